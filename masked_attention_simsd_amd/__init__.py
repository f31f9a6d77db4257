"""SimSD verification hot path for MI355X (gfx950).

The compute path is libsimsd.so (HIP kernels behind the C ABI of
include/simsd.h); ``binding`` exposes its entry points to Python under the
same names (every name in ``binding.EXPORTS``, plus the binding's flags,
status codes and helpers), and they are re-exported here on first use.
``synth`` draws the seeded synthetic inputs.
"""
import importlib

_SUBMODULES = ("binding", "synth", "build")


def __getattr__(name):
    # lazy: importing the package does not load torch or the library
    if name.startswith("_") or name in _SUBMODULES:
        raise AttributeError(name)
    binding = importlib.import_module(__name__ + ".binding")
    if hasattr(binding, name):
        return getattr(binding, name)
    raise AttributeError(name)
