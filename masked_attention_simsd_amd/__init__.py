"""SimSD verification hot path for MI355X (gfx950).

The compute path is libsimsd.so (HIP kernels behind the C ABI of
include/simsd.h); ``binding`` exposes its entry points to Python under the
same names. ``synth`` draws the seeded synthetic inputs.
"""

_BINDING_NAMES = (
    "simsd_rope_copy", "simsd_verify_attention", "simsd_verify_attention_workspace",
    "simsd_accept", "SimsdError", "load_library",
)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
