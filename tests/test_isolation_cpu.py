"""The product path and the oracle stay apart, and the product path has no
fallback: the HIP library's sources and its binding never name the oracle,
the oracle never names the HIP path, importing the binding loads no oracle
module, and a missing library is an error rather than a silent substitute."""
import glob
import os
import subprocess
import sys

import pytest

from masked_attention_simsd_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sources(*patterns):
    out = []
    for p in patterns:
        out += glob.glob(os.path.join(ROOT, p), recursive=True)
    assert out, patterns
    return out


def test_product_sources_never_name_the_oracle():
    files = _sources("masked_attention_simsd_amd/**/*.py", "masked_attention_simsd_amd/csrc/*.hip",
                     "masked_attention_simsd_amd/csrc/*.h", "include/*.h")
    for f in files:
        text = open(f).read()
        for word in ("import oracle", "from oracle", "simsd_oracle", "oracle/"):
            assert word not in text, f"{os.path.relpath(f, ROOT)} names the oracle ({word!r})"


def test_oracle_never_names_the_hip_path():
    for f in _sources("oracle/*.py", "oracle/*.c"):
        text = open(f).read()
        for word in ("masked_attention_simsd_amd", "simsd_internal", "libsimsd.so", "include/simsd.h",
                     "#include \"simsd"):
            assert word not in text, f"{os.path.relpath(f, ROOT)} names the HIP path ({word!r})"


def test_importing_the_binding_loads_no_oracle():
    code = "import sys, masked_attention_simsd_amd.binding, masked_attention_simsd_amd.synth; " \
           "sys.exit(1 if any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules) else 0)"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-500:]


def test_missing_library_is_an_error(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        binding.load_library(str(tmp_path / "libsimsd.so"))


def test_package_reexports_every_entry_point():
    import masked_attention_simsd_amd as pkg
    from masked_attention_simsd_amd import binding
    # every C entry point the binding wraps under its own name (the status
    # string and last-error calls are used inside the binding only)
    wrapped = [n for n in binding.EXPORTS if hasattr(binding, n)]
    assert len(wrapped) >= len(binding.EXPORTS) - 2
    for name in wrapped + ["SimsdError", "load_library", "tuning", "SIMSD_ROPE_POSITIONS"]:
        assert getattr(pkg, name) is getattr(binding, name), name


def test_exp2_fraction_table_is_correctly_rounded():
    # the statistics pass's table of 2^(j/256): every entry the fp64 value
    # nearest the exact one (80-digit decimal arithmetic here)
    import re
    from decimal import Decimal, getcontext
    src = open(os.path.join(ROOT, "masked_attention_simsd_amd", "csrc", "accept.hip")).read()
    body = src[src.index("kExp2Frac[256] = {"):]
    body = body[:body.index("};")]
    vals = [float.fromhex(h) for h in re.findall(r"0x[0-9a-f.]+p[+-]\d+", body)]
    assert len(vals) == 256
    getcontext().prec = 80
    for j, v in enumerate(vals):
        exact = Decimal(2) ** (Decimal(j) / 256)
        assert v == float(exact), j
        # neither neighbouring double is closer to the exact value
        import math
        for nb in (math.nextafter(v, 0.0), math.nextafter(v, 4.0)):
            assert abs(Decimal(nb) - exact) >= abs(Decimal(v) - exact), j
