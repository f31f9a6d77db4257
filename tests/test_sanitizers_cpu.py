"""CPU-only sanitizer runs (AddressSanitizer + UndefinedBehaviorSanitizer).

1. The oracle, built with gcc's ASan/UBSan, runs its pin tests (loaded through
   the oracle's alternate-library hook, in a child process with gcc's ASan
   runtime preloaded).
2. The library's host code -- every entry point's argument checks in
   simsd_api.hip -- built with clang's ASan/UBSan on the host side only (the
   gfx950 device code is built as usual), runs the C-ABI tests in a child
   process with clang's ASan runtime preloaded. Those tests stop every call
   before a kernel launch, so no GPU is needed.
3. Canaries: a planted heap overflow and a planted signed overflow in a tiny C
   file, built each way, must abort the child -- proof that each sanitizer
   setup is live.
Nothing here touches a GPU."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
OPTS = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1", "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
PIN_FILES = sorted(os.path.join(ROOT, "tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_oracle_") and f.endswith(".py") and f != "test_oracle_mutants.py")

CANARY = r"""
#include <limits.h>
#include <stdlib.h>
int heap_overflow(int i) { int* p = (int*)malloc(4 * sizeof(int)); int v = p[4 + i]; free(p); return v; }
int signed_overflow(int x) { return x + INT_MAX; }
"""


def _gcc_runtime():
    return subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()


def _clang_runtime():
    found = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return found[0] if found else None


def _run(code, runtime, *args):
    env = dict(os.environ, LD_PRELOAD=runtime, **OPTS)
    return subprocess.run([sys.executable, "-c", code, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=600)


CALL_CANARY = "import ctypes, sys; lib = ctypes.CDLL(sys.argv[1]); print(getattr(lib, sys.argv[2])(int(sys.argv[3])))"


def _canaries(lib, runtime):
    r = _run(CALL_CANARY, runtime, lib, "heap_overflow", "0")
    # (either sanitizer may report the read first)
    assert r.returncode != 0 and ("heap-buffer-overflow" in r.stderr or "runtime error" in r.stderr), r.stderr[-500:]
    r = _run(CALL_CANARY, runtime, lib, "signed_overflow", "5")
    assert r.returncode != 0 and "overflow" in r.stderr, r.stderr[-500:]


def test_oracle_pins_under_gcc_sanitizers(tmp_path):
    flags = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-fPIC", "-shared"]
    src = tmp_path / "canary.c"
    src.write_text(CANARY)
    subprocess.check_call(["gcc", *flags, str(src), "-o", str(tmp_path / "canary.so")])
    _canaries(str(tmp_path / "canary.so"), _gcc_runtime())
    lib = tmp_path / "liboracle_asan.so"
    subprocess.check_call(["gcc", *flags, "-std=c11", "-ffp-contract=off",
                           os.path.join(ROOT, "oracle", "simsd_oracle.c"), "-o", str(lib), "-lm"])
    env_code = ("import os, sys, pytest; os.environ['SIMSD_ORACLE_MUTANT_LIB'] = sys.argv[1]; "
                "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu', *sys.argv[2:]]))")
    r = _run(env_code, _gcc_runtime(), str(lib), *PIN_FILES)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-2000:])
    assert " passed" in r.stdout


def test_host_checks_under_clang_sanitizers(tmp_path):
    runtime = _clang_runtime()
    build = os.path.join(ROOT, "masked_attention_simsd_amd", "_build")
    objs = [os.path.join(build, f"{n}.o") for n in ("rope_copy", "verify_attention", "accept", "commit_kv")]
    if runtime is None or not all(os.path.exists(o) for o in objs):
        pytest.skip("clang ASan runtime or built objects missing")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    src = tmp_path / "canary.c"
    src.write_text(CANARY)
    clang = "/opt/rocm/lib/llvm/bin/clang"
    subprocess.check_call([clang, "-O1", "-g", "-fPIC", "-shared", "-shared-libsan", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", str(src), "-o", str(tmp_path / "canary.so")])
    _canaries(str(tmp_path / "canary.so"), runtime)
    api = tmp_path / "api.o"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
                           "-fno-omit-frame-pointer", *san, "-Xclang", "-target-feature", "-Xclang",
                           "-packed-fp32-ops", f"-I{ROOT}/include", f"-I{ROOT}/masked_attention_simsd_amd/csrc",
                           "-c", os.path.join(ROOT, "masked_attention_simsd_amd", "csrc", "simsd_api.hip"),
                           "-o", str(api)], stderr=subprocess.DEVNULL)
    lib = tmp_path / "libsimsd_asan.so"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan", *san, str(api),
                           *objs, "-o", str(lib)])
    code = ("import sys; sys.path.insert(0, '.'); from masked_attention_simsd_amd import binding; "
            "binding.load_library(sys.argv[1]); import pytest; "
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', 'tests/test_abi_cpu.py']))")
    r = _run(code, runtime, str(lib))
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-2000:])
    assert " passed" in r.stdout
