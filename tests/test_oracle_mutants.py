"""The pins of the oracle catch plausible mistakes.

Each mutant below is a copy of the C oracle with one planted mistake of the
kind the pins are meant to catch (an off-by-one in the temporal mask, a
dropped term, a wrong sign, index or operand). Every mutant is compiled the
way the oracle is, and the oracle's pin tests are run against it in a child
process (the oracle loads the mutant through its MUTANT_ENV hook): at least
one pin must fail for every mutant, and none for an unaltered copy. Nothing
here touches a GPU or the HIP library."""
import json
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = sorted(
    os.path.join("tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
    if f.startswith("test_oracle_") and f.endswith(".py") and f != os.path.basename(__file__))

# name -> list of (text in the oracle source, replacement); each text occurs once.
# (Leaving the ratio min(1, p/q) uncapped is not among them: with u in [0, 1)
# the decision u < r is the same for every r >= 1, so it is no mistake.)
MUTANTS = {
    # temporal mask ([nl]/[fr] Methodologie 2)
    "slot_sees_data_of_its_own_step": [("if (!k_is_slot) return tj < ti;", "if (!k_is_slot) return tj <= ti;")],
    "slot_misses_itself": [("    return tj >= ti;\n  }", "    return tj > ti;\n  }")],
    "data_rows_see_slots": [("  if (k_is_slot) return 0;", "  if (k_is_slot) return 1;")],
    "data_rule_reversed": [("  return tj <= ti;\n}", "  return tj >= ti;\n}")],
    # attention
    "slots_lose_the_prefix": [("ok[j] = 1; /* the whole cached prefix is visible */", "ok[j] = qr < B;")],
    "scale_dropped": [("    s[j] = dot * scale;", "    s[j] = dot;")],
    "lse_without_max": [("  *lse = m + log(denom);", "  *lse = log(denom);")],
    "gqa_head_by_modulo": [("h / G, r,", "h % Hkv, r,")],
    "prefix_head_stride_transposed": [("kj = k_pre + ((size_t)j * Hkv + g) * d;",
                                       "kj = k_pre + ((size_t)g * P + j) * d;")],
    "values_read_from_keys": [("const double* vj = j < P ? v_pre + ((size_t)j * Hkv + g) * d",
                               "const double* vj = j < P ? k_pre + ((size_t)j * Hkv + g) * d")],
    "block_head_offset_dropped": [("kj = k_blk + ((size_t)(j - P) * Hkv + g) * d;",
                                   "kj = k_blk + ((size_t)(j - P) * Hkv) * d;")],
    # RoPE with the copy rule ([nl]/[fr] Methodologie 3)
    "rope_sign": [("v[bb] = xb * c + xa * sn;", "v[bb] = xb * c - xa * sn;")],
    "rope_frequency_exponent": [("pow(base, -2.0 * i / d)", "pow(base, -1.0 * i / d)")],
    "rope_no_copy_rule": [("int k = r < B ? r : r - B;", "int k = r;")],
    "rope_pairs_mirrored": [("int bb = interleaved ? 2 * i + 1 : i + half;",
                             "int bb = interleaved ? 2 * i + 1 : d - 1 - i;")],
    "rope_position_off_by_one": [("(long)start_pos[s] + k;", "(long)start_pos[s] + k + 1;")],
    "rope_positions_of_the_first_pair": [("(long)positions[(size_t)s * B + k]", "(long)positions[(size_t)s * B]")],
    # acceptance ([nl]/[fr] Methodologie 4)
    "accept_non_strict": [("if (!(us[t - 1] < r)) {", "if (!(us[t - 1] <= r)) {")],
    "accept_in_position_order": [("      int k = inv[t - 1];\n", "      int k = t - 1;\n")],
    "ratio_inverted": [("          r = a / c;\n", "          r = c / a;\n")],
    "residual_sign": [("float rho = pk[y] - qk[y];", "float rho = qk[y] - pk[y];"),
                      ("        w = pk[y] - qk[y];", "        w = qk[y] - pk[y];")],
    "correction_row_by_position": [("int kstar = inv[L];", "int kstar = L;")],
    "correction_uniform_of_step": [("double T = (double)us[B] * Z", "double T = (double)us[L] * Z")],
    "cdf_not_strict": [("if (pick < 0 && C > T) {", "if (pick < 0 && C >= T) {")],
    "q_zero_rule_rejects": [("          r = a > 0.0f ? 1.0f : 0.0f;", "          r = 0.0f;")],
    # softmax at a temperature
    "softmax_temperature_multiplies": [("s += exp(((double)zr[y] - m) / temperature);",
                                        "s += exp(((double)zr[y] - m) * temperature);"),
                                       ("o[y] = (float)(exp(((double)zr[y] - m) / temperature) / s);",
                                        "o[y] = (float)(exp(((double)zr[y] - m) * temperature) / s);")],
    "softmax_unnormalised": [("o[y] = (float)(exp(((double)zr[y] - m) / temperature) / s);",
                              "o[y] = (float)(exp(((double)zr[y] - m) / temperature));")],
    # attention under an explicit block mask
    "explicit_mask_transposed": [("ok[j] = (char)(arow[j - P] != 0);",
                                  "ok[j] = (char)(allowed[((size_t)s * R + (j - P)) * R + r] != 0);")],
}


# Mutants of the Python-side row movement (commit_kv, pack_regions): the child
# re-executes the oracle module's source with the edit applied, in place, before
# running the pins.
PY_MUTANTS = {
    "commit_in_position_order": [("k = int(inv[step])", "k = step")],
    "commit_mask_slot_rows": [("kc[:, row] = kb[s, k]\n", "kc[:, row] = kb[s, k + B]\n"),
                              ("kc[row] = kb[s, k]\n", "kc[row] = kb[s, k + B]\n"),
                              ("vc[:, row] = vb[s, k]\n", "vc[:, row] = vb[s, k + B]\n"),
                              ("vc[row] = vb[s, k]\n", "vc[row] = vb[s, k + B]\n")],
    "commit_row_off_by_one": [("row = int(off[s]) + int(ln[s]) + step", "row = int(off[s]) + int(ln[s]) + step + 1")],
    "commit_length_kept": [("ln[s] += L", "ln[s] += 0")],
    "commit_overflow_off_by_one": [("int(ln[s]) + L > cap", "int(ln[s]) + L > cap + 1")],
    "commit_values_from_keys": [("vc[:, row] = vb[s, k]", "vc[:, row] = kb[s, k]"),
                                ("vc[row] = vb[s, k]", "vc[row] = kb[s, k]")],
    "next_correction_not_first": [("row.append(int(ps[s, inv[L]]))  # the correction's position\n", ""),
                                  ("for j in range(L + 1, B))", "for j in range(L, B))")],
    "next_frontier_off_by_one": [("frontier = int(ps[s].max()) + 1", "frontier = int(ps[s].max())")],
    "next_reopens_an_accepted_position": [("for j in range(L + 1, B))", "for j in range(L - 1 if L else 1, B))"),
                                          ("row += [frontier + i for i in range(L)]",
                                           "row += [frontier + i for i in range(L)]\n        row = row[:B]")],
    "committed_in_position_order": [("out.append([int(ps[s, inv[j]]) for j in range(L)]",
                                     "out.append([int(ps[s, j]) for j in range(L)]")],
    "pack_whole_regions": [("np.arange(off[s], off[s] + ln[s])", "np.arange(off[s], off[s + 1])")],
    "pack_offsets_of_regions": [("po[1:] = np.cumsum(ln)", "po[1:] = np.cumsum(np.diff(off))")],
}

_PY_CHILD = """
import json, os, sys
import oracle
src = open(oracle.__file__).read()
for old, new in json.loads(os.environ["ORACLE_PY_EDITS"]):
    assert src.count(old) == 1, old
    src = src.replace(old, new)
exec(compile(src, oracle.__file__, "exec"), oracle.__dict__)
import pytest
sys.exit(pytest.main(sys.argv[1:]))
"""


def _mutate(src: str, edits) -> str:
    for old, new in edits:
        assert src.count(old) == 1, f"mutation anchor not unique or missing: {old!r}"
        src = src.replace(old, new)
    return src


def _run_pins(lib_path: str, py_edits=None):
    env = dict(os.environ)
    env[oracle.MUTANT_ENV] = lib_path
    args = ["-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *PIN_FILES]
    if py_edits:
        env["ORACLE_PY_EDITS"] = json.dumps(py_edits)
        cmd = [sys.executable, "-c", _PY_CHILD, *args]
    else:
        cmd = [sys.executable, "-m", "pytest", *args]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    lines = r.stdout.strip().splitlines()
    return r.returncode, lines[-1] if lines else r.stderr[-300:]


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    src = open(oracle.SRC).read()
    d = tmp_path_factory.mktemp("oracle_mutants")
    libs = {}
    for name, edits in [("unaltered", [])] + list(MUTANTS.items()):
        c = d / f"{name}.c"
        c.write_text(_mutate(src, edits))
        lib = str(d / f"{name}.so")
        oracle.compile_source(str(c), lib)
        libs[name] = lib
    with ThreadPoolExecutor(max_workers=4) as ex:
        futs = {name: ex.submit(_run_pins, lib) for name, lib in libs.items()}
        futs.update({name: ex.submit(_run_pins, libs["unaltered"], edits) for name, edits in PY_MUTANTS.items()})
        return {name: f.result() for name, f in futs.items()}


def test_unaltered_copy_passes_every_pin(outcomes):
    rc, summary = outcomes["unaltered"]
    assert rc == 0, summary


@pytest.mark.parametrize("name", sorted(MUTANTS) + sorted(PY_MUTANTS))
def test_pins_catch_mutant(outcomes, name):
    rc, summary = outcomes[name]
    # a pin must fail (an assertion, reported by pytest), not the process crash
    assert rc == 1 and "failed" in summary, f"mutant {name} survived the pins: {summary}"
