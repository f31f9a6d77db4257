"""The benchmark's host-side parts, without a GPU: the algorithmic bytes and
flops it divides by (against the closed forms of the per-block work), the
rule that counter traffic is reported only for the kernel source it was
measured on, the rocprofv3 summary, and the single-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from masked_attention_simsd_amd import synth  # noqa: E402


def test_algorithmic_bytes_and_flops_of_the_b8_workload():
    # per sequence (prefix P = 4096, B = 8, 32/8 heads, d = 128): the prefix K and V
    # 4 d Hkv P, Q and O plus block K and V 8 B d (Hq + Hkv), tau and offset 4 B + 4;
    # flops 4 d Hq (2 B P + B^2 + B (B + 1) / 2)
    w = synth.CONFIGS["b8"]
    nbytes, flops = bench.attn_bytes_flops(w, [4096] * 16, fused=False)
    per_seq = 4 * 128 * 8 * 4096 + 8 * 8 * 128 * 40 + 4 * 8 + 4
    assert nbytes == 16 * per_seq == 273_678_912
    assert flops == 16 * 4 * 128 * 32 * (2 * 8 * 4096 + 64 + 36) == 17_206_083_584
    # the fused form also writes the rotated block keys and reads the start position
    nb_f, fl_f = bench.attn_bytes_flops(w, [4096] * 16, fused=True)
    assert nb_f - nbytes == 16 * (4 * 8 * 128 * 8 + 4) and fl_f == flops
    # ragged prefixes add up per sequence
    nb_r, _ = bench.attn_bytes_flops(w, [512, 8192], fused=False)
    assert nb_r == bench.attn_bytes_flops(w, [512], False)[0] + bench.attn_bytes_flops(w, [8192], False)[0]


def test_counter_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    f = tmp_path / "verify_attention_b8_counters.txt"
    f.write_text("# a summary\nsource_sha256_16: abcdef0123456789\nhbm_bytes_per_launch: 123.5\n")
    monkeypatch.setattr(bench, "counter_file", lambda workload: str(f))
    monkeypatch.setattr(bench, "attn_source_hash", lambda: "abcdef0123456789")
    assert bench.counter_summary("b8", "hbm_bytes_per_launch") == 123.5
    assert bench.counter_summary("b8", "missing_key") is None
    monkeypatch.setattr(bench, "attn_source_hash", lambda: "0000000000000000")
    assert bench.counter_summary("b8", "hbm_bytes_per_launch") is None


def test_committed_counter_summaries_name_a_source_hash():
    for w in ("b8", "b16", "ragged"):
        text = open(bench.counter_file(w)).read()
        assert "source_sha256_16:" in text, w


def test_rocprof_summary(tmp_path, capsys):
    (tmp_path / "run").mkdir()
    (tmp_path / "run" / "t_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"verify_attn_kernel<128>",4,200000,50000.0,90.0,49000,51000,800.0\n')
    bench.summarize_rocprof(str(tmp_path))
    out = capsys.readouterr().out
    assert "verify_attn_kernel<128>" in out and "avg_us     50.000" in out and "calls      4" in out


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_committed_bench_lines_follow_the_contract():
    # every line in profiles/bench_lines.txt carries the contract's keys, and
    # its roofline figures are the algorithmic bytes over the reported launch
    # time (no figure typed in by hand)
    import json
    lines = [l for l in open(os.path.join(ROOT, "profiles", "bench_lines.txt")) if not l.startswith("#")]
    assert len(lines) == 3
    for l in lines:
        w, j = l.split(": ", 1)
        d = json.loads(j)
        for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                    "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "parity"):
            assert key in d, (w, key)
        assert d["n_gpus"] == 1 and d["dtype"] == "bf16" and d["metric"] == bench.METRIC
        r = d["roofline"]
        x = synth.make_inputs(w, with_accept=False, with_attn=False)
        nbytes, _ = bench.attn_bytes_flops(synth.CONFIGS[w], x["prefix_lens"].tolist(), fused=False)
        assert r["algorithmic_bytes_per_launch"] == nbytes
        assert abs(r["achieved"] - nbytes / r["avg_launch_us"] / 1e3) <= 0.1
        assert abs(r["frac"] - r["achieved"] / r["peak"]) <= 1e-4
        assert r["avg_launch_us"] == d["kernels_us"]["verify_attention"]["in_steps"]["mean_us"]
        assert abs(d["value"] - d["config"]["global_batch"] / d["ms_per_step"] * 1e3) / d["value"] < 2e-3
        if w == "b8":
            assert d["cpu_baseline"] is not None and d["parity"]["accept_len_equal"] == 16
