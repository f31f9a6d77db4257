"""Verify attention on the GPU against the oracle.

Tolerance: max-abs 2e-2 for bf16 output (bf16 inputs, fp32 accumulation);
the fp32-output path is held to 4e-3 to separate kernel arithmetic from the
final bf16 rounding."""

import numpy as np
import pytest
import torch

import oracle
from masked_attention_simsd_amd import binding, synth
from gpu_util import ORACLE_THREADS, f64, inputs, say, subset_sequences, to_dev

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_F32 = 4e-3


def head_major(x):
    """The same inputs with the prefix cache stored [Hkv][sum P][d]."""
    y = dict(x)
    y["k_pre"] = x["k_pre"].transpose(0, 1).contiguous()
    y["v_pre"] = x["v_pre"].transpose(0, 1).contiguous()
    return y


def run_gpu(x, flags=0, max_prefix=None, status=None, lse=True):
    if flags & binding.SIMSD_KV_HEAD_MAJOR:
        x = head_major(x)
    g = to_dev(x)
    if flags & binding.SIMSD_KV_PAIRED:
        # one buffer [..][..][2][d]: each token's key row, then its value row
        kv = torch.stack([g["k_pre"], g["v_pre"]], dim=2).contiguous()
        g["k_pre"], g["v_pre"] = binding.kv_pair_views(kv)
    b, twoB, Hq, _ = x["q_blk"].shape
    if max_prefix is None:
        lens = x["prefix_offsets"][1:] - x["prefix_offsets"][:-1]
        max_prefix = int(lens.max())
    lse_t = torch.full((b, twoB, Hq), float("nan"), device="cuda") if lse else None
    out = binding.simsd_verify_attention(g["q_blk"], g["k_blk"], g["v_blk"], g["k_pre"], g["v_pre"],
                                         g["prefix_offsets"], g["tau"], lse=lse_t,
                                         max_prefix=max_prefix, flags=flags, status=status)
    torch.cuda.synchronize()
    return out, lse_t


def run_oracle(x, rule=0):
    return oracle.verify_attention(f64(x["q_blk"]), f64(x["k_blk"]), f64(x["v_blk"]),
                                   f64(x["k_pre"]), f64(x["v_pre"]), x["prefix_offsets"].numpy(),
                                   x["tau"].numpy(), data_rule=rule, threads=ORACLE_THREADS)


def compare(out, lse, ref, ref_lse, rule, tol, what):
    got = f64(out)
    rows = slice(None) if rule != 2 else slice(ref.shape[1] // 2, None)
    err = float(np.abs(got[:, rows] - ref[:, rows]).max())
    lerr = float(np.abs(f64(lse)[:, rows] - ref_lse[:, rows]).max()) if lse is not None else 0.0
    say(f"  {what}: max-abs {err:.3e}, lse max-abs {lerr:.3e}")
    assert err <= tol, what
    assert lerr <= 2e-3, what


SHAPES = [
    # (b, Hq, Hkv, d, B, prefix range)   -- tails, tiny and empty prefixes, wide and narrow groups
    (1, 1, 1, 64, 4, (32, 32)),
    (2, 4, 1, 64, 3, (0, 70)),
    (3, 8, 2, 128, 8, (100, 700)),
    (2, 32, 8, 128, 4, (1000, 4100)),
    (1, 8, 8, 128, 1, (0, 0)),
    (2, 16, 2, 128, 8, (63, 65)),
    (1, 32, 8, 128, 16, (2049, 2049)),
    (1, 4, 1, 64, 64, (130, 130)),
    (4, 32, 4, 128, 5, (1, 3000)),
    (2, 32, 8, 128, 64, (100, 1500)),  # the largest block (B = 64): 512 rows per KV head in 4 slices
]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
@pytest.mark.parametrize("rule", [0, 1, 2])
def test_shapes_match_oracle(shape, rule):
    b, Hq, Hkv, d, B, pre = shape
    w = synth.custom(b=b, Hq=Hq, Hkv=Hkv, d=d, B=B, prefix=pre)
    say(f"attention shape={shape} rule={rule}")
    x = synth.make_inputs(w, with_accept=False, seed=hash(shape) % 1000)
    ref, ref_lse = run_oracle(x, rule)
    out, lse = run_gpu(x, flags=rule | binding.SIMSD_OUT_F32)
    compare(out, lse, ref, ref_lse, rule, TOL_F32, "fp32 out")
    out, lse = run_gpu(x, flags=rule)
    compare(out, lse, ref, ref_lse, rule, TOL_BF16, "bf16 out")
    out, lse = run_gpu(x, flags=rule | binding.SIMSD_OUT_F32 | binding.SIMSD_KV_HEAD_MAJOR)
    compare(out, lse, ref, ref_lse, rule, TOL_F32, "fp32 out, head-major cache")


@pytest.mark.parametrize("B", [8, 16], ids=["64_rows", "128_rows"])
def test_every_kernel_variant_matches_oracle(B):
    # Each key-tile ring / wave layout the launcher can select (tuning key
    # attn_pipe) on a batch with several tiles per split, ragged tails and an
    # empty prefix.
    w = synth.custom(b=3, Hq=32, Hkv=8, d=128, B=B, prefix=(0, 2100))
    x = synth.make_inputs(w, with_accept=False, seed=31 + B)
    ref, ref_lse = run_oracle(x)
    for pipe in range(10):
        with binding.tuning(attn_pipe=pipe, attn_chunk_max=512):
            out, lse = run_gpu(x, flags=binding.SIMSD_OUT_F32 | binding.SIMSD_KV_HEAD_MAJOR)
        compare(out, lse, ref, ref_lse, 0, TOL_F32, f"pipe {pipe}")


_WORKLOAD_REFS = {}  # oracle results per (workload, sequences): the layout does not change them


# The last layout is the one the benchmark times (paired head-major); on ragged
# it runs the longest-first schedule.
@pytest.mark.parametrize("layout", [0, binding.SIMSD_KV_HEAD_MAJOR,
                                    binding.SIMSD_KV_HEAD_MAJOR | binding.SIMSD_KV_PAIRED],
                         ids=["token_major", "head_major", "paired_head_major"])
@pytest.mark.parametrize("cfg,seqs", [("tiny", None), ("b4", None), ("b8", None), ("b16", None), ("ragged", None)])
def test_workloads_match_oracle(cfg, seqs, layout):
    # every sequence of every workload, element by element (the oracle result
    # of a workload is computed once and reused for the three layouts)
    say(f"attention workload {cfg} layout {layout}")
    x = inputs(cfg)
    out, lse = run_gpu(x, flags=layout)
    key = (cfg, None if seqs is None else tuple(seqs))
    if key not in _WORKLOAD_REFS:
        _WORKLOAD_REFS[key] = run_oracle(x if seqs is None else subset_sequences(x, seqs))
    ref, ref_lse = _WORKLOAD_REFS[key]
    if seqs is None:
        compare(out, lse, ref, ref_lse, 0, TOL_BF16, cfg)
    else:
        idx = torch.tensor(seqs, device="cuda")
        compare(out[idx], lse[idx], ref, ref_lse, 0, TOL_BF16, f"{cfg} seqs {seqs}")


def test_hidden_keys_do_not_change_slot_rows_bit_exact():
    # Large finite changes to keys/values a mask slot must not see leave its
    # output bit-identical (masked keys are excluded, not down-weighted).
    w = synth.custom(b=2, Hq=8, Hkv=2, d=128, B=8, prefix=(300, 300))
    x = synth.make_inputs(w, with_accept=False, seed=77)
    base, _ = run_gpu(x)
    tau = x["tau"]
    for s in range(2):
        for i in range(8):
            y = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in x.items()}
            hidden_d = [j for j in range(8) if tau[s, j] >= tau[s, i]]
            hidden_t = [8 + j for j in range(8) if tau[s, j] < tau[s, i]]
            for c in hidden_d + hidden_t:
                y["k_blk"][s, c] = 30.0
                y["v_blk"][s, c] = -1000.0
            out, _ = run_gpu(y)
            assert torch.equal(out[s, 8 + i], base[s, 8 + i]), (s, i)


@pytest.mark.parametrize("value", [float("nan"), float("inf"), float("-inf")], ids=["nan", "inf", "-inf"])
@pytest.mark.parametrize("shape", [(2, 8, 2, 128, 8, 300), (1, 32, 8, 128, 16, 600), (2, 4, 1, 64, 5, 90)],
                         ids=["b2_B8", "b1_B16_128rows", "d64_B5"])
def test_non_finite_hidden_keys_do_not_change_slot_rows(shape, value):
    # NaN or Inf in the key AND value rows of every block key a mask slot may
    # not see leave that slot's output and lse bit-identical; a mask slot that
    # sees such a value propagates it exactly as the oracle's plain softmax
    b, Hq, Hkv, d, B, P = shape
    say(f"non-finite hidden keys {shape} value {value}")
    w = synth.custom(b=b, Hq=Hq, Hkv=Hkv, d=d, B=B, prefix=(P, P))
    x = synth.make_inputs(w, with_accept=False, seed=78)
    fl = binding.SIMSD_OUT_F32
    base, base_lse = run_gpu(x, flags=fl)
    tau = x["tau"]
    for s in range(b):
        for i in range(B):
            y = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in x.items()}
            hidden_d = [j for j in range(B) if tau[s, j] >= tau[s, i]]
            hidden_t = [B + j for j in range(B) if tau[s, j] < tau[s, i]]
            for c in hidden_d + hidden_t:
                y["k_blk"][s, c] = value
                y["v_blk"][s, c] = value
            out, lse = run_gpu(y, flags=fl)
            assert torch.equal(out[s, B + i], base[s, B + i]), (s, i)
            assert torch.equal(lse[s, B + i], base_lse[s, B + i]), (s, i)
            # every other sequence is untouched
            others = [t for t in range(b) if t != s]
            assert torch.equal(out[others], base[others])
    # visible: a value vector of one data token with a NaN / Inf entry reaches
    # exactly the rows that see that token, as in the oracle
    y = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in x.items()}
    j = int((tau[0] == 1).nonzero()[0, 0])  # step 1: seen by every later mask slot
    y["v_blk"][0, j, :, 3] = value
    out, lse = run_gpu(y, flags=fl)
    ref, ref_lse = run_oracle(y)
    o, r = out.cpu().double().numpy(), ref
    assert np.array_equal(np.isnan(o), np.isnan(r)) and np.array_equal(np.isinf(o), np.isinf(r))
    fin = np.isfinite(r)
    assert np.abs(o[fin] - r[fin]).max() <= TOL_F32


def test_deterministic_and_split_independent():
    x = inputs("b8")
    a, _ = run_gpu(x, flags=binding.SIMSD_OUT_F32)
    b, _ = run_gpu(x, flags=binding.SIMSD_OUT_F32)
    assert torch.equal(a, b), "two identical calls differ"
    for target in (1, 4096):
        with binding.tuning(attn_target_wg=target):
            c, _ = run_gpu(x, flags=binding.SIMSD_OUT_F32)
        err = float((c - a).abs().max())
        say(f"  target {target}: max diff vs default {err:.2e}")
        assert err < 2e-3


def test_status_bits():
    # tau not a permutation of 1..B: a repeated label, a label 0, a label past B
    w = synth.custom(b=4, Hq=4, Hkv=2, d=64, B=4, prefix=(50, 90))
    x = synth.make_inputs(w, with_accept=False, seed=5)
    x["tau"][1] = torch.tensor([1, 1, 2, 3], dtype=torch.int32)
    x["tau"][2] = torch.tensor([0, 1, 2, 3], dtype=torch.int32)
    x["tau"][3] = torch.tensor([1, 2, 3, 5], dtype=torch.int32)
    status = torch.zeros(4, dtype=torch.int32, device="cuda")
    lens = (x["prefix_offsets"][1:] - x["prefix_offsets"][:-1]).tolist()
    short = int(min(lens))
    run_gpu(x, status=status, max_prefix=short)
    st = status.cpu().tolist()
    for s in range(4):
        assert bool(st[s] & binding.SIMSD_DEV_BAD_PREFIX) == (lens[s] > short)
        assert bool(st[s] & binding.SIMSD_DEV_BAD_TAU) == (s != 0)


def test_one_workspace_shared_by_calls_of_different_shapes():
    # Calls of different shapes leave partial results in the shared workspace;
    # none of them may disturb the counter words the next shape relies on.
    shapes = [synth.custom(b=2, Hq=32, Hkv=8, d=128, B=4, prefix=(1000, 4100)),
              synth.custom(b=1, Hq=32, Hkv=8, d=128, B=16, prefix=(2049, 2049)),
              synth.custom(b=3, Hq=4, Hkv=1, d=64, B=3, prefix=(0, 700))]
    xs = [synth.make_inputs(w, with_accept=False, seed=40 + i) for i, w in enumerate(shapes)]
    xs.append(inputs("b8"))
    refs = [run_oracle(x)[0] for x in xs]
    need = max(binding.simsd_verify_attention_workspace(
        x["q_blk"].shape[0], x["q_blk"].shape[1] // 2, x["q_blk"].shape[2], x["k_blk"].shape[2],
        x["q_blk"].shape[3], int((x["prefix_offsets"][1:] - x["prefix_offsets"][:-1]).max()))
        for x in xs)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    gs = [to_dev(x) for x in xs]
    for rnd in range(2):
        for i in (0, 3, 1, 3, 2, 3):
            g, x = gs[i], xs[i]
            out = binding.simsd_verify_attention(
                g["q_blk"], g["k_blk"], g["v_blk"], g["k_pre"], g["v_pre"], g["prefix_offsets"],
                g["tau"], flags=binding.SIMSD_DATA_CAUSAL | binding.SIMSD_OUT_F32, workspace=ws,
                max_prefix=int((x["prefix_offsets"][1:] - x["prefix_offsets"][:-1]).max()))
            torch.cuda.synchronize()
            err = float(np.abs(f64(out) - refs[i]).max())
            assert err <= TOL_F32, (rnd, i, err)
    assert int(ws[:262144].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("b,prefix,layout", [
    (40, (16, 3000), binding.SIMSD_KV_HEAD_MAJOR | binding.SIMSD_KV_PAIRED),  # > 256 units, longest first
    (72, (16, 600), binding.SIMSD_KV_HEAD_MAJOR),                             # > 64 sequences: two per CU
    (72, (0, 900), 0),
], ids=["lpt_b40", "b72_head_major", "b72_token_major"])
def test_large_batch_schedules_match_oracle(b, prefix, layout):
    """Unsplit launches of more than 256 workgroups: the longest-first order
    (at most 64 sequences) and the plain order beyond 64 sequences, checked on
    a sample of sequences that includes the longest and the shortest."""
    say(f"large batch b={b} prefix={prefix} layout={layout}")
    w = synth.custom(b=b, Hq=32, Hkv=8, d=128, B=8, prefix=prefix)
    x = synth.make_inputs(w, with_accept=False, seed=31 + b)
    out, lse = run_gpu(x, flags=layout)
    lens = (x["prefix_offsets"][1:] - x["prefix_offsets"][:-1]).tolist()
    seqs = sorted({0, 1, b // 2, b - 1, int(np.argmin(lens)), int(np.argmax(lens))})
    ref, ref_lse = run_oracle(subset_sequences(x, seqs))
    idx = torch.tensor(seqs, device="cuda")
    compare(out[idx], lse[idx], ref, ref_lse, 0, TOL_BF16, f"b={b} seqs {seqs}")
