"""KV commit (simsd_commit_kv) and attention over cache regions with room to
grow (SIMSD_PREFIX_LENS) on the GPU: the commit is bit-exact against the
oracle (rows, lengths, status), attention over regions equals attention over
the same rows packed (and never reads past the used rows), and several rounds
of RoPE-copy -> attention -> acceptance -> commit, all on the device with no
host round trip, follow the oracle's own chain."""
import numpy as np
import pytest
import torch

import oracle
from masked_attention_simsd_amd import binding, synth
from gpu_util import ORACLE_THREADS, bf16_round, bf16_ulp, f64, say

pytestmark = pytest.mark.gpu

NAN_BF16 = float("nan")


def regions(rng, caps):
    off = np.zeros(len(caps) + 1, np.int32)
    off[1:] = np.cumsum(caps)
    return off


@pytest.mark.parametrize("shape", [(5, 8, 2, 128, False), (3, 16, 8, 128, True), (4, 1, 1, 64, False),
                                   (2, 64, 4, 64, True)])
def test_commit_matches_oracle(shape):
    b, B, Hkv, d, head_major = shape
    say(f"commit {shape}")
    rng = np.random.default_rng(b * 100 + B)
    lens = rng.integers(0, 50, size=b).astype(np.int32)
    caps = lens + rng.integers(0, B + 3, size=b)
    off = regions(rng, caps)
    C = int(off[-1])
    gen = torch.Generator().manual_seed(B)
    kb = torch.randn(b, 2 * B, Hkv, d, generator=gen).to(torch.bfloat16)
    vb = torch.randn(b, 2 * B, Hkv, d, generator=gen).to(torch.bfloat16)
    shape_c = (Hkv, C, d) if head_major else (C, Hkv, d)
    kc = torch.randn(*shape_c, generator=gen).to(torch.bfloat16)
    vc = torch.randn(*shape_c, generator=gen).to(torch.bfloat16)
    tau = np.stack([rng.permutation(B) + 1 for _ in range(b)]).astype(np.int32)
    L = rng.integers(0, B + 1, size=b).astype(np.int32)
    if b >= 3:
        tau[1, 0] = tau[1, -1] if B > 1 else 2  # not a permutation
        L[2] = B  # may overflow its region
    ek, ev, el, est = oracle.commit_kv(f64(kb), f64(vb), tau, L, f64(kc), f64(vc), off, lens, head_major)
    # this round's positions: scattered, unordered, distinct per sequence
    pos = np.stack([rng.choice(100000, size=B, replace=False) for _ in range(b)]).astype(np.int32)
    enext = oracle.next_positions(pos, tau, L)
    enext[est != 0] = pos[est != 0]  # a sequence that commits nothing keeps its block
    ext = torch.tensor(np.concatenate([off, lens]), dtype=torch.int32, device="cuda")
    status = torch.zeros(b, dtype=torch.int32, device="cuda")
    gk, gv = kc.cuda(), vc.cuda()
    gpos = torch.from_numpy(pos).cuda()
    gnext = torch.full_like(gpos, -7)
    binding.simsd_commit_kv(kb.cuda(), vb.cuda(), torch.from_numpy(tau).cuda(), torch.from_numpy(L).cuda(),
                            gk, gv, ext[:b + 1], ext[b + 1:], pos=gpos, next_pos=gnext,
                            flags=binding.SIMSD_KV_HEAD_MAJOR if head_major else 0, status=status)
    torch.cuda.synchronize()
    say(f"  L {L.tolist()} status {status.cpu().tolist()} lens {ext[b + 1:].cpu().tolist()}")
    assert np.array_equal(ext[b + 1:].cpu().numpy(), el)
    assert np.array_equal(status.cpu().numpy(), est)
    assert np.array_equal(f64(gk), ek) and np.array_equal(f64(gv), ev)
    assert np.array_equal(gnext.cpu().numpy(), enext)
    # in place: next_pos may be pos itself
    kc2, vc2 = kc.cuda(), vc.cuda()
    ext2 = torch.tensor(np.concatenate([off, lens]), dtype=torch.int32, device="cuda")
    binding.simsd_commit_kv(kb.cuda(), vb.cuda(), torch.from_numpy(tau).cuda(), torch.from_numpy(L).cuda(),
                            kc2, vc2, ext2[:b + 1], ext2[b + 1:], pos=gpos, next_pos=gpos,
                            flags=binding.SIMSD_KV_HEAD_MAJOR if head_major else 0)
    torch.cuda.synchronize()
    assert np.array_equal(gpos.cpu().numpy(), enext)


def grown_cache(x, caps, head_major, fill=NAN_BF16):
    """The packed prefix of x spread into regions of the given capacities; the
    unused rows hold `fill` (NaN proves they are never read)."""
    off = x["prefix_offsets"].numpy()
    lens = np.diff(off).astype(np.int32)
    roff = np.zeros(len(lens) + 1, np.int32)
    roff[1:] = np.cumsum(caps)
    Hkv, d = x["k_pre"].shape[1:]
    k = torch.full((int(roff[-1]), Hkv, d), fill, dtype=torch.bfloat16)
    v = torch.full((int(roff[-1]), Hkv, d), fill, dtype=torch.bfloat16)
    for s in range(len(lens)):
        k[roff[s]:roff[s] + lens[s]] = x["k_pre"][off[s]:off[s + 1]]
        v[roff[s]:roff[s] + lens[s]] = x["v_pre"][off[s]:off[s + 1]]
    if head_major:
        k, v = k.transpose(0, 1).contiguous(), v.transpose(0, 1).contiguous()
    return k, v, roff, lens


@pytest.mark.parametrize("head_major", [False, True])
def test_attention_over_regions_equals_packed(head_major):
    say(f"attention over grown regions, head_major={head_major}")
    w = synth.custom(b=4, Hq=16, Hkv=4, d=128, B=8, prefix=(0, 1500))
    x = synth.make_inputs(w, with_accept=False, seed=31)
    lens = np.diff(x["prefix_offsets"].numpy())
    caps = lens + np.array([0, 5, 200, 64])
    k, v, roff, lens = grown_cache(x, caps, head_major)
    ext = torch.tensor(np.concatenate([roff, lens]), dtype=torch.int32, device="cuda")
    fl = (binding.SIMSD_KV_HEAD_MAJOR if head_major else 0) | binding.SIMSD_OUT_F32
    kp, vp = x["k_pre"], x["v_pre"]
    if head_major:
        kp, vp = kp.transpose(0, 1).contiguous(), vp.transpose(0, 1).contiguous()
    g = {n: x[n].cuda() for n in ("q_blk", "k_blk", "v_blk", "tau", "prefix_offsets")}
    maxp = int(caps.max())
    lse0 = torch.empty(4, 16, 16, device="cuda")
    lse1 = torch.empty(4, 16, 16, device="cuda")
    ref = binding.simsd_verify_attention(g["q_blk"], g["k_blk"], g["v_blk"], kp.cuda(), vp.cuda(),
                                         g["prefix_offsets"], g["tau"], lse=lse0, max_prefix=maxp, flags=fl)
    out = binding.simsd_verify_attention(g["q_blk"], g["k_blk"], g["v_blk"], k.cuda(), v.cuda(), ext, g["tau"],
                                         lse=lse1, max_prefix=maxp, flags=fl | binding.SIMSD_PREFIX_LENS)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert torch.equal(out, ref) and torch.equal(lse1, lse0)
    # the explicit-mask entry point reads the same regions
    allowed = np.stack([oracle.mask_matrix(t) for t in x["tau"].numpy()])
    from gpu_util import pack_mask
    m = pack_mask(allowed).cuda()
    out_m = binding.simsd_verify_attention_mask(g["q_blk"], g["k_blk"], g["v_blk"], k.cuda(), v.cuda(), ext, m,
                                                max_prefix=maxp, flags=fl | binding.SIMSD_PREFIX_LENS)
    torch.cuda.synchronize()
    assert torch.equal(out_m, ref)


def test_lengths_past_the_region_are_flagged_and_clamped():
    say("prefix length past its region")
    w = synth.custom(b=3, Hq=8, Hkv=2, d=128, B=4, prefix=(100, 300))
    x = synth.make_inputs(w, with_accept=False, seed=32)
    lens = np.diff(x["prefix_offsets"].numpy())
    k, v, roff, lens = grown_cache(x, lens + 10, False, fill=0.0)
    g = {n: x[n].cuda() for n in ("q_blk", "k_blk", "v_blk", "tau")}
    bad = lens.copy()
    bad[1] = lens[1] + 11  # one row past its region
    bad[2] = -3
    ext = torch.tensor(np.concatenate([roff, bad]), dtype=torch.int32, device="cuda")
    status = torch.zeros(3, dtype=torch.int32, device="cuda")
    out = binding.simsd_verify_attention(g["q_blk"], g["k_blk"], g["v_blk"], k.cuda(), v.cuda(), ext, g["tau"],
                                         max_prefix=int(lens.max()) + 10, flags=binding.SIMSD_PREFIX_LENS,
                                         status=status)
    # sequence 1 computed over its full region, sequence 2 over an empty prefix
    full = lens.copy()
    full[1] += 10
    full[2] = 0
    ext2 = torch.tensor(np.concatenate([roff, full]), dtype=torch.int32, device="cuda")
    ref = binding.simsd_verify_attention(g["q_blk"], g["k_blk"], g["v_blk"], k.cuda(), v.cuda(), ext2, g["tau"],
                                         max_prefix=int(lens.max()) + 10, flags=binding.SIMSD_PREFIX_LENS)
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0, binding.SIMSD_DEV_BAD_PREFIX, binding.SIMSD_DEV_BAD_PREFIX]
    assert torch.equal(out, ref)


@pytest.mark.parametrize("head_major", [True, False])
def test_rounds_follow_the_oracle_chain(head_major):
    # Rounds of RoPE-copy (explicit positions) -> attention over the grown
    # cache -> acceptance -> commit, the positions of each round written by the
    # previous commit on the device. After a rejection the committed
    # correction token enters the next round as the data token of the first
    # pair (the rejected position) at temporal step 1, with draft probability
    # equal to the target's, so it is accepted and its key/value row committed.
    rounds, b, Hq, Hkv, d, B, V = 4, 8, 8, 2, 128, 8, 256
    say(f"{rounds} rounds, head_major={head_major}")
    w0 = synth.custom(b=b, Hq=Hq, Hkv=Hkv, d=d, B=B, V=V, prefix=(40, 400))
    x0 = synth.make_inputs(w0, with_accept=False, seed=40)
    lens0 = np.diff(x0["prefix_offsets"].numpy()).astype(np.int32)
    caps = lens0 + rounds * B
    k, v, roff, lens = grown_cache(x0, caps, head_major, fill=0.0)
    fl = binding.SIMSD_KV_HEAD_MAJOR if head_major else 0
    # device state: cache, one [2b+1] array (bounds, then lengths), positions
    gk, gv = k.cuda(), v.cuda()
    ext = torch.tensor(np.concatenate([roff, lens]), dtype=torch.int32, device="cuda")
    glens = ext[b + 1:]
    gpos = torch.from_numpy((lens0[:, None] + np.arange(B)[None, :]).astype(np.int32)).cuda()
    # oracle state (fp64 copies of the same bf16 values)
    ok_, ov_, olens = f64(k), f64(v), lens.copy()
    opos = gpos.cpu().numpy()
    cached = [[] for _ in range(b)]  # positions committed after the prompt
    maxp = int(caps.max())
    prev_L = prev_corr = None
    partial = 0  # rounds of a sequence with tau != identity and 0 < L < B
    for r in range(rounds):
        x = synth.make_inputs(w0, seed=41 + r)  # this round's block, drafts and probabilities
        tau, draft, q, p = x["tau"].clone(), x["draft"].clone(), x["q"].clone(), x["p"]
        if r > 0:
            for s in range(b):
                if prev_L[s] < B:
                    j = int((tau[s] == 1).nonzero()[0, 0])
                    tau[s, j], tau[s, 0] = tau[s, 0].clone(), 1
                    draft[s, 0] = int(prev_corr[s])
                    q[s, 0] = p[s, 0]
        qg, kg, vg, tg = x["q_blk"].cuda(), x["k_blk"].cuda(), x["v_blk"].cuda(), tau.cuda()
        binding.simsd_rope_copy(qg, kg, gpos, w0.rope_base, binding.SIMSD_ROPE_POSITIONS)
        out = binding.simsd_verify_attention(qg, kg, vg, gk, gv, ext, tg, max_prefix=maxp,
                                             flags=fl | binding.SIMSD_PREFIX_LENS | binding.SIMSD_OUT_F32)
        L, corr = binding.simsd_accept(p.cuda(), q.cuda(), draft.cuda(), tg, x["u"].cuda())
        status = torch.zeros(b, dtype=torch.int32, device="cuda")
        gnext = torch.empty_like(gpos)
        binding.simsd_commit_kv(kg, vg, tg, L, gk, gv, ext[:b + 1], glens, pos=gpos, next_pos=gnext,
                                flags=fl, status=status)
        torch.cuda.synchronize()

        tn = tau.numpy()
        q_r = bf16_round(oracle.rope_copy(f64(x["q_blk"]), opos, w0.rope_base))
        k_r = bf16_round(oracle.rope_copy(f64(x["k_blk"]), opos, w0.rope_base))
        kp, po = oracle.pack_regions(ok_, roff, olens, head_major)
        vp, _ = oracle.pack_regions(ov_, roff, olens, head_major)
        if head_major:
            kp, vp = kp.transpose(1, 0, 2), vp.transpose(1, 0, 2)
        ref, _ = oracle.verify_attention(q_r, k_r, f64(x["v_blk"]), kp, vp, po, tn, threads=ORACLE_THREADS)
        acc = oracle.accept(p.numpy(), q.numpy(), draft.numpy(), tn, x["u"].numpy())
        ok_, ov_, olens, ost = oracle.commit_kv(k_r, f64(x["v_blk"]), tn, acc["accept_len"], ok_, ov_, roff,
                                                olens, head_major)
        onext = oracle.next_positions(opos, tn, acc["accept_len"])
        done = oracle.committed_positions(opos, tn, acc["accept_len"])
        err = float(np.abs(f64(out) - ref).max())
        Lh, ch = L.cpu().numpy(), corr.cpu().numpy()
        say(f"  round {r}: attention max-abs {err:.3e}, accepted {Lh.tolist()}, lens {glens.cpu().tolist()}")
        assert err <= 4e-3
        assert np.array_equal(Lh, acc["accept_len"])
        assert not ((ch != acc["correction"]) & (acc["boundary"] == 0)).any()
        assert status.cpu().tolist() == [0] * b and ost.tolist() == [0] * b
        assert np.array_equal(glens.cpu().numpy(), olens)
        # values are copied bit for bit; keys carry the RoPE-copy result (within 1 bf16 ulp of the oracle's)
        assert np.array_equal(f64(gv), ov_)
        assert (np.abs(f64(gk) - ok_) <= bf16_ulp(ok_)).all()
        nx = gnext.cpu().numpy()
        assert np.array_equal(nx, onext)
        for s in range(b):
            if r > 0 and prev_L[s] < B:
                assert Lh[s] >= 1, "the committed correction token was not accepted"
            cached[s] += done[s]
            seen = cached[s] + nx[s].tolist()
            # committed plus next-round positions: each once, no gap after the prompt
            assert len(seen) == len(set(seen)) and sorted(seen) == list(range(lens0[s], max(seen) + 1)), s
            if 0 < Lh[s] < B and not (tn[s] == np.arange(1, B + 1)).all():
                partial += 1
        prev_L, prev_corr = Lh, ch
        gpos, opos = gnext, onext
    say(f"  rounds with tau != identity and 0 < L < B: {partial}")
    assert partial >= 4
