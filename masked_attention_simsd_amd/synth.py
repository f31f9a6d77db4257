"""Seeded synthetic inputs for the SimSD verification path.

This module draws inputs only; it holds none of the method's arithmetic. The
same CPU tensors feed the HIP path (after a device copy) and the CPU oracle.

The pages report results on trained SDAR models over GSM8K, MBPP, TriviaQA
and MMLU; none of those models or datasets is used. Random tensors with the
shapes below stand in for them.

Workloads (one attention layer of the verification forward, plus acceptance):
  tiny   : 1 sequence, 1/1 heads, d 64, prefix 32, B 4, vocab 256; target
           logits N(0,1), draft logits = target + N(0,0.5)
  b4     : 1 sequence, 32/8 heads, d 128, prefix 1024, B 4, vocab 32768;
           target logits N(0,2), draft = target + N(0,0.5)
  b8     : 16 sequences, 32/8 heads, d 128, prefix 4096, B 8, vocab 32768,
           logits as b4 (the headline workload)
  b16    : 8 sequences, 32/8 heads, d 128, prefix 16384, B 16, vocab 151936;
           target logits N(0,3), draft = target + N(0,1)
  ragged : 64 sequences, prefix lengths uniform in [512, 8192], B 8, 32/8 heads,
           d 128, vocab 32768, logits as b4; sequences s % 8 == 0 use the
           identity step map, s % 8 == 1 the reversed one, the rest random.
N(0, s) means standard deviation s. Q/K/V of every workload are drawn fp32
N(0,1) and rounded to bf16 (the oracle runs on the rounded values).
p = softmax(target) and q = softmax(draft) are computed in fp64 and stored as
fp32; draft tokens are drawn from q; uniforms are fp32 in [0, 1).
The prefix K/V are treated as already rotated (they come from the cache).

Draw order (fixed): prefix lengths, K_pre, V_pre, Q_blk, K_blk, V_blk, tau,
then per sequence its target logits and draft noise, then draft tokens, then
uniforms. Seed = 1000 + index of the workload in CONFIG_ORDER.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

CONFIG_ORDER = ("tiny", "b4", "b8", "b16", "ragged")


@dataclass(frozen=True)
class Workload:
    name: str
    b: int
    Hq: int
    Hkv: int
    d: int
    B: int
    V: int
    prefix: tuple  # (lo, hi) inclusive; lo == hi for fixed length
    logit_std: float
    noise_std: float
    tau_mode: str = "random"  # random | mixed
    rope_base: float = 10000.0

    @property
    def seed(self) -> int:
        return 1000 + CONFIG_ORDER.index(self.name)

    def describe(self) -> str:
        pre = (f"prefix {self.prefix[0]}" if self.prefix[0] == self.prefix[1]
               else f"prefix U[{self.prefix[0]},{self.prefix[1]}]")
        return (f"batch {self.b}, {self.Hq}/{self.Hkv} heads, head_dim {self.d}, {pre}, "
                f"B={self.B} ({2 * self.B} block rows), bf16 Q/K/V, vocab {self.V}")


CONFIGS = {
    "tiny": Workload("tiny", 1, 1, 1, 64, 4, 256, (32, 32), 1.0, 0.5),
    "b4": Workload("b4", 1, 32, 8, 128, 4, 32768, (1024, 1024), 2.0, 0.5),
    "b8": Workload("b8", 16, 32, 8, 128, 8, 32768, (4096, 4096), 2.0, 0.5),
    "b16": Workload("b16", 8, 32, 8, 128, 16, 151936, (16384, 16384), 3.0, 1.0),
    "ragged": Workload("ragged", 64, 32, 8, 128, 8, 32768, (512, 8192), 2.0, 0.5,
                       tau_mode="mixed"),
}


def custom(name="custom", **kw) -> Workload:
    """A workload of arbitrary shape (used by tests for ragged tails and edge
    cases). make_inputs seeds it with 1000 + len(CONFIG_ORDER) unless given a
    seed."""
    base = dict(b=1, Hq=1, Hkv=1, d=64, B=4, V=256, prefix=(32, 32), logit_std=1.0, noise_std=0.5)
    base.update(kw)
    return Workload(name, **base)


def _randn_bf16(shape, g):
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    return x.to(torch.bfloat16)


def make_inputs(w: Workload | str, seed: int | None = None, with_accept: bool = True,
                with_attn: bool = True) -> dict:
    """Draw one batch of inputs on the CPU. Returns a dict of tensors:

    prefix_lens [b] int64, prefix_offsets [b+1] int32, start_pos [b] int32,
    k_pre / v_pre [sum P][Hkv][d] bf16, q_blk [b][2B][Hq][d] bf16,
    k_blk / v_blk [b][2B][Hkv][d] bf16, tau [b][B] int32 (labels 1..B),
    p / q [b][B][V] fp32 (softmax of target_logits / draft_logits [b][B][V]
    fp32), draft [b][B] int32, u [b][B+1] fp32.
    """
    if isinstance(w, str):
        w = CONFIGS[w]
    if seed is None:
        seed = w.seed if w.name in CONFIG_ORDER else 1000 + len(CONFIG_ORDER)
    g = torch.Generator().manual_seed(seed)
    b, B, Hq, Hkv, d = w.b, w.B, w.Hq, w.Hkv, w.d
    lo, hi = w.prefix
    if lo == hi:
        lens = torch.full((b,), lo, dtype=torch.int64)
    else:
        lens = torch.randint(lo, hi + 1, (b,), generator=g, dtype=torch.int64)
    offsets = torch.zeros(b + 1, dtype=torch.int32)
    offsets[1:] = torch.cumsum(lens, 0).to(torch.int32)
    total = int(offsets[-1])
    out = dict(workload=w, seed=seed, prefix_lens=lens, prefix_offsets=offsets,
               start_pos=lens.to(torch.int32))
    if with_attn:
        out["k_pre"] = _randn_bf16((total, Hkv, d), g)
        out["v_pre"] = _randn_bf16((total, Hkv, d), g)
        out["q_blk"] = _randn_bf16((b, 2 * B, Hq, d), g)
        out["k_blk"] = _randn_bf16((b, 2 * B, Hkv, d), g)
        out["v_blk"] = _randn_bf16((b, 2 * B, Hkv, d), g)
    tau = torch.stack([torch.randperm(B, generator=g) for _ in range(b)]).to(torch.int32) + 1
    if w.tau_mode == "mixed":
        for s in range(b):
            if s % 8 == 0:
                tau[s] = torch.arange(1, B + 1, dtype=torch.int32)
            elif s % 8 == 1:
                tau[s] = torch.arange(B, 0, -1, dtype=torch.int32)
    out["tau"] = tau.contiguous()
    if with_accept:
        V = w.V
        p = torch.empty((b, B, V), dtype=torch.float32)
        q = torch.empty((b, B, V), dtype=torch.float32)
        zt = torch.empty((b, B, V), dtype=torch.float32)
        zd = torch.empty((b, B, V), dtype=torch.float32)
        for s in range(b):  # per sequence to bound fp64 temporaries
            tgt = torch.randn((B, V), generator=g, dtype=torch.float64) * w.logit_std
            drf = tgt + torch.randn((B, V), generator=g, dtype=torch.float64) * w.noise_std
            # the logits are stored in fp32; the probabilities are their fp64
            # softmax rounded to fp32
            zt[s] = tgt.to(torch.float32)
            zd[s] = drf.to(torch.float32)
            p[s] = torch.softmax(zt[s].to(torch.float64), dim=-1).to(torch.float32)
            q[s] = torch.softmax(zd[s].to(torch.float64), dim=-1).to(torch.float32)
        draft = torch.multinomial(q.reshape(b * B, V).to(torch.float64), 1, generator=g)
        out["p"], out["q"] = p, q
        out["target_logits"], out["draft_logits"] = zt, zd
        out["draft"] = draft.reshape(b, B).to(torch.int32).contiguous()
        out["u"] = torch.rand((b, B + 1), generator=g, dtype=torch.float32)
    return out
