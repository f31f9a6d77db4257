"""Helpers shared by the GPU parity tests (no test functions here)."""
from __future__ import annotations

import functools
import os
import sys

import numpy as np
import torch

from masked_attention_simsd_amd import synth

ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def say(*args):
    """Print and flush (names the case before a GPU step)."""
    print(*args, flush=True)
    sys.stdout.flush()


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Exact round-to-nearest-even of fp64 values to bf16 (normal range)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    _, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(1.0, e - 8)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


@functools.lru_cache(maxsize=4)
def inputs(name: str):
    return synth.make_inputs(name)


def to_dev(x: dict, dev="cuda:0") -> dict:
    return {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in x.items()}


def subset_sequences(x: dict, seqs) -> dict:
    """Inputs of the chosen sequences only (for oracle runs on a sample)."""
    off = x["prefix_offsets"].tolist()
    kp = torch.cat([x["k_pre"][off[s]:off[s + 1]] for s in seqs])
    vp = torch.cat([x["v_pre"][off[s]:off[s + 1]] for s in seqs])
    lens = torch.tensor([off[s + 1] - off[s] for s in seqs], dtype=torch.int64)
    noff = torch.zeros(len(seqs) + 1, dtype=torch.int32)
    noff[1:] = torch.cumsum(lens, 0).to(torch.int32)
    idx = torch.tensor(list(seqs))
    return dict(k_pre=kp, v_pre=vp, prefix_offsets=noff, q_blk=x["q_blk"][idx],
                k_blk=x["k_blk"][idx], v_blk=x["v_blk"][idx], tau=x["tau"][idx])


def pack_mask(allowed) -> torch.Tensor:
    """bool [b][R][R] -> int64 [b][R][ceil(R/64)] bit words (bit c % 64 of
    word c // 64 of row r set when row r sees block key c)."""
    a = np.asarray(allowed, dtype=bool)
    b, R, _ = a.shape
    W = (R + 63) // 64
    words = np.zeros((b, R, W), dtype=np.uint64)
    for c in range(R):
        words[:, :, c // 64] |= a[:, :, c].astype(np.uint64) << np.uint64(c % 64)
    return torch.from_numpy(words.view(np.int64))
