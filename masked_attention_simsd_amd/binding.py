"""ctypes binding of libsimsd (the C ABI in include/simsd.h).

Argument marshalling only: each function checks tensor devices, dtypes and
shapes, passes raw device pointers and the current HIP stream, and raises
SimsdError on a nonzero return code. All computation happens in the HIP
kernels of libsimsd.so; there is no fallback path. If the library has not
been built the first call raises (build it with
``python -m masked_attention_simsd_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsimsd.so")

# flag and status values, as in include/simsd.h
SIMSD_ROPE_HALF, SIMSD_ROPE_INTERLEAVED, SIMSD_ROPE_NO_COPY, SIMSD_ROPE_POSITIONS = 0, 1, 2, 4
SIMSD_DATA_CAUSAL, SIMSD_DATA_BIDIR, SIMSD_DATA_SKIP, SIMSD_OUT_F32 = 0, 1, 2, 4
SIMSD_KV_HEAD_MAJOR, SIMSD_PREFIX_LENS, SIMSD_KV_PAIRED = 8, 16, 32
SIMSD_DEV_BAD_TAU, SIMSD_DEV_ZERO_RESIDUAL, SIMSD_DEV_Q_ZERO = 1, 2, 4
SIMSD_DEV_BAD_TOKEN, SIMSD_DEV_BAD_PREFIX, SIMSD_DEV_SYNC_TIMEOUT = 8, 16, 32
SIMSD_DEV_COMMIT_OVERFLOW = 64
# simsd_set_tuning keys
TUNE_KEYS = {"attn_pipe": 0, "attn_target_wg": 1, "attn_chunk_max": 2, "attn_xcd_remap": 3,
             "attn_rotate": 4, "attn_lpt": 5, "attn_shift": 6, "accept_per": 7, "rowstat_per": 8}

EXPORTS = (
    "simsd_rope_copy", "simsd_verify_attention", "simsd_verify_attention_rope",
    "simsd_verify_attention_workspace", "simsd_verify_attention_mask",
    "simsd_verify_attention_mask_workspace",
    "simsd_accept", "simsd_accept_workspace", "simsd_accept_logits", "simsd_accept_logits_workspace",
    "simsd_commit_kv", "simsd_status_string", "simsd_last_hip_error", "simsd_set_tuning",
    "simsd_verify_attention_noalloc",
)
SIMSD_ERR_SCRATCH = 11
NOALLOC_SCRATCH_BYTES = 32 << 20


class SimsdError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} returned {code}: {msg}")
        self.code = code


_lib = None
_lock = threading.Lock()


def load_library(path: str = LIB_PATH):
    """Load libsimsd.so (in-tree). Raises if it is missing: there is no fallback."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m masked_attention_simsd_amd.build`")
        lib = ctypes.CDLL(path)
        P, I, U, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32, ctypes.c_float, ctypes.c_size_t
        lib.simsd_rope_copy.argtypes = [P, P, P, I, I, I, I, I, F, U, P]
        lib.simsd_rope_copy.restype = I
        lib.simsd_verify_attention.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, U, P, P, Z, P]
        lib.simsd_verify_attention.restype = I
        lib.simsd_verify_attention_rope.argtypes = [P, P, P, P, P, P, P, P, F, U, P, P, P, I, I, I, I, I, I,
                                                    F, U, P, P, Z, P]
        lib.simsd_verify_attention_rope.restype = I
        lib.simsd_verify_attention_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, U, P, P]
        lib.simsd_verify_attention_noalloc.restype = I
        lib.simsd_verify_attention_workspace.argtypes = [I, I, I, I, I, I]
        lib.simsd_verify_attention_workspace.restype = Z
        lib.simsd_verify_attention_mask.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, U, P, P, Z, P]
        lib.simsd_verify_attention_mask.restype = I
        lib.simsd_verify_attention_mask_workspace.argtypes = [I, I, I, I, I, I]
        lib.simsd_verify_attention_mask_workspace.restype = Z
        lib.simsd_accept.argtypes = [P, P, P, P, P, I, I, I, P, P, P, P, Z, P]
        lib.simsd_accept.restype = I
        lib.simsd_accept_workspace.argtypes = [I, I, I]
        lib.simsd_accept_workspace.restype = Z
        lib.simsd_accept_logits.argtypes = [P, P, F, P, P, P, I, I, I, P, P, P, P, Z, P]
        lib.simsd_accept_logits.restype = I
        lib.simsd_commit_kv.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, U, P, P]
        lib.simsd_commit_kv.restype = I
        lib.simsd_accept_logits_workspace.argtypes = [I, I, I]
        lib.simsd_accept_logits_workspace.restype = Z
        lib.simsd_status_string.argtypes = [I]
        lib.simsd_status_string.restype = ctypes.c_char_p
        lib.simsd_last_hip_error.argtypes = []
        lib.simsd_last_hip_error.restype = I
        lib.simsd_set_tuning.argtypes = [I, I]
        lib.simsd_set_tuning.restype = I
        _lib = lib
        return lib


def _check(fn: str, rc: int):
    if rc != 0:
        lib = load_library()
        msg = lib.simsd_status_string(rc).decode()
        if rc == 8:
            msg += f" (hipError {lib.simsd_last_hip_error()})"
        raise SimsdError(fn, rc, msg)


def simsd_set_tuning(key, value: int):
    """Override one kernel-plan choice process-wide (key: a name of TUNE_KEYS
    or its number; value -1 restores the default)."""
    k = TUNE_KEYS[key] if isinstance(key, str) else int(key)
    _check("simsd_set_tuning", load_library().simsd_set_tuning(k, int(value)))


class tuning:
    """Context manager: tuning overrides for the calls made inside it, e.g.
    ``with binding.tuning(attn_pipe=7): ...``; restores the defaults after."""

    def __init__(self, **kw):
        self.kw = kw

    def __enter__(self):
        for k, v in self.kw.items():
            simsd_set_tuning(k, v)
        return self

    def __exit__(self, *exc):
        for k in self.kw:
            simsd_set_tuning(k, -1)
        return False


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def kv_pair_views(kv):
    """The key and value halves of a paired cache buffer (SIMSD_KV_PAIRED):
    kv is [rows][Hkv][2][d] (token-major) or [Hkv][rows][2][d] (head-major),
    contiguous; returns the two [..][..][d] views to pass as k / v."""
    _need(kv, "kv", torch.bfloat16, 4)
    if kv.shape[2] != 2:
        raise ValueError("a paired cache buffer has shape [..][..][2][d]")
    return kv[:, :, 0, :], kv[:, :, 1, :]


def _need_kv(k, v, names, flags):
    """Prefix or cache tensors: contiguous 3-D bf16 tensors, or with
    SIMSD_KV_PAIRED the two halves of one contiguous [..][..][2][d] buffer
    (see kv_pair_views)."""
    if not flags & SIMSD_KV_PAIRED:
        _need(k, names[0], torch.bfloat16, 3)
        _need(v, names[1], torch.bfloat16, 3)
        return
    for t, n in ((k, names[0]), (v, names[1])):
        if not torch.is_tensor(t) or t.dtype != torch.bfloat16 or not t.is_cuda or t.dim() != 3:
            raise ValueError(f"{n} must be a 3-dim bf16 device tensor")
    d = k.shape[2]
    want = (k.shape[1] * 2 * d, 2 * d, 1)
    if (tuple(k.stride()) != want or tuple(v.stride()) != want or v.shape != k.shape
            or v.data_ptr() != k.data_ptr() + 2 * d):
        raise ValueError(f"with SIMSD_KV_PAIRED, {names[0]} / {names[1]} must be the halves of one "
                         "contiguous [..][..][2][d] buffer (kv_pair_views)")


def _need(t, name, dtype, dims=None, device=True):
    if not torch.is_tensor(t):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, got shape {tuple(t.shape)}")


def _offsets_len(b: int, flags: int) -> int:
    """prefix_offsets holds b+1 bounds, followed by b used lengths with SIMSD_PREFIX_LENS."""
    return 2 * b + 1 if flags & SIMSD_PREFIX_LENS else b + 1


def _max_prefix(prefix_offsets, b: int) -> int:
    """The largest region (a bound on every prefix length; a device-to-host copy)."""
    off = prefix_offsets[:b + 1].cpu()
    return int((off[1:] - off[:-1]).max()) if b > 0 else 0


def _need_positions(start_pos, b, B, flags):
    """start_pos: int32 [b], or [b][B] (one position per pair) with SIMSD_ROPE_POSITIONS."""
    if flags & SIMSD_ROPE_POSITIONS:
        _need(start_pos, "start_pos", torch.int32, 2)
        if tuple(start_pos.shape) != (b, B):
            raise ValueError("with SIMSD_ROPE_POSITIONS start_pos must be [b][B]")
    else:
        _need(start_pos, "start_pos", torch.int32, 1)
        if start_pos.shape[0] != b:
            raise ValueError("start_pos must have b entries")


def simsd_rope_copy(q_blk, k_blk, start_pos, rope_base: float = 10000.0, flags: int = 0,
                    stream=None):
    """In-place RoPE with the copy rule. q_blk [b][2B][Hq][d], k_blk [b][2B][Hkv][d] bf16,
    start_pos int32 [b] (pair k at start_pos[s] + k), or [b][B] positions with
    SIMSD_ROPE_POSITIONS."""
    _need(q_blk, "q_blk", torch.bfloat16, 4)
    _need(k_blk, "k_blk", torch.bfloat16, 4)
    b, twoB, Hq, d = q_blk.shape
    if twoB % 2 or k_blk.shape[0] != b or k_blk.shape[1] != twoB or k_blk.shape[3] != d:
        raise ValueError("q_blk / k_blk shapes disagree")
    _need_positions(start_pos, b, twoB // 2, flags)
    rc = load_library().simsd_rope_copy(_ptr(q_blk), _ptr(k_blk), _ptr(start_pos), b, twoB // 2,
                                        Hq, k_blk.shape[2], d, float(rope_base), flags,
                                        _stream(stream))
    _check("simsd_rope_copy", rc)


def simsd_verify_attention_workspace(b: int, B: int, Hq: int, Hkv: int, d: int,
                                     max_prefix: int) -> int:
    return int(load_library().simsd_verify_attention_workspace(b, B, Hq, Hkv, d, max_prefix))


_ws_cache: dict = {}


def _cached_workspace(kind: str, device, nbytes: int):
    key = (kind, torch.device(device))
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=key[1])
        _ws_cache[key] = ws
    return ws


def attention_workspace(device, nbytes: int):
    """A zero-initialised workspace of at least nbytes on `device` for
    simsd_verify_attention, reused across calls (every call leaves its counter
    words zero). Calls sharing it must not overlap, so use it from one stream."""
    return _cached_workspace("attention", device, nbytes)


def accept_workspace(device, nbytes: int):
    """As attention_workspace, for simsd_accept (the whole buffer starts zero;
    every call leaves it zero)."""
    return _cached_workspace("accept", device, nbytes)


def simsd_accept_workspace(b: int, B: int, V: int) -> int:
    return int(load_library().simsd_accept_workspace(b, B, V))


def simsd_verify_attention(q_blk, k_blk, v_blk, k_pre, v_pre, prefix_offsets, tau, out=None,
                           lse=None, max_prefix: int | None = None, scale: float = 0.0,
                           flags: int = 0, status=None, workspace=None, stream=None):
    """Verify attention. Returns out ([b][2B][Hq][d], bf16 or fp32 with SIMSD_OUT_F32).

    k_pre / v_pre are [sum P][Hkv][d], or [Hkv][sum P][d] with SIMSD_KV_HEAD_MAJOR;
    with SIMSD_KV_PAIRED the two halves of one [..][..][2][d] buffer (kv_pair_views).

    max_prefix: host int >= every prefix length; if None it is read back from
    prefix_offsets (a device-to-host copy, so not for timed loops).
    """
    return _attention("simsd_verify_attention", q_blk, k_blk, v_blk, k_pre, v_pre, prefix_offsets,
                      tau, out, lse, max_prefix, scale, flags, status, workspace, stream, None)


def simsd_verify_attention_noalloc(q_blk, k_blk, v_blk, k_pre, v_pre, prefix_offsets, tau, out, lse=None,
                                   max_prefix: int | None = None, scale: float = 0.0, flags: int = 0,
                                   status=None, stream=None):
    """simsd_verify_attention without a workspace argument: the library uses
    its fixed per-GPU scratch buffer and allocates nothing (so `out` must be
    given). Calls on one GPU must not overlap."""
    return _attention("simsd_verify_attention_noalloc", q_blk, k_blk, v_blk, k_pre, v_pre, prefix_offsets,
                      tau, out, lse, max_prefix, scale, flags, status, None, stream, "noalloc")


def simsd_verify_attention_rope(q_blk, k_blk, v_blk, k_pre, v_pre, prefix_offsets, tau, start_pos,
                                rope_base: float = 10000.0, rope_flags: int = 0, k_rot=None, out=None,
                                lse=None, max_prefix: int | None = None, scale: float = 0.0,
                                flags: int = 0, status=None, workspace=None, stream=None):
    """RoPE-copy fused into verify attention: q_blk / k_blk are the block rows
    BEFORE RoPE and are not modified; k_rot (optional, [b][2B][Hkv][d] bf16,
    not overlapping k_blk) receives the rotated block keys. Returns out."""
    _need_positions(start_pos, q_blk.shape[0], q_blk.shape[1] // 2, rope_flags)
    if k_rot is not None:
        _need(k_rot, "k_rot", torch.bfloat16, 4)
        if tuple(k_rot.shape) != tuple(k_blk.shape):
            raise ValueError("k_rot shape must equal k_blk shape")
    return _attention("simsd_verify_attention_rope", q_blk, k_blk, v_blk, k_pre, v_pre, prefix_offsets,
                      tau, out, lse, max_prefix, scale, flags, status, workspace, stream,
                      (start_pos, float(rope_base), int(rope_flags), k_rot))


def _attention(fn, q_blk, k_blk, v_blk, k_pre, v_pre, prefix_offsets, tau, out, lse, max_prefix,
               scale, flags, status, workspace, stream, rope):
    for t, n in ((q_blk, "q_blk"), (k_blk, "k_blk"), (v_blk, "v_blk")):
        _need(t, n, torch.bfloat16, 4)
    _need_kv(k_pre, v_pre, ("k_pre", "v_pre"), flags)
    _need(prefix_offsets, "prefix_offsets", torch.int32, 1)
    _need(tau, "tau", torch.int32, 2)
    b, twoB, Hq, d = q_blk.shape
    B = twoB // 2
    Hkv = k_blk.shape[2]
    head_major = bool(flags & SIMSD_KV_HEAD_MAJOR)
    pre_ok = (k_pre.shape[0] == Hkv and k_pre.shape[2] == d) if head_major else k_pre.shape[1:] == (Hkv, d)
    if (twoB % 2 or tuple(k_blk.shape) != (b, twoB, Hkv, d) or tuple(v_blk.shape) != (b, twoB, Hkv, d)
            or not pre_ok or v_pre.shape != k_pre.shape
            or prefix_offsets.shape[0] != _offsets_len(b, flags) or tuple(tau.shape) != (b, B)):
        raise ValueError("inconsistent shapes")
    if max_prefix is None:
        max_prefix = _max_prefix(prefix_offsets, b)
    out_f32 = bool(flags & SIMSD_OUT_F32)
    if out is None and rope != "noalloc":
        out = torch.empty_like(q_blk, dtype=torch.float32 if out_f32 else torch.bfloat16)
    if out is None:
        raise ValueError("simsd_verify_attention_noalloc needs an output tensor (it allocates nothing)")
    _need(out, "out", torch.float32 if out_f32 else torch.bfloat16, 4)
    if tuple(out.shape) != tuple(q_blk.shape):
        raise ValueError("out shape must equal q_blk shape")
    if lse is not None:
        _need(lse, "lse", torch.float32, 3)
    if status is not None:
        _need(status, "status", torch.int32, 1)
    if rope == "noalloc":
        if out is None:
            raise ValueError("simsd_verify_attention_noalloc needs an output tensor (it allocates nothing)")
    else:
        need = simsd_verify_attention_workspace(b, B, Hq, Hkv, d, max_prefix)
        if workspace is None:
            workspace = attention_workspace(q_blk.device, need)
    head = (_ptr(q_blk), _ptr(k_blk), _ptr(v_blk), _ptr(k_pre) if k_pre.numel() else None,
            _ptr(v_pre) if v_pre.numel() else None, _ptr(prefix_offsets), _ptr(tau))
    lib = load_library()
    if rope == "noalloc":
        rc = lib.simsd_verify_attention_noalloc(*head, _ptr(out), _ptr(lse), b, B, Hq, Hkv, d, int(max_prefix),
                                                float(scale), flags, _ptr(status), _stream(stream))
        _check(fn, rc)
        return out
    tail = (_ptr(out), _ptr(lse), b, B, Hq, Hkv, d, int(max_prefix), float(scale), flags, _ptr(status),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if rope is None:
        rc = lib.simsd_verify_attention(*head, *tail)
    else:
        start_pos, base, rflags, k_rot = rope
        rc = lib.simsd_verify_attention_rope(*head, _ptr(start_pos), base, rflags, _ptr(k_rot), *tail)
    _check(fn, rc)
    return out


def simsd_verify_attention_mask_workspace(b: int, R: int, Hq: int, Hkv: int, d: int, max_prefix: int) -> int:
    return int(load_library().simsd_verify_attention_mask_workspace(b, R, Hq, Hkv, d, max_prefix))


def simsd_verify_attention_mask(q_blk, k_blk, v_blk, k_pre, v_pre, prefix_offsets, block_mask, out=None,
                                lse=None, max_prefix: int | None = None, scale: float = 0.0, flags: int = 0,
                                status=None, workspace=None, stream=None):
    """Attention of R block rows under an explicit block mask: block_mask is an
    int64 tensor [b][R][ceil(R/64)] holding the uint64 bit words (bit c % 64 of
    word c // 64 of row r: row r sees block key c). Returns out."""
    for t, n in ((q_blk, "q_blk"), (k_blk, "k_blk"), (v_blk, "v_blk")):
        _need(t, n, torch.bfloat16, 4)
    _need_kv(k_pre, v_pre, ("k_pre", "v_pre"), flags)
    _need(prefix_offsets, "prefix_offsets", torch.int32, 1)
    _need(block_mask, "block_mask", torch.int64, 3)
    b, R, Hq, d = q_blk.shape
    Hkv = k_blk.shape[2]
    head_major = bool(flags & SIMSD_KV_HEAD_MAJOR)
    pre_ok = (k_pre.shape[0] == Hkv and k_pre.shape[2] == d) if head_major else k_pre.shape[1:] == (Hkv, d)
    if (tuple(k_blk.shape) != (b, R, Hkv, d) or tuple(v_blk.shape) != (b, R, Hkv, d) or not pre_ok
            or v_pre.shape != k_pre.shape or prefix_offsets.shape[0] != _offsets_len(b, flags)
            or tuple(block_mask.shape) != (b, R, (R + 63) // 64)):
        raise ValueError("inconsistent shapes")
    if max_prefix is None:
        max_prefix = _max_prefix(prefix_offsets, b)
    out_f32 = bool(flags & SIMSD_OUT_F32)
    if out is None:
        out = torch.empty_like(q_blk, dtype=torch.float32 if out_f32 else torch.bfloat16)
    _need(out, "out", torch.float32 if out_f32 else torch.bfloat16, 4)
    if lse is not None:
        _need(lse, "lse", torch.float32, 3)
    if status is not None:
        _need(status, "status", torch.int32, 1)
    need = simsd_verify_attention_mask_workspace(b, R, Hq, Hkv, d, max_prefix)
    if workspace is None:
        workspace = attention_workspace(q_blk.device, need)
    rc = load_library().simsd_verify_attention_mask(
        _ptr(q_blk), _ptr(k_blk), _ptr(v_blk), _ptr(k_pre) if k_pre.numel() else None,
        _ptr(v_pre) if v_pre.numel() else None, _ptr(prefix_offsets), _ptr(block_mask), _ptr(out), _ptr(lse),
        b, R, Hq, Hkv, d, int(max_prefix), float(scale), flags, _ptr(status), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check("simsd_verify_attention_mask", rc)
    return out


def simsd_accept(p, q, draft_tokens, tau, uniforms, accept_len=None, correction_token=None,
                 status=None, workspace=None, stream=None):
    """Rejection-sampling acceptance. Returns (accept_len, correction_token), int32 [b]."""
    _need(p, "p", torch.float32, 3)
    _need(q, "q", torch.float32, 3)
    _need(draft_tokens, "draft_tokens", torch.int32, 2)
    _need(tau, "tau", torch.int32, 2)
    _need(uniforms, "uniforms", torch.float32, 2)
    b, B, V = p.shape
    if (tuple(q.shape) != (b, B, V) or tuple(draft_tokens.shape) != (b, B)
            or tuple(tau.shape) != (b, B) or tuple(uniforms.shape) != (b, B + 1)):
        raise ValueError("inconsistent shapes")
    if accept_len is None:
        accept_len = torch.empty(b, dtype=torch.int32, device=p.device)
    if correction_token is None:
        correction_token = torch.empty(b, dtype=torch.int32, device=p.device)
    _need(accept_len, "accept_len", torch.int32, 1)
    _need(correction_token, "correction_token", torch.int32, 1)
    if status is not None:
        _need(status, "status", torch.int32, 1)
    need = simsd_accept_workspace(b, B, V)
    if workspace is None:
        workspace = accept_workspace(p.device, need)
    rc = load_library().simsd_accept(_ptr(p), _ptr(q), _ptr(draft_tokens), _ptr(tau),
                                     _ptr(uniforms), b, B, V, _ptr(accept_len),
                                     _ptr(correction_token), _ptr(status), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(),
                                     _stream(stream))
    _check("simsd_accept", rc)
    return accept_len, correction_token


def simsd_accept_logits_workspace(b: int, B: int, V: int) -> int:
    return int(load_library().simsd_accept_logits_workspace(b, B, V))


def simsd_accept_logits(target_logits, draft_logits, draft_tokens, tau, uniforms, temperature: float = 1.0,
                        accept_len=None, correction_token=None, status=None, workspace=None, stream=None):
    """Acceptance from fp32 logits [b][B][V] (softmax at `temperature`).
    Returns (accept_len, correction_token), int32 [b]."""
    _need(target_logits, "target_logits", torch.float32, 3)
    _need(draft_logits, "draft_logits", torch.float32, 3)
    _need(draft_tokens, "draft_tokens", torch.int32, 2)
    _need(tau, "tau", torch.int32, 2)
    _need(uniforms, "uniforms", torch.float32, 2)
    b, B, V = target_logits.shape
    if (tuple(draft_logits.shape) != (b, B, V) or tuple(draft_tokens.shape) != (b, B)
            or tuple(tau.shape) != (b, B) or tuple(uniforms.shape) != (b, B + 1)):
        raise ValueError("inconsistent shapes")
    if accept_len is None:
        accept_len = torch.empty(b, dtype=torch.int32, device=target_logits.device)
    if correction_token is None:
        correction_token = torch.empty(b, dtype=torch.int32, device=target_logits.device)
    if status is not None:
        _need(status, "status", torch.int32, 1)
    need = simsd_accept_logits_workspace(b, B, V)
    if workspace is None:
        workspace = _cached_workspace("accept_logits", target_logits.device, need)
    rc = load_library().simsd_accept_logits(_ptr(target_logits), _ptr(draft_logits), float(temperature),
                                            _ptr(draft_tokens), _ptr(tau), _ptr(uniforms), b, B, V,
                                            _ptr(accept_len), _ptr(correction_token), _ptr(status),
                                            _ptr(workspace), workspace.numel() * workspace.element_size(),
                                            _stream(stream))
    _check("simsd_accept_logits", rc)
    return accept_len, correction_token


def cache_offsets_with_lens(offsets, lens):
    """One int32 device array [2b+1]: region bounds then used lengths. Pass it
    as prefix_offsets with SIMSD_PREFIX_LENS; its tail view ([b+1:]) is the
    cache_lens of simsd_commit_kv (and, before the first round, the start
    position of each sequence's first block)."""
    return torch.cat([offsets.to(torch.int32), lens.to(torch.int32)]).contiguous()


def simsd_commit_kv(k_blk, v_blk, tau, accept_len, k_cache, v_cache, cache_offsets, cache_lens,
                    pos=None, next_pos=None, flags: int = 0, status=None, stream=None):
    """Append each sequence's accepted drafts (tau(k) <= accept_len[s]) to its
    cache region, in temporal order, and advance cache_lens in place; with
    next_pos, also write the positions the next round verifies.

    k_blk / v_blk [b][2B][Hkv][d] bf16; k_cache / v_cache [C][Hkv][d] (or
    [Hkv][C][d] with SIMSD_KV_HEAD_MAJOR) bf16; cache_offsets int32 [b+1];
    cache_lens int32 [b] (may be a view into the array built by
    cache_offsets_with_lens); pos / next_pos int32 [b][B] (this round's
    positions and the next round's; next_pos may be pos)."""
    for t, n in ((k_blk, "k_blk"), (v_blk, "v_blk")):
        _need(t, n, torch.bfloat16, 4)
    _need_kv(k_cache, v_cache, ("k_cache", "v_cache"), flags)
    _need(tau, "tau", torch.int32, 2)
    _need(accept_len, "accept_len", torch.int32, 1)
    _need(cache_offsets, "cache_offsets", torch.int32, 1)
    _need(cache_lens, "cache_lens", torch.int32, 1)
    b, twoB, Hkv, d = k_blk.shape
    B = twoB // 2
    head_major = bool(flags & SIMSD_KV_HEAD_MAJOR)
    cache_ok = (k_cache.shape[0] == Hkv and k_cache.shape[2] == d) if head_major else k_cache.shape[1:] == (Hkv, d)
    if (twoB % 2 or tuple(v_blk.shape) != tuple(k_blk.shape) or not cache_ok or v_cache.shape != k_cache.shape
            or tuple(tau.shape) != (b, B) or accept_len.shape[0] != b or cache_offsets.shape[0] < b + 1
            or cache_lens.shape[0] != b):
        raise ValueError("inconsistent shapes")
    if status is not None:
        _need(status, "status", torch.int32, 1)
    for t, n in ((pos, "pos"), (next_pos, "next_pos")):
        if t is not None:
            _need(t, n, torch.int32, 2)
            if tuple(t.shape) != (b, B):
                raise ValueError(f"{n} must be [b][B]")
    rc = load_library().simsd_commit_kv(_ptr(k_blk), _ptr(v_blk), _ptr(tau), _ptr(accept_len), _ptr(k_cache),
                                        _ptr(v_cache), _ptr(cache_offsets), _ptr(cache_lens), _ptr(pos),
                                        _ptr(next_pos), b, B, Hkv, d, flags, _ptr(status), _stream(stream))
    _check("simsd_commit_kv", rc)
