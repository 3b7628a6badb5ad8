"""Block-diffusion attention and the confidence commit on MI355X (gfx950).

A thin ctypes binding over ``libbda.so`` (C ABI declared in ``include/bda.h``).
Tensors are torch CUDA (HIP) tensors; this module only checks dtypes, shapes
and devices, allocates outputs/workspaces with torch, and passes raw device
pointers plus torch's current HIP stream to the library.  Every step of the
computation runs in the library's kernels.  There is no CPU fallback: if the
library is missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbda.so")

MODE = {"hybrid": 0, "decode": 1, "causal": 2}
BF16, F32 = 0, 1
TILE_FULL, TILE_EMPTY, TILE_PARTIAL = 0, 1, 2

_ENTRY_POINTS = (
    "bda_attn_fwd", "bda_attn_workspace_bytes", "bda_commit", "bda_commit_workspace_bytes",
    "bda_verify", "bda_verify_workspace_bytes", "bda_classify_tile", "bda_strerror",
    "bda_last_error", "bda_version", "bda_row_stats", "bda_row_stats_workspace_bytes",
    "bda_attn_fwd_lse", "bda_attn_bwd", "bda_attn_bwd_workspace_bytes", "bda_sprint_prune",
    "bda_sprint_workspace_bytes", "bda_sprint_kept_count", "bda_attn_fwd_varlen", "bda_kv_append",
    "bda_verify_crop", "bda_commit_entropy", "bda_commit_entropy_workspace_bytes", "bda_adaptive_stop",
    "bda_row_stats_commit", "bda_row_stats_commit_workspace_bytes",
)


class BdaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {lib.bda_strerror(code).decode()} ({lib.bda_last_error().decode()})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m block_masked_attention_amd.build` "
                          "(or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    P, I, S, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    L.bda_attn_fwd.argtypes = [P, P, P, P, I, I, I, I, I, I, I, P, S, P]
    L.bda_attn_fwd.restype = I
    L.bda_attn_fwd_lse.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, P, S, P]
    L.bda_attn_fwd_lse.restype = I
    L.bda_attn_fwd_varlen.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, P, S, P]
    L.bda_attn_fwd_varlen.restype = I
    L.bda_kv_append.argtypes = [P, P, P, P, P, I, I, I, I, I, P]
    L.bda_kv_append.restype = I
    L.bda_verify_crop.argtypes = [P, I, P, P, P, P, I, I, I, I, P, S, P]
    L.bda_verify_crop.restype = I
    L.bda_commit_entropy.argtypes = [P, I, P, P, F, F, I, I, I, I, P, S, P]
    L.bda_commit_entropy.restype = I
    L.bda_commit_entropy_workspace_bytes.argtypes = [I, I, I]
    L.bda_commit_entropy_workspace_bytes.restype = S
    L.bda_adaptive_stop.argtypes = [P, P, P, P, P, I, I, I, F, P, P]
    L.bda_adaptive_stop.restype = I
    L.bda_attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, S, P]
    L.bda_attn_bwd.restype = I
    L.bda_attn_bwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    L.bda_attn_bwd_workspace_bytes.restype = S
    L.bda_attn_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    L.bda_attn_workspace_bytes.restype = S
    L.bda_commit.argtypes = [P, I, P, P, F, I, I, I, I, P, S, P]
    L.bda_commit.restype = I
    L.bda_commit_noalloc.argtypes = [P, I, P, P, F, I, I, I, I, P]
    L.bda_commit_noalloc.restype = I
    L.bda_commit_workspace_bytes.argtypes = [I, I, I]
    L.bda_commit_workspace_bytes.restype = S
    L.bda_verify.argtypes = [P, I, P, P, P, I, I, I, P, S, P]
    L.bda_verify.restype = I
    L.bda_verify_workspace_bytes.argtypes = [I, I, I]
    L.bda_verify_workspace_bytes.restype = S
    L.bda_row_stats.argtypes = [P, I, P, P, P, P, P, I, I, I, P, S, P]
    L.bda_row_stats.restype = I
    L.bda_row_stats_workspace_bytes.argtypes = [I, I, I]
    L.bda_row_stats_workspace_bytes.restype = S
    L.bda_row_stats_commit.argtypes = [P, I, P, P, F, I, P, P, P, P, I, I, I, P, S, P]
    L.bda_row_stats_commit.restype = I
    L.bda_row_stats_commit_workspace_bytes.argtypes = [I, I, I]
    L.bda_row_stats_commit_workspace_bytes.restype = S
    L.bda_sprint_prune.argtypes = [P, P, P, P, F, F, F, P, P, I, P, P, P, I, I, I, I, P, S, P]
    L.bda_sprint_prune.restype = I
    L.bda_sprint_workspace_bytes.argtypes = [I, I]
    L.bda_sprint_workspace_bytes.restype = S
    L.bda_sprint_kept_count.argtypes = [I, I, F, F]
    L.bda_sprint_kept_count.restype = I
    L.bda_classify_tile.argtypes = [I, I, I, I, I, I, I]
    L.bda_classify_tile.restype = I
    for name in ("bda_strerror",):
        getattr(L, name).argtypes = [I]
        getattr(L, name).restype = ctypes.c_char_p
    for name in ("bda_last_error", "bda_version"):
        getattr(L, name).argtypes = []
        getattr(L, name).restype = ctypes.c_char_p
    return L


lib = _load()


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _check_dev(*ts):
    dev = ts[0].device
    for t in ts:
        if t is None:
            continue
        if t.device.type != "cuda" or t.device != dev:
            raise ValueError("all tensors must be on the same HIP device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def _workspace(nbytes: int, device, ws):
    if nbytes == 0:
        return None
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace needs {nbytes} bytes")
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def attn_workspace_bytes(B, Hq, Hkv, L, d, block, mode) -> int:
    return int(lib.bda_attn_workspace_bytes(B, Hq, Hkv, L, d, block, MODE[mode] if isinstance(mode, str) else mode))


def attn_fwd(q, k, v, mode: str, block: int, out=None, workspace=None, lse=None):
    """Masked attention forward (bf16).  HYBRID: q/k/v [B,H,2L,d] over
    [x_t ; x_0]; DECODE/CAUSAL: q [B,Hq,n,d] with n = ``block`` and k/v
    [B,Hkv,L,d].  Returns ``out`` shaped like q.  With ``lse`` (float32
    [B,Hq,rows]) the per-row natural-log log-sum-exp is written too."""
    m = MODE[mode]
    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or t.dim() != 4:
            raise ValueError("q, k, v must be 4-D bfloat16")
    dev = _check_dev(q, k, v)
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k/v shape mismatch")
    if m == 0:
        if Sq != Sk or Sq % 2:
            raise ValueError("hybrid form needs q, k, v of 2L rows")
        L = Sq // 2
    else:
        if Sq != block:
            raise ValueError("decode/causal: q rows must equal block")
        L = Sk
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != torch.bfloat16:
        raise ValueError("out must match q")
    _check_dev(q, out)
    need = attn_workspace_bytes(B, Hq, Hkv, L, d, block, m)
    ws = _workspace(need, dev, workspace)
    if lse is None:
        rc = lib.bda_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, L, d, block, m,
                              _ptr(ws), need, _stream(dev))
    else:
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Sq):
            raise ValueError("lse must be float32 [B, Hq, rows]")
        _check_dev(q, lse)
        rc = lib.bda_attn_fwd_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, L, d, block,
                                  m, _ptr(ws), need, _stream(dev))
    if rc:
        raise BdaError(rc, "bda_attn_fwd")
    return out


def attn_bwd(q, k, v, out, dout, lse, block: int, workspace=None):
    """Backward of the training form (hybrid mask): returns (dq, dk, dv) for
    loss = sum(dout * out); ``lse`` from attn_fwd(..., lse=...)."""
    for t in (q, k, v, out, dout):
        if t.dtype != torch.bfloat16 or t.dim() != 4:
            raise ValueError("q, k, v, out, dout must be 4-D bfloat16")
    dev = _check_dev(q, k, v, out, dout, lse)
    B, Hq, Sq, d = q.shape
    Hkv = k.shape[1]
    if Sq % 2 or k.shape != v.shape or k.shape[2] != Sq or out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("lse must be float32 [B, Hq, 2L]")
    L = Sq // 2
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    need = int(lib.bda_attn_bwd_workspace_bytes(B, Hq, Hkv, L, d, block, 0))
    ws = _workspace(need, dev, workspace)
    rc = lib.bda_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                          _ptr(dv), B, Hq, Hkv, L, d, block, 0, _ptr(ws), need, _stream(dev))
    if rc:
        raise BdaError(rc, "bda_attn_bwd")
    return dq, dk, dv


def commit(logits, tokens, masked, threshold: float, k_min: int, workspace=None):
    """In-place confidence commit on logits [G,R,V] (bf16 or fp32);
    ``tokens`` int64 [G,R] and ``masked`` uint8 [G,R] are updated."""
    if logits.dim() != 3:
        raise ValueError("logits must be [G, R, V]")
    G, R, V = logits.shape
    dt = {torch.bfloat16: BF16, torch.float32: F32}.get(logits.dtype)
    if dt is None:
        raise ValueError("logits must be bfloat16 or float32")
    if tokens.dtype != torch.int64 or masked.dtype != torch.uint8:
        raise ValueError("tokens int64, masked uint8")
    if tuple(tokens.shape) != (G, R) or tuple(masked.shape) != (G, R):
        raise ValueError("tokens/masked must be [G, R]")
    dev = _check_dev(logits, tokens, masked)
    need = int(lib.bda_commit_workspace_bytes(G, R, V))
    ws = _workspace(need, dev, workspace)
    rc = lib.bda_commit(_ptr(logits), dt, _ptr(tokens), _ptr(masked), float(threshold), int(k_min),
                        G, R, V, _ptr(ws), need, _stream(dev))
    if rc:
        raise BdaError(rc, "bda_commit")
    return tokens, masked


def commit_noalloc(logits, tokens, masked, threshold: float, k_min: int):
    """bda_commit over the library's static scratch: nothing is allocated
    (calls on one GPU must not overlap in time)."""
    if logits.dim() != 3:
        raise ValueError("logits must be [G, R, V]")
    G, R, V = logits.shape
    dt = {torch.bfloat16: BF16, torch.float32: F32}.get(logits.dtype)
    if dt is None:
        raise ValueError("logits must be bfloat16 or float32")
    if tokens.dtype != torch.int64 or masked.dtype != torch.uint8:
        raise ValueError("tokens int64, masked uint8")
    if tuple(tokens.shape) != (G, R) or tuple(masked.shape) != (G, R):
        raise ValueError("tokens/masked must be [G, R]")
    dev = _check_dev(logits, tokens, masked)
    rc = lib.bda_commit_noalloc(_ptr(logits), dt, _ptr(tokens), _ptr(masked), float(threshold), int(k_min),
                                G, R, V, _stream(dev))
    if rc:
        raise BdaError(rc, "bda_commit_noalloc")
    return tokens, masked


def attn_fwd_varlen(q, k, v, kv_len, mode: str, block: int, out=None, workspace=None):
    """DECODE/CAUSAL forward over a cache with per-row key counts: q
    [B,Hq,n,d] with n = ``block``, k/v [B,Hkv,L_cap,d], ``kv_len`` int32 [B]
    on the device (row b uses its first kv_len[b] keys, clamped to [n, L_cap];
    its last n keys are the block)."""
    m = MODE[mode]
    if m == 0:
        raise ValueError("per-row key counts apply to the decode and causal forms")
    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or t.dim() != 4:
            raise ValueError("q, k, v must be 4-D bfloat16")
    dev = _check_dev(q, k, v, kv_len)
    B, Hq, Sq, d = q.shape
    Hkv, Lc = k.shape[1], k.shape[2]
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d or Sq != block:
        raise ValueError("shape mismatch")
    if kv_len.dtype != torch.int32 or tuple(kv_len.shape) != (B,):
        raise ValueError("kv_len must be int32 [B]")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != torch.bfloat16:
        raise ValueError("out must match q")
    _check_dev(q, out)
    need = attn_workspace_bytes(B, Hq, Hkv, Lc, d, block, m)
    ws = _workspace(need, dev, workspace)
    rc = lib.bda_attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(kv_len), B, Hq, Hkv, Lc, d, block, m,
                                 _ptr(ws), need, _stream(dev))
    if rc:
        raise BdaError(rc, "bda_attn_fwd_varlen")
    return out


def kv_append(k_cache, v_cache, k_new, v_new, kv_len):
    """Write the block rows k_new/v_new [B,Hkv,n,d] at rows kv_len[b]-n ..
    kv_len[b]-1 of the caches [B,Hkv,L_cap,d] (in place)."""
    for t in (k_cache, v_cache, k_new, v_new):
        if t.dtype != torch.bfloat16 or t.dim() != 4:
            raise ValueError("caches and new rows must be 4-D bfloat16")
    if k_cache.shape != v_cache.shape or k_new.shape != v_new.shape:
        raise ValueError("k and v shapes differ")
    B, Hkv, Lc, d = k_cache.shape
    n = k_new.shape[2]
    if k_new.shape[0] != B or k_new.shape[1] != Hkv or k_new.shape[3] != d:
        raise ValueError("new rows do not match the cache")
    if kv_len.dtype != torch.int32 or tuple(kv_len.shape) != (B,):
        raise ValueError("kv_len must be int32 [B]")
    dev = _check_dev(k_cache, v_cache, k_new, v_new, kv_len)
    rc = lib.bda_kv_append(_ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(kv_len), B, Hkv, Lc, n, d,
                           _stream(dev))
    if rc:
        raise BdaError(rc, "bda_kv_append")


def verify_crop(logits, drafts, kv_len, kv_cap: int, argmax_out=None, accept_len=None, workspace=None):
    """verify, then kv_len[b] = min(kv_len[b] + accept_len[b], kv_cap) on the
    device.  Returns (argmax [B,R] int64, accept_len [B] int32)."""
    if logits.dim() != 3:
        raise ValueError("logits must be [B, R, V]")
    B, R, V = logits.shape
    dt = {torch.bfloat16: BF16, torch.float32: F32}.get(logits.dtype)
    if dt is None:
        raise ValueError("logits must be bfloat16 or float32")
    if drafts.dtype != torch.int64 or tuple(drafts.shape) != (B, R):
        raise ValueError("drafts must be int64 [B, R]")
    if kv_len.dtype != torch.int32 or tuple(kv_len.shape) != (B,):
        raise ValueError("kv_len must be int32 [B]")
    dev = _check_dev(logits, drafts, kv_len, argmax_out, accept_len)
    am = torch.empty(B, R, dtype=torch.int64, device=dev) if argmax_out is None else argmax_out
    acc = torch.empty(B, dtype=torch.int32, device=dev) if accept_len is None else accept_len
    if am.dtype != torch.int64 or tuple(am.shape) != (B, R) or acc.dtype != torch.int32 or tuple(acc.shape) != (B,):
        raise ValueError("argmax_out must be int64 [B, R], accept_len int32 [B]")
    need = int(lib.bda_verify_workspace_bytes(B, R, V))
    ws = _workspace(need, dev, workspace)
    rc = lib.bda_verify_crop(_ptr(logits), dt, _ptr(drafts), _ptr(am), _ptr(acc), _ptr(kv_len), kv_cap, B, R, V,
                             _ptr(ws), need, _stream(dev))
    if rc:
        raise BdaError(rc, "bda_verify_crop")
    return am, acc


def commit_entropy(logits, tokens, masked, entropy_bound: float, temperature: float = 1.0, k_min: int = 1,
                   workspace=None):
    """Entropy-bound commit on logits [G,R,V] (bf16 or fp32): updates
    ``tokens`` (int64 [G,R]) and ``masked`` (uint8 [G,R]) in place."""
    if logits.dim() != 3:
        raise ValueError("logits must be [G, R, V]")
    G, R, V = logits.shape
    dt = {torch.bfloat16: BF16, torch.float32: F32}.get(logits.dtype)
    if dt is None:
        raise ValueError("logits must be bfloat16 or float32")
    if tokens.dtype != torch.int64 or masked.dtype != torch.uint8 or tuple(tokens.shape) != (G, R) \
            or tuple(masked.shape) != (G, R):
        raise ValueError("tokens must be int64 [G, R] and masked uint8 [G, R]")
    dev = _check_dev(logits, tokens, masked)
    need = int(lib.bda_commit_entropy_workspace_bytes(G, R, V))
    ws = _workspace(need, dev, workspace)
    rc = lib.bda_commit_entropy(_ptr(logits), dt, _ptr(tokens), _ptr(masked), entropy_bound, temperature, k_min,
                                G, R, V, _ptr(ws), need, _stream(dev))
    if rc:
        raise BdaError(rc, "bda_commit_entropy")


def adaptive_stop(argmax, prev_argmax, stable_steps, frozen, mean_entropy, stability_threshold: int = 1,
                  confidence_threshold: float = 0.005, n_frozen=None):
    """One adaptive-stopping step on device state (updated in place):
    argmax / prev_argmax int64 [G,R], stable_steps int32 [G], frozen uint8
    [G], mean_entropy float32 [G]; n_frozen (int32 [1]) if given receives the
    number of frozen examples."""
    G = frozen.shape[0]
    R = argmax.shape[1] if argmax.dim() == 2 else 0
    if argmax.dtype != torch.int64 or prev_argmax.dtype != torch.int64 or tuple(argmax.shape) != (G, R) \
            or tuple(prev_argmax.shape) != (G, R):
        raise ValueError("argmax and prev_argmax must be int64 [G, R]")
    if stable_steps.dtype != torch.int32 or frozen.dtype != torch.uint8 or mean_entropy.dtype != torch.float32:
        raise ValueError("stable_steps int32 [G], frozen uint8 [G], mean_entropy float32 [G]")
    if tuple(stable_steps.shape) != (G,) or tuple(mean_entropy.shape) != (G,):
        raise ValueError("stable_steps and mean_entropy must be [G]")
    if n_frozen is not None and (n_frozen.dtype != torch.int32 or n_frozen.numel() < 1):
        raise ValueError("n_frozen must be int32 with at least one element")
    dev = _check_dev(argmax, prev_argmax, stable_steps, frozen, mean_entropy, n_frozen)
    rc = lib.bda_adaptive_stop(_ptr(argmax), _ptr(prev_argmax), _ptr(stable_steps), _ptr(frozen),
                               _ptr(mean_entropy), G, R, stability_threshold, confidence_threshold, _ptr(n_frozen),
                               _stream(dev))
    if rc:
        raise BdaError(rc, "bda_adaptive_stop")


def verify(logits, drafts, workspace=None):
    """Argmax per row and longest matching prefix: returns (argmax [B,R]
    int64, accept_len [B] int32)."""
    if logits.dim() != 3:
        raise ValueError("logits must be [B, R, V]")
    B, R, V = logits.shape
    dt = {torch.bfloat16: BF16, torch.float32: F32}.get(logits.dtype)
    if dt is None:
        raise ValueError("logits must be bfloat16 or float32")
    if drafts.dtype != torch.int64 or tuple(drafts.shape) != (B, R):
        raise ValueError("drafts must be int64 [B, R]")
    dev = _check_dev(logits, drafts)
    am = torch.empty(B, R, dtype=torch.int64, device=dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    need = int(lib.bda_verify_workspace_bytes(B, R, V))
    ws = _workspace(need, dev, workspace)
    rc = lib.bda_verify(_ptr(logits), dt, _ptr(drafts), _ptr(am), _ptr(acc), B, R, V,
                        _ptr(ws), need, _stream(dev))
    if rc:
        raise BdaError(rc, "bda_verify")
    return am, acc


def row_stats(logits, masked=None, workspace=None, out=None):
    """Per-row softmax statistics of logits [G,R,V] (bf16 or fp32): returns
    (conf [G,R] float32, argmax [G,R] int64, entropy [G,R] float32 in nats,
    mean_entropy [G] float32).  With ``masked`` (uint8 [G,R]) only rows with
    masked != 0 are computed; the other rows' outputs are NaN / -1 and the
    group means cover the computed rows only.  ``out`` = the four output
    tensors, written in place (rows not computed keep their contents)."""
    if logits.dim() != 3:
        raise ValueError("logits must be [G, R, V]")
    G, R, V = logits.shape
    dt = {torch.bfloat16: BF16, torch.float32: F32}.get(logits.dtype)
    if dt is None:
        raise ValueError("logits must be bfloat16 or float32")
    if masked is not None and (masked.dtype != torch.uint8 or tuple(masked.shape) != (G, R)):
        raise ValueError("masked must be uint8 [G, R]")
    dev = _check_dev(logits, masked)
    if out is not None:
        conf, am, ent, mean = out
        for t, dt_, shp in ((conf, torch.float32, (G, R)), (am, torch.int64, (G, R)), (ent, torch.float32, (G, R)),
                            (mean, torch.float32, (G,))):
            if t.dtype != dt_ or tuple(t.shape) != shp or not t.is_contiguous() or t.device != dev:
                raise ValueError("out tensors must be contiguous conf/entropy float32 [G,R], argmax int64 [G,R], "
                                 "mean float32 [G] on the logits' device")
    else:
        conf = torch.full((G, R), float("nan"), dtype=torch.float32, device=dev)
        am = torch.full((G, R), -1, dtype=torch.int64, device=dev)
        ent = torch.full((G, R), float("nan"), dtype=torch.float32, device=dev)
        mean = torch.empty(G, dtype=torch.float32, device=dev)
    need = int(lib.bda_row_stats_workspace_bytes(G, R, V))
    ws = _workspace(need, dev, workspace)
    rc = lib.bda_row_stats(_ptr(logits), dt, _ptr(masked), _ptr(conf), _ptr(am), _ptr(ent), _ptr(mean),
                           G, R, V, _ptr(ws), need, _stream(dev))
    if rc:
        raise BdaError(rc, "bda_row_stats")
    return conf, am, ent, mean


def row_stats_commit(logits, tokens, masked, threshold: float, k_min: int, workspace=None, out=None):
    """Row statistics of every row and the confidence commit of the masked
    rows from one pass over logits [G,R,V] (bf16 or fp32): the results of
    row_stats(logits) and then commit(logits, tokens, masked, threshold,
    k_min).  ``tokens`` int64 [G,R] and ``masked`` uint8 [G,R] are updated in
    place.  Returns (conf, argmax, entropy, mean_entropy), written into
    ``out`` when given (four tensors as for row_stats)."""
    if logits.dim() != 3:
        raise ValueError("logits must be [G, R, V]")
    G, R, V = logits.shape
    dt = {torch.bfloat16: BF16, torch.float32: F32}.get(logits.dtype)
    if dt is None:
        raise ValueError("logits must be bfloat16 or float32")
    if tokens.dtype != torch.int64 or masked.dtype != torch.uint8:
        raise ValueError("tokens int64, masked uint8")
    if tuple(tokens.shape) != (G, R) or tuple(masked.shape) != (G, R):
        raise ValueError("tokens/masked must be [G, R]")
    dev = _check_dev(logits, tokens, masked)
    if out is not None:
        conf, am, ent, mean = out
        for t, dt_, shp in ((conf, torch.float32, (G, R)), (am, torch.int64, (G, R)), (ent, torch.float32, (G, R)),
                            (mean, torch.float32, (G,))):
            if t.dtype != dt_ or tuple(t.shape) != shp or not t.is_contiguous() or t.device != dev:
                raise ValueError("out tensors must be contiguous conf/entropy float32 [G,R], argmax int64 [G,R], "
                                 "mean float32 [G] on the logits' device")
    else:
        conf = torch.empty((G, R), dtype=torch.float32, device=dev)
        am = torch.empty((G, R), dtype=torch.int64, device=dev)
        ent = torch.empty((G, R), dtype=torch.float32, device=dev)
        mean = torch.empty(G, dtype=torch.float32, device=dev)
    need = int(lib.bda_row_stats_commit_workspace_bytes(G, R, V))
    ws = _workspace(need, dev, workspace)
    rc = lib.bda_row_stats_commit(_ptr(logits), dt, _ptr(tokens), _ptr(masked), float(threshold), int(k_min),
                                  _ptr(conf), _ptr(am), _ptr(ent), _ptr(mean), G, R, V, _ptr(ws), need,
                                  _stream(dev))
    if rc:
        raise BdaError(rc, "bda_row_stats_commit")
    return conf, am, ent, mean


def sprint_kept_count(n_image: int, n_text: int, r_img: float = 0.8, r_text: float = 1.0) -> int:
    K = int(lib.bda_sprint_kept_count(n_image, n_text, r_img, r_text))
    if K < 0:
        raise ValueError("bad SPRINT counts or ratios")
    return K


def sprint_prune(k, v, conf, modality, alpha: float = 0.5, r_img: float = 0.8, r_text: float = 1.0,
                 gather: bool = True, scores: bool = False, workspace=None, n_text=None):
    """SPRINT prefix pruning of the cache k, v [B,Hkv,L,d] (bf16) with
    per-position confidence ``conf`` (float32 [B,L]) and ``modality`` (uint8
    [L], 0 = text).  Returns (k_out, v_out [B,Hkv,K,d] or None, kept int32
    [B,L] (-1 padded), scores float32 [B,L] or None).  K is computed on the
    host from the modality counts: pass ``n_text`` (the number of zeros in
    ``modality``) when it is known, else it is read back from the device."""
    for t in (k, v):
        if t.dtype != torch.bfloat16 or t.dim() != 4:
            raise ValueError("k, v must be 4-D bfloat16")
    if k.shape != v.shape:
        raise ValueError("k and v must have one shape")
    B, Hkv, L, d = k.shape
    if conf.dtype != torch.float32 or tuple(conf.shape) != (B, L):
        raise ValueError("conf must be float32 [B, L]")
    if modality.dtype != torch.uint8 or tuple(modality.shape) != (L,):
        raise ValueError("modality must be uint8 [L]")
    dev = _check_dev(k, v, conf, modality)
    if n_text is None:
        n_text = int((modality == 0).sum().item())
    K = sprint_kept_count(L - n_text, n_text, r_img, r_text)
    cap = K if gather else 0
    k_out = torch.empty((B, Hkv, cap, d), dtype=torch.bfloat16, device=dev) if gather else None
    v_out = torch.empty((B, Hkv, cap, d), dtype=torch.bfloat16, device=dev) if gather else None
    kept = torch.empty((B, L), dtype=torch.int32, device=dev)
    sc = torch.empty((B, L), dtype=torch.float32, device=dev) if scores else None
    need = int(lib.bda_sprint_workspace_bytes(B, L))
    ws = _workspace(need, dev, workspace)
    rc = lib.bda_sprint_prune(_ptr(k), _ptr(v), _ptr(conf), _ptr(modality), alpha, r_img, r_text,
                              _ptr(k_out) if cap else None, _ptr(v_out) if cap else None, cap, _ptr(kept), None,
                              _ptr(sc), B, Hkv, L, d, _ptr(ws), need, _stream(dev))
    if rc:
        raise BdaError(rc, "bda_sprint_prune")
    return k_out, v_out, kept, sc


def classify_tile(mode, L, block, q0, q1, k0, k1) -> int:
    return int(lib.bda_classify_tile(MODE[mode] if isinstance(mode, str) else mode, L, block, q0, q1, k0, k1))


def version() -> str:
    return lib.bda_version().decode()
