"""CPU oracle for block-diffusion attention, the confidence commit and verify.

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU
baseline leg may import this package; the library and its binding never do.
It shares no code with the HIP path.  The arithmetic lives in ``bda_oracle.c``
(double precision, explicit dense mask, scalar loops); this module only
marshals numpy arrays into it, plus a dense-mask tile reduction in numpy.

Pins: every function here is pinned by ``tests/test_oracle_pins.py`` against
closed forms, torch CPU fp64 SDPA special cases, brute force and hand-derived
fixtures.  The absolute attention/commit values on the synthetic workloads are
not printed anywhere on the pages, so those values themselves are pinned only
through the identities above (the pages give no worked numeric example).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bda_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

MODES = {"hybrid": 0, "decode": 1, "causal": 2}
FULL, EMPTY, PARTIAL = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP, -O2, strict IEEE: no fast-math)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build(force=True)
    lib = ctypes.CDLL(LIB)
    P, L, I, F = ctypes.c_void_p, ctypes.c_long, ctypes.c_int, ctypes.c_float
    lib.oracle_mask_shape.argtypes = [I, L, L, P, P]
    lib.oracle_mask.argtypes = [I, L, L, P]
    lib.oracle_attention.argtypes = [I, P, P, P, P, L, L, L, L, L, L, P, L, I]
    lib.oracle_commit.argtypes = [P, P, P, F, L, L, L, L, P, P, P, P, I]
    lib.oracle_verify.argtypes = [P, P, P, P, L, L, L, I]
    lib.oracle_row_stats.argtypes = [P, P, P, P, P, P, L, L, L, I]
    lib.oracle_attention_bwd.argtypes = [I, P, P, P, P, P, P, P, P, L, L, L, L, L, L, I]
    lib.oracle_sprint.argtypes = [P, P, P, ctypes.c_double, ctypes.c_double, ctypes.c_double, L, L, L, L, P, P]
    lib.oracle_sprint.restype = L
    lib.oracle_commit_entropy.argtypes = [P, P, P, ctypes.c_double, ctypes.c_double, L, L, L, L, P, P, I]
    lib.oracle_max_threads.restype = I
    for f in (lib.oracle_mask_shape, lib.oracle_mask, lib.oracle_attention,
              lib.oracle_commit, lib.oracle_verify, lib.oracle_row_stats, lib.oracle_attention_bwd,
              lib.oracle_commit_entropy):
        f.restype = I
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _f32(x) -> np.ndarray:
    """float32 contiguous copy of a numpy array or a (CPU) torch tensor."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.ascontiguousarray(x, dtype=np.float32)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def mask(mode: str, L: int, block: int) -> np.ndarray:
    """Dense mask (bool).  HYBRID: [2L, 2L] over [x_t ; x_0]; DECODE/CAUSAL:
    [block, L] (block = number of query rows)."""
    lib = _load()
    rows, keys = ctypes.c_long(), ctypes.c_long()
    if lib.oracle_mask_shape(MODES[mode], L, block, ctypes.byref(rows), ctypes.byref(keys)):
        raise ValueError("bad mask geometry")
    M = np.zeros((rows.value, keys.value), dtype=np.uint8)
    lib.oracle_mask(MODES[mode], L, block, _ptr(M))
    return M.astype(bool)


def attention(mode: str, q, k, v, L: int, block: int, sel=None, nthreads: int = 0) -> np.ndarray:
    """Masked attention in double.  q [B,Hq,rows,d], k/v [B,Hkv,keys,d].
    Returns [B,Hq,rows,d] float64, or [len(sel), d] for (b, h, i) triples."""
    lib = _load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, Hq, rows, d = q.shape
    Hkv = k.shape[1]
    if sel is None:
        out = np.empty((B, Hq, rows, d), dtype=np.float64)
        sel_arr, nsel = None, 0
    else:
        sel_arr = np.ascontiguousarray(np.asarray(sel, dtype=np.int64).reshape(-1, 3))
        nsel = sel_arr.shape[0]
        out = np.empty((nsel, d), dtype=np.float64)
    rc = lib.oracle_attention(MODES[mode], _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, L, d,
                              block, _ptr(sel_arr), nsel, nthreads)
    if rc:
        raise ValueError("oracle_attention: bad arguments")
    return out


def attention_bwd(mode: str, q, k, v, dout, L: int, block: int, nthreads: int = 0):
    """Gradients of sum(dout * attention(q, k, v)) in double: (dq, dk, dv,
    lse) with lse the natural-log log-sum-exp of each query row's scores."""
    lib = _load()
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, Hq, rows, d = q.shape
    Hkv = k.shape[1]
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.empty(k.shape, dtype=np.float64)
    dv = np.empty(v.shape, dtype=np.float64)
    lse = np.empty((B, Hq, rows), dtype=np.float64)
    rc = lib.oracle_attention_bwd(MODES[mode], _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk),
                                  _ptr(dv), _ptr(lse), B, Hq, Hkv, L, d, block, nthreads)
    if rc:
        raise ValueError("oracle_attention_bwd: bad arguments")
    return dq, dk, dv, lse


def sprint(k, conf, modality, alpha: float = 0.5, r_img: float = 0.8, r_text: float = 1.0):
    """SPRINT prefix retention in double: (kept [B, L] int64, -1 padded;
    scores [B, L] float64; K kept positions per batch)."""
    lib = _load()
    kk = _f32(k)
    B, Hkv, L, d = kk.shape
    cf = np.ascontiguousarray(np.asarray(conf, dtype=np.float32).reshape(B, L))
    md = np.ascontiguousarray(np.asarray(modality, dtype=np.uint8).reshape(L))
    kept = np.empty((B, L), dtype=np.int64)
    sc = np.empty((B, L), dtype=np.float64)
    # the ratios are fp32 parameters (as the library takes them); counts use their double values
    K = lib.oracle_sprint(_ptr(kk), _ptr(cf), _ptr(md), float(np.float32(alpha)), float(np.float32(r_img)),
                          float(np.float32(r_text)), B, Hkv, L, d, _ptr(kept), _ptr(sc))
    if K < 0:
        raise ValueError("oracle_sprint: bad arguments")
    return kept, sc, int(K)


def commit(logits, masked, tokens, threshold: float, k_min: int, nthreads: int = 0):
    """Confidence commit on logits [G,R,V].  Returns (tokens, masked, info)
    with new arrays; info holds p64, argmax, margin (|p - tau|) and gap."""
    lib = _load()
    lg = _f32(logits)
    G, R, V = lg.shape
    m = np.ascontiguousarray(np.asarray(masked, dtype=np.uint8)).copy()
    t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64)).copy()
    p64 = np.empty(G * R, dtype=np.float64)
    am = np.empty(G * R, dtype=np.int64)
    margin = np.empty(G * R, dtype=np.float64)
    gap = np.empty(max(G, 1), dtype=np.float64)
    rc = lib.oracle_commit(_ptr(lg), _ptr(t), _ptr(m), ctypes.c_float(threshold), k_min, G, R, V,
                           _ptr(p64), _ptr(am), _ptr(margin), _ptr(gap), nthreads)
    if rc:
        raise ValueError("oracle_commit: bad arguments")
    info = dict(p64=p64.reshape(G, R), argmax=am.reshape(G, R), margin=margin.reshape(G, R),
                gap=gap[:G])
    return t, m, info


def verify(logits, drafts, nthreads: int = 0):
    """Per-row argmax (lowest index) and longest matching prefix length."""
    lib = _load()
    lg = _f32(logits)
    B, R, V = lg.shape
    dr = np.ascontiguousarray(np.asarray(drafts, dtype=np.int64))
    am = np.empty((B, R), dtype=np.int64)
    acc = np.empty(B, dtype=np.int32)
    rc = lib.oracle_verify(_ptr(lg), _ptr(dr), _ptr(am), _ptr(acc), B, R, V, nthreads)
    if rc:
        raise ValueError("oracle_verify: bad arguments")
    return am, acc


def row_stats(logits, masked=None, nthreads: int = 0):
    """Per-row softmax statistics in double: (conf, argmax, entropy [nats],
    group mean entropy).  Rows with masked == 0 are not computed (NaN / -1)."""
    lib = _load()
    lg = _f32(logits)
    G, R, V = lg.shape
    m = None if masked is None else np.ascontiguousarray(np.asarray(masked, dtype=np.uint8))
    conf = np.full((G, R), np.nan)
    am = np.full((G, R), -1, dtype=np.int64)
    ent = np.full((G, R), np.nan)
    mean = np.empty(G)
    rc = lib.oracle_row_stats(_ptr(lg), _ptr(m), _ptr(conf), _ptr(am), _ptr(ent), _ptr(mean), G, R, V,
                              nthreads)
    if rc:
        raise ValueError("oracle_row_stats: bad arguments")
    return conf, am, ent, mean


def commit_entropy(logits, masked, tokens, bound: float, temperature: float, k_min: int, nthreads: int = 0):
    """Entropy-bound commit in double on logits [G,R,V].  bound and
    temperature are fp32 parameters (as the library takes them) used at their
    double values.  Returns (tokens, masked, entropy [G,R] (NaN where not
    masked), argmax [G,R] (-1 where not masked)) as new arrays."""
    lib = _load()
    lg = _f32(logits)
    G, R, V = lg.shape
    m = np.ascontiguousarray(np.asarray(masked, dtype=np.uint8)).copy()
    t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64)).copy()
    ent = np.full((G, R), np.nan)
    am = np.full((G, R), -1, dtype=np.int64)
    rc = lib.oracle_commit_entropy(_ptr(lg), _ptr(t), _ptr(m), float(np.float32(bound)),
                                   float(np.float32(temperature)), k_min, G, R, V, _ptr(ent), _ptr(am), nthreads)
    if rc:
        raise ValueError("oracle_commit_entropy: bad arguments")
    return t, m, ent, am


def adaptive_stop_step(argmax, prev, stable, frozen, mean_entropy, stability_threshold: int,
                       confidence_threshold: float):
    """One step of adaptive stopping ([DGemma] "Adaptive stopping"), per
    example g of argmax [G,R]: an example already frozen keeps its state;
    otherwise stable[g] counts the consecutive steps whose argmax equals the
    previous step's (reset to 0 on any change; prev = -1 counts as a change),
    prev becomes this step's argmax, and the example freezes once stable[g]
    >= stability_threshold and mean_entropy[g] < confidence_threshold (a
    float32 parameter).  Plain loops; returns new (prev, stable, frozen)."""
    argmax = np.asarray(argmax, dtype=np.int64)
    prev = np.array(prev, dtype=np.int64, copy=True)
    stable = np.array(stable, dtype=np.int64, copy=True)
    frozen = np.array(frozen, dtype=np.uint8, copy=True)
    thr = float(np.float32(confidence_threshold))
    G, R = argmax.shape
    for g in range(G):
        if frozen[g]:
            continue
        same = all(int(argmax[g, r]) == int(prev[g, r]) for r in range(R))
        stable[g] = stable[g] + 1 if same else 0
        for r in range(R):
            prev[g, r] = argmax[g, r]
        if stable[g] >= stability_threshold and float(np.float32(mean_entropy[g])) < thr:
            frozen[g] = 1
    return prev, stable, frozen


def tile_class(M: np.ndarray, q0: int, q1: int, k0: int, k1: int) -> int:
    """FULL / EMPTY / PARTIAL of the dense-mask rectangle [q0,q1) x [k0,k1)."""
    sub = M[q0:q1, k0:k1]
    if sub.size == 0 or not sub.any():
        return EMPTY
    if sub.all():
        return FULL
    return PARTIAL


def pair_count(mode: str, L: int, block: int) -> int:
    """Number of allowed (query, key) pairs, counted on the dense mask."""
    return int(mask(mode, L, block).sum())
