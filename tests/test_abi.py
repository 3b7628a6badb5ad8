"""Host-only checks of the C ABI: the library loads, exports what the header
declares, rejects bad arguments before touching a device, and its tile
classifier agrees with the oracle's dense-mask reduction."""
import ctypes
import math
import os
import re

import pytest

import oracle
import block_masked_attention_amd as bda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bda.h")

# Distinct, 16-byte aligned, far-apart fake device addresses: every call below
# fails validation before any HIP call, so nothing dereferences them.
A, Bp, Cp, Dp, Wp = (ctypes.c_void_p(x << 32) for x in (1, 2, 3, 4, 5))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bda_\w+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(bda.lib, n), n


def test_strings():
    for code in range(5):
        assert bda.lib.bda_strerror(code)
    assert bda.lib.bda_strerror(99) == b"unknown error code"
    assert bda.version().startswith("bda")


def _attn(B=1, Hq=4, Hkv=2, L=64, d=128, block=8, mode=0, q=A, k=Bp, v=Cp, out=Dp, ws=None, nbytes=0):
    return bda.lib.bda_attn_fwd(q, k, v, out, B, Hq, Hkv, L, d, block, mode, ws, nbytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(out=None), 1), (dict(Hq=3, Hkv=2), 1), (dict(d=96), 2), (dict(d=256), 2),
    (dict(block=0), 1), (dict(block=65), 1), (dict(mode=3), 1), (dict(B=0), 1), (dict(L=0), 1),
    (dict(q=ctypes.c_void_p((1 << 32) + 8)), 1),                      # misaligned
    (dict(out=ctypes.c_void_p((1 << 32) + 4096)), 1),                 # out overlaps q
    (dict(mode=1, L=4124, block=28, Hq=32, Hkv=8), 3),                # split workspace missing
])
def test_attn_validation(kw, code):
    assert _attn(**kw) == code
    assert bda.lib.bda_last_error()


def test_attn_workspace_sizes():
    assert bda.attn_workspace_bytes(4, 32, 8, 2048, 128, 32, "hybrid") == 0
    # 32 x 8 (batch, kv head) items give every CU one: no key split
    assert bda.attn_workspace_bytes(32, 32, 8, 4124, 128, 28, "decode") == 0
    need = bda.attn_workspace_bytes(16, 32, 8, 8220, 128, 28, "causal")   # 128 items: two splits
    assert need == 2 * 16 * 32 * 28 * (128 * 4 + 8)
    assert _attn(mode=2, L=8220, block=28, Hq=32, Hkv=8, B=16, ws=Wp, nbytes=need - 1) == 3
    assert bda.attn_workspace_bytes(1, 3, 2, 10, 128, 2, "hybrid") == 0     # invalid -> 0


def test_commit_validation():
    c = bda.lib.bda_commit
    assert c(A, 0, Bp, Cp, 0.9, 1, 0, 5, 10, None, 0, None) == 0             # nothing to do
    assert c(A, 2, Bp, Cp, 0.9, 1, 1, 5, 10, Wp, 1 << 20, None) == 1         # dtype
    assert c(A, 0, Bp, Cp, float("nan"), 1, 1, 5, 10, Wp, 1 << 20, None) == 1
    assert c(A, 0, Bp, Cp, 0.9, -1, 1, 5, 10, Wp, 1 << 20, None) == 1
    assert c(A, 0, Bp, Cp, 0.9, 1, 1, 5, 0, Wp, 1 << 20, None) == 1          # V
    assert c(None, 0, Bp, Cp, 0.9, 1, 1, 5, 10, Wp, 1 << 20, None) == 1
    assert c(A, 0, None, Cp, 0.9, 1, 1, 5, 10, Wp, 1 << 20, None) == 1
    assert c(A, 0, Bp, Cp, 0.9, 1, 1, 5, 10, None, 0, None) == 3             # workspace
    need = bda.lib.bda_commit_workspace_bytes(1, 5, 10)
    assert c(A, 0, Bp, Cp, 0.9, 1, 1, 5, 10, Wp, need - 1, None) == 3
    assert c(A, 0, ctypes.c_void_p((1 << 32) + 16), Cp, 0.9, 1, 1, 5, 10, Wp, need, None) == 1  # overlap


def test_verify_validation():
    f = bda.lib.bda_verify
    assert f(A, 0, Bp, Cp, Dp, 0, 28, 100, None, 0, None) == 0
    assert f(A, 0, Bp, Cp, None, 2, 28, 100, Wp, 1 << 20, None) == 1
    assert f(A, 7, Bp, Cp, Dp, 2, 28, 100, Wp, 1 << 20, None) == 1
    assert f(A, 0, Bp, Cp, Dp, 2, 28, 100, None, 0, None) == 3


def _sweep():
    for L in (1, 5, 16, 37, 64):
        for b in sorted({1, 2, 3, 4, 7, 16, 32, L} & set(range(1, L + 1))):
            yield "hybrid", L, b
    for L, n in ((1, 1), (40, 7), (64, 28), (64, 64), (97, 33)):
        yield "decode", L, n
        yield "causal", L, n


@pytest.mark.parametrize("mode,L,b", list(_sweep()))
def test_classifier_matches_dense_mask(mode, L, b):
    M = oracle.mask(mode, L, b)
    rows, keys = M.shape
    for tq in (1, 3, 8, 32):
        for tk in (1, 5, 32, 64):
            for q0 in range(0, rows, tq):
                for k0 in range(0, keys, tk):
                    q1, k1 = min(rows, q0 + tq), min(keys, k0 + tk)
                    assert bda.classify_tile(mode, L, b, q0, q1, k0, k1) == oracle.tile_class(M, q0, q1, k0, k1), \
                        (mode, L, b, q0, q1, k0, k1)
    assert bda.classify_tile(mode, L, b, 0, rows + 1, 0, 1) == -1
    assert bda.classify_tile(mode, L, b, 0, 1, 2, 1) == -1


def test_row_stats_validation():
    f = bda.lib.bda_row_stats
    # logits, dtype, masked, conf, argmax, entropy, mean, G, R, V, ws, ws_bytes, stream
    assert f(A, 0, None, Bp, None, None, None, 0, 5, 10, None, 0, None) == 0          # nothing to do
    assert f(A, 3, None, Bp, None, None, None, 1, 5, 10, Wp, 1 << 20, None) == 1      # dtype
    assert f(A, 0, None, Bp, None, None, None, 1, 5, 0, Wp, 1 << 20, None) == 1       # V
    assert f(None, 0, None, Bp, None, None, None, 1, 5, 10, Wp, 1 << 20, None) == 1   # logits
    assert f(A, 0, None, Bp, None, None, None, 1, 5, 10, None, 0, None) == 3          # workspace
    need = bda.lib.bda_row_stats_workspace_bytes(1, 5, 10)
    assert need > 0
    assert f(A, 0, None, Bp, None, None, None, 1, 5, 10, Wp, need - 1, None) == 3
    assert f(A, 0, None, ctypes.c_void_p((1 << 32) + 16), None, None, None, 1, 5, 10, Wp, need, None) == 1  # overlap


def test_row_stats_commit_validation():
    f = bda.lib.bda_row_stats_commit
    T, M = ctypes.c_void_p(6 << 32), ctypes.c_void_p(7 << 32)
    # logits, dtype, tokens, masked, threshold, k_min, conf, argmax, entropy, mean, G, R, V, ws, ws_bytes, stream
    assert f(A, 0, T, M, 0.9, 1, None, None, None, None, 0, 5, 10, None, 0, None) == 0        # nothing to do
    assert f(A, 3, T, M, 0.9, 1, None, None, None, None, 1, 5, 10, Wp, 1 << 20, None) == 1    # dtype
    assert f(A, 0, T, M, float("nan"), 1, None, None, None, None, 1, 5, 10, Wp, 1 << 20, None) == 1
    assert f(A, 0, T, M, 0.9, -1, None, None, None, None, 1, 5, 10, Wp, 1 << 20, None) == 1   # k_min
    assert f(A, 0, None, M, 0.9, 1, None, None, None, None, 1, 5, 10, Wp, 1 << 20, None) == 1  # tokens
    assert f(A, 0, T, M, 0.9, 1, None, None, None, None, 1, 5, 10, None, 0, None) == 3        # workspace
    need = bda.lib.bda_row_stats_commit_workspace_bytes(1, 5, 10)
    assert need == bda.lib.bda_commit_workspace_bytes(1, 5, 10) > 0
    assert f(A, 0, T, M, 0.9, 1, None, None, None, None, 1, 5, 10, Wp, need - 1, None) == 3
    assert f(A, 0, T, M, 0.9, 1, ctypes.c_void_p((1 << 32) + 16), None, None, None, 1, 5, 10, Wp, need,
             None) == 1                                                                        # conf overlaps logits
    assert f(A, 0, T, M, 0.9, 1, None, ctypes.c_void_p((7 << 32) + 2), None, None, 1, 5, 10, Wp, need,
             None) == 1                                                                        # argmax overlaps masked


def test_sprint_validation():
    f = bda.lib.bda_sprint_prune
    E, Fp, Gp = (ctypes.c_void_p(x << 32) for x in (6, 7, 8))
    need = bda.lib.bda_sprint_workspace_bytes(2, 64)
    assert need >= 2 * 64 * 4 + 2 * 64          # norms and kept flags

    # k, v, conf, modality, alpha, r_img, r_text, k_out, v_out, cap, kept, kept_count, scores,
    # B, Hkv, L, d, ws, ws_bytes, stream
    def call(**kw):
        a = dict(k=A, v=Bp, conf=Cp, mod=Dp, alpha=0.5, r_img=0.8, r_text=1.0, ko=E, vo=Fp, cap=16,
                 kept=Gp, kc=None, sc=None, B=2, H=8, L=64, d=128, ws=Wp, wsb=need)
        a.update(kw)
        return f(a["k"], a["v"], a["conf"], a["mod"], a["alpha"], a["r_img"], a["r_text"], a["ko"], a["vo"],
                 a["cap"], a["kept"], a["kc"], a["sc"], a["B"], a["H"], a["L"], a["d"], a["ws"], a["wsb"], None)

    assert call(d=96) == 2                       # head dim
    assert call(L=16385) == 2                    # LDS-resident sort bound
    assert call(B=0) == 1
    assert call(alpha=1.5) == 1
    assert call(r_img=-0.1) == 1
    assert call(r_text=float("nan")) == 1
    assert call(cap=-1) == 1
    assert call(conf=None) == 1
    assert call(kept=None) == 1
    assert call(ko=None) == 1                    # gather requested without outputs
    assert call(ws=None) == 3
    assert call(wsb=need - 1) == 3
    assert call(ko=ctypes.c_void_p((1 << 32) + 8)) == 1     # misaligned
    assert call(ko=ctypes.c_void_p((1 << 32) + 4096)) == 1  # k_out inside k
    assert call(kept=ctypes.c_void_p((2 << 32) + 64)) == 1  # kept inside v
    assert call(conf=ctypes.c_void_p((3 << 32) + 2)) == 1   # misaligned confidence
    assert call(sc=ctypes.c_void_p((9 << 32) + 1)) == 1     # misaligned scores


def test_sprint_kept_count():
    kc = bda.lib.bda_sprint_kept_count
    assert kc(3080, 1016, 0.8, 1.0) == 2464 + 1016
    assert kc(5, 3, 0.5, 0.5) == 3 + 2             # floor(2.5 + 0.5), floor(1.5 + 0.5)
    assert kc(0, 0, 0.8, 1.0) == 0
    assert kc(-1, 0, 0.8, 1.0) == -1
    assert kc(1, 1, 1.5, 1.0) == -1
    # the oracle's count for the same modality mix
    for n_img, n_txt, ri, rt in ((7, 3, 0.8, 1.0), (10, 10, 0.35, 0.65), (1, 0, 0.5, 0.5)):
        L = n_img + n_txt
        md = [1] * n_img + [0] * n_txt
        k = [[[[1.0] * 4 for _ in range(L)]]]
        conf = [[0.5] * L]
        _, _, K = oracle.sprint(k, conf, md, 0.5, ri, rt)
        assert kc(n_img, n_txt, ri, rt) == K


def test_varlen_cache_validation():
    f = bda.lib.bda_attn_fwd_varlen
    E = ctypes.c_void_p(6 << 32)
    # q, k, v, out, kv_len, B, Hq, Hkv, L_cap, d, block, mode, ws, ws_bytes, stream
    assert f(A, Bp, Cp, Dp, E, 2, 32, 8, 256, 128, 28, 0, None, 0, None) == 2        # hybrid
    assert f(A, Bp, Cp, Dp, None, 2, 32, 8, 256, 128, 28, 1, None, 0, None) == 1     # no lengths
    assert f(A, Bp, Cp, Dp, ctypes.c_void_p((6 << 32) + 2), 2, 32, 8, 256, 128, 28, 1, None, 0, None) == 1
    assert f(A, Bp, Cp, Dp, ctypes.c_void_p((4 << 32) + 16), 2, 32, 8, 256, 128, 28, 2, None, 0, None) == 1  # in out
    assert f(A, Bp, Cp, Dp, E, 2, 32, 8, 20, 128, 28, 1, None, 0, None) == 1          # block > capacity
    a = bda.lib.bda_kv_append
    # k_cache, v_cache, k_new, v_new, kv_len, B, Hkv, L_cap, n, d, stream
    assert a(A, Bp, Cp, Dp, E, 0, 8, 256, 28, 128, None) == 0                          # nothing to do
    assert a(A, Bp, Cp, Dp, E, 2, 8, 256, 28, 96, None) == 2
    assert a(A, Bp, Cp, Dp, E, 2, 8, 20, 28, 128, None) == 1
    assert a(A, Bp, None, Dp, E, 2, 8, 256, 28, 128, None) == 1
    assert a(A, ctypes.c_void_p((1 << 32) + 4096), Cp, Dp, E, 2, 8, 256, 28, 128, None) == 1   # caches overlap
    assert a(A, Bp, Cp, Dp, ctypes.c_void_p((1 << 32) + 64), 2, 8, 256, 28, 128, None) == 1    # lengths in a cache
    c = bda.lib.bda_verify_crop
    # logits, dtype, drafts, argmax, accept, kv_len, kv_cap, B, R, V, ws, ws_bytes, stream
    assert c(A, 0, Bp, Cp, Dp, None, 100, 2, 28, 100, Wp, 1 << 20, None) == 1
    assert c(A, 0, Bp, Cp, Dp, E, 0, 2, 28, 100, Wp, 1 << 20, None) == 1
    assert c(A, 0, Bp, Cp, Dp, ctypes.c_void_p((4 << 32) + 4), 100, 2, 28, 100, Wp, 1 << 20, None) == 1  # in accept
    assert c(A, 0, Bp, Cp, Dp, E, 100, 2, 28, 100, None, 0, None) == 3


def test_entropy_commit_and_adaptive_stop_validation():
    f = bda.lib.bda_commit_entropy
    # logits, dtype, tokens, masked, bound, temperature, k_min, G, R, V, ws, ws_bytes, stream
    need = bda.lib.bda_commit_entropy_workspace_bytes(2, 28, 1000)
    assert need == bda.lib.bda_commit_workspace_bytes(2, 28, 1000)
    assert f(A, 0, Bp, Cp, 1.0, 1.0, 1, 0, 28, 1000, None, 0, None) == 0            # nothing to do
    assert f(A, 0, Bp, Cp, 1.0, 0.0, 1, 2, 28, 1000, Wp, need, None) == 1           # temperature
    assert f(A, 0, Bp, Cp, 1.0, float("inf"), 1, 2, 28, 1000, Wp, need, None) == 1
    assert f(A, 0, Bp, Cp, float("nan"), 1.0, 1, 2, 28, 1000, Wp, need, None) == 1
    assert f(A, 0, Bp, Cp, 1.0, 1.0, -1, 2, 28, 1000, Wp, need, None) == 1          # k_min
    assert f(A, 0, Bp, Cp, 1.0, 1.0, 1, 2, 4097, 1000, Wp, 1 << 30, None) == 2      # rows per group
    assert f(A, 0, Bp, Cp, 1.0, 1.0, 1, 2, 28, 1000, Wp, need - 1, None) == 3
    assert f(A, 0, None, Cp, 1.0, 1.0, 1, 2, 28, 1000, Wp, need, None) == 1
    s = bda.lib.bda_adaptive_stop
    # argmax, prev, stable, frozen, mean_entropy, G, R, stability, conf, n_frozen, stream
    assert s(A, Bp, Cp, Dp, Wp, -1, 28, 1, 0.005, None, None) == 1
    assert s(A, Bp, Cp, Dp, Wp, 2, 28, -1, 0.005, None, None) == 1
    assert s(A, Bp, Cp, Dp, Wp, 2, 28, 1, float("nan"), None, None) == 1
    assert s(A, None, Cp, Dp, Wp, 2, 28, 1, 0.005, None, None) == 1
    assert s(ctypes.c_void_p((1 << 32) + 4), Bp, Cp, Dp, Wp, 2, 28, 1, 0.005, None, None) == 1   # misaligned
    assert s(A, ctypes.c_void_p((1 << 32) + 64), Cp, Dp, Wp, 2, 28, 1, 0.005, None, None) == 1   # prev in argmax
    assert s(A, Bp, Cp, Dp, Wp, 0, 28, 1, 0.005, None, None) == 0                   # nothing to do
