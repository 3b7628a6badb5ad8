"""Pins of the CPU oracle against facts that do not depend on it.

Each test checks the oracle against a closed form, a textbook routine (torch
CPU fp64 scaled_dot_product_attention), a hand-derived fixture, or a brute
force written differently (``oracle/brute.py``), so that a dropped term, a
swapped half, a wrong inequality or a transposed operand in the oracle fails
at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_mask(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([c == "1" for c in line.replace(" ", "")])
    return np.array(rows, dtype=bool)


def _rand(shape, seed, dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(dtype)


def _sdpa(q, k, v, mask=None, causal=False):
    """torch CPU fp64 SDPA on [B,H,S,d] with repeat-interleaved kv heads."""
    q, k, v = (torch.as_tensor(np.asarray(x, dtype=np.float64)) for x in (q, k, v))
    G = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(G, dim=1)
    v = v.repeat_interleave(G, dim=1)
    m = None if mask is None else torch.as_tensor(mask)
    return F.scaled_dot_product_attention(q, k, v, attn_mask=m, is_causal=causal).numpy()


# ---------------------------------------------------------------- masks

@pytest.mark.parametrize("L", range(1, 13))
def test_hybrid_mask_three_constructions(L):
    for b in range(1, L + 1):
        M = oracle.mask("hybrid", L, b)
        kron = np.array(brute.hybrid_mask_kron(L, b), dtype=bool)
        enum = np.array(brute.hybrid_mask_enum(L, b), dtype=bool)
        assert (M == kron).all(), (L, b)
        assert (M == enum).all(), (L, b)
        assert M[np.arange(2 * L), np.arange(2 * L)].all()   # every row sees itself
        assert not M[L:, :L].any()                            # x_0 never sees x_t


def test_mask_golden_fixtures():
    assert (oracle.mask("hybrid", 6, 2) == _read_mask("hybrid_mask_L6_b2.txt")).all()
    assert (oracle.mask("hybrid", 5, 2) == _read_mask("hybrid_mask_L5_b2.txt")).all()
    assert (oracle.mask("causal", 6, 3) == _read_mask("causal_mask_L6_n3.txt")).all()


@pytest.mark.parametrize("L,n", [(1, 1), (5, 1), (5, 5), (9, 4), (33, 28)])
def test_decode_causal_masks(L, n):
    assert (oracle.mask("decode", L, n) == np.array(brute.decode_mask_enum(L, n), bool)).all()
    assert (oracle.mask("causal", L, n) == np.array(brute.causal_mask_enum(L, n), bool)).all()


def test_pair_counts_closed_form():
    for L in (1, 7, 16, 64, 100):
        for b in sorted({1, 2, 3, 4, 7, 32, L} & set(range(1, L + 1))):
            starts = range(0, L, b)
            closed = 2 * sum(min(b, L - s) * (s + min(b, L - s)) for s in starts)
            assert oracle.pair_count("hybrid", L, b) == closed
            if L % b == 0:
                assert closed == L * (L + b)
    for L, n in ((10, 3), (64, 64), (4124, 28)):
        assert oracle.pair_count("decode", L, n) == n * L
        assert oracle.pair_count("causal", L, n) == n * (L - n) + n * (n + 1) // 2
    # the training-form workload: L=2048, b=32 -> L(L+b) pairs per head
    assert 2048 * (2048 + 32) * 4 * 128 * 4 * 32 == 279172874240


# ---------------------------------------------------------------- attention

def _hybrid_inputs(L, d=8, Hq=2, Hkv=1, B=1, seed=0):
    q = _rand((B, Hq, 2 * L, d), seed)
    k = _rand((B, Hkv, 2 * L, d), seed + 1)
    v = _rand((B, Hkv, 2 * L, d), seed + 2)
    return q, k, v


def test_block1_is_causal():
    L = 24
    q, k, v = _hybrid_inputs(L, Hq=4, Hkv=2)
    out = oracle.attention("hybrid", q, k, v, L, 1)
    ref0 = _sdpa(q[:, :, L:], k[:, :, L:], v[:, :, L:], causal=True)
    np.testing.assert_allclose(out[:, :, L:], ref0, rtol=0, atol=1e-12)
    # x_t half equals causal attention over x_0 once x_t's keys/values equal x_0's
    k2, v2 = k.clone(), v.clone()
    k2[:, :, :L] = k[:, :, L:]
    v2[:, :, :L] = v[:, :, L:]
    out2 = oracle.attention("hybrid", q, k2, v2, L, 1)
    ref_t = _sdpa(q[:, :, :L], k[:, :, L:], v[:, :, L:], causal=True)
    np.testing.assert_allclose(out2[:, :, :L], ref_t, rtol=0, atol=1e-12)


def test_block_L_is_per_half_bidirectional():
    L = 20
    q, k, v = _hybrid_inputs(L, Hq=2, Hkv=2)
    out = oracle.attention("hybrid", q, k, v, L, L)
    np.testing.assert_allclose(out[:, :, :L], _sdpa(q[:, :, :L], k[:, :, :L], v[:, :, :L]), atol=1e-12, rtol=0)
    np.testing.assert_allclose(out[:, :, L:], _sdpa(q[:, :, L:], k[:, :, L:], v[:, :, L:]), atol=1e-12, rtol=0)


def test_decode_is_unmasked_sdpa():
    q = _rand((2, 4, 5, 16), 3)
    k = _rand((2, 2, 37, 16), 4)
    v = _rand((2, 2, 37, 16), 5)
    out = oracle.attention("decode", q, k, v, 37, 5)
    np.testing.assert_allclose(out, _sdpa(q, k, v), atol=1e-12, rtol=0)


def test_causal_is_bottom_right_sdpa():
    n, L = 7, 40
    q = _rand((1, 4, n, 16), 6)
    k = _rand((1, 1, L, 16), 7)
    v = _rand((1, 1, L, 16), 8)
    out = oracle.attention("causal", q, k, v, L, n)
    br = torch.ones(n, L, dtype=torch.bool).tril(diagonal=L - n)
    np.testing.assert_allclose(out, _sdpa(q, k, v, mask=br), atol=1e-12, rtol=0)
    # top-left alignment would differ: guard against that reading
    assert not np.allclose(out, _sdpa(q, k, v, causal=True), atol=1e-6)


def test_cross_mode_identities():
    L, b = 21, 5
    q, k, v = _hybrid_inputs(L, Hq=4, Hkv=2, seed=11)
    out = oracle.attention("hybrid", q, k, v, L, b)
    for s in range(0, L, b):
        e = min(L, s + b)
        # noisy block = decode over (clean blocks before it) + (that noisy block)
        kk = torch.cat([k[:, :, L:L + s], k[:, :, s:e]], dim=2)
        vv = torch.cat([v[:, :, L:L + s], v[:, :, s:e]], dim=2)
        dec = oracle.attention("decode", q[:, :, s:e], kk, vv, kk.shape[2], e - s)
        np.testing.assert_allclose(out[:, :, s:e], dec, atol=1e-12, rtol=0)
        # clean block = decode over clean blocks up to and including it
        kk = k[:, :, L:L + e]
        vv = v[:, :, L:L + e]
        dec = oracle.attention("decode", q[:, :, L + s:L + e], kk, vv, e, e - s)
        np.testing.assert_allclose(out[:, :, L + s:L + e], dec, atol=1e-12, rtol=0)
    # causal(L, n) = last n rows of causal(L, L)
    qc = _rand((1, 2, 30, 8), 12)
    kc = _rand((1, 2, 30, 8), 13)
    vc = _rand((1, 2, 30, 8), 14)
    full = oracle.attention("causal", qc, kc, vc, 30, 30)
    part = oracle.attention("causal", qc[:, :, -6:], kc, vc, 30, 6)
    np.testing.assert_allclose(part, full[:, :, -6:], atol=1e-12, rtol=0)
    # GQA = MHA with repeat-interleaved kv heads (head h uses kv head h // G)
    mha = oracle.attention("hybrid", q, k.repeat_interleave(2, 1), v.repeat_interleave(2, 1), L, b)
    np.testing.assert_allclose(out, mha, atol=0, rtol=0)


def test_weights_rows_sum_to_one_and_masked_are_zero():
    # With V = identity over the keys, each output row IS the weight row.
    for mode, L, b in (("hybrid", 9, 2), ("hybrid", 8, 3), ("causal", 12, 5), ("decode", 7, 3)):
        rows = 2 * L if mode == "hybrid" else b
        keys = 2 * L if mode == "hybrid" else L
        q = _rand((1, 1, rows, 4), 20)
        k = _rand((1, 1, keys, 4), 21)
        v = torch.eye(keys).reshape(1, 1, keys, keys)
        q4 = torch.nn.functional.pad(q, (0, keys - 4))        # d = keys; zero-pad keeps q.k
        k4 = torch.nn.functional.pad(k, (0, keys - 4))
        W = oracle.attention(mode, q4, k4, v, L, b)[0, 0]
        M = oracle.mask(mode, L, b)
        np.testing.assert_allclose(W.sum(axis=1), 1.0, atol=1e-12, rtol=0)
        assert (W[~M] == 0.0).all()
        assert (W[M] > 0.0).all()


def test_masked_perturbation_changes_nothing():
    L, b = 16, 4
    q, k, v = _hybrid_inputs(L, Hq=2, Hkv=1, seed=30)
    M = oracle.mask("hybrid", L, b)
    base = oracle.attention("hybrid", q, k, v, L, b)
    for qb in range(0, 2 * L, b):
        rows = slice(qb, qb + b)
        seen = M[rows].any(axis=0)
        k2, v2 = k.clone(), v.clone()
        noise = _rand(k.shape, 31 + qb) * 1e4
        k2[:, :, ~torch.as_tensor(seen)] = noise[:, :, ~torch.as_tensor(seen)]
        v2[:, :, ~torch.as_tensor(seen)] = -noise[:, :, ~torch.as_tensor(seen)]
        out = oracle.attention("hybrid", q, k2, v2, L, b)
        assert np.array_equal(out[:, :, rows], base[:, :, rows])


def test_closed_forms():
    L, b = 10, 3
    q, k, _ = _hybrid_inputs(L, seed=40)
    v = torch.full((1, 1, 2 * L, 8), 0.0)
    v[..., :] = torch.arange(8, dtype=torch.float32)           # every value row identical
    out = oracle.attention("hybrid", q, k, v, L, b)
    np.testing.assert_allclose(out, np.broadcast_to(np.arange(8.0), out.shape), atol=1e-12, rtol=0)
    # identical keys -> uniform weights -> mean of the visible value rows
    k1 = torch.ones_like(k) * 0.5
    v1 = _rand((1, 1, 2 * L, 8), 41)
    out = oracle.attention("hybrid", q, k1, v1, L, b)
    M = oracle.mask("hybrid", L, b)
    ref = np.stack([v1[0, 0].numpy()[M[i]].astype(np.float64).mean(axis=0) for i in range(2 * L)])
    np.testing.assert_allclose(out[0, 0], ref, atol=1e-12, rtol=0)


def test_brute_loops_agree():
    L, b, d = 6, 4, 5
    q, k, v = _hybrid_inputs(L, d=d, seed=50)
    out = oracle.attention("hybrid", q, k, v, L, b)[0, 0]
    M = brute.hybrid_mask_enum(L, b)
    ref = brute.attention_loops(q[0, 0].double().tolist(), k[0, 0].double().tolist(),
                                v[0, 0].double().tolist(), M, 1 / math.sqrt(d))
    np.testing.assert_allclose(out, np.array(ref), atol=1e-13, rtol=0)


# ---------------------------------------------------------------- commit

def _commit(logits, masked, tau, k_min, tokens=None):
    G, R, _ = logits.shape
    if tokens is None:
        tokens = np.full((G, R), -7, dtype=np.int64)
    return oracle.commit(logits, masked, tokens, tau, k_min)


def test_commit_uniform_row_probability():
    for V in (1, 2, 4, 1000, 131072):
        lg = np.full((1, 1, V), 0.375, dtype=np.float32)
        _, _, info = _commit(lg, np.ones((1, 1), np.uint8), 0.5, 0)
        assert info["p64"][0, 0] == pytest.approx(1.0 / V, rel=1e-12)
        assert info["argmax"][0, 0] == 0                         # ties -> lowest id


def test_commit_single_peak_closed_form_and_threshold_side():
    V, tau = 1000, 0.85
    for side in (+1e-3, -1e-3):
        target = tau + side
        delta = math.log((V - 1) * target / (1 - target))        # p = 1/(1+(V-1)e^-delta)
        lg = np.zeros((1, 1, V), dtype=np.float32)
        lg[0, 0, 417] = np.float32(delta)
        toks, m, info = _commit(lg, np.ones((1, 1), np.uint8), tau, 0)
        p_closed = 1.0 / (1.0 + (V - 1) * math.exp(-float(np.float32(delta))))
        assert info["p64"][0, 0] == pytest.approx(p_closed, rel=1e-12)
        committed = side > 0
        assert (m[0, 0] == 0) == committed
        assert (toks[0, 0] == 417) == committed


def test_commit_strict_threshold():
    lg = np.zeros((1, 2, 4), dtype=np.float32)                   # p = 0.25 exactly
    t, m, _ = _commit(lg, np.ones((1, 2), np.uint8), 0.25, 0)
    assert m.tolist() == [[1, 1]] and t.tolist() == [[-7, -7]]
    t, m, _ = _commit(lg, np.ones((1, 2), np.uint8), float(np.nextafter(np.float32(0.25), 0)), 0)
    assert m.tolist() == [[0, 0]] and t.tolist() == [[0, 0]]


def test_commit_argmax_ties_lowest_index():
    lg = np.zeros((1, 3, 50), dtype=np.float32)
    lg[0, 0, [7, 9, 30]] = 5.0
    lg[0, 1, [49, 48]] = 2.5
    lg[0, 2, [0, 1]] = 1.0
    t, m, info = _commit(lg, np.ones((1, 3), np.uint8), 0.0, 0)
    assert info["argmax"][0].tolist() == [7, 48, 0]
    assert t[0].tolist() == [7, 48, 0] and m[0].tolist() == [0, 0, 0]


def test_commit_brute_force_subsets():
    rng = np.random.default_rng(123)
    for trial in range(120):
        R = int(rng.integers(1, 13))
        V = int(rng.integers(2, 40))
        lg = (rng.standard_normal((1, R, V)) * rng.uniform(0.5, 6)).astype(np.float32)
        if trial % 5 == 0:                 # plant exact probability ties across rows
            lg[0, R // 2] = lg[0, 0]
        masked = (rng.random((1, R)) < 0.7).astype(np.uint8)
        tau = float(np.float32(rng.uniform(0.05, 0.95)))
        k_min = int(rng.integers(0, R + 3))
        tokens0 = np.full((1, R), -7, dtype=np.int64)
        t, m, info = oracle.commit(lg, masked, tokens0, tau, k_min)
        p32 = [float(np.float32(x)) if masked[0, r] else 0.0 for r, x in enumerate(info["p64"][0])]
        S = brute.commit_subset(p32, masked[0].tolist(), tau, k_min)
        committed = tuple(r for r in range(R) if masked[0, r] and not m[0, r])
        assert committed == S, (trial, committed, S)
        for r in range(R):
            lg64 = lg[0, r].astype(np.float64)
            if r in S:
                assert t[0, r] == int(np.flatnonzero(lg64 == lg64.max())[0])
            else:
                assert t[0, r] == -7 and m[0, r] == masked[0, r]


def test_commit_groups_are_independent_and_kmin_saturates():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((3, 6, 30)).astype(np.float32)
    masked = np.array([[1, 1, 0, 1, 0, 1], [0, 0, 0, 0, 0, 0], [1, 1, 1, 1, 1, 1]], np.uint8)
    t, m, _ = _commit(lg, masked, 0.999, 100)       # k_min above #masked -> all masked commit
    assert not m.any()
    assert (t[1] == -7).all()
    t, m, _ = _commit(lg, masked, 0.999, 1)
    assert (masked - m).sum(axis=1).tolist() == [1, 0, 1]


# ---------------------------------------------------------------- verify

def test_verify_planted_prefix():
    import synth
    g = torch.Generator().manual_seed(99)
    logits, idx = synth.planted_logits(6, 10, 300, 3.0, g, dtype=torch.float32)
    drafts, acc = synth.verify_drafts(idx, seed=3, p=0.3, V=300)
    am, accept = oracle.verify(logits, drafts)
    assert (am == idx.numpy()).all()
    assert accept.tolist() == acc.tolist()
    d2 = idx.numpy().copy()                  # all drafts right -> R
    am, accept = oracle.verify(logits, d2)
    assert accept.tolist() == [10] * 6


def test_tile_class_reduction():
    M = oracle.mask("hybrid", 8, 2)
    assert oracle.tile_class(M, 0, 2, 0, 2) == oracle.FULL
    assert oracle.tile_class(M, 0, 2, 2, 4) == oracle.EMPTY
    assert oracle.tile_class(M, 0, 4, 0, 4) == oracle.PARTIAL
    assert oracle.tile_class(M, 8, 16, 0, 8) == oracle.EMPTY


# ---- row statistics: confidence, argmax, entropy ([DGemma] adaptive stopping)

def test_row_stats_uniform_row():
    V = 1000
    conf, am, ent, mean = oracle.row_stats(np.full((1, 3, V), 0.75, np.float32))
    assert np.allclose(conf, 1.0 / V, rtol=1e-14) and (am == 0).all()
    assert np.allclose(ent, math.log(V), rtol=1e-13) and np.isclose(mean[0], math.log(V), rtol=1e-13)


@pytest.mark.parametrize("V,delta", [(2, 0.5), (1000, 3.0), (131072, 12.0), (50, 40.0)])
def test_row_stats_single_peak_closed_form(V, delta):
    row = np.zeros((1, 1, V), np.float32)
    row[0, 0, V // 3] = delta
    conf, am, ent, _ = oracle.row_stats(row)
    den = 1.0 + (V - 1) * math.exp(-delta)
    p1, q = 1.0 / den, math.exp(-delta) / den
    H = -p1 * math.log(p1) - (V - 1) * q * math.log(q)
    assert am[0, 0] == V // 3 and math.isclose(conf[0, 0], p1, rel_tol=1e-12)
    assert math.isclose(ent[0, 0], H, rel_tol=1e-10, abs_tol=1e-14)


def test_row_stats_two_levels_closed_form():
    V, k, a = 4096, 17, 2.5
    row = np.zeros((1, 1, V), np.float32)
    row[0, 0, 100:100 + k] = a
    _, am, ent, _ = oracle.row_stats(row)
    den = k * math.exp(a) + (V - k)
    pa, p0 = math.exp(a) / den, 1.0 / den
    H = -k * pa * math.log(pa) - (V - k) * p0 * math.log(p0)
    assert am[0, 0] == 100                         # ties: lowest index
    assert math.isclose(ent[0, 0], H, rel_tol=1e-12)


def test_row_stats_matches_scipy_entropy_and_shift_invariance():
    import scipy.special
    import scipy.stats
    g = np.random.default_rng(11)
    lg = (np.round(g.standard_normal((3, 5, 700)) * 3 * 256) / 256).astype(np.float32)   # k/256: shifts exact
    conf, am, ent, mean = oracle.row_stats(lg)
    p = scipy.special.softmax(lg.astype(np.float64), axis=-1)
    assert np.allclose(ent, scipy.stats.entropy(p, axis=-1), rtol=1e-11)
    assert np.allclose(conf, p.max(-1), rtol=1e-12) and (am == lg.argmax(-1)).all()
    assert np.allclose(mean, ent.mean(-1), rtol=1e-12)
    c2, a2, e2, _ = oracle.row_stats(lg + np.float32(64.0))   # exact shift in fp32 at these magnitudes
    assert np.allclose(e2, ent, rtol=1e-11) and (a2 == am).all()


def test_row_stats_masked_rows_and_group_mean():
    g = np.random.default_rng(12)
    lg = g.standard_normal((2, 6, 64)).astype(np.float32)
    m = np.array([[1, 0, 1, 0, 0, 1], [0, 0, 0, 0, 0, 0]], np.uint8)
    conf, am, ent, mean = oracle.row_stats(lg, m)
    _, _, ent_all, _ = oracle.row_stats(lg)
    assert np.isnan(ent[m == 0]).all() and (am[m == 0] == -1).all()
    assert np.allclose(ent[m == 1], ent_all[m == 1], rtol=0, atol=0)
    assert math.isclose(mean[0], ent_all[0, [0, 2, 5]].mean(), rel_tol=1e-14) and mean[1] == 0.0


# ---- backward of the masked attention (training form)

def _torch_attention64(mode, q, k, v, L, block):
    """Masked softmax attention in torch float64 on the oracle's dense mask
    (the mask itself is pinned above); GQA by repeating kv heads."""
    M = torch.from_numpy(oracle.mask(mode, L, block).astype(bool))
    G = q.shape[1] // k.shape[1]
    kk = k.repeat_interleave(G, dim=1)
    vv = v.repeat_interleave(G, dim=1)
    s = (q @ kk.transpose(-1, -2)) / math.sqrt(q.shape[-1])
    s = s.masked_fill(~M, float("-inf"))
    return torch.softmax(s, dim=-1) @ vv, torch.logsumexp(s, dim=-1)


BWD_CASES = [("hybrid", 1, 4, 2, 12, 3, 8), ("hybrid", 2, 2, 1, 10, 4, 16), ("hybrid", 1, 2, 2, 7, 7, 4),
             ("decode", 1, 4, 2, 15, 5, 8), ("causal", 2, 2, 1, 13, 6, 8), ("causal", 1, 2, 2, 9, 9, 4)]


def _bwd_inputs(mode, B, Hq, Hkv, L, blk, d, seed):
    g = torch.Generator().manual_seed(seed)
    rows = 2 * L if mode == "hybrid" else blk
    keys = 2 * L if mode == "hybrid" else L
    mk = lambda *s: torch.randn(*s, generator=g).to(torch.float32)
    return mk(B, Hq, rows, d), mk(B, Hkv, keys, d), mk(B, Hkv, keys, d), mk(B, Hq, rows, d)


@pytest.mark.parametrize("mode,B,Hq,Hkv,L,blk,d", BWD_CASES)
def test_attention_bwd_matches_autograd(mode, B, Hq, Hkv, L, blk, d):
    q, k, v, do = _bwd_inputs(mode, B, Hq, Hkv, L, blk, d, seed=L * 7 + d)
    dq, dk, dv, lse = oracle.attention_bwd(mode, q, k, v, do, L, blk)
    q6, k6, v6 = (t.double().requires_grad_(True) for t in (q, k, v))
    out, lse_t = _torch_attention64(mode, q6, k6, v6, L, blk)
    (out * do.double()).sum().backward()
    assert np.allclose(dq, q6.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dk, k6.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dv, v6.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(lse, lse_t.detach().numpy(), rtol=1e-12)


def test_attention_bwd_finite_differences():
    mode, B, Hq, Hkv, L, blk, d = "hybrid", 1, 2, 1, 6, 2, 4
    q, k, v, do = _bwd_inputs(mode, B, Hq, Hkv, L, blk, d, seed=5)
    dq, dk, dv, _ = oracle.attention_bwd(mode, q, k, v, do, L, blk)
    base = {"q": q.double(), "k": k.double(), "v": v.double()}

    def loss(**kw):
        t = dict(base, **kw)
        out, _ = _torch_attention64(mode, t["q"], t["k"], t["v"], L, blk)
        return float((out * do.double()).sum())

    g = np.random.default_rng(3)
    eps = 1e-6
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        for _ in range(6):
            idx = tuple(int(g.integers(s)) for s in base[name].shape)
            plus, minus = base[name].clone(), base[name].clone()
            plus[idx] += eps
            minus[idx] -= eps
            fd = (loss(**{name: plus}) - loss(**{name: minus})) / (2 * eps)
            assert math.isclose(grad[idx], fd, rel_tol=1e-6, abs_tol=1e-8), (name, idx, grad[idx], fd)


def test_attention_bwd_zero_upstream_rows_send_nothing_to_their_private_keys():
    # x_t keys of block j are seen only by the x_t rows of block j: zero dout
    # there and those keys get no gradient at all.
    mode, L, blk = "hybrid", 8, 2
    q, k, v, do = _bwd_inputs(mode, 1, 2, 1, L, blk, 8, seed=9)
    do[:, :, 2:4] = 0.0                       # x_t rows of block 1
    _, dk, dv, _ = oracle.attention_bwd(mode, q, k, v, do, L, blk)
    assert np.abs(dk[:, :, 2:4]).max() == 0.0 and np.abs(dv[:, :, 2:4]).max() == 0.0
    assert np.abs(dk[:, :, 4:6]).max() > 0.0


# ---- SPRINT sparse prefix retention ([LLaDA] SPRINT)

def _sprint_brute(k, conf, modality, alpha, r_img, r_text):
    """Pure-Python restatement on tiny inputs: norms by loops, then a sort by
    (score descending, position ascending) per modality."""
    B, H, L, d = k.shape
    r = {1: float(np.float32(r_img)), 0: float(np.float32(r_text))}
    a = float(np.float32(alpha))
    out = []
    for b in range(B):
        n = [math.sqrt(sum(float(k[b, h, i, c]) ** 2 for h in range(H) for c in range(d))) for i in range(L)]
        mean = sum(n) / L
        s = [a * n[i] / mean + (1 - a) * float(conf[b, i]) for i in range(L)]
        keep = set()
        for m in (0, 1):
            pos = [i for i in range(L) if int(modality[i]) == m]
            cnt = math.floor(r[m] * len(pos) + 0.5)
            keep.update(sorted(pos, key=lambda i: (-s[i], i))[:cnt])
        out.append(sorted(keep))
    return out


@pytest.mark.parametrize("seed", range(4))
def test_sprint_brute_force(seed):
    g = np.random.default_rng(40 + seed)
    B, H, L, d = 2, 2, 37, 5
    k = g.standard_normal((B, H, L, d)).astype(np.float32) * g.uniform(0.2, 3.0, (1, 1, L, 1)).astype(np.float32)
    conf = g.uniform(0, 1, (B, L)).astype(np.float32)
    mod = (g.uniform(size=L) < 0.6).astype(np.uint8)
    kept, sc, K = oracle.sprint(k, conf, mod, 0.5, 0.8, 1.0)
    ref = _sprint_brute(k, conf, mod, 0.5, 0.8, 1.0)
    for b in range(B):
        assert list(kept[b, :K]) == ref[b] and (kept[b, K:] == -1).all()


def test_sprint_equal_norms_rank_by_confidence_and_ratios():
    L, d = 40, 8
    base = np.arange(1, d + 1, dtype=np.float32)
    k = np.stack([np.roll(base, i) for i in range(L)])[None, None]      # every key has the same norm
    conf = np.linspace(0.0, 1.0, L, dtype=np.float32)[::-1].copy()[None]  # position 0 most confident
    mod = np.array([1] * 30 + [0] * 10, dtype=np.uint8)
    kept, sc, K = oracle.sprint(k, conf, mod, 0.5, 0.8, 1.0)
    assert np.allclose(sc, 0.5 + 0.5 * conf.astype(np.float64), rtol=1e-12)   # I_i = 1
    assert K == 24 + 10 and list(kept[0, :K]) == list(range(24)) + list(range(30, 40))
    kept1, _, K1 = oracle.sprint(k, conf, mod, 0.5, 1.0, 1.0)
    assert K1 == L and list(kept1[0]) == list(range(L))
    kept0, _, K0 = oracle.sprint(k, conf, mod, 0.5, 0.0, 1.0)
    assert K0 == 10 and list(kept0[0, :K0]) == list(range(30, 40))


def test_sprint_equal_confidence_ranks_by_key_norm():
    L = 16
    k = np.zeros((1, 2, L, 4), np.float32)
    norms = np.array([3, 1, 4, 1, 5, 9, 2, 6, 5, 3, 5, 8, 9, 7, 9, 3], np.float32)
    k[0, 0, :, 0] = norms                                                 # one kv head carries the norm
    mod = np.ones(L, np.uint8)
    kept, sc, K = oracle.sprint(k, np.full((1, L), 0.4, np.float32), mod, 0.5, 0.5, 1.0)
    n64 = norms.astype(np.float64)
    assert np.allclose(sc[0], 0.5 * n64 / n64.mean() + 0.5 * float(np.float32(0.4)), rtol=1e-12)
    order = sorted(range(L), key=lambda i: (-norms[i], i))[:K]
    assert K == 8 and list(kept[0, :K]) == sorted(order)                  # ties (the 9s, 5s) by position


# ---- Entropy-bound commit ([DGemma] Schedulers, EntropyBoundScheduler)

def _entropy_commit_brute(logits, masked, bound, temperature, k_min):
    """Restatement with scipy's softmax and entropy, Python sorting and sums."""
    import scipy.special
    import scipy.stats
    G, R, V = logits.shape
    T = float(np.float32(temperature))
    b = float(np.float32(bound))
    committed = np.zeros((G, R), bool)
    for g in range(G):
        rows = [r for r in range(R) if masked[g, r]]
        H = {r: float(scipy.stats.entropy(scipy.special.softmax(logits[g, r].astype(np.float64) / T))) for r in rows}
        order = sorted(rows, key=lambda r: (H[r], r))
        n, acc = 0, 0.0
        for j, r in enumerate(order):
            acc += H[r]
            if acc <= b:
                n = j + 1
            else:
                break
        n = max(n, min(k_min, len(rows)))
        for r in order[:n]:
            committed[g, r] = True
    return committed


@pytest.mark.parametrize("seed", range(5))
def test_entropy_commit_matches_restatement(seed):
    g = np.random.default_rng(70 + seed)
    G, R, V = 3, 9, 50
    logits = (g.standard_normal((G, R, V)) * g.uniform(0.5, 6.0, (G, R, 1))).astype(np.float32)
    masked = (g.uniform(size=(G, R)) < 0.7).astype(np.uint8)
    bound, T, k_min = float(g.uniform(0.5, 8.0)), float(g.choice([0.4, 0.8, 1.0, 1.7])), int(g.integers(0, 3))
    tokens = np.full((G, R), -1, np.int64)
    t, m, ent, am = oracle.commit_entropy(logits, masked, tokens, bound, T, k_min)
    want = _entropy_commit_brute(logits, masked, bound, T, k_min)
    assert np.array_equal((masked == 1) & (m == 0), want)
    assert np.array_equal(t[want], logits.argmax(-1)[want])          # argmax: lowest index of the max
    assert (t[~want] == -1).all() and (m[~want] == masked[~want]).all()


def test_entropy_commit_temperature_and_closed_forms():
    g = np.random.default_rng(80)
    G, R, V = 2, 6, 64
    logits = (g.standard_normal((G, R, V)) * 3).astype(np.float32)
    masked = np.ones((G, R), np.uint8)
    tok = np.full((G, R), -1, np.int64)
    # softmax(l / 0.5) is softmax((2 l) / 1): same entropies
    _, _, e_half, _ = oracle.commit_entropy(logits, masked, tok, 1.0, 0.5, 0)
    _, _, e_two, _ = oracle.commit_entropy(2 * logits, masked, tok, 1.0, 1.0, 0)
    assert np.allclose(e_half, e_two, rtol=1e-14, atol=0)
    # uniform rows: H = log V at any temperature; ties go to the lower row
    uni = np.zeros((1, 5, V), np.float32)
    m1 = np.ones((1, 5), np.uint8)
    t, m, e, _ = oracle.commit_entropy(uni, m1, np.full((1, 5), -1, np.int64), 2.5 * np.log(V), 0.8, 0)
    assert np.allclose(e, np.log(V), rtol=1e-14)
    assert list(m[0]) == [0, 0, 1, 1, 1] and list(t[0, :2]) == [0, 0]
    # bound below every entropy: exactly min(k_min, #masked) rows, the lowest-entropy ones
    peaked = np.zeros((1, 4, V), np.float32)
    for r, gap in enumerate([1.0, 9.0, 3.0, 30.0]):
        peaked[0, r, 7 + r] = gap                                     # larger gap, lower entropy
    _, m, e, _ = oracle.commit_entropy(peaked, np.ones((1, 4), np.uint8), np.full((1, 4), -1, np.int64), -1.0, 1.0, 2)
    assert list(m[0]) == [1, 0, 1, 0]
    _, m, _, _ = oracle.commit_entropy(peaked, np.ones((1, 4), np.uint8), np.full((1, 4), -1, np.int64), -1.0, 1.0, 0)
    assert list(m[0]) == [1, 1, 1, 1]
    # a bound above the total commits every masked row
    _, m, e, _ = oracle.commit_entropy(peaked, np.array([[1, 0, 1, 1]], np.uint8), np.full((1, 4), -1, np.int64),
                                       1e9, 1.0, 0)
    assert list(m[0]) == [0, 0, 0, 0] and np.isnan(e[0, 1])
    # single-peak closed form: H = log Z - (gap e^gap) / Z, Z = e^gap + V - 1
    gap = 3.0
    Z = np.exp(gap) + V - 1
    assert abs(e[0, 2] - (np.log(Z) - gap * np.exp(gap) / Z)) < 1e-12


def test_adaptive_stop_steps():
    G, R = 3, 4
    prev = np.full((G, R), -1, np.int64)
    stable = np.zeros(G, np.int64)
    frozen = np.zeros(G, np.uint8)
    a0 = np.arange(G * R).reshape(G, R)
    low, high = np.array([0.001, 0.001, 0.1]), np.array([0.001, 0.01, 0.001])
    # first step: prev unset, nothing is stable yet
    prev, stable, frozen = oracle.adaptive_stop_step(a0, prev, stable, frozen, low, 1, 0.005)
    assert list(stable) == [0, 0, 0] and list(frozen) == [0, 0, 0] and np.array_equal(prev, a0)
    # unchanged argmax: stable 1; example 0 freezes (entropy below), 1 not (0.01), 2 not (0.1)
    a1 = a0.copy()
    a1[1, 3] = a0[1, 3]                                               # unchanged
    prev, stable, frozen = oracle.adaptive_stop_step(a1, prev, stable, frozen, high * 0 + [0.001, 0.01, 0.1], 1, 0.005)
    assert list(stable) == [1, 1, 1] and list(frozen) == [1, 0, 0]
    # example 1 changes one position: counter resets; example 2 stays and its entropy drops
    a2 = a1.copy()
    a2[1, 0] += 100
    a2[0, 0] += 100                                                   # example 0 is frozen: ignored
    prev, stable, frozen = oracle.adaptive_stop_step(a2, prev, stable, frozen, np.array([0.5, 0.001, 0.001]), 1, 0.005)
    assert list(stable) == [1, 0, 2] and list(frozen) == [1, 0, 1]
    assert prev[0, 0] == a1[0, 0] and prev[1, 0] == a2[1, 0]
    # a threshold of 2 needs two unchanged steps; equality with the confidence threshold does not freeze
    p, s, f = oracle.adaptive_stop_step(a0[:1], a0[:1], [0], [0], [0.0], 2, 0.005)
    assert list(s) == [1] and list(f) == [0]
    p, s, f = oracle.adaptive_stop_step(a0[:1], p, s, f, [0.0], 2, 0.005)
    assert list(s) == [2] and list(f) == [1]
    p, s, f = oracle.adaptive_stop_step(a0[:1], a0[:1], [5], [0], [np.float32(0.005)], 1, 0.005)
    assert list(f) == [0]
