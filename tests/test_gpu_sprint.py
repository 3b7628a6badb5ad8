"""GPU parity of SPRINT prefix pruning ([LLaDA] SPRINT) against the fp64 oracle.

The kernels compute key norms, the mean norm and the scores in fp32; the
oracle in fp64.  Scores must agree within SCORE_TOL (a few fp32 ulps of a
score near 1).  The kept sets must be equal, except for positions whose
oracle score lies within SCORE_TOL of the cut of their modality (the
count-th best score), where fp32 rounding may legitimately decide; the GPU's
own selection must in any case be exactly the top of its own scores
(score descending, position ascending) per modality.  Gathered K/V rows must
be bit-identical to the rows the kept list names, and decode attention over
the pruned cache must match the oracle's over the oracle's pruned cache.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close_attn, dev, sample_rows, say

pytestmark = pytest.mark.gpu

bda = pytest.importorskip("block_masked_attention_amd")

SCORE_TOL = 4e-6


def _check(k, v, conf, mod, alpha, r_img, r_text, what, gather=True):
    B, H, L, d = k.shape
    say(f"[sprint] {what}: B={B} Hkv={H} L={L} d={d} alpha={alpha} r_img={r_img} r_text={r_text}")
    ko, vo, kept, sc = bda.sprint_prune(k.to(dev()), v.to(dev()), conf.to(dev()), mod.to(dev()), alpha, r_img,
                                        r_text, gather=gather, scores=True)
    torch.cuda.synchronize()
    rk, rs, K = oracle.sprint(k, conf, mod.numpy(), alpha, r_img, r_text)
    gk, gs = kept.cpu().numpy().astype(np.int64), sc.cpu().numpy().astype(np.float64)
    md = mod.numpy().astype(bool)
    err = np.abs(gs - rs)
    assert err.max() <= SCORE_TOL, f"{what}: score error {err.max():.3e}"
    assert K == bda.sprint_kept_count(int(md.sum()), int((~md).sum()), r_img, r_text)
    exact = True
    for b in range(B):
        row = gk[b]
        assert (row[K:] == -1).all(), f"{what}: batch {b} padding"
        sel = row[:K]
        assert (np.diff(sel) > 0).all() and sel.min(initial=0) >= 0 and sel.max(initial=0) < L
        # the GPU's selection is the top of its own scores per modality
        for m in (False, True):
            pos = np.nonzero(md == m)[0]
            cnt = int(np.count_nonzero(md[sel] == m))
            order = sorted(pos, key=lambda i: (-np.float32(gs[b, i]), i))
            assert sorted(order[:cnt]) == list(sel[md[sel] == m]), f"{what}: batch {b} not the top of its scores"
        # against the oracle, up to the guard band at the cut
        diff = set(sel.tolist()) ^ set(rk[b, :K].tolist())
        if diff:
            exact = False
            for i in diff:
                m = md[i]
                pos = np.nonzero(md == m)[0]
                cnt = int(np.count_nonzero(md[rk[b, :K]] == m))
                cut = np.sort(rs[b, pos])[::-1][cnt - 1] if cnt else np.inf
                assert abs(rs[b, i] - cut) <= SCORE_TOL, f"{what}: batch {b} position {i} kept set differs"
    if gather:
        assert tuple(ko.shape) == (B, H, K, d)
        ko_c, vo_c = ko.cpu(), vo.cpu()
        for b in range(B):
            idx = torch.from_numpy(gk[b, :K])
            assert torch.equal(ko_c[b].view(torch.int16), k[b][:, idx].view(torch.int16)), f"{what}: k rows"
            assert torch.equal(vo_c[b].view(torch.int16), v[b][:, idx].view(torch.int16)), f"{what}: v rows"
    say(f"[sprint] {what}: K={K} max score err {err.max():.2e} kept sets {'equal' if exact else 'equal up to the cut'}")
    return ko, vo, rk, K, exact


def test_sprint_multimodal_prefix_and_decode():
    """The 4096-position image+text prefix (3080 image, 1016 text), then one
    decode step of a 28-query block over the pruned cache."""
    k, v, conf = synth.sprint_prefix()
    mod = synth.prefix_modality()
    ko, vo, rk, K, exact = _check(k, v, conf, mod, 0.5, 0.8, 1.0, "multimodal prefix")
    assert K == 2464 + 1016 and exact
    B, H = k.shape[:2]
    n, Hq = 28, 32
    q, kb, vb, _, _ = synth.multimodal_step(0, n, B=B, Hq=Hq, Hkv=H, d=k.shape[3])
    kc = torch.cat([ko, kb.to(dev())], dim=2)
    vc = torch.cat([vo, vb.to(dev())], dim=2)
    out = bda.attn_fwd(q.to(dev()), kc, vc, "decode", n)
    torch.cuda.synchronize()
    kr = torch.cat([torch.stack([k[b][:, torch.from_numpy(rk[b, :K])] for b in range(B)]), kb], dim=2)
    vr = torch.cat([torch.stack([v[b][:, torch.from_numpy(rk[b, :K])] for b in range(B)]), vb], dim=2)
    sel = sample_rows(B, Hq, n, 24, seed=77, must=[(0, 0, 0), (B - 1, Hq - 1, n - 1)])
    got = np.stack([out[b, h, i].float().cpu().numpy() for (b, h, i) in sel])
    ref = oracle.attention("decode", q, kr, vr, K + n, n, sel=sel)
    assert_close_attn(got, ref, "decode over the pruned cache")


@pytest.mark.parametrize("case", [
    # (seed, B, Hkv, L, d, alpha, r_img, r_text, p_image)
    (1, 3, 2, 37, 64, 0.5, 0.35, 0.65, 0.6),     # ragged, tiny
    (2, 2, 4, 5000, 32, 0.3, 0.8, 1.0, 0.7),     # non-power-of-two L
    (3, 1, 1, 1, 128, 0.5, 0.8, 1.0, 1.0),       # one position
    (4, 2, 8, 1024, 128, 0.0, 0.5, 0.5, 0.5),    # confidence only
    (5, 2, 8, 1024, 128, 1.0, 0.5, 0.5, 0.5),    # key norm only
    (6, 2, 2, 700, 64, 0.5, 0.0, 1.0, 0.8),      # drop every image position
    (7, 2, 2, 700, 64, 0.5, 1.0, 1.0, 0.8),      # keep everything
    (8, 2, 2, 513, 64, 0.5, 0.8, 0.5, 0.0),      # text only
    (9, 1, 8, 16384, 128, 0.5, 0.8, 1.0, 0.75),  # largest supported L
])
def test_sprint_cases(case):
    seed, B, H, L, d, alpha, r_img, r_text, p_img = case
    k, v, conf = synth.sprint_prefix(seed=seed, B=B, Hkv=H, d=d, L=L)
    g = torch.Generator().manual_seed(500 + seed)
    mod = (torch.rand(L, generator=g) < p_img).to(torch.uint8)
    ko, vo, rk, K, _ = _check(k, v, conf, mod, alpha, r_img, r_text, f"case {seed}")
    if r_img == 1.0 and r_text == 1.0:
        assert K == L and torch.equal(ko.cpu().view(torch.int16), k.view(torch.int16))


def test_sprint_kept_only_and_repeat():
    """gather=False writes only the kept list; a second call on the same
    workspace gives the same answer."""
    k, v, conf = synth.sprint_prefix(seed=11, B=2, Hkv=4, d=64, L=900)
    mod = (torch.arange(900) % 3 != 0).to(torch.uint8)
    _, _, kept1, _ = bda.sprint_prune(k.to(dev()), v.to(dev()), conf.to(dev()), mod.to(dev()), gather=False)
    ws = torch.empty(int(bda.lib.bda_sprint_workspace_bytes(2, 900)), dtype=torch.uint8, device=dev())
    _, _, kept2, _ = bda.sprint_prune(k.to(dev()), v.to(dev()), conf.to(dev()), mod.to(dev()), workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(kept1, kept2)
    rk = oracle.sprint(k, conf, mod.numpy())[0]
    assert np.array_equal(kept1.cpu().numpy(), rk)
