"""GPU parity of the per-row statistics pass (confidence, argmax, entropy,
group mean entropy) against the fp64 oracle.

argmax is compared exactly.  conf and entropy are fp32 results of sums over
the vocabulary; the bound used is derived in the design notes: each lane sums
at most 64 terms, merges are pairwise over <= 2^11 partials, and v_exp_f32 is
within 1 ulp, so the relative error of Z and T stays below ~2^-16; the
entropy log Z - T/Z then carries at most ~2^-16 * (1 + H) absolute error.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dev, say

pytestmark = pytest.mark.gpu

bda = pytest.importorskip("block_masked_attention_amd")

CONF_RTOL = 2.0 ** -16
ENT_TOL = 2.0 ** -16


def _compare(logits, masked, what):
    conf, am, ent, mean = bda.row_stats(logits.to(dev()), None if masked is None else masked.to(dev()))
    torch.cuda.synchronize()
    rc, ra, re, rm = oracle.row_stats(logits, None if masked is None else masked.numpy())
    sel = np.ones(rc.shape, bool) if masked is None else masked.numpy() != 0
    conf, am, ent, mean = conf.cpu().numpy(), am.cpu().numpy(), ent.cpu().numpy(), mean.cpu().numpy()
    assert (am[sel] == ra[sel]).all(), f"{what}: argmax differs"
    assert (am[~sel] == -1).all() and np.isnan(ent[~sel]).all(), f"{what}: unselected rows written"
    ce = np.abs(conf[sel] - rc[sel]) / rc[sel]
    ee = np.abs(ent[sel] - re[sel]) / (1.0 + re[sel])
    me = np.abs(mean - rm) / (1.0 + rm)
    say(f"[stats] {what}: max conf rel err {ce.max() if ce.size else 0:.2e}, "
        f"max entropy err/(1+H) {ee.max() if ee.size else 0:.2e}, mean {me.max():.2e}")
    assert (ce <= CONF_RTOL).all(), f"{what}: conf out of tolerance"
    assert (ee <= ENT_TOL).all(), f"{what}: entropy out of tolerance"
    assert (me <= ENT_TOL).all(), f"{what}: group mean entropy out of tolerance"


def test_stats_decode_logits_full():
    logits, _, _ = synth.commit_logits()
    _compare(logits, None, "decode logits 32x28x131072 bf16")


def test_stats_decode_logits_masked_subset():
    logits, _, _ = synth.commit_logits()
    g = torch.Generator().manual_seed(21)
    masked = (torch.rand(32, 28, generator=g) < 0.4).to(torch.uint8)
    masked[3] = 0                                   # a group with no selected row: mean 0
    _compare(logits, masked, "decode logits, 40% of rows selected")


@pytest.mark.parametrize("G,R,V,dtype", [
    (3, 12, 1001, torch.bfloat16),    # V not a multiple of 8: scalar path
    (2, 5, 3, torch.float32),
    (1, 7, 1, torch.bfloat16),        # V = 1: conf 1, entropy 0
    (4, 40, 20000, torch.float32),    # two vocabulary chunks, ragged second chunk
    (2, 300, 64, torch.bfloat16),     # R above the finalize block size
])
def test_stats_edges(G, R, V, dtype):
    g = torch.Generator().manual_seed(G * 100 + R + V)
    logits = (torch.randn(G, R, V, generator=g) * 2.0).to(dtype)
    _compare(logits, None, f"[{G},{R},{V}] {dtype}")


def test_stats_closed_forms_on_gpu():
    V = 131072
    lg = torch.zeros(2, 3, V, dtype=torch.bfloat16)
    lg[1, :, 777] = 10.0                            # single peak rows
    conf, am, ent, _ = bda.row_stats(lg.to(dev()))
    torch.cuda.synchronize()
    ent = ent.cpu().numpy()
    assert np.allclose(ent[0], math.log(V), rtol=ENT_TOL)
    den = 1.0 + (V - 1) * math.exp(-10.0)
    p1, q = 1.0 / den, math.exp(-10.0) / den
    H = -p1 * math.log(p1) - (V - 1) * q * math.log(q)
    assert np.allclose(ent[1], H, rtol=0, atol=ENT_TOL * (1 + H))
    assert (am.cpu().numpy()[0] == 0).all() and (am.cpu().numpy()[1] == 777).all()
