"""GPU parity of the fused row statistics + confidence commit
(bda_row_stats_commit): one pass over a denoising step's logits for the
stopping statistics ([DGemma] "Adaptive stopping") and the commit ([DGemma]
"Schedulers"; [LLaDA] SPRINT).

Each case checks two things.  (1) The fused call returns, bit for bit, what
bda_row_stats over every row followed by bda_commit return on the same
inputs.  (2) Against the oracle: committed tokens and commit masks exactly
(decisions outside the guard band, as in the commit tests), argmax exactly,
and confidence, entropy and group mean entropy within the row-statistics
bounds (relative 2^-16 for the confidence, 2^-16 (1 + H) for entropies).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from commit_util import close_rows, guarded
from gpu_util import dev, say

pytestmark = pytest.mark.gpu

bda = pytest.importorskip("block_masked_attention_amd")

TOL = 2.0 ** -16


def _bits_equal(a, b):
    if a.dtype.is_floating_point:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def _run(logits, masked, tau, k_min, what):
    G, R, _ = logits.shape
    lg = logits.to(dev())
    tokens = torch.full((G, R), -1, dtype=torch.int64)
    # separate calls
    t1, m1 = tokens.clone().to(dev()), masked.clone().to(dev())
    sep = bda.row_stats(lg)
    bda.commit(lg, t1, m1, tau, k_min)
    # fused call
    t2, m2 = tokens.clone().to(dev()), masked.clone().to(dev())
    fused = bda.row_stats_commit(lg, t2, m2, tau, k_min)
    torch.cuda.synchronize()
    names = ("conf", "argmax", "entropy", "mean entropy")
    for n, a, b in zip(names, sep, fused):
        assert _bits_equal(a, b), f"{what}: {n} differs from the separate row statistics call"
    assert torch.equal(t1, t2) and torch.equal(m1, m2), f"{what}: commit differs from the separate commit call"
    # oracle
    rt, rm, _ = oracle.commit(logits, masked.numpy(), tokens.numpy(), tau, k_min)
    assert np.array_equal(m2.cpu().numpy(), rm), f"{what}: commit masks differ from the oracle"
    assert np.array_equal(t2.cpu().numpy(), rt), f"{what}: committed tokens differ from the oracle"
    rc, ra, re, rmean = oracle.row_stats(logits, None)
    conf, am, ent, mean = (x.cpu().numpy() for x in fused)
    assert (am == ra).all(), f"{what}: argmax differs from the oracle"
    ce = np.abs(conf - rc) / rc if rc.size else np.zeros(1)
    ee = np.abs(ent - re) / (1.0 + re) if re.size else np.zeros(1)
    me = np.abs(mean - rmean) / (1.0 + rmean)
    say(f"[stats+commit] {what}: committed {int((masked.numpy() - rm).sum())}, conf rel err {ce.max():.2e}, "
        f"entropy err/(1+H) {ee.max():.2e}, mean {me.max():.2e}")
    assert (ce <= TOL).all() and (ee <= TOL).all() and (me <= TOL).all(), f"{what}: statistics out of tolerance"


def test_decode_workload():
    logits, idx, masked = synth.commit_logits()
    logits, _ = guarded(logits, idx, masked, 0.85, 1, 3.0, seed=4)
    _run(logits, masked, 0.85, 1, "decode commit 32x28x131072")


@pytest.mark.parametrize("step", range(2))
def test_canvas_step(step):
    _, _, _, logits, idx = synth.multimodal_step(step, 28, B=2)
    masked = torch.ones(2, 28, dtype=torch.uint8)
    masked[:, : 9 * step] = 0
    logits, _ = guarded(logits, idx, masked, 0.9, 1, 3.0, seed=70 + step)
    _run(logits, masked, 0.9, 1, f"canvas step {step}")


def _uniform(G, R, V, seed, dtype, scale):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(G, R, V, generator=g) * scale).to(dtype)


@pytest.mark.parametrize("G,R,V,dtype,tau,k_min", [
    (3, 12, 1001, torch.bfloat16, 0.3, 2),     # V not a multiple of 8: scalar path
    (1, 7, 1, torch.bfloat16, 0.5, 0),         # V = 1: p = 1, entropy 0
    (4, 40, 20000, torch.float32, 0.99, 5),    # two vocabulary chunks, fallback only
    (2, 300, 64, torch.bfloat16, 0.2, 3),      # R above the finalize block size
    (2, 2100, 64, torch.bfloat16, 0.2, 3),     # R above the rows the finalize keeps in LDS
])
def test_edges(G, R, V, dtype, tau, k_min):
    g = torch.Generator().manual_seed(V + R)
    masked = (torch.rand(G, R, generator=g) < 0.75).to(torch.uint8)
    tokens = torch.full((G, R), -1, dtype=torch.int64)
    for attempt in range(16):
        logits = _uniform(G, R, V, G * 1000 + R + V + 7919 * attempt, dtype, 2.0 if V > 4 else 0.7)
        _, _, info = oracle.commit(logits, masked.numpy(), tokens.numpy(), tau, k_min)
        if V == 1 or not close_rows(info, masked.numpy(), tau, k_min):
            break
    else:
        raise AssertionError("no seed left the guard band")
    _run(logits, masked, tau, k_min, f"G={G} R={R} V={V} {dtype}")


def test_banned_tokens():
    """-inf logits: single banned ids in every row and a whole banned
    16384-entry chunk in some rows."""
    G, R, V = 2, 6, 40000
    logits = _uniform(G, R, V, 5, torch.float32, 2.0)
    logits[:, :, 7] = -float("inf")
    logits[0, ::2, 16384:32768] = -float("inf")
    logits[0, 3, 123] = 30.0                    # one confident row per group: no fallback ranking
    logits[1, 1, 39000] = 30.0
    masked = torch.ones(G, R, dtype=torch.uint8)
    for dtype in (torch.float32, torch.bfloat16):
        _run(logits.to(dtype), masked, 0.9, 1, f"banned ids {dtype}")


def test_no_rows_and_errors():
    lg = torch.zeros(2, 0, 10, dtype=torch.bfloat16, device=dev())
    t = torch.zeros(2, 0, dtype=torch.int64, device=dev())
    m = torch.zeros(2, 0, dtype=torch.uint8, device=dev())
    conf, am, ent, mean = bda.row_stats_commit(lg, t, m, 0.9, 1)
    torch.cuda.synchronize()
    assert mean.cpu().tolist() == [0.0, 0.0]
    lg = torch.zeros(1, 3, 10, dtype=torch.bfloat16, device=dev())
    t = torch.zeros(1, 3, dtype=torch.int64, device=dev())
    m = torch.ones(1, 3, dtype=torch.uint8, device=dev())
    with pytest.raises(bda.BdaError):
        bda.row_stats_commit(lg, t, m, float("nan"), 1)
    with pytest.raises(bda.BdaError):
        bda.row_stats_commit(lg, t, m, 0.5, -1)
