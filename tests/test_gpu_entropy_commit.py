"""GPU parity of the entropy-bound commit and of adaptive stopping ([DGemma]
"Schedulers" and "Adaptive stopping") against the oracle.

The kernels compute each row's entropy in fp32 (error below 2^-16 (1 + H)
nats, as for the row statistics) and sum the ranked entropies in fp32.  The
committed sets must equal the oracle's exactly once the bound keeps clear of
every partial sum by the accumulated tolerance and the rows on either side of
each group's cut differ by more than theirs; the bound of each case is the
first candidate that satisfies this (the candidates are fixed, so the case is
deterministic).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dev, say

pytestmark = pytest.mark.gpu

bda = pytest.importorskip("block_masked_attention_amd")


def _tol(h):
    return 2.0 ** -16 * (1.0 + h)


def _clear(ent, masked, bound, k_min):
    """True when no fp32 rounding of the entropies or their sums can change
    the committed set for this bound."""
    b = float(np.float32(bound))
    for g in range(ent.shape[0]):
        rows = np.nonzero(masked[g])[0]
        if len(rows) == 0:
            continue
        h = np.array(sorted(ent[g, rows]))
        s = np.cumsum(h)
        tol = np.cumsum(_tol(h)) + 1e-6 * np.abs(s)
        if np.any(np.abs(s - b) <= tol):
            return False
        n = max(int(np.count_nonzero(s <= b)), min(k_min, len(rows)))
        if 0 < n < len(h) and h[n] - h[n - 1] <= _tol(h[n]) + _tol(h[n - 1]):
            return False
    return True


def _pick_bound(ent, masked, k_min):
    sums = [np.sort(ent[g, np.nonzero(masked[g])[0]]).sum() for g in range(ent.shape[0])]
    top = max(sums) if sums else 1.0
    for frac in (0.31, 0.17, 0.47, 0.09, 0.63, 0.23, 0.39, 0.55, 0.05, 0.71):
        b = float(np.float32(frac * top))
        if _clear(ent, masked, b, k_min):
            return b
    raise AssertionError("no clear bound among the candidates")


def _run(logits, masked, bound, temperature, k_min, what):
    G, R, V = logits.shape
    tokens = torch.full((G, R), -1, dtype=torch.int64)
    if bound is None:
        _, _, ent, _ = oracle.commit_entropy(logits.float(), masked.numpy(), tokens.numpy(), 0.0, temperature, 0)
        bound = _pick_bound(ent, masked.numpy(), k_min)
    rt, rm, ent, _ = oracle.commit_entropy(logits.float(), masked.numpy(), tokens.numpy(), bound, temperature, k_min)
    assert _clear(ent, masked.numpy(), bound, k_min), f"{what}: bound too close to a decision"
    gt, gm = tokens.to(dev()), masked.clone().to(dev())
    bda.commit_entropy(logits.to(dev()), gt, gm, bound, temperature, k_min)
    torch.cuda.synchronize()
    n = int(masked.sum()) - int(rm.sum())
    say(f"[entropy commit] {what}: G={G} R={R} V={V} T={temperature} bound={bound:.4f} k_min={k_min}: "
        f"{n} of {int(masked.sum())} masked rows committed")
    assert np.array_equal(gm.cpu().numpy(), rm), f"{what}: committed rows differ"
    assert np.array_equal(gt.cpu().numpy(), rt), f"{what}: tokens differ"
    return n


@pytest.mark.parametrize("case", [
    # (seed, G, R, V, temperature, k_min, dtype)
    (1, 8, 28, 32768, 1.0, 1, torch.bfloat16),
    (2, 8, 28, 32768, 0.8, 1, torch.bfloat16),
    (3, 4, 37, 1000, 0.4, 2, torch.float32),      # ragged rows and vocabulary, fp32 logits
    (4, 3, 256, 4096, 2.0, 0, torch.bfloat16),
    (5, 2, 1, 50000, 1.0, 1, torch.bfloat16),     # one row per group
    (8, 3, 64, 2048, 1.0, 3, torch.bfloat16),     # largest group ranked by one wavefront
    (9, 2, 65, 2048, 0.7, 1, torch.bfloat16),     # smallest group ranked by the whole workgroup
])
def test_entropy_commit(case):
    seed, G, R, V, T, k_min, dt = case
    logits = synth.spread_logits(seed, G, R, V, dtype=dt)
    g = torch.Generator().manual_seed(900 + seed)
    masked = (torch.rand(G, R, generator=g) < 0.75).to(torch.uint8)
    _run(logits, masked, None, T, k_min, f"case {seed}")


def test_entropy_commit_decode_workload():
    """The decode workload's logits [32, 28, 131072] bf16, every row masked."""
    logits, _, masked = synth.commit_logits()
    _run(logits, masked, None, 1.0, 1, "decode workload")


def test_entropy_commit_bounds():
    logits = synth.spread_logits(7, 4, 28, 4096)
    masked = torch.ones(4, 28, dtype=torch.uint8)
    assert _run(logits, masked, -1.0, 1.0, 3, "bound below every entropy") == 4 * 3
    assert _run(logits, masked, -1.0, 1.0, 0, "nothing allowed") == 0
    assert _run(logits, masked, 1e9, 1.0, 0, "bound above the total") == 4 * 28
    empty = torch.zeros(4, 28, dtype=torch.uint8)
    assert _run(logits, empty, 5.0, 1.0, 2, "nothing masked") == 0


def test_adaptive_stop_sequence():
    """Step by step against the oracle: argmax sequences where examples keep,
    change or partly change their predictions, mean entropies around the
    threshold, stability thresholds 1 and 2."""
    G, R = 6, 28
    g = torch.Generator().manual_seed(321)
    for stab in (1, 2):
        prev = torch.full((G, R), -1, dtype=torch.int64)
        stable = torch.zeros(G, dtype=torch.int32)
        frozen = torch.zeros(G, dtype=torch.uint8)
        gp, gs, gf = prev.to(dev()), stable.to(dev()), frozen.to(dev())
        nf = torch.zeros(1, dtype=torch.int32, device=dev())
        cur = torch.randint(0, 1000, (G, R), generator=g)
        for step in range(8):
            change = torch.rand(G, generator=g) < torch.tensor([0.0, 0.2, 0.5, 0.8, 0.1, 0.3])
            pos = torch.randint(0, R, (G,), generator=g)
            for e in range(G):
                if change[e]:
                    cur[e, pos[e]] = (cur[e, pos[e]] + 1) % 1000
            ment = (torch.rand(G, generator=g) * 0.01).to(torch.float32)
            prev, stable, frozen = (torch.from_numpy(x) for x in oracle.adaptive_stop_step(
                cur.numpy(), prev.numpy(), stable.numpy(), frozen.numpy(), ment.numpy(), stab, 0.005))
            bda.adaptive_stop(cur.to(dev()), gp, gs, gf, ment.to(dev()), stab, 0.005, n_frozen=nf)
            torch.cuda.synchronize()
            assert torch.equal(gp.cpu(), prev), f"step {step}: prev"
            assert torch.equal(gs.cpu().long(), stable.long()), f"step {step}: stable"
            assert torch.equal(gf.cpu(), frozen.to(torch.uint8)), f"step {step}: frozen"
            assert int(nf.item()) == int(frozen.sum())
        say(f"[adaptive stop] stability {stab}: frozen after 8 steps {frozen.tolist()}")
