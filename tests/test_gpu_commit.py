"""GPU parity of the commit and verify kernels against the oracle: committed
token ids, commit masks, argmaxes and accept lengths must be bit-identical.

Threshold and fallback-ranking decisions are compared only where the oracle's
fp64 probability is more than GUARD away from the threshold / from the next
candidate; generated rows inside that band are redrawn (seeded) before the
comparison, and the tiny fixed-seed case instead asserts its margin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from commit_util import close_rows as _close_rows
from commit_util import guarded as _guarded
from gpu_util import GUARD, dev, say

pytestmark = pytest.mark.gpu

bda = pytest.importorskip("block_masked_attention_amd")


def _gpu_commit(logits, masked, tokens, tau, k_min, workspace=None):
    t = tokens.clone().to(dev())
    m = masked.clone().to(dev())
    bda.commit(logits.to(dev()), t, m, tau, k_min, workspace=workspace)
    torch.cuda.synchronize()
    return t.cpu(), m.cpu()


def _check(logits, masked, tau, k_min, what, workspace=None):
    tokens = torch.full(masked.shape, -1, dtype=torch.int64)
    rt, rm, info = oracle.commit(logits, masked.numpy(), tokens.numpy(), tau, k_min)
    gt, gm = _gpu_commit(logits, masked, tokens, tau, k_min, workspace)
    assert np.array_equal(gm.numpy(), rm), f"{what}: commit masks differ"
    assert np.array_equal(gt.numpy(), rt), f"{what}: committed tokens differ"
    return rt, rm, info


def test_tiny_commit_fp32():
    _, logits, masked = synth.tiny()
    tau, k_min = 0.85, 1
    tokens = torch.full(masked.shape, -1, dtype=torch.int64)
    _, _, info = oracle.commit(logits, masked.numpy(), tokens.numpy(), tau, k_min)
    gap = float(info["gap"][0])
    say(f"[commit tiny] fallback gap {gap:.3e}, max p {np.nanmax(info['p64']):.4f}")
    assert gap > GUARD, "tiny case decision inside the guard band; parity not well-posed"
    rt, rm, _ = _check(logits, masked, tau, k_min, "tiny")
    assert int((masked.numpy() - rm).sum()) == 1          # only the fallback commits


def test_decode_commit_full():
    logits, idx, masked = synth.commit_logits()
    logits, info = _guarded(logits, idx, masked, 0.85, 1, 3.0, seed=4)
    say(f"[commit full] pass rate {float((info['p64'] > 0.85).mean()):.3f}")
    rt, rm, _ = _check(logits, masked, 0.85, 1, "decode commit 32x28x131072")
    committed = masked.numpy() - rm
    assert committed.sum() > 0
    assert (rt[committed == 1] == idx.numpy()[committed == 1]).all()   # planted peak wins


@pytest.mark.parametrize("step", range(3))
def test_canvas_commit_steps(step):
    """Per-step canvas commit, threshold 0.9, with earlier commits applied."""
    _, _, _, logits, idx = synth.multimodal_step(step, 28, B=2)
    masked = torch.ones(2, 28, dtype=torch.uint8)
    masked[:, : 7 * step] = 0
    logits, _ = _guarded(logits, idx, masked, 0.9, 1, 3.0, seed=50 + step)
    _check(logits, masked, 0.9, 1, f"canvas step {step}")


def _uniform(G, R, V, seed, dtype, scale=2.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(G, R, V, generator=g) * scale).to(dtype)


@pytest.mark.parametrize("G,R,V,dtype,tau,k_min", [
    (3, 12, 1001, torch.bfloat16, 0.3, 2),     # V not a multiple of 8: scalar path
    (2, 5, 3, torch.float32, 0.5, 1),
    (1, 7, 1, torch.bfloat16, 0.5, 0),         # V = 1: p = 1 everywhere
    (4, 40, 20000, torch.float32, 0.99, 5),    # two vocabulary chunks, fallback only
    (2, 300, 64, torch.bfloat16, 0.2, 3),      # R above the finalize block size
    (2, 2100, 64, torch.bfloat16, 0.2, 3),     # R above the rows the finalize keeps in LDS
    (2, 9, 4096, torch.bfloat16, 0.0, 0),      # tau = 0: every masked row passes
    (2, 9, 4096, torch.bfloat16, 1.0, 100),    # nothing passes, k_min > #masked
])
def test_commit_edges(G, R, V, dtype, tau, k_min):
    g = torch.Generator().manual_seed(V)
    masked = (torch.rand(G, R, generator=g) < 0.75).to(torch.uint8)
    tokens = torch.full((G, R), -1, dtype=torch.int64)
    for attempt in range(16):    # deterministic re-seeding until no decision is inside the band
        logits = _uniform(G, R, V, seed=G * 1000 + R + V + 7919 * attempt, dtype=dtype,
                          scale=2.0 if V > 4 else 0.7)
        _, _, info = oracle.commit(logits, masked.numpy(), tokens.numpy(), tau, k_min)
        if V == 1 or not _close_rows(info, masked.numpy(), tau, k_min):
            break
    else:
        raise AssertionError("no seed left the guard band")
    say(f"[commit edge] G={G} R={R} V={V} {dtype} tau={tau} k_min={k_min}")
    _check(logits, masked, tau, k_min, "edge")


def test_commit_closed_form_threshold_sides():
    V, tau = 131072, 0.85
    rows = []
    for side in (+1e-3, -1e-3, +3e-3, -3e-3):
        target = tau + side
        delta = math.log((V - 1) * target / (1 - target))
        r = torch.zeros(V)
        r[12345 + int(side * 1e6)] = delta
        rows.append(r)
    logits = torch.stack(rows).reshape(1, 4, V)
    masked = torch.ones(1, 4, dtype=torch.uint8)
    _, rm, _ = _check(logits, masked, tau, 0, "closed form fp32")
    assert rm.tolist() == [[0, 1, 0, 1]]


def test_commit_ties():
    V = 131072
    lg = torch.zeros(2, 3, V)
    lg[0, 0, [70000, 5, 130000]] = 9.0          # argmax tie across vocabulary chunks
    lg[0, 1] = lg[0, 0]                          # identical rows: ranking tie -> lower row
    lg[0, 2, 99] = 1.0
    lg[1, :, 131071] = 4.0
    lg[1, 1, 0] = 4.0
    masked = torch.ones(2, 3, dtype=torch.uint8)
    rt, rm, _ = _check(lg.to(torch.bfloat16), masked, 0.99, 1, "ties")
    assert rt[0, 0] == 5 and rm[0].tolist() == [0, 1, 1]
    assert rt[1, 0] == 131071 or rm[1, 0] == 1


def test_commit_workspace_any_contents_and_reuse():
    """The workspace needs no initial contents: filled with constant or
    random bytes before the first call, then reused by calls over fewer
    groups, every call matches the oracle."""
    G, R, V = 6, 28, 40000
    ws = torch.empty(bda.lib.bda_commit_workspace_bytes(G, R, V), dtype=torch.uint8, device=dev())
    g = torch.Generator().manual_seed(77)
    fills = [lambda: ws.fill_(0xFF), lambda: ws.fill_(0xAB),
             lambda: ws.copy_(torch.randint(0, 256, ws.shape, generator=g, dtype=torch.uint8).to(dev()))]
    for i, fill in enumerate(fills):
        fill()
        for G1 in (G, 3, 1):
            masked = (torch.rand(G1, R, generator=g) < 0.8).to(torch.uint8)
            tokens = torch.full((G1, R), -1, dtype=torch.int64)
            for attempt in range(16):
                logits = _uniform(G1, R, V, seed=100 * i + 10 * G1 + attempt, dtype=torch.bfloat16)
                _, _, info = oracle.commit(logits, masked.numpy(), tokens.numpy(), 0.3, 2)
                if not _close_rows(info, masked.numpy(), 0.3, 2):
                    break
            else:
                raise AssertionError("no seed left the guard band")
            say(f"[commit workspace] fill {i} G={G1}")
            _check(logits, masked, 0.3, 2, f"fill {i} G={G1}", workspace=ws)


def test_commit_noop_and_errors():
    logits = torch.zeros(0, 5, 10, device=dev())
    t = torch.zeros(0, 5, dtype=torch.int64, device=dev())
    m = torch.zeros(0, 5, dtype=torch.uint8, device=dev())
    bda.commit(logits, t, m, 0.9, 1)
    logits = torch.zeros(1, 5, 10, device=dev())
    t = torch.zeros(1, 5, dtype=torch.int64, device=dev())
    m = torch.zeros(1, 5, dtype=torch.uint8, device=dev())
    with pytest.raises(bda.BdaError):
        bda.commit(logits, t, m, float("nan"), 1)


# ------------------------------------------------------------------ verify

def test_verify_full():
    logits, idx, _ = synth.commit_logits(seed=6, G=16, R=28)
    drafts, planted_accept = synth.verify_drafts(idx)
    say(f"[verify full] planted accept lengths {planted_accept.tolist()}")
    am, acc = bda.verify(logits.to(dev()), drafts.to(dev()))
    torch.cuda.synchronize()
    ram, racc = oracle.verify(logits, drafts)
    assert np.array_equal(am.cpu().numpy(), ram)
    assert np.array_equal(acc.cpu().numpy(), racc)
    assert acc.cpu().tolist() == planted_accept.tolist()


@pytest.mark.parametrize("B,R,V,dtype", [(3, 1, 1001, torch.float32), (2, 28, 7, torch.bfloat16),
                                         (5, 300, 4096, torch.bfloat16), (1, 0, 10, torch.float32)])
def test_verify_edges(B, R, V, dtype):
    logits = _uniform(B, R, V, seed=B + R + V, dtype=dtype)
    ram0, _ = oracle.verify(logits, np.zeros((B, R), np.int64)) if R else (np.zeros((B, 0), np.int64), None)
    drafts = torch.as_tensor(ram0.copy())
    if R > 2:
        drafts[0, R // 2] = (drafts[0, R // 2] + 1) % V
    am, acc = bda.verify(logits.to(dev()), drafts.to(dev()))
    torch.cuda.synchronize()
    ram, racc = oracle.verify(logits, drafts.numpy()) if R else (np.zeros((B, 0), np.int64), np.zeros(B, np.int32))
    assert np.array_equal(am.cpu().numpy(), ram)
    assert np.array_equal(acc.cpu().numpy(), racc)
