"""Logits set to -inf (banned tokens) in the commit, row statistics and
entropy-bound commit, against the oracle.

A -inf logit has probability exactly 0: it adds nothing to Z, nothing to the
entropy (the oracle skips p = 0 terms), and never wins the argmax.  Every row
keeps at least one finite logit.  Cases cover one -inf per row and whole
16384-entry vocabulary chunks of -inf (the chunk a streaming workgroup reads
whole), for bf16 and fp32 logits, on the aligned whole-chunk path (V =
131072) and the ragged path (V = 20000).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from commit_util import close_rows
from gpu_util import dev, say
from test_gpu_entropy_commit import _run as run_entropy_commit
from test_gpu_stats import _compare as compare_stats

pytestmark = pytest.mark.gpu

bda = pytest.importorskip("block_masked_attention_amd")

CHUNK = 16384


def _ban(logits, idx, rows, kind, seed):
    """Write -inf into the listed (g, r) rows as `kind` says; the planted peak
    is never banned."""
    g = torch.Generator().manual_seed(seed)
    V = logits.shape[-1]
    ninf = float("-inf")
    for gi, r in rows:
        peak = int(idx[gi, r])
        if kind == "one":
            j = int(torch.randint(V, (1,), generator=g))
            if j == peak:
                j = (j + 1) % V
            logits[gi, r, j] = ninf
        elif kind == "chunk":
            c = 0 if peak >= CHUNK else 1      # the first whole chunk without the peak
            logits[gi, r, c * CHUNK:min(V, (c + 1) * CHUNK)] = ninf
        elif kind == "all_but_peak_chunk":
            keep = peak // CHUNK
            for c in range((V + CHUNK - 1) // CHUNK):
                if c != keep:
                    logits[gi, r, c * CHUNK:min(V, (c + 1) * CHUNK)] = ninf


def _banned(kind, G, R, V, dtype, seed, tau=None):
    """Planted-peak logits (noise sigma 3, a peak per row as in the decode
    workload) with -inf written where `kind` says.  With tau, rows whose
    commit decision falls inside the guard band are redrawn and banned again
    (seeded), as the other commit tests do."""
    logits, idx = synth.planted_logits(G, R, V, 3.0, torch.Generator().manual_seed(seed), dtype=dtype)
    _ban(logits, idx, [(g, r) for g in range(G) for r in range(R)], kind, seed + 1)
    if tau is None:
        return logits, idx
    masked = np.ones((G, R), dtype=np.uint8)
    for it in range(8):
        _, _, info = oracle.commit(logits, masked, np.full((G, R), -1, dtype=np.int64), tau, 1)
        bad = close_rows(info, masked, tau, 1)
        if not bad:
            return logits, idx
        synth.redraw_rows(logits, idx, bad, seed=seed * 100 + it, sigma=3.0)
        _ban(logits, idx, bad, kind, seed + 2 + it)
    raise AssertionError("could not leave the guard band")


CASES = [
    # kind, G, R, V, dtype
    ("one", 4, 28, 131072, torch.bfloat16),
    ("one", 4, 28, 131072, torch.float32),
    ("chunk", 4, 28, 131072, torch.bfloat16),
    ("chunk", 4, 28, 131072, torch.float32),
    ("all_but_peak_chunk", 2, 28, 131072, torch.bfloat16),
    ("one", 3, 12, 20000, torch.bfloat16),
    ("chunk", 3, 12, 20000, torch.float32),
]


@pytest.mark.parametrize("kind,G,R,V,dtype", CASES)
def test_banned_commit(kind, G, R, V, dtype):
    say(f"[banned] commit {kind} G={G} R={R} V={V} {dtype}")
    logits, idx = _banned(kind, G, R, V, dtype, seed=700 + G + V, tau=0.85)
    masked = torch.ones(G, R, dtype=torch.uint8)
    tokens = torch.full((G, R), -1, dtype=torch.int64)
    rt, rm, _ = oracle.commit(logits, masked.numpy(), tokens.numpy(), 0.85, 1)
    t, m = tokens.to(dev()), masked.clone().to(dev())
    bda.commit(logits.to(dev()), t, m, 0.85, 1)
    torch.cuda.synchronize()
    assert np.array_equal(m.cpu().numpy(), rm), "commit masks differ"
    assert np.array_equal(t.cpu().numpy(), rt), "committed tokens differ"
    assert int(masked.sum()) - int(rm.sum()) >= G


@pytest.mark.parametrize("kind,G,R,V,dtype", CASES)
def test_banned_row_stats(kind, G, R, V, dtype):
    logits, _ = _banned(kind, G, R, V, dtype, seed=800 + G + V)
    compare_stats(logits, None, f"banned {kind} [{G},{R},{V}] {dtype}")


@pytest.mark.parametrize("kind,G,R,V,dtype", CASES)
def test_banned_entropy_commit(kind, G, R, V, dtype):
    logits, _ = _banned(kind, G, R, V, dtype, seed=900 + G + V)
    masked = torch.ones(G, R, dtype=torch.uint8)
    run_entropy_commit(logits, masked, None, 1.0, 1, f"banned {kind}")


def test_banned_verify():
    logits, idx = _banned("chunk", 4, 28, 131072, torch.bfloat16, seed=1000)
    drafts, _ = synth.verify_drafts(idx)
    am, acc = bda.verify(logits.to(dev()), drafts.to(dev()))
    torch.cuda.synchronize()
    ram, racc = oracle.verify(logits, drafts.numpy())
    assert np.array_equal(am.cpu().numpy(), ram) and np.array_equal(acc.cpu().numpy(), racc)
