"""Guard-band handling shared by the commit parity tests (test logic only:
the decisions come from the oracle's fp64 probabilities)."""
import numpy as np
import torch

import oracle
import synth
from gpu_util import GUARD, say


def close_rows(info, masked, tau, k_min):
    """Rows whose decision lies inside the guard band (from the oracle)."""
    p = info["p64"]
    G, R = p.shape
    bad = set()
    for g in range(G):
        rows = [r for r in range(R) if masked[g, r]]
        for r in rows:
            if abs(p[g, r] - tau) <= GUARD:
                bad.add((g, r))
        below = sorted((r for r in rows if np.float32(p[g, r]) <= np.float32(tau)),
                       key=lambda r: (-float(np.float32(p[g, r])), r))
        need = min(k_min, len(rows)) - (len(rows) - len(below))
        if 0 < need < len(below) and p[g, below[need - 1]] - p[g, below[need]] <= GUARD:
            bad.update({(g, below[need - 1]), (g, below[need])})
    return sorted(bad)


def guarded(logits, idx, masked, tau, k_min, sigma, seed):
    for it in range(8):
        tokens = torch.full(masked.shape, -1, dtype=torch.int64)
        _, _, info = oracle.commit(logits, masked.numpy(), tokens.numpy(), tau, k_min)
        bad = close_rows(info, masked.numpy(), tau, k_min)
        if not bad:
            return logits, info
        say(f"  redrawing {len(bad)} rows inside the guard band")
        synth.redraw_rows(logits, idx, bad, seed=seed * 100 + it, sigma=sigma)
    raise AssertionError("could not leave the guard band")


