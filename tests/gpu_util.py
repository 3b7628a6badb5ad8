"""Helpers shared by the GPU tests (no method arithmetic here)."""
import sys

import numpy as np
import torch

ATOL, RTOL = 2e-2, 1e-2      # bf16 attention outputs: |gpu - ref| <= ATOL + RTOL * |ref|
GUARD = 1e-4                  # decisions closer than this to the threshold / ranking are redrawn


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def assert_close_attn(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance; "
                           f"max err {err.max():.3e}")
    return float(err.max())


def sample_rows(B, H, rows, n, seed, must=()):
    g = np.random.default_rng(seed)
    sel = [tuple(x) for x in must]
    sel += [(int(g.integers(B)), int(g.integers(H)), int(g.integers(rows))) for _ in range(n)]
    return sel
