"""bda_commit_noalloc (the commit over the library's static scratch, for
callers that cannot allocate) against bda_commit through the C ABI: tokens
and masks must be bit-identical on two calls in a row, the second on a
smaller input, and a size above the static scratch is refused before any
launch."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from commit_util import guarded
from gpu_util import dev, say

pytestmark = pytest.mark.gpu

bda = pytest.importorskip("block_masked_attention_amd")


def _inputs(G, R, V, seed, tau):
    logits, idx, masked = synth.commit_logits(seed=seed, G=G, R=R, V=V)
    g = torch.Generator().manual_seed(seed + 1)
    masked = (torch.rand(G, R, generator=g) < 0.8).to(torch.uint8)
    logits, _ = guarded(logits, idx, masked, tau, 1, 3.0, seed=seed)
    return logits, masked


def _both(logits, masked, tau, k_min):
    G, R, V = logits.shape
    lg = logits.to(dev())
    t0 = torch.full((G, R), -1, dtype=torch.int64, device=dev())
    m0 = masked.clone().to(dev())
    ws = torch.empty(int(bda.lib.bda_commit_workspace_bytes(G, R, V)), dtype=torch.uint8, device=dev())
    rc = bda.lib.bda_commit(bda._ptr(lg), bda.BF16, bda._ptr(t0), bda._ptr(m0), float(tau), int(k_min), G, R, V,
                            bda._ptr(ws), ws.numel(), bda._stream(dev()))
    assert rc == 0, bda.lib.bda_last_error()
    t1 = torch.full((G, R), -1, dtype=torch.int64, device=dev())
    m1 = masked.clone().to(dev())
    rc = bda.lib.bda_commit_noalloc(bda._ptr(lg), bda.BF16, bda._ptr(t1), bda._ptr(m1), float(tau), int(k_min),
                                    G, R, V, bda._stream(dev()))
    assert rc == 0, bda.lib.bda_last_error()
    torch.cuda.synchronize()
    return (t0.cpu().numpy(), m0.cpu().numpy()), (t1.cpu().numpy(), m1.cpu().numpy())


def test_noalloc_matches_commit_on_two_calls():
    # first call: the decode workload's shape; second: smaller, so stale
    # partials of the first call sit in the scratch beyond its rows
    for (G, R, V, seed, tau, k_min) in ((32, 28, 131072, 4, 0.85, 1), (3, 10, 50000, 40, 0.9, 2)):
        say(f"[noalloc] G={G} R={R} V={V} tau={tau} k_min={k_min}")
        logits, masked = _inputs(G, R, V, seed, tau)
        (ta, ma), (tb, mb) = _both(logits, masked, tau, k_min)
        assert np.array_equal(ma, mb), "masks differ"
        assert np.array_equal(ta, tb), "tokens differ"
        assert int(masked.sum()) - int(mb.sum()) >= 1


def test_noalloc_refuses_sizes_above_the_static_scratch():
    G, R, V = 64, 128, 131072               # 8192 rows x 8 chunks: about 1.1 MB of scratch
    need = int(bda.lib.bda_commit_workspace_bytes(G, R, V))
    assert need > (1 << 20)
    big = ctypes.c_void_p(1 << 40)          # never dereferenced: refused on the host
    rc = bda.lib.bda_commit_noalloc(big, bda.BF16, ctypes.c_void_p(2 << 40), ctypes.c_void_p(3 << 40), 0.9, 1,
                                    G, R, V, None)
    assert rc == 3 and b"static scratch" in bda.lib.bda_last_error()
