"""Offsets beyond 2^31 elements.

A decode call over a 32768-key cache for 80 sequences (K and V hold 2.7 G
elements each) and row statistics over [128, 160, 131072] logits (2.7 G
elements).  Inputs are drawn on the device; sampled outputs of the first
batch or group, of those where the byte offset passes 2^31 and where the
element offset passes 2^31, and of the last one are checked against the
oracle, to the tolerances of the smaller parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close_attn, dev, say

pytestmark = pytest.mark.gpu

bda = pytest.importorskip("block_masked_attention_amd")

CONF_RTOL = 2.0 ** -16


def _fill(t, g, scale=1.0):
    """Standard normal * scale in bf16, one leading index at a time (bounds
    the fp32 temporary)."""
    for i in range(t.shape[0]):
        t[i] = (torch.randn(t.shape[1:], generator=g, device=t.device) * scale).to(t.dtype)


def test_decode_offsets_beyond_2g():
    B, Hq, Hkv, L, d, n = 80, 32, 8, 32768, 128, 28
    g = torch.Generator(device=dev()).manual_seed(11)
    q = torch.empty(B, Hq, n, d, dtype=torch.bfloat16, device=dev())
    k = torch.empty(B, Hkv, L, d, dtype=torch.bfloat16, device=dev())
    v = torch.empty_like(k)
    for t in (q, k, v):
        _fill(t, g)
    per_batch = Hkv * L * d
    assert k.numel() > 2 ** 31 and (B - 1) * per_batch > 2 ** 31
    say(f"[large] decode B={B} Hq={Hq} Hkv={Hkv} L={L} d={d} n={n}: K, V {k.numel() / 1e9:.2f} G elements each")
    out = bda.attn_fwd(q, k, v, "decode", n)
    torch.cuda.synchronize()
    # batch 32 starts at 2^31 bytes of K, batch 64 at 2^31 elements
    for b in (0, 2 ** 30 // per_batch, 2 ** 31 // per_batch, B - 1):
        sel = [(0, 0, 0), (0, Hq - 1, n - 1), (0, 13, 7), (0, 21, 20)]
        ref = oracle.attention("decode", q[b:b + 1].cpu(), k[b:b + 1].cpu(), v[b:b + 1].cpu(), L, n, sel=sel)
        got = np.stack([out[b, h, i].float().cpu().numpy() for (_, h, i) in sel])
        assert_close_attn(got, ref, f"decode batch {b}")
    del q, k, v, out
    torch.cuda.empty_cache()


def test_row_stats_offsets_beyond_2g():
    G, R, V = 128, 160, 131072
    g = torch.Generator(device=dev()).manual_seed(12)
    logits = torch.empty(G, R, V, dtype=torch.bfloat16, device=dev())
    _fill(logits, g, 3.0)
    per_group = R * V
    assert logits.numel() > 2 ** 31 and (G - 1) * per_group > 2 ** 31
    say(f"[large] row statistics [{G}, {R}, {V}] bf16: {logits.numel() / 1e9:.2f} G elements")
    conf, am, ent, _ = bda.row_stats(logits)
    torch.cuda.synchronize()
    # groups 51 and 102 hold byte 2^31 and element 2^31 of the logits
    for grp in (0, 2 ** 30 // per_group, 2 ** 31 // per_group, G - 1):
        rc, ra, re, _ = oracle.row_stats(logits[grp:grp + 1].cpu())
        gc, ga, ge = conf[grp].cpu().numpy(), am[grp].cpu().numpy(), ent[grp].cpu().numpy()
        assert np.array_equal(ga, ra[0]), f"group {grp}: argmax"
        assert (np.abs(gc - rc[0]) / rc[0] <= CONF_RTOL).all(), f"group {grp}: conf"
        assert (np.abs(ge - re[0]) <= 2.0 ** -16 * (1.0 + re[0])).all(), f"group {grp}: entropy"
        say(f"[large] group {grp}: argmax equal, max conf rel err {(np.abs(gc - rc[0]) / rc[0]).max():.2e}")
    del logits
    torch.cuda.empty_cache()
