"""GPU parity over the multimodal canvas trajectory.

The 4096-token image+text prefix (55x55 merged image tokens, 55 row breaks,
1016 text tokens) fills the cache; the 256-position canvas is then decoded
block by block (nine blocks of 28 and a last block of 4) with threshold 0.9
and at least one commit per step, until every position of a block is
committed; a finished block's K/V rows join the cache.  Per step the inputs
(the active block's queries and fresh K/V rows, the canvas logits) are the
seeded synthetic draws of the multimodal workload.

Every step's committed token ids and commit masks, updated in place on the
device across steps, must equal the oracle's exactly (rows inside the
guard band are redrawn first).  The decode attention of the first step of
every block is compared with the oracle on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from commit_util import guarded
from gpu_util import assert_close_attn, dev, sample_rows, say

pytestmark = pytest.mark.gpu

bda = pytest.importorskip("block_masked_attention_amd")

TAU, K_MIN = 0.9, 1


def test_canvas_trajectory():
    pre = synth.multimodal_prefill()
    B, Hq = pre.q.shape[:2]
    kc, vc = pre.k, pre.v
    canvas = torch.full((B, synth.CANVAS), -1, dtype=torch.int64)
    step, pos = 0, 0
    for bi, n in enumerate(synth.canvas_blocks()):
        masked = torch.ones(B, n, dtype=torch.uint8)
        tokens = torch.full((B, n), -1, dtype=torch.int64)
        g_masked, g_tokens = masked.to(dev()), tokens.to(dev())
        first = True
        while bool(masked.any()):
            assert step < 400, "canvas did not finish"
            q, kb, vb, logits, idx = synth.multimodal_step(step, n, B=B)
            k = torch.cat([kc, kb], dim=2)
            v = torch.cat([vc, vb], dim=2)
            L = k.shape[2]
            out = bda.attn_fwd(q.to(dev()), k.to(dev()), v.to(dev()), "decode", n)
            torch.cuda.synchronize()
            if first:
                sel = sample_rows(B, Hq, n, 24, seed=300 + bi, must=[(0, 0, 0), (B - 1, Hq - 1, n - 1)])
                got = np.stack([out[b, h, i].float().cpu().numpy() for (b, h, i) in sel])
                ref = oracle.attention("decode", q, k, v, L, n, sel=sel)
                assert_close_attn(got, ref, f"canvas block {bi} step {step} attention (KV {L})")
            logits, _ = guarded(logits, idx, masked, TAU, K_MIN, 3.0, seed=1000 + step)
            rt, rm, _ = oracle.commit(logits, masked.numpy(), tokens.numpy(), TAU, K_MIN)
            bda.commit(logits.to(dev()), g_tokens, g_masked, TAU, K_MIN)
            torch.cuda.synchronize()
            assert np.array_equal(g_masked.cpu().numpy(), rm), f"step {step}: commit masks differ"
            assert np.array_equal(g_tokens.cpu().numpy(), rt), f"step {step}: committed tokens differ"
            assert int(masked.sum()) - int(rm.sum()) >= min(K_MIN, int(masked.sum()))
            tokens, masked = torch.from_numpy(rt), torch.from_numpy(rm)
            step += 1
            first = False
        kc, vc = k, v                      # the finished block's rows join the cache
        canvas[:, pos:pos + n] = tokens
        pos += n
    say(f"[canvas] {step} denoise steps for {synth.CANVAS} positions; final KV {kc.shape[2]}")
    assert pos == synth.CANVAS and bool((canvas >= 0).all())
    assert kc.shape[2] == synth.PREFIX + synth.CANVAS
