"""GPU parity of the training-form backward (dq, dk, dv) against the fp64
oracle, elementwise, on shapes that span several tiles and ragged tails, and
on the full training form.

The GPU path runs the forward with log-sum-exp output, then the backward on
the forward's bf16 output; the oracle differentiates the exact attention of
the same bf16 inputs.  Tolerance (derived from the arithmetic; see
bwd_emul.py): a CPU computation that rounds at the GPU path's bf16 points
gives the error that precision implies; the GPU's largest and mean absolute
errors against the oracle must stay within twice that computation's own
(plus 1e-3 of the gradient's rms for the max), and so must every element's
(plus 2^-6 of the element's magnitude and of the gradient's rms).
"""
import numpy as np
import pytest
import torch

import bwd_emul
import oracle
from gpu_util import dev, say

pytestmark = pytest.mark.gpu

bda = pytest.importorskip("block_masked_attention_amd")


# Per element: |gpu - ref| <= 2 |emul - ref| + EPS_REL (|ref| + rms).  The
# GPU and the emulation take the same bf16 forward output and round at the
# same points, but from fp32 values summed in different orders, so a bf16
# rounding of P, dS or the stored gradient can land one step apart (2^-8
# relative); EPS_REL = 2^-6 covers such a step in the stored value and a few
# in the terms summed into it, and the rms term does the same for elements
# whose exact value is near zero.
EPS_REL = 2.0 ** -6


def _check(got, ref, emul, what):
    got = got.float().cpu().numpy().astype(np.float64)
    emul = emul.numpy()
    rms = float(np.sqrt(np.mean(ref * ref))) + 1e-30
    err, eref = np.abs(got - ref), np.abs(emul - ref)
    bound = 2 * eref + EPS_REL * (np.abs(ref) + rms)
    worst = float((err / bound).max())
    say(f"[bwd] {what}: max err {err.max() / rms:.3e} rms (bf16-rounding yardstick {eref.max() / rms:.3e}), "
        f"mean err {err.mean() / rms:.3e} rms (yardstick {eref.mean() / rms:.3e}), "
        f"largest err / per-element bound {worst:.3f}")
    assert np.isfinite(got).all(), f"{what}: non-finite"
    assert err.max() <= 2 * eref.max() + 1e-3 * rms, f"{what}: largest error beyond the bound"
    assert err.mean() <= 2 * eref.mean() + 1e-6 * rms, f"{what}: mean error beyond the bound"
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} elements beyond the per-element bound"


CASES = [
    # B, Hq, Hkv, L, d, block
    (1, 4, 1, 64, 128, 16),      # 4-wave dq workgroups, one 128-key tile per half
    (1, 8, 2, 300, 128, 32),     # 8-wave dq workgroups, ragged key tiles (300 = 2*128 + 44)
    (2, 4, 4, 130, 64, 7),       # G = 1, block not dividing anything
    (1, 32, 1, 96, 32, 96),      # G = 32, block = L
    (1, 2, 1, 40, 128, 1),       # block 1
    (1, 16, 2, 257, 128, 28),    # G = 8, ragged
]


@pytest.mark.parametrize("B,Hq,Hkv,L,d,blk", CASES)
def test_bwd_elementwise(B, Hq, Hkv, L, d, blk):
    g = torch.Generator().manual_seed(B * 1000 + Hq * 10 + L + d + blk)
    mk = lambda H: torch.randn(B, H, 2 * L, d, generator=g).to(torch.bfloat16)
    q, k, v, do = mk(Hq), mk(Hkv), mk(Hkv), mk(Hq)
    qd, kd, vd, dod = (t.to(dev()) for t in (q, k, v, do))
    lse = torch.empty(B, Hq, 2 * L, dtype=torch.float32, device=dev())
    out = bda.attn_fwd(qd, kd, vd, "hybrid", blk, lse=lse)
    dq, dk, dv = bda.attn_bwd(qd, kd, vd, out, dod, lse, blk)
    torch.cuda.synchronize()
    rq, rk, rv, rl = oracle.attention_bwd("hybrid", q, k, v, do, L, blk)
    eq, ek, ev = bwd_emul.grads(q, k, v, do, L, blk, o=out.cpu())
    assert np.allclose(lse.cpu().numpy(), rl, rtol=0, atol=2e-3), "forward log-sum-exp"
    what = f"B={B} Hq={Hq} Hkv={Hkv} L={L} d={d} b={blk}"
    _check(dq, rq, eq, what + " dq")
    _check(dk, rk, ek, what + " dk")
    _check(dv, rv, ev, what + " dv")


@pytest.mark.parametrize("B,Hq,Hkv,L,d,blk", [(1, 8, 2, 300, 128, 32), (1, 4, 1, 130, 64, 7)])
def test_bwd_growing_scores(B, Hq, Hkv, L, d, blk):
    """Scores that rise by about 8 (natural-log units) per 64 keys of position
    in both halves, so each row's weights sit on its last visible keys and
    its log-sum-exp is far from 0: P is rebuilt from large scores minus a
    large log-sum-exp."""
    g = torch.Generator().manual_seed(4000 + L + d)
    mk = lambda H: torch.randn(B, H, 2 * L, d, generator=g)
    q, k, v, do = mk(Hq), mk(Hkv), mk(Hkv), mk(Hq)
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    c = 8.0 * (torch.arange(2 * L, dtype=torch.float32) % L) / 64.0 * (d ** 0.5) / 8.0
    q, k = q + 8.0 * u, k + c[:, None] * u
    q, k, v, do = (t.to(torch.bfloat16) for t in (q, k, v, do))
    qd, kd, vd, dod = (t.to(dev()) for t in (q, k, v, do))
    lse = torch.empty(B, Hq, 2 * L, dtype=torch.float32, device=dev())
    out = bda.attn_fwd(qd, kd, vd, "hybrid", blk, lse=lse)
    dq, dk, dv = bda.attn_bwd(qd, kd, vd, out, dod, lse, blk)
    torch.cuda.synchronize()
    rq, rk, rv, rl = oracle.attention_bwd("hybrid", q, k, v, do, L, blk)
    eq, ek, ev = bwd_emul.grads(q, k, v, do, L, blk, o=out.cpu())
    assert np.allclose(lse.cpu().numpy(), rl, rtol=0, atol=2e-3), "forward log-sum-exp"
    what = f"growing scores B={B} Hq={Hq} L={L} d={d} b={blk}"
    _check(dq, rq, eq, what + " dq")
    _check(dk, rk, ek, what + " dk")
    _check(dv, rv, ev, what + " dv")


def test_bwd_rejects_other_modes():
    q = torch.zeros(1, 2, 8, 32, dtype=torch.bfloat16, device=dev())
    k = torch.zeros(1, 1, 16, 32, dtype=torch.bfloat16, device=dev())
    lse = torch.zeros(1, 2, 8, dtype=torch.float32, device=dev())
    ws = torch.empty(1 << 16, dtype=torch.uint8, device=dev())
    rc = bda.lib.bda_attn_bwd(q.data_ptr(), k.data_ptr(), k.data_ptr(), q.data_ptr(), q.data_ptr(),
                              lse.data_ptr(), q.data_ptr(), k.data_ptr(), k.data_ptr(), 1, 2, 1, 16, 32, 8, 1,
                              ws.data_ptr(), 1 << 16, None)
    assert rc == 2


def test_bwd_training_form_full_size_batch0():
    """The full training form (B=4, L=2048, b=32, Hq=32, Hkv=8, d=128) in the
    launch configuration the benchmark times; batch 0's gradients (which
    depend on batch 0's inputs only) are compared elementwise."""
    import synth
    case = synth.hybrid_train()
    B, Hq, S, d = case.q.shape
    g = torch.Generator().manual_seed(31)
    do = torch.randn(case.q.shape, generator=g).to(torch.bfloat16)
    qd, kd, vd, dod = (t.to(dev()) for t in (case.q, case.k, case.v, do))
    lse = torch.empty(B, Hq, S, dtype=torch.float32, device=dev())
    out = bda.attn_fwd(qd, kd, vd, "hybrid", case.block, lse=lse)
    dq, dk, dv = bda.attn_bwd(qd, kd, vd, out, dod, lse, case.block)
    torch.cuda.synchronize()
    rq, rk, rv, _ = oracle.attention_bwd("hybrid", case.q[:1], case.k[:1], case.v[:1], do[:1], case.L, case.block)
    eq, ek, ev = bwd_emul.grads(case.q[:1], case.k[:1], case.v[:1], do[:1], case.L, case.block, o=out[:1].cpu())
    _check(dq[:1], rq, eq, "training form batch 0 dq")
    _check(dk[:1], rk, ek, "training form batch 0 dk")
    _check(dv[:1], rv, ev, "training form batch 0 dv")
