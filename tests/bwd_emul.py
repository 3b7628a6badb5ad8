"""Error yardstick for the backward parity tests (test logic only).

The GPU backward rounds at fixed points: the forward's output O is bf16 (it
enters the row deltas D = rowsum(dO * O)), P and dS are rounded to bf16 as
MFMA operands, and the gradients are stored in bf16.  This torch CPU
computation rounds at exactly those points and computes everything else in
fp32; its distance to the exact fp64 gradients is the rounding error that
choice of precision implies, against which the GPU error is judged.  It
takes the same bf16 forward output O that the GPU backward is given (an
input of the backward), so that the two differ only by the backward's own
rounding.
"""
import math

import torch

import oracle


def _bf(x):
    return x.to(torch.bfloat16).to(torch.float32)


def grads(q, k, v, do, L, block, o=None):
    """dq, dk, dv (float64 tensors) of the hybrid-mask attention with the
    rounding points described above.  q, do: [B,Hq,2L,d]; k, v: [B,Hkv,2L,d].
    o (optional, [B,Hq,2L,d] bf16): the forward output the backward is given;
    when absent it is the bf16 rounding of the fp32 attention output."""
    M = torch.from_numpy(oracle.mask("hybrid", L, block).astype(bool))
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    qf, kf, vf, gf = (t.to(torch.float32) for t in (q, k, v, do))
    dq = torch.empty(B, Hq, S, d, dtype=torch.float32)
    dk = torch.zeros(B, Hkv, S, d, dtype=torch.float32)
    dv = torch.zeros(B, Hkv, S, d, dtype=torch.float32)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            s = (qf[b, h] @ kf[b, g].T) * scale
            s = s.masked_fill(~M, float("-inf"))
            lse = torch.logsumexp(s.double(), dim=-1).float()
            p = torch.exp(s - lse[:, None])
            ob = _bf(p @ vf[b, g]) if o is None else o[b, h].to(torch.float32)
            D = (gf[b, h] * ob).sum(-1)
            dp = gf[b, h] @ vf[b, g].T
            ds = _bf(p * (dp - D[:, None]))
            dq[b, h] = _bf(scale * (ds @ kf[b, g]))
            dk[b, g] += scale * (ds.T @ qf[b, h])
            dv[b, g] += _bf(p).T @ gf[b, h]
    return dq.double(), _bf(dk).double(), _bf(dv).double()
