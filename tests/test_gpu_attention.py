"""GPU parity of the attention kernels against the fp64 oracle.

Small cases are compared element by element (every output); the full-size
workloads are compared on sampled rows that the oracle computes one by one,
in the same launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import ATOL, assert_close_attn, dev, sample_rows, say

pytestmark = pytest.mark.gpu

bda = pytest.importorskip("block_masked_attention_amd")


def _case(mode, B, Hq, Hkv, L, d, blk, seed):
    g = torch.Generator().manual_seed(seed)
    if mode == "hybrid":
        q = synth.normal((B, Hq, 2 * L, d), 1.0, g)
        k = synth.normal((B, Hkv, 2 * L, d), 1.0, g)
        v = synth.normal((B, Hkv, 2 * L, d), 1.0, g)
    else:
        q = synth.normal((B, Hq, blk, d), 1.0, g)
        k = synth.normal((B, Hkv, L, d), 1.0, g)
        v = synth.normal((B, Hkv, L, d), 1.0, g)
    return q, k, v


def _run(mode, q, k, v, blk):
    out = bda.attn_fwd(q.to(dev()), k.to(dev()), v.to(dev()), mode, blk)
    torch.cuda.synchronize()
    return out.float().cpu()


SMALL = [
    # mode, B, Hq, Hkv, L, d, block
    ("hybrid", 2, 8, 2, 200, 128, 28),     # ragged last block (200 = 7*28 + 4)
    ("hybrid", 1, 4, 1, 130, 64, 7),
    ("hybrid", 1, 4, 4, 96, 128, 1),       # block 1
    ("hybrid", 1, 4, 2, 96, 128, 96),      # block = L
    ("hybrid", 2, 16, 2, 300, 128, 32),    # 8-wave workgroups, G = 8
    ("hybrid", 1, 32, 8, 512, 128, 32),    # training-form head layout
    ("hybrid", 1, 3, 3, 50, 32, 50),
    ("hybrid", 1, 6, 2, 257, 64, 16),
    ("hybrid", 1, 2, 1, 1, 32, 1),         # smallest
    ("decode", 2, 32, 8, 300, 128, 28),
    ("decode", 1, 8, 8, 1000, 64, 5),
    ("decode", 3, 4, 2, 77, 32, 77),
    ("decode", 1, 32, 8, 4124, 128, 28),
    ("causal", 2, 32, 8, 333, 128, 28),
    ("causal", 1, 8, 2, 300, 128, 300),    # prefill (n = L)
    ("causal", 2, 4, 1, 700, 64, 150),
    ("causal", 1, 2, 1, 65, 32, 1),
    ("decode", 1, 8, 2, 512, 128, 128),    # 8-wave persistent walk, items of full tiles only
    ("causal", 1, 8, 2, 256, 128, 129),    # last query tile (one row) sees all 256 keys
    ("decode", 1, 4, 1, 20, 128, 20),      # fewer keys than half a tile: one key group sees none
]


@pytest.mark.parametrize("mode,B,Hq,Hkv,L,d,blk", SMALL)
def test_small_elementwise(mode, B, Hq, Hkv, L, d, blk):
    say(f"[attn small] {mode} B={B} Hq={Hq} Hkv={Hkv} L={L} d={d} block={blk}")
    q, k, v = _case(mode, B, Hq, Hkv, L, d, blk, seed=1000 + L + d + blk)
    got = _run(mode, q, k, v, blk)
    ref = oracle.attention(mode, q, k, v, L, blk)
    assert_close_attn(got.numpy(), ref, f"{mode} L={L} b={blk}")


def test_tiny_config_fp32_inputs_rounded():
    """Tiny workload: fp32 Q/K/V are rounded to bf16 (RNE) before the kernel;
    the oracle reads the same rounded values."""
    case, _, _ = synth.tiny()
    q, k, v = (t.to(torch.bfloat16) for t in (case.q, case.k, case.v))
    say("[attn tiny] hybrid L=64 b=4 Hq=Hkv=2 d=32")
    got = _run("hybrid", q, k, v, case.block)
    ref = oracle.attention("hybrid", q, k, v, case.L, case.block)
    assert_close_attn(got.numpy(), ref, "tiny")


def _sampled(case, sel, what):
    mode, L, blk = case.mode, case.L, case.block
    say(f"[attn full] {what}: shapes q={tuple(case.q.shape)} k={tuple(case.k.shape)}")
    out = bda.attn_fwd(case.q.to(dev()), case.k.to(dev()), case.v.to(dev()), mode, blk)
    torch.cuda.synchronize()
    out = out.cpu()
    got = np.stack([out[b, h, i].float().numpy() for (b, h, i) in sel])
    ref = oracle.attention(mode, case.q, case.k, case.v, L, blk, sel=sel)
    return assert_close_attn(got, ref, what)


def test_full_training_form_sampled():
    case = synth.hybrid_train()
    B, H, R = case.q.shape[:3]
    L = case.L
    must = [(0, 0, 0), (0, 0, L - 1), (0, 0, L), (3, 31, 2 * L - 1), (1, 5, L + 31), (2, 17, 32), (3, 0, L - 32)]
    _sampled(case, sample_rows(B, H, R, 384, seed=7, must=must), "training form B=4 L=2048 b=32")


def test_full_decode_sampled():
    case = synth.decode_block()
    B, H, R = case.q.shape[:3]
    must = [(0, 0, r) for r in range(28)] + [(31, 31, r) for r in range(28)]
    _sampled(case, sample_rows(B, H, R, 200, seed=8, must=must), "decode B=32 n=28 KV=4124")


def test_full_verify_sampled():
    case = synth.verify_block()
    B, H, R = case.q.shape[:3]
    must = [(0, 0, r) for r in range(28)] + [(15, 31, r) for r in range(28)]
    _sampled(case, sample_rows(B, H, R, 200, seed=9, must=must), "verify B=16 n=28 KV=8220")


def test_full_prefill_sampled():
    case = synth.multimodal_prefill()
    B, H, R = case.q.shape[:3]
    must = [(0, 0, 0), (0, 0, 1), (1, 31, R - 1), (1, 3, 4095), (0, 8, 2048)]
    _sampled(case, sample_rows(B, H, R, 256, seed=10, must=must), "prefill B=2 n=L=4096")


def test_masked_perturbation_bitwise():
    """Large finite noise in keys/values a query block may not see leaves
    that block's outputs bitwise unchanged."""
    L, blk = 256, 32
    q, k, v = _case("hybrid", 1, 8, 2, L, 128, blk, seed=77)
    base = _run("hybrid", q, k, v, blk)
    M = oracle.mask("hybrid", L, blk)
    for qb in (0, 3 * blk, L + 5 * blk, 2 * L - blk):
        rows = slice(qb, qb + blk)
        hidden = torch.as_tensor(~M[rows].any(axis=0))
        g = torch.Generator().manual_seed(qb)
        k2, v2 = k.clone(), v.clone()
        noise = (torch.randn(k.shape, generator=g) * 3e3).to(torch.bfloat16)
        k2[:, :, hidden] = noise[:, :, hidden]
        v2[:, :, hidden] = -noise[:, :, hidden]
        say(f"[attn perturb] query block starting at row {qb}")
        out = _run("hybrid", q, k2, v2, blk)
        assert torch.equal(out[:, :, rows], base[:, :, rows])


def test_decode_perturbation_bitwise_causal():
    L, n = 500, 28
    q, k, v = _case("causal", 2, 8, 2, L, 128, n, seed=78)
    base = _run("causal", q, k, v, n)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, L - n + 1:] = 1e3        # the first query sees keys 0..L-n only
    v2[:, :, L - n + 1:] = -1e3
    out = _run("causal", q, k2, v2, n)
    assert torch.equal(out[:, :, 0], base[:, :, 0])


def test_deterministic_bitwise():
    for mode, blk, L in (("hybrid", 32, 512), ("decode", 28, 3000), ("causal", 28, 3000)):
        q, k, v = _case(mode, 2, 32, 8, L, 128, blk, seed=5)
        a = _run(mode, q, k, v, blk)
        b = _run(mode, q, k, v, blk)
        assert torch.equal(a, b), mode


def test_cross_mode_on_gpu():
    """Clean-half rows of block j of the training form equal the decode form
    over the clean keys up to block j (both computed by the kernels)."""
    L, blk = 320, 32
    q, k, v = _case("hybrid", 1, 8, 2, L, 128, blk, seed=90)
    hyb = _run("hybrid", q, k, v, blk)
    for j in (0, 4, 9):
        s, e = j * blk, (j + 1) * blk
        dec = _run("decode", q[:, :, L + s:L + e].contiguous(), k[:, :, L:L + e].contiguous(),
                   v[:, :, L:L + e].contiguous(), blk)
        assert (hyb[:, :, L + s:L + e] - dec).abs().max().item() <= ATOL
    # causal prefill: its last n rows equal the n-row verify over the same keys
    qc, kc, vc = _case("causal", 1, 8, 2, 400, 128, 400, seed=91)
    full = _run("causal", qc, kc, vc, 400)
    part = _run("causal", qc[:, :, -28:].contiguous(), kc, vc, 28)
    assert (full[:, :, -28:] - part).abs().max().item() <= ATOL


def test_errors_raise():
    q = torch.zeros(1, 3, 8, 128, dtype=torch.bfloat16, device=dev())
    k = torch.zeros(1, 2, 8, 128, dtype=torch.bfloat16, device=dev())
    with pytest.raises(bda.BdaError):
        bda.attn_fwd(q, k, k, "hybrid", 2)
