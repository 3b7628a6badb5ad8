"""GPU parity of the attention kernels against the fp64 oracle.

Every case is compared element by element (every output), the full-size
workloads included, in the same launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import ATOL, assert_close_attn, dev, say

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
    ("causal", 1, 4, 1, 2048, 128, 128),   # persistent walk with 8 key splits (partials, then the combine)
    # split-key walk prologues: walks of at most 8 tiles start on tile 0 while
    # tiles 1..3 load, longer walks wait for four tiles first
    ("decode", 4, 32, 8, 4096, 128, 28),   # 8 splits of exactly 8 tiles (the short prologue's largest walk)
    ("decode", 4, 32, 8, 4608, 128, 28),   # 8 splits of 9 tiles (the long prologue's smallest walk)
    ("causal", 4, 32, 8, 4100, 128, 28),   # 7 splits of 9 tiles and a ragged last split of 2 tiles: both in one launch
    # persistent training-form walk at d = 32 and 64 (one 8-wave workgroup per
    # CU for d = 128, two below), items of one block's rows with 32-key
    # boundary ranges
    ("hybrid", 1, 4, 1, 512, 32, 16),
    ("hybrid", 2, 8, 2, 640, 64, 32),
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


# Element-wise cases whose persistent walk takes several items per
# workgroup (the grid is one workgroup per compute unit at d = 128, two at
# d = 64 and 32), so the DMA ring carried from one item into the next and the
# boundary tile that ends every item are checked on every output.
MULTI_ITEM = [
    # mode, B, Hq, Hkv, L, d, block               items per workgroup (256 CUs)
    ("hybrid", 4, 32, 8, 1024, 128, 32),         # 1024 items: 4
    ("hybrid", 4, 32, 8, 2048, 64, 32),          # 2048 items on 512: 4
    ("hybrid", 4, 32, 8, 1536, 32, 28),          # 1536 items on 512: 3, ragged blocks
    ("hybrid", 3, 32, 8, 1000, 128, 7),          # ragged tail of the sequence, short blocks
    ("causal", 2, 32, 8, 2048, 128, 2048),       # prefill form: 512 items, 2
    ("causal", 4, 32, 8, 2100, 64, 2100),        # prefill, 1056 items on 512, ragged last query tile
]


@pytest.mark.parametrize("mode,B,Hq,Hkv,L,d,blk", MULTI_ITEM)
def test_multi_item_elementwise(mode, B, Hq, Hkv, L, d, blk):
    say(f"[attn multi-item] {mode} B={B} Hq={Hq} Hkv={Hkv} L={L} d={d} block={blk}")
    q, k, v = _case(mode, B, Hq, Hkv, L, d, blk, seed=2000 + L + d + blk)
    got = _run(mode, q, k, v, blk)
    ref = oracle.attention(mode, q, k, v, L, blk)
    assert_close_attn(got.numpy(), ref, f"{mode} B={B} L={L} d={d} b={blk}")


# Scores that grow along the walk: a key component along one direction u
# rises by RATE (natural-log units of score) per 64 keys of its position, and
# every query carries A along u.  A later subtile's weights then exceed the
# running maximum's by e^4 or more, so the online softmax moves its maximum
# and rescales O on nearly every subtile (inside the fast loop, in boundary
# tiles, across items), the two key-half groups of the split walk merge
# different maxima, and key splits combine partials whose maxima differ by
# hundreds.  Normal inputs reach that path only on a walk's first subtile.
GROWING = [
    # mode, B, Hq, Hkv, L, d, block
    ("hybrid", 1, 8, 2, 512, 128, 32),       # one item per workgroup
    ("hybrid", 2, 32, 8, 1024, 128, 32),     # 512 items: two per workgroup
    ("hybrid", 1, 6, 2, 257, 64, 16),        # d = 64, ragged
    ("decode", 2, 32, 8, 2000, 128, 28),     # split walk, group merge
    ("causal", 1, 4, 1, 2048, 128, 128),     # persistent walk with key splits, then the combine
    ("causal", 2, 8, 2, 700, 128, 700),      # prefill form
]
RATE, A = 8.0, 8.0


@pytest.mark.parametrize("mode,B,Hq,Hkv,L,d,blk", GROWING)
def test_growing_scores_elementwise(mode, B, Hq, Hkv, L, d, blk):
    say(f"[attn growing scores] {mode} B={B} Hq={Hq} Hkv={Hkv} L={L} d={d} block={blk}")
    q, k, v = _case(mode, B, Hq, Hkv, L, d, blk, seed=3000 + L + d + blk)
    g = torch.Generator().manual_seed(L + d)
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    pos = torch.arange(k.shape[2], dtype=torch.float32)
    if mode == "hybrid":
        pos = pos % L                         # both halves grow along the position
    c = RATE * pos / 64.0 * (d ** 0.5) / A
    q = (q.float() + A * u).to(torch.bfloat16)
    k = (k.float() + c[:, None] * u).to(torch.bfloat16)
    got = _run(mode, q, k, v, blk)
    ref = oracle.attention(mode, q, k, v, L, blk)
    assert_close_attn(got.numpy(), ref, f"growing scores {mode} B={B} L={L} d={d} b={blk}")


def _dense(case, what):
    """Every output element of a full-size workload against the oracle, in
    the launch configuration the benchmark times."""
    mode, L, blk = case.mode, case.L, case.block
    say(f"[attn full dense] {what}: shapes q={tuple(case.q.shape)} k={tuple(case.k.shape)}")
    out = bda.attn_fwd(case.q.to(dev()), case.k.to(dev()), case.v.to(dev()), mode, blk)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    del out
    ref = oracle.attention(mode, case.q, case.k, case.v, L, blk)
    err = assert_close_attn(got, ref, what)
    say(f"[attn full dense] {what}: max err {err:.3e}")


def test_full_training_form_dense():
    _dense(synth.hybrid_train(), "training form B=4 L=2048 b=32 (every row)")


def test_full_prefill_dense():
    _dense(synth.multimodal_prefill(), "prefill B=2 n=L=4096 (every row)")


def test_full_decode_dense():
    _dense(synth.decode_block(), "decode B=32 n=28 KV=4124 (every row)")


def test_full_verify_dense():
    _dense(synth.verify_block(), "verify B=16 n=28 KV=8220 (every row)")


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
