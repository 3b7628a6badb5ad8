"""GPU parity of the per-sequence cache lengths of linear speculative
decoding ([NLD-3x] sec. 2 and its KV-cache strategy): DECODE / CAUSAL
attention where batch row b sees only its first kv_len[b] keys, the append of
a block's K/V rows at each row's own position, and the verify pass that crops
each row's length to its accepted drafts.  References: the fp64 oracle on
each batch row cut to its own length; the append and the crop are checked
exactly."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close_attn, dev, say

pytestmark = pytest.mark.gpu

bda = pytest.importorskip("block_masked_attention_amd")

CASES = [
    # (mode, B, Hq, Hkv, d, n, cap, lengths)
    ("decode", 4, 32, 8, 128, 28, 4124, [28, 1000, 4124, 3001]),     # key splits, ragged
    ("causal", 4, 32, 8, 128, 28, 8220, [28, 5000, 8220, 77]),
    ("decode", 3, 8, 2, 64, 5, 300, [5, 150, 299]),
    ("causal", 2, 4, 4, 32, 130, 700, [130, 611]),                    # long block
    ("decode", 2, 16, 2, 128, 128, 2000, [128, 1777]),
    ("causal", 2, 32, 8, 128, 28, 1000, [0, 99999]),                   # clamped to [n, cap]
]


def _sel(B, Hq, n, k, seed):
    g = np.random.default_rng(seed)
    out = []
    for b in range(B):
        out += [(b, 0, 0), (b, Hq - 1, n - 1)]
        out += [(b, int(g.integers(Hq)), int(g.integers(n))) for _ in range(k)]
    return out


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_varlen_attention(ci):
    mode, B, Hq, Hkv, d, n, cap, lens = CASES[ci]
    say(f"[varlen] case {ci}: {mode} B={B} Hq={Hq} Hkv={Hkv} d={d} n={n} cap={cap} lens={lens}")
    q, k, v = synth.varlen_case(30 + ci, B, Hq, Hkv, d, n, cap)
    kl = torch.tensor(lens, dtype=torch.int32)
    out = bda.attn_fwd_varlen(q.to(dev()), k.to(dev()), v.to(dev()), kl.to(dev()), mode, n)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    for b in range(B):
        Lb = min(cap, max(n, lens[b]))
        sel = [(0, h, i) for (bb, h, i) in _sel(B, Hq, n, 12, 7 + ci) if bb == b]
        ref = oracle.attention(mode, q[b:b + 1], k[b:b + 1, :, :Lb], v[b:b + 1, :, :Lb], Lb, n, sel=sel)
        got = np.stack([out[b, h, i] for (_, h, i) in sel])
        assert_close_attn(got, ref, f"{mode} row {b} (keys {Lb})")


@pytest.mark.parametrize("mode", ["decode", "causal"])
def test_varlen_full_length_matches_fixed_length(mode):
    """Every row at the capacity: bit-identical to the fixed-length call."""
    B, Hq, Hkv, d, n, cap = 4, 32, 8, 128, 28, 4124
    q, k, v = synth.varlen_case(40, B, Hq, Hkv, d, n, cap)
    q, k, v = q.to(dev()), k.to(dev()), v.to(dev())
    a = bda.attn_fwd_varlen(q, k, v, torch.full((B,), cap, dtype=torch.int32, device=dev()), mode, n)
    b = bda.attn_fwd(q, k, v, mode, n)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_kv_append():
    B, Hkv, d, n, cap = 3, 8, 128, 28, 600
    k, v, _ = synth.spec_prefix(seed=41, prefix=(10, 300, 572), cap=cap, n=n, Hkv=Hkv, d=d)
    lens = [0, 328, 10000]                      # clamped to n, 328, cap
    kn = synth.normal((B, Hkv, n, d), 1.0, synth._gen(42))
    vn = synth.normal((B, Hkv, n, d), 1.0, synth._gen(43))
    gk, gv = k.to(dev()), v.to(dev())
    bda.kv_append(gk, gv, kn.to(dev()), vn.to(dev()), torch.tensor(lens, dtype=torch.int32, device=dev()))
    torch.cuda.synchronize()
    ek, ev = k.clone(), v.clone()
    for b, L in enumerate(lens):
        Lb = min(cap, max(n, L))
        ek[b, :, Lb - n:Lb] = kn[b]
        ev[b, :, Lb - n:Lb] = vn[b]
    assert torch.equal(gk.cpu().view(torch.int16), ek.view(torch.int16))
    assert torch.equal(gv.cpu().view(torch.int16), ev.view(torch.int16))


def test_verify_crop():
    B, R, V, cap = 16, 28, synth.VOCAB, 4200
    vl, vidx, _ = synth.commit_logits(seed=6, G=B, R=R)
    drafts, _ = synth.verify_drafts(vidx)
    kv0 = torch.tensor([4199 - 3 * b for b in range(B)], dtype=torch.int32)    # some rows reach the cap
    kl = kv0.to(dev())
    am, acc = bda.verify_crop(vl.to(dev()), drafts.to(dev()), kl, cap)
    torch.cuda.synchronize()
    ram, racc = oracle.verify(vl, drafts)
    assert np.array_equal(am.cpu().numpy(), ram)
    assert np.array_equal(acc.cpu().numpy(), racc)
    want = np.minimum(kv0.numpy().astype(np.int64) + racc, cap)
    assert np.array_equal(kl.cpu().numpy(), want)
    assert (want == cap).any() and (want < cap).any()
