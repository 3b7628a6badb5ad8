"""The linear speculative loop of [NLD-3x] sec. 2 on the device, captured in
a HIP graph.

One step: write the draft block's K/V rows at each sequence's own position;
DECODE attention of the draft queries over each sequence's cache; the drafts
are the argmax of the draft logits; write the validation pass's K/V rows over
them; CAUSAL attention of the validation queries; verify against the drafts
and crop each sequence's length to its accepted drafts.  Logits and fresh
K/V rows stand in for the model (seeded draws with planted accept lengths).

The step is captured once and replayed for several steps, the per-sequence
lengths changing on the device in between.  Every replay is checked against
the same step run eagerly (bit for bit) and against the oracle's trajectory:
attention on sampled rows within the bf16 tolerance, drafts, argmax, accept
lengths, lengths and cache contents exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close_attn, dev, say

pytestmark = pytest.mark.gpu

bda = pytest.importorskip("block_masked_attention_amd")

STEPS = 5
B, Hq, Hkv, d, n, V, CAP = 4, 32, 8, 128, 28, 32768, 3328
PREFIX = (517, 1000, 2345, 3000)


class Loop:
    """State (cache, lengths), static inputs and outputs of the loop."""

    def __init__(self, k, v, kv_len):
        D = dev()
        bf = torch.bfloat16
        self.kc, self.vc, self.kl = k.to(D).clone(), v.to(D).clone(), kv_len.to(D).clone()
        self.qd = torch.empty(B, Hq, n, d, dtype=bf, device=D)
        self.qv = torch.empty_like(self.qd)
        self.kd = torch.empty(B, Hkv, n, d, dtype=bf, device=D)
        self.vd, self.kv, self.vv = torch.empty_like(self.kd), torch.empty_like(self.kd), torch.empty_like(self.kd)
        self.dlog = torch.empty(B, n, V, dtype=bf, device=D)
        self.vlog = torch.empty_like(self.dlog)
        self.od, self.ov = torch.empty_like(self.qd), torch.empty_like(self.qd)
        self.drafts = torch.empty(B, n, dtype=torch.int64, device=D)
        self.am = torch.empty(B, n, dtype=torch.int64, device=D)
        self.acc = torch.empty(B, dtype=torch.int32, device=D)
        u8 = torch.uint8
        self.ws_d = torch.empty(max(1, bda.attn_workspace_bytes(B, Hq, Hkv, CAP, d, n, "decode")), dtype=u8, device=D)
        self.ws_v = torch.empty(max(1, bda.attn_workspace_bytes(B, Hq, Hkv, CAP, d, n, "causal")), dtype=u8, device=D)
        self.n_s = int(bda.lib.bda_row_stats_workspace_bytes(B, n, V))
        self.ws_s = torch.empty(self.n_s, dtype=u8, device=D)
        self.ws_c = torch.empty(int(bda.lib.bda_verify_workspace_bytes(B, n, V)), dtype=u8, device=D)

    def load(self, s):
        for name in ("qd", "kd", "vd", "dlog", "qv", "kv", "vv", "vlog"):
            getattr(self, name).copy_(s[name])

    def run(self):
        st = bda._stream(dev())
        bda.kv_append(self.kc, self.vc, self.kd, self.vd, self.kl)
        bda.attn_fwd_varlen(self.qd, self.kc, self.vc, self.kl, "decode", n, out=self.od, workspace=self.ws_d)
        rc = bda.lib.bda_row_stats(bda._ptr(self.dlog), bda.BF16, None, None, bda._ptr(self.drafts), None, None,
                                   B, n, V, bda._ptr(self.ws_s), self.n_s, st)
        assert rc == 0
        bda.kv_append(self.kc, self.vc, self.kv, self.vv, self.kl)
        bda.attn_fwd_varlen(self.qv, self.kc, self.vc, self.kl, "causal", n, out=self.ov, workspace=self.ws_v)
        bda.verify_crop(self.vlog, self.drafts, self.kl, CAP, argmax_out=self.am, accept_len=self.acc,
                        workspace=self.ws_c)

    def snapshot(self):
        return {k: getattr(self, k).clone() for k in ("od", "ov", "drafts", "am", "acc", "kl", "kc", "vc")}


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def _sampled(out, q, k, v, lens, mode, seed):
    g = np.random.default_rng(seed)
    for b in range(B):
        Lb = int(lens[b])
        sel = [(0, 0, 0), (0, Hq - 1, n - 1)] + [(0, int(g.integers(Hq)), int(g.integers(n))) for _ in range(6)]
        ref = oracle.attention(mode, q[b:b + 1], k[b:b + 1, :, :Lb], v[b:b + 1, :, :Lb], Lb, n, sel=sel)
        got = np.stack([out[b, h, i].float().cpu().numpy() for (_, h, i) in sel])
        assert_close_attn(got, ref, f"{mode} sequence {b} (keys {Lb})")


def test_speculative_loop_graph():
    k0, v0, kl0 = synth.spec_prefix(prefix=PREFIX, cap=CAP, n=n, Hkv=Hkv, d=d)
    warm = Loop(k0, v0, kl0)                  # first launches outside the capture
    warm.load(synth.spec_step(0, B, n, Hq, Hkv, d, V))
    warm.run()
    torch.cuda.synchronize()
    del warm
    gl, el = Loop(k0, v0, kl0), Loop(k0, v0, kl0)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gl.run()
    torch.cuda.synchronize()
    # the oracle's trajectory on the host
    kh, vh, lens = k0.clone(), v0.clone(), kl0.numpy().astype(np.int64)
    total = 0
    for t in range(STEPS):
        s = synth.spec_step(t, B, n, Hq, Hkv, d, V)
        say(f"[spec] step {t}: lengths {lens.tolist()} planted accept {s['accept'].tolist()}")
        gl.load(s)
        el.load(s)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        gs = gl.snapshot()
        el.run()
        torch.cuda.synchronize()
        es = el.snapshot()
        for key in gs:
            assert _same(gs[key], es[key]), f"step {t}: graph replay and eager run differ in {key}"
        # oracle: draft pass
        for b in range(B):
            kh[b, :, lens[b] - n:lens[b]] = s["kd"][b]
            vh[b, :, lens[b] - n:lens[b]] = s["vd"][b]
        _sampled(gs["od"], s["qd"], kh, vh, lens, "decode", 100 + t)
        drafts_o, _ = oracle.verify(s["dlog"], np.zeros((B, n), np.int64))
        assert np.array_equal(gs["drafts"].cpu().numpy(), drafts_o)
        assert np.array_equal(drafts_o, s["drafts"].numpy())               # the planted peaks
        # oracle: validation pass
        for b in range(B):
            kh[b, :, lens[b] - n:lens[b]] = s["kv"][b]
            vh[b, :, lens[b] - n:lens[b]] = s["vv"][b]
        _sampled(gs["ov"], s["qv"], kh, vh, lens, "causal", 200 + t)
        am_o, acc_o = oracle.verify(s["vlog"], drafts_o)
        assert np.array_equal(gs["am"].cpu().numpy(), am_o)
        assert np.array_equal(gs["acc"].cpu().numpy(), acc_o)
        assert np.array_equal(acc_o, s["accept"].numpy())                  # the planted accept lengths
        lens = np.minimum(lens + acc_o, CAP)
        assert np.array_equal(gs["kl"].cpu().numpy(), lens)
        assert _same(gs["kc"].cpu(), kh) and _same(gs["vc"].cpu(), vh), f"step {t}: cache contents"
        total += int(acc_o.sum())
    say(f"[spec] {STEPS} replays, {total} drafts accepted; final lengths {lens.tolist()}")
