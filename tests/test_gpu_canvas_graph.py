"""One denoise step of the multimodal canvas captured in a HIP graph.

The step of [DGemma] "정적 캐시 및 컴파일" (a static cache, so the decoder
step can be captured) with the stopping rule of "적응형 중단": write the
active block's K/V rows into the cache; DECODE attention of the block's
queries over the cache; row statistics (confidence, argmax, entropy and the
group mean entropy); the adaptive-stop update; the confidence commit.  The
statistics and the commit run as two calls or as the one call that reads
the logits once.  Seeded queries, rows and logits stand in for the model.

The step is captured once and replayed for several steps, with fresh inputs
copied in and other work run eagerly between the replays.  Every replay is
compared bit for bit with the same step run eagerly from the same state:
attention output, statistics, stopping state, tokens and commit mask (the
kernels are deterministic, so any difference is a capture fault).  Each call
is checked against the oracle by its own tests.
"""
import pytest
import torch

import synth
from gpu_util import dev, say

pytestmark = pytest.mark.gpu

bda = pytest.importorskip("block_masked_attention_amd")

STEPS = 6
B, Hq, Hkv, d = 2, 32, 8, 128
n = synth.CANVAS_BLOCK
V = synth.VOCAB
CAP = synth.PREFIX + synth.CANVAS


class Canvas:
    """State (cache, commit and stopping state), inputs and outputs of a step."""

    def __init__(self, kc0, vc0):
        D = dev()
        bf, u8, i32, i64, f32 = torch.bfloat16, torch.uint8, torch.int32, torch.int64, torch.float32
        self.kc, self.vc = kc0.to(D).clone(), vc0.to(D).clone()
        self.kl = torch.full((B,), synth.PREFIX + n, dtype=i32, device=D)
        self.q = torch.empty(B, Hq, n, d, dtype=bf, device=D)
        self.kb = torch.empty(B, Hkv, n, d, dtype=bf, device=D)
        self.vb = torch.empty_like(self.kb)
        self.logits = torch.empty(B, n, V, dtype=bf, device=D)
        self.out = torch.empty_like(self.q)
        self.tokens = torch.full((B, n), -1, dtype=i64, device=D)
        self.masked = torch.ones(B, n, dtype=u8, device=D)
        self.conf = torch.empty(B, n, dtype=f32, device=D)
        self.am = torch.empty(B, n, dtype=i64, device=D)
        self.ent = torch.empty(B, n, dtype=f32, device=D)
        self.mean = torch.empty(B, dtype=f32, device=D)
        self.prev = torch.full((B, n), -1, dtype=i64, device=D)
        self.stable = torch.zeros(B, dtype=i32, device=D)
        self.frozen = torch.zeros(B, dtype=u8, device=D)
        self.nfz = torch.zeros(1, dtype=i32, device=D)
        self.ws_a = torch.empty(max(1, bda.attn_workspace_bytes(B, Hq, Hkv, CAP, d, n, "decode")), dtype=u8, device=D)
        self.ws_s = torch.empty(int(bda.lib.bda_row_stats_workspace_bytes(B, n, V)), dtype=u8, device=D)
        self.ws_c = torch.empty(int(bda.lib.bda_commit_workspace_bytes(B, n, V)), dtype=u8, device=D)

    def load(self, s):
        q, kb, vb, lg, _ = s
        self.q.copy_(q)
        self.kb.copy_(kb)
        self.vb.copy_(vb)
        self.logits.copy_(lg)

    def run(self, fused):
        bda.kv_append(self.kc, self.vc, self.kb, self.vb, self.kl)
        bda.attn_fwd_varlen(self.q, self.kc, self.vc, self.kl, "decode", n, out=self.out, workspace=self.ws_a)
        stats = (self.conf, self.am, self.ent, self.mean)
        if fused:      # statistics and commit from one pass over the logits
            bda.row_stats_commit(self.logits, self.tokens, self.masked, 0.9, 1, workspace=self.ws_c, out=stats)
            bda.adaptive_stop(self.am, self.prev, self.stable, self.frozen, self.mean, 1, 0.005, n_frozen=self.nfz)
        else:
            bda.row_stats(self.logits, workspace=self.ws_s, out=stats)
            bda.adaptive_stop(self.am, self.prev, self.stable, self.frozen, self.mean, 1, 0.005, n_frozen=self.nfz)
            bda.commit(self.logits, self.tokens, self.masked, 0.9, 1, workspace=self.ws_c)

    def snapshot(self):
        names = ("out", "conf", "am", "ent", "mean", "prev", "stable", "frozen", "nfz", "tokens", "masked")
        snap = {k: getattr(self, k).clone() for k in names}
        snap["block_rows"] = self.kc[:, :, synth.PREFIX:synth.PREFIX + n].clone()
        return snap


def _same(a, b):
    if a.dtype.is_floating_point:
        return torch.equal(a.view(torch.int16 if a.element_size() == 2 else torch.int32),
                           b.view(torch.int16 if b.element_size() == 2 else torch.int32))
    return torch.equal(a, b)


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
def test_canvas_step_graph_replays_match_eager(fused):
    g = torch.Generator().manual_seed(31)
    kc0 = (torch.randn(B, Hkv, CAP, d, generator=g) * 0.5).to(torch.bfloat16)
    vc0 = (torch.randn(B, Hkv, CAP, d, generator=g) * 0.5).to(torch.bfloat16)
    steps = [synth.multimodal_step(t, n, B=B) for t in range(STEPS)]
    say(f"[canvas graph] B={B} n={n} cache {CAP} keys {synth.PREFIX + n} V={V}: warm-up launches")
    warm = Canvas(kc0, vc0)                    # first launches outside the capture
    warm.load(steps[0])
    warm.run(fused)
    torch.cuda.synchronize()
    del warm
    gc, ec = Canvas(kc0, vc0), Canvas(kc0, vc0)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gc.run(fused)
    torch.cuda.synchronize()
    spare = torch.randn(1 << 20, device=dev())
    for t in range(STEPS):
        say(f"[canvas graph] step {t}")
        gc.load(steps[t])
        ec.load(steps[t])
        spare.mul_(1.0001).add_(0.5)            # other work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        gs = gc.snapshot()
        ec.run(fused)
        torch.cuda.synchronize()
        es = ec.snapshot()
        for key in gs:
            assert _same(gs[key], es[key]), f"step {t}: graph replay and eager run differ in {key}"
        assert torch.isfinite(gs["out"].float()).all() and torch.isfinite(gs["conf"]).all()
    # the commit made progress: at least one token per group and step (k_min = 1)
    committed = (gs["masked"] == 0).sum(dim=1)
    assert (committed >= STEPS).all(), committed.tolist()
