"""Seeded synthetic inputs for block-diffusion attention and the confidence commit.

This module only draws random numbers and lays them out.  It holds none of the
method's arithmetic (no mask, no softmax, no argmax search): both the HIP path
and the CPU oracle consume the bytes it returns, and neither imports the other.

All draws use ``torch.Generator().manual_seed(seed)`` on the CPU, in the order
written below.  Floating values are drawn as fp32 ``randn() * sigma`` (sigma is
a standard deviation) and cast to bfloat16 with round-to-nearest-even where the
workload is bf16.

Workload shapes follow the pages' parameters: block 28 and threshold 0.85
(Nemotron-Labs-Diffusion-VLM-8B usage page, "basic usage"), canvas 256 and 48
steps with threshold 0.9 (diffusers DiffusionGemma page, "Usage" and
"Schedulers"), a 1540x1540 image cut into 14x14 patches with a 2x2 merge
(VLM-8B page, "high-resolution image support").
"""
from __future__ import annotations

import dataclasses
import math

import torch

VOCAB = 131072


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(int(seed))
    return g


def normal(shape, sigma: float, g: torch.Generator, dtype=torch.bfloat16) -> torch.Tensor:
    """fp32 N(0, sigma^2) draw, cast to ``dtype`` (RNE for bf16)."""
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if sigma != 1.0:
        x = x * sigma
    return x.to(dtype)


def planted_logits(G: int, R: int, V: int, sigma: float, g: torch.Generator,
                   dtype=torch.bfloat16, lo: float = 2.0, hi: float = 12.0, idx=None):
    """Noise logits with one planted peak per row.

    Each row is N(0, sigma^2) noise (cast to ``dtype``); a uniformly drawn
    index (or the given ``idx`` [G, R]) is then overwritten with (largest
    noise value of that row) + U(lo, hi), cast to ``dtype``.  The planted index
    is returned: it is the row's unique largest entry by construction (the gap
    is at least ``lo`` before rounding).  Draw order: noise, planted indices
    (when not given), offsets.
    """
    noise = normal((G, R, V), sigma, g, dtype)
    if idx is None:
        idx = torch.randint(0, V, (G, R), generator=g, dtype=torch.int64)
    else:
        idx = idx.to(torch.int64).clone()
    off = lo + (hi - lo) * torch.rand(G, R, generator=g, dtype=torch.float32)
    top = noise.float().amax(dim=-1)
    peak = (top + off).to(dtype)
    noise.scatter_(-1, idx.unsqueeze(-1), peak.unsqueeze(-1))
    return noise, idx


def redraw_rows(logits: torch.Tensor, idx: torch.Tensor, rows, seed: int, sigma: float,
                lo: float = 2.0, hi: float = 12.0):
    """Deterministically redraw the listed (g, r) rows in place.

    Used to keep threshold decisions away from the guard band: the caller
    decides which rows to redraw; this function only draws new noise and a new
    plant for them from ``seed``, in the listed order.
    """
    g = _gen(seed)
    V = logits.shape[-1]
    for (gi, ri) in rows:
        row = normal((V,), sigma, g, logits.dtype)
        j = int(torch.randint(0, V, (1,), generator=g).item())
        off = lo + (hi - lo) * torch.rand(1, generator=g).item()
        row[j] = (row.float().max() + off).to(logits.dtype)
        logits[gi, ri] = row
        idx[gi, ri] = j
    return logits, idx


# --------------------------------------------------------------------------
# Workloads (shapes and seeds).  "L" below is the per-half length in the
# training form and the total KV length in the decode/verify forms.
# --------------------------------------------------------------------------

@dataclasses.dataclass
class AttnCase:
    mode: str            # "hybrid" | "decode" | "causal"
    q: torch.Tensor      # [B, Hq, Sq, d]
    k: torch.Tensor      # [B, Hkv, Sk, d]
    v: torch.Tensor      # [B, Hkv, Sk, d]
    L: int
    block: int


def tiny(seed_qkv: int = 0, seed_mask: int = 1):
    """Tiny case: B=1, L=64 per half, block 4, Hq=Hkv=2, d=32, fp32 N(0,1)
    Q/K/V; then fp32 logits [1,64,1000] with sigma 2 from the same stream;
    masked [1,64] ~ Bernoulli(0.5) from ``seed_mask``."""
    g = _gen(seed_qkv)
    q = normal((1, 2, 128, 32), 1.0, g, torch.float32)
    k = normal((1, 2, 128, 32), 1.0, g, torch.float32)
    v = normal((1, 2, 128, 32), 1.0, g, torch.float32)
    logits = normal((1, 64, 1000), 2.0, g, torch.float32)
    gm = _gen(seed_mask)
    masked = (torch.rand(1, 64, generator=gm) < 0.5).to(torch.uint8)
    return AttnCase("hybrid", q, k, v, L=64, block=4), logits, masked


def hybrid_train(seed: int = 2, B: int = 4, L: int = 2048, block: int = 32,
                 Hq: int = 32, Hkv: int = 8, d: int = 128) -> AttnCase:
    """Training form over [x_t ; x_0]: Q [B,Hq,2L,d], K/V [B,Hkv,2L,d] bf16 N(0,1)."""
    g = _gen(seed)
    q = normal((B, Hq, 2 * L, d), 1.0, g)
    k = normal((B, Hkv, 2 * L, d), 1.0, g)
    v = normal((B, Hkv, 2 * L, d), 1.0, g)
    return AttnCase("hybrid", q, k, v, L=L, block=block)


def decode_block(seed: int = 3, B: int = 32, prefix: int = 4096, n: int = 28,
                 Hq: int = 32, Hkv: int = 8, d: int = 128) -> AttnCase:
    """Decode form: an active block of n queries over prefix + own block keys."""
    g = _gen(seed)
    q = normal((B, Hq, n, d), 1.0, g)
    k = normal((B, Hkv, prefix + n, d), 1.0, g)
    v = normal((B, Hkv, prefix + n, d), 1.0, g)
    return AttnCase("decode", q, k, v, L=prefix + n, block=n)


def verify_block(seed: int = 5, B: int = 16, cache: int = 8192, n: int = 28,
                 Hq: int = 32, Hkv: int = 8, d: int = 128) -> AttnCase:
    """Verify form: n drafted queries, causal over cache + drafts (bottom-right)."""
    g = _gen(seed)
    q = normal((B, Hq, n, d), 1.0, g)
    k = normal((B, Hkv, cache + n, d), 1.0, g)
    v = normal((B, Hkv, cache + n, d), 1.0, g)
    return AttnCase("causal", q, k, v, L=cache + n, block=n)


def commit_logits(seed: int = 4, G: int = 32, R: int = 28, V: int = VOCAB, sigma: float = 3.0):
    """bf16 logits [G,R,V] with planted peaks; every position still masked."""
    g = _gen(seed)
    logits, idx = planted_logits(G, R, V, sigma, g)
    masked = torch.ones(G, R, dtype=torch.uint8)
    return logits, idx, masked


def verify_drafts(planted_idx: torch.Tensor, seed: int = 7, p: float = 0.2, V: int = VOCAB):
    """Drafts that agree with the planted peaks for a geometric-length prefix.

    accept_b ~ Geometric(p) - 1 (number of failures before the first success),
    capped at R.  drafts[b, j] = planted[b, j] for j < accept_b; at j = accept_b
    the draft is (planted + 1 + r) mod V with r ~ U[0, V-1) so it differs; later
    positions are uniform ids.  Returns (drafts int64 [B,R], planted accept [B]).
    """
    B, R = planted_idx.shape
    g = _gen(seed)
    u = torch.rand(B, generator=g, dtype=torch.float64)
    acc = torch.floor(torch.log1p(-u) / math.log1p(-p)).to(torch.int64).clamp(max=R)
    r = torch.randint(0, V - 1, (B,), generator=g, dtype=torch.int64)
    rest = torch.randint(0, V, (B, R), generator=g, dtype=torch.int64)
    drafts = rest.clone()
    for b in range(B):
        a = int(acc[b])
        drafts[b, :a] = planted_idx[b, :a]
        if a < R:
            drafts[b, a] = (planted_idx[b, a] + 1 + r[b]) % V
    return drafts, acc


# --------------------------------------------------------------------------
# Long multimodal prefill + canvas
# --------------------------------------------------------------------------

IMAGE_SIDE = 1540
PATCH = 14
MERGE = 2
GRID = IMAGE_SIDE // PATCH // MERGE          # 55 merged tokens per image row
IMAGE_TOKENS = GRID * GRID                   # 3025
ROW_BREAKS = GRID                            # one break token per image row
TEXT_TOKENS = 1016
PREFIX = IMAGE_TOKENS + ROW_BREAKS + TEXT_TOKENS   # 4096
CANVAS = 256
CANVAS_BLOCK = 28


def canvas_blocks(canvas: int = CANVAS, block: int = CANVAS_BLOCK):
    """Block lengths of the canvas: full blocks, then a short last block."""
    out = [block] * (canvas // block)
    if canvas % block:
        out.append(canvas % block)
    return out


def multimodal_prefill(seed: int = 8, B: int = 2, Hq: int = 32, Hkv: int = 8, d: int = 128) -> AttnCase:
    g = _gen(seed)
    q = normal((B, Hq, PREFIX, d), 1.0, g)
    k = normal((B, Hkv, PREFIX, d), 1.0, g)
    v = normal((B, Hkv, PREFIX, d), 1.0, g)
    return AttnCase("causal", q, k, v, L=PREFIX, block=PREFIX)


def multimodal_step(step: int, n: int, B: int = 2, Hq: int = 32, Hkv: int = 8, d: int = 128,
                    V: int = VOCAB, sigma: float = 3.0):
    """Per denoise step ``step`` (seed 100+step): the active block's queries,
    its fresh K/V rows (written into the cache at the block's position) and
    the canvas logits [B, n, V] with planted peaks."""
    g = _gen(100 + step)
    q = normal((B, Hq, n, d), 1.0, g)
    kb = normal((B, Hkv, n, d), 1.0, g)
    vb = normal((B, Hkv, n, d), 1.0, g)
    logits, idx = planted_logits(B, n, V, sigma, g)
    return q, kb, vb, logits, idx


def prefix_modality() -> torch.Tensor:
    """Modality of the multimodal prefix positions (uint8 [PREFIX]): the image
    span (merged image tokens and their row breaks) is 1, the text tail 0."""
    m = torch.zeros(PREFIX, dtype=torch.uint8)
    m[:IMAGE_TOKENS + ROW_BREAKS] = 1
    return m


def sprint_prefix(seed: int = 9, B: int = 2, Hkv: int = 8, d: int = 128, L: int = PREFIX,
                  key_spread: float = 0.25):
    """Prefix cache and per-position confidence for SPRINT pruning.

    k, v [B, Hkv, L, d] bf16: N(0, 1) draws; each key row of position (b, i)
    is scaled (in fp32, before the bf16 cast) by exp(key_spread * z_{b,i}),
    z ~ N(0, 1) shared by the kv heads, so key norms vary across positions.
    conf [B, L] fp32: U(0.05, 1).  Draw order: k, z, v, conf."""
    g = _gen(seed)
    k = torch.randn(B, Hkv, L, d, generator=g, dtype=torch.float32)
    z = torch.randn(B, 1, L, 1, generator=g, dtype=torch.float32)
    k = (k * torch.exp(key_spread * z)).to(torch.bfloat16)
    v = normal((B, Hkv, L, d), 1.0, g)
    conf = 0.05 + 0.95 * torch.rand(B, L, generator=g, dtype=torch.float32)
    return k, v, conf


# --------------------------------------------------------------------------
# Linear speculative loop with per-sequence cache lengths
# --------------------------------------------------------------------------

def spec_prefix(seed: int = 20, prefix=(517, 1000, 2345, 3000), cap: int = 3328, n: int = 28,
                Hkv: int = 8, d: int = 128):
    """Cache [B, Hkv, cap, d] bf16 N(0, 1) (rows past each prefix are filled
    too, so a read past a sequence's length would show) and the starting
    per-sequence key counts kv_len = prefix + n (int32)."""
    g = _gen(seed)
    B = len(prefix)
    k = normal((B, Hkv, cap, d), 1.0, g)
    v = normal((B, Hkv, cap, d), 1.0, g)
    kv_len = torch.tensor([p + n for p in prefix], dtype=torch.int32)
    return k, v, kv_len


def spec_step(step: int, B: int = 4, n: int = 28, Hq: int = 32, Hkv: int = 8, d: int = 128,
              V: int = 32768, sigma: float = 3.0, p: float = 0.25):
    """Inputs of speculative step ``step`` (seed 200 + step), in draw order:
    draft queries and block K/V rows, draft logits [B, n, V] with planted
    peaks (the drafts are their argmax), verify queries and block K/V rows,
    accept lengths a_b ~ Geometric(p) - 1 capped at n, and verify logits
    planted at the drafts for j < a_b, at a different id for j = a_b and at
    uniform ids after."""
    g = _gen(200 + step)
    qd = normal((B, Hq, n, d), 1.0, g)
    kd = normal((B, Hkv, n, d), 1.0, g)
    vd = normal((B, Hkv, n, d), 1.0, g)
    dlog, drafts = planted_logits(B, n, V, sigma, g)
    qv = normal((B, Hq, n, d), 1.0, g)
    kv = normal((B, Hkv, n, d), 1.0, g)
    vv = normal((B, Hkv, n, d), 1.0, g)
    u = torch.rand(B, generator=g, dtype=torch.float64)
    acc = torch.floor(torch.log1p(-u) / math.log1p(-p)).to(torch.int64).clamp(max=n)
    r = torch.randint(0, V - 1, (B,), generator=g, dtype=torch.int64)
    vidx = torch.randint(0, V, (B, n), generator=g, dtype=torch.int64)
    for b in range(B):
        a = int(acc[b])
        vidx[b, :a] = drafts[b, :a]
        if a < n:
            vidx[b, a] = (drafts[b, a] + 1 + r[b]) % V
    vlog, _ = planted_logits(B, n, V, sigma, g, idx=vidx)
    return dict(qd=qd, kd=kd, vd=vd, dlog=dlog, drafts=drafts, qv=qv, kv=kv, vv=vv, vlog=vlog, accept=acc)


def varlen_case(seed: int, B: int, Hq: int, Hkv: int, d: int, n: int, cap: int):
    """q [B, Hq, n, d] and a cache k, v [B, Hkv, cap, d], bf16 N(0, 1), drawn
    in that order."""
    g = _gen(seed)
    q = normal((B, Hq, n, d), 1.0, g)
    k = normal((B, Hkv, cap, d), 1.0, g)
    v = normal((B, Hkv, cap, d), 1.0, g)
    return q, k, v


def spread_logits(seed: int, G: int, R: int, V: int, dtype=torch.bfloat16):
    """Logits [G, R, V] whose rows range from nearly uniform to sharply
    peaked: row noise N(0, sigma_r^2) with sigma_r ~ U(0.3, 4), then, in about
    half the rows, one uniformly drawn index raised to the row's largest noise
    value + U(0, 12).  Draw order: sigmas, noise, peak flags, indices, offsets."""
    g = _gen(seed)
    sig = 0.3 + 3.7 * torch.rand(G, R, 1, generator=g, dtype=torch.float32)
    x = torch.randn(G, R, V, generator=g, dtype=torch.float32) * sig
    flag = torch.rand(G, R, generator=g, dtype=torch.float32) < 0.5
    idx = torch.randint(0, V, (G, R), generator=g, dtype=torch.int64)
    off = 12.0 * torch.rand(G, R, generator=g, dtype=torch.float32)
    x = x.to(dtype)
    top = x.float().amax(dim=-1)
    peak = (top + off).to(dtype)
    cur = x.gather(-1, idx.unsqueeze(-1)).squeeze(-1)
    x.scatter_(-1, idx.unsqueeze(-1), torch.where(flag, peak, cur).unsqueeze(-1))
    return x
