#!/usr/bin/env python3
"""Benchmark of the block-diffusion hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary] [--no-cpu]

Headline step: one training-form hybrid attention forward over [x_t ; x_0]
(B=4, L=2048 per half, block 32, Hq=32, Hkv=8, d=128, bf16, synthetic
N(0,1) inputs resident in HBM).  `value` = unmasked TFLOP/s, counting
4*d FLOPs per allowed (query, key) pair per query head.

Secondary lines (same JSON object): decode-form and verify-form attention,
the confidence commit (committed tokens/s and HBM GB/s) and verify, each
timed per launch with HIP events on the stream the kernels run on, with
rotated input buffers for the HBM-bound ones so that the 256 MB last-level
cache cannot serve repeated reads.

`--copy-calibration` runs only a plain device copy of known size (for
scaling rocprofv3 FETCH_SIZE/WRITE_SIZE counters to bytes).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0
METRIC = "block-diffusion attn TFLOP/s (unmasked) & %MFMA peak; commit tokens/s & %HBM peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def hybrid_pairs(L, b):
    """Allowed (query, key) pairs of one head of the training form (closed form)."""
    tot = 0
    for s in range(0, L, b):
        n = min(b, L - s)
        tot += n * (s + n)
    return 2 * tot


def decode_pairs(L, n):
    return n * L


def causal_pairs(L, n):
    return n * (L - n) + n * (n + 1) // 2


_FILL = None   # (source, destination, ms per copy) of the queue filler


def _queue_fill(ms):
    """Keep the GPU streaming memory for about ms milliseconds: device copies
    between two 512 MB buffers, enqueued in well under a millisecond.  A GPU
    left nearly idle instead (a one-workgroup spin) lets the memory-side
    clocks drop, and HBM-bound calls queued behind it then ran ~15% slower
    than in steady state (decode attention 127 against 110 us)."""
    global _FILL
    import torch
    if _FILL is None:
        src = torch.zeros(1 << 28, dtype=torch.float16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(5):
            dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        _FILL = (src, dst, max(a.elapsed_time(b) / 5, 1e-3))
    src, dst, per = _FILL
    for _ in range(int(ms / per) + 1):
        dst.copy_(src)


def time_launches(fn, iters, warmup, pre=None, queue=True):
    """Mean and median per-launch ms of fn(i) with HIP events on the current
    stream.  The timed launches are queued behind enough memory-streaming
    work for the host to enqueue all of them, so each event pair measures the
    GPU's back-to-back time for the call and not the host's launch overhead
    (the ctypes call and argument checks take tens of microseconds, as long
    as a small kernel).  queue=False times each call as the host issues it."""
    import time
    import torch
    t0 = time.perf_counter()
    for i in range(warmup):
        if pre:
            pre(i)
        fn(i)
    torch.cuda.synchronize()
    host_ms = (time.perf_counter() - t0) * 1e3 / max(warmup, 1)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    if queue:
        _queue_fill(min(2.0 * host_ms * iters + 1.0, 200.0))
    for i in range(iters):
        if pre:
            pre(i)
        starts[i].record()
        fn(i)
        ends[i].record()
    torch.cuda.synchronize()
    ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return sum(ms) / len(ms), ms[len(ms) // 2]


def copy_calibration():
    import torch
    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n, "launches": 5}))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads():
    """Threads the CPU baseline runs on, and what they were derived from: the
    CPUs this process may run on (affinity), capped by OMP_NUM_THREADS when
    it is set (the host's CPU share where the machine is shared)."""
    nproc = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = nproc
    omp_env = os.environ.get("OMP_NUM_THREADS")
    threads = affinity
    try:
        if omp_env is not None and int(omp_env.split(",")[0]) > 0:
            threads = min(threads, int(omp_env.split(",")[0]))
    except ValueError:
        pass
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as fh:
            q, per = fh.read().split()[:2]
            if q != "max":
                quota = round(int(q) / int(per), 2)
    except (OSError, ValueError):
        pass
    return threads, {"nproc": nproc, "affinity": affinity, "OMP_NUM_THREADS": omp_env, "cgroup_cpus": quota}


def cpu_baseline_attention(case, budget_s=20.0, min_s=10.0):
    """The oracle, untuned, on a bounded sample of the same workload: every
    row of the query heads of the first kv head(s) of batch 0, the number of
    kv heads doubled until one call takes about a quarter of budget_s, then
    repeated until at least min_s seconds have been timed."""
    import oracle
    L, blk = case.L, case.block
    rows = 2 * L
    pairs_per_head = hybrid_pairs(L, blk)
    d = case.q.shape[-1]
    G = case.q.shape[1] // case.k.shape[1]
    Hkv, B = case.k.shape[1], case.q.shape[0]
    nt, host = host_threads()
    kvh, nb = 1, 1
    while True:
        heads = G * kvh
        t0 = time.perf_counter()
        oracle.attention("hybrid", case.q[:nb, :heads], case.k[:nb, :kvh], case.v[:nb, :kvh], L, blk, nthreads=nt)
        dt = time.perf_counter() - t0
        flops = 4 * d * pairs_per_head * heads * nb
        if dt > budget_s / 4 or (kvh == Hkv and nb == B):
            break
        if kvh < Hkv:
            kvh = min(Hkv, kvh * 2)
        else:
            nb = min(B, nb * 2)
    # the whole workload can take less than min_s: repeat it and take the mean
    calls, total = 1, dt
    while total < min_s:
        t0 = time.perf_counter()
        oracle.attention("hybrid", case.q[:nb, :heads], case.k[:nb, :kvh], case.v[:nb, :kvh], L, blk, nthreads=nt)
        total += time.perf_counter() - t0
        calls += 1
    # one thread, on one kv head of batch 0 (its G query heads)
    t0 = time.perf_counter()
    oracle.attention("hybrid", case.q[:1, :G], case.k[:1, :1], case.v[:1, :1], L, blk, nthreads=1)
    dt1 = time.perf_counter() - t0
    flops1 = 4 * d * pairs_per_head * G
    return {"value": flops * calls / total / 1e12, "unit": "TFLOP/s", "cores": nt, "kind": "oracle",
            "cpu": _cpu_model(), "host": host, "sample": f"all {rows} rows of {heads} query heads ({kvh} kv heads) of {nb} batch(es) "
                      f"({flops / 1e9:.1f} GFLOP per call, {calls} call(s), {total:.1f} s)",
            "single_thread": {"value": flops1 / dt1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                              "sample": f"all {rows} rows of {G} query heads (1 kv head) of batch 0 "
                                        f"({flops1 / 1e9:.1f} GFLOP, {dt1:.1f} s)"}}


def cpu_baseline_commit(logits, masked, tau, k_min, min_s=10.0):
    import numpy as np
    import oracle
    G = logits.shape[0]
    g = G                                   # the whole commit call is well under a minute of CPU work
    tokens = np.full((g, logits.shape[1]), -1, dtype=np.int64)
    nt, host = host_threads()
    calls, dt = 0, 0.0
    while dt < min_s:                       # the oracle returns new arrays: every call does the whole commit
        t0 = time.perf_counter()
        _, m, _ = oracle.commit(logits[:g], masked[:g].numpy(), tokens, tau, k_min, nthreads=nt)
        dt += time.perf_counter() - t0
        calls += 1
    committed = int(masked[:g].numpy().sum() - m.sum())
    t0 = time.perf_counter()
    oracle.commit(logits[:g], masked[:g].numpy(), tokens, tau, k_min, nthreads=1)
    dt1 = time.perf_counter() - t0
    return {"value": committed * calls / dt, "unit": "committed tokens/s", "cores": nt,
            "kind": "oracle", "cpu": _cpu_model(), "host": host,
            "sample": f"{g} of {G} groups ({committed} tokens per call, {calls} calls, {dt:.1f} s)",
            "single_thread": {"value": committed / dt1, "unit": "committed tokens/s", "cores": 1,
                              "sample": f"{g} of {G} groups, one call ({dt1:.2f} s)"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="untimed launches continue for this many seconds after the warm-up steps")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the kernels run on one GPU's share "
              "of the work, and sharding across GPUs is not implemented.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    import block_masked_attention_amd as bda
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---------------- headline: training-form hybrid attention
    case = synth.hybrid_train()
    B, Hq, S2, d = case.q.shape
    Hkv, L, blk = case.k.shape[1], case.L, case.block
    flops = 4 * d * hybrid_pairs(L, blk) * B * Hq
    q, k, v = case.q.to(dev), case.k.to(dev), case.v.to(dev)
    out = torch.empty_like(q)
    log(f"[bench] training form: {flops / 1e9:.1f} GFLOP unmasked per step")
    for _ in range(args.warmup):
        bda.attn_fwd(q, k, v, "hybrid", blk, out=out)
    torch.cuda.synchronize()
    # Settle: the first few dozen launches of a fresh process run up to 30%
    # slower (clocks still ramping), so untimed launches continue for at
    # least settle_s seconds of GPU time before the K timed steps.
    settle_n, t_set = 0, time.perf_counter()
    while time.perf_counter() - t_set < args.settle_s:
        for _ in range(10):
            bda.attn_fwd(q, k, v, "hybrid", blk, out=out)
        settle_n += 10
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_set
    log(f"[bench] settle: {settle_n} untimed launches over {settle_s:.2f} s after {args.warmup} warm-up launches")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        bda.attn_fwd(q, k, v, "hybrid", blk, out=out)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"[bench] training form: {ms * 1e3:.1f} us/step, {tflops:.1f} TFLOP/s "
        f"({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of bf16 MFMA peak)")
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "attn_hybrid_B4_L2048_b32_traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            tr = json.load(f)
        if tr.get("kernel_source_sha") == _kernel_sha():
            traffic = tr.get("bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"launches": settle_n, "seconds": round(settle_s, 3)},
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "training-form block-diffusion attention over [x_t;x_0]",
                   "B": B, "L": L, "seq_2L": S2, "block": blk, "Hq": Hq, "Hkv": Hkv, "head_dim": d,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
    }
    del q, k, v, out

    if not args.no_secondary:
        result["secondary"] = secondary(bda, synth, torch, dev, args)
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a sample of the training form")
        result["cpu_baseline"] = cpu_baseline_attention(case)
        log(f"[bench] cpu baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)


def _kernel_sha():
    import hashlib
    h = hashlib.sha256()
    for f in ("attn.hip", "attn_index.h", "common.h", "geometry.h", "tiles.h"):
        with open(os.path.join(ROOT, "block_masked_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def secondary(bda, synth, torch, dev, args):
    res = {}
    iters = max(20, args.steps)
    # ---- decode-form attention (B=32, 28 queries over 4096 + 28 keys)
    for name, maker, pairs in (("decode_attention", synth.decode_block, decode_pairs),
                               ("verify_attention", synth.verify_block, causal_pairs)):
        case = maker()
        B, Hq, n, d = case.q.shape
        L = case.L
        fl = 4 * d * pairs(L, n) * B * Hq
        sets = [(case.q.to(dev), case.k.to(dev), case.v.to(dev))]
        g = torch.Generator(device=dev).manual_seed(1)
        for _ in range(2):     # two more K/V sets so repeated launches stream from HBM
            sets.append((sets[0][0], torch.randn(case.k.shape, generator=g, device=dev).to(torch.bfloat16),
                         torch.randn(case.v.shape, generator=g, device=dev).to(torch.bfloat16)))
        out = torch.empty_like(sets[0][0])
        ws = torch.empty(max(1, bda.attn_workspace_bytes(B, Hq, case.k.shape[1], L, d, n, case.mode)),
                         dtype=torch.uint8, device=dev)
        mean, med = time_launches(lambda i: bda.attn_fwd(*sets[i % 3], case.mode, n, out=out, workspace=ws),
                                  iters, 5)
        byts = (case.q.numel() * 2 * 2) + case.k.numel() * 2 * 2
        res[name] = {"B": B, "n": n, "kv_len": L, "us_per_call": round(mean * 1e3, 2),
                     "TFLOP/s": round(fl / (mean * 1e-3) / 1e12, 2),
                     "mfma_frac": round(fl / (mean * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "GB/s": round(byts / (mean * 1e-3) / 1e9, 1),
                     "hbm_frac": round(byts / (mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "algorithmic_bytes": byts}
        log(f"[bench] {name}: {res[name]}")
        del sets, out, ws
        torch.cuda.empty_cache()

    # ---- training-form backward (dq, dk, dv) on the headline workload:
    # 2.5x the forward's unmasked FLOPs (dS, dP, dQ, dK, dV: five products)
    case = synth.hybrid_train()
    B, Hq, S, d = case.q.shape
    q, k, v = case.q.to(dev), case.k.to(dev), case.v.to(dev)
    do = torch.randn(q.shape, generator=torch.Generator(device=dev).manual_seed(3), device=dev).to(torch.bfloat16)
    lse = torch.empty(B, Hq, S, dtype=torch.float32, device=dev)
    out = bda.attn_fwd(q, k, v, "hybrid", case.block, lse=lse)
    bws = torch.empty(bda.lib.bda_attn_bwd_workspace_bytes(B, Hq, k.shape[1], case.L, d, case.block, 0),
                      dtype=torch.uint8, device=dev)
    mean, med = time_launches(lambda i: bda.attn_bwd(q, k, v, out, do, lse, case.block, workspace=bws), iters, 5)
    fl = 2.5 * 4 * d * hybrid_pairs(case.L, case.block) * B * Hq
    res["training_backward"] = {"B": B, "L": case.L, "block": case.block, "us_per_call": round(mean * 1e3, 2),
                                "TFLOP/s": round(fl / (mean * 1e-3) / 1e12, 2),
                                "mfma_frac": round(fl / (mean * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    log(f"[bench] training_backward: {res['training_backward']}")
    del q, k, v, do, lse, out, bws
    torch.cuda.empty_cache()

    # ---- multimodal prefill: causal over the 4096-token prefix, B=2
    case = synth.multimodal_prefill()
    B, Hq, n, d = case.q.shape
    L = case.L
    fl = 4 * d * causal_pairs(L, n) * B * Hq
    q, k, v = case.q.to(dev), case.k.to(dev), case.v.to(dev)
    out = torch.empty_like(q)
    mean, med = time_launches(lambda i: bda.attn_fwd(q, k, v, "causal", n, out=out), iters, 5)
    res["prefill_attention"] = {"B": B, "n": n, "kv_len": L, "us_per_call": round(mean * 1e3, 2),
                                "TFLOP/s": round(fl / (mean * 1e-3) / 1e12, 2),
                                "mfma_frac": round(fl / (mean * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    log(f"[bench] prefill_attention: {res['prefill_attention']}")
    del q, k, v, out
    torch.cuda.empty_cache()

    # ---- one canvas denoise step mid-canvas: decode attention of the 28-row
    # block over prefix + four finished blocks, then the commit (threshold
    # 0.9) on its [2, 28, 131072] logits.  Both are launch-latency bound; the
    # floors are their HBM bytes at 8 TB/s (the cache also fits the 256 MB
    # last-level cache, as it would between real steps).
    qs, kb, vb, lg, _ = synth.multimodal_step(0, 28)
    pre_k = torch.randn(2, 8, synth.PREFIX + 4 * 28, 128, generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    k = torch.cat([pre_k, kb], dim=2).to(dev)
    v = torch.cat([pre_k.flip(2), vb], dim=2).to(dev)
    qs, lg = qs.to(dev), lg.to(dev)
    L = k.shape[2]
    out = torch.empty_like(qs)
    ws = torch.empty(max(1, bda.attn_workspace_bytes(2, 32, 8, L, 128, 28, "decode")), dtype=torch.uint8, device=dev)
    t_att, _ = time_launches(lambda i: bda.attn_fwd(qs, k, v, "decode", 28, out=out, workspace=ws), iters, 5)
    tok = torch.full((2, 28), -1, dtype=torch.int64, device=dev)
    msk = torch.ones(2, 28, dtype=torch.uint8, device=dev)
    cws = torch.empty(bda.lib.bda_commit_workspace_bytes(2, 28, synth.VOCAB), dtype=torch.uint8, device=dev)
    t_com, _ = time_launches(lambda i: bda.commit(lg, tok, msk, 0.9, 1, workspace=cws), iters, 5,
                             pre=lambda i: msk.fill_(1))
    att_bytes = (qs.numel() * 2 * 2) + k.numel() * 2 * 2
    com_bytes = lg.numel() * 2
    res["canvas_step"] = {"B": 2, "n": 28, "kv_len": L, "attention_us": round(t_att * 1e3, 2),
                          "attention_floor_us": round(att_bytes / PEAK_HBM_GBS / 1e3, 2),
                          "commit_us": round(t_com * 1e3, 2),
                          "commit_floor_us": round(com_bytes / PEAK_HBM_GBS / 1e3, 2)}
    log(f"[bench] canvas_step: {res['canvas_step']}")
    del k, v, qs, lg, out, ws, cws
    torch.cuda.empty_cache()

    # ---- the canvas denoise step captured as one HIP graph: append the
    # active block's fresh K/V rows, DECODE attention over the cache (per-row
    # lengths on the device), row statistics, adaptive stopping and the
    # commit; and the number of steps the whole 256-position canvas takes
    res["canvas_graph"] = canvas_graph(bda, synth, torch, dev, iters)
    log(f"[bench] canvas_graph: {res['canvas_graph']}")
    torch.cuda.empty_cache()

    # ---- commit on decode-form logits [32, 28, 131072] bf16, threshold 0.85
    logits, idx, masked0 = synth.commit_logits()
    G, R, V = logits.shape
    sets = [logits.to(dev)]
    for j in range(2):
        sets.append(sets[0].roll(shifts=j + 1, dims=0).contiguous())
    tokens = torch.full((G, R), -1, dtype=torch.int64, device=dev)
    masked = masked0.to(dev)
    ws = torch.empty(bda.lib.bda_commit_workspace_bytes(G, R, V), dtype=torch.uint8, device=dev)
    committed = []

    def pre(i):
        masked.fill_(1)

    def run(i):
        bda.commit(sets[i % 3], tokens, masked, 0.85, 1, workspace=ws)

    mean, med = time_launches(run, iters, 5, pre=pre)
    torch.cuda.synchronize()
    n_commit = int(G * R - masked.sum().item())
    byts = G * R * V * 2
    res["commit"] = {"G": G, "R": R, "V": V, "threshold": 0.85, "k_min": 1,
                     "us_per_call": round(mean * 1e3, 2), "committed_per_call": n_commit,
                     "committed_tokens_per_s": round(n_commit / (mean * 1e-3), 1),
                     "GB/s": round(byts / (mean * 1e-3) / 1e9, 1),
                     "hbm_frac": round(byts / (mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "algorithmic_bytes": byts}
    log(f"[bench] commit: {res['commit']}")
    if not args.no_cpu:
        res["commit"]["cpu_baseline"] = cpu_baseline_commit(logits, masked0, 0.85, 1)

    # ---- row statistics (confidence, argmax, entropy) on the same logits
    sws = torch.empty(bda.lib.bda_row_stats_workspace_bytes(G, R, V), dtype=torch.uint8, device=dev)
    souts = (torch.empty(G, R, device=dev), torch.empty(G, R, dtype=torch.int64, device=dev),
             torch.empty(G, R, device=dev), torch.empty(G, device=dev))
    mean, med = time_launches(lambda i: bda.row_stats(sets[i % 3], workspace=sws, out=souts), iters, 5)
    res["row_stats"] = {"G": G, "R": R, "V": V, "us_per_call": round(mean * 1e3, 2),
                        "GB/s": round(byts / (mean * 1e-3) / 1e9, 1),
                        "hbm_frac": round(byts / (mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                        "algorithmic_bytes": byts}
    log(f"[bench] row_stats: {res['row_stats']}")

    # ---- entropy-bound commit on the same logits (bound 14 nats per group,
    # temperature 1, at least one commit)
    ews = torch.empty(bda.lib.bda_commit_entropy_workspace_bytes(G, R, V), dtype=torch.uint8, device=dev)

    def erun(i):
        bda.commit_entropy(sets[i % 3], tokens, masked, 14.0, 1.0, 1, workspace=ews)

    mean, med = time_launches(erun, iters, 5, pre=pre)
    torch.cuda.synchronize()
    n_commit = int(G * R - masked.sum().item())
    res["entropy_commit"] = {"G": G, "R": R, "V": V, "entropy_bound": 14.0, "us_per_call": round(mean * 1e3, 2),
                             "committed_per_call": n_commit,
                             "GB/s": round(byts / (mean * 1e-3) / 1e9, 1),
                             "hbm_frac": round(byts / (mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                             "algorithmic_bytes": byts}
    log(f"[bench] entropy_commit: {res['entropy_commit']}")

    # ---- SPRINT pruning of the multimodal prefix (B=2, 8 kv heads, 4096
    # positions: 3080 image, 1016 text; keep 0.8 of the image, all text), and
    # one decode step of a 28-row block over the pruned vs the full cache.
    pk, pv, pconf = synth.sprint_prefix()
    pmod = synth.prefix_modality()
    n_text = int((pmod == 0).sum())
    pk, pv, pconf, pmod = pk.to(dev), pv.to(dev), pconf.to(dev), pmod.to(dev)
    B, Hkv, L, d = pk.shape
    spws = torch.empty(bda.lib.bda_sprint_workspace_bytes(B, L), dtype=torch.uint8, device=dev)
    t_pr, _ = time_launches(lambda i: bda.sprint_prune(pk, pv, pconf, pmod, workspace=spws, n_text=n_text), iters, 5)
    ko, vo, _, _ = bda.sprint_prune(pk, pv, pconf, pmod, workspace=spws, n_text=n_text)
    K = ko.shape[2]
    qs, kb, vb, _, _ = synth.multimodal_step(0, 28)
    qs, kb, vb = qs.to(dev), kb.to(dev), vb.to(dev)
    step_us = {}
    for tag, (kk, vv) in (("full", (pk, pv)), ("pruned", (ko, vo))):
        kc, vc = torch.cat([kk, kb], dim=2), torch.cat([vv, vb], dim=2)
        out = torch.empty_like(qs)
        ws = torch.empty(max(1, bda.attn_workspace_bytes(B, 32, Hkv, kc.shape[2], d, 28, "decode")),
                         dtype=torch.uint8, device=dev)
        t, _ = time_launches(lambda i: bda.attn_fwd(qs, kc, vc, "decode", 28, out=out, workspace=ws), iters, 5)
        step_us[tag] = round(t * 1e3, 2)
    byts = pk.numel() * 2 + 2 * 2 * B * Hkv * K * d * 2          # norms read K; gather reads and writes K and V rows
    res["sprint_prune"] = {"B": B, "kv_heads": Hkv, "prefix": L, "kept": K, "us_per_call": round(t_pr * 1e3, 2),
                           "hbm_floor_us": round(byts / PEAK_HBM_GBS / 1e3, 2),
                           "decode_step_us_full_cache": step_us["full"],
                           "decode_step_us_pruned_cache": step_us["pruned"]}
    log(f"[bench] sprint_prune: {res['sprint_prune']}")
    del pk, pv, pconf, pmod, ko, vo, spws
    torch.cuda.empty_cache()

    # ---- one linear speculative step on the device, eager launches vs one
    # HIP graph replay: append the draft rows, DECODE attention, drafts =
    # argmax of the draft logits, append the validation rows, CAUSAL
    # attention, verify + crop.  16 sequences of ~8k cached keys, 28 drafts,
    # vocabulary 131072 (the verify workload's shapes); the lengths are reset
    # before each timed call.
    res["speculative_step"] = speculative_step(bda, synth, torch, dev, iters)
    log(f"[bench] speculative_step: {res['speculative_step']}")
    torch.cuda.empty_cache()

    # ---- verify on [16, 28, 131072] bf16
    vl, vidx, _ = synth.commit_logits(seed=6, G=16, R=28)
    drafts, _ = synth.verify_drafts(vidx)
    vsets = [vl.to(dev)] + [vl.to(dev).roll(shifts=j + 1, dims=0).contiguous() for j in range(2)]
    dr = drafts.to(dev)
    mean, med = time_launches(lambda i: bda.verify(vsets[i % 3], dr), iters, 5)
    byts = vl.numel() * 2
    res["verify"] = {"B": 16, "R": 28, "V": V, "us_per_call": round(mean * 1e3, 2),
                     "GB/s": round(byts / (mean * 1e-3) / 1e9, 1),
                     "hbm_frac": round(byts / (mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "algorithmic_bytes": byts}
    log(f"[bench] verify: {res['verify']}")
    return res


def canvas_graph(bda, synth, torch, dev, iters):
    """One denoise step of the multimodal canvas (B=2, 28-row active block,
    threshold 0.9, at least one commit) as eager launches and as one HIP
    graph replay, beside the HBM floors of its attention and commit (the
    step with row statistics and commit from one pass over the logits, and
    for comparison with the two as separate calls); then
    the whole canvas run block by block with the graph (the host reads the
    commit mask after each step to move to the next block), reporting the
    steps it took against the 48-step budget."""
    B, Hq, Hkv, d, V = 2, 32, 8, 128, synth.VOCAB
    n = synth.CANVAS_BLOCK
    cap = synth.PREFIX + synth.CANVAS
    pre = synth.multimodal_prefill()
    kc = torch.zeros(B, Hkv, cap, d, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    kc[:, :, :synth.PREFIX] = pre.k.to(dev)
    vc[:, :, :synth.PREFIX] = pre.v.to(dev)
    del pre
    u8, i32, i64, f32 = torch.uint8, torch.int32, torch.int64, torch.float32
    kl = torch.full((B,), synth.PREFIX + n, dtype=i32, device=dev)
    st = {}

    def buffers(nb):
        if nb in st:
            return st[nb]
        x = dict(q=torch.empty(B, Hq, nb, d, dtype=torch.bfloat16, device=dev),
                 kb=torch.empty(B, Hkv, nb, d, dtype=torch.bfloat16, device=dev),
                 logits=torch.empty(B, nb, V, dtype=torch.bfloat16, device=dev),
                 tokens=torch.full((B, nb), -1, dtype=i64, device=dev),
                 masked=torch.ones(B, nb, dtype=u8, device=dev),
                 conf=torch.empty(B, nb, dtype=f32, device=dev), am=torch.empty(B, nb, dtype=i64, device=dev),
                 ent=torch.empty(B, nb, dtype=f32, device=dev), mean=torch.empty(B, dtype=f32, device=dev),
                 prev=torch.full((B, nb), -1, dtype=i64, device=dev), stable=torch.zeros(B, dtype=i32, device=dev),
                 frozen=torch.zeros(B, dtype=u8, device=dev), nfz=torch.zeros(1, dtype=i32, device=dev))
        x["vb"] = torch.empty_like(x["kb"])
        x["out"] = torch.empty_like(x["q"])
        x["ws_a"] = torch.empty(max(1, bda.attn_workspace_bytes(B, Hq, Hkv, cap, d, nb, "decode")), dtype=u8,
                                device=dev)
        x["ws_c"] = torch.empty(bda.lib.bda_commit_workspace_bytes(B, nb, V), dtype=u8, device=dev)
        x["ws_s"] = torch.empty(bda.lib.bda_row_stats_workspace_bytes(B, nb, V), dtype=u8, device=dev)
        st[nb] = x
        return x

    def attention(x, nb):
        bda.attn_fwd_varlen(x["q"], kc, vc, kl, "decode", nb, out=x["out"], workspace=x["ws_a"])

    def step(x, nb):
        # the statistics and the commit from one pass over the logits
        bda.kv_append(kc, vc, x["kb"], x["vb"], kl)
        attention(x, nb)
        bda.row_stats_commit(x["logits"], x["tokens"], x["masked"], 0.9, 1, workspace=x["ws_c"],
                             out=(x["conf"], x["am"], x["ent"], x["mean"]))
        bda.adaptive_stop(x["am"], x["prev"], x["stable"], x["frozen"], x["mean"], 1, 0.005, n_frozen=x["nfz"])

    def step_separate(x, nb):
        # the same step with the statistics and the commit as two calls
        bda.kv_append(kc, vc, x["kb"], x["vb"], kl)
        attention(x, nb)
        bda.row_stats(x["logits"], workspace=x["ws_s"], out=(x["conf"], x["am"], x["ent"], x["mean"]))
        bda.adaptive_stop(x["am"], x["prev"], x["stable"], x["frozen"], x["mean"], 1, 0.005, n_frozen=x["nfz"])
        bda.commit(x["logits"], x["tokens"], x["masked"], 0.9, 1, workspace=x["ws_c"])

    def load(x, s_, nb):
        q, kb, vb, lg, _ = synth.multimodal_step(s_, nb, B=B)
        x["q"].copy_(q)
        x["kb"].copy_(kb)
        x["vb"].copy_(vb)
        x["logits"].copy_(lg)

    x = buffers(n)
    load(x, 0, n)
    graphs = {}

    def graph_of(nb, fn):
        key = (nb, fn.__name__)
        if key not in graphs:
            xb = buffers(nb)
            for _ in range(2):
                fn(xb, nb)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn(xb, nb)
            torch.cuda.synchronize()
            graphs[key] = g
        return graphs[key]

    def reset(i):
        x["masked"].fill_(1)

    t_eager, _ = time_launches(lambda i: step(x, n), iters, 5, pre=reset)
    t_eager_sep, _ = time_launches(lambda i: step_separate(x, n), iters, 5, pre=reset)
    g_sep = graph_of(n, step_separate)
    t_graph_sep, _ = time_launches(lambda i: g_sep.replay(), iters, 5, pre=reset)
    g_step = graph_of(n, step)
    t_graph, _ = time_launches(lambda i: g_step.replay(), iters, 5, pre=reset)
    t_graph_host, _ = time_launches(lambda i: g_step.replay(), iters, 5, pre=reset, queue=False)
    g_att = graph_of(n, attention)
    t_att_graph, _ = time_launches(lambda i: g_att.replay(), iters, 5)
    t_att_eager, _ = time_launches(lambda i: attention(x, n), iters, 5)
    L0 = synth.PREFIX + n
    att_bytes = B * Hq * n * d * 2 * 2 + B * Hkv * L0 * d * 2 * 2
    com_bytes = B * n * V * 2
    floor = (att_bytes + com_bytes + B * Hkv * n * d * 2 * 2) / PEAK_HBM_GBS / 1e3   # logits read once

    # the whole canvas: blocks of 28 (a last one of 4) in lockstep over the batch
    kl.fill_(synth.PREFIX)
    steps, pos, committed = 0, 0, 0
    for nb in synth.canvas_blocks():
        xb = buffers(nb)
        xb["masked"].fill_(1)
        xb["tokens"].fill_(-1)
        kl.add_(nb)                                  # the block's rows join the cache
        g = graph_of(nb, step)
        while True:
            load(xb, steps, nb)
            g.replay()
            steps += 1
            left = int(xb["masked"].sum().item())
            if left == 0 or steps >= 400:
                break
        committed += B * nb - left
        pos += nb
    torch.cuda.synchronize()
    return {"B": B, "n": n, "kv_len_first_block": L0, "V": V,
            "us_per_step_eager": round(t_eager * 1e3, 2), "us_per_step_graph": round(t_graph * 1e3, 2),
            "us_per_step_graph_as_issued": round(t_graph_host * 1e3, 2),
            "us_per_step_eager_separate_stats_commit": round(t_eager_sep * 1e3, 2),
            "us_per_step_graph_separate_stats_commit": round(t_graph_sep * 1e3, 2),
            "attention_us_graph": round(t_att_graph * 1e3, 2), "attention_us_eager": round(t_att_eager * 1e3, 2),
            "attention_floor_us": round(att_bytes / PEAK_HBM_GBS / 1e3, 2),
            "step_hbm_floor_us": round(floor, 2),
            "canvas_positions": pos, "canvas_steps": steps, "step_budget": 48, "committed_tokens": committed}


def speculative_step(bda, synth, torch, dev, iters):
    B, Hq, Hkv, d, n, V = 16, 32, 8, 128, 28, synth.VOCAB
    prefix = tuple(8192 - 37 * b for b in range(B))
    cap = 8192 + n + 8 * n
    k0, v0, kl0 = synth.spec_prefix(seed=21, prefix=prefix, cap=cap, n=n, Hkv=Hkv, d=d)
    s = synth.spec_step(0, B=B, n=n, Hq=Hq, Hkv=Hkv, d=d, V=V)
    kc, vc, kl, kl_init = k0.to(dev), v0.to(dev), kl0.to(dev), kl0.to(dev)
    x = {key: s[key].to(dev) for key in ("qd", "kd", "vd", "dlog", "qv", "kv", "vv", "vlog")}
    od, ov = torch.empty_like(x["qd"]), torch.empty_like(x["qd"])
    drafts = torch.empty(B, n, dtype=torch.int64, device=dev)
    am = torch.empty(B, n, dtype=torch.int64, device=dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    u8 = torch.uint8
    ws_d = torch.empty(max(1, bda.attn_workspace_bytes(B, Hq, Hkv, cap, d, n, "decode")), dtype=u8, device=dev)
    ws_v = torch.empty(max(1, bda.attn_workspace_bytes(B, Hq, Hkv, cap, d, n, "causal")), dtype=u8, device=dev)
    n_s = int(bda.lib.bda_row_stats_workspace_bytes(B, n, V))
    ws_s = torch.empty(n_s, dtype=u8, device=dev)
    ws_c = torch.empty(int(bda.lib.bda_verify_workspace_bytes(B, n, V)), dtype=u8, device=dev)

    def step():
        bda.kv_append(kc, vc, x["kd"], x["vd"], kl)
        bda.attn_fwd_varlen(x["qd"], kc, vc, kl, "decode", n, out=od, workspace=ws_d)
        rc = bda.lib.bda_row_stats(bda._ptr(x["dlog"]), bda.BF16, None, None, bda._ptr(drafts), None, None, B, n, V,
                                   bda._ptr(ws_s), n_s, bda._stream(dev))
        if rc:
            raise RuntimeError("bda_row_stats failed")
        bda.kv_append(kc, vc, x["kv"], x["vv"], kl)
        bda.attn_fwd_varlen(x["qv"], kc, vc, kl, "causal", n, out=ov, workspace=ws_v)
        bda.verify_crop(x["vlog"], drafts, kl, cap, argmax_out=am, accept_len=acc, workspace=ws_c)

    def reset(i):
        kl.copy_(kl_init)

    step()
    torch.cuda.synchronize()
    accepted = int(acc.sum().item())
    t_eager, _ = time_launches(lambda i: step(), iters, 5, pre=reset)
    t_eager_host, _ = time_launches(lambda i: step(), iters, 5, pre=reset, queue=False)
    graph = torch.cuda.CUDAGraph()
    reset(0)
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    t_graph, _ = time_launches(lambda i: graph.replay(), iters, 5, pre=reset)
    t_graph_host, _ = time_launches(lambda i: graph.replay(), iters, 5, pre=reset, queue=False)
    keys = sum(prefix) + B * n
    byts = 2 * (keys * Hkv * d * 2 * 2) + 2 * B * n * V * 2 + 4 * B * n * Hq * d * 2
    return {"B": B, "drafts": n, "kv_len": [min(prefix) + n, max(prefix) + n], "V": V,
            "us_per_step_eager": round(t_eager * 1e3, 2), "us_per_step_graph": round(t_graph * 1e3, 2),
            "us_per_step_eager_as_issued": round(t_eager_host * 1e3, 2),
            "us_per_step_graph_as_issued": round(t_graph_host * 1e3, 2),
            "hbm_floor_us": round(byts / PEAK_HBM_GBS / 1e3, 2), "accepted_per_step": accepted,
            "accepted_tokens_per_s_graph": round(accepted / (t_graph * 1e-3), 1)}


if __name__ == "__main__":
    main()
