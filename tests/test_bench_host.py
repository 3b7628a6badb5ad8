"""Host-side checks of bench.py: the CPU baselines carry the fields the
benchmark line reports (kind, cores, sample, a single-thread figure) and time
at least the requested minimum, and a request for more than one GPU is
refused with a message."""
import os
import subprocess
import sys

import numpy as np

import bench
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _check_fields(r, unit):
    assert r["kind"] == "oracle" and r["unit"] == unit
    assert r["value"] > 0 and r["cores"] >= 1 and r["sample"]
    st = r["single_thread"]
    assert st["cores"] == 1 and st["unit"] == unit and st["value"] > 0 and st["sample"]


def test_cpu_baseline_attention_tiny():
    case, _, _ = synth.tiny()
    r = bench.cpu_baseline_attention(case, budget_s=0.01, min_s=0.2)
    _check_fields(r, "TFLOP/s")
    # the tiny case is reached at once (one kv head of one batch is all of it)
    # and repeated until the minimum is timed
    calls = int(r["sample"].split(" call(s)")[0].rsplit(" ", 1)[1])
    assert calls >= 1
    total_s = float(r["sample"].split(" call(s), ")[1].split(" s)")[0])
    assert total_s >= 0.2 - 0.05


def test_cpu_baseline_commit_counts_what_the_oracle_commits():
    _, logits, masked = synth.tiny()
    r = bench.cpu_baseline_commit(logits, masked, 0.85, 1, min_s=0.05)
    _check_fields(r, "committed tokens/s")
    tokens = np.full(tuple(masked.shape), -1, dtype=np.int64)
    _, m, _ = oracle.commit(logits, masked.numpy(), tokens, 0.85, 1)
    committed = int(masked.numpy().sum() - m.sum())
    assert committed >= 1                          # k_min = 1 guarantees one
    assert f"({committed} tokens per call" in r["sample"]


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert p.returncode != 0
    assert "one GPU" in (p.stdout + p.stderr)


def test_single_thread_call_leaves_the_default_thread_count():
    """A call with nthreads=1 sets the count for its own parallel regions
    only: the process-wide OpenMP default that later calls see is unchanged."""
    before = oracle.max_threads()
    case, logits, masked = synth.tiny()
    oracle.commit(logits, masked.numpy(), np.full(tuple(masked.shape), -1, dtype=np.int64), 0.85, 1, nthreads=1)
    oracle.attention("hybrid", case.q, case.k, case.v, case.L, case.block, nthreads=1)
    assert oracle.max_threads() == before


def test_baseline_records_its_thread_count_and_host(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "2")
    nt, host = bench.host_threads()
    assert nt == min(2, host["affinity"]) and host["OMP_NUM_THREADS"] == "2"
    assert host["nproc"] >= host["affinity"] >= 1
    case, _, _ = synth.tiny()
    r = bench.cpu_baseline_attention(case, budget_s=0.01, min_s=0.05)
    assert r["cores"] == nt and r["host"]["affinity"] == host["affinity"]
