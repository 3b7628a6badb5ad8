"""Host-side sanitizer runs (CPU only).

* The oracle (plain C) is built with AddressSanitizer and
  UndefinedBehaviorSanitizer together with tests/host/oracle_driver.c, which
  calls every oracle entry point on small and edge-case inputs; any
  out-of-bounds access, leak or undefined operation fails the run.
* The library's sources are built with the sanitizers on their host code
  only (hipcc -Xarch_host; the gfx950 device code is compiled as usual) and
  linked with tests/host/abi_driver.cpp, which drives every path that runs
  before a launch: argument validation of every entry point, the plans
  behind the workspace-size queries, the tile classifier, the SPRINT keep
  counts; and with tests/host/index_replay.cpp, which replays the attention
  kernels' index arithmetic (attn_index.h) for the benchmark's workloads,
  multi-item and ragged cases and workloads past 2^31 elements, checking
  item coverage, tile bounds, key coverage, every global offset against
  its tensor and the persistent walk's DMA ring protocol (run once more
  without the walk's stand-in loads, where it must fail).  Nothing touches
  a device.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
CSRC = os.path.join(ROOT, "block_masked_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(exe, env):
    p = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    out = p.stdout + p.stderr
    assert p.returncode == 0 and "ok" in p.stdout, out[-4000:]
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall", "-Wextra",
                           os.path.join(HOST, "oracle_driver.c"), os.path.join(ROOT, "oracle", "bda_oracle.c"),
                           "-o", exe, "-lm"])
    _run(exe, SAN_ENV)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_library_host_code_under_asan_ubsan(tmp_path):
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    srcs = [os.path.join(CSRC, f) for f in ("attn.hip", "bwd.hip", "cache.hip", "commit.hip", "sprint.hip",
                                             "api.cpp")] + [os.path.join(HOST, "abi_driver.cpp"),
                                                            os.path.join(HOST, "index_replay.cpp")]
    procs = []
    for s in srcs:
        o = str(tmp_path / (os.path.basename(s) + ".o"))
        objs.append(o)
        procs.append(subprocess.Popen([HIPCC, *flags, "-x", "hip", "-c", s, "-o", o],
                                      stdout=subprocess.DEVNULL, stderr=subprocess.PIPE, text=True))
    for p in procs:
        _, err = p.communicate(timeout=900)
        assert p.returncode == 0, err[-4000:]
    lib_objs, drivers = objs[:-2], objs[-2:]
    for drv in drivers:
        exe = drv[:-2]
        subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                               "-fsanitize=undefined", *lib_objs, drv, "-o", exe])
        # the HIP runtime itself is not instrumented: leak reports would be its own
        _run(exe, dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=0"))
    # the ring replay must catch a walk that stops issuing once its stream is
    # exhausted: the last fast step of a workgroup's last item, when that
    # item has one boundary tile (the causal prefill), would read a tile
    # whose loads may still be in flight
    p = subprocess.run([drivers[1][:-2], "no-stand-in"], capture_output=True, text=True, timeout=600,
                       env=dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=0"))
    assert p.returncode != 0 and "before it landed" in p.stderr, (p.stdout + p.stderr)[-4000:]
