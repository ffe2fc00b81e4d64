"""bench.py on the CPU: byte accounting and the one-GPU contract."""
import json
import subprocess
import sys
import os

import pytest

import bench
from synth import recipes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bytes_per_param():
    assert bench.bytes_per_param(recipes.full7p5b()) == (30, 28)
    assert bench.bytes_per_param(recipes.zero1_7p5b()) == (30, 28)
    assert bench.bytes_per_param(recipes.reduce8()) == (50, 30)       # 2*8 + 4 + 4 + 26
    assert bench.bytes_per_param(recipes.tiny()) == (42, 30)
    # 16-bit reduce output: the reduce writes 2 B and the Adam pass reads 2 B
    assert bench.bytes_per_param(recipes.reduce8(), 1, True) == (16 + 2 + 2 + 26, 28)
    assert bench.bytes_per_param(recipes.full7p5b(), 1, True) == (30, 28)
    # micro-steps: first accumulation writes the accumulator, later ones read and write it
    assert bench.bytes_per_param(recipes.reduce8(), 2) == ((16 + 4) + (16 + 8) + 30, 30)
    assert bench.bytes_per_param(recipes.reduce8(), 4) == ((16 + 4) + 2 * (16 + 8) + (16 + 8) + 30, 30)
    # one already-reduced source: the last intake only reads the accumulator and the source,
    # the Adam pass reads both again
    assert bench.bytes_per_param(recipes.full7p5b(), 2) == ((2 + 4) + (2 + 4) + 32, 32)
    assert bench.bytes_per_param(recipes.zero1_7p5b(), 3) == ((2 + 4) + (2 + 8) + (2 + 4) + 32, 32)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "8"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_traffic_summary_is_tied_to_the_kernel_source():
    # a committed summary is only used for the shard size it was taken on
    assert bench.traffic_from_profiles("full7p5b", 0, 1) == (None, None)
    assert bench.traffic_from_profiles("no_such_config", 0, 1) == (None, None)


def test_threaded_oracle_baseline_runs_the_same_step():
    """The threaded oracle baseline performs the same step as the single-threaded one:
    after three steps of a pre-reduced and of an 8-way reduce workload (a ragged last
    piece, no clipping at these sizes) the master, moments and 16-bit slice agree bit
    for bit, and the counters match."""
    import numpy as np
    for w in (recipes.full7p5b(), recipes.reduce8()):
        n = (1 << 18) + 1234
        _, _, a = bench.cpu_baseline(w, n, 3, keep=True)
        _, _, b = bench.cpu_baseline(w, n, 3, threads=4, piece=1 << 16, keep=True)
        for name in ("w", "m", "v"):
            assert (getattr(a, name).view(np.uint32) == getattr(b, name).view(np.uint32)).all(), name
        assert (a.p16 == b.p16).all()
        assert a.counters.t == b.counters.t == 3 and a.counters.p1 == b.counters.p1


def test_host_info_fields():
    h = bench.host_info()
    assert h["nproc"] >= 1 and 1 <= h["usable_cpus"] <= h["nproc"]


def test_committed_traffic_summaries():
    """Where the committed counter summaries of the target workloads match the current
    kernel source, the benchmark reads the Adam and statistics traffic for their shards,
    and both are within 5% of the algorithmic bytes (the bar for redundant traffic)."""
    import pytest
    found = 0
    for cfg, valid in (("full7p5b", 7_500_000_000), ("zero1_7p5b", 117_187_520)):
        adam, stats = bench.traffic_from_profiles(cfg, 0, 28 * valid)
        if adam is None:
            continue
        found += 1
        assert stats is not None, cfg
        assert 1.0 <= adam / (28 * valid) <= 1.05 and 1.0 <= stats / (2 * valid) <= 1.05, cfg
    if not found:
        pytest.skip("the committed summaries were taken on another kernel source")


def test_hbm_side_bytes():
    """Where the gradient slice fits in the 256 MiB Infinity Cache (the ZeRO-1 7.5B/64 shard,
    234 MB), the Adam pass's re-read is not counted as HBM traffic: 28 B/param for the step and
    26 for the Adam pass, against the fabric counts 30 and 28.  Of a larger slice (the GPT-2
    shard's 389 MB) only the 256 MiB tail left in the cache is taken off, nothing beyond 4 GiB
    (the full state) and nothing with tracked segments (the Adam pass then walks forward).  The same holds for the
    last 192 MiB of the local reduce's output.  Micro-steps keep the fabric count."""
    approx = pytest.approx
    assert bench.hbm_side(recipes.zero1_7p5b(), 117_187_520, 1, False, 30, 28)[:2] == (28, 26)
    tail = 256 * 2**20
    assert bench.hbm_side(recipes.full7p5b(), 7_500_000_000, 1, False, 30, 28)[:2] == (30, 28)   # 15 GB: no tail
    assert bench.hbm_side(recipes.gpt2_shard(), 194_409_856, 1, False, 30, 28)[:2] == approx(
        (30 - tail / 194_409_856, 28 - tail / 194_409_856))
    assert bench.hbm_side(recipes.gpt2_shard(), 194_409_856, 1, False, 30, 28, segments=64)[:2] == (30, 28)
    # the local reduce's output: its last 192 MiB are re-read from the cache (all of a smaller output)
    rtail = 192 * 2**20
    assert bench.hbm_side(recipes.reduce8(), 187_500_032, 1, False, 50, 30)[:2] == approx(
        (50 - rtail / 187_500_032, 30 - rtail / 187_500_032))
    assert bench.hbm_side(recipes.reduce8(), 187_500_032, 1, True, 46, 28)[:2] == approx(
        (46 - rtail / 187_500_032, 28 - rtail / 187_500_032))
    assert bench.hbm_side(recipes.reduce8(), 187_500_032, 1, False, 50, 30, segments=8)[:2] == (50, 30)
    assert bench.hbm_side(recipes.tiny(), 262_144, 1, False, 42, 30)[:2] == (38, 26)
    # with micro-steps the accumulator is re-read instead: no adjustment
    assert bench.hbm_side(recipes.zero1_7p5b(), 117_187_520, 2, False, 44, 32)[:2] == (44, 32)


def test_probe_library_checks_its_grid_on_the_host():
    """The bandwidth probes load and refuse shapes they cannot cover before any device work:
    an element count that is not a multiple of 4, a block span that is not a multiple of
    4 x the block size, an unsupported block size or quad count (hipErrorInvalidValue = 1)."""
    import ctypes
    import probes
    L = probes.lib()
    P = ctypes.c_void_p(1 << 20)
    assert L.zprobe_adam_mix(P, 0, P, P, P, P, 6, 2048, 2, 256, 1, 1, None) == 1
    assert L.zprobe_adam_mix(P, 0, P, P, P, P, 4096, 1000, 2, 256, 1, 1, None) == 1
    assert L.zprobe_adam_mix(P, 0, P, P, P, P, 4096, 2048, 3, 256, 1, 1, None) == 1
    assert L.zprobe_copy32(P, P, 4096, 2048, 2, 128, 1, None) == 1
    assert L.zprobe_reduce_mix((ctypes.c_void_p * 3)(P, P, P), 3, P, 4096, 2048, 2, 256, 1, None) == 1
    assert L.zprobe_adam_mix(P, 0, P, P, P, P, 0, 2048, 2, 256, 1, 1, None) == 0      # nothing to do
