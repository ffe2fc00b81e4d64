"""Benchmark: one data-parallel rank's partitioned optimizer step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic
gradients: [local reduce of N_d rank buffers] + unscale + overflow flag +
sum of squares (one pass), global norm and clip, Adam with bias correction
and decoupled weight decay, and the fused 16-bit write-back.  All inputs are
resident in HBM before the timed region; the timed region is exactly K steps
bracketed by device synchronisation.

Prints one JSON line.  `value` is shard parameters updated per second;
`roofline` reports the dominant kernel (the Adam pass) against the HBM peak;
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "shard params/s per optimizer step and achieved HBM GB/s (% of peak), 1 GPU"
DTYPE_NAME = {1: "fp16", 2: "bf16"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=30,
                   help="untimed steps first; on the full state a process's step time can shift once "
                        "by about 0.5%% within its first ~30 back-to-back steps")
    p.add_argument("--config", default="full7p5b", choices=["tiny", "gpt2", "zero1_7p5b", "reduce8", "full7p5b"])
    p.add_argument("--rank", type=int, default=None, help="data-parallel rank whose shard is stepped")
    p.add_argument("--micro-steps", type=int, default=1,
                   help="gradient-accumulation micro-steps per optimizer step (K - 1 accumulations, then the "
                        "step's own intake)")
    p.add_argument("--dynamic-loss-scale", action="store_true",
                   help="device-resident dynamic loss scale starting at the workload's loss scale (growth 2, "
                        "backoff 0.5, interval 1000, floor 1)")
    p.add_argument("--reduce-output16", action="store_true",
                   help="the local reduce delivers its sum rounded to the 16-bit dtype (the reduce-scatter's "
                        "16-bit result), which the step then takes in")
    p.add_argument("--segments", type=int, default=0,
                   help="track the write-back in this many segments; a second stream waits for each segment and "
                        "copies it out (a stand-in for the segment's all-gather)")
    p.add_argument("--segment-consumer", default="copy", choices=["copy", "wait", "none"],
                   help="with --segments: per segment, wait and copy it out; only wait; or no consumer (the "
                        "tracking cost alone)")
    p.add_argument("--offload", action="store_true",
                   help="ZeRO-Offload: fp32 state in host memory, the step on the host cores, the gradient slice "
                        "copied to the host and the 16-bit slice back to the device (pre-reduced gradients only)")
    p.add_argument("--host-threads", type=int, default=0, help="with --offload: host worker threads (0: all)")
    p.add_argument("--offload-host-stats", action="store_true",
                   help="with --offload: the host computes the flag and sum of squares from the copied gradient "
                        "(default: the device does, and the host update overlaps the copy)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=1 << 26, help="elements of the oracle's timed sample")
    p.add_argument("--cpu-steps", type=int, default=7)
    p.add_argument("--cpu-threads", type=int, default=16,
                   help="threads of the threaded oracle baseline (at most the usable CPUs)")
    p.add_argument("--graph", action="store_true",
                   help="also time the step captured into a HIP graph and replayed (after the timed steps)")
    p.add_argument("--no-cold-cache", action="store_true",
                   help="skip the per-step timing after a cache-evicting read, and after a write "
                        "(after the timed steps)")
    p.add_argument("--no-copy-ceiling", action="store_true",
                   help="skip the device-to-device copy measurement after the timed steps")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run one 1 GiB read + 1 GiB write elementwise kernel first (scales the traffic counters)")
    p.add_argument("--no-probes", action="store_true",
                   help="skip the bandwidth probes (the step's access patterns without its arithmetic) after the "
                        "timed steps")
    p.add_argument("--state-pitch-gib", type=float, default=0.0,
                   help="place the shard's fp32 state arrays this many GiB apart inside one allocation (the gaps "
                        "are allocated too); 0: one allocation per array (default).  An experiment on the DRAM "
                        "address mapping, not the benchmark's layout")
    p.add_argument("--secondary", default="auto",
                   choices=["auto", "none", "tiny", "gpt2", "zero1_7p5b", "reduce8", "full7p5b"],
                   help="a second configuration measured the same way after the first, reported as `secondary` "
                        "(auto: the ZeRO-1 7.5B/64 shard after the full-state one, else none)")
    return p.parse_args()


def kernel_source_sha():
    """Hash of the device code's source (kernels.hip and zs_internal.h) with // comments and
    blank lines removed: counter summaries stay valid across comment-only edits."""
    h = hashlib.sha256()
    for f in ("kernels.hip", "zs_internal.h"):
        with open(os.path.join(ROOT, "zero_partitioned_mixed_reduce_amd", "csrc", f)) as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


class Workload:
    """Device-resident inputs and the library handle for one rank."""

    def __init__(self, w, rank, micro_steps=1, dynamic_loss_scale=False, segments=0, consumer="copy",
                 reduce_out16=False):
        import torch
        import synth
        from zero_partitioned_mixed_reduce_amd.shard import ZeroShard

        self.w, self.rank, self.micro_steps = w, rank, micro_steps
        dt = w.dtype
        psi = w.psi
        starts = [0]
        for n in w.numel:
            starts.append(starts[-1] + n)
        self.starts = starts
        mstream = synth.stream_id(synth.MASTER)

        def filled16(n, first, sigma, stream, zero=False):
            t = torch.empty(n, dtype=torch.int16, device="cuda")
            synth.gpu_normal_16(t, dt, w.seed, stream, first=first, sigma=sigma,
                                zero_seed=w.seed if zero else 0, zero_mod=w.zero_mod if zero else 0)
            return t

        # 16-bit parameters: RNE16 of the master values, full model (the all-gather target)
        if w.param_mode == "flat":
            self.params = filled16(psi, 0, w.master_sigma, mstream)
        else:
            self.params = [filled16(n, starts[k], w.master_sigma, mstream) for k, n in enumerate(w.numel)]
        # gradients
        self.rank_grads, grads_reg = [], None
        gstream = synth.stream_id(synth.GRAD, 0, 0)
        if w.grad_mode == "reduce":
            self.rank_grads = [filled16(psi, 0, w.grad_sigma, synth.stream_id(synth.GRAD, q, 0), zero=True)
                               for q in range(w.nd)]
        elif w.grad_mode == "flat":
            grads_reg = filled16(psi, 0, w.grad_sigma, gstream)
        else:
            grads_reg = [filled16(n, starts[k], w.grad_sigma, gstream) for k, n in enumerate(w.numel)]
        self.grads_reg = grads_reg
        # fp32 master of this shard (logical order) -> library state
        import zero_partitioned_mixed_reduce_amd as zpm
        from zero_partitioned_mixed_reduce_amd import shard as shmod
        info = zpm.zero_shard_plan(shmod.make_desc(w.numel, w.nd, rank, dt, self.params, grads_reg))
        b, valid = info.shard_begin, info.valid_elems
        mi = torch.empty(max(valid, 1), dtype=torch.float32, device="cuda")[:valid]
        if valid:
            synth.gpu_normal_f32(mi, w.seed, mstream, first=b, sigma=w.master_sigma)
        self.shard = ZeroShard(w.numel, w.nd, rank, dt, self.params, grads=grads_reg,
                               master_init=mi if w.master_given else None,
                               with_red=(w.grad_mode == "reduce" or micro_steps > 1))
        del mi
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        self.info = self.shard.info
        if reduce_out16 and w.grad_mode == "reduce":
            self.shard.zero_set_reduce_output(True)
        self.inv = 1.0 / w.loss_scale
        self.intake_inv = self.inv
        if dynamic_loss_scale:
            from zero_partitioned_mixed_reduce_amd import ZERO_DEVICE_LOSS_SCALE
            self.shard.zero_enable_dynamic_loss_scale(w.loss_scale, 2.0, 0.5, 1000, 1.0)
            self.intake_inv = ZERO_DEVICE_LOSS_SCALE
        self.segments = []
        if segments:
            n = self.shard.zero_set_segments(segments)
            self.segments = [self.shard.zero_segment_range(k) for k in range(n)]
            self.consumer = torch.cuda.Stream()
            self.consumer_mode = consumer
            self.gather = torch.empty(max(valid, 1), dtype=torch.int16, device="cuda")
        # the other ranks' sum of squares: the expected value under the synthetic distribution
        sig_u = w.grad_sigma * self.inv * (w.nd ** 0.5 if w.grad_mode == "reduce" else 1.0)
        self.other_sumsq = float(psi - valid) * sig_u * sig_u

    def step(self, ev=None):
        s, w = self.shard, self.w
        if self.segments:
            import torch
            torch.cuda.current_stream().wait_stream(self.consumer)   # the previous step's gathers are done
        for _ in range(self.micro_steps - 1):
            s.zero_accumulate_grads(self.rank_grads)      # the same gradient buffers every micro-step
        if ev:
            ev[0].record()
        s.zero_reduce_grads(self.rank_grads, self.intake_inv)
        if ev:
            ev[1].record()
        s.zero_check_overflow(False)
        s.zero_grad_norm(self.other_sumsq, w.max_norm)
        s.zero_adam_step(w.hp["lr"], w.hp["beta1"], w.hp["beta2"], w.hp["eps"], w.hp["weight_decay"],
                         fuse_cast=True)
        if ev:
            ev[2].record()
        if self.segments and self.consumer_mode != "none":
            self._consume(ev)

    def _consume(self, ev):
        """Per segment: wait for its write-back, then copy its 16-bit slice out (the
        all-gather of that segment would start here)."""
        import torch
        b = self.info.shard_begin
        flat = self.params if not isinstance(self.params, list) else None
        with torch.cuda.stream(self.consumer):
            for k, (lo, ln) in enumerate(self.segments):
                self.shard.zero_wait_segment(k, self.consumer)
                if ev and k == 0:
                    ev[3].record(self.consumer)
                if flat is not None and self.consumer_mode == "copy":
                    self.gather[lo:lo + ln].copy_(flat[b + lo:b + lo + ln])
            if ev:
                ev[4].record(self.consumer)


def bytes_per_param(w, micro_steps=1, reduce_out16=False):
    """Dependency-minimal HBM bytes per shard parameter for the whole step, and for the Adam pass.

    One micro-step reads its sources (2 B per rank buffer, or 2 B of already-reduced
    gradient); the first accumulation writes the fp32 accumulator (4 B), later ones
    read and write it (8 B).  The step's intake on top of an accumulation: from rank
    buffers it reads the accumulator and writes u (8 B) and the Adam pass reads u
    (4 B); from one already-reduced source it only reads the accumulator (4 B) and
    the Adam pass reads the accumulator and the source again (4 + 2 B).  With a 16-bit
    reduce output the reduce writes, and the Adam pass reads, 2 B."""
    src = 2 * w.nd if w.grad_mode == "reduce" else 2
    if micro_steps <= 1:
        if w.grad_mode == "reduce" and reduce_out16:
            return src + 2 + 2 + 26, 2 + 12 + 12 + 2      # write the 16-bit result; Adam reads it
        if w.grad_mode == "reduce":
            return src + 4 + 4 + 26, 4 + 12 + 12 + 2      # write fp32 u; Adam reads u
        return src + 2 + 12 + 12 + 2, 2 + 12 + 12 + 2    # statistics pass, then Adam re-reads the gradient
    if w.grad_mode == "reduce":
        step = (src + 4) + (micro_steps - 2) * (src + 8) + (src + 8) + (4 + 12 + 12 + 2)
        return step, 4 + 12 + 12 + 2
    adam = 4 + src + 12 + 12 + 2
    return (src + 4) + (micro_steps - 2) * (src + 8) + (src + 4) + adam, adam


def cpu_baseline(w, sample, steps, threads=1, piece=1 << 20, keep=False):
    """The oracle on the first `sample` elements of the workload's gradient and state
    (pre-reduced or N_d-way reduce, as configured), `steps` steps of statistics, clip,
    Adam and cast.  Returns (elements per second, seconds[, final state if keep]).

    threads == 1: the oracle's whole-array calls, single-threaded.  threads > 1: the
    oracle's own functions called from that many threads over consecutive pieces of
    `piece` elements (ctypes releases the interpreter lock for the duration of each
    call).  Per step: the statistics of every piece, their sums of squares added in
    piece order, the clip, the step's bias-correction scalars and one advance of the
    counters (an Adam call over no elements), then Adam with those scalars and the
    cast, per piece."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    import synth
    n = sample
    if w.grad_mode == "reduce":
        gs = [synth.normal_16(n, w.dtype, w.seed, synth.stream_id(synth.GRAD, q, 0), 0, w.grad_sigma, w.seed,
                              w.zero_mod) for q in range(w.nd)]
    else:
        gs = [synth.normal_16(n, w.dtype, w.seed, synth.stream_id(synth.GRAD, 0, 0), 0, w.grad_sigma)]
    st = oracle.RankState(w.dtype, synth.normal_16(n, w.dtype, w.seed, synth.stream_id(synth.MASTER), 0,
                                                   w.master_sigma),
                          synth.normal_f32(n, w.seed, synth.stream_id(synth.MASTER), 0, w.master_sigma))
    hp = oracle.HParams(w.hp["lr"], w.hp["beta1"], w.hp["beta2"], w.hp["eps"], w.hp["weight_decay"])
    inv = 1.0 / w.loss_scale
    if threads <= 1:
        t0 = time.perf_counter()
        for _ in range(steps):
            u, flag, ss = oracle.grad_stats(w.dtype, gs, inv)
            clip, _ = oracle.clip_coef(ss, w.max_norm)
            oracle.adam(flag, u, clip, hp, st.counters, st.w, st.m, st.v)
            if not flag:
                oracle.cast(w.dtype, st.w, st.p16)
        dt = time.perf_counter() - t0
    else:
        spans = [(lo, min(lo + piece, n)) for lo in range(0, n, piece)]
        none = np.empty(0, np.float32)
        with ThreadPoolExecutor(threads) as ex:
            t0 = time.perf_counter()
            for _ in range(steps):
                stats = list(ex.map(lambda sp: oracle.grad_stats(w.dtype, [g[sp[0]:sp[1]] for g in gs], inv), spans))
                flag = any(x[1] for x in stats)
                ss = 0.0
                for x in stats:
                    ss = ss + x[2]
                clip, _ = oracle.clip_coef(ss, w.max_norm)
                if flag:
                    continue
                bc1, bc2 = oracle.next_scalars(hp, st.counters)
                oracle.adam(False, none, clip, hp, st.counters, none, none, none)

                def update(k, clip=clip, bc1=bc1, bc2=bc2, stats=stats):
                    lo, hi = spans[k]
                    oracle.adam_elems(stats[k][0], clip, hp, bc1, bc2, st.w[lo:hi], st.m[lo:hi], st.v[lo:hi])
                    oracle.cast(w.dtype, st.w[lo:hi], st.p16[lo:hi])

                list(ex.map(update, range(len(spans))))
            dt = time.perf_counter() - t0
    assert np.isfinite(st.w).all()
    return (n * steps / dt, dt, st) if keep else (n * steps / dt, dt)


def cold_cache_steps(wl, steps, evict="read", flush_bytes=1 << 30):
    """Median duration (ms) of `steps` steps each timed on its own after a 1 GiB pass over
    a scratch buffer that evicts the 256 MB Infinity Cache and the L2s: per step, the
    eviction, then the step between two HIP events on the step's stream, then a wait for
    it.  evict="read": a reduction over the buffer, which leaves the cache holding clean
    lines; evict="write": a fill, which leaves up to 256 MB of dirty lines whose
    write-back then falls inside the timed step."""
    import statistics

    import torch
    scratch = torch.ones(flush_bytes // 4, dtype=torch.float32, device="cuda")
    times = []
    for k in range(steps):
        if evict == "write":
            scratch.fill_(float(k))
        else:
            torch.sum(scratch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        wl.step()
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    torch.cuda.synchronize()
    del scratch
    return statistics.median(times)


def graph_steps(wl, steps):
    """The step captured once into a HIP graph (torch.cuda.CUDAGraph) and replayed
    `steps` times back to back; returns ms per replay.  Each replay is one more step
    (the step counters live on the device)."""
    import torch
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        wl.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del graph
    return ms


def host_info():
    """The host the benchmark ran on: logical CPUs, those this process may use, the CPU
    model and the memory size."""
    model, mem_kib = None, None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal:"):
                    mem_kib = int(line.split()[1])
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0)), "cpu_model": model,
            "mem_gib": None if mem_kib is None else round(mem_kib / 2 ** 20, 1)}


def copy_ceiling(nbytes=4 << 30, reps=5):
    """Measured device-to-device copy rates on this GPU over nbytes: the runtime's
    memcpy (torch copy_) and a plain elementwise kernel (torch.mul by 1), best of
    `reps`, bytes read + written per second."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    best = {"memcpy": 0.0, "elementwise": 0.0}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    for _ in range(reps):
        ev[0].record()
        dst.copy_(src)
        ev[1].record()
        torch.mul(src, 1.0, out=dst)
        ev[2].record()
        ev[2].synchronize()
        best["memcpy"] = max(best["memcpy"], 2 * nbytes / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9)
        best["elementwise"] = max(best["elementwise"], 2 * nbytes / (ev[1].elapsed_time(ev[2]) * 1e-3) / 1e9)
    del src, dst
    torch.cuda.empty_cache()
    return best


def traffic_from_profiles(cfg, rank, adam_launch_bytes):
    """HBM bytes per launch of the Adam kernel and of the statistics kernel from the
    committed rocprofv3 counter summary (profiles/adam_<config>_traffic.txt), when it
    was taken on the current kernel source and the same shard size; else (None, None)."""
    path = os.path.join(ROOT, "profiles", f"adam_{cfg}_traffic.txt")
    if not os.path.exists(path):
        return None, None
    kv = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_sha():
        return None, None
    if int(kv.get("algorithmic_bytes_per_launch", -1)) != adam_launch_bytes:
        return None, None
    stats = kv.get("stats_traffic_bytes_per_launch")
    return int(kv["traffic_bytes_per_launch"]), (int(stats) if stats is not None else None)


def host_probe_gbps(threads, nbytes=1 << 31):
    """Measured host memory bandwidth with `threads` threads over nbytes buffers, best of
    three each: a copy split over the threads (numpy's copy, i.e. the C library's memcpy;
    bytes read + written), torch's read-only sum and torch's write-only fill.  The host has
    no published per-VM figure, so the best of these stands for its peak."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch
    torch.set_num_threads(threads)
    src = np.ones(nbytes // 4, np.float32)
    dst = np.empty_like(src)
    edges = np.linspace(0, src.size, threads + 1).astype(np.int64)
    parts = list(zip(edges[:-1], edges[1:]))
    ts, td = torch.from_numpy(src), torch.from_numpy(dst)

    def cp(b):
        np.copyto(dst[b[0]:b[1]], src[b[0]:b[1]])

    best = {"copy": 0.0, "read": 0.0, "write": 0.0}
    with ThreadPoolExecutor(threads) as ex:
        for _ in range(3):
            t0 = time.perf_counter()
            list(ex.map(cp, parts))
            t1 = time.perf_counter()
            float(ts.sum())
            t2 = time.perf_counter()
            td.fill_(2.0)
            t3 = time.perf_counter()
            best["copy"] = max(best["copy"], 2 * nbytes / (t1 - t0) / 1e9)
            best["read"] = max(best["read"], nbytes / (t2 - t1) / 1e9)
            best["write"] = max(best["write"], nbytes / (t3 - t2) / 1e9)
    del src, dst, ts, td
    return best


def bench_offload(a, w, rank):
    """The offloaded step: fetch (device to host, 2 B/param) -> host statistics ->
    host Adam + 16-bit cast with the host-to-device copy of each finished block
    (2 B/param), then the stream synchronised.  Inputs are resident (16-bit
    parameters and gradients on the device, fp32 state on the host) before timing."""
    import torch
    import synth
    from zero_partitioned_mixed_reduce_amd.offload import ZeroOffload

    if w.grad_mode == "reduce":
        print(json.dumps({"error": "--offload takes an already-reduced gradient (not the N_d-buffer reduce)"}),
              flush=True)
        sys.exit(2)
    torch.cuda.set_device(0)
    dt = w.dtype
    starts = [0]
    for n in w.numel:
        starts.append(starts[-1] + n)
    mstream = synth.stream_id(synth.MASTER)
    gstream = synth.stream_id(synth.GRAD, 0, 0)

    def filled16(n, first, sigma, stream):
        t = torch.empty(n, dtype=torch.int16, device="cuda")
        synth.gpu_normal_16(t, dt, w.seed, stream, first=first, sigma=sigma)
        return t

    t_setup = time.perf_counter()
    if w.param_mode == "flat":
        params = filled16(w.psi, 0, w.master_sigma, mstream)
    else:
        params = [filled16(n, starts[k], w.master_sigma, mstream) for k, n in enumerate(w.numel)]
    if w.grad_mode == "flat":
        grads = filled16(w.psi, 0, w.grad_sigma, gstream)
    else:
        grads = [filled16(n, starts[k], w.grad_sigma, gstream) for k, n in enumerate(w.numel)]
    from zero_partitioned_mixed_reduce_amd import shard as shmod
    import zero_partitioned_mixed_reduce_amd as zpm
    info = zpm.zero_shard_plan(shmod.make_desc(w.numel, w.nd, rank, dt, params, grads))
    b, valid = info.shard_begin, info.valid_elems
    master = synth.normal_f32(valid, w.seed, mstream, b, w.master_sigma) if w.master_given else None
    h = ZeroOffload(w.numel, w.nd, rank, dt, params=params, grads=grads, master_init=master,
                    num_threads=a.host_threads, device_stats=not a.offload_host_stats)
    del master
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    threads = a.host_threads if a.host_threads > 0 else os.cpu_count()
    inv = 1.0 / w.loss_scale
    sig_u = w.grad_sigma * inv
    other = float(w.psi - valid) * sig_u * sig_u
    hp = w.hp

    def step(times=None):
        t0 = time.perf_counter()
        h.zero_offload_fetch_grads(inv)
        h.zero_offload_grad_stats(inv)
        t1 = time.perf_counter()
        h.zero_offload_adam_step(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], False, other,
                                 w.max_norm, push=True)
        t2 = time.perf_counter()
        torch.cuda.current_stream().synchronize()
        t3 = time.perf_counter()
        if times is not None:
            times["stats"] += t1 - t0
            times["adam"] += t2 - t1
            times["drain"] += t3 - t2

    for _ in range(a.warmup):
        step()
    q = h.query()
    assert not q["skipped"] and q["t"] == a.warmup, q
    times = {"stats": 0.0, "adam": 0.0, "drain": 0.0}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step(times)
    wall = time.perf_counter() - t0
    q = h.query()
    assert not q["skipped"] and q["t"] == a.warmup + a.steps, q
    # device-to-host rate on its own: the fetch alone, timed with events on its stream
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    h.zero_offload_fetch_grads(inv)
    ev[1].record()
    ev[1].synchronize()
    d2h_ms = ev[0].elapsed_time(ev[1])
    h.zero_offload_grad_stats(inv)
    h.zero_offload_adam_step(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], False, other,
                             w.max_norm, push=False)
    ev[0].record()
    h.zero_offload_push_params()
    ev[1].record()
    torch.cuda.synchronize()
    h2d_ms = ev[0].elapsed_time(ev[1])
    h.close()
    ms_step = wall * 1e3 / a.steps
    stats_ms, adam_ms, drain_ms = (times[k] * 1e3 / a.steps for k in ("stats", "adam", "drain"))
    probes = host_probe_gbps(threads)
    host_peak = max(probes.values())
    adam_bytes = 28 * valid
    achieved = adam_bytes / (adam_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": valid / (ms_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name + "_offload", "psi": w.psi, "dp_size": w.nd, "dp_rank": rank,
                   "shard_params": valid, "param_grad_dtype": DTYPE_NAME[dt], "grad_source": w.grad_mode,
                   "tensors": len(w.numel), "loss_scale": w.loss_scale, "max_norm": w.max_norm,
                   "offload": "fp32 master/m/v on the host; host step; gradient to host, 16-bit slice to device",
                   "host_threads": threads,
                   "statistics": "host" if a.offload_host_stats else "device, overlapping the copy",
                   "adam": w.hp},
        "breakdown_ms": {"fetch_and_stats": stats_ms, "host_adam_cast_and_push": adam_ms,
                         "push_drain": drain_ms},
        "pcie": {"d2h_gbps": 2 * valid / (d2h_ms * 1e-3) / 1e9, "h2d_gbps": 2 * valid / (h2d_ms * 1e-3) / 1e9,
                 "d2h_ms": d2h_ms, "h2d_ms": h2d_ms, "bytes_each_way": 2 * valid,
                 "peak_gbps": 64.0, "peak_source": "PCIe 5.0 x16, one direction"},
        "roofline": {"kernel": "host Adam + 16-bit cast (AVX-512, all worker threads)", "bound": "host-dram",
                     "achieved": achieved, "peak": host_peak, "unit": "GB/s", "frac": achieved / host_peak,
                     "traffic": None, "algorithmic_bytes_per_launch": adam_bytes, "bytes_per_param": 28,
                     "avg_launch_ms": adam_ms,
                     "peak_source": f"measured on this host with {threads} threads over 2 GiB: the best of a "
                                    "threaded memcpy, a read-only sum and a write-only fill (no published "
                                    "per-VM figure)",
                     "host_probes_gbps": probes},
        "setup_s": setup_s,
    }
    out["host"] = host_info()
    if not a.no_cpu_baseline:
        n = min(a.cpu_sample, valid)
        rate, secs = cpu_baseline(w, n, a.cpu_steps)
        out["cpu_baseline"] = {"value": rate, "unit": "params/s", "cores": 1, "kind": "oracle",
                               "sample": f"first {n} elements of the shard's workload, {a.cpu_steps} steps "
                                         f"(statistics, clip, Adam, cast), {secs:.1f} s single-threaded"}
        threads = max(1, min(out["host"]["usable_cpus"], a.cpu_threads))
        rate, secs = cpu_baseline(w, n, a.cpu_steps, threads)
        out["cpu_baseline_threaded"] = {"value": rate, "unit": "params/s", "cores": threads,
                                        "kind": "oracle, threaded over 1M-element pieces",
                                        "sample": f"the same {n} elements and {a.cpu_steps} steps, {secs:.1f} s"}
    print(json.dumps(out), flush=True)


INFINITY_CACHE_BYTES = 256 << 20


STATS_TAIL_BYTES = 256 << 20   # a larger slice's tail that the statistics pass leaves in the cache
REDUCE_TAIL_BYTES = 192 << 20  # the part of the local reduce's output stored to stay in the cache


def hbm_side(w, valid, micro_steps, reduce_out16, step_b, adam_b, segments=0):
    """HBM-side bytes per parameter where they differ from the fabric-side (L2-requested)
    count.  A 16-bit gradient slice that fits in the 256 MiB Infinity Cache is read by the
    statistics pass with plain loads and re-read by the Adam pass from the cache, so the
    second read does not reach HBM.  Of a larger slice the statistics pass reads the last
    256 MiB with plain loads and the Adam pass (walking from the end, unless the write-back
    tracks segments) re-reads those from the cache, up to slices of 4 GiB.  Likewise the local reduce stores the
    last 192 MiB of its output (all of it if smaller) with plain stores, and the Adam pass
    reads them from the cache.  Returns (step, adam, note)."""
    slice_bytes = 2 * valid
    fabric = "HBM-side bytes equal the fabric count"
    unseen = "(no hardware counter separates the two on gfx950)"
    if micro_steps > 1 or valid == 0:
        return step_b, adam_b, "the step's re-reads are not counted apart with micro-steps: " + fabric
    if w.grad_mode == "reduce":
        out_bytes = (2 if reduce_out16 else 4) * valid
        if out_bytes > REDUCE_TAIL_BYTES and segments:
            return step_b, adam_b, ("with tracked segments the Adam pass walks forward and re-reads no cached part of "
                                    "the reduce output: " + fabric)
        d = min(out_bytes, REDUCE_TAIL_BYTES) / valid
        return step_b - d, adam_b - d, (f"{min(out_bytes, REDUCE_TAIL_BYTES) / 2**20:.0f} MiB of the local reduce's "
                                        f"{out_bytes / 1e6:.0f} MB output stay in the Infinity Cache for the Adam pass: "
                                        f"HBM moves {d:.4f} B/param less than the fabric count " + unseen)
    if slice_bytes <= INFINITY_CACHE_BYTES:
        return step_b - 2, adam_b - 2, (f"the {slice_bytes / 1e6:.0f} MB gradient slice fits in the 256 MiB Infinity "
                                        "Cache: the Adam pass re-reads it from there, so HBM moves 2 B/param less "
                                        "than the fabric count " + unseen)
    if segments:
        return step_b, adam_b, "with tracked segments the Adam pass walks forward and re-reads no cached tail: " + fabric
    if slice_bytes > 16 * STATS_TAIL_BYTES:
        return step_b, adam_b, "a slice beyond 16 x 256 MiB leaves no tail in the cache: " + fabric
    d = STATS_TAIL_BYTES / valid
    return step_b - d, adam_b - d, (f"the last 256 MiB of the {slice_bytes / 1e6:.0f} MB gradient slice stay in the "
                                    "Infinity Cache for the Adam pass, which starts there: HBM moves "
                                    f"{d:.4f} B/param less than the fabric count " + unseen)


def probe_ceiling(wl, adam_gbps, stats_gbps):
    """The step's access patterns without its arithmetic, on the workload's own buffers
    (probes/): the Adam pass's stream mix in the kernel's own grid, block and
    non-temporal policy, and two nearby shapes; the statistics pass's (or the local
    reduce's) read pattern; pure fp32 read, write and copy streams over the state arrays.
    Runs after every step measurement (it overwrites the state).  GB/s, medians of 3."""
    import torch
    import probes
    st = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    w, sh = wl.w, wl.shard
    valid, b = wl.info.valid_elems, wl.info.shard_begin
    n = valid // 4 * 4
    if n < 4096:
        return None
    scratch = []

    def flat16(t):
        if t is not None and not isinstance(t, list):
            return t.data_ptr() + 2 * b                 # this rank's slice of a flat buffer
        x = torch.empty(n, dtype=torch.int16, device="cuda")  # ragged tensors: one flat stand-in of the slice's size
        x.fill_(0x3C00)
        scratch.append(x)
        return x.data_ptr()

    def timed(fn, reps=3):
        fn()
        ts = []
        for _ in range(reps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record()
            fn()
            e[1].record()
            e[1].synchronize()
            ts.append(e[0].elapsed_time(e[1]))
        return sorted(ts)[len(ts) // 2]

    gbps = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9
    wp, mp, vp = sh.master.data_ptr(), sh.m.data_ptr(), sh.v.data_ptr()
    p16 = flat16(wl.params)
    out = {"unit": "GB/s", "elements": n,
           "buffers": "the benchmark's own fp32 state arrays and the shard's 16-bit slices (ragged tensor lists: a "
                      "flat 16-bit stand-in of the slice's size), after the timed steps",
           "note": "each probe streams all its bytes through memory: an Adam pass that starts on the part of its "
                   "gradient input the intake left in the Infinity Cache (a slice between 256 MiB and 4 GiB, or "
                   "a local reduce's output) can run above its probe"}
    reduce_mode = w.grad_mode == "reduce"
    if reduce_mode:
        g, g32, mix_b = sh.red.data_ptr(), True, 30             # the Adam pass reads fp32 u after a local reduce
    else:
        g, g32, mix_b = flat16(wl.grads_reg), False, 28
    shapes = {"kernel_shape": (2048, 2, 256), "u4_bs512": (2048, 4, 512), "epb1024_u4": (1024, 4, 256)}
    mix = {}
    for name, (epb, u, bs) in shapes.items():
        mix[name] = gbps(mix_b * n, timed(lambda: probes.adam_mix(g, wp, mp, vp, p16, n, st(), epb, u, bs, 1, 1,
                                                                   g32)))
    out["adam_mix_bytes_per_param"] = mix_b
    out["adam_mix"] = mix
    best = max(mix.values())
    out["adam_mix_best"] = best
    out["adam_frac_of_ceiling"] = adam_gbps / best
    out["adam_frac_of_same_pattern_probe"] = adam_gbps / mix["kernel_shape"]
    sink = torch.empty(n // 1024 + 1, device="cuda")
    if reduce_mode:
        srcs = [x.data_ptr() + 2 * b for x in wl.rank_grads]
        out["reduce_mix"] = {f: gbps((2 * len(srcs) + 4) * n, timed(lambda: probes.reduce_mix(
            srcs, sh.red.data_ptr(), n, st(), epb, u, bs, 1))) for f, (epb, u, bs) in
            {"kernel_shape": (8192, 2, 256), "epb4096_bs512": (4096, 2, 512), "epb1024": (1024, 2, 256)}.items()}
        out["reduce_frac_of_ceiling"] = stats_gbps / max(out["reduce_mix"].values())
    else:
        nt = int(2 * valid > INFINITY_CACHE_BYTES)               # the statistics pass's load policy
        out["read16_grad"] = {f: gbps(2 * n, timed(lambda: probes.read16(g, n, sink.data_ptr(), st(), epb, u, bs, nt)))
                              for f, (epb, u, bs) in {"kernel_shape": (8192, 4, 256),
                                                      "epb32768_bs512": (32768, 2, 512)}.items()}
        out["stats_frac_of_ceiling"] = stats_gbps / max(out["read16_grad"].values())
    out["read32"] = gbps(4 * n, timed(lambda: probes.read32(wp, n, sink.data_ptr(), st(), 2048, 1, 256, 1)))
    out["write32"] = gbps(4 * n, timed(lambda: probes.write32(mp, n, st(), 2048, 2, 512, 1)))
    out["copy32"] = gbps(8 * n, timed(lambda: probes.copy32(wp, mp, n, st(), 2048, 2, 512, 1)))
    del scratch, sink
    return out


def measure(a, config, rank, primary=True):
    """Builds the workload, runs the warm-up and the timed steps, and returns the bench
    fields for one configuration (the workload is freed before returning)."""
    import torch
    from synth import recipes

    w = recipes.ALL[config]()
    rank = rank if rank is not None else w.ranks[0]
    from zero_partitioned_mixed_reduce_amd.shard import ZeroShard
    pitch = int(getattr(a, "state_pitch_gib", 0.0) * (1 << 30)) // 256 * 256
    ZeroShard.state_pitch = pitch if pitch > 0 else None
    t_setup = time.perf_counter()
    wl = Workload(w, rank, a.micro_steps, a.dynamic_loss_scale, a.segments, a.segment_consumer, a.reduce_output16)
    setup_s = time.perf_counter() - t_setup
    valid = wl.info.valid_elems
    step_b, adam_b = bytes_per_param(w, a.micro_steps, a.reduce_output16)

    if a.copy_calibration and primary:
        # a plain elementwise kernel of known traffic (reads 1 GiB, writes 1 GiB), used to scale
        # the FETCH_SIZE / WRITE_SIZE counters of the same run
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(a.warmup):
        wl.step()
    torch.cuda.synchronize()
    q = wl.shard.query()
    assert not q["skipped"] and q["t"] == a.warmup, q

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(a.steps):
        wl.step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    q = wl.shard.query()
    assert not q["skipped"] and q["t"] == a.warmup + a.steps, q

    ms_step = wall * 1e3 / a.steps
    stats_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / a.steps
    adam_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / a.steps
    adam_bytes = adam_b * valid
    achieved = adam_bytes / (adam_ms * 1e-3) / 1e9
    traffic, stats_traffic = traffic_from_profiles(config, rank, adam_bytes)
    out = {
        "metric": METRIC,
        "value": valid / (ms_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "psi": w.psi, "dp_size": w.nd, "dp_rank": rank, "shard_params": valid,
                   "param_grad_dtype": DTYPE_NAME[w.dtype], "grad_source": w.grad_mode,
                   "tensors": len(w.numel), "loss_scale": w.loss_scale, "max_norm": w.max_norm,
                   "loss_scale_mode": "dynamic, device-resident" if a.dynamic_loss_scale else "static",
                   "micro_steps": a.micro_steps,
                   "reduce_output": "16-bit" if a.reduce_output16 and w.grad_mode == "reduce" else "fp32",
                   "state_placement": (f"one allocation, arrays {pitch / (1 << 30):g} GiB apart" if pitch > 0
                                       else "one allocation per array"),
                   "adam": w.hp},
        "hbm_gbps_step": step_b * valid / (ms_step * 1e-3) / 1e9,
        "hbm_frac_step": step_b * valid / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "bytes_per_param_step": step_b,
        "bytes_counted": "fabric side: the dependency-minimal bytes the L2s request (the gradient read twice)",
        "breakdown_ms": {"accumulate": ms_step - stats_ms - adam_ms if a.micro_steps > 1 else 0.0,
                         "intake_stats": stats_ms, "norm_adam_cast": adam_ms},
        "roofline": {"kernel": "adam_kernel (Adam + fused 16-bit write-back)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "traffic_counts": "FETCH_SIZE + WRITE_SIZE per launch (scaled by a known copy): requests "
                                       "below the L2s, Infinity Cache hits included",
                     "algorithmic_bytes_per_launch": adam_bytes, "bytes_per_param": adam_b,
                     "avg_launch_ms": adam_ms},
        "setup_s": setup_s,
    }
    # the same step rate at 28 B/param (the read of g, w, m, v and the writes of w, m, v, p16, plus
    # 2 B per rank buffer when reducing): the second read of the gradient is not counted
    ns_b = 28 + (2 * w.nd if w.grad_mode == "reduce" else 0)
    out["hbm_gbps_step_28b"] = ns_b * valid / (ms_step * 1e-3) / 1e9
    out["bytes_per_param_28b"] = ns_b
    hs_step, hs_adam, hs_note = hbm_side(w, valid, a.micro_steps, a.reduce_output16, step_b, adam_b, a.segments)
    if traffic is not None and stats_traffic is not None and a.micro_steps == 1 and w.grad_mode != "reduce":
        # counter-measured bytes of the step's two kernels (profiles/), over the measured step time
        step_traffic = traffic + stats_traffic
        out["counter_traffic_step"] = {"bytes": step_traffic, "ratio_to_algorithmic": step_traffic / (step_b * valid),
                                       "gbps": step_traffic / (ms_step * 1e-3) / 1e9,
                                       "frac": step_traffic / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    if wl.segments:
        out["config"]["segments"] = len(wl.segments)
        copies = a.segment_consumer == "copy" and not isinstance(wl.params, list)
        out["pipeline"] = {
            "segments": len(wl.segments),
            "consumer": {"copy": "wait per segment, then copy its 16-bit slice" if copies else "wait per segment",
                         "wait": "wait per segment", "none": "none"}[a.segment_consumer],
            "adam_ms": adam_ms,
            "timeouts": wl.shard.zero_segment_timeouts(),
        }
        if a.segment_consumer != "none":
            out["pipeline"]["first_segment_ready_ms"] = sum(e[1].elapsed_time(e[3]) for e in evs) / a.steps
            out["pipeline"]["last_segment_done_ms"] = sum(e[1].elapsed_time(e[4]) for e in evs) / a.steps
    if a.graph and not wl.segments:
        t_before = wl.shard.query()["t"]
        g_ms = graph_steps(wl, a.steps)
        q = wl.shard.query()
        assert not q["skipped"] and q["t"] == t_before + a.steps, q
        out["graph_replay"] = {"ms_per_step": g_ms, "value": valid / (g_ms * 1e-3),
                               "hbm_frac_step": step_b * valid / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                               "steps": a.steps,
                               "protocol": "after the timed steps: the step captured once into a HIP graph, "
                                           "then replayed back to back, bracketed by synchronisation"}
    cold_ms = None
    if not a.no_cold_cache:
        cold_ms = cold_cache_steps(wl, a.steps, "read")
        cold_w_ms = cold_cache_steps(wl, a.steps, "write")
        out["cold_cache"] = {"ms_per_step_median": cold_ms, "value": valid / (cold_ms * 1e-3),
                             "hbm_frac_step": step_b * valid / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                             "ms_per_step_median_after_write": cold_w_ms,
                             "steps": a.steps,
                             "protocol": "after the timed steps: per step a 1 GiB read of a scratch buffer "
                                         "(evicts the Infinity Cache and L2s, leaving clean lines), then the "
                                         "step alone between two events; median.  After a 1 GiB write "
                                         "instead, the write-back of the dirty lines it leaves falls inside "
                                         "the step"}
    hs = {"bytes_per_param_step": hs_step, "bytes_per_param_adam": hs_adam, "note": hs_note,
          "gbps_step": hs_step * valid / (ms_step * 1e-3) / 1e9,
          "frac_step": hs_step * valid / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
          "gbps_adam": hs_adam * valid / (adam_ms * 1e-3) / 1e9,
          "frac_adam": hs_adam * valid / (adam_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    if cold_ms is not None:
        hs["frac_step_cold_cache"] = hs_step * valid / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS
    out["hbm_side"] = hs
    if not a.no_probes:
        stats_gbps = ((2 * w.nd + 4) if w.grad_mode == "reduce" else 2) * valid / (stats_ms * 1e-3) / 1e9
        ceil = probe_ceiling(wl, achieved, stats_gbps)
        if ceil is not None:
            out["roofline"]["ceiling"] = ceil
    del wl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out, w, rank, achieved


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": f"this benchmark runs one data-parallel rank on one GPU; --gpus {a.gpus} "
                                   "is not supported (the path has no collectives: each rank would run this "
                                   "step on its own shard, with the reduce-scatter before it, a two-scalar "
                                   "all-reduce between its passes and the all-gather after it)"}), flush=True)
        sys.exit(2)
    import torch
    from synth import recipes

    if a.offload:
        w = recipes.ALL[a.config]()
        bench_offload(a, w, a.rank if a.rank is not None else w.ranks[0])
        return
    torch.cuda.set_device(0)
    out, w, rank, achieved = measure(a, a.config, a.rank)
    secondary = a.secondary if a.secondary != "auto" else ("zero1_7p5b" if a.config == "full7p5b" else "none")
    if secondary != "none" and secondary != a.config:
        sec, _, _, _ = measure(a, secondary, None, primary=False)
        keep = ("value", "unit", "ms_per_step", "steps", "warmup", "config", "hbm_gbps_step", "hbm_frac_step",
                "bytes_per_param_step", "bytes_counted", "hbm_gbps_step_28b", "bytes_per_param_28b",
                "breakdown_ms", "roofline", "counter_traffic_step", "cold_cache", "hbm_side")
        out["secondary"] = {k: sec[k] for k in keep if k in sec}
    if not a.no_copy_ceiling:
        cc = copy_ceiling()
        top = max(cc.values())
        out["copy_ceiling"] = {"unit": "GB/s", "bytes": 4 << 30, "memcpy_d2d": cc["memcpy"],
                               "elementwise_copy": cc["elementwise"],
                               "adam_frac_of_copy": achieved / top, "step_frac_of_copy": out["hbm_gbps_step"] / top}
    out["host"] = host_info()
    if not a.no_cpu_baseline:
        valid = out["config"]["shard_params"]
        n = min(a.cpu_sample, valid)
        rate, secs = cpu_baseline(w, n, a.cpu_steps)
        out["cpu_baseline"] = {"value": rate, "unit": "params/s", "cores": 1, "kind": "oracle",
                               "sample": f"first {n} elements of the shard's workload, {a.cpu_steps} steps "
                                         f"(statistics, clip, Adam, cast), {secs:.1f} s single-threaded"}
        threads = max(1, min(out["host"]["usable_cpus"], a.cpu_threads))
        rate, secs = cpu_baseline(w, n, a.cpu_steps, threads)
        out["cpu_baseline_threaded"] = {"value": rate, "unit": "params/s", "cores": threads,
                                        "kind": "oracle, threaded over 1M-element pieces",
                                        "sample": f"the same {n} elements and {a.cpu_steps} steps, {secs:.1f} s"}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
