"""Full-size parity: the large workloads in the benchmark's own launch
configuration, checked against the oracle on sampled elements.

The oracle computes this rank's sum of squares over the whole shard (host
threads over fixed chunks, partials added in chunk order), the clip
coefficient and bias corrections, then every sampled element one by one:
shard ends, both sides of every tensor-piece and chunk boundary, and random
positions.  Two applied steps with the benchmark's gradient.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import recipes
from tests.gpu_harness import assert_16_close, assert_f32_close

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu(need_gpu):
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def host_grad(w, q, idx_or_range):
    """16-bit gradient of rank buffer q (or the reduced buffer) at flat indices."""
    stream = synth.stream_id(synth.GRAD, q, 0)
    zs, zm = (w.seed, w.zero_mod) if w.grad_mode == "reduce" else (0, 0)
    if isinstance(idx_or_range, tuple):
        lo, n = idx_or_range
        return synth.normal_16(n, w.dtype, w.seed, stream, lo, w.grad_sigma, zs, zm)
    return synth.gather_16(idx_or_range, w.dtype, w.seed, stream, w.grad_sigma, zs, zm)


def oracle_u(w, srcs, inv, micro_steps, r16=False):
    """The oracle's unscaled gradient for one run of elements: the benchmark feeds the
    same sources to every micro-step.  r16: the reduce delivers its sum in 16 bits."""
    if r16 and len(srcs) >= 2:
        srcs = [oracle.reduce_to16(w.dtype, srcs)]
    if micro_steps <= 1:
        return oracle.grad_stats(w.dtype, srcs, inv)
    acc = np.zeros(srcs[0].size, np.float32)
    for k in range(micro_steps):
        oracle.accumulate(w.dtype, srcs, acc, first=(k == 0))
    return oracle.stats_f32(acc, inv)


def oracle_local_sumsq(w, b, valid, inv, micro_steps=1, r16=False):
    nsrc = w.nd if w.grad_mode == "reduce" else 1
    step = 1 << 24
    blocks = [(lo, min(step, valid - lo)) for lo in range(0, valid, step)]

    def part(blk):
        lo, n = blk
        srcs = [host_grad(w, q, (b + lo, n)) for q in range(nsrc)]
        _, flag, ss = oracle_u(w, srcs, inv, micro_steps, r16)
        return flag, ss

    synth.set_host_threads(1)          # the pool below already uses every core
    try:
        with ThreadPoolExecutor(16) as ex:
            parts = list(ex.map(part, blocks))
    finally:
        synth.set_host_threads(0)
    total = 0.0
    for _, ss in parts:
        total = total + ss
    return any(f for f, _ in parts), total


def sample_positions(info, pieces, rng):
    valid = info.valid_elems
    S = []
    S.append(np.arange(min(4096, valid)))
    S.append(np.arange(max(0, valid - 4096), valid))
    for (_, _, soff, _, ln) in pieces:
        for edge in (soff, soff + ln):
            S.append(np.arange(max(0, edge - 64), min(valid, edge + 64)))
    # inside a tensor piece, around element offsets 2^31 and 2^32 from its start
    for (_, _, soff, _, ln) in pieces:
        for big in (1 << 31, 1 << 32):
            if ln > big:
                S.append(np.arange(soff + big - 64, soff + big + 64))
    # chunk boundaries (multiples of 4096 from a piece start, shifted by < 8 for alignment): 4000 of them
    starts = np.array([p[2] for p in pieces], np.int64)
    lens = np.array([p[4] for p in pieces], np.int64)
    k = rng.integers(0, len(pieces), size=4000)
    e = starts[k] + (rng.integers(0, 1 << 40, size=4000) % np.maximum(lens[k] // 4096, 1)) * 4096
    S.append((e[:, None] + np.arange(-8, 8)[None, :]).ravel().clip(0, valid - 1))
    S.append(rng.integers(0, valid, size=200_000))
    return np.unique(np.concatenate(S).astype(np.int64))


def state_index(pieces, pos):
    soffs = np.array([p[2] for p in pieces], np.int64)
    stoffs = np.array([p[3] for p in pieces], np.int64)
    k = np.searchsorted(soffs, pos, side="right") - 1
    return stoffs[k] + (pos - soffs[k])


def gpu_params_at(wl, flat_idx):
    if not isinstance(wl.params, list):
        t = torch.from_numpy(flat_idx).cuda()
        return wl.params[t].cpu().numpy().view(np.uint16)
    starts = np.array(wl.starts[:-1], np.int64)
    k = np.searchsorted(starts, flat_idx, side="right") - 1
    out = np.empty(flat_idx.size, np.uint16)
    for kk in np.unique(k):
        sel = np.flatnonzero(k == kk)
        off = torch.from_numpy(flat_idx[sel] - starts[kk]).cuda()
        out[sel] = wl.params[kk][off].cpu().numpy().view(np.uint16)
    return out


@pytest.mark.parametrize("cfg,rank,micro,r16,seg", [
    ("zero1_7p5b", 0, 1, False, 0), ("zero1_7p5b", 63, 1, False, 0), ("gpt2", 7, 1, False, 0),
    ("gpt2", 3, 1, False, 0), ("reduce8", 7, 1, False, 0), ("reduce8", 0, 1, False, 0), ("full7p5b", 0, 1, False, 0),
    ("reduce8", 7, 3, False, 0), ("zero1_7p5b", 0, 2, False, 0), ("reduce8", 7, 1, True, 0), ("reduce8", 0, 2, True, 0),
    ("big_tensor", 0, 1, False, 0),
    # tracked segments: the Adam pass walks forward past the intake's cached tail
    ("gpt2", 7, 1, False, 16), ("reduce8", 7, 1, True, 16)])
def test_full_size_sampled(cfg, rank, micro, r16, seg):
    """The shard's slices beyond the 256 MiB Infinity Cache (GPT-2, the local reduce's output)
    take the paths where the intake leaves a tail in the cache and the Adam pass starts at the
    end (or, with tracked segments, walks forward)."""
    import bench
    w = recipes.ALL[cfg]() if cfg in recipes.ALL else getattr(recipes, cfg)()
    print(f"\n[fullsize] {cfg} rank {rank} micro-steps {micro} 16-bit reduce output {r16} segments {seg}: setting up",
          flush=True)
    wl = bench.Workload(w, rank, micro, reduce_out16=r16, segments=seg)
    info = wl.info
    b, valid = info.shard_begin, info.valid_elems
    pieces = wl.shard.pieces()
    for _ in range(2):
        wl.step()
    torch.cuda.synchronize()
    q = wl.shard.query()
    assert q["t"] == 2 and not q["skipped"]
    if seg:
        assert wl.shard.zero_segment_timeouts() == 0

    print(f"[fullsize] {cfg}: oracle sum of squares over {valid} elements", flush=True)
    flag, local = oracle_local_sumsq(w, b, valid, wl.inv, micro, r16)
    assert not flag
    clip, norm = oracle.clip_coef(local + wl.other_sumsq, w.max_norm)
    assert q["clip"] == clip, (q, clip)
    assert abs(q["norm"] - norm) <= 1e-9 * norm       # the device's fp64 sum agrees to ~1e-12

    rng = np.random.default_rng(2024)
    pos = sample_positions(info, pieces, rng)
    flat = b + pos
    nsrc = w.nd if w.grad_mode == "reduce" else 1
    u, _, _ = oracle_u(w, [host_grad(w, qq, flat) for qq in range(nsrc)], wl.inv, micro, r16)
    mstream = synth.stream_id(synth.MASTER)
    if w.master_given:
        wv = synth.gather_f32(flat, w.seed, mstream, w.master_sigma)
    else:
        wv = oracle.decode16(w.dtype, synth.gather_16(flat, w.dtype, w.seed, mstream, w.master_sigma))
    mv = np.zeros_like(wv)
    vv = np.zeros_like(wv)
    hp = oracle.HParams(w.hp["lr"], w.hp["beta1"], w.hp["beta2"], w.hp["eps"], w.hp["weight_decay"])
    ctr = oracle.Counters.fresh()
    none = np.empty(0, np.float32)
    for _ in range(2):
        bc1, bc2 = oracle.next_scalars(hp, ctr)
        oracle.adam_elems(u, clip, hp, bc1, bc2, wv, mv, vv)
        oracle.adam(False, none, clip, hp, ctr, none, none, none)     # advances the counters
    p16 = oracle.encode16(w.dtype, wv)

    sidx = torch.from_numpy(state_index(pieces, pos)).cuda()
    s = wl.shard
    nonexact = assert_f32_close(s.master[sidx].cpu().numpy(), wv, f"{cfg} master")
    nonexact += assert_f32_close(s.m[sidx].cpu().numpy(), mv, f"{cfg} m")
    nonexact += assert_f32_close(s.v[sidx].cpu().numpy(), vv, f"{cfg} v")
    nonexact += assert_16_close(gpu_params_at(wl, flat), p16, f"{cfg} p16")
    assert nonexact == 0, f"{nonexact} sampled values within tolerance but not bit-exact"
    # parameters outside this rank's shard are untouched: check around both shard edges
    outside = np.concatenate([np.arange(max(0, b - 2048), b), np.arange(b + valid, min(w.psi, b + valid + 2048))])
    if outside.size:
        exp = synth.gather_16(outside, w.dtype, w.seed, mstream, w.master_sigma)
        assert (gpu_params_at(wl, outside) == exp).all()
    print(f"[fullsize] {cfg}: {pos.size} sampled elements match", flush=True)
    wl.shard.close()
    del wl


@pytest.mark.parametrize("cfg,rank", [("zero1_7p5b", 63), ("gpt2", 3), ("reduce8", 7)])
def test_full_shard_every_element(cfg, rank):
    """Every element of a full-size shard after two steps, in the benchmark's launch
    configuration: the ZeRO-1 7.5B shard of the last rank (fp16, loss scale 2^16, a
    padded tail), a middle GPT-2 shard (bf16, 386 tensor pieces) and the last rank of
    the 8-way local reduce (fp16, exact zeros shared by all buffers).  The oracle runs
    the whole shard (its own reduce, statistics, clip and Adam) and the master, m, v
    and 16-bit slice are compared bit for bit."""
    import bench
    w = recipes.ALL[cfg]()
    print(f"\n[fullshard] {cfg} rank {rank}: setting up", flush=True)
    wl = bench.Workload(w, rank)
    b, valid = wl.info.shard_begin, wl.info.valid_elems
    for _ in range(2):
        wl.step()
    torch.cuda.synchronize()
    q = wl.shard.query()
    assert q["t"] == 2 and not q["skipped"]

    print(f"[fullshard] {cfg}: oracle over {valid} elements", flush=True)
    mstream = synth.stream_id(synth.MASTER)
    nsrc = w.nd if w.grad_mode == "reduce" else 1
    g = [host_grad(w, qq, (b, valid)) for qq in range(nsrc)]
    u, flag, local = oracle.grad_stats(w.dtype, g, wl.inv)
    assert not flag
    clip, _ = oracle.clip_coef(local + wl.other_sumsq, w.max_norm)
    assert q["clip"] == clip, (q, clip)
    p16 = synth.normal_16(valid, w.dtype, w.seed, mstream, b, w.master_sigma)
    mst = synth.normal_f32(valid, w.seed, mstream, b, w.master_sigma) if w.master_given else None
    st = oracle.RankState(w.dtype, p16, mst)
    hp = oracle.HParams(w.hp["lr"], w.hp["beta1"], w.hp["beta2"], w.hp["eps"], w.hp["weight_decay"])
    for _ in range(2):
        oracle.adam(False, u, clip, hp, st.counters, st.w, st.m, st.v)
        oracle.cast(w.dtype, st.w, st.p16)
    del u, g

    s = wl.shard
    for name, exp in (("master", st.w), ("m", st.m), ("v", st.v)):
        got = s.export(name).cpu().numpy()
        bad = np.flatnonzero(got.view(np.uint32) != exp.view(np.uint32))
        assert bad.size == 0, f"{cfg} {name}: {bad.size} elements differ, first at {bad[:5]}"
        del got
    if isinstance(wl.params, list):
        dev = np.concatenate([t.cpu().numpy().view(np.uint16) for t in wl.params])[b:b + valid]
    else:
        dev = wl.params[b:b + valid].cpu().numpy().view(np.uint16)
    bad = np.flatnonzero(dev != st.p16)
    assert bad.size == 0, f"{cfg} p16: {bad.size} elements differ, first at {bad[:5]}"
    print(f"[fullshard] {cfg}: all {valid} elements match", flush=True)
    wl.shard.close()
    del wl


def test_full_state_every_element():
    """Every element of the full-state 7.5B shard (N_d = 1, 292 bf16 tensors, 7.5e9
    elements) after two steps in the benchmark's launch configuration, streamed in
    2^25-element pieces: the oracle's statistics over the whole shard give the clip,
    then each piece's master, m, v and 16-bit values from the oracle (two Adam steps
    and the cast, host threads over pieces) are compared bit for bit with the device."""
    from concurrent.futures import ThreadPoolExecutor

    import bench
    w = recipes.full7p5b()
    print("\n[fullstate] setting up", flush=True)
    wl = bench.Workload(w, 0)
    b, valid = wl.info.shard_begin, wl.info.valid_elems
    for _ in range(2):
        wl.step()
    torch.cuda.synchronize()
    q = wl.shard.query()
    assert q["t"] == 2 and not q["skipped"]
    print(f"[fullstate] oracle sum of squares over {valid} elements", flush=True)
    flag, local = oracle_local_sumsq(w, b, valid, wl.inv)
    assert not flag
    clip, _ = oracle.clip_coef(local + wl.other_sumsq, w.max_norm)
    assert q["clip"] == clip, (q, clip)
    hp = oracle.HParams(w.hp["lr"], w.hp["beta1"], w.hp["beta2"], w.hp["eps"], w.hp["weight_decay"])
    mstream = synth.stream_id(synth.MASTER)
    exports = {name: wl.shard.export(name) for name in ("master", "m", "v")}
    starts = np.array(wl.starts, np.int64)

    def device16(lo, n):
        """The device's 16-bit parameters of logical shard elements [lo, lo + n)."""
        parts, a, e = [], b + lo, b + lo + n
        k = int(np.searchsorted(starts, a, side="right")) - 1
        while a < e:
            hi = min(e, int(starts[k + 1]))
            parts.append(wl.params[k][a - starts[k]:hi - starts[k]])
            a, k = hi, k + 1
        return torch.cat(parts).cpu().numpy().view(np.uint16)

    def oracle_piece(blk):
        lo, n = blk
        g = host_grad(w, 0, (b + lo, n))
        u, _, _ = oracle.grad_stats(w.dtype, [g], wl.inv)
        st = oracle.RankState(w.dtype, synth.normal_16(n, w.dtype, w.seed, mstream, b + lo, w.master_sigma),
                              synth.normal_f32(n, w.seed, mstream, b + lo, w.master_sigma))
        for _ in range(2):
            oracle.adam(False, u, clip, hp, st.counters, st.w, st.m, st.v)
            oracle.cast(w.dtype, st.w, st.p16)
        return lo, n, st

    step = 1 << 25
    blocks = [(lo, min(step, valid - lo)) for lo in range(0, valid, step)]
    checked = 0
    synth.set_host_threads(1)
    try:
        with ThreadPoolExecutor(16) as ex:
            for wave in range(0, len(blocks), 16):          # bounded: 16 pieces in memory at a time
                for lo, n, st in ex.map(oracle_piece, blocks[wave:wave + 16]):
                    for name, exp in (("master", st.w), ("m", st.m), ("v", st.v)):
                        got = exports[name][lo:lo + n].cpu().numpy()
                        bad = np.flatnonzero(got.view(np.uint32) != exp.view(np.uint32))
                        assert bad.size == 0, f"{name}: {bad.size} elements differ in [{lo}, {lo + n}), first {bad[:5]}"
                    bad = np.flatnonzero(device16(lo, n) != st.p16)
                    assert bad.size == 0, f"p16: {bad.size} elements differ in [{lo}, {lo + n}), first {bad[:5]}"
                    checked += n
                print(f"[fullstate] {checked} of {valid} elements match", flush=True)
    finally:
        synth.set_host_threads(0)
    assert checked == valid
    del exports
    wl.shard.close()
    del wl
