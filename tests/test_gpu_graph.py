"""The step captured into a HIP graph and replayed, and the ranks' exchange of
their statistics done in place on the device.

Each replay of a captured step is one more step: the step counters, the loss
scale and the choice of counter slot live in the workspace.  Between replays
the test writes the next gradient into the registered buffers, runs eager work
(exports, queries) and synchronises; after every replay the state is compared
with the oracle element by element (bit-exact), with the step count, skip
decision, clip and loss scale checked as well.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import recipes
from tests.gpu_harness import Sim, dev16

pytestmark = pytest.mark.gpu
F16, BF16 = oracle.F16, oracle.BF16


@pytest.fixture(autouse=True)
def _gpu(need_gpu):
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def hp_of(d):
    return oracle.HParams(d["lr"], d["beta1"], d["beta2"], d["eps"], d["weight_decay"])


def write_registered(sim, g_full):
    sim._device_grads([g_full])
    torch.cuda.synchronize()


def stats_views(s):
    """torch views of a shard's device-resident sum of squares (fp64) and flag (int32)."""
    ss_ptr, fl_ptr = s.zero_local_stats_device()
    base = s.workspace.data_ptr()
    o_ss, o_fl = ss_ptr - base, fl_ptr - base
    assert 0 <= o_ss and o_ss + 8 <= s.workspace.numel() and 0 <= o_fl and o_fl + 4 <= s.workspace.numel()
    return s.workspace[o_ss:o_ss + 8].view(torch.float64), s.workspace[o_fl:o_fl + 4].view(torch.int32)


def check_after(sim, res, max_norm):
    """Device reports and state against the oracle's step results."""
    for r in sim.ranks:
        q = sim.shards[r].query()
        assert q["skipped"] == res[r]["skipped"], (r, q, res[r])
        assert q["t"] == sim.ostates[r].counters.t, (r, q)
        if not q["skipped"]:
            assert q["clip"] == res[r]["clip"], (r, q, res[r])
    sim.compare()


@pytest.mark.parametrize("dynamic", [False, True])
def test_captured_step_replays(dynamic):
    """One rank (N_d = 1) of the ragged mini list with registered per-tensor gradients:
    one eager step, then the step captured once and replayed six times, with an
    overflow in the third replay.  bf16 with a static scale, or fp16 with the
    device-resident dynamic scale (growth every 2 good steps)."""
    w = recipes.ragged_mini(1)
    dtype = F16 if dynamic else BF16
    psi = w.psi
    master = synth.normal_f32(psi, w.seed, synth.stream_id(synth.MASTER), 0, w.master_sigma)
    p16 = synth.normal_16(psi, dtype, w.seed, synth.stream_id(synth.MASTER), 0, w.master_sigma)
    sim = Sim(w.numel, 1, dtype, p16, master, "ragged", per_tensor_params=True)
    sim.p16_initial = p16.copy()
    hp = hp_of(w.hp)
    scale = 1024.0
    sigma = w.grad_sigma * (scale if dynamic else 1.0) * 30.0      # clipping active
    if dynamic:
        sim.enable_dynamic(init_scale=scale, growth=2.0, backoff=0.5, interval=2, min_scale=1.0)

    def grads(step):
        g = synth.normal_16(psi, dtype, w.seed, synth.stream_id(synth.GRAD, 0, step), 0, sigma)
        if step == 4:
            g[psi // 3] = 0x7C00 if dtype == F16 else 0x7F80     # +inf: the third replay skips
        return g

    # step 1, eager (also loads the kernels before capture)
    res = sim.step([grads(1)], 1.0, w.max_norm, hp)
    assert not res[0]["skipped"] and res[0]["clip"] < 1.0
    sim.compare()

    s = sim.shards[0]
    inv_oracle, inv_dev = sim._intake_inv(1.0)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        s.zero_reduce_grads([], inv_dev)
        s.zero_check_overflow(False)
        s.zero_grad_norm(0.0, w.max_norm)
        s.zero_adam_step(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, fuse_cast=True)
    torch.cuda.synchronize()
    assert s.query()["t"] == 1            # capturing runs nothing

    for step in range(2, 8):
        g = grads(step)
        inv_oracle, _ = sim._intake_inv(1.0)
        res = oracle.step_ranks(sim.ostates, [g], sim.begins, inv_oracle, w.max_norm, hp)
        write_registered(sim, g)
        graph.replay()
        torch.cuda.synchronize()
        assert res[0]["skipped"] == (step == 4)
        check_after(sim, res, w.max_norm)
        sim._after_step(res)               # with the dynamic scale: the oracle's scaler, and the device's
    assert sim.ostates[0].counters.t == 6
    if dynamic:
        # 6 applied steps with a backoff at the fourth: 1024 -> 2048 -> 1024 -> 2048 (growth every 2)
        assert sim.scaler.scale.value == 2048.0


def test_captured_multi_rank_step_with_device_exchange():
    """Two ranks of N_d = 2 on one GPU, their whole step captured into one graph:
    both intakes, the exchange of the two scalars done in place on the device (the sum
    of squares added in rank order, the flags combined by max) into each rank's
    workspace, then each rank's overflow check, norm and Adam with zero for the other
    ranks.  Replayed five times with an overflow in one rank's slice at the second
    replay; the oracle adds the ranks' sums in the same order, so clip and state
    are expected bit-exact."""
    w = recipes.ragged_mini(2)
    psi = w.psi
    master = synth.normal_f32(psi, w.seed, synth.stream_id(synth.MASTER), 0, w.master_sigma)
    p16 = synth.normal_16(psi, w.dtype, w.seed, synth.stream_id(synth.MASTER), 0, w.master_sigma)
    sim = Sim(w.numel, 2, w.dtype, p16, master, "ragged", per_tensor_params=True)
    sim.p16_initial = p16.copy()
    hp = hp_of(w.hp)
    S = sim.plans[0][1]

    def grads(step):
        g = synth.normal_16(psi, w.dtype, w.seed, synth.stream_id(synth.GRAD, 0, step), 0, w.grad_sigma * 40.0)
        if step == 3:
            g[S + 17] = 0x7FC0                                   # NaN in rank 1's slice only
        return g

    res = sim.step([grads(1)], 1.0, w.max_norm, hp)              # eager step 1
    sim.compare()

    shards = [sim.shards[r] for r in (0, 1)]
    views = [stats_views(s) for s in shards]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in shards:
            s.zero_reduce_grads([], 1.0)
        tot = views[0][0] + views[1][0]                          # rank order
        flag = torch.maximum(views[0][1], views[1][1])
        for ss, fl in views:
            ss.copy_(tot)
            fl.copy_(flag)
        for s in shards:
            s.zero_check_overflow(False)
            s.zero_grad_norm(0.0, w.max_norm)
            s.zero_adam_step(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, fuse_cast=True)
    torch.cuda.synchronize()

    for step in range(2, 7):
        g = grads(step)
        res = oracle.step_ranks(sim.ostates, [g], sim.begins, 1.0, w.max_norm, hp)
        write_registered(sim, g)
        graph.replay()
        torch.cuda.synchronize()
        assert all(x["skipped"] == (step == 3) for x in res)
        glob = res[0]["local_sumsq"] + res[1]["local_sumsq"]
        for ss, fl in views:
            assert int(fl.item()) == int(step == 3)
            if step != 3:
                assert abs(ss.item() - glob) <= 1e-9 * glob       # the device's order of the per-rank terms
        check_after(sim, res, w.max_norm)
    assert sim.ostates[0].counters.t == 5


def test_device_exchange_eager():
    """The same device-side exchange without a graph, on three ranks of a flat
    pre-reduced gradient: after each rank's intake the sums are added in rank order
    and the flags combined on the device, written back in place, and every rank
    steps with zero for the other ranks."""
    w = recipes.tiny()
    psi, nd = 150_001, 3
    master = synth.normal_f32(psi, w.seed, synth.stream_id(synth.MASTER), 0, w.master_sigma)
    p16 = synth.normal_16(psi, w.dtype, w.seed, synth.stream_id(synth.MASTER), 0, w.master_sigma)
    sim = Sim([psi], nd, w.dtype, p16, master, "flat")
    sim.p16_initial = p16.copy()
    hp = hp_of(w.hp)
    inv = 1.0 / w.loss_scale
    for step in range(1, 4):
        g = synth.normal_16(psi, w.dtype, w.seed, synth.stream_id(synth.GRAD, 0, step), 0, w.grad_sigma * 3.0)
        if step == 2:
            g[2 * sim.plans[0][1] + 5] = 0xFC00                 # -inf in rank 2's slice
        res = oracle.step_ranks(sim.ostates, [g], sim.begins, inv, w.max_norm, hp)
        dg = [dev16(g)]
        shards = [sim.shards[r] for r in range(nd)]
        views = [stats_views(s) for s in shards]
        for s in shards:
            s.zero_reduce_grads(dg, inv)
        tot = views[0][0].clone()
        for ss, _ in views[1:]:
            tot = tot + ss
        flag = views[0][1].clone()
        for _, fl in views[1:]:
            flag = torch.maximum(flag, fl)
        for ss, fl in views:
            ss.copy_(tot)
            fl.copy_(flag)
        for s in shards:
            s.zero_check_overflow(False)
            s.zero_grad_norm(0.0, w.max_norm)
            s.zero_adam_step(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, fuse_cast=True)
        torch.cuda.synchronize()
        assert all(x["skipped"] == (step == 2) for x in res)
        check_after(sim, res, w.max_norm)


def test_captured_accumulation_replays():
    """Two micro-steps per step captured into one graph (an accumulation from a flat
    buffer, then the intake of a second flat buffer on top of it, the Adam pass
    recomputing u from the accumulator): four replays with new contents written into the
    two device buffers between replays, an overflow in the first micro-step of the
    third replay."""
    w = recipes.ragged_mini(1)
    psi = w.psi
    master = synth.normal_f32(psi, w.seed, synth.stream_id(synth.MASTER), 0, w.master_sigma)
    p16 = synth.normal_16(psi, w.dtype, w.seed, synth.stream_id(synth.MASTER), 0, w.master_sigma)
    sim = Sim([psi], 1, w.dtype, p16, master, "flat", with_red=True)
    sim.p16_initial = p16.copy()
    hp = hp_of(w.hp)

    def micro(step):
        gs = [synth.normal_16(psi, w.dtype, w.seed, synth.stream_id(synth.GRAD, 0, 10 * step + k), 0,
                              w.grad_sigma * 20.0) for k in range(2)]
        if step == 4:
            gs[0][psi - 3] = 0xFF80                            # -inf in the first micro-step
        return gs

    res = sim.step_accumulated([[g] for g in micro(1)], 1.0, w.max_norm, hp)     # eager step 1
    sim.compare()
    s = sim.shards[0]
    bufs = [torch.empty(psi, dtype=torch.int16, device="cuda") for _ in range(2)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        s.zero_accumulate_grads([bufs[0]])
        s.zero_reduce_grads([bufs[1]], 1.0)
        s.zero_check_overflow(False)
        s.zero_grad_norm(0.0, w.max_norm)
        s.zero_adam_step(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, fuse_cast=True)
    torch.cuda.synchronize()
    for step in range(2, 6):
        gs = micro(step)
        res = oracle.step_ranks_accumulated(sim.ostates, [[g] for g in gs], sim.begins, 1.0, w.max_norm, hp)
        for buf, g in zip(bufs, gs):
            buf.copy_(dev16(g))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert res[0]["skipped"] == (step == 4)
        check_after(sim, res, w.max_norm)
    assert sim.ostates[0].counters.t == 4
