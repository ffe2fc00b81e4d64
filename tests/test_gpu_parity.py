"""Parity of the HIP path with the oracle, element by element (MI355X).

Sizes span many chunks and ragged tails; every rank of the data-parallel group
is simulated so the shard boundaries and the exchange are exercised.
Tolerance (stated for the method): fp32 master/m/v within 2 ulp or 1e-6
relative, 16-bit parameters within 1 ulp, flags and skip decisions and t
exact, norm within 1e-6 relative (local sums of squares within 1e-9).  Past
that bar the values are also required to be bit-exact: the kernels take the
oracle's operation order with correctly rounded fp32 arithmetic.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import recipes
from tests.gpu_harness import Layout, Sim, dev16, host16

pytestmark = pytest.mark.gpu
F16, BF16 = oracle.F16, oracle.BF16


@pytest.fixture(autouse=True)
def _gpu(need_gpu):
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def hp_of(d):
    return oracle.HParams(d["lr"], d["beta1"], d["beta2"], d["eps"], d["weight_decay"])


def grads_for(w, step, psi, nranks):
    return [synth.normal_16(psi, w.dtype, w.seed, synth.stream_id(synth.GRAD, q, step), 0, w.grad_sigma,
                            zero_seed=w.seed if w.zero_mod else 0, zero_mod=w.zero_mod) for q in range(nranks)]


def master_of(w, psi):
    m = synth.normal_f32(psi, w.seed, synth.stream_id(synth.MASTER), 0, w.master_sigma)
    return m, synth.normal_16(psi, w.dtype, w.seed, synth.stream_id(synth.MASTER), 0, w.master_sigma)


# --------------------------------------------------------------------------
# the tiny workload: 4 ranks, fp16, loss scale 1024, 5 steps, inf injected at step 2


@pytest.mark.parametrize("bad,where,at_step", [
    (np.inf, "own", 2), (-np.inf, "own", 2), (np.nan, "own", 2), (np.inf, "other", 2), (np.inf, "own", 1)])
def test_tiny_workload_all_ranks(bad, where, at_step):
    w = recipes.tiny()
    psi = w.psi
    master, p16 = master_of(w, psi)
    sim = Sim(w.numel, w.nd, w.dtype, p16, master, "reduce")
    sim.p16_initial = p16.copy()
    hp = hp_of(w.hp)
    S = sim.plans[0][1]
    for step in range(1, w.steps + 1):
        g = grads_for(w, step, psi, w.nd)
        if step == at_step:
            r_bad = 3 if where == "own" else 1
            g[0][r_bad * S + 777] = oracle.encode16(F16, np.array([bad], np.float32))[0]
        res = sim.step(g, 1.0 / w.loss_scale, w.max_norm, hp)
        assert all(x["skipped"] == (step == at_step) for x in res)
        sim.compare()
    assert all(st.counters.t == w.steps - 1 for st in sim.ostates)


# --------------------------------------------------------------------------
# ragged per-tensor list with shard cuts inside rows


@pytest.mark.parametrize("nd", [3, 7])
@pytest.mark.parametrize("fuse", [True, False])
def test_ragged_mini_all_ranks(nd, fuse):
    w = recipes.ragged_mini(nd)
    psi = w.psi
    master, p16 = master_of(w, psi)
    # at least one shard boundary falls strictly inside a row of a 2-D tensor
    starts = np.cumsum([0] + w.numel)
    cut_mid_row = False
    for r in range(1, nd):
        b = oracle.plan(w.numel, nd, r)[2]
        k = int(np.searchsorted(starts, b, side="right") - 1)
        if w.numel[k] > 256 and (b - starts[k]) % 256 != 0:
            cut_mid_row = True
    assert cut_mid_row
    sim = Sim(w.numel, nd, w.dtype, p16, None, "ragged", per_tensor_params=True)
    sim.p16_initial = p16.copy()
    hp = hp_of(w.hp)
    for step in range(1, w.steps + 1):
        sim.step(grads_for(w, step, psi, 1), 1.0, w.max_norm, hp, fuse=fuse)
        sim.compare()
    # the layout reported by the library is the oracle's partition
    for r in sim.ranks:
        pieces = sim.shards[r].pieces()
        _, _, b, valid = sim.plans[r]
        exp = oracle.shard_pieces(w.numel, b, valid)
        assert [(p[0], p[1], p[2], p[4]) for p in pieces] == exp


# --------------------------------------------------------------------------
# one already-reduced flat gradient (the ZeRO-1 path), fp16 with loss scale 2^16


@pytest.mark.parametrize("nd,psi", [(5, 300_001), (2, 64 * 8192 + 3), (1, 77_777)])
def test_flat_prereduced_all_ranks(nd, psi):
    w = recipes.zero1_7p5b()
    w.tensors = [("flat", psi)]
    master, p16 = master_of(w, psi)
    sim = Sim(w.numel, nd, w.dtype, p16, master, "flat")
    sim.p16_initial = p16.copy()
    hp = hp_of(w.hp)
    for step in range(1, 4):
        sim.step(grads_for(w, step, psi, 1), 1.0 / w.loss_scale, w.max_norm, hp)
        sim.compare()


@pytest.mark.parametrize("nd", [2, 3, 8, 11, 64])
def test_reduce_fan_in(nd):
    """Local reduce with the specialised (2, 8) and the generic (3, 11, and the maximum
    64) fan-ins."""
    w = recipes.reduce8()
    psi = (40_000 if nd <= 11 else 4_000) * nd + 13
    w.tensors = [("flat", psi)]
    master, p16 = master_of(w, psi)
    sim = Sim(w.numel, nd, w.dtype, p16, master, "reduce", ranks=[0, nd - 1])
    sim.p16_initial = p16.copy()
    for step in range(1, 3):
        sim.step(grads_for(w, step, psi, nd), 1.0, w.max_norm, hp_of(w.hp))
        sim.compare()


# --------------------------------------------------------------------------
# edge cases


def test_ranks_without_elements_and_tiny_tensors():
    # psi below N_d * 64: the last ranks own nothing; tensors of 0, 1 and 7 elements
    numel = [0, 1, 7, 50, 0, 3]
    w = recipes.ragged_mini(5)
    psi = sum(numel)
    master, p16 = master_of(w, psi)
    sim = Sim(numel, 5, BF16, p16, None, "ragged", per_tensor_params=True)
    sim.p16_initial = p16.copy()
    assert [p[3] for p in sim.plans] == [61, 0, 0, 0, 0]
    for step in range(1, 3):
        sim.step(grads_for(w, step, psi, 1), 1.0, 1.0, hp_of(w.hp))
        sim.compare()


def test_empty_model():
    """Every tensor empty (psi = 0): no elements anywhere, yet each step is a step --
    zero norm, no overflow, t advances -- for every rank."""
    numel = [0, 0, 0]
    w = recipes.ragged_mini(3)
    p16 = np.zeros(0, np.uint16)
    sim = Sim(numel, 3, BF16, p16, None, "ragged", per_tensor_params=True)
    assert [p[3] for p in sim.plans] == [0, 0, 0]
    for step in range(1, 3):
        res = sim.step([np.zeros(0, np.uint16)], 1.0, 1.0, hp_of(w.hp))
        assert not any(x["skipped"] for x in res) and all(x["norm"] == 0.0 for x in res)
        sim.compare()
    assert all(st.counters.t == 2 for st in sim.ostates)


@pytest.mark.parametrize("hp", [dict(lr=1e-3, beta1=0.0, beta2=0.0, eps=1e-8, weight_decay=0.0),
                                dict(lr=0.0, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1),
                                dict(lr=1e-2, beta1=0.5, beta2=0.5, eps=1e-3, weight_decay=0.5)])
def test_degenerate_hyperparameters(hp):
    """beta = 0 (m = g, v = g^2, no bias correction left), lr = 0 (nothing moves), and
    large eps / weight decay, on the tiny workload's shapes (4 ranks, fp16, scale 1024)."""
    w = recipes.tiny()
    psi = 100_003
    master, p16 = master_of(w, psi)
    sim = Sim([psi], w.nd, w.dtype, p16, master, "reduce")
    sim.p16_initial = p16.copy()
    for step in range(1, 4):
        sim.step(grads_for(w, step, psi, w.nd), 1.0 / w.loss_scale, w.max_norm, hp_of(hp))
        sim.compare()
    if hp["lr"] == 0.0:
        for r in sim.ranks:
            _, _, b, valid = sim.plans[r]
            assert (sim.shards[r].export("master").cpu().numpy().view(np.uint32) ==
                    master[b:b + valid].view(np.uint32)).all()


def test_eps_zero_with_exact_zero_gradients():
    """eps = 0 where the reduced gradient is exactly zero: m = v = 0 there, so the update is
    0/0 = NaN, the master turns NaN and the 16-bit write-back takes the canonical NaN, on the
    GPU as in the oracle (elsewhere the step is ordinary)."""
    w = recipes.tiny()
    psi = 100_003
    master, p16 = master_of(w, psi)
    sim = Sim([psi], w.nd, w.dtype, p16, master, "reduce")
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=0.0, weight_decay=0.01)
    zeros = np.arange(5, psi, 97)
    for step in range(1, 3):
        g = grads_for(w, step, psi, w.nd)
        for x in g:
            x[zeros] = 0                                   # +0.0 in every rank: an exact zero sum
        sim.step(g, 1.0 / w.loss_scale, w.max_norm, hp_of(hp))
        sim.compare()
    for r in sim.ranks:
        _, _, b, valid = sim.plans[r]
        got = sim.shards[r].export("master").cpu().numpy()
        mine = zeros[(zeros >= b) & (zeros < b + valid)] - b
        # (other elements whose four fp16 terms cancel exactly are NaN too, on both sides)
        assert np.isnan(got[mine]).all() and (np.isnan(got) == np.isnan(sim.ostates[r].w)).all()


@pytest.mark.parametrize("cap", ["1", "3"])
def test_capped_grid(cap, monkeypatch):
    """ZERO_SHARD_BLOCKS_PER_CU caps the streaming grids (init, accumulation, Adam, cast,
    export) at that many blocks per CU, so every block walks several work items: all
    ranks of the ragged list with two micro-steps per step, 8 tracked segments, and the
    cast fused or not, against the oracle."""
    monkeypatch.setenv("ZERO_SHARD_BLOCKS_PER_CU", cap)
    w = recipes.ragged_mini(3)
    psi = w.psi
    master, p16 = master_of(w, psi)
    sim = Sim(w.numel, 3, w.dtype, p16, master, "ragged", per_tensor_params=True, with_red=True, segments=8)
    sim.p16_initial = p16.copy()
    for step in range(1, 4):
        sim.step_accumulated(micro_grads(w, step, psi, 1, 2), 1.0, w.max_norm, hp_of(w.hp), fuse=(step != 2),
                             last_fused=(step != 3))
        sim.compare()


@pytest.mark.parametrize("align,mode,nd", [(8, "reduce", 3), (8, "ragged", 5), (256, "reduce", 4), (1024, "ragged", 3)])
def test_shard_alignment(align, mode, nd):
    """Shard lengths rounded to `align` elements other than the default 64: 8 (shard
    boundaries at 16-byte steps of the 16-bit data, so the rank slices start at every
    phase the kernels peel), 256 and 1024 (larger padding at the last rank).  Every rank
    against the oracle's partition with the same alignment, two steps."""
    w = recipes.ragged_mini(nd) if mode == "ragged" else recipes.tiny()
    numel = w.numel if mode == "ragged" else [100_003]
    psi = sum(numel)
    master, p16 = master_of(w, psi)
    sim = Sim(numel, nd, w.dtype, p16, master, mode, per_tensor_params=(mode == "ragged"), align=align)
    sim.p16_initial = p16.copy()
    for r in range(nd):
        _, S, b, _ = sim.plans[r]
        assert S % align == 0 and b == r * S
        assert sim.shards[r].info.shard_elems == S
    inv = 1.0 / w.loss_scale
    for step in range(1, 3):
        sim.step(grads_for(w, step, psi, nd if mode == "reduce" else 1), inv, w.max_norm, hp_of(w.hp))
        sim.compare()


@pytest.mark.parametrize("pmis,gmis", [((1, 3, 5, 7), (0,)), ((2,), (1,)), ((3,), (3,)), ((1, 2), (2, 1))])
def test_misaligned_tensors(pmis, gmis):
    """Per-tensor parameters and gradients starting at odd element offsets: the
    kernels peel heads or fall back to one element per lane, same results."""
    numel = [5000, 1, 8193, 64, 12345, 3]
    w = recipes.ragged_mini(3)
    psi = sum(numel)
    master, p16 = master_of(w, psi)
    sim = Sim(numel, 3, F16, p16, master, "ragged", per_tensor_params=True, param_misalign=pmis,
              grad_misalign=gmis)
    sim.p16_initial = p16.copy()
    for step in range(1, 3):
        sim.step(grads_for(w, step, psi, 1), 1.0, 1.0, hp_of(w.hp))
        sim.compare()


def test_extreme_values_and_clipping_off():
    """Gradients at the fp16 extremes (subnormals, 65504) and clipping disabled."""
    psi, nd = 70_000, 2
    w = recipes.tiny()
    master, p16 = master_of(w, psi)
    vals = np.array([6e-8, -6e-8, 1e-7, 65504.0, -65504.0, 0.0, -0.0, 1.0, 3e-5], np.float32)
    g = np.resize(oracle.encode16(F16, vals), psi)
    g2 = np.resize(oracle.encode16(F16, vals[::-1].copy()), psi)
    sim = Sim([psi], nd, F16, p16, master, "reduce")
    sim.p16_initial = p16.copy()
    sim.step([g, g2], 1.0, 0.0, hp_of(w.hp))
    sim.compare()
    sim.step([g2, g], 1.0 / 65536, 1e30, hp_of(w.hp))
    sim.compare()


def test_step_order_is_enforced():
    from zero_partitioned_mixed_reduce_amd import ZeroError
    from zero_partitioned_mixed_reduce_amd._abi import ZERO_ESTATE, ZERO_EINVAL
    psi = 4096
    w = recipes.tiny()
    _, p16 = master_of(w, psi)
    from zero_partitioned_mixed_reduce_amd.shard import ZeroShard
    params = dev16(p16)
    s = ZeroShard([psi], 1, 0, F16, params)
    g = dev16(grads_for(w, 1, psi, 1)[0])
    with pytest.raises(ZeroError) as e:
        s.zero_adam_step(1e-3, 0.9, 0.999, 1e-8, 0.0)
    assert e.value.status == ZERO_ESTATE
    with pytest.raises(ZeroError) as e:
        s.zero_reduce_grads([], 1.0)          # no registered gradient
    assert e.value.status == ZERO_EINVAL
    s.zero_reduce_grads([g], 1.0)
    with pytest.raises(ZeroError):
        s.zero_grad_norm(0.0, 1.0)            # check_overflow first
    s.zero_check_overflow(False)
    s.zero_grad_norm(0.0, 1.0)
    s.zero_adam_step(1e-3, 0.9, 0.999, 1e-8, 0.0, fuse_cast=False)
    with pytest.raises(ZeroError):
        s.zero_reduce_grads([g], 1.0)         # cast pending
    s.zero_cast_params()
    s.zero_cast_params()                      # already done: no-op
    s.zero_reduce_grads([g], 1.0)
    assert s.query()["t"] == 1


def test_statistics_are_deterministic():
    psi = 3_000_000
    w = recipes.gpt2_shard()
    _, p16 = master_of(w, psi)
    from zero_partitioned_mixed_reduce_amd.shard import ZeroShard
    s = ZeroShard([psi], 1, 0, BF16, dev16(p16))
    g = dev16(grads_for(w, 1, psi, 1)[0])
    vals = set()
    for _ in range(10):
        s.zero_reduce_grads([g], 1.0)
        vals.add(s.zero_local_stats()[1])
    assert len(vals) == 1


def test_device_generator_matches_host_generator():
    n = 5_000_003
    t = torch.empty(n, dtype=torch.int16, device="cuda")
    synth.gpu_normal_16(t, F16, 77, 5, first=123, sigma=3.0, zero_seed=9, zero_mod=100)
    assert (host16(t) == synth.normal_16(n, F16, 77, 5, 123, 3.0, 9, 100)).all()
    f = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.gpu_normal_f32(f, 77, 6, first=5, sigma=0.02)
    assert (f.cpu().numpy().view(np.uint32) == synth.normal_f32(n, 77, 6, 5, 0.02).view(np.uint32)).all()


# --------------------------------------------------------------------------
# gradient accumulation over micro-steps


def micro_grads(w, step, psi, nranks, K):
    return [[synth.normal_16(psi, w.dtype, w.seed, synth.stream_id(synth.GRAD, q, 100 * step + k), 0, w.grad_sigma)
             for q in range(nranks)] for k in range(K)]


@pytest.mark.parametrize("last_fused", [True, False])
def test_accumulation_tiny_all_ranks(last_fused):
    w = recipes.tiny()
    psi = w.psi
    master, p16 = master_of(w, psi)
    sim = Sim(w.numel, w.nd, w.dtype, p16, master, "reduce")
    sim.p16_initial = p16.copy()
    hp = hp_of(w.hp)
    S = sim.plans[0][1]
    for step in range(1, 4):
        micro = micro_grads(w, step, psi, w.nd, 3)
        if step == 2:
            micro[1][2][1 * S + 5] = 0x7C00           # inf in rank 1's slice, micro-step 2 of step 2
        res = sim.step_accumulated(micro, 1.0 / w.loss_scale, w.max_norm, hp, last_fused=last_fused)
        assert all(x["skipped"] == (step == 2) for x in res)
        sim.compare()


@pytest.mark.parametrize("mode,nd,K", [("flat", 5, 4), ("ragged", 3, 2), ("reduce", 3, 2), ("reduce", 8, 2)])
def test_accumulation_modes(mode, nd, K):
    w = recipes.ragged_mini(nd) if mode == "ragged" else recipes.tiny()
    psi = w.psi if mode == "ragged" else 200_003
    numel = w.numel if mode == "ragged" else [psi]
    master, p16 = master_of(w, psi)
    sim = Sim(numel, nd, w.dtype, p16, None if mode == "ragged" else master, mode,
              per_tensor_params=(mode == "ragged"), ranks=None if nd <= 5 else [0, nd - 1], with_red=True)
    sim.p16_initial = p16.copy()
    for step in range(1, 3):
        micro = micro_grads(w, step, psi, nd if mode == "reduce" else 1, K)
        sim.step_accumulated(micro, 1.0 / w.loss_scale, w.max_norm, hp_of(w.hp), last_fused=(step == 1))
        sim.compare()


@pytest.mark.parametrize("last_fused", [True, False])
def test_accumulation_misaligned_tensors(last_fused):
    """Registered per-tensor gradients at odd offsets, accumulated over three micro-steps;
    the last one through the intake itself (the Adam pass then re-reads the registered
    gradient next to the accumulator) or accumulated too (ZERO_ACCUMULATED)."""
    numel = [5000, 1, 8193, 64, 12345, 3]
    w = recipes.ragged_mini(3)
    psi = sum(numel)
    master, p16 = master_of(w, psi)
    sim = Sim(numel, 3, F16, p16, master, "ragged", per_tensor_params=True, param_misalign=(1, 3),
              grad_misalign=(2,), with_red=True)
    sim.p16_initial = p16.copy()
    for step in (1, 2):
        sim.step_accumulated(micro_grads(w, step, psi, 1, 3), 1.0, 1.0, hp_of(w.hp), last_fused=last_fused)
        sim.compare()


def test_accumulation_step_order():
    from zero_partitioned_mixed_reduce_amd import ZeroError, ZERO_ACCUMULATED
    from zero_partitioned_mixed_reduce_amd._abi import ZERO_ESTATE, ZERO_EINVAL
    from zero_partitioned_mixed_reduce_amd.shard import ZeroShard
    psi = 4096
    w = recipes.tiny()
    _, p16 = master_of(w, psi)
    g = dev16(grads_for(w, 1, psi, 1)[0])
    s = ZeroShard([psi], 1, 0, F16, dev16(p16), with_red=True)
    with pytest.raises(ZeroError) as e:
        s.zero_reduce_grads(ZERO_ACCUMULATED, 1.0)           # nothing accumulated
    assert e.value.status == ZERO_ESTATE
    s.zero_accumulate_grads([g])
    s.zero_reduce_grads([g], 1.0)
    with pytest.raises(ZeroError) as e:
        s.zero_accumulate_grads([g])                         # after the step's intake
    assert e.value.status == ZERO_ESTATE
    s2 = ZeroShard([psi], 1, 0, F16, dev16(p16))             # no bufs.red
    with pytest.raises(ZeroError) as e:
        s2.zero_accumulate_grads([g])
    assert e.value.status == ZERO_EINVAL


# --------------------------------------------------------------------------
# dynamic loss scale kept on the device


def _poison(g, idx, dtype):
    g[idx] = oracle.encode16(dtype, np.array([np.inf], np.float32))[0]


def test_dynamic_loss_scale_tiny_all_ranks():
    """Backoff to the floor, growth after `interval` good steps, overflow in another
    rank's slice; the scale sequence is also checked against the rule by hand."""
    w = recipes.tiny()
    psi = w.psi
    master, p16 = master_of(w, psi)
    sim = Sim(w.numel, w.nd, w.dtype, p16, master, "reduce")
    sim.p16_initial = p16.copy()
    sim.enable_dynamic(init_scale=8.0, growth=2.0, backoff=0.5, interval=3, min_scale=2.0)
    hp = hp_of(w.hp)
    S = sim.plans[0][1]
    bad = {2: 0, 3: 3, 4: 1, 9: 2}                  # step -> rank slice holding an inf
    expect = {1: 8, 2: 4, 3: 2, 4: 2, 5: 2, 6: 2, 7: 4, 8: 4, 9: 2, 10: 2, 11: 2, 12: 4}
    for step in range(1, 13):
        g = grads_for(w, step, psi, w.nd)
        if step in bad:
            _poison(g[step % w.nd], bad[step] * S + 11 * step, w.dtype)
        res = sim.step(g, None, w.max_norm, hp)
        assert all(x["skipped"] == (step in bad) for x in res)
        assert sim.scaler.scale.value == expect[step], step
        sim.compare()
    assert all(st.counters.t == 12 - len(bad) for st in sim.ostates)


@pytest.mark.parametrize("mode,nd,fuse", [("flat", 3, True), ("ragged", 3, False), ("registered_flat", 2, True)])
def test_dynamic_loss_scale_modes(mode, nd, fuse):
    w = recipes.ragged_mini(nd) if mode == "ragged" else recipes.tiny()
    psi = w.psi if mode == "ragged" else 150_001
    numel = w.numel if mode == "ragged" else [psi]
    master, p16 = master_of(w, psi)
    sim = Sim(numel, nd, w.dtype, p16, None if mode == "ragged" else master, mode,
              per_tensor_params=(mode == "ragged"))
    sim.p16_initial = p16.copy()
    sim.enable_dynamic(init_scale=2.0 ** 12, growth=2.0, backoff=0.25, interval=2, min_scale=1.0)
    for step in range(1, 7):
        g = grads_for(w, step, psi, 1)
        if step in (3, 4):
            _poison(g[0], psi - 1 - 5 * step, w.dtype)
        res = sim.step(g, None, w.max_norm, hp_of(w.hp), fuse=fuse)
        assert all(x["skipped"] == (step in (3, 4)) for x in res)
        sim.compare()


@pytest.mark.parametrize("mode,last_fused", [("reduce", True), ("reduce", False), ("flat", True), ("flat", False)])
def test_dynamic_loss_scale_with_accumulation(mode, last_fused):
    """Device loss scale with two micro-steps: 3 rank buffers (u stored by the intake) or
    one already-reduced flat source (u recomputed by the Adam pass from the accumulator);
    an overflow in the first micro-step is seen only through the accumulator."""
    w = recipes.tiny()
    psi = 120_007
    master, p16 = master_of(w, psi)
    sim = Sim([psi], 3, F16, p16, master, mode, with_red=True)
    sim.p16_initial = p16.copy()
    sim.enable_dynamic(init_scale=1024.0, growth=2.0, backoff=0.5, interval=1, min_scale=1.0)
    S = sim.plans[0][1]
    for step in range(1, 5):
        micro = micro_grads(w, step, psi, 3 if mode == "reduce" else 1, 2)
        if step == 2:
            _poison(micro[0][min(1, len(micro[0]) - 1)], 2 * S + 3, F16)   # first micro-step only
        res = sim.step_accumulated(micro, None, w.max_norm, hp_of(w.hp), last_fused=last_fused)
        assert all(x["skipped"] == (step == 2) for x in res)
        sim.compare()


def test_dynamic_loss_scale_errors():
    from zero_partitioned_mixed_reduce_amd import ZeroError, ZERO_DEVICE_LOSS_SCALE
    from zero_partitioned_mixed_reduce_amd._abi import ZERO_ESTATE, ZERO_EINVAL
    from zero_partitioned_mixed_reduce_amd.shard import ZeroShard
    psi = 4096
    w = recipes.tiny()
    _, p16 = master_of(w, psi)
    g = dev16(grads_for(w, 1, psi, 1)[0])
    s = ZeroShard([psi], 1, 0, F16, dev16(p16))
    for bad_inv in (-1.0, float("inf"), float("nan")):
        with pytest.raises(ZeroError) as e:
            s.zero_reduce_grads([g], bad_inv)
        assert e.value.status == ZERO_EINVAL
    with pytest.raises(ZeroError) as e:
        s.zero_reduce_grads([g], ZERO_DEVICE_LOSS_SCALE)     # not enabled
    assert e.value.status == ZERO_EINVAL
    with pytest.raises(ZeroError) as e:
        s.zero_loss_scale()
    assert e.value.status == ZERO_ESTATE
    for cfg in [dict(init_scale=0.0), dict(growth_factor=0.5), dict(backoff_factor=1.5), dict(growth_interval=0),
                dict(min_scale=0.0)]:
        with pytest.raises(ZeroError) as e:
            s.zero_enable_dynamic_loss_scale(**cfg)
        assert e.value.status == ZERO_EINVAL
    s.zero_reduce_grads([g], 1.0)
    with pytest.raises(ZeroError) as e:
        s.zero_enable_dynamic_loss_scale()                   # inside a step
    assert e.value.status == ZERO_ESTATE
    s.zero_check_overflow(False)
    s.zero_grad_norm(0.0, 1.0)
    s.zero_adam_step(1e-3, 0.9, 0.999, 1e-8, 0.0)
    s.zero_enable_dynamic_loss_scale(init_scale=256.0)       # between steps
    assert s.zero_loss_scale() == (256.0, 0)
    with pytest.raises(ZeroError) as e:
        s.zero_reduce_grads([g], 1.0)                        # a host scale while dynamic
    assert e.value.status == ZERO_EINVAL
    s.zero_reduce_grads([g], ZERO_DEVICE_LOSS_SCALE)
    s.zero_check_overflow(False)
    s.zero_grad_norm(0.0, 1.0)
    s.zero_adam_step(1e-3, 0.9, 0.999, 1e-8, 0.0)
    assert s.query()["t"] == 2
    assert s.zero_loss_scale() == (256.0, 1)


# --------------------------------------------------------------------------
# chunk-pipelined step: per-segment completion of the 16-bit write-back


@pytest.mark.parametrize("fuse,segments", [(True, 3), (False, 7), (True, 256)])
def test_segmented_write_back_tiny_all_ranks(fuse, segments):
    """Tracking segments changes no result (the inf at step 2 skips)."""
    w = recipes.tiny()
    psi = w.psi
    master, p16 = master_of(w, psi)
    sim = Sim(w.numel, w.nd, w.dtype, p16, master, "reduce", segments=segments)
    sim.p16_initial = p16.copy()
    S = sim.plans[0][1]
    for step in range(1, 4):
        g = grads_for(w, step, psi, w.nd)
        if step == 2:
            _poison(g[1], 2 * S + 99, w.dtype)
        sim.step(g, 1.0 / w.loss_scale, w.max_norm, hp_of(w.hp), fuse=fuse)
        sim.compare()
    assert all(s.zero_segment_timeouts() == 0 for s in sim.shards.values())


def _segment_ranges(s, n):
    return [s.zero_segment_range(k) for k in range(n)]


@pytest.mark.parametrize("mode,nd,rank,segments", [("flat", 1, 0, 16), ("ragged", 3, 1, 9), ("flat", 5, 4, 256)])
def test_segment_consumer_sees_each_step(mode, nd, rank, segments):
    """A consumer stream waits for each segment, then copies it (standing in for the
    segment's all-gather): every copy equals the step's final 16-bit slice, also for
    a skipped step and for the unfused write-back."""
    w = recipes.ragged_mini(nd) if mode == "ragged" else recipes.gpt2_shard()
    psi = w.psi if mode == "ragged" else 3_000_017
    numel = w.numel if mode == "ragged" else [psi]
    master, p16 = master_of(w, psi)
    sim = Sim(numel, nd, w.dtype, p16, None, mode, per_tensor_params=(mode == "ragged"), ranks=[rank])
    s = sim.shards[rank]
    n = s.zero_set_segments(segments)
    assert n == min(segments, s.info.num_chunks)
    _, _, b, valid = sim.plans[rank]
    ranges = _segment_ranges(s, n)
    assert ranges[0][0] == 0 and sum(ln for _, ln in ranges) == valid
    assert all(ranges[k][0] + ranges[k][1] == ranges[k + 1][0] for k in range(n - 1))
    store, views = sim.params[rank]
    consumer = torch.cuda.Stream()
    for step in range(1, 5):
        g = grads_for(w, step, psi, 1)
        if step == 3:
            _poison(g[0], b + valid // 2, w.dtype)
        fuse = step != 2
        sim.step(g, 1.0, w.max_norm, hp_of(w.hp), fuse=fuse)
        flat_params = store if views is None else None
        got = torch.zeros(valid, dtype=torch.int16, device="cuda")
        main = torch.cuda.current_stream()
        consumer.wait_stream(main)         # the consumer's own inputs (got) are ready
        with torch.cuda.stream(consumer):
            for k, (lo, ln) in enumerate(ranges):
                s.zero_wait_segment(k, consumer)
                if flat_params is not None:
                    got[lo:lo + ln].copy_(flat_params[b + lo:b + lo + ln])
        torch.cuda.synchronize()
        exp = sim.ostates[rank].p16
        if flat_params is not None:
            assert (host16(got) == exp).all(), step
        sim.compare()
    assert s.zero_segment_timeouts() == 0


def test_segment_api_errors():
    from zero_partitioned_mixed_reduce_amd import ZeroError
    from zero_partitioned_mixed_reduce_amd._abi import ZERO_ESTATE, ZERO_EINVAL
    from zero_partitioned_mixed_reduce_amd.shard import ZeroShard
    psi = 100_000
    w = recipes.tiny()
    _, p16 = master_of(w, psi)
    g = dev16(grads_for(w, 1, psi, 1)[0])
    s = ZeroShard([psi], 1, 0, F16, dev16(p16))
    assert s.zero_set_segments(0) == 0
    for bad in (-1, 257):
        with pytest.raises(ZeroError) as e:
            s.zero_set_segments(bad)
        assert e.value.status == ZERO_EINVAL
    n = s.zero_set_segments(4)
    assert n == 4
    with pytest.raises(ZeroError) as e:
        s.zero_segment_range(4)
    assert e.value.status == ZERO_EINVAL
    with pytest.raises(ZeroError) as e:
        s.zero_wait_segment(0)                       # no step yet
    assert e.value.status == ZERO_ESTATE
    s.zero_reduce_grads([g], 1.0)
    with pytest.raises(ZeroError) as e:
        s.zero_set_segments(2)                       # inside a step
    assert e.value.status == ZERO_ESTATE
    s.zero_check_overflow(False)
    s.zero_grad_norm(0.0, 1.0)
    s.zero_adam_step(1e-3, 0.9, 0.999, 1e-8, 0.0, fuse_cast=False)
    with pytest.raises(ZeroError) as e:
        s.zero_wait_segment(0)                       # write-back not enqueued yet
    assert e.value.status == ZERO_ESTATE
    s.zero_cast_params()
    for k in range(n):
        s.zero_wait_segment(k)
    torch.cuda.synchronize()
    assert s.zero_segment_timeouts() == 0


# --------------------------------------------------------------------------
# 16-bit output of the local reduce ("DeepSpeed ZeRO", ZeRO Stage 2 基本思想: the fp32
# gradient shard comes from the reduce-scatter's bf16 result)


@pytest.mark.parametrize("bad,at_step", [(np.inf, 2), (np.nan, 1)])
def test_reduce16_tiny_all_ranks(bad, at_step):
    """The tiny workload with the 16-bit reduce output: fp16, loss scale 1024, 5 steps."""
    w = recipes.tiny()
    psi = w.psi
    master, p16 = master_of(w, psi)
    sim = Sim(w.numel, w.nd, w.dtype, p16, master, "reduce")
    sim.p16_initial = p16.copy()
    sim.set_reduce_out16()
    hp = hp_of(w.hp)
    S = sim.plans[0][1]
    for step in range(1, w.steps + 1):
        g = grads_for(w, step, psi, w.nd)
        if step == at_step:
            g[2][1 * S + 4321] = oracle.encode16(F16, np.array([bad], np.float32))[0]
        res = sim.step(g, 1.0 / w.loss_scale, w.max_norm, hp)
        assert all(x["skipped"] == (step == at_step) for x in res)
        sim.compare()


@pytest.mark.parametrize("nd,dtype,per_tensor", [(2, BF16, False), (3, F16, True), (8, BF16, False),
                                                 (11, F16, False)])
def test_reduce16_fan_in_and_layouts(nd, dtype, per_tensor):
    """Specialised (2, 8) and generic (3, 11) fan-ins; per-tensor parameters at odd
    offsets make the 16-bit result's alignment differ from the flat rank buffers'."""
    w = recipes.reduce8()
    numel = [40_000 * nd + 13] if not per_tensor else [5000, 1, 8193, 64, 12345, 3]
    psi = sum(numel)
    master, p16 = master_of(w, psi)
    sim = Sim(numel, nd, dtype, p16, master, "reduce", per_tensor_params=per_tensor, param_misalign=(1, 3, 2),
              ranks=None if nd <= 3 else [0, nd - 1])
    sim.p16_initial = p16.copy()
    sim.set_reduce_out16()
    for step in range(1, 3):
        g = [synth.normal_16(psi, dtype, w.seed, synth.stream_id(synth.GRAD, q, step), 0, 0.5) for q in range(nd)]
        sim.step(g, 1.0, 1.0, hp_of(w.hp))
        sim.compare()


def test_reduce16_fp16_overflow_skips():
    """A sum beyond 65504 becomes inf in the fp16 reduce output: every rank skips,
    while the fp32 reduce output of the same gradients steps normally."""
    w = recipes.tiny()
    psi, nd = 5000, 8
    master, p16 = master_of(w, psi)
    g = [synth.normal_16(psi, F16, w.seed, synth.stream_id(synth.GRAD, q, 1), 0, 1.0) for q in range(nd)]
    big = oracle.encode16(F16, np.array([10000.0], np.float32))[0]
    for q in range(nd):
        g[q][77] = big
    sim = Sim([psi], nd, F16, p16, master, "reduce", ranks=[0, nd - 1])
    sim.p16_initial = p16.copy()
    sim.set_reduce_out16()
    res = sim.step(g, 1.0 / 65536, 1.0, hp_of(w.hp))
    assert all(x["skipped"] for x in res) and res[0]["flag"]
    sim.compare()
    sim.set_reduce_out16(False)
    res = sim.step(g, 1.0 / 65536, 1.0, hp_of(w.hp))
    assert not any(x["skipped"] for x in res)
    sim.compare()


@pytest.mark.parametrize("last_fused", [True, False])
def test_reduce16_with_accumulation(last_fused):
    """Each micro-step's sum is rounded to 16 bits, then accumulated in fp32."""
    w = recipes.tiny()
    psi, nd = 150_001, 4
    master, p16 = master_of(w, psi)
    sim = Sim([psi], nd, F16, p16, master, "reduce")
    sim.p16_initial = p16.copy()
    sim.set_reduce_out16()
    for step in range(1, 3):
        micro = micro_grads(w, step, psi, nd, 3)
        sim.step_accumulated(micro, 1.0 / w.loss_scale, w.max_norm, hp_of(w.hp), last_fused=last_fused)
        sim.compare()


def test_reduce16_api():
    from zero_partitioned_mixed_reduce_amd import ZeroError
    from zero_partitioned_mixed_reduce_amd._abi import ZERO_ESTATE, ZERO_EINVAL
    from zero_partitioned_mixed_reduce_amd.shard import ZeroShard
    psi = 4096
    w = recipes.tiny()
    _, p16 = master_of(w, psi)
    gh = grads_for(w, 1, psi, 2)
    g = [dev16(x) for x in gh]
    s = ZeroShard([psi], 2, 0, F16, dev16(p16))
    with pytest.raises(ZeroError) as e:
        s.zero_set_reduce_output(True)                  # no bufs.red
    assert e.value.status == ZERO_EINVAL
    s.close()
    s = ZeroShard([psi], 2, 0, F16, dev16(p16), with_red=True)
    s.zero_set_reduce_output(True)
    s.zero_accumulate_grads(g)
    with pytest.raises(ZeroError) as e:
        s.zero_set_reduce_output(False)                 # while micro-steps are accumulated
    assert e.value.status == ZERO_ESTATE
    s.zero_reduce_grads(g, 1.0)
    with pytest.raises(ZeroError) as e:
        s.zero_set_reduce_output(False)                 # inside a step
    assert e.value.status == ZERO_ESTATE
    s.zero_check_overflow(False)
    s.zero_grad_norm(0.0, 1.0)
    s.zero_adam_step(1e-3, 0.9, 0.999, 1e-8, 0.0)
    s.export("red")                                     # an accumulated intake keeps fp32 values
    s.zero_reduce_grads(g, 1.0)
    with pytest.raises(ZeroError) as e:
        s.export("red")                                 # red now holds the 16-bit result
    assert e.value.status == ZERO_ESTATE
    s.zero_check_overflow(False)
    s.zero_grad_norm(0.0, 1.0)
    s.zero_adam_step(1e-3, 0.9, 0.999, 1e-8, 0.0)
    s.zero_accumulate_grads(g)                          # red holds an fp32 accumulator again
    acc = s.export("red").cpu().numpy()
    exp = oracle.decode16(F16, oracle.reduce_to16(F16, [x[:psi // 2] for x in gh]))
    assert (acc.view(np.uint32) == exp.view(np.uint32)).all()
    s.zero_reduce_grads(g, 1.0)
    s.zero_check_overflow(False)
    s.zero_grad_norm(0.0, 1.0)
    s.zero_adam_step(1e-3, 0.9, 0.999, 1e-8, 0.0)
    s.zero_set_reduce_output(False)
    torch.cuda.synchronize()
    s.close()


# --------------------------------------------------------------------------
# the write-back's NaN rule: every NaN is written as the canonical quiet NaN


def _nan_payload_values(n, seed):
    """n float32 values mixing payload NaNs of both signs (quiet and signalling), +-inf
    and ordinary N(0, 0.02) values."""
    r = np.random.default_rng(seed)
    x = (r.standard_normal(n) * 0.02).astype(np.float32)
    bits = x.view(np.uint32)
    kind = r.integers(0, 6, size=n)
    payload = r.integers(1, 1 << 23, size=n, dtype=np.uint32)
    sign = r.integers(0, 2, size=n, dtype=np.uint32) << 31
    nan_bits = sign | np.uint32(0x7F800000) | payload
    bits[kind == 0] = nan_bits[kind == 0]
    bits[kind == 1] = np.uint32(0x7F800000) | sign[kind == 1]            # +-inf
    return x


@pytest.mark.parametrize("dtype,fuse", [(F16, True), (F16, False), (BF16, True), (BF16, False)])
def test_nan_and_inf_master_write_back(dtype, fuse):
    """2 ranks; the given fp32 master holds payload NaNs of both signs and +-inf in both
    ranks' slices.  After two steps every NaN and inf master value has become a NaN (the
    decoupled decay of an infinite weight is inf - inf) and the 16-bit slice holds exactly
    the canonical quiet NaN there; everything else bit-exact with the oracle."""
    w = recipes.tiny()
    psi, nd = 70_001, 2
    master = _nan_payload_values(psi, 7 + dtype)
    p16 = oracle.encode16(dtype, master)
    sim = Sim([psi], nd, dtype, p16, master, "flat")
    sim.p16_initial = p16.copy()
    hp = hp_of(w.hp)
    for step in (1, 2):
        g = synth.normal_16(psi, dtype, w.seed, synth.stream_id(synth.GRAD, 0, step), 0, 1e-3)
        res = sim.step([g], 1.0, w.max_norm, hp, fuse=fuse)
        assert not any(x["skipped"] for x in res)
        sim.compare()
    canonical = 0x7E00 if dtype == F16 else 0x7FC0
    nonfinite = ~np.isfinite(master)
    assert nonfinite.sum() > psi // 4
    for r in sim.ranks:
        _, _, b, valid = sim.plans[r]
        store, views = sim.params[r]
        got = Layout.flat_of(views if views is not None else store)[b:b + valid]
        assert (got[nonfinite[b:b + valid]] == canonical).all()


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_nan_payload_16bit_params_upcast(dtype):
    """No master given: the master is the upcast of 16-bit parameters holding payload NaNs
    and +-inf; the step writes the canonical NaN back wherever the master is NaN."""
    w = recipes.tiny()
    psi, nd = 40_003, 2
    r = np.random.default_rng(11)
    p16 = oracle.encode16(dtype, (r.standard_normal(psi) * 0.02).astype(np.float32))
    e_bits, f_bits = (5, 10) if dtype == F16 else (8, 7)
    exp_all = ((1 << e_bits) - 1) << f_bits
    pick = r.integers(0, 5, size=psi)
    pay = r.integers(1, 1 << f_bits, size=psi).astype(np.uint16)
    sgn = (r.integers(0, 2, size=psi) << 15).astype(np.uint16)
    p16[pick == 0] = (sgn | np.uint16(exp_all) | pay)[pick == 0]
    p16[pick == 1] = (sgn | np.uint16(exp_all))[pick == 1]
    sim = Sim([psi], nd, dtype, p16, None, "flat")
    sim.p16_initial = p16.copy()
    g = synth.normal_16(psi, dtype, w.seed, synth.stream_id(synth.GRAD, 0, 1), 0, 1e-3)
    res = sim.step([g], 1.0, w.max_norm, hp_of(w.hp))
    assert not any(x["skipped"] for x in res)
    sim.compare()


# --------------------------------------------------------------------------
# the global sum of squares: one rank-order sum given to every rank


def test_global_sum_gives_every_rank_the_same_clip():
    """Local sums 1, 2^-53, 2^-53 (bf16 gradients 1.0 on rank 0, two of 2^-27 on ranks 1
    and 2): with zero_grad_norm_global every rank takes norm 1 and the same clip, and
    the state is bit-exact with the oracle's rank-order reading."""
    psi, nd = 3 * 64, 3
    master, _ = master_of(recipes.tiny(), psi)
    p16 = oracle.encode16(BF16, master)
    sim = Sim([psi], nd, BF16, p16, master, "flat")
    sim.p16_initial = p16.copy()
    g = np.zeros(psi, np.uint16)
    g[0] = oracle.encode16(BF16, np.array([1.0], np.float32))[0]
    tiny = oracle.encode16(BF16, np.array([2.0 ** -27], np.float32))[0]
    S = sim.plans[0][1]
    g[S] = g[S + 1] = g[2 * S] = g[2 * S + 1] = tiny
    res = sim.step([g], 1.0, 0.5, hp_of(recipes.tiny().hp))
    assert all(x["global_sumsq"] == 1.0 for x in res)
    qs = [sim.shards[r].query() for r in range(nd)]
    assert all(q["norm"] == 1.0 for q in qs) and len({q["clip"] for q in qs}) == 1
    sim.compare()


def test_others_norm_mode_on_exact_sums():
    """The older per-rank form (zero_grad_norm with the other ranks' sum) on gradients
    whose squares and sums are exact in fp64 in any order (multiples of 2^-8 up to 1/4,
    unscaled by 2^-10), so it must agree with the oracle's rank-order global sum bit for
    bit; clipping active."""
    w = recipes.tiny()
    psi, nd = 200_003, 4
    master, p16 = master_of(w, psi)
    sim = Sim([psi], nd, F16, p16, master, "reduce")
    sim.norm_mode = "others"
    sim.p16_initial = p16.copy()
    r = np.random.default_rng(5)
    for step in (1, 2):
        g = [oracle.encode16(F16, (r.integers(-64, 65, size=psi) * 2.0 ** -8).astype(np.float32))
             for _ in range(nd)]
        res = sim.step(g, 1.0 / 1024, 1e-3, hp_of(w.hp))
        assert not any(x["skipped"] for x in res) and res[0]["clip"] < 1.0
        sim.compare()


# --------------------------------------------------------------------------
# argument checks that need a handle (and so a device)


def test_reduce_rejects_a_fan_in_other_than_the_ranks():
    from zero_partitioned_mixed_reduce_amd import ZeroError
    from zero_partitioned_mixed_reduce_amd._abi import ZERO_EINVAL
    from zero_partitioned_mixed_reduce_amd.shard import ZeroShard
    from zero_partitioned_mixed_reduce_amd import _abi
    w = recipes.tiny()
    psi, nd = 8192, 4
    _, p16 = master_of(w, psi)
    g = [dev16(x) for x in grads_for(w, 1, psi, nd)]
    s = ZeroShard([psi], nd, 1, F16, dev16(p16), with_red=True)
    for bad in (g[:3], g[:2], g + g[:1]):                         # N_d - 1, 2, N_d + 1 buffers
        with pytest.raises(ZeroError) as e:
            s.zero_reduce_grads(bad, 1.0)
        assert e.value.status == ZERO_EINVAL and "dp_size" in str(e.value)
        with pytest.raises(ZeroError) as e:
            s.zero_accumulate_grads(bad)
        assert e.value.status == ZERO_EINVAL
    arr = (ctypes.c_void_p * nd)(*[x.data_ptr() for x in g])
    for n in (-2, -5, 65):
        assert _abi.lib().zero_reduce_grads(s.h, arr, n, 1.0, None) == ZERO_EINVAL
        assert _abi.lib().zero_accumulate_grads(s.h, arr, n, None) == ZERO_EINVAL
    with pytest.raises(ZeroError) as e:
        s.zero_grad_norm_global(-1.0, 1.0)                        # outside a step: order first
    s.zero_reduce_grads(g, 1.0)                                   # N_d buffers: accepted
    s.zero_check_overflow(False)
    for bad in (-1.0, -float("inf")):
        with pytest.raises(ZeroError) as e:
            s.zero_grad_norm_global(bad, 1.0)
        assert e.value.status == ZERO_EINVAL
    s.zero_grad_norm_global(0.0, 1.0)
    s.zero_adam_step(1e-3, 0.9, 0.999, 1e-8, 0.0)
    torch.cuda.synchronize()
    assert s.query()["t"] == 1
    s.close()


# --------------------------------------------------------------------------
# the dynamic loss scale never grows to infinity


def test_dynamic_loss_scale_growth_stops_below_infinity():
    """From 2^126 with growth 2 every good step: 2^127, then the growth would overflow and
    the scale stays at 2^127 (torch's rule); an overflow backs it off to 2^126; state and
    scale checked against the oracle each step."""
    w = recipes.tiny()
    psi, nd = 50_001, 2
    master, p16 = master_of(w, psi)
    sim = Sim([psi], nd, BF16, p16, master, "flat")
    sim.p16_initial = p16.copy()
    sim.enable_dynamic(init_scale=2.0 ** 126, growth=2.0, backoff=0.5, interval=1, min_scale=1.0)
    expect = {1: 2.0 ** 127, 2: 2.0 ** 127, 3: 2.0 ** 127, 4: 2.0 ** 126, 5: 2.0 ** 127}
    for step in range(1, 6):
        g = synth.normal_16(psi, BF16, w.seed, synth.stream_id(synth.GRAD, 0, step), 0, 1e30)
        if step == 4:
            _poison(g, psi // 2, BF16)
        res = sim.step([g], None, w.max_norm, hp_of(w.hp))
        assert all(x["skipped"] == (step == 4) for x in res)
        assert sim.scaler.scale.value == expect[step], step
        sim.compare()


# --------------------------------------------------------------------------
# seeded random small configurations, every rank against the oracle


@pytest.mark.parametrize("seed", range(16))
def test_random_small_configurations(seed):
    """A seeded random configuration per case: a tensor list of 1-11 tensors (sizes 0-40000,
    some empty), N_d 1-7, shard alignment 8, 64 or 256, fp16 or bf16, the gradient as N_d rank
    buffers, one flat buffer, per-tensor registered or flat registered, parameters flat or
    per tensor at element misalignments, a given or upcast master; three steps with a
    non-finite value injected at a random step and place (or none), clipping off, loose or
    active, the cast fused or standalone.  Every rank's state and 16-bit slice must match the
    oracle bit for bit, and nothing outside each rank's slice may change."""
    r = np.random.default_rng(0x5EED1000 + seed)
    T = int(r.integers(1, 12))
    numel = [int(x) if r.random() > 0.1 else 0 for x in r.integers(1, 40001, size=T)]
    if sum(numel) == 0:
        numel[0] = 12345
    psi = sum(numel)
    nd = int(r.integers(1, 8))
    align = int(r.choice([8, 64, 256]))
    dtype = int(r.choice([F16, BF16]))
    mode = str(r.choice(["reduce", "flat", "ragged", "registered_flat"]))
    per_tensor = bool(r.random() < 0.5)
    pmis = tuple(int(x) for x in r.integers(0, 8, size=3))
    gmis = tuple(int(x) for x in r.integers(0, 8, size=2))
    master_given = bool(r.random() < 0.7)
    fuse = bool(r.random() < 0.5)
    max_norm = float(r.choice([0.0, 1.0, 1e-3]))
    hp = oracle.HParams(float(r.choice([1e-4, 1e-3, 1e-2])), 0.9, 0.999, 1e-8, float(r.choice([0.0, 0.01, 0.1])))
    seed_w = 0x5EED2000 + seed
    print(f"[random {seed}] T {T} psi {psi} N_d {nd} align {align} dtype {dtype} mode {mode} "
          f"per_tensor {per_tensor} master {master_given} fuse {fuse} max_norm {max_norm}", flush=True)
    master = synth.normal_f32(psi, seed_w, synth.stream_id(synth.MASTER), 0, 0.02)
    p16 = oracle.encode16(dtype, master) if master_given else \
        synth.normal_16(psi, dtype, seed_w, synth.stream_id(synth.MASTER), 0, 0.02)
    sim = Sim(numel, nd, dtype, p16, master if master_given else None, mode, per_tensor_params=per_tensor,
              param_misalign=pmis, grad_misalign=gmis, align=align)
    sim.p16_initial = p16.copy()
    scale = 1024.0 if dtype == F16 else 1.0
    bad_step = int(r.integers(1, 5))              # 4: no injection
    bad_val = float(r.choice([np.inf, -np.inf, np.nan]))
    nbuf = nd if mode == "reduce" else 1
    for step in range(1, 4):
        g = [synth.normal_16(psi, dtype, seed_w, synth.stream_id(synth.GRAD, q, step), 0, 1e-3 * scale * 30)
             for q in range(nbuf)]
        if step == bad_step:
            g[int(r.integers(0, nbuf))][int(r.integers(0, psi))] = oracle.encode16(
                dtype, np.array([bad_val], np.float32))[0]
        res = sim.step(g, 1.0 / scale, max_norm, hp, fuse=fuse)
        assert all(x["skipped"] == (step == bad_step) for x in res)
        sim.compare()


@pytest.mark.parametrize("seed", range(12))
def test_random_configurations_with_the_next_rows(seed):
    """Seeded random configurations that combine the step's extensions: 1-3 micro-steps
    (the last one fused into the intake or accumulated and taken with ZERO_ACCUMULATED), the
    device-resident dynamic loss scale, the 16-bit output of the local reduce and a tracked
    segmented write-back, over random tensor lists, N_d, dtypes, gradient modes and layouts;
    three steps with a non-finite value injected into a random micro-step of a random step (or
    none).  Every rank's state, 16-bit slice and loss scale must match the oracle bit for bit."""
    r = np.random.default_rng(0x5EED3000 + seed)
    T = int(r.integers(1, 9))
    numel = [int(x) for x in r.integers(1, 30001, size=T)]
    psi = sum(numel)
    nd = int(r.integers(1, 6))
    dtype = int(r.choice([F16, BF16]))
    mode = str(r.choice(["reduce", "flat", "ragged", "registered_flat"]))
    K = int(r.integers(1, 4))
    last_fused = bool(r.random() < 0.5)
    out16 = mode == "reduce" and nd >= 2 and bool(r.random() < 0.5)
    dynamic = bool(r.random() < 0.6)
    segments = int(r.choice([0, 3, 17]))
    fuse = bool(r.random() < 0.6)
    per_tensor = bool(r.random() < 0.5)
    max_norm = float(r.choice([0.0, 1.0, 1e-3]))
    hp = oracle.HParams(1e-3, 0.9, 0.999, 1e-8, float(r.choice([0.0, 0.01])))
    seed_w = 0x5EED4000 + seed
    print(f"[random-next {seed}] T {T} psi {psi} N_d {nd} dtype {dtype} mode {mode} K {K} last_fused {last_fused} "
          f"out16 {out16} dynamic {dynamic} segments {segments} fuse {fuse} per_tensor {per_tensor}", flush=True)
    master = synth.normal_f32(psi, seed_w, synth.stream_id(synth.MASTER), 0, 0.02)
    p16 = oracle.encode16(dtype, master)
    sim = Sim(numel, nd, dtype, p16, master, mode, per_tensor_params=per_tensor, param_misalign=(0, 3),
              grad_misalign=(1,), with_red=True, segments=segments)
    sim.p16_initial = p16.copy()
    if out16:
        sim.set_reduce_out16(True)
    scale = 1024.0 if dtype == F16 else 1.0
    if dynamic:
        sim.enable_dynamic(init_scale=float(2.0 ** int(r.integers(4, 12))), growth=2.0, backoff=0.5,
                           interval=int(r.integers(1, 3)), min_scale=1.0)
    bad_step = int(r.integers(1, 5))
    bad_micro = int(r.integers(0, K))
    nbuf = nd if mode == "reduce" else 1
    for step in range(1, 4):
        micro = [[synth.normal_16(psi, dtype, seed_w, synth.stream_id(synth.GRAD, q, 100 * step + k), 0, 30e-3 * scale)
                  for q in range(nbuf)] for k in range(K)]
        if step == bad_step:
            micro[bad_micro][int(r.integers(0, nbuf))][int(r.integers(0, psi))] = oracle.encode16(
                dtype, np.array([np.inf], np.float32))[0]
        inv = None if dynamic else 1.0 / scale
        if K == 1:
            res = sim.step(micro[0], inv, max_norm, hp, fuse=fuse)
        else:
            res = sim.step_accumulated(micro, inv, max_norm, hp, fuse=fuse, last_fused=last_fused)
        assert all(x["skipped"] == (step == bad_step) for x in res)
        sim.compare()
