"""zero_shard_init_static (the handle's workspace in the library's static device array,
for callers that cannot allocate device memory) against zero_shard_init (a caller
workspace), through the C ABI on one GPU.

Two static initialisations in a row, the second with a smaller shard: each static handle
is stepped next to a handle with its own workspace on the same inputs, and master, m, v,
the 16-bit slice, t, the skip decision, norm and clip must agree bit for bit after every
step (the same kernels run on the same data; the bar of the method's tolerance is met a
fortiori).  The second static initialisation retires the first static handle."""
import numpy as np
import pytest
import torch

import synth
from synth import recipes
from tests.gpu_harness import Layout, dev16, host16
from zero_partitioned_mixed_reduce_amd import ZeroError, _abi
from zero_partitioned_mixed_reduce_amd.shard import ZeroShard

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu(need_gpu):
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def same_state(a, b, params_a, params_b, what):
    for name in ("master", "m", "v"):
        ea, eb = a.export(name).cpu().numpy(), b.export(name).cpu().numpy()
        assert (ea.view(np.uint32) == eb.view(np.uint32)).all(), f"{what}: {name}"
    pa = Layout.flat_of(params_a)
    pb = Layout.flat_of(params_b)
    assert (pa == pb).all(), f"{what}: 16-bit parameters"
    qa, qb = a.query(), b.query()
    assert qa == qb, (what, qa, qb)
    return qa


def step_both(handles, srcs, inv, other_sumsq, max_norm, hp):
    for h in handles:
        h.zero_reduce_grads(srcs, inv)
        h.zero_check_overflow(False)
        h.zero_grad_norm(other_sumsq, max_norm)
        h.zero_adam_step(*hp, fuse_cast=True)


def test_static_workspace_matches_caller_workspace_twice():
    hp = (1e-3, 0.9, 0.999, 1e-8, 0.01)
    w = recipes.tiny()

    # call 1: flat fp16, N_d = 2, rank 1, the local reduce of 2 rank buffers, loss scale 1024
    psi, nd, rank = 3_000_017, 2, 1
    print(f"[no-alloc] call 1: flat fp16 psi {psi} N_d {nd} rank {rank}", flush=True)
    p16 = synth.normal_16(psi, w.dtype, w.seed, synth.stream_id(synth.MASTER), 0, w.master_sigma)
    pa, pb = dev16(p16), dev16(p16)
    a = ZeroShard([psi], nd, rank, w.dtype, pa, with_red=True)
    s1 = ZeroShard([psi], nd, rank, w.dtype, pb, with_red=True, static_workspace=True)
    assert s1.workspace is None and s1.bufs.workspace is None
    assert a.info.workspace_bytes <= _abi.ZERO_STATIC_WORKSPACE_BYTES
    for step in range(1, 4):
        g = [synth.normal_16(psi, w.dtype, w.seed, synth.stream_id(synth.GRAD, q, step), 0, w.grad_sigma * 1024)
             for q in range(nd)]
        if step == 2:
            g[0][psi - 5] = 0x7C00                                     # +inf in this rank's slice: skip
        step_both((a, s1), [dev16(x) for x in g], 1.0 / 1024, 1.0, 0.5, hp)
        q = same_state(a, s1, pa, pb, f"call 1 step {step}")
        assert q["skipped"] == (step == 2) and q["t"] == (step if step < 2 else step - 1)
    a.close()

    # call 2: a smaller shard -- the ragged per-tensor list, bf16, N_d = 7, rank 3, one
    # already-reduced flat gradient, clipping active
    m = recipes.ragged_mini(7)
    nd, rank = 7, 3
    numel = m.numel
    psi = sum(numel)
    print(f"[no-alloc] call 2: ragged bf16 psi {psi} N_d {nd} rank {rank}", flush=True)
    p16 = synth.normal_16(psi, m.dtype, m.seed, synth.stream_id(synth.MASTER), 0, m.master_sigma)
    lay = Layout(numel, True, (0, 1, 3))
    sa, va = lay.make(p16)
    sb, vb = lay.make(p16)
    b = ZeroShard(numel, nd, rank, m.dtype, va)
    s2 = ZeroShard(numel, nd, rank, m.dtype, vb, static_workspace=True)
    assert s2.info.valid_elems < s1.info.valid_elems
    # the first static handle's workspace now belongs to s2
    with pytest.raises(ZeroError) as e:
        s1.zero_reduce_grads([dev16(g[0]), dev16(g[1])], 1.0)
    assert e.value.status == _abi.ZERO_ESTATE and "taken over" in str(e.value)
    with pytest.raises(ZeroError):
        s1.query()
    s1.close()
    for step in range(1, 4):
        g = synth.normal_16(psi, m.dtype, m.seed, synth.stream_id(synth.GRAD, 0, step), 0, m.grad_sigma * 50)
        step_both((b, s2), [dev16(g)], 1.0, 0.0, m.max_norm, hp)
        q = same_state(b, s2, va, vb, f"call 2 step {step}")
        assert not q["skipped"] and q["t"] == step and q["clip"] < 1.0
    b.close()
    s2.close()


def test_static_workspace_at_its_largest_shard():
    """The largest flat shard whose workspace fits the static array (about 8.2e8 elements at
    N_d = 1, so its 16-bit slice is larger than the Infinity Cache and the statistics pass
    leaves a cached tail for an Adam pass that walks from the end): two steps on the static
    handle and on a caller-workspace handle, compared bit for bit on the device."""
    from zero_partitioned_mixed_reduce_amd.shard import make_desc
    probe = torch.empty(1, dtype=torch.int16, device="cuda")
    lo, hi = 1 << 20, 1 << 31                                  # the plan's workspace grows with psi
    while hi - lo > 8192:
        mid = (lo + hi) // 2
        fits = _abi.zero_shard_plan(make_desc([mid], 1, 0, _abi.ZERO_BF16, probe)).workspace_bytes
        lo, hi = (mid, hi) if fits <= _abi.ZERO_STATIC_WORKSPACE_BYTES else (lo, mid)
    psi = lo
    w = recipes.tiny()
    print(f"[no-alloc] largest static shard: flat bf16 psi {psi} N_d 1", flush=True)
    p16 = torch.empty(psi, dtype=torch.int16, device="cuda")
    synth.gpu_normal_16(p16, _abi.ZERO_BF16, w.seed, synth.stream_id(synth.MASTER), 0, w.master_sigma)
    pa, pb = p16.clone(), p16
    a = ZeroShard([psi], 1, 0, _abi.ZERO_BF16, pa)
    s = ZeroShard([psi], 1, 0, _abi.ZERO_BF16, pb, static_workspace=True)
    assert a.info.workspace_bytes <= _abi.ZERO_STATIC_WORKSPACE_BYTES and 2 * psi > 256 << 20
    g = torch.empty(psi, dtype=torch.int16, device="cuda")
    hp = (1e-3, 0.9, 0.999, 1e-8, 0.01)
    for step in range(1, 3):
        synth.gpu_normal_16(g, _abi.ZERO_BF16, w.seed, synth.stream_id(synth.GRAD, 0, step), 0, 1e-4)
        step_both((a, s), [g], 1.0, 0.0, 1.0, hp)
        for name in ("master", "m", "v"):
            assert torch.equal(a.export(name).view(torch.int32), s.export(name).view(torch.int32)), (step, name)
        assert torch.equal(pa, pb), (step, "16-bit parameters")
        qa, qs = a.query(), s.query()
        assert qa == qs and not qa["skipped"] and qa["t"] == step and qa["clip"] < 1.0, (qa, qs)
    a.close()
    s.close()


def test_static_workspace_size_limit():
    """A shard whose workspace exceeds the static array is refused before any device work
    (and a caller workspace passed to the static call is refused too)."""
    big = [2_000_000_000]
    flat = torch.empty(1, dtype=torch.int16, device="cuda")
    from zero_partitioned_mixed_reduce_amd.shard import make_desc
    d = make_desc(big, 1, 0, _abi.ZERO_BF16, flat)
    info = _abi.zero_shard_plan(d)
    assert info.workspace_bytes > _abi.ZERO_STATIC_WORKSPACE_BYTES
    bufs = _abi.zero_shard_bufs_t()
    bufs.master = bufs.m = bufs.v = 1 << 20                       # never dereferenced: refused first
    bufs.state_capacity = info.state_elems
    with pytest.raises(ZeroError) as e:
        _abi.zero_shard_init_static(d, bufs, None, None)
    assert e.value.status == _abi.ZERO_EINVAL and "ZERO_STATIC_WORKSPACE_BYTES" in str(e.value)
    small = make_desc([4096], 1, 0, _abi.ZERO_BF16, flat)
    bufs.workspace = 1 << 21
    with pytest.raises(ZeroError) as e:
        _abi.zero_shard_init_static(small, bufs, None, None)
    assert e.value.status == _abi.ZERO_EINVAL and "NULL" in str(e.value)
