"""The offloaded (host) step with its device copies on the MI355X, against the
oracle element by element: the gradient slice fetched from device memory
(registered per-tensor views at odd element offsets, a registered flat buffer,
or a flat buffer passed at fetch time), the host update, and the updated
16-bit slice pushed back into the device parameters block by block while the
update runs.  Nothing outside each rank's slice of the device parameters may
change.  Host state and 16-bit values are expected bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import recipes
from tests.gpu_harness import Layout, dev16, host16
from zero_partitioned_mixed_reduce_amd.offload import ZeroOffload

pytestmark = pytest.mark.gpu
F16, BF16 = oracle.F16, oracle.BF16


@pytest.fixture(autouse=True)
def _gpu(need_gpu):
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def hp_of(d):
    return oracle.HParams(d["lr"], d["beta1"], d["beta2"], d["eps"], d["weight_decay"])


def sumsq_tol(n):
    """Relative bound on the difference between two fp64 sums of the same n non-negative
    terms added in different orders: each is within (n - 1) * 2^-53 of the exact sum."""
    return max(2.0 * n * 2.0 ** -53, 1e-15)


class OffloadSim:
    """Every rank's offload handle with its own copy of the device parameters."""

    def __init__(self, numel, nd, dtype, p16_full, master_full, grad_mode, per_tensor, misalign=(0,),
                 device_stats=True):
        self.numel, self.nd, self.dtype, self.grad_mode = list(numel), nd, dtype, grad_mode
        self.psi = sum(numel)
        self.p16_initial = p16_full.copy()
        self.plans = [oracle.plan(numel, nd, r) for r in range(nd)]
        self.ostates, self.handles, self.params = [], [], []
        self.player = Layout(numel, per_tensor, misalign)
        self.glayout = Layout(numel, grad_mode == "ragged", misalign[::-1])
        self.gstore, self.gviews = None, None
        if grad_mode in ("ragged", "registered_flat"):
            self.gstore, self.gviews = self.glayout.make(np.zeros(self.psi, np.uint16))
        for r in range(nd):
            _, _, b, valid = self.plans[r]
            mst = None if master_full is None else master_full[b:b + valid]
            self.ostates.append(oracle.RankState(dtype, p16_full[b:b + valid], mst))
            store, views = self.player.make(p16_full)
            self.params.append((store, views))
            grads = {"ragged": self.gviews, "registered_flat": self.gstore}.get(grad_mode)
            self.handles.append(ZeroOffload(numel, nd, r, dtype, params=views if views is not None else store,
                                            grads=grads, master_init=mst, num_threads=(0, 3, 5)[r % 3],
                                            device_stats=device_stats))
        torch.cuda.synchronize()

    def step(self, g_full, inv, max_norm, hp, fused_push=True):
        res = oracle.step_ranks(self.ostates, [g_full], [p[2] for p in self.plans], inv, max_norm, hp)
        src = dev16(g_full)
        if self.gviews is not None:
            start = 0
            for v, n in zip(self.gviews, self.numel):
                v.copy_(src[start:start + n])
                start += n
        elif self.gstore is not None:
            self.gstore.copy_(src)
        loc = []
        for h in self.handles:
            h.zero_offload_fetch_grads(inv, src if self.grad_mode == "flat" else None)
            loc.append(h.zero_offload_grad_stats(inv))
        glob = 0.0
        for x in loc:
            glob = glob + x[1]                  # the ranks' local sums, once, in rank order
        for r, h in enumerate(self.handles):
            other_flag = any(loc[q][0] for q in range(self.nd) if q != r)
            h.zero_offload_adam_step_global(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, other_flag, glob,
                                            max_norm, push=fused_push)
            if not fused_push:
                h.zero_offload_push_params()
            q = h.query()
            valid = self.plans[r][3]
            assert loc[r][0] == res[r]["flag"] and q["skipped"] == res[r]["skipped"], (r, loc[r], q, res[r])
            if np.isfinite(res[r]["local_sumsq"]):
                # host statistics: two fp64 orders of the same terms; device statistics: within the
                # device step's bound
                tol = sumsq_tol(valid) if h.workspace is None else 1e-9
                assert abs(loc[r][1] - res[r]["local_sumsq"]) <= tol * max(res[r]["local_sumsq"], 1e-300)
            if not q["skipped"]:
                assert q["clip"] == res[r]["clip"]
            assert q["t"] == self.ostates[r].counters.t
        torch.cuda.synchronize()
        return res

    def compare(self):
        for r, (h, o) in enumerate(zip(self.handles, self.ostates)):
            _, _, b, valid = self.plans[r]
            for name, exp in (("master", o.w), ("m", o.m), ("v", o.v)):
                assert (h.host(name).view(np.uint32) == exp.view(np.uint32)).all(), f"rank {r} {name}"
            assert (h.host16("param16") == o.p16).all(), f"rank {r} host param16"
            store, views = self.params[r]
            flat = Layout.flat_of(views if views is not None else store)
            assert (flat[b:b + valid] == o.p16).all(), f"rank {r} device parameters"
            assert (flat[:b] == self.p16_initial[:b]).all() and \
                (flat[b + valid:] == self.p16_initial[b + valid:]).all(), f"rank {r} wrote outside its slice"

    def close(self):
        for h in self.handles:
            h.close()


@pytest.mark.parametrize("grad_mode,per_tensor,master_given,fused_push,device_stats", [
    ("ragged", True, True, True, True),
    ("ragged", True, False, False, True),
    ("registered_flat", False, True, True, True),
    ("flat", False, False, True, True),
    ("flat", True, True, False, True),
    ("ragged", True, True, True, False),
    ("flat", False, False, False, False),
])
def test_offload_device_copies_match_oracle(grad_mode, per_tensor, master_given, fused_push, device_stats):
    """The ragged mini list (4 layers, d 256, MLP 688, vocab 2000) at N_d = 3, bf16, 4 steps
    with an inf in step 2; tensors sit at odd element offsets in device memory.  With device
    statistics the host update consumes the gradient blocks as they land; without, the host
    computes the statistics first."""
    w = recipes.ragged_mini(3)
    psi = w.psi
    master = synth.normal_f32(psi, w.seed, synth.stream_id(synth.MASTER), 0, w.master_sigma)
    p16 = synth.normal_16(psi, w.dtype, w.seed, synth.stream_id(synth.MASTER), 0, w.master_sigma)
    sim = OffloadSim(w.numel, w.nd, w.dtype, p16, master if master_given else None, grad_mode, per_tensor,
                     misalign=(0, 1, 3, 6), device_stats=device_stats)
    if not master_given:
        for h, o in zip(sim.handles, sim.ostates):
            assert (h.host("master").view(np.uint32) == o.w.view(np.uint32)).all()
    hp = hp_of(w.hp)
    for step in range(1, 5):
        g = synth.normal_16(psi, w.dtype, w.seed, synth.stream_id(synth.GRAD, 0, step), 0, w.grad_sigma)
        if step == 2:
            g[psi - 5] = 0x7F80
        res = sim.step(g, 1.0, w.max_norm, hp, fused_push)
        assert all(x["skipped"] == (step == 2) for x in res)
        sim.compare()
    sim.close()


@pytest.mark.parametrize("device_stats", [True, False])
def test_offload_fp16_loss_scale_many_blocks(device_stats):
    """fp16 with loss scale 1024 over several copy blocks (4M elements each) and a
    ragged tail, one rank of N_d = 2; the gradient slice is fetched from a flat buffer."""
    n, nd, dtype, seed = (1 << 22) * 2 + 12345, 2, F16, 0x5EED0700
    psi = n * nd - 100
    master = synth.normal_f32(psi, seed, synth.stream_id(synth.MASTER), 0, 0.02)
    p16 = synth.normal_16(psi, dtype, seed, synth.stream_id(synth.MASTER), 0, 0.02)
    sim = OffloadSim([psi], nd, dtype, p16, master, "flat", False, device_stats=device_stats)
    hp = oracle.HParams(1e-3, 0.9, 0.999, 1e-8, 0.01)
    for step in (1, 2):
        g = synth.normal_16(psi, dtype, seed, synth.stream_id(synth.GRAD, 0, step), 0, 1e-3 * 1024)
        sim.step(g, 1.0 / 1024, 1.0, hp)
        sim.compare()
    sim.close()


def test_offload_gpt2_shard_full_size():
    """The GPT-2 1.5B-shaped list at N_d = 8, rank 7 (the padded last shard), as the
    benchmark runs it: flat bf16 parameters and a registered flat gradient on the device,
    two applied steps, every element of the 194M-element shard compared."""
    w = recipes.gpt2_shard()
    r = 7
    psi, S, b, valid = oracle.plan(w.numel, w.nd, r)
    mstream = synth.stream_id(synth.MASTER)
    params = torch.empty(psi, dtype=torch.int16, device="cuda")
    synth.gpu_normal_16(params, w.dtype, w.seed, mstream, first=0, sigma=w.master_sigma)
    grads = torch.empty(psi, dtype=torch.int16, device="cuda")
    master = synth.normal_f32(valid, w.seed, mstream, b, w.master_sigma)
    st = oracle.RankState(w.dtype, synth.normal_16(valid, w.dtype, w.seed, mstream, b, w.master_sigma), master)
    h = ZeroOffload(w.numel, w.nd, r, w.dtype, params=params, grads=grads, master_init=master)
    hp = hp_of(w.hp)
    other = float(psi - valid) * w.grad_sigma * w.grad_sigma
    for step in (1, 2):
        gstream = synth.stream_id(synth.GRAD, 0, step)
        synth.gpu_normal_16(grads, w.dtype, w.seed, gstream, first=0, sigma=w.grad_sigma)
        torch.cuda.synchronize()
        h.zero_offload_fetch_grads(1.0)
        flag, ss = h.zero_offload_grad_stats(1.0)
        g = synth.normal_16(valid, w.dtype, w.seed, gstream, b, w.grad_sigma)
        u, oflag, oss = oracle.grad_stats(w.dtype, [g], 1.0)
        assert flag == oflag is False and abs(ss - oss) <= 1e-9 * oss    # the device's statistics
        h.zero_offload_adam_step(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, False, other, w.max_norm,
                                 push=True)
        clip, _ = oracle.clip_coef(oss + other, w.max_norm)
        assert h.query()["clip"] == clip
        oracle.adam(False, u, clip, hp, st.counters, st.w, st.m, st.v)
        oracle.cast(w.dtype, st.w, st.p16)
        torch.cuda.synchronize()
        for name, exp in (("master", st.w), ("m", st.m), ("v", st.v)):
            assert (h.host(name).view(np.uint32) == exp.view(np.uint32)).all(), name
        dev = host16(params)
        assert (dev[b:b + valid] == st.p16).all()
    h.close()


def test_offload_destroy_mid_step():
    """Handles destroyed with work still pending -- a gradient fetch in flight with its
    device statistics unread, or statistics read but no update -- release their events
    and streams cleanly, many times over, and a new handle then steps normally."""
    w = recipes.ragged_mini(2)
    psi = w.psi
    p16 = synth.normal_16(psi, w.dtype, w.seed, synth.stream_id(synth.MASTER), 0, w.master_sigma)
    params = dev16(p16)
    g = dev16(synth.normal_16(psi, w.dtype, w.seed, synth.stream_id(synth.GRAD, 0, 1), 0, w.grad_sigma))
    for k in range(40):
        h = ZeroOffload(w.numel, 2, k % 2, w.dtype, params=params, num_threads=2)
        h.zero_offload_fetch_grads(1.0, g)
        if k % 3 == 1:
            h.zero_offload_grad_stats(1.0)
        h.close()
    sim = OffloadSim(w.numel, 2, w.dtype, p16, None, "flat", False)
    hp = hp_of(w.hp)
    sim.step(synth.normal_16(psi, w.dtype, w.seed, synth.stream_id(synth.GRAD, 0, 1), 0, w.grad_sigma), 1.0,
             w.max_norm, hp)
    sim.compare()
    sim.close()
