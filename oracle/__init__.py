"""Oracle for one data-parallel rank's partitioned mixed-precision optimizer step.

TEST INFRASTRUCTURE ONLY: the plain, slow CPU statement of what the step
computes.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import it; the product path never does.  It shares no code with the HIP
library.  The arithmetic lives in zero_oracle.c (see its header for the
passages it follows); this module is its ctypes binding plus the multi-rank
driver that simulates the exchange of flags and norms between ranks.

Parity status: every function here is pinned by tests/test_oracle_pins.py.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F16, BF16 = 1, 2
_lib = None


class HParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float)]


class Counters(ctypes.Structure):
    _fields_ = [("t", ctypes.c_int64), ("p1", ctypes.c_double), ("p2", ctypes.c_double)]

    @classmethod
    def fresh(cls):
        return cls(0, 1.0, 1.0)

    def copy(self):
        return Counters(self.t, self.p1, self.p2)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        i64p = ctypes.POINTER(ctypes.c_int64)
        L.orc_plan.argtypes = [i64p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                               i64p, i64p, i64p, i64p]
        L.orc_plan.restype = ctypes.c_int
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f32.restype = ctypes.c_float
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_grad_stats.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_int64,
                                     ctypes.c_float, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)]
        L.orc_grad_stats.restype = ctypes.c_int
        L.orc_accumulate.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_int64,
                                     ctypes.c_void_p, ctypes.c_int]
        L.orc_reduce_to16.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_int64,
                                      ctypes.c_void_p]
        L.orc_stats_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                                    ctypes.POINTER(ctypes.c_double)]
        L.orc_stats_f32.restype = ctypes.c_int
        L.orc_loss_scale_update.argtypes = [ctypes.c_int, ctypes.c_float, ctypes.c_float, ctypes.c_int, ctypes.c_float,
                                            ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int)]
        L.orc_inv_scale.argtypes = [ctypes.c_float]
        L.orc_inv_scale.restype = ctypes.c_float
        L.orc_clip_coef.argtypes = [ctypes.c_double, ctypes.c_float, ctypes.POINTER(ctypes.c_double)]
        L.orc_clip_coef.restype = ctypes.c_float
        L.orc_next_scalars.argtypes = [ctypes.POINTER(HParams), ctypes.POINTER(Counters),
                                       ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float)]
        L.orc_adam.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                               ctypes.POINTER(HParams), ctypes.POINTER(Counters),
                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.orc_adam_elems.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.POINTER(HParams),
                                     ctypes.c_float, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]
        for name in ("orc_cast", "orc_encode_many"):
            getattr(L, name).argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        for name in ("orc_upcast", "orc_decode_many"):
            getattr(L, name).argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        _lib = L
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def _f32(a):
    a = np.asarray(a)
    assert a.dtype == np.float32 and a.flags.c_contiguous
    return a


def _u16(a):
    a = np.asarray(a)
    assert a.dtype == np.uint16 and a.flags.c_contiguous
    return a


def plan(numel, nd, rank, align=64):
    """(psi, S, begin, valid) of `rank` for the flattened tensor list `numel`."""
    arr = np.ascontiguousarray(np.asarray(numel, dtype=np.int64))
    out = [ctypes.c_int64() for _ in range(4)]
    rc = lib().orc_plan(arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(arr), nd, rank, align,
                        *[ctypes.byref(o) for o in out])
    if rc != 0:
        raise ValueError("bad partition arguments")
    return tuple(o.value for o in out)


def shard_pieces(numel, begin, valid):
    """Intersections of the shard [begin, begin+valid) with each tensor of the
    flattened list: (tensor, tensor_offset, shard_offset, length) in order."""
    out, start = [], 0
    end = begin + valid
    for k, n in enumerate(numel):
        lo, hi = max(start, begin), min(start + n, end)
        if lo < hi:
            out.append((k, lo - start, lo - begin, hi - lo))
        start += n
    return out


def decode16(dtype, h):
    h = _u16(np.ascontiguousarray(h))
    out = np.empty(h.shape, np.float32)
    lib().orc_decode_many(dtype, _ptr(h), h.size, _ptr(out))
    return out


def encode16(dtype, x):
    x = _f32(np.ascontiguousarray(x, dtype=np.float32))
    out = np.empty(x.shape, np.uint16)
    lib().orc_encode_many(dtype, _ptr(x), x.size, _ptr(out))
    return out


def grad_stats(dtype, srcs, inv_loss_scale, sumsq_acc=0.0):
    """Reduce (rank order, fp32) + unscale + non-finite flag + fp64 sum of squares.
    srcs: list of uint16 arrays of equal length (one = already reduced).
    Returns (u, flag, sumsq) where sumsq continues from sumsq_acc."""
    srcs = [_u16(np.ascontiguousarray(s)) for s in srcs]
    n = srcs[0].size
    assert all(s.size == n for s in srcs)
    arr = (ctypes.c_void_p * len(srcs))(*[s.ctypes.data for s in srcs])
    u = np.empty(n, np.float32)
    acc = ctypes.c_double(sumsq_acc)
    flag = lib().orc_grad_stats(dtype, arr, len(srcs), n, ctypes.c_float(inv_loss_scale), _ptr(u),
                                ctypes.byref(acc))
    return u, bool(flag), acc.value


def reduce_to16(dtype, srcs):
    """16-bit output of the local reduce: RNE16 of the rank-order fp32 sum of srcs."""
    srcs = [_u16(np.ascontiguousarray(x)) for x in srcs]
    n = srcs[0].size
    assert all(x.size == n for x in srcs)
    arr = (ctypes.c_void_p * len(srcs))(*[x.ctypes.data for x in srcs])
    out = np.empty(n, np.uint16)
    lib().orc_reduce_to16(dtype, arr, len(srcs), n, _ptr(out))
    return out


def _intake_sources(dtype, srcs, reduce_out16):
    """The sources as the step takes them in: with a 16-bit reduce output, N_d >= 2
    rank buffers become the one 16-bit reduce-scatter result."""
    if reduce_out16 and len(srcs) >= 2:
        return [reduce_to16(dtype, srcs)]
    return srcs


def accumulate(dtype, srcs, acc, first):
    """acc (float32, in place) = s or acc + s, with s the rank-order fp32 sum of srcs."""
    srcs = [_u16(np.ascontiguousarray(x)) for x in srcs]
    acc = _f32(acc)
    assert all(x.size == acc.size for x in srcs)
    arr = (ctypes.c_void_p * len(srcs))(*[x.ctypes.data for x in srcs])
    lib().orc_accumulate(dtype, arr, len(srcs), acc.size, _ptr(acc), int(bool(first)))


def stats_f32(acc, inv_loss_scale, sumsq_acc=0.0):
    """(u, flag, sumsq) of an accumulated fp32 gradient."""
    acc = _f32(np.ascontiguousarray(acc, dtype=np.float32))
    u = np.empty(acc.size, np.float32)
    ss = ctypes.c_double(sumsq_acc)
    flag = lib().orc_stats_f32(_ptr(acc), acc.size, ctypes.c_float(inv_loss_scale), _ptr(u), ctypes.byref(ss))
    return u, bool(flag), ss.value


def clip_coef(global_sumsq, max_norm):
    norm = ctypes.c_double()
    c = lib().orc_clip_coef(global_sumsq, ctypes.c_float(max_norm), ctypes.byref(norm))
    return np.float32(c), norm.value


def next_scalars(hp, counters):
    b1, b2 = ctypes.c_float(), ctypes.c_float()
    lib().orc_next_scalars(ctypes.byref(hp), ctypes.byref(counters), ctypes.byref(b1), ctypes.byref(b2))
    return np.float32(b1.value), np.float32(b2.value)


def adam(skip, u, clip, hp, counters, w, m, v):
    """In place on w, m, v (float32 arrays) and counters."""
    u, w, m, v = _f32(u), _f32(w), _f32(m), _f32(v)
    assert u.size == w.size == m.size == v.size
    lib().orc_adam(int(skip), _ptr(u), u.size, ctypes.c_float(clip), ctypes.byref(hp), ctypes.byref(counters),
                   _ptr(w), _ptr(m), _ptr(v))


def adam_elems(u, clip, hp, bc1, bc2, w, m, v):
    """In place on sampled elements, with the step's bias-correction scalars given."""
    u, w, m, v = _f32(u), _f32(w), _f32(m), _f32(v)
    lib().orc_adam_elems(_ptr(u), u.size, ctypes.c_float(clip), ctypes.byref(hp), ctypes.c_float(bc1),
                         ctypes.c_float(bc2), _ptr(w), _ptr(m), _ptr(v))


def cast(dtype, w, p16):
    w, p16 = _f32(w), _u16(p16)
    assert w.size == p16.size
    lib().orc_cast(dtype, _ptr(w), w.size, _ptr(p16))


def upcast(dtype, p16):
    p16 = _u16(np.ascontiguousarray(p16))
    w = np.empty(p16.size, np.float32)
    lib().orc_upcast(dtype, _ptr(p16), p16.size, _ptr(w))
    return w


class LossScaler:
    """Dynamic loss scale state of the oracle (see orc_loss_scale_update)."""

    def __init__(self, init_scale=65536.0, growth=2.0, backoff=0.5, interval=1000, min_scale=1.0):
        self.scale = ctypes.c_float(init_scale)
        self.good = ctypes.c_int(0)
        self.growth, self.backoff, self.interval, self.min_scale = growth, backoff, interval, min_scale

    @property
    def inv(self):
        return float(lib().orc_inv_scale(self.scale))

    def update(self, skipped):
        lib().orc_loss_scale_update(int(bool(skipped)), ctypes.c_float(self.growth), ctypes.c_float(self.backoff),
                                    int(self.interval), ctypes.c_float(self.min_scale), ctypes.byref(self.scale),
                                    ctypes.byref(self.good))


class RankState:
    """One rank's logical shard state: fp32 w, m, v and its 16-bit parameter slice."""

    def __init__(self, dtype, p16_slice, master=None):
        self.dtype = dtype
        self.p16 = np.array(p16_slice, dtype=np.uint16, copy=True)
        self.w = upcast(dtype, self.p16) if master is None else np.array(master, np.float32, copy=True)
        self.m = np.zeros_like(self.w)
        self.v = np.zeros_like(self.w)
        self.counters = Counters.fresh()


def step_ranks_accumulated(states, micro_grads, begins, inv_loss_scale, max_norm, hp, extra_found_inf=False,
                           reduce_out16=False):
    """One optimizer step over K micro-steps: micro_grads[k] is the list of flat
    uint16 buffers of micro-step k (one already-reduced buffer, or one per rank).
    Each rank accumulates its slice over the micro-steps in fp32, then the step
    proceeds as in step_ranks on the accumulated gradient.  reduce_out16: each
    micro-step's reduce delivers its sum in 16 bits, which is what gets accumulated."""
    nd = len(states)
    locs = []
    for r, st in enumerate(states):
        n, b = st.w.size, begins[r]
        acc = np.zeros(n, np.float32)
        for k, grads in enumerate(micro_grads):
            srcs = _intake_sources(st.dtype, [g[b:b + n] for g in grads], reduce_out16)
            accumulate(st.dtype, srcs, acc, first=(k == 0))
        locs.append(stats_f32(acc, inv_loss_scale))
    return _finish_step(states, locs, nd, max_norm, hp, extra_found_inf)


def step_ranks(states, rank_grads, begins, inv_loss_scale, max_norm, hp, extra_found_inf=False,
               reduce_out16=False):
    """One optimizer step of every simulated rank.

    states[r] holds rank r's shard (valid elements from begins[r]).  rank_grads
    is a list of full flat uint16 buffers: one already-reduced buffer, or one per
    rank to be summed.  Each rank computes its local flag and sum of squares;
    the exchange gives every rank the same global flag (the OR of all ranks'
    flags) and the same global sum of squares, the ranks' local sums added in
    rank order (see _finish_step).
    reduce_out16: the reduce of N_d >= 2 buffers delivers its sum in 16 bits
    (reduce_to16), which the step then takes in.
    Returns a list of per-rank dicts (flag, local_sumsq, global_sumsq, norm,
    clip, skipped)."""
    nd = len(states)
    locs = []
    for r, st in enumerate(states):
        n = st.w.size
        b = begins[r]
        srcs = _intake_sources(st.dtype, [g[b:b + n] for g in rank_grads], reduce_out16)
        u, flag, ss = grad_stats(st.dtype, srcs, inv_loss_scale)
        locs.append((u, flag, ss))
    return _finish_step(states, locs, nd, max_norm, hp, extra_found_inf)


def _finish_step(states, locs, nd, max_norm, hp, extra_found_inf):
    """Exchange of flags and sums between the ranks, then each rank's update and cast.

    The global decision and norm are formed once and given to every rank: the
    flag is the OR of all ranks' flags (and extra_found_inf, a flag from outside
    the simulated ranks); the global sum of squares is 0 + ss_0 + ss_1 + ... +
    ss_{N_d-1} in fp64, in rank order.  Partition invariance ("DeepSpeed ZeRO",
    ZeRO Stage 2 数学推导: the shards together make exactly the unpartitioned
    update) needs the same clip on every rank; a per-rank sum such as ss_r +
    (sum of the others) can round differently on different ranks."""
    global_flag = any(loc[1] for loc in locs) or bool(extra_found_inf)
    global_ss = 0.0
    for q in range(nd):
        global_ss = global_ss + locs[q][2]
    clip, norm = clip_coef(global_ss, max_norm)
    out = []
    for r, st in enumerate(states):
        u, flag, ss = locs[r]
        skip = global_flag
        adam(skip, u, clip, hp, st.counters, st.w, st.m, st.v)
        if not skip:
            cast(st.dtype, st.w, st.p16)
        out.append(dict(flag=flag, local_sumsq=ss, global_sumsq=global_ss, norm=norm, clip=clip, skipped=skip))
    return out
