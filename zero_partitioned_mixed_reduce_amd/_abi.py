"""ctypes binding of libzero_shard.so: the C ABI declared in include/zero_shard.h,
with the same function and struct names.  Argument marshalling only."""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libzero_shard.so")

ZERO_OK, ZERO_EINVAL, ZERO_ENOMEM, ZERO_EHIP, ZERO_ESTATE = 0, -1, -2, -3, -4
ZERO_F16, ZERO_BF16 = 1, 2
ZERO_ACCUMULATED = -1
ZERO_DEVICE_LOSS_SCALE = 0.0
ZERO_STATIC_WORKSPACE_BYTES = 8 * 1024 * 1024

c_i64p = ctypes.POINTER(ctypes.c_int64)


class zero_shard_desc_t(ctypes.Structure):
    _fields_ = [("dp_size", ctypes.c_int32), ("dp_rank", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("align", ctypes.c_int32), ("num_tensors", ctypes.c_int64), ("numel", c_i64p),
                ("param16", ctypes.POINTER(ctypes.c_void_p)), ("flat_param16", ctypes.c_void_p),
                ("grad16", ctypes.POINTER(ctypes.c_void_p)), ("flat_grad16", ctypes.c_void_p)]


class zero_shard_info_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("psi", "shard_elems", "shard_begin", "valid_elems", "state_elems",
                                              "num_pieces", "num_chunks", "workspace_bytes",
                                              "model_state_bytes")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class zero_shard_bufs_t(ctypes.Structure):
    _fields_ = [("master", ctypes.c_void_p), ("m", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("red", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("state_capacity", ctypes.c_int64),
                ("workspace_capacity", ctypes.c_int64)]


class zero_loss_scaler_t(ctypes.Structure):
    _fields_ = [("init_scale", ctypes.c_float), ("growth_factor", ctypes.c_float), ("backoff_factor", ctypes.c_float),
                ("growth_interval", ctypes.c_int32), ("min_scale", ctypes.c_float)]


class zero_offload_bufs_t(ctypes.Structure):
    _fields_ = [("master", ctypes.c_void_p), ("m", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("grad16", ctypes.c_void_p), ("param16", ctypes.c_void_p), ("capacity", ctypes.c_int64),
                ("workspace", ctypes.c_void_p), ("workspace_capacity", ctypes.c_int64)]


class zero_adam_hparams_t(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float)]


_PROTOS = {
    "zero_shard_plan": [ctypes.POINTER(zero_shard_desc_t), ctypes.POINTER(zero_shard_info_t)],
    "zero_shard_init": [ctypes.POINTER(zero_shard_desc_t), ctypes.POINTER(zero_shard_bufs_t), ctypes.c_void_p,
                        ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)],
    "zero_shard_init_static": [ctypes.POINTER(zero_shard_desc_t), ctypes.POINTER(zero_shard_bufs_t), ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)],
    "zero_reduce_grads": [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32, ctypes.c_float,
                          ctypes.c_void_p],
    "zero_accumulate_grads": [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32, ctypes.c_void_p],
    "zero_set_reduce_output": [ctypes.c_void_p, ctypes.c_int32],
    "zero_local_stats": [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double),
                         ctypes.c_void_p],
    "zero_local_stats_device": [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p)],
    "zero_check_overflow": [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p],
    "zero_grad_norm": [ctypes.c_void_p, ctypes.c_double, ctypes.c_float, ctypes.POINTER(ctypes.c_double),
                       ctypes.c_void_p],
    "zero_grad_norm_global": [ctypes.c_void_p, ctypes.c_double, ctypes.c_float, ctypes.POINTER(ctypes.c_double),
                              ctypes.c_void_p],
    "zero_adam_step": [ctypes.c_void_p, ctypes.POINTER(zero_adam_hparams_t), ctypes.c_int32, ctypes.c_void_p],
    "zero_cast_params": [ctypes.c_void_p, ctypes.c_void_p],
    "zero_shard_info": [ctypes.c_void_p, ctypes.POINTER(zero_shard_info_t)],
    "zero_enable_dynamic_loss_scale": [ctypes.c_void_p, ctypes.POINTER(zero_loss_scaler_t), ctypes.c_void_p],
    "zero_loss_scale": [ctypes.c_void_p, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32),
                        ctypes.c_void_p],
    "zero_set_segments": [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)],
    "zero_segment_range": [ctypes.c_void_p, ctypes.c_int32, c_i64p, c_i64p],
    "zero_wait_segment": [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p],
    "zero_segment_timeouts": [ctypes.c_void_p, c_i64p, ctypes.c_void_p],
    "zero_shard_pieces": [ctypes.c_void_p, c_i64p, ctypes.c_int64],
    "zero_shard_query": [ctypes.c_void_p, c_i64p, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double),
                         ctypes.POINTER(ctypes.c_float), ctypes.c_void_p],
    "zero_export_state": [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p],
    "zero_shard_destroy": [ctypes.c_void_p],
    # offloaded (host) step, include/zero_offload.h
    "zero_offload_init": [ctypes.POINTER(zero_shard_desc_t), ctypes.POINTER(zero_offload_bufs_t), ctypes.c_void_p,
                          ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)],
    "zero_offload_fetch_grads": [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p],
    "zero_offload_grad_stats": [ctypes.c_void_p, ctypes.c_float, ctypes.POINTER(ctypes.c_int32),
                                ctypes.POINTER(ctypes.c_double)],
    "zero_offload_adam_step": [ctypes.c_void_p, ctypes.POINTER(zero_adam_hparams_t), ctypes.c_int32, ctypes.c_double,
                               ctypes.c_float, ctypes.c_int32, ctypes.c_void_p],
    "zero_offload_adam_step_global": [ctypes.c_void_p, ctypes.POINTER(zero_adam_hparams_t), ctypes.c_int32,
                                      ctypes.c_double, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p],
    "zero_offload_push_params": [ctypes.c_void_p, ctypes.c_void_p],
    "zero_offload_query": [ctypes.c_void_p, c_i64p, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double),
                           ctypes.POINTER(ctypes.c_float)],
    "zero_offload_destroy": [ctypes.c_void_p],
}

_lib = None


def lib():
    """Load libzero_shard.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(the HIP library is the only implementation)")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _PROTOS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.zero_last_error.argtypes = []
        L.zero_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


class ZeroError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = lib().zero_last_error().decode(errors="replace")
        super().__init__(f"{fn} returned {status}: {msg}")


def check(fn, status):
    if status != ZERO_OK:
        raise ZeroError(fn, status)


def _call(name, *args):
    check(name, getattr(lib(), name)(*args))


def zero_shard_plan(desc):
    info = zero_shard_info_t()
    _call("zero_shard_plan", ctypes.byref(desc), ctypes.byref(info))
    return info


def zero_shard_init(desc, bufs, master_init_ptr, stream):
    h = ctypes.c_void_p()
    _call("zero_shard_init", ctypes.byref(desc), ctypes.byref(bufs), master_init_ptr, stream, ctypes.byref(h))
    return h


def zero_shard_init_static(desc, bufs, master_init_ptr, stream):
    h = ctypes.c_void_p()
    _call("zero_shard_init_static", ctypes.byref(desc), ctypes.byref(bufs), master_init_ptr, stream, ctypes.byref(h))
    return h


def zero_reduce_grads(h, rank_grad_ptrs, inv_loss_scale, stream):
    """rank_grad_ptrs: list of device pointers, or ZERO_ACCUMULATED."""
    if rank_grad_ptrs is ZERO_ACCUMULATED or rank_grad_ptrs == ZERO_ACCUMULATED:
        _call("zero_reduce_grads", h, None, ZERO_ACCUMULATED, inv_loss_scale, stream)
        return
    n = len(rank_grad_ptrs)
    arr = (ctypes.c_void_p * max(n, 1))(*rank_grad_ptrs)
    _call("zero_reduce_grads", h, arr if n else None, n, inv_loss_scale, stream)


def zero_set_reduce_output(h, out_16bit):
    _call("zero_set_reduce_output", h, int(bool(out_16bit)))


def zero_accumulate_grads(h, rank_grad_ptrs, stream):
    n = len(rank_grad_ptrs)
    arr = (ctypes.c_void_p * max(n, 1))(*rank_grad_ptrs)
    _call("zero_accumulate_grads", h, arr if n else None, n, stream)


def zero_local_stats(h, stream):
    f, s = ctypes.c_int32(), ctypes.c_double()
    _call("zero_local_stats", h, ctypes.byref(f), ctypes.byref(s), stream)
    return bool(f.value), s.value


def zero_local_stats_device(h):
    """Device addresses (ints) of this rank's fp64 sum of squares and int32 flag."""
    s, f = ctypes.c_void_p(), ctypes.c_void_p()
    _call("zero_local_stats_device", h, ctypes.byref(s), ctypes.byref(f))
    return s.value, f.value


def zero_check_overflow(h, other_ranks_found_inf, stream, sync=False):
    out = ctypes.c_int32(-1)
    _call("zero_check_overflow", h, int(bool(other_ranks_found_inf)), ctypes.byref(out) if sync else None, stream)
    return bool(out.value) if sync else None


def zero_grad_norm(h, other_ranks_sumsq, max_norm, stream, sync=False):
    out = ctypes.c_double(float("nan"))
    _call("zero_grad_norm", h, other_ranks_sumsq, max_norm, ctypes.byref(out) if sync else None, stream)
    return out.value if sync else None


def zero_grad_norm_global(h, global_sumsq, max_norm, stream, sync=False):
    out = ctypes.c_double(float("nan"))
    _call("zero_grad_norm_global", h, global_sumsq, max_norm, ctypes.byref(out) if sync else None, stream)
    return out.value if sync else None


def zero_adam_step(h, hp, fuse_cast, stream):
    _call("zero_adam_step", h, ctypes.byref(hp), int(bool(fuse_cast)), stream)


def zero_cast_params(h, stream):
    _call("zero_cast_params", h, stream)


def zero_set_segments(h, n_segments):
    n = ctypes.c_int32()
    _call("zero_set_segments", h, n_segments, ctypes.byref(n))
    return n.value


def zero_segment_range(h, k):
    b, n = ctypes.c_int64(), ctypes.c_int64()
    _call("zero_segment_range", h, k, ctypes.byref(b), ctypes.byref(n))
    return b.value, n.value


def zero_wait_segment(h, k, stream):
    _call("zero_wait_segment", h, k, stream)


def zero_segment_timeouts(h, stream):
    n = ctypes.c_int64()
    _call("zero_segment_timeouts", h, ctypes.byref(n), stream)
    return n.value


def zero_enable_dynamic_loss_scale(h, cfg, stream):
    _call("zero_enable_dynamic_loss_scale", h, ctypes.byref(cfg), stream)


def zero_loss_scale(h, stream):
    sc, good = ctypes.c_float(), ctypes.c_int32()
    _call("zero_loss_scale", h, ctypes.byref(sc), ctypes.byref(good), stream)
    return sc.value, good.value


def zero_shard_info(h):
    info = zero_shard_info_t()
    _call("zero_shard_info", h, ctypes.byref(info))
    return info


def zero_shard_pieces(h, n):
    out = (ctypes.c_int64 * (5 * max(n, 1)))()
    _call("zero_shard_pieces", h, out, n)
    return [tuple(out[5 * p:5 * p + 5]) for p in range(n)]


def zero_shard_query(h, stream):
    t, sk, nrm, clip = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_double(), ctypes.c_float()
    _call("zero_shard_query", h, ctypes.byref(t), ctypes.byref(sk), ctypes.byref(nrm), ctypes.byref(clip), stream)
    return dict(t=t.value, skipped=bool(sk.value), norm=nrm.value, clip=clip.value)


def zero_export_state(h, which, dst_ptr, stream):
    _call("zero_export_state", h, which, dst_ptr, stream)


def zero_shard_destroy(h):
    _call("zero_shard_destroy", h)


def zero_offload_init(desc, bufs, master_init_ptr, num_threads, stream):
    h = ctypes.c_void_p()
    _call("zero_offload_init", ctypes.byref(desc), ctypes.byref(bufs), master_init_ptr, num_threads, stream,
          ctypes.byref(h))
    return h


def zero_offload_fetch_grads(h, flat_grad16_ptr, inv_loss_scale, stream):
    _call("zero_offload_fetch_grads", h, flat_grad16_ptr, inv_loss_scale, stream)


def zero_offload_grad_stats(h, inv_loss_scale):
    f, s = ctypes.c_int32(), ctypes.c_double()
    _call("zero_offload_grad_stats", h, inv_loss_scale, ctypes.byref(f), ctypes.byref(s))
    return bool(f.value), s.value


def zero_offload_adam_step(h, hp, other_ranks_found_inf, other_ranks_sumsq, max_norm, push, stream):
    _call("zero_offload_adam_step", h, ctypes.byref(hp), int(bool(other_ranks_found_inf)), other_ranks_sumsq,
          max_norm, int(bool(push)), stream)

def zero_offload_adam_step_global(h, hp, other_ranks_found_inf, global_sumsq, max_norm, push, stream):
    _call("zero_offload_adam_step_global", h, ctypes.byref(hp), int(bool(other_ranks_found_inf)), global_sumsq,
          max_norm, int(bool(push)), stream)


def zero_offload_push_params(h, stream):
    _call("zero_offload_push_params", h, stream)


def zero_offload_query(h):
    t, sk, nrm, clip = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_double(), ctypes.c_float()
    _call("zero_offload_query", h, ctypes.byref(t), ctypes.byref(sk), ctypes.byref(nrm), ctypes.byref(clip))
    return dict(t=t.value, skipped=bool(sk.value), norm=nrm.value, clip=clip.value)


def zero_offload_destroy(h):
    _call("zero_offload_destroy", h)


def zero_last_error():
    return lib().zero_last_error().decode(errors="replace")
