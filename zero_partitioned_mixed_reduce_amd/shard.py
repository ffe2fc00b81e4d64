"""Torch-side convenience around the C ABI: allocates the caller-owned device
buffers with torch and passes torch's current HIP stream.  Every step of the
path runs in libzero_shard.so; this module only marshals arguments."""
import ctypes

import torch

from . import _abi as abi

_TDT = {abi.ZERO_F16: torch.float16, abi.ZERO_BF16: torch.bfloat16}


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_desc(numel, dp_size, dp_rank, dtype, params, grads=None, align=0):
    """params / grads: one flat tensor, or a list of per-tensor tensors (or None: no device pointers)."""
    numel = [int(n) for n in numel]
    keep = {}
    d = abi.zero_shard_desc_t()
    d.dp_size, d.dp_rank, d.dtype, d.align = dp_size, dp_rank, dtype, align
    arr = (ctypes.c_int64 * len(numel))(*numel)
    keep["numel"] = arr
    d.num_tensors = len(numel)
    d.numel = ctypes.cast(arr, abi.c_i64p)

    def ptrs(ts):
        a = (ctypes.c_void_p * len(ts))(*[t.data_ptr() if t is not None else None for t in ts])
        return a

    if isinstance(params, (list, tuple)):
        keep["p"] = ptrs(params)
        d.param16 = ctypes.cast(keep["p"], ctypes.POINTER(ctypes.c_void_p))
    elif params is not None:
        d.flat_param16 = params.data_ptr()
    if grads is not None:
        if isinstance(grads, (list, tuple)):
            keep["g"] = ptrs(grads)
            d.grad16 = ctypes.cast(keep["g"], ctypes.POINTER(ctypes.c_void_p))
        else:
            d.flat_grad16 = grads.data_ptr()
    d._keep = keep
    return d


class ZeroShard:
    """One rank's shard: plan, caller-owned buffers (torch), handle."""

    def __init__(self, numel, dp_size, dp_rank, dtype, params, grads=None, master_init=None, with_red=False,
                 device="cuda", align=0, static_workspace=False):
        """static_workspace: no workspace is allocated; the handle uses the library's static
        device workspace (zero_shard_init_static)."""
        self.dtype = dtype
        self.desc = make_desc(numel, dp_size, dp_rank, dtype, params, grads, align)
        self._params, self._grads = params, grads
        self.info = abi.zero_shard_plan(self.desc)
        n = self.info.state_elems
        self.master, self.m, self.v, self.red = self._alloc_state(n, with_red, device)
        self.workspace = None
        if not static_workspace:
            self.workspace = torch.empty(self.info.workspace_bytes, dtype=torch.uint8, device=device)
        b = abi.zero_shard_bufs_t()
        b.master, b.m, b.v = self.master.data_ptr(), self.m.data_ptr(), self.v.data_ptr()
        b.red = self.red.data_ptr() if self.red is not None else None
        b.workspace = self.workspace.data_ptr() if self.workspace is not None else None
        b.state_capacity = n
        b.workspace_capacity = self.info.workspace_bytes if self.workspace is not None else 0
        self.bufs = b
        mi = None
        if master_init is not None:
            assert master_init.dtype == torch.float32 and master_init.numel() == self.info.valid_elems
            mi = master_init.data_ptr()
        init = abi.zero_shard_init_static if static_workspace else abi.zero_shard_init
        self.h = init(self.desc, b, mi, _stream())

    # Placement of the state arrays (master, m, v, red).  None: one allocation per array.
    # state_stagger (floats): carved from one allocation, each n + state_stagger floats after
    # the previous one.  state_pitch (bytes, a multiple of 256): carved from one allocation,
    # each starting state_pitch bytes after the previous one; the gaps are allocated too.
    state_stagger = None
    state_pitch = None

    def _alloc_state(self, n, with_red, device):
        k = 4 if with_red else 3
        if self.state_pitch is not None:
            pitch = self.state_pitch // 4
            assert self.state_pitch % 256 == 0 and pitch >= n, "state_pitch must hold one array"
            self._state_store = torch.empty((k - 1) * pitch + n, dtype=torch.float32, device=device)
            arrs = [self._state_store[i * pitch:i * pitch + n] for i in range(k)]
        elif self.state_stagger is None:
            arrs = [torch.empty(n, dtype=torch.float32, device=device) for _ in range(k)]
        else:
            pitch = n + self.state_stagger
            self._state_store = torch.empty(k * pitch, dtype=torch.float32, device=device)
            arrs = [self._state_store[i * pitch:i * pitch + n] for i in range(k)]
        return arrs[0], arrs[1], arrs[2], (arrs[3] if with_red else None)

    # step calls (same names as the C ABI)
    def zero_reduce_grads(self, rank_grads, inv_loss_scale):
        """rank_grads: list of 16-bit tensors ([] for the registered gradient) or
        abi.ZERO_ACCUMULATED."""
        if isinstance(rank_grads, int):
            abi.zero_reduce_grads(self.h, rank_grads, inv_loss_scale, _stream())
            return
        ptrs = [g.data_ptr() for g in rank_grads] if rank_grads else []
        abi.zero_reduce_grads(self.h, ptrs, inv_loss_scale, _stream())

    def zero_set_reduce_output(self, out_16bit):
        """Deliver the local reduce's sum in the 16-bit dtype (True) or keep it in fp32 (False)."""
        abi.zero_set_reduce_output(self.h, out_16bit)

    def zero_accumulate_grads(self, rank_grads):
        ptrs = [g.data_ptr() for g in rank_grads] if rank_grads else []
        abi.zero_accumulate_grads(self.h, ptrs, _stream())

    def zero_local_stats(self):
        return abi.zero_local_stats(self.h, _stream())

    def zero_local_stats_device(self):
        """(sumsq, found_inf): device addresses of this rank's fp64 sum of squares and int32
        flag in the workspace, for an in-place all-reduce across ranks."""
        return abi.zero_local_stats_device(self.h)

    def zero_check_overflow(self, other_ranks_found_inf=False, sync=False):
        return abi.zero_check_overflow(self.h, other_ranks_found_inf, _stream(), sync)

    def zero_grad_norm(self, other_ranks_sumsq=0.0, max_norm=1.0, sync=False):
        return abi.zero_grad_norm(self.h, other_ranks_sumsq, max_norm, _stream(), sync)

    def zero_grad_norm_global(self, global_sumsq, max_norm=1.0, sync=False):
        """The norm from the global sum of squares (all ranks' local sums, added once in
        rank order and given to every rank)."""
        return abi.zero_grad_norm_global(self.h, global_sumsq, max_norm, _stream(), sync)

    def zero_adam_step(self, lr, beta1, beta2, eps, weight_decay, fuse_cast=True):
        hp = abi.zero_adam_hparams_t(lr, beta1, beta2, eps, weight_decay)
        abi.zero_adam_step(self.h, hp, fuse_cast, _stream())

    def zero_cast_params(self):
        abi.zero_cast_params(self.h, _stream())

    def zero_set_segments(self, n_segments):
        """Track completion of the 16-bit write-back in up to n_segments segments; returns
        the number of segments (0 turns tracking off)."""
        return abi.zero_set_segments(self.h, n_segments)

    def zero_segment_range(self, k):
        """(first logical shard element, number of elements) of segment k."""
        return abi.zero_segment_range(self.h, k)

    def zero_wait_segment(self, k, stream=None):
        """Enqueue on `stream` (a torch stream; default: the current one) a wait for
        segment k of the latest step's write-back."""
        s = _stream() if stream is None else ctypes.c_void_p(stream.cuda_stream)
        abi.zero_wait_segment(self.h, k, s)

    def zero_segment_timeouts(self):
        return abi.zero_segment_timeouts(self.h, _stream())

    def zero_enable_dynamic_loss_scale(self, init_scale=65536.0, growth_factor=2.0, backoff_factor=0.5,
                                       growth_interval=1000, min_scale=1.0):
        cfg = abi.zero_loss_scaler_t(init_scale, growth_factor, backoff_factor, growth_interval, min_scale)
        abi.zero_enable_dynamic_loss_scale(self.h, cfg, _stream())

    def zero_loss_scale(self):
        """(current dynamic loss scale, good steps since it last changed)."""
        return abi.zero_loss_scale(self.h, _stream())

    def query(self):
        return abi.zero_shard_query(self.h, _stream())

    def pieces(self):
        return abi.zero_shard_pieces(self.h, self.info.num_pieces)

    def export(self, which):
        """State buffer `which` ('master', 'm', 'v', 'red') in logical shard order (device fp32)."""
        idx = {"master": 0, "m": 1, "v": 2, "red": 3}[which]
        out = torch.empty(self.info.valid_elems, dtype=torch.float32, device=self.master.device)
        abi.zero_export_state(self.h, idx, out.data_ptr() if out.numel() else None, _stream())
        return out

    def close(self):
        if self.h:
            abi.zero_shard_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
