"""Torch-side convenience around the offloaded (host) step of the C ABI
(include/zero_offload.h): allocates the caller-owned host buffers with torch --
the two 16-bit staging arrays pinned when a GPU is present, so the copies run
on the DMA engines -- and passes torch's current HIP stream.  The step runs in
libzero_shard.so; this module only marshals arguments."""
import ctypes

import numpy as np
import torch

from . import _abi as abi
from .shard import make_desc


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream) if torch.cuda.is_available() else None


class ZeroOffload:
    """One rank's shard with its fp32 state in host memory.

    params / grads: device tensors as for ZeroShard (flat or per tensor), or
    params=None for a host-only handle (then fill grad16 / param16 yourself).
    master_init: host fp32 tensor or array of the shard's valid elements, or None (then the
    master is the upcast of the shard's 16-bit parameters: read from the device, or, for a
    host-only handle, taken from param16_init).
    device_stats: with device parameters, give the library a device workspace so the step's
    flag and sum of squares are taken on the GPU and the host update overlaps the copy."""

    def __init__(self, numel, dp_size, dp_rank, dtype, params=None, grads=None, master_init=None, num_threads=0,
                 param16_init=None, device_stats=True):
        self.dtype = dtype
        self.host_only = params is None
        if self.host_only:
            self.desc = make_desc(numel, dp_size, dp_rank, dtype, None, None)
        else:
            self.desc = make_desc(numel, dp_size, dp_rank, dtype, params, grads)
        self._params, self._grads = params, grads
        plan_desc = self.desc if not self.host_only else make_desc(numel, dp_size, dp_rank, dtype,
                                                                   _FakeFlat(), None)
        self.info = abi.zero_shard_plan(plan_desc)
        n = max(self.info.valid_elems, 1)
        pin = torch.cuda.is_available()
        self.master = torch.empty(n, dtype=torch.float32)
        self.m = torch.empty(n, dtype=torch.float32)
        self.v = torch.empty(n, dtype=torch.float32)
        self.grad16 = torch.empty(n, dtype=torch.int16, pin_memory=pin)
        self.param16 = torch.empty(n, dtype=torch.int16, pin_memory=pin)
        b = abi.zero_offload_bufs_t()
        b.master, b.m, b.v = self.master.data_ptr(), self.m.data_ptr(), self.v.data_ptr()
        b.grad16, b.param16 = self.grad16.data_ptr(), self.param16.data_ptr()
        b.capacity = n
        self.workspace = None
        if device_stats and not self.host_only:
            self.workspace = torch.empty(self.info.workspace_bytes, dtype=torch.uint8, device="cuda")
            b.workspace = self.workspace.data_ptr()
            b.workspace_capacity = self.info.workspace_bytes
        self.bufs = b
        if param16_init is not None:
            self.host16("param16")[:] = np.asarray(param16_init, dtype=np.uint16)
        self._mi = None
        mi = None
        if master_init is not None:
            t = torch.as_tensor(np.ascontiguousarray(master_init, dtype=np.float32) if not torch.is_tensor(master_init)
                                else master_init.detach().cpu().contiguous())
            assert t.dtype == torch.float32 and t.numel() == self.info.valid_elems
            self._mi = t
            mi = t.data_ptr() if t.numel() else None
        self.h = abi.zero_offload_init(self.desc, b, mi, num_threads, _stream())

    # host views of the state (logical shard order)
    def host(self, which):
        t = {"master": self.master, "m": self.m, "v": self.v}[which]
        return t[:self.info.valid_elems].numpy()

    def host16(self, which):
        t = {"grad16": self.grad16, "param16": self.param16}[which]
        return t[:self.info.valid_elems].numpy().view(np.uint16)

    # step calls (same names as the C ABI)
    def zero_offload_fetch_grads(self, inv_loss_scale=1.0, flat_grad=None):
        abi.zero_offload_fetch_grads(self.h, flat_grad.data_ptr() if flat_grad is not None else None,
                                     inv_loss_scale, _stream())

    def zero_offload_grad_stats(self, inv_loss_scale):
        return abi.zero_offload_grad_stats(self.h, inv_loss_scale)

    def zero_offload_adam_step(self, lr, beta1, beta2, eps, weight_decay, other_ranks_found_inf=False,
                               other_ranks_sumsq=0.0, max_norm=1.0, push=True):
        hp = abi.zero_adam_hparams_t(lr, beta1, beta2, eps, weight_decay)
        abi.zero_offload_adam_step(self.h, hp, other_ranks_found_inf, other_ranks_sumsq, max_norm,
                                   push and not self.host_only, _stream())

    def zero_offload_adam_step_global(self, lr, beta1, beta2, eps, weight_decay, other_ranks_found_inf=False,
                                      global_sumsq=0.0, max_norm=1.0, push=True):
        hp = abi.zero_adam_hparams_t(lr, beta1, beta2, eps, weight_decay)
        abi.zero_offload_adam_step_global(self.h, hp, other_ranks_found_inf, global_sumsq, max_norm,
                                          push and not self.host_only, _stream())

    def zero_offload_push_params(self):
        abi.zero_offload_push_params(self.h, _stream())

    def query(self):
        return abi.zero_offload_query(self.h)

    def close(self):
        if self.h:
            abi.zero_offload_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class _FakeFlat:
    """Stands in for a flat parameter tensor when only the partition is needed."""

    @staticmethod
    def data_ptr():
        return 256
