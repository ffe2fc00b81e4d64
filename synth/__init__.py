"""Seeded synthetic inputs for tests and the benchmark.

A counter-based generator (SplitMix64 words -> Irwin-Hall(8) approximately
normal values, see zsynth_core.h): every element is a pure function of
(seed, stream, index), produced bit-identically by the host filler (for the
oracle side) and the device filler (to create multi-gigabyte inputs in HBM).
Holds none of the optimizer's arithmetic.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F16, BF16 = 1, 2
_host = None
_gpu = None


def host():
    global _host
    if _host is None:
        if not os.path.exists(_build.HOST_LIB):
            raise RuntimeError("synth host library not built: run __graft_entry__.build()")
        L = ctypes.CDLL(_build.HOST_LIB)
        L.zs_fill_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint64,
                                  ctypes.c_int64, ctypes.c_double]
        L.zs_fill_16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                 ctypes.c_int64, ctypes.c_double, ctypes.c_uint64, ctypes.c_uint32]
        L.zs_gather_16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double, ctypes.c_uint64,
                                   ctypes.c_uint32]
        L.zs_set_threads.argtypes = [ctypes.c_int]
        L.zs_gather_f32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                    ctypes.c_uint64, ctypes.c_double]
        _host = L
    return _host


def gpu():
    global _gpu
    if _gpu is None:
        if not os.path.exists(_build.GPU_LIB):
            raise RuntimeError("synth device library not built: run __graft_entry__.build()")
        L = ctypes.CDLL(_build.GPU_LIB)
        L.zs_gpu_fill_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint64,
                                      ctypes.c_int64, ctypes.c_double, ctypes.c_void_p]
        L.zs_gpu_fill_f32.restype = ctypes.c_int
        L.zs_gpu_fill_16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint64,
                                     ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_uint64,
                                     ctypes.c_uint32, ctypes.c_void_p]
        L.zs_gpu_fill_16.restype = ctypes.c_int
        _gpu = L
    return _gpu


def set_host_threads(n: int) -> None:
    """OpenMP threads per host fill call (0 = default); global for the process."""
    host().zs_set_threads(n)


def stream_id(array: int, rank: int = 0, step: int = 0) -> int:
    """One generator stream per (array, rank, step)."""
    return (array << 48) | (rank << 24) | step


MASTER, GRAD, PARAM = 1, 2, 3


def normal_f32(n, seed, stream, first=0, sigma=1.0):
    out = np.empty(n, np.float32)
    host().zs_fill_f32(out.ctypes.data, n, seed, stream, first, sigma)
    return out


def normal_16(n, dtype, seed, stream, first=0, sigma=1.0, zero_seed=0, zero_mod=0):
    out = np.empty(n, np.uint16)
    host().zs_fill_16(out.ctypes.data, n, dtype, seed, stream, first, sigma, zero_seed, zero_mod)
    return out


def gather_16(idx, dtype, seed, stream, sigma=1.0, zero_seed=0, zero_mod=0):
    idx = np.ascontiguousarray(idx, np.int64)
    out = np.empty(idx.size, np.uint16)
    host().zs_gather_16(out.ctypes.data, idx.ctypes.data, idx.size, dtype, seed, stream, sigma, zero_seed, zero_mod)
    return out


def gather_f32(idx, seed, stream, sigma=1.0):
    idx = np.ascontiguousarray(idx, np.int64)
    out = np.empty(idx.size, np.float32)
    host().zs_gather_f32(out.ctypes.data, idx.ctypes.data, idx.size, seed, stream, sigma)
    return out


def gpu_normal_f32(tensor, seed, stream, first=0, sigma=1.0, hip_stream=None):
    """Fill a contiguous float32 torch CUDA tensor on the given (or current) stream."""
    import torch
    assert tensor.is_cuda and tensor.dtype == torch.float32 and tensor.is_contiguous()
    s = hip_stream if hip_stream is not None else torch.cuda.current_stream().cuda_stream
    rc = gpu().zs_gpu_fill_f32(tensor.data_ptr(), tensor.numel(), seed, stream, first, sigma, s)
    if rc != 0:
        raise RuntimeError(f"zs_gpu_fill_f32 failed: hip error {rc}")


def gpu_normal_16(tensor, dtype, seed, stream, first=0, sigma=1.0, zero_seed=0, zero_mod=0, hip_stream=None):
    """Fill a contiguous 16-bit torch CUDA tensor (float16/bfloat16/int16/uint16 storage)."""
    import torch
    assert tensor.is_cuda and tensor.element_size() == 2 and tensor.is_contiguous()
    s = hip_stream if hip_stream is not None else torch.cuda.current_stream().cuda_stream
    rc = gpu().zs_gpu_fill_16(tensor.data_ptr(), tensor.numel(), dtype, seed, stream, first, sigma, zero_seed,
                              zero_mod, s)
    if rc != 0:
        raise RuntimeError(f"zs_gpu_fill_16 failed: hip error {rc}")
