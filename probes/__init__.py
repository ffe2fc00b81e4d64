"""Bandwidth probes for the benchmark (libzprobe.so): streaming kernels with the
memory-access patterns of the optimizer step's kernels and none of its
arithmetic, timed on the same GPU to give the ceiling each pattern reaches.
Not part of the optimizer library; the benchmark is their only user."""
import ctypes
import os

from . import build as _build

_lib = None
_I64, _I32, _P = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            raise RuntimeError("probe library not built: run __graft_entry__.build()")
        L = ctypes.CDLL(_build.LIB)
        L.zprobe_adam_mix.argtypes = [_P, _I32, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _P]
        for name in ("zprobe_read32", "zprobe_read16"):
            getattr(L, name).argtypes = [_P, _I64, _P, _I32, _I32, _I32, _I32, _P]
        L.zprobe_write32.argtypes = [_P, _I64, _I32, _I32, _I32, _I32, _P]
        L.zprobe_copy32.argtypes = [_P, _P, _I64, _I32, _I32, _I32, _I32, _P]
        L.zprobe_reduce_mix.argtypes = [ctypes.POINTER(_P), _I32, _P, _I64, _I32, _I32, _I32, _I32, _P]
        for name in ("zprobe_adam_mix", "zprobe_read32", "zprobe_read16", "zprobe_write32", "zprobe_copy32",
                     "zprobe_reduce_mix"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(name, rc):
    if rc != 0:
        raise RuntimeError(f"{name} failed with hipError {rc}")


def adam_mix(g, w, m, v, p16, n, stream, epb=2048, u=2, bs=256, nt_load=1, nt_store=1, g32=False):
    """Reads g (16-bit, or fp32 with g32), w, m, v; writes w, m, v and p16: 28 (30) B per element."""
    _check("zprobe_adam_mix", lib().zprobe_adam_mix(g, int(bool(g32)), w, m, v, p16, n, epb, u, bs, nt_load,
                                                    nt_store, stream))


def read32(src, n, sink, stream, epb=2048, u=2, bs=256, nt=1):
    _check("zprobe_read32", lib().zprobe_read32(src, n, sink, epb, u, bs, nt, stream))


def read16(src, n, sink, stream, epb=8192, u=4, bs=256, nt=1):
    _check("zprobe_read16", lib().zprobe_read16(src, n, sink, epb, u, bs, nt, stream))


def write32(dst, n, stream, epb=2048, u=2, bs=256, nt=1):
    _check("zprobe_write32", lib().zprobe_write32(dst, n, epb, u, bs, nt, stream))


def copy32(src, dst, n, stream, epb=2048, u=2, bs=256, nt=1):
    _check("zprobe_copy32", lib().zprobe_copy32(src, dst, n, epb, u, bs, nt, stream))


def reduce_mix(srcs, out, n, stream, epb=8192, u=2, bs=256, nt=1):
    arr = (_P * len(srcs))(*srcs)
    _check("zprobe_reduce_mix", lib().zprobe_reduce_mix(arr, len(srcs), out, n, epb, u, bs, nt, stream))
