"""One data-parallel rank's partitioned mixed-precision optimizer step (ZeRO
stage 1/2) on AMD Instinct MI355X: a thin binding of libzero_shard.so.

The C ABI's calls and structs are available here under their C names
(zero_shard_init, zero_reduce_grads, ...); ZeroShard and ZeroOffload hold the
caller-owned buffers of one handle and call them."""
from . import _abi
from ._abi import ZERO_ACCUMULATED, ZERO_BF16, ZERO_DEVICE_LOSS_SCALE, ZERO_F16, ZeroError

_C_NAMES = sorted(n for n in vars(_abi) if n.startswith("zero_"))
globals().update({n: getattr(_abi, n) for n in _C_NAMES})

__all__ = ["ZERO_F16", "ZERO_BF16", "ZERO_ACCUMULATED", "ZERO_DEVICE_LOSS_SCALE", "ZeroError", "ZeroShard",
           "ZeroOffload"] + _C_NAMES


def __getattr__(name):
    if name == "ZeroShard":
        from .shard import ZeroShard
        return ZeroShard
    if name == "ZeroOffload":
        from .offload import ZeroOffload
        return ZeroOffload
    raise AttributeError(name)
