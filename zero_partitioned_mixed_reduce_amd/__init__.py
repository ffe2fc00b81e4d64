"""One data-parallel rank's partitioned mixed-precision optimizer step (ZeRO
stage 1/2) on AMD Instinct MI355X: a thin binding of libzero_shard.so."""
from . import _abi
from ._abi import (ZERO_ACCUMULATED, ZERO_BF16, ZERO_DEVICE_LOSS_SCALE, ZERO_F16, ZeroError, zero_accumulate_grads,
                   zero_adam_hparams_t, zero_adam_step, zero_cast_params, zero_enable_dynamic_loss_scale,
                   zero_loss_scale, zero_loss_scaler_t, zero_set_reduce_output,
                   zero_check_overflow, zero_export_state, zero_grad_norm, zero_last_error, zero_local_stats,
                   zero_local_stats_device,
                   zero_reduce_grads, zero_shard_bufs_t, zero_shard_desc_t, zero_shard_destroy, zero_shard_info,
                   zero_shard_info_t, zero_shard_init, zero_shard_pieces, zero_shard_plan, zero_shard_query,
                   zero_set_segments, zero_segment_range, zero_wait_segment, zero_segment_timeouts,
                   zero_offload_bufs_t, zero_offload_init, zero_offload_fetch_grads, zero_offload_grad_stats,
                   zero_offload_adam_step, zero_offload_push_params, zero_offload_query, zero_offload_destroy)

__all__ = ["ZERO_F16", "ZERO_BF16", "ZERO_ACCUMULATED", "ZERO_DEVICE_LOSS_SCALE", "ZeroError", "zero_shard_plan",
           "zero_shard_init", "zero_enable_dynamic_loss_scale", "zero_loss_scale", "zero_loss_scaler_t", "zero_set_reduce_output",
           "zero_accumulate_grads", "zero_reduce_grads",
           "zero_local_stats", "zero_local_stats_device", "zero_check_overflow", "zero_grad_norm", "zero_adam_step", "zero_cast_params",
           "zero_shard_info", "zero_shard_pieces", "zero_shard_query", "zero_export_state", "zero_shard_destroy",
           "zero_last_error", "zero_shard_desc_t", "zero_shard_bufs_t", "zero_shard_info_t",
           "zero_adam_hparams_t", "zero_set_segments", "zero_segment_range", "zero_wait_segment",
           "zero_segment_timeouts", "zero_offload_bufs_t", "zero_offload_init", "zero_offload_fetch_grads",
           "zero_offload_grad_stats", "zero_offload_adam_step", "zero_offload_push_params", "zero_offload_query",
           "zero_offload_destroy", "ZeroShard", "ZeroOffload"]


def __getattr__(name):
    if name == "ZeroShard":
        from .shard import ZeroShard
        return ZeroShard
    if name == "ZeroOffload":
        from .offload import ZeroOffload
        return ZeroOffload
    raise AttributeError(name)
