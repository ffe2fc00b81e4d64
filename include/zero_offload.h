/* zero_offload.h -- C ABI of the offloaded optimizer step (ZeRO-Offload) of
 * one data-parallel rank's shard, on an AMD Instinct MI355X host.
 *
 * What it computes is the step of zero_shard.h -- unscale, overflow flag and
 * skip, global L2 norm and clip, Adam with bias correction and decoupled
 * weight decay, the round-to-nearest-even 16-bit write-back -- with the same
 * per-element fp32 arithmetic, but where the pages put it under ZeRO-Offload:
 *   - the fp32 master weights, the optimizer states (momentum, variance) and
 *     the 16-bit gradients are kept in host memory, while the 16-bit weights
 *     stay on the GPU for the forward and backward passes ("DeepSpeed ZeRO",
 *     ZeRO-Offload, 参数更新; "千亿参数模型如何塞进有限显卡", ZeRO-Offload：
 *     利用CPU内存);
 *   - after the backward pass the gradients are moved to the host
 *     asynchronously, the host cores run the optimizer update, and only the
 *     16-bit weights are copied back to the GPU ("DeepSpeed ZeRO",
 *     ZeRO-Offload, 异步调度策略).
 *
 * The host side is this library's own runtime: a pool of worker threads runs
 * AVX-512 loops over fixed tiles of the shard.  The device-to-host copy of the
 * gradient slice proceeds in blocks.  With a device workspace the step's flag
 * and sum of squares come from the GPU, where the gradient already is, and the
 * host update starts on each block as soon as it lands, overlapping the copy;
 * without one, a host statistics pass consumes the blocks as they land and the
 * update follows.  The host-to-device copy of each block of updated 16-bit
 * weights is enqueued as soon as that block is written.  Host results do not
 * depend on the thread count: the host sum of squares is formed per tile and
 * the tile sums are added in tile order.
 *
 * Conventions as in zero_shard.h (zero_status_t returns, zero_last_error(),
 * caller-owned memory, int64 sizes), plus:
 *   - Host arrays are in the shard's logical order (element i is flat model
 *     element shard_begin + i), valid_elems long; no alignment beyond the
 *     element size is required.  The two 16-bit staging arrays should be pinned
 *     (hipHostMalloc, or torch's pin_memory) so the copies run asynchronously
 *     on the DMA engines.
 *   - One step is: [zero_offload_fetch_grads] -> zero_offload_grad_stats ->
 *     zero_offload_adam_step [-> zero_offload_push_params].  Out-of-order calls
 *     return ZERO_ESTATE and change nothing.
 *   - The host calls return when their host work is done; the copies they
 *     enqueue run on the given stream.
 *   - The host cores must support AVX-512 (F, BW, VL) and F16C; init returns
 *     ZERO_EINVAL otherwise.  There is no other code path.
 */
#ifndef ZERO_OFFLOAD_H
#define ZERO_OFFLOAD_H

#include <stdint.h>

#include "zero_shard.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct zero_offload* zero_offload_t; /* opaque host handle */

/* Caller-allocated host buffers, each at least `capacity` elements. */
typedef struct {
  float* master;   /* fp32 master weights of the shard                                      */
  float* m;        /* fp32 first moment                                                      */
  float* v;        /* fp32 second moment                                                     */
  void* grad16;    /* 16-bit gradient slice: where zero_offload_fetch_grads lands it, or     */
                   /* where the caller writes it                                             */
  void* param16;   /* 16-bit parameter slice written by zero_offload_adam_step and copied    */
                   /* to the device from here                                                */
  int64_t capacity;/* elements of each array (>= valid_elems of the plan)                    */
  void* workspace; /* optional device workspace of zero_shard_plan's workspace_bytes         */
                   /* (256-byte aligned): the flag and sum of squares are then taken on the  */
                   /* GPU while the gradient is copied, and the host update starts on each   */
                   /* block as it lands; NULL: the host computes them from the copied slice  */
  int64_t workspace_capacity; /* bytes of workspace                                          */
} zero_offload_bufs_t;

/* Builds the handle: partition as zero_shard_plan (same description, same
 * sizes; zero_shard_plan gives valid_elems), m = v = 0, no step applied.
 * desc's device pointers (param16 / flat_param16, grad16 / flat_grad16) are
 * used only by the copy calls; a host-only handle gives neither param16 nor
 * flat_param16 (the copy calls then return ZERO_EINVAL).  The master is
 * master_init (host fp32 [valid_elems], logical order) or, when that is NULL,
 * the exact fp32 value of the shard's 16-bit parameters: copied from the
 * device into bufs.param16 on `stream` (synchronised), or, for a host-only
 * handle, as the caller left them in bufs.param16.  num_threads <= 0 uses the
 * host's hardware concurrency; at most 256.  EINVAL on a bad description,
 * null buffers, a capacity below valid_elems, or a host without AVX-512;
 * ENOMEM when host memory or the worker threads cannot be obtained. */
zero_status_t zero_offload_init(const zero_shard_desc_t* desc, const zero_offload_bufs_t* bufs,
                                const float* master_init, int32_t num_threads, void* stream, zero_offload_t* out);

/* Enqueues on `stream` the device-to-host copy of this rank's already-reduced
 * 16-bit gradient slice into bufs.grad16, block by block, and returns without
 * waiting.  flat_grad16: a device [psi] flat gradient, or NULL for the
 * gradient registered at init (grad16 / flat_grad16).  With a device
 * workspace, the step's flag and sum of squares of u = g * inv_loss_scale are
 * first computed on the device, over the gradient in device memory, by the
 * statistics kernel of zero_reduce_grads; pass the same inv_loss_scale to
 * zero_offload_grad_stats.  The gradient must stay unchanged until the step's
 * zero_offload_adam_step returns.  EINVAL for a host-only handle, without a
 * source, or for an inv_loss_scale that is not finite and positive; ESTATE
 * after zero_offload_grad_stats of the same step. */
zero_status_t zero_offload_fetch_grads(zero_offload_t h, const void* flat_grad16, float inv_loss_scale,
                                       void* stream);

/* The step's statistics: u = g * inv_loss_scale (fp32), found_inf = any u not
 * finite, sumsq = sum of u*u in fp64.  After a fetch on a handle with a device
 * workspace they are the device's (this call waits for the statistics kernel
 * only, not for the copies); otherwise the host computes them from
 * bufs.grad16, waiting for each block of a pending fetch as it lands.  Both
 * outputs are nullable.  EINVAL unless inv_loss_scale is finite and positive
 * (and, after a device fetch, equal to the fetch's). */
zero_status_t zero_offload_grad_stats(zero_offload_t h, float inv_loss_scale, int32_t* found_inf, double* sumsq);

/* The optimizer step on the host cores.  skip = this rank's flag OR
 * other_ranks_found_inf; norm = sqrt(sumsq + other_ranks_sumsq); clip =
 * max_norm / (norm + 1e-6) when that is below 1, else 1 (max_norm <= 0: no
 * clipping).  Unless skipped: t += 1, beta^t advance as fp64 running products,
 * bc = 1 - beta^t rounded to fp32, and per element, in fp32 with every
 * operation rounded to nearest even and no fused multiply-add,
 *   g = u * clip; m = b1 m + (1-b1) g; v = b2 v + (1-b2) g g;
 *   w = w - lr * ((m / bc1) / (sqrt(v / bc2) + eps) + wd * w);
 *   param16 = round-to-nearest-even 16-bit value of w (a NaN w: the positive
 *             canonical quiet NaN, as zero_cast_params writes it)
 * ("DeepSpeed ZeRO", ZeRO Stage 1, 以 AdaW 为例, with the readings of
 * zero_adam_step).  A skipped step changes nothing and copies nothing
 * ("DeepSpeed ZeRO", 权重更新的触发条件).  push != 0 (needs a device handle)
 * enqueues on `stream` the host-to-device copy of each block of bufs.param16
 * into the device parameters as soon as the block is updated.  Returns when
 * the update is done and every copy is enqueued.  Waits first for the copies
 * of the previous push, which read bufs.param16.  EINVAL on a null hparams
 * pointer or push on a host-only handle; ESTATE before zero_offload_grad_stats.
 * A gradient copy still in flight is consumed block by block: each block is
 * updated as soon as it lands. */
zero_status_t zero_offload_adam_step(zero_offload_t h, const zero_adam_hparams_t* hp, int32_t other_ranks_found_inf,
                                     double other_ranks_sumsq, float max_norm, int32_t push, void* stream);

/* As zero_offload_adam_step, but from the global sum of squares: norm =
 * sqrt(global_sumsq), with global_sumsq the sum over all ranks of their local
 * sums (zero_offload_grad_stats), formed once in rank order and given to every
 * rank, so every rank takes the same clip (see zero_grad_norm_global).  EINVAL
 * also if global_sumsq is negative. */
zero_status_t zero_offload_adam_step_global(zero_offload_t h, const zero_adam_hparams_t* hp,
                                            int32_t other_ranks_found_inf, double global_sumsq, float max_norm,
                                            int32_t push, void* stream);

/* Enqueues on `stream` the host-to-device copy of bufs.param16 (this rank's
 * valid elements) into the device parameters; nothing after a skipped step.
 * EINVAL on a host-only handle; ESTATE unless the last call was
 * zero_offload_adam_step. */
zero_status_t zero_offload_push_params(zero_offload_t h, void* stream);

/* Applied steps t, whether the last step skipped, and the global norm and
 * clip coefficient it used.  All outputs nullable. */
zero_status_t zero_offload_query(zero_offload_t h, int64_t* t, int32_t* last_skipped, double* last_norm,
                                 float* last_clip);

/* Waits for the handle's pending copies and frees it (never caller memory). */
zero_status_t zero_offload_destroy(zero_offload_t h);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_OFFLOAD_H */
