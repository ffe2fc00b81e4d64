/* zero_shard.h -- C ABI of one data-parallel rank's partitioned mixed-precision
 * optimizer step (ZeRO stage 1/2) on one AMD Instinct MI355X (gfx950).
 *
 * What the step computes (the pages on DeepSpeed ZeRO):
 *   - model states are fp16/bf16 parameters and gradients plus fp32 master
 *     weights, momentum and variance ("ZeRO 技术原理" section 3; "DeepSpeed ZeRO"
 *     表格计算);
 *   - the flattened, padded model is cut into N_d equal shards and rank r owns
 *     and updates only shard r ("ZeRO 技术原理" 3.1.1 and 3.3.1;
 *     "DeepSpeed ZeRO" ZeRO Stage 3 基本流程);
 *   - the shard's gradient is the reduce-scatter of the ranks' gradients
 *     ("DeepSpeed ZeRO" ZeRO Stage 2 基本思想); this library performs the local
 *     reduction half on buffers already resident on the GPU;
 *   - a nan/inf gradient skips the update entirely ("DeepSpeed ZeRO"
 *     权重更新的触发条件);
 *   - Adam updates the fp32 master, momentum and variance ("DeepSpeed ZeRO"
 *     ZeRO Stage 1, 以 AdaW 为例), here with bias correction, decoupled weight
 *     decay and global-norm clipping;
 *   - the updated fp32 slice is written back in place into the 16-bit
 *     parameters for the all-gather that follows ("DeepSpeed ZeRO" 具体训练步骤).
 *
 * Conventions
 *   - Every call returns a zero_status_t; on failure zero_last_error() gives a
 *     message (thread-local, valid until the next call on the same thread).
 *   - Device memory is owned by the caller (parameters, gradients, fp32 state
 *     and the workspace); the library owns only the host-side handle and never
 *     frees caller memory.  All pointers given to zero_shard_init must stay
 *     valid until zero_shard_destroy.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue work
 *     on it and return without waiting, except where a host_* output pointer is
 *     non-NULL (the call then synchronises the stream) and for the query calls.
 *   - One step is: zero_reduce_grads -> zero_check_overflow -> zero_grad_norm
 *     -> zero_adam_step [-> zero_cast_params].  Calls out of that order return
 *     ZERO_ESTATE and change nothing.
 *   - Element counts and offsets are int64 (a 7.5e9-element model is fine).
 *   - Calls on one handle must not overlap (one host thread, one stream at a
 *     time); different handles are independent.
 *   - A step's calls (without host_* outputs or segments) only enqueue kernels,
 *     and the step counters, the loss scale and the choice between the two
 *     counter slots live in the workspace, so a step captured into a HIP graph
 *     can be replayed: each replay is one more step.  Host queries after
 *     replays read the device state.  The arguments of the captured calls
 *     (inv_loss_scale, other_ranks_*, max_norm, hyperparameters, pointers) are
 *     fixed in the graph; see zero_local_stats_device for taking the other
 *     ranks' values from device memory.  Segment tracking counts steps on the
 *     host and is not for replays.
 *
 * Typical use, one rank of N_d (error checks omitted):
 *   zero_shard_plan(&desc, &info);                    sizes: state_elems, workspace_bytes
 *   allocate master, m, v (and red) of info.state_elems floats, the workspace
 *   zero_shard_init(&desc, &bufs, master_init_or_NULL, stream, &h);
 *   per step:
 *     zero_reduce_grads(h, rank_bufs, N_d, 1.0f / loss_scale, stream);
 *     exchange this rank's flag and sum of squares with the other ranks, on the
 *       host (zero_local_stats) or in place on the device (zero_local_stats_device)
 *     zero_check_overflow(h, other_ranks_found_inf, NULL, stream);
 *     zero_grad_norm(h, other_ranks_sumsq, max_norm, NULL, stream);
 *     zero_adam_step(h, &hparams, 1, stream);          16-bit slice written back
 *     all-gather the 16-bit slices
 *   zero_shard_destroy(h);
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ZERO_OK = 0,
  ZERO_EINVAL = -1, /* bad argument: null pointer, size, dtype, alignment, rank count */
  ZERO_ENOMEM = -2, /* host memory or worker threads could not be obtained           */
  ZERO_EHIP = -3,   /* a HIP runtime call failed (message names it)                  */
  ZERO_ESTATE = -4  /* call out of the step order                                    */
} zero_status_t;

typedef enum { ZERO_F16 = 1, ZERO_BF16 = 2 } zero_dtype_t;

typedef struct zero_shard* zero_shard_t; /* opaque host handle */

/* Description of the model and of this rank.  Host memory, read during the call. */
typedef struct {
  int32_t dp_size;            /* N_d >= 1                                                     */
  int32_t dp_rank;            /* 0 <= dp_rank < N_d                                           */
  int32_t dtype;              /* zero_dtype_t of the 16-bit parameters and gradients         */
  int32_t align;              /* shard length is a multiple of this many elements; 0 -> 64;  */
                              /* must be a multiple of 8                                      */
  int64_t num_tensors;        /* 1 <= T <= 2^31 - 1 tensors, flattened in this order         */
  const int64_t* numel;       /* host [T], each >= 0; psi = sum <= 2^60                       */
  void* const* param16;       /* host [T] of device pointers, one per tensor, or NULL         */
  void* flat_param16;         /* device [psi] flat 16-bit parameters, or NULL                 */
                              /* (exactly one of param16 / flat_param16)                      */
  const void* const* grad16;  /* host [T] of device pointers: the already-reduced 16-bit      */
                              /* gradient per tensor, or NULL                                 */
  const void* flat_grad16;    /* device [psi] already-reduced flat gradient, or NULL          */
                              /* (at most one of grad16 / flat_grad16; used by                */
                              /* zero_reduce_grads with n_ranks == 0)                         */
} zero_shard_desc_t;

/* Sizes of this rank's shard (zero_shard_plan / zero_shard_info). */
typedef struct {
  int64_t psi;               /* total parameters                                              */
  int64_t shard_elems;       /* S: every rank's shard length (multiple of align)             */
  int64_t shard_begin;       /* r * S: flat index of this rank's first element               */
  int64_t valid_elems;       /* elements of [r*S, r*S + S) inside [0, psi)                    */
  int64_t state_elems;       /* floats the caller allocates for each of master, m, v (and red) */
  int64_t num_pieces;        /* tensor pieces the shard touches                               */
  int64_t num_chunks;        /* work items of the kernels                                     */
  int64_t workspace_bytes;   /* device workspace the caller allocates (256-byte aligned)      */
  int64_t model_state_bytes; /* bytes this rank keeps for the method's model states:          */
                             /* full 16-bit params and grads + 12 * state_elems (ZeRO-1 view) */
} zero_shard_info_t;

/* Caller-allocated device buffers, each 16-byte aligned. */
typedef struct {
  float* master;             /* [state_capacity] fp32 master weights                          */
  float* m;                  /* [state_capacity] fp32 first moment                            */
  float* v;                  /* [state_capacity] fp32 second moment                           */
  float* red;                /* [state_capacity] fp32 reduced gradient; required only for     */
                             /* zero_reduce_grads with n_ranks >= 2, else may be NULL         */
  void* workspace;           /* [workspace_bytes], 256-byte aligned                           */
  int64_t state_capacity;    /* floats allocated per state buffer (>= state_elems)            */
  int64_t workspace_capacity;/* bytes allocated for the workspace (>= workspace_bytes)        */
} zero_shard_bufs_t;

typedef struct {
  float lr, beta1, beta2, eps, weight_decay;
} zero_adam_hparams_t;

/* Partition and sizes only; no GPU work.  psi = sum(numel); S = align *
 * ceil(ceil(psi / N_d) / align); this rank owns flat [r*S, r*S + S) clipped to
 * [0, psi) -- the flatten-and-pad partition of "DeepSpeed ZeRO" ZeRO Stage 3
 * 基本流程 with start = partition size * rank as in "ZeRO 技术原理" 3.3.1.
 * The fp32 state is laid out in tensor pieces, each placed so that it has the
 * same 16-byte alignment as its 16-bit parameters (a few padding floats per
 * piece), hence state_elems >= valid_elems.  EINVAL on a bad description;
 * ENOMEM when the host tables do not fit in host memory. */
zero_status_t zero_shard_plan(const zero_shard_desc_t* desc, zero_shard_info_t* out);

/* Builds the handle: copies the work table into the workspace, zeroes the
 * state, sets the master to master_init (device fp32 [valid_elems], this
 * shard in logical order) or, when master_init is NULL, to the exact fp32
 * value of this shard's 16-bit parameters (the partition_fp16.copy().float()
 * of "DeepSpeed ZeRO" ZeRO Stage 1); m = v = 0 and no step applied yet.
 * Synchronises the stream before returning.  EINVAL on a bad description,
 * null or misaligned buffers, or capacities below zero_shard_plan's sizes;
 * ENOMEM when the handle's host tables cannot be allocated. */
zero_status_t zero_shard_init(const zero_shard_desc_t* desc, const zero_shard_bufs_t* bufs,
                              const float* master_init, void* stream, zero_shard_t* out);

/* Size in bytes of the library's static device workspace (one per device): the
 * largest workspace_bytes a handle made by zero_shard_init_static may need.
 * 8 MiB holds the workspace of shards of up to about 100,000 work items (one
 * flat tensor of about 8.2e8 elements; fewer elements when a ragged tensor
 * list cuts the shard into more pieces). */
#define ZERO_STATIC_WORKSPACE_BYTES (8 * 1024 * 1024)

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: as
 * zero_shard_init, but the handle's workspace is the library's own static
 * device array of ZERO_STATIC_WORKSPACE_BYTES on the current device, held
 * from the first such call on the device until the process ends.
 * bufs->workspace must be NULL (bufs->workspace_capacity is ignored); the
 * caller still passes the state buffers (master, m, v, red) and the 16-bit
 * inputs and outputs.  Makes no device allocation: no hipMalloc, hipFree or
 * allocating library routine (the handle itself is host memory).
 *   - EINVAL if zero_shard_plan's workspace_bytes for the description exceeds
 *     ZERO_STATIC_WORKSPACE_BYTES (use zero_shard_init with a workspace then),
 *     or if bufs->workspace is not NULL; otherwise the errors of
 *     zero_shard_init.
 *   - One array per device: every zero_shard_init_static on a device takes it
 *     over (re-initialising all of it, so nothing of an earlier handle
 *     carries over), after which calls on earlier such handles of that device
 *     return ZERO_ESTATE (zero_shard_destroy still frees them).  Work that an
 *     earlier handle already enqueued must have completed before the new call,
 *     and calls on such handles must not overlap on one device: they would
 *     race on the array. */
zero_status_t zero_shard_init_static(const zero_shard_desc_t* desc, const zero_shard_bufs_t* bufs,
                                     const float* master_init, void* stream, zero_shard_t* out);

/* Chunk-pipelined step ("DeepSpeed ZeRO", ZeRO Stage 1, 通信与计算重叠: the
 * all-gather of updated parameters can start on each part as soon as it is
 * updated, alongside the update of the rest).  The shard's chunks are split
 * into up to 256 contiguous segments; the kernel that writes the 16-bit slice
 * (zero_adam_step with fuse_cast, else zero_cast_params) marks each segment
 * complete on the device as soon as its last element is written, and a consumer
 * stream can wait for one segment and then start that segment's all-gather
 * while later segments are still being updated.  A skipped step marks every
 * segment complete at once (nothing is written).  While segments are tracked
 * the fused write-back walks the shard from its first segment, so segments
 * complete roughly in order (without them the Adam pass may start at the end
 * of a large shard, where the intake left part of its input in the cache). */

/* Splits the write-back into min(n_segments, num_chunks) segments of equal
 * chunk counts (0 turns tracking off; the default).  Between steps only
 * (ESTATE otherwise); EINVAL unless 0 <= n_segments <= 256.  *out_segments
 * (nullable) receives the number of segments. */
zero_status_t zero_set_segments(zero_shard_t h, int32_t n_segments, int32_t* out_segments);

/* Segment k covers the logical shard elements [*shard_begin, *shard_begin +
 * *len) (valid elements only; flat model index = shard_begin of the shard plus
 * these).  EINVAL if there is no segment k. */
zero_status_t zero_segment_range(zero_shard_t h, int32_t k, int64_t* shard_begin, int64_t* len);

/* Enqueues on `stream` a wait that ends when segment k of the latest step's
 * 16-bit write-back is complete; work enqueued after it on `stream` sees the
 * segment's 16-bit parameters of that step.  `stream` first waits (event) until
 * the step's own stream reaches the write-back kernel; then one polling lane
 * watches the segment's flag.  Call it after the write-back was enqueued with
 * segments on (ESTATE otherwise), typically on a stream other than the
 * step's.  If the segment is not complete within about 2 s of polling the wait
 * gives up and the count returned by zero_segment_timeouts increases (work
 * after it then runs without that segment's guarantee).  Each wait polls on
 * its own; an earlier timeout does not shorten later waits. */
zero_status_t zero_wait_segment(zero_shard_t h, int32_t k, void* stream);

/* Number of segment waits that gave up since init (synchronises the stream). */
zero_status_t zero_segment_timeouts(zero_shard_t h, int64_t* timeouts, void* stream);

/* Dynamic loss scale kept on the device ("DeepSpeed ZeRO" 配置说明: fp16.loss_scale
 * = 0 selects dynamic scaling, starting at 2^initial_scale_power).  The pages give
 * no update rule; the one applied, by zero_adam_step on the device, is: after a
 * skipped (overflow) step scale = max(scale * backoff_factor, min_scale) and the
 * good-step count restarts; after growth_interval consecutive good steps scale =
 * scale * growth_factor and the count restarts. */
typedef struct {
  float init_scale;       /* e.g. 65536 = 2^16                      */
  float growth_factor;    /* >= 1, e.g. 2                           */
  float backoff_factor;   /* in (0, 1], e.g. 0.5                    */
  int32_t growth_interval;/* good steps before growing, >= 1        */
  float min_scale;        /* floor of the scale, > 0, e.g. 1        */
} zero_loss_scaler_t;

/* Value of inv_loss_scale for zero_reduce_grads: unscale by 1 / the
 * device-resident dynamic scale (fp32), as zero_adam_step last left it. */
#define ZERO_DEVICE_LOSS_SCALE 0.0f

/* Switches this handle to the device-resident dynamic loss scale, starting at
 * cfg->init_scale.  Between steps only (ESTATE otherwise).  Afterwards every
 * zero_reduce_grads must pass ZERO_DEVICE_LOSS_SCALE.  Synchronises the
 * stream.  EINVAL on an invalid configuration. */
zero_status_t zero_enable_dynamic_loss_scale(zero_shard_t h, const zero_loss_scaler_t* cfg, void* stream);

/* The current dynamic loss scale (what the next step's backward should scale
 * the loss by) and the count of good steps since it last changed.  Synchronises
 * the stream.  ESTATE if dynamic scaling is not enabled. */
zero_status_t zero_loss_scale(zero_shard_t h, float* host_scale, int32_t* host_good, void* stream);

/* Gradient accumulation ("DeepSpeed ZeRO", ZeRO Stage 2 under gradient
 * accumulation: every micro-step's backward is reduce-scattered and the rank
 * adds its 1/N_d slice to what it has accumulated).  Sources as in
 * zero_reduce_grads (0: the registered gradient, 1: a flat already-reduced
 * gradient, N_d: the ranks' buffers); s = their rank-order fp32 sum on this
 * shard; the first micro-step of a step sets acc = s, later ones acc = acc + s,
 * with acc in bufs.red (required).  No statistics.  The step then calls
 * zero_reduce_grads, which adds its own sources (the last micro-step) to acc,
 * or, with n_ranks = ZERO_ACCUMULATED, uses acc as it is, before unscaling.
 * ESTATE after the step's zero_reduce_grads or with a cast pending; EINVAL on
 * an n_ranks other than 0, 1 or N_d (dp_size), null pointers, or without
 * bufs.red. */
zero_status_t zero_accumulate_grads(zero_shard_t h, const void* const* rank_grads, int32_t n_ranks, void* stream);

/* 16-bit output of the local reduce ("DeepSpeed ZeRO", ZeRO Stage 2 基本思想:
 * the rank's fp32 gradient shard is taken from the reduce-scatter's bf16
 * result).  With out_16bit = 1, the rank-order fp32 sum of N_d >= 2 rank
 * buffers (zero_reduce_grads, zero_accumulate_grads) is delivered rounded once,
 * to nearest even, in the handle's 16-bit dtype, and the step takes that
 * value in: without accumulation the 16-bit result is stored in bufs.red
 * (2 bytes per element of the state layout) and the unscale, flag, sum of
 * squares and Adam read it (for fp16 a sum beyond 65504 becomes inf and skips
 * the step); with accumulation each micro-step's rounded result is added to
 * the fp32 accumulator.  Sources of one already-reduced buffer are 16-bit
 * already and are taken in unchanged.  out_16bit = 0 (the default) keeps the
 * fp32 sum.  Between steps only (ESTATE otherwise, also while micro-steps are
 * accumulated); EINVAL unless out_16bit is 0 or 1, or for 1 without bufs.red.
 * While bufs.red holds a 16-bit intake (until the next micro-step or intake),
 * zero_export_state of red (3) returns ESTATE. */
zero_status_t zero_set_reduce_output(zero_shard_t h, int32_t out_16bit);

/* n_ranks value for zero_reduce_grads: no new gradient, use the accumulated one. */
#define ZERO_ACCUMULATED (-1)

/* Gradient intake of one step: the local reduce, the unscale, and this rank's
 * overflow flag and sum of squares, in one pass over the gradient.
 *   n_ranks == 0: use the already-reduced gradient registered at init
 *                 (grad16 or flat_grad16); rank_grads is ignored.
 *   n_ranks == 1: rank_grads[0] is an already-reduced flat 16-bit gradient
 *                 [psi] (the ZeRO-1 all-reduce result); only this rank's slice
 *                 is read.  It must stay unchanged until zero_adam_step.
 *   n_ranks == N_d >= 2: rank_grads[q] is rank q's flat 16-bit gradient [psi];
 *                 this rank's slice is summed in fp32 in rank order
 *                 g_0 + g_1 + ... + g_{N_d-1} (the local half of the
 *                 reduce-scatter, "DeepSpeed ZeRO" ZeRO Stage 2) and the
 *                 unscaled sum is kept in bufs.red (or, after
 *                 zero_set_reduce_output(h, 1), the sum rounded to 16 bits).
 *                 N_d <= 64.
 *   after zero_accumulate_grads: the sources above (or none, n_ranks =
 *                 ZERO_ACCUMULATED) are added to the accumulated gradient in
 *                 bufs.red first: acc + s.  With N_d >= 2 rank buffers u is
 *                 stored in bufs.red; with one source or none bufs.red keeps
 *                 acc, and zero_adam_step recomputes u = (acc + s) * inv with
 *                 the same fp32 operations (so the source, registered or
 *                 rank_grads[0], must stay unchanged until zero_adam_step).
 * u = gradient * inv_loss_scale (fp32), or gradient * (1 / device scale) with
 * ZERO_DEVICE_LOSS_SCALE; flag = any u not finite; sum of squares = sum of u*u
 * in fp64.  rank_grads is a host array of device pointers.  EINVAL on an
 * n_ranks other than 0, 1, N_d (dp_size) or ZERO_ACCUMULATED, on null
 * pointers, or on an inv_loss_scale that is not finite and positive
 * (or, with dynamic scaling, not ZERO_DEVICE_LOSS_SCALE); ESTATE if the previous
 * step's cast is still pending, or for ZERO_ACCUMULATED with nothing
 * accumulated. */
zero_status_t zero_reduce_grads(zero_shard_t h, const void* const* rank_grads, int32_t n_ranks,
                                float inv_loss_scale, void* stream);

/* This rank's local overflow flag and fp64 sum of squares from the last
 * zero_reduce_grads, for the caller's exchange with the other ranks.
 * Synchronises the stream.  ESTATE before a zero_reduce_grads. */
zero_status_t zero_local_stats(zero_shard_t h, int32_t* found_inf, double* sumsq, void* stream);

/* Device addresses, inside the workspace and fixed for the handle's lifetime,
 * of where zero_reduce_grads leaves this rank's fp64 sum of squares and its
 * int32 overflow flag (0 or 1).  For a step that never waits on the host, the
 * exchange with the other ranks can happen in place on the device: after
 * zero_reduce_grads, all-reduce *sumsq (sum) and *found_inf (max, or sum) across
 * the ranks on the step's stream, then pass other_ranks_found_inf = 0 and
 * other_ranks_sumsq = 0; zero_adam_step then takes the skip, norm and clip from
 * the global values.  (The pages exchange these scalars to decide the skip,
 * "DeepSpeed ZeRO" 权重更新的触发条件; the library fixes no transport.)  EINVAL
 * on null arguments. */
zero_status_t zero_local_stats_device(zero_shard_t h, double** sumsq, int32_t** found_inf);

/* Global overflow decision: this rank's flag OR other_ranks_found_inf (the
 * other ranks' flags, combined by the caller).  If host_found_inf is non-NULL
 * the stream is synchronised and the global flag stored there.  A set flag
 * makes zero_adam_step and zero_cast_params change nothing ("DeepSpeed ZeRO"
 * 权重更新的触发条件). */
zero_status_t zero_check_overflow(zero_shard_t h, int32_t other_ranks_found_inf, int32_t* host_found_inf,
                                  void* stream);

/* Global L2 norm and clip over the whole model's unscaled, reduced gradient, as
 * if it were one flat buffer (the codezrq ZeRO optimizer page, 一. 优化前,
 * Temporary buffers: gradient-norm computation runs over all parameters fused
 * into one buffer; here each rank contributes its shard's sum of squares).
 * norm = sqrt(this rank's local sum of squares + other_ranks_sumsq); the clip
 * coefficient is max_norm / (norm + 1e-6) when that is below 1, else 1;
 * max_norm <= 0 disables clipping (the pages give no clipping rule; this is
 * the common one).  The device computes it in fp64 when zero_adam_step runs; a
 * set overflow flag skips the step regardless.  If host_norm is non-NULL the
 * stream is synchronised and the norm stored there.  Launches nothing.
 * Since ranks add the same terms in different orders here, the rounding of the
 * global sum can differ between ranks; zero_grad_norm_global avoids that.
 * ESTATE unless it follows zero_check_overflow. */
zero_status_t zero_grad_norm(zero_shard_t h, double other_ranks_sumsq, float max_norm, double* host_norm,
                             void* stream);

/* As zero_grad_norm, but from the global sum of squares: norm =
 * sqrt(global_sumsq), where global_sumsq is the sum over all N_d ranks of their
 * local sums (zero_local_stats), formed once by the caller -- in rank order,
 * 0 + ss_0 + ss_1 + ... -- and given to every rank, so that every rank takes
 * the same clip coefficient by construction, as the partition-invariance of the
 * update requires ("DeepSpeed ZeRO", ZeRO Stage 2 数学推导: the shards' updates
 * together make the unpartitioned update).  This rank's own sum is not added
 * again (a non-finite local sum, from a non-finite gradient, makes the global
 * sum non-finite, and the overflow flag skips the step).  host_norm (nullable)
 * receives the norm without a synchronisation.  EINVAL if global_sumsq is
 * negative; ESTATE unless it follows zero_check_overflow. */
zero_status_t zero_grad_norm_global(zero_shard_t h, double global_sumsq, float max_norm, double* host_norm,
                                    void* stream);

/* Adam on this rank's fp32 master, m and v ("DeepSpeed ZeRO" ZeRO Stage 1,
 * 以 AdaW 为例), with bias correction and decoupled weight decay.  Unless the
 * step is skipped: t += 1, beta^t advance as fp64 running products,
 * bc = 1 - beta^t rounded to fp32, and per element (fp32, each operation
 * rounded to nearest even, no fused multiply-add):
 *   g = u * clip; m = b1 m + (1-b1) g; v = b2 v + (1-b2) g g;
 *   w = w - lr * ((m / bc1) / (sqrt(v / bc2) + eps) + wd * w).
 * The skip decision is read on the device; a skipped step writes nothing.
 * fuse_cast != 0 also writes the 16-bit parameters in the same pass (then
 * zero_cast_params is a no-op).  EINVAL on a null hparams pointer. */
zero_status_t zero_adam_step(zero_shard_t h, const zero_adam_hparams_t* hp, int32_t fuse_cast, void* stream);

/* In-place write-back p16 = round-to-nearest-even(master) of this rank's
 * valid elements ("DeepSpeed ZeRO" 权重更新的触发条件, step 4: fp32 copied
 * into fp16 in place); nothing outside the shard is touched, nothing at all
 * after a skipped step.  fp16: IEEE binary16 with subnormals, overflow to
 * +-inf; bf16: the top half of the binary32, rounded.  Every NaN master value,
 * whatever its sign and payload, is written as the format's positive
 * canonical quiet NaN (0x7E00, 0x7FC0): IEEE 754 leaves an arithmetic NaN's
 * sign and payload open and machines differ, so keeping them would make the
 * written bits machine-dependent.  The same encoding serves the fused cast of
 * zero_adam_step.  No-op when the step fused the cast. */
zero_status_t zero_cast_params(zero_shard_t h, void* stream);

/* Plan sizes of an initialised handle. */
zero_status_t zero_shard_info(zero_shard_t h, zero_shard_info_t* out);

/* The state layout: for each piece p < min(num_pieces, cap), out[5p .. 5p+4] =
 * {tensor index, offset in tensor, offset in shard (logical), offset in the
 * state buffers, length}.  Host memory. */
zero_status_t zero_shard_pieces(zero_shard_t h, int64_t* out, int64_t cap);

/* Applied steps t, whether the last zero_adam_step skipped, and the global
 * norm and clip coefficient it used.  Synchronises the stream. */
zero_status_t zero_shard_query(zero_shard_t h, int64_t* t, int32_t* last_skipped, double* last_norm,
                               float* last_clip, void* stream);

/* Copies state buffer `which` (0 master, 1 m, 2 v, 3 red) of this shard into
 * dst (device fp32 [valid_elems]) in logical order.  ESTATE for red while it
 * holds a 16-bit intake (zero_set_reduce_output). */
zero_status_t zero_export_state(zero_shard_t h, int32_t which, float* dst, void* stream);

/* Frees the host handle (never caller memory). */
zero_status_t zero_shard_destroy(zero_shard_t h);

/* Message of the last failed call on this thread ("" if none). */
const char* zero_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_SHARD_H */
