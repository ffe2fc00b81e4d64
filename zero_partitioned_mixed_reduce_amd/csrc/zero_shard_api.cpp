// C ABI of one data-parallel rank's partitioned mixed-precision optimizer step.
// Host side: argument checks, the step-order state machine, the device scalar
// block and kernel launches.  The arithmetic is in kernels.hip.
#include <hip/hip_runtime.h>
#include <math.h>

#include <cmath>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "zero_shard.h"
#include "zs_host.h"
#include "zs_internal.h"


namespace {

thread_local std::string g_err;

zero_status_t fail(zero_status_t s, const std::string& msg) {
  g_err = msg;
  return s;
}

zero_status_t hip_fail(const char* what, hipError_t e) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return ZERO_EHIP;
}

#define ZS_HIP(call)                              \
  do {                                            \
    hipError_t e_ = (call);                       \
    if (e_ != hipSuccess) return hip_fail(#call, e_); \
  } while (0)

enum Phase { kReady, kReduced, kChecked, kNormed, kStepped };
using zs::kGradAcc;
using zs::kGradAccChunk16;
using zs::kGradAccFlat16;
using zs::kGradChunk16;
using zs::kGradFlat16;
using zs::kGradRed;
using zs::kGradRed16;

}  // namespace

zero_status_t zs::set_error(zero_status_t s, const std::string& msg) { return fail(s, msg); }

struct zero_shard {
  zero_shard_info_t info;
  std::vector<zs::Piece> pieces;
  int dtype;
  int device;
  bool has_registered_grads;
  float *master, *m, *v, *red;
  zs::DevScalars* sc;
  zs::IntakeParts parts;       // partial sums of the intake passes (workspace)
  zs::Chunk* chunks;
  int64_t n_chunks;
  std::vector<int64_t> chunk_begin;  // logical shard offset of each chunk, plus the end
  zs::SegState* seg;
  int32_t n_seg;                     // segments of the write-back (0: not tracked)
  int64_t seg_per;                   // chunks per segment
  bool seg_tracked;                  // the latest write-back tracked the current segments
  hipEvent_t wb_event;               // recorded just before each tracked write-back launch
  int64_t grid_main;
  Phase phase;
  bool cast_pending;
  bool accumulating;   // micro-steps summed into red since the last intake
  bool reduce_out16;   // the local reduce delivers its sum in the 16-bit type
  bool red_holds16;    // red holds the last intake's 16-bit reduce output (not fp32 values)
  int64_t dp_size;
  bool dynamic;        // device-resident dynamic loss scale enabled
  zero_loss_scaler_t dyn_cfg;
  // current step
  int grad_source;
  const uint16_t* step_flat_g;
  float inv;
  int32_t other_flag;
  double other_sumsq;  // the other ranks' sum of squares, or (sumsq_global) the global sum
  bool sumsq_global;   // zero_grad_norm_global: other_sumsq is the global sum, the local one is not added
  float max_norm;
  int64_t adam_calls;  // zero_adam_step calls (the segments' epoch)
  uint64_t static_gen; // 0: caller workspace; else which zero_shard_init_static on this device made it
};

namespace {

struct DeviceGuard {
  int prev = -1;
  bool changed = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) == hipSuccess && prev != dev) changed = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    if (changed) (void)hipSetDevice(prev);
  }
};

// Grid cap of the streaming kernels, in blocks per CU.  The default leaves the
// grid at one block per work item (the hardware dispatcher balances the load);
// ZERO_SHARD_BLOCKS_PER_CU caps it to make the kernels persistent instead.
int64_t blocks_per_cu() {
  const char* e = getenv("ZERO_SHARD_BLOCKS_PER_CU");
  if (e) {
    long v = strtol(e, nullptr, 10);
    if (v >= 1 && v <= 65536) return v;
  }
  return 65536;
}

// Between an intake and its zero_adam_step (the device has flipped cur_slot).
bool in_step(const zero_shard* h) { return h->phase == kReduced || h->phase == kChecked || h->phase == kNormed; }

// The slot holding the latest step counters (see DevScalars).
const zs::Slot& latest_slot(const zero_shard* h, const zs::DevScalars& sc) {
  return sc.slot[in_step(h) ? sc.cur_slot & 1u : (sc.cur_slot & 1u) ^ 1u];
}

zero_status_t sync_read_scalars(zero_shard* h, hipStream_t st, zs::DevScalars* out) {
  ZS_HIP(hipStreamSynchronize(st));
  ZS_HIP(hipMemcpy(out, h->sc, sizeof(zs::DevScalars), hipMemcpyDeviceToHost));
  return ZERO_OK;
}

// The library's own workspace for handles made by zero_shard_init_static (for callers that
// cannot allocate device memory).  Each device holds its own copy of the array, at its own
// address, until the process ends.  In host code the array's name is only a host-side
// stand-in: the device address comes from hipGetSymbolAddress (static_workspace below), and
// only that address is ever handed to kernels or copies.
static_assert(ZERO_STATIC_WORKSPACE_BYTES % 256 == 0, "static workspace size");
__device__ __align__(256) static unsigned char scratch[ZERO_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices];     // device address of `scratch` on each device (null until looked up)
uint64_t g_static_gen[kMaxDevices];  // zero_shard_init_static calls on each device

// Takes the static workspace of device `dev` (the current device) for a new handle: looks up
// its device address on the first call on that device, and advances the device's generation,
// which retires every earlier handle on it.
zero_status_t static_workspace(int dev, char** ws, uint64_t* gen) {
  if (dev < 0 || dev >= kMaxDevices) return fail(ZERO_EINVAL, "device index beyond the static workspaces");
  std::lock_guard<std::mutex> lk(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail("hipGetSymbolAddress(static workspace)", e);
    if (!ptr || ((uintptr_t)ptr & 255u) != 0) return fail(ZERO_EHIP, "static workspace address is not 256-byte aligned");
    g_static_ptr[dev] = ptr;
  }
  *ws = static_cast<char*>(g_static_ptr[dev]);
  *gen = ++g_static_gen[dev];
  return ZERO_OK;
}

// A handle on the static workspace is usable until the next zero_shard_init_static on its device.
zero_status_t check_workspace(const zero_shard* h) {
  if (h->static_gen == 0) return ZERO_OK;
  std::lock_guard<std::mutex> lk(g_static_mu);
  if (g_static_gen[h->device] != h->static_gen)
    return fail(ZERO_ESTATE, "this handle's static workspace was taken over by a later zero_shard_init_static "
                             "on the same device");
  return ZERO_OK;
}

#define ZS_OWNER(h)                             \
  do {                                          \
    zero_status_t o_ = check_workspace(h);      \
    if (o_ != ZERO_OK) return o_;               \
  } while (0)

}  // namespace

extern "C" {

const char* zero_last_error(void) { return g_err.c_str(); }

}  // extern "C"

namespace {

zero_status_t shard_plan(const zero_shard_desc_t* desc, zero_shard_info_t* out) {
  if (!out) return fail(ZERO_EINVAL, "null output");
  zs::Plan p;
  zero_status_t s = zs::build_plan(desc, &p, &g_err);
  if (s != ZERO_OK) return s;
  *out = p.info;
  return ZERO_OK;
}

// zero_shard_init (use_static false: the caller's workspace) and zero_shard_init_static (the
// library's static workspace of the current device).
zero_status_t shard_init(const zero_shard_desc_t* desc, const zero_shard_bufs_t* bufs, const float* master_init,
                         void* stream, zero_shard_t* out, bool use_static) {
  if (!bufs || !out) return fail(ZERO_EINVAL, "null buffers or output handle");
  *out = nullptr;
  zs::Plan p;
  zero_status_t s = zs::build_plan(desc, &p, &g_err);
  if (s != ZERO_OK) return s;
  if (!bufs->master || !bufs->m || !bufs->v) return fail(ZERO_EINVAL, "master, m and v must be non-null");
  auto mis16 = [](const void* q) { return ((uintptr_t)q & 15u) != 0; };
  if (mis16(bufs->master) || mis16(bufs->m) || mis16(bufs->v) || (bufs->red && mis16(bufs->red)))
    return fail(ZERO_EINVAL, "state buffers must be 16-byte aligned");
  if (bufs->state_capacity < p.info.state_elems)
    return fail(ZERO_EINVAL, "state_capacity " + std::to_string(bufs->state_capacity) + " < state_elems " +
                                 std::to_string(p.info.state_elems));
  if (use_static) {
    if (bufs->workspace) return fail(ZERO_EINVAL, "zero_shard_init_static takes no workspace: bufs->workspace "
                                                  "must be NULL");
    if (p.info.workspace_bytes > (int64_t)ZERO_STATIC_WORKSPACE_BYTES)
      return fail(ZERO_EINVAL, "the shard needs a workspace of " + std::to_string(p.info.workspace_bytes) +
                                   " bytes, beyond the static workspace of " +
                                   std::to_string((int64_t)ZERO_STATIC_WORKSPACE_BYTES) +
                                   " bytes (ZERO_STATIC_WORKSPACE_BYTES); use zero_shard_init with a workspace");
  } else {
    if (!bufs->workspace) return fail(ZERO_EINVAL, "workspace must be non-null");
    if (((uintptr_t)bufs->workspace & 255u) != 0) return fail(ZERO_EINVAL, "workspace must be 256-byte aligned");
    if (bufs->workspace_capacity < p.info.workspace_bytes)
      return fail(ZERO_EINVAL, "workspace_capacity " + std::to_string(bufs->workspace_capacity) +
                                   " < workspace_bytes " + std::to_string(p.info.workspace_bytes));
  }
  if (master_init && mis16(master_init)) return fail(ZERO_EINVAL, "master_init must be 16-byte aligned");

  hipStream_t st = static_cast<hipStream_t>(stream);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  int cus = 0;
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice/hipDeviceGetAttribute", e);
  char* ws = static_cast<char*>(bufs->workspace);
  uint64_t gen = 0;
  if (use_static) {
    s = static_workspace(dev, &ws, &gen);
    if (s != ZERO_OK) return s;
  }
  zero_shard* h = new (std::nothrow) zero_shard();
  if (!h) return fail(ZERO_ENOMEM, "out of host memory");
  h->static_gen = gen;
  h->info = p.info;
  h->pieces = std::move(p.pieces);
  h->dtype = desc->dtype;
  h->device = dev;
  h->has_registered_grads = desc->grad16 || desc->flat_grad16;
  h->master = bufs->master;
  h->m = bufs->m;
  h->v = bufs->v;
  h->red = bufs->red;
  h->sc = reinterpret_cast<zs::DevScalars*>(ws);
  const zs::IntakeLayout il = zs::intake_layout((int64_t)p.chunks.size());
  h->parts.part = reinterpret_cast<uint64_t*>(ws + il.part_off);
  h->parts.gcount = reinterpret_cast<zs::GroupCount*>(ws + il.gcount_off);
  h->parts.gpart = reinterpret_cast<uint64_t*>(ws + il.gpart_off);
  h->chunks = reinterpret_cast<zs::Chunk*>(ws + zs::kChunksOff);
  h->n_chunks = (int64_t)p.chunks.size();
  h->seg = reinterpret_cast<zs::SegState*>(ws + zs::kSegOff);
  h->n_seg = 0;
  h->seg_per = 1;
  h->seg_tracked = false;
  h->wb_event = nullptr;
  h->chunk_begin.resize(p.chunks.size() + 1);
  for (size_t c = 0; c < p.chunks.size(); ++c) h->chunk_begin[c] = p.chunks[c].shard_off;
  h->chunk_begin[p.chunks.size()] = p.chunks.empty() ? 0 : p.chunks.back().shard_off + p.chunks.back().len;
  h->grid_main = (int64_t)cus * blocks_per_cu();
  h->phase = kReady;
  h->cast_pending = false;
  h->accumulating = false;
  h->reduce_out16 = false;
  h->red_holds16 = false;
  h->dp_size = desc->dp_size;
  h->dynamic = false;
  memset(&h->dyn_cfg, 0, sizeof(h->dyn_cfg));
  h->adam_calls = 0;

  zs::DevScalars init_sc;
  memset(&init_sc, 0, sizeof(init_sc));
  init_sc.slot[0] = zs::Slot{0, 1.0, 1.0, 1.0f, 0};
  init_sc.slot[1] = zs::Slot{0, 1.0, 1.0, 1.0f, 0};
  init_sc.clip = 1.0f;
  zero_status_t rs = ZERO_OK;
  do {
    if ((e = hipMemcpyAsync(h->sc, &init_sc, sizeof(init_sc), hipMemcpyHostToDevice, st)) != hipSuccess) {
      rs = hip_fail("hipMemcpyAsync(scalars)", e);
      break;
    }
    static const zs::SegState zero_segs[zs::kMaxSegments] = {};
    if ((e = hipMemcpyAsync(h->seg, zero_segs, sizeof(zero_segs), hipMemcpyHostToDevice, st)) != hipSuccess) {
      rs = hip_fail("hipMemcpyAsync(segments)", e);
      break;
    }
    if (!p.chunks.empty() &&
        (e = hipMemcpyAsync(h->chunks, p.chunks.data(), p.chunks.size() * sizeof(zs::Chunk), hipMemcpyHostToDevice,
                            st)) != hipSuccess) {
      rs = hip_fail("hipMemcpyAsync(chunk table)", e);
      break;
    }
    // the intake passes' group counters start at zero (and are re-armed by every pass)
    const int64_t n_groups = zs::intake_groups(h->n_chunks);
    if ((e = zs::launch_fill_zero(reinterpret_cast<float*>(h->parts.gcount),
                                  n_groups * (int64_t)(sizeof(zs::GroupCount) / sizeof(float)), st)) != hipSuccess) {
      rs = hip_fail("group counters", e);
      break;
    }
    if ((e = zs::launch_init(h->dtype, h->chunks, h->n_chunks, h->master, h->m, h->v, h->info.state_elems,
                             master_init, h->grid_main, st)) != hipSuccess) {
      rs = hip_fail("init kernels", e);
      break;
    }
    if ((e = hipStreamSynchronize(st)) != hipSuccess) {
      rs = hip_fail("hipStreamSynchronize(init)", e);
      break;
    }
  } while (0);
  if (rs != ZERO_OK) {
    // copies already enqueued may still read init_sc and the plan's chunk table
    (void)hipStreamSynchronize(st);
    if (h->wb_event) (void)hipEventDestroy(h->wb_event);
    delete h;
    return rs;
  }
  *out = h;
  return ZERO_OK;
}

}  // namespace

extern "C" {

// The plan's host tables may not fit in host memory: no exception leaves the C ABI.
zero_status_t zero_shard_plan(const zero_shard_desc_t* desc, zero_shard_info_t* out) {
  try {
    return shard_plan(desc, out);
  } catch (const std::exception& e) {
    return fail(ZERO_ENOMEM, std::string("host resources: ") + e.what());
  }
}

zero_status_t zero_shard_init(const zero_shard_desc_t* desc, const zero_shard_bufs_t* bufs,
                              const float* master_init, void* stream, zero_shard_t* out) {
  try {
    return shard_init(desc, bufs, master_init, stream, out, false);
  } catch (const std::exception& e) {
    return fail(ZERO_ENOMEM, std::string("host resources: ") + e.what());
  }
}

zero_status_t zero_shard_init_static(const zero_shard_desc_t* desc, const zero_shard_bufs_t* bufs,
                                     const float* master_init, void* stream, zero_shard_t* out) {
  try {
    return shard_init(desc, bufs, master_init, stream, out, true);
  } catch (const std::exception& e) {
    return fail(ZERO_ENOMEM, std::string("host resources: ") + e.what());
  }
}

namespace {
// Checks a gradient source list: 0 (registered), 1 (flat, already reduced) or the N_d rank
// buffers (2 <= N_d <= 64): summing fewer or more buffers than there are ranks is an error.
zero_status_t check_sources(zero_shard* h, const void* const* rank_grads, int32_t n_ranks) {
  if (n_ranks == 0) {
    if (!h->has_registered_grads) return fail(ZERO_EINVAL, "n_ranks == 0 needs gradients registered at init");
    return ZERO_OK;
  }
  if (n_ranks < 0 || n_ranks > zs::kMaxRanks) return fail(ZERO_EINVAL, "n_ranks must be 0..64");
  if (n_ranks >= 2 && n_ranks != h->dp_size)
    return fail(ZERO_EINVAL, "the local reduce takes one buffer per rank: n_ranks " + std::to_string(n_ranks) +
                                 " != dp_size " + std::to_string(h->dp_size));
  if (!rank_grads) return fail(ZERO_EINVAL, "rank_grads is null");
  for (int q = 0; q < n_ranks; ++q)
    if (!rank_grads[q]) return fail(ZERO_EINVAL, "rank_grads[" + std::to_string(q) + "] is null");
  return ZERO_OK;
}
}  // namespace

zero_status_t zero_set_reduce_output(zero_shard_t h, int32_t out_16bit) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  ZS_OWNER(h);
  if (out_16bit != 0 && out_16bit != 1) return fail(ZERO_EINVAL, "out_16bit must be 0 or 1");
  if (!(h->phase == kReady || h->phase == kStepped) || h->cast_pending || h->accumulating)
    return fail(ZERO_ESTATE, "the reduce output is set between steps");
  if (out_16bit && !h->red) return fail(ZERO_EINVAL, "the 16-bit reduce output is kept in bufs.red");
  h->reduce_out16 = out_16bit != 0;
  return ZERO_OK;
}

zero_status_t zero_accumulate_grads(zero_shard_t h, const void* const* rank_grads, int32_t n_ranks, void* stream) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  ZS_OWNER(h);
  if (h->phase == kReduced || h->phase == kChecked || h->phase == kNormed)
    return fail(ZERO_ESTATE, "micro-steps are accumulated before the step's zero_reduce_grads");
  if (h->phase == kStepped && h->cast_pending)
    return fail(ZERO_ESTATE, "zero_cast_params of the previous step is pending");
  if (!h->red) return fail(ZERO_EINVAL, "accumulation needs bufs.red");
  zero_status_t s = check_sources(h, rank_grads, n_ranks);
  if (s != ZERO_OK) return s;
  DeviceGuard dg(h->device);
  hipError_t e = zs::launch_accumulate(h->dtype, h->chunks, h->n_chunks, rank_grads, n_ranks, !h->accumulating,
                                       h->reduce_out16, h->red, h->grid_main, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("accumulate kernel", e);
  h->accumulating = true;
  h->red_holds16 = false;
  h->phase = kReady;
  h->cast_pending = false;
  return ZERO_OK;
}

zero_status_t zero_reduce_grads(zero_shard_t h, const void* const* rank_grads, int32_t n_ranks, float inv_loss_scale,
                                void* stream) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  ZS_OWNER(h);
  if (h->phase == kStepped && h->cast_pending)
    return fail(ZERO_ESTATE, "zero_cast_params of the previous step is pending");
  bool dyn = false;
  if (inv_loss_scale == ZERO_DEVICE_LOSS_SCALE) {
    if (!h->dynamic) return fail(ZERO_EINVAL, "ZERO_DEVICE_LOSS_SCALE needs zero_enable_dynamic_loss_scale");
    dyn = true;
  } else if (h->dynamic) {
    return fail(ZERO_EINVAL, "with dynamic loss scaling pass inv_loss_scale = ZERO_DEVICE_LOSS_SCALE");
  } else if (!(inv_loss_scale > 0.0f) || !std::isfinite(inv_loss_scale)) {
    return fail(ZERO_EINVAL, "inv_loss_scale must be finite and positive");
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  DeviceGuard dg(h->device);
  // the step's first intake advances the device-side counter slot (a repeated one does not)
  const bool flip = !in_step(h);
  hipError_t e;
  if (h->accumulating) {
    // last micro-step (or none: ZERO_ACCUMULATED) on top of the accumulated gradient.  From one
    // source or none the pass only takes the statistics: red keeps the accumulator and the Adam
    // pass recomputes u = (acc + g) * inv from it and the (unchanged) source, which moves fewer
    // bytes than storing u and reading it back; from rank buffers u is stored.
    if (n_ranks != ZERO_ACCUMULATED) {
      zero_status_t s = check_sources(h, rank_grads, n_ranks);
      if (s != ZERO_OK) return s;
    }
    const bool keep_acc = n_ranks == 0 || n_ranks == 1 || n_ranks == ZERO_ACCUMULATED;
    e = zs::launch_reduce(h->dtype, h->chunks, h->n_chunks, h->info.valid_elems, rank_grads, n_ranks, true, h->reduce_out16, keep_acc,
                          inv_loss_scale, dyn, flip, h->red, h->sc, h->parts, st);
    if (e != hipSuccess) return hip_fail("reduce kernel", e);
    h->grad_source = !keep_acc ? kGradRed : n_ranks == 0 ? kGradAccChunk16 : n_ranks == 1 ? kGradAccFlat16 : kGradAcc;
    h->step_flat_g = n_ranks == 1 ? static_cast<const uint16_t*>(rank_grads[0]) : nullptr;
    h->accumulating = false;
  } else if (n_ranks == ZERO_ACCUMULATED) {
    return fail(ZERO_ESTATE, "ZERO_ACCUMULATED without zero_accumulate_grads in this step");
  } else if (n_ranks == 0) {
    if (!h->has_registered_grads) return fail(ZERO_EINVAL, "n_ranks == 0 needs gradients registered at init");
    e = zs::launch_stats16(h->dtype, h->chunks, h->n_chunks, h->info.valid_elems, nullptr, inv_loss_scale, dyn, flip,
                           h->sc, h->parts, st);
    if (e != hipSuccess) return hip_fail("statistics kernel", e);
    h->grad_source = kGradChunk16;
    h->step_flat_g = nullptr;
  } else if (n_ranks == 1) {
    if (!rank_grads || !rank_grads[0]) return fail(ZERO_EINVAL, "rank_grads[0] is null");
    const uint16_t* g = static_cast<const uint16_t*>(rank_grads[0]);
    e = zs::launch_stats16(h->dtype, h->chunks, h->n_chunks, h->info.valid_elems, g, inv_loss_scale, dyn, flip,
                           h->sc, h->parts, st);
    if (e != hipSuccess) return hip_fail("statistics kernel", e);
    h->grad_source = kGradFlat16;
    h->step_flat_g = g;
  } else {
    zero_status_t sc = check_sources(h, rank_grads, n_ranks);  // n_ranks < -1 or >= 2 here
    if (sc != ZERO_OK) return sc;
    if (!h->red) return fail(ZERO_EINVAL, "reducing N_d >= 2 buffers needs bufs.red");
    e = zs::launch_reduce(h->dtype, h->chunks, h->n_chunks, h->info.valid_elems, rank_grads, n_ranks, false, h->reduce_out16, false,
                          inv_loss_scale, dyn, flip, h->red, h->sc, h->parts, st);
    if (e != hipSuccess) return hip_fail("reduce kernel", e);
    h->grad_source = h->reduce_out16 ? kGradRed16 : kGradRed;
    h->step_flat_g = nullptr;
  }
  h->red_holds16 = h->grad_source == kGradRed16;
  h->inv = inv_loss_scale;
  h->other_flag = 0;
  h->other_sumsq = 0.0;
  h->sumsq_global = false;
  h->max_norm = 0.0f;
  h->phase = kReduced;
  h->cast_pending = false;
  return ZERO_OK;
}

zero_status_t zero_local_stats(zero_shard_t h, int32_t* found_inf, double* sumsq, void* stream) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  ZS_OWNER(h);
  if (h->phase == kReady || h->phase == kStepped) return fail(ZERO_ESTATE, "no gradient intake in this step yet");
  DeviceGuard dg(h->device);
  zs::DevScalars sc;
  zero_status_t s = sync_read_scalars(h, static_cast<hipStream_t>(stream), &sc);
  if (s != ZERO_OK) return s;
  if (found_inf) *found_inf = sc.local_flag;
  if (sumsq) *sumsq = sc.local_sumsq;
  return ZERO_OK;
}

zero_status_t zero_local_stats_device(zero_shard_t h, double** sumsq, int32_t** found_inf) {
  if (!h || !sumsq || !found_inf) return fail(ZERO_EINVAL, "null handle or output");
  ZS_OWNER(h);
  *sumsq = &h->sc->local_sumsq;
  *found_inf = &h->sc->local_flag;
  return ZERO_OK;
}

zero_status_t zero_check_overflow(zero_shard_t h, int32_t other_ranks_found_inf, int32_t* host_found_inf,
                                  void* stream) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  ZS_OWNER(h);
  if (h->phase != kReduced && h->phase != kChecked)
    return fail(ZERO_ESTATE, "zero_check_overflow must follow zero_reduce_grads");
  h->other_flag = other_ranks_found_inf ? 1 : 0;
  h->phase = kChecked;
  if (host_found_inf) {
    DeviceGuard dg(h->device);
    zs::DevScalars sc;
    zero_status_t s = sync_read_scalars(h, static_cast<hipStream_t>(stream), &sc);
    if (s != ZERO_OK) return s;
    *host_found_inf = (sc.local_flag | h->other_flag) ? 1 : 0;
  }
  return ZERO_OK;
}

namespace {
// The norm call of a step: sumsq is the other ranks' sum (global false) or the global sum.
zero_status_t grad_norm(zero_shard_t h, double sumsq, bool global, float max_norm, double* host_norm, void* stream) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  ZS_OWNER(h);
  if (h->phase != kChecked && h->phase != kNormed)
    return fail(ZERO_ESTATE, "the norm call must follow zero_check_overflow");
  if (global && sumsq < 0.0) return fail(ZERO_EINVAL, "global_sumsq must not be negative");
  h->other_sumsq = sumsq;
  h->sumsq_global = global;
  h->max_norm = max_norm;
  h->phase = kNormed;
  if (host_norm) {
    if (global) {
      *host_norm = sqrt(sumsq);
      return ZERO_OK;
    }
    DeviceGuard dg(h->device);
    zs::DevScalars sc;
    zero_status_t s = sync_read_scalars(h, static_cast<hipStream_t>(stream), &sc);
    if (s != ZERO_OK) return s;
    *host_norm = sqrt(sc.local_sumsq + sumsq);
  }
  return ZERO_OK;
}
}  // namespace

zero_status_t zero_grad_norm(zero_shard_t h, double other_ranks_sumsq, float max_norm, double* host_norm,
                             void* stream) {
  return grad_norm(h, other_ranks_sumsq, false, max_norm, host_norm, stream);
}

zero_status_t zero_grad_norm_global(zero_shard_t h, double global_sumsq, float max_norm, double* host_norm,
                                    void* stream) {
  return grad_norm(h, global_sumsq, true, max_norm, host_norm, stream);
}

namespace {
zs::SegArgs seg_args(const zero_shard* h, int64_t epoch) {
  return zs::SegArgs{h->seg, h->seg_per, h->n_chunks, h->n_seg, (uint64_t)epoch};
}
}  // namespace

zero_status_t zero_adam_step(zero_shard_t h, const zero_adam_hparams_t* hp, int32_t fuse_cast, void* stream) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  ZS_OWNER(h);
  if (!hp) return fail(ZERO_EINVAL, "null hyperparameters");
  if (h->phase != kNormed) return fail(ZERO_ESTATE, "zero_adam_step must follow zero_grad_norm");
  DeviceGuard dg(h->device);
  const zs::SegArgs seg = seg_args(h, h->adam_calls + 1);
  const bool track = h->n_seg > 0 && fuse_cast != 0;
  if (track) ZS_HIP(hipEventRecord(h->wb_event, static_cast<hipStream_t>(stream)));
  hipError_t e = zs::launch_adam_step(h->dtype, h->grad_source, fuse_cast != 0, h->chunks, h->n_chunks,
                                      h->info.valid_elems, h->step_flat_g, h->red, h->master, h->m, h->v, h->sc,
                                      h->other_flag,
                                      h->other_sumsq, h->sumsq_global, h->max_norm,
                                      h->inv, hp, h->dynamic ? &h->dyn_cfg : nullptr, h->n_seg ? &seg : nullptr,
                                      h->grid_main, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("adam kernel", e);
  h->seg_tracked = track;
  h->adam_calls += 1;
  h->phase = kStepped;
  h->cast_pending = fuse_cast == 0;
  return ZERO_OK;
}

zero_status_t zero_cast_params(zero_shard_t h, void* stream) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  ZS_OWNER(h);
  if (h->phase != kStepped) return fail(ZERO_ESTATE, "zero_cast_params must follow zero_adam_step");
  if (!h->cast_pending) return ZERO_OK;
  DeviceGuard dg(h->device);
  const zs::SegArgs seg = seg_args(h, h->adam_calls);
  if (h->n_seg > 0) ZS_HIP(hipEventRecord(h->wb_event, static_cast<hipStream_t>(stream)));
  hipError_t e = zs::launch_cast(h->dtype, h->chunks, h->n_chunks, h->master, h->sc, h->n_seg ? &seg : nullptr,
                                 h->grid_main, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("cast kernel", e);
  h->seg_tracked = h->n_seg > 0;
  h->cast_pending = false;
  return ZERO_OK;
}

zero_status_t zero_set_segments(zero_shard_t h, int32_t n_segments, int32_t* out_segments) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  ZS_OWNER(h);
  if (n_segments < 0 || n_segments > zs::kMaxSegments) return fail(ZERO_EINVAL, "n_segments must be 0..256");
  if (h->phase != kReady && h->phase != kStepped) return fail(ZERO_ESTATE, "set segments between steps");
  if (h->phase == kStepped && h->cast_pending) return fail(ZERO_ESTATE, "zero_cast_params is pending");
  if (n_segments > 0 && h->n_chunks > 0 && !h->wb_event) {
    DeviceGuard dg(h->device);
    ZS_HIP(hipEventCreateWithFlags(&h->wb_event, hipEventDisableTiming));
  }
  // every counter is re-armed once a write-back completes, so the layout may change between steps
  if (n_segments == 0 || h->n_chunks == 0) {
    h->n_seg = 0;
    h->seg_per = 1;
  } else {
    h->seg_per = (h->n_chunks + n_segments - 1) / n_segments;
    h->n_seg = (int32_t)((h->n_chunks + h->seg_per - 1) / h->seg_per);
  }
  h->seg_tracked = false;
  if (out_segments) *out_segments = h->n_seg;
  return ZERO_OK;
}

zero_status_t zero_segment_range(zero_shard_t h, int32_t k, int64_t* shard_begin, int64_t* len) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  if (k < 0 || k >= h->n_seg) return fail(ZERO_EINVAL, "no segment " + std::to_string(k));
  const int64_t c0 = (int64_t)k * h->seg_per;
  const int64_t c1 = c0 + h->seg_per < h->n_chunks ? c0 + h->seg_per : h->n_chunks;
  if (shard_begin) *shard_begin = h->chunk_begin[c0];
  if (len) *len = h->chunk_begin[c1] - h->chunk_begin[c0];
  return ZERO_OK;
}

zero_status_t zero_wait_segment(zero_shard_t h, int32_t k, void* stream) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  ZS_OWNER(h);
  if (k < 0 || k >= h->n_seg) return fail(ZERO_EINVAL, "no segment " + std::to_string(k));
  if (h->adam_calls == 0 || h->phase != kStepped || h->cast_pending)
    return fail(ZERO_ESTATE, "the write-back of this step has not been enqueued");
  if (!h->seg_tracked) return fail(ZERO_ESTATE, "the latest write-back did not track these segments");
  DeviceGuard dg(h->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // The polling lane starts only once the step's stream has reached the write-back kernel, so
  // it spins for at most that kernel's run time; about 2 s of polls (s_sleep 32 is about 2048
  // clocks each) bound it in any case.
  ZS_HIP(hipStreamWaitEvent(st, h->wb_event, 0));
  const int64_t max_polls = 1000000;
  hipError_t e = zs::launch_seg_wait(h->seg, k, (uint64_t)h->adam_calls, max_polls, h->sc,
                                     st);
  if (e != hipSuccess) return hip_fail("segment wait kernel", e);
  return ZERO_OK;
}

zero_status_t zero_segment_timeouts(zero_shard_t h, int64_t* timeouts, void* stream) {
  if (!h || !timeouts) return fail(ZERO_EINVAL, "null handle or output");
  ZS_OWNER(h);
  DeviceGuard dg(h->device);
  zs::DevScalars sc;
  zero_status_t s = sync_read_scalars(h, static_cast<hipStream_t>(stream), &sc);
  if (s != ZERO_OK) return s;
  *timeouts = sc.wait_timeouts;
  return ZERO_OK;
}

zero_status_t zero_enable_dynamic_loss_scale(zero_shard_t h, const zero_loss_scaler_t* cfg, void* stream) {
  if (!h || !cfg) return fail(ZERO_EINVAL, "null handle or configuration");
  ZS_OWNER(h);
  if (h->phase != kReady && h->phase != kStepped) return fail(ZERO_ESTATE, "enable loss scaling between steps");
  if (h->phase == kStepped && h->cast_pending) return fail(ZERO_ESTATE, "zero_cast_params is pending");
  if (h->accumulating) return fail(ZERO_ESTATE, "enable loss scaling before accumulating micro-steps");
  if (!(cfg->init_scale > 0.0f) || !std::isfinite(cfg->init_scale) || !(cfg->growth_factor >= 1.0f) ||
      !(cfg->backoff_factor > 0.0f && cfg->backoff_factor <= 1.0f) || cfg->growth_interval < 1 ||
      !(cfg->min_scale > 0.0f))
    return fail(ZERO_EINVAL, "need init_scale > 0, growth_factor >= 1, 0 < backoff_factor <= 1, "
                             "growth_interval >= 1, min_scale > 0");
  DeviceGuard dg(h->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  struct {
    float scale;
    int32_t good;
  } v = {cfg->init_scale, 0};
  static_assert(sizeof(v) == 8, "scale and good are adjacent in the slot");
  // both slots: whichever holds the latest counters, the next intake finds the scale there
  for (int k = 0; k < 2; ++k)
    ZS_HIP(hipMemcpyAsync(&h->sc->slot[k].scale, &v, sizeof(v), hipMemcpyHostToDevice, st));
  ZS_HIP(hipStreamSynchronize(st));
  h->dynamic = true;
  h->dyn_cfg = *cfg;
  return ZERO_OK;
}

zero_status_t zero_loss_scale(zero_shard_t h, float* host_scale, int32_t* host_good, void* stream) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  ZS_OWNER(h);
  if (!h->dynamic) return fail(ZERO_ESTATE, "dynamic loss scaling is not enabled");
  DeviceGuard dg(h->device);
  zs::DevScalars sc;
  zero_status_t s = sync_read_scalars(h, static_cast<hipStream_t>(stream), &sc);
  if (s != ZERO_OK) return s;
  const zs::Slot& cur = latest_slot(h, sc);
  if (host_scale) *host_scale = cur.scale;
  if (host_good) *host_good = cur.good;
  return ZERO_OK;
}

zero_status_t zero_shard_info(zero_shard_t h, zero_shard_info_t* out) {
  if (!h || !out) return fail(ZERO_EINVAL, "null handle or output");
  *out = h->info;
  return ZERO_OK;
}

zero_status_t zero_shard_pieces(zero_shard_t h, int64_t* out, int64_t cap) {
  if (!h || (!out && cap > 0)) return fail(ZERO_EINVAL, "null handle or output");
  for (int64_t p = 0; p < cap && p < (int64_t)h->pieces.size(); ++p) {
    const zs::Piece& pc = h->pieces[p];
    out[5 * p + 0] = pc.tensor;
    out[5 * p + 1] = pc.tensor_off;
    out[5 * p + 2] = pc.shard_off;
    out[5 * p + 3] = pc.state_off;
    out[5 * p + 4] = pc.len;
  }
  return ZERO_OK;
}

zero_status_t zero_shard_query(zero_shard_t h, int64_t* t, int32_t* last_skipped, double* last_norm,
                               float* last_clip, void* stream) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  ZS_OWNER(h);
  DeviceGuard dg(h->device);
  zs::DevScalars sc;
  zero_status_t s = sync_read_scalars(h, static_cast<hipStream_t>(stream), &sc);
  if (s != ZERO_OK) return s;
  if (t) *t = latest_slot(h, sc).t;
  if (last_skipped) *last_skipped = h->adam_calls ? sc.skipped : 0;
  if (last_norm) *last_norm = sc.norm;
  if (last_clip) *last_clip = sc.clip;
  return ZERO_OK;
}

zero_status_t zero_export_state(zero_shard_t h, int32_t which, float* dst, void* stream) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  ZS_OWNER(h);
  const float* src = which == 0 ? h->master : which == 1 ? h->m : which == 2 ? h->v : which == 3 ? h->red : nullptr;
  if (!src) return fail(ZERO_EINVAL, "which must be 0 (master), 1 (m), 2 (v) or 3 (red, when allocated)");
  if (which == 3 && h->red_holds16)
    return fail(ZERO_ESTATE, "bufs.red holds the last intake's 16-bit reduce output, not fp32 values");
  if (!dst && h->info.valid_elems > 0) return fail(ZERO_EINVAL, "null destination");
  DeviceGuard dg(h->device);
  hipError_t e = zs::launch_export(h->chunks, h->n_chunks, src, dst, h->grid_main, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("export kernel", e);
  return ZERO_OK;
}

zero_status_t zero_shard_destroy(zero_shard_t h) {
  if (h && h->wb_event) (void)hipEventDestroy(h->wb_event);
  delete h;
  return ZERO_OK;
}

}  // extern "C"
