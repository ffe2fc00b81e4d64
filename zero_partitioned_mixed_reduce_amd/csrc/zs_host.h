// Host-only internals shared by the library's C ABI sources.
#pragma once
#include <hip/hip_runtime_api.h>

#include <string>

#include "zero_shard.h"
#include "zs_internal.h"

namespace zs {

// Sets the calling thread's message for zero_last_error() and returns s.
zero_status_t set_error(zero_status_t s, const std::string& msg);

}  // namespace zs

// Kernel launchers (kernels.hip).
namespace zs {
hipError_t launch_stats16(int dtype, const Chunk* chunks, int64_t n_chunks, int64_t slice_elems,
                          const uint16_t* flat_g, float inv, bool dyn, bool flip, DevScalars* sc,
                          const IntakeParts& parts, hipStream_t st);
hipError_t launch_reduce(int dtype, const Chunk* chunks, int64_t n_chunks, int64_t slice_elems, const void* const* ranks,
                         int32_t n_ranks, bool accumulate, bool r16, bool keep_acc, float inv, bool dyn, bool flip,
                         float* red, DevScalars* sc, const IntakeParts& parts, hipStream_t st);
hipError_t launch_accumulate(int dtype, const Chunk* chunks, int64_t n_chunks, const void* const* ranks,
                             int32_t n_ranks, bool first, bool r16, float* red, int64_t grid_cap, hipStream_t st);
struct AdamArgs;
hipError_t launch_cast(int dtype, const Chunk* chunks, int64_t n_chunks, const float* master,
                       const DevScalars* sc, const SegArgs* seg, int64_t grid_cap, hipStream_t st);
hipError_t launch_seg_wait(const SegState* seg, int32_t k, uint64_t epoch, int64_t max_polls, DevScalars* sc,
                           hipStream_t st);
hipError_t launch_init(int dtype, const Chunk* chunks, int64_t n_chunks, float* master, float* m, float* v,
                       int64_t state_elems, const float* master_init, int64_t grid_cap, hipStream_t st);
hipError_t launch_export(const Chunk* chunks, int64_t n_chunks, const float* src, float* dst, int64_t grid_cap,
                         hipStream_t st);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st);
hipError_t launch_adam_step(int dtype, int grad_source, bool cast, const Chunk* chunks, int64_t n_chunks,
                            int64_t slice_elems, const uint16_t* flat_g, const float* red, float* master, float* m,
                            float* v, DevScalars* sc, int32_t other_flag, double other_sumsq, bool sumsq_global,
                            float max_norm, float inv, const zero_adam_hparams_t* hp, const zero_loss_scaler_t* dyn,
                            const SegArgs* seg, int64_t grid_cap, hipStream_t st);
}  // namespace zs
