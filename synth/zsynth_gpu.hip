// Device filler for the counter-based synthetic inputs (same definitions as the
// host filler; see zsynth_core.h).  Used by tests and the benchmark to create
// multi-gigabyte inputs directly in HBM.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "zsynth_core.h"

namespace {

__global__ void __launch_bounds__(256) fill_f32_kernel(float* out, int64_t n, uint64_t key, int64_t first,
                                                       double sigma) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
    out[j] = (float)(zs_std(key, (uint64_t)(first + j)) * sigma);
}

__global__ void __launch_bounds__(256) fill_16_kernel(uint16_t* out, int64_t n, int dtype, uint64_t key,
                                                      int64_t first, double sigma, uint64_t zkey,
                                                      uint32_t zero_mod) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride) {
    uint64_t idx = (uint64_t)(first + j);
    out[j] = zs_is_zero(zkey, idx, zero_mod) ? (uint16_t)0 : zs_value16(key, idx, sigma, dtype);
  }
}

unsigned grid_for(int64_t n) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  return (unsigned)blocks;
}

}  // namespace

extern "C" int zs_gpu_fill_f32(float* out, int64_t n, uint64_t seed, uint64_t stream, int64_t first,
                               double sigma, hipStream_t s) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(n)), dim3(256), 0, s, out, n, zs_key(seed, stream), first,
                     sigma);
  return (int)hipGetLastError();
}

extern "C" int zs_gpu_fill_16(uint16_t* out, int64_t n, int dtype, uint64_t seed, uint64_t stream,
                              int64_t first, double sigma, uint64_t zero_seed, uint32_t zero_mod,
                              hipStream_t s) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(fill_16_kernel, dim3(grid_for(n)), dim3(256), 0, s, out, n, dtype, zs_key(seed, stream),
                     first, sigma, zs_mix64(zero_seed), zero_mod);
  return (int)hipGetLastError();
}
