/* Host filler for the counter-based synthetic inputs (see zsynth_core.h). */
#include <stddef.h>
#include <stdint.h>
#include "zsynth_core.h"

#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads for the host fillers: 0 = the OpenMP default (callers that already run
 * several fills in parallel pass 1). */
static int g_threads = 0;
void zs_set_threads(int n) { g_threads = n < 0 ? 0 : n; }
#define ZS_NT (g_threads > 0 ? g_threads : omp_get_max_threads())

/* out[j] = sigma * N(seed, stream, first + j), rounded once to float */
void zs_fill_f32(float* out, int64_t n, uint64_t seed, uint64_t stream, int64_t first, double sigma) {
  uint64_t key = zs_key(seed, stream);
#pragma omp parallel for schedule(static) num_threads(ZS_NT)
  for (int64_t j = 0; j < n; ++j) out[j] = (float)(zs_std(key, (uint64_t)(first + j)) * sigma);
}

/* out[j] = 16-bit round-to-nearest-even of the same float value; when zero_mod != 0,
 * elements whose index hashes (with zero_seed) to 0 mod zero_mod are an exact +0. */
void zs_fill_16(uint16_t* out, int64_t n, int dtype, uint64_t seed, uint64_t stream, int64_t first,
                double sigma, uint64_t zero_seed, uint32_t zero_mod) {
  uint64_t key = zs_key(seed, stream);
  uint64_t zkey = zs_mix64(zero_seed);
#pragma omp parallel for schedule(static) num_threads(ZS_NT)
  for (int64_t j = 0; j < n; ++j) {
    uint64_t idx = (uint64_t)(first + j);
    out[j] = zs_is_zero(zkey, idx, zero_mod) ? (uint16_t)0 : zs_value16(key, idx, sigma, dtype);
  }
}

/* Gathered variant: out[j] = value at index idx[j] (for sampled checks of huge inputs). */
void zs_gather_16(uint16_t* out, const int64_t* idx, int64_t n, int dtype, uint64_t seed, uint64_t stream,
                  double sigma, uint64_t zero_seed, uint32_t zero_mod) {
  uint64_t key = zs_key(seed, stream);
  uint64_t zkey = zs_mix64(zero_seed);
#pragma omp parallel for schedule(static) num_threads(ZS_NT)
  for (int64_t j = 0; j < n; ++j) {
    uint64_t i = (uint64_t)idx[j];
    out[j] = zs_is_zero(zkey, i, zero_mod) ? (uint16_t)0 : zs_value16(key, i, sigma, dtype);
  }
}

void zs_gather_f32(float* out, const int64_t* idx, int64_t n, uint64_t seed, uint64_t stream, double sigma) {
  uint64_t key = zs_key(seed, stream);
#pragma omp parallel for schedule(static) num_threads(ZS_NT)
  for (int64_t j = 0; j < n; ++j) out[j] = (float)(zs_std(key, (uint64_t)idx[j]) * sigma);
}
