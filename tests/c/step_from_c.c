/* A whole optimizer step driven from plain C through the C ABI on the GPU,
 * checked against the C oracle element by element (bit for bit).
 *
 * Model: three tensors (5000, 77, 70001 elements) flattened, fp16, N_d = 2,
 * this process is rank 1; two rank gradient buffers are reduced on the device
 * (the local half of the reduce-scatter), loss scale 1024, clipping at 1.0,
 * three steps with an overflow in the second.  Device memory comes from
 * hipMalloc; nothing else than the library and the HIP runtime is involved.
 * The oracle (test infrastructure) computes both ranks' statistics and this
 * rank's state.  Built as a shared library (tests/c/build.py) and called
 * in-process: step_from_c() prints one line per check and returns non-zero on
 * the first mismatch. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zero_shard.h"

/* The oracle's C entry points and structs (oracle/zero_oracle.c). */
typedef struct {
  float lr, beta1, beta2, eps, weight_decay;
} orc_hparams;
typedef struct {
  int64_t t;
  double p1, p2;
} orc_counters;
int orc_plan(const int64_t* numel, int64_t num_tensors, int32_t nd, int32_t rank, int32_t align, int64_t* psi,
             int64_t* shard, int64_t* begin, int64_t* valid);
uint16_t orc_f32_to_f16(float x);
int orc_grad_stats(int dtype, const uint16_t* const* src, int n_src, int64_t n, float inv_loss_scale, float* u,
                   double* sumsq_acc);
float orc_clip_coef(double global_sumsq, float max_norm, double* norm_out);
void orc_adam(int skip, const float* u, int64_t n, float clip, const orc_hparams* hp, orc_counters* c, float* w,
              float* m, float* v);
void orc_cast(int dtype, const float* w, int64_t n, uint16_t* p16);

#define HIPCHECK(call)                                                       \
  do {                                                                       \
    hipError_t e_ = (call);                                                  \
    if (e_ != hipSuccess) {                                                  \
      printf("FAIL %s: %s\n", #call, hipGetErrorString(e_));                 \
      fflush(stdout);                                                        \
      return 1;                                                              \
    }                                                                        \
  } while (0)
#define ZCHECK(call)                                                         \
  do {                                                                       \
    zero_status_t s_ = (call);                                               \
    if (s_ != ZERO_OK) {                                                     \
      printf("FAIL %s: %d %s\n", #call, (int)s_, zero_last_error());         \
      fflush(stdout);                                                        \
      return 1;                                                              \
    }                                                                        \
  } while (0)

/* SplitMix64 words mapped to roughly normal values (sum of four uniforms). */
static uint64_t mix(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}
static float normalish(uint64_t seed, uint64_t i) {
  double s = 0.0;
  for (int k = 0; k < 4; ++k) s += (double)(mix(seed * 0x100000001B3ull + 4 * i + k) >> 11) * 0x1.0p-53;
  return (float)((s - 2.0) * 1.7320508075688772);
}

int step_from_c(void) {
  const int64_t numel[3] = {5000, 77, 70001};
  const int32_t nd = 2, rank = 1;
  const float inv = 1.0f / 1024.0f, max_norm = 1.0f;
  const orc_hparams ohp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f};
  const zero_adam_hparams_t hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f};
  int64_t psi, S, b, valid;
  if (orc_plan(numel, 3, nd, rank, 64, &psi, &S, &b, &valid) != 0) return 1;

  /* host model: fp32 master, its fp16 parameters, two rank gradients per step */
  float* master = malloc(sizeof(float) * psi);
  uint16_t* p16 = malloc(2 * psi);
  uint16_t* g[2] = {malloc(2 * psi), malloc(2 * psi)};
  for (int64_t i = 0; i < psi; ++i) {
    master[i] = 0.02f * normalish(1, i);
    p16[i] = orc_f32_to_f16(master[i]);
  }

  /* device buffers */
  void *d_p16, *d_g[2], *d_ws;
  float *d_master0, *d_state[4], *d_out;
  HIPCHECK(hipMalloc(&d_p16, 2 * psi));
  HIPCHECK(hipMalloc(&d_g[0], 2 * psi));
  HIPCHECK(hipMalloc(&d_g[1], 2 * psi));
  HIPCHECK(hipMemcpy(d_p16, p16, 2 * psi, hipMemcpyHostToDevice));
  zero_shard_desc_t d;
  memset(&d, 0, sizeof d);
  d.dp_size = nd;
  d.dp_rank = rank;
  d.dtype = ZERO_F16;
  d.num_tensors = 3;
  d.numel = numel;
  d.flat_param16 = d_p16;
  zero_shard_info_t info;
  ZCHECK(zero_shard_plan(&d, &info));
  if (info.shard_begin != b || info.valid_elems != valid) {
    printf("FAIL plan differs from the oracle's\n");
    fflush(stdout);
    return 1;
  }
  for (int k = 0; k < 4; ++k) HIPCHECK(hipMalloc((void**)&d_state[k], sizeof(float) * info.state_elems));
  HIPCHECK(hipMalloc(&d_ws, info.workspace_bytes));
  HIPCHECK(hipMalloc((void**)&d_master0, sizeof(float) * valid));
  HIPCHECK(hipMalloc((void**)&d_out, sizeof(float) * valid));
  HIPCHECK(hipMemcpy(d_master0, master + b, sizeof(float) * valid, hipMemcpyHostToDevice));
  zero_shard_bufs_t bufs;
  memset(&bufs, 0, sizeof bufs);
  bufs.master = d_state[0];
  bufs.m = d_state[1];
  bufs.v = d_state[2];
  bufs.red = d_state[3];
  bufs.workspace = d_ws;
  bufs.state_capacity = info.state_elems;
  bufs.workspace_capacity = info.workspace_bytes;
  zero_shard_t h;
  ZCHECK(zero_shard_init(&d, &bufs, d_master0, NULL, &h));
  printf("ok init: rank %d of %d, %lld of %lld elements\n", rank, nd, (long long)valid, (long long)psi);

  /* oracle state of this rank */
  float* w = malloc(sizeof(float) * valid);
  float* m = calloc(valid, sizeof(float));
  float* v = calloc(valid, sizeof(float));
  float* u = malloc(sizeof(float) * psi);
  uint16_t* o16 = malloc(2 * valid);
  memcpy(w, master + b, sizeof(float) * valid);
  memcpy(o16, p16 + b, 2 * valid);
  orc_counters ctr = {0, 1.0, 1.0};

  for (int step = 1; step <= 3; ++step) {
    for (int q = 0; q < 2; ++q)
      for (int64_t i = 0; i < psi; ++i) g[q][i] = orc_f32_to_f16(1024.0f * 1e-2f * normalish(100 * step + q, i));
    if (step == 2) g[0][b + 17] = 0x7C00; /* +inf in this rank's slice */
    HIPCHECK(hipMemcpy(d_g[0], g[0], 2 * psi, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(d_g[1], g[1], 2 * psi, hipMemcpyHostToDevice));

    /* oracle: both ranks' statistics (rank order), this rank's update */
    double local[2];
    int flag[2];
    for (int r = 0; r < nd; ++r) {
      int64_t pr, sr, br, vr;
      orc_plan(numel, 3, nd, r, 64, &pr, &sr, &br, &vr);
      const uint16_t* src[2] = {g[0] + br, g[1] + br};
      local[r] = 0.0;
      flag[r] = orc_grad_stats(ZERO_F16, src, 2, vr, inv, u, &local[r]);
    }
    const uint16_t* mine[2] = {g[0] + b, g[1] + b};
    double mysum = 0.0;
    orc_grad_stats(ZERO_F16, mine, 2, valid, inv, u, &mysum);
    double norm;
    const float clip = orc_clip_coef(local[0] + local[1], max_norm, &norm);
    const int skip = flag[0] | flag[1];
    orc_adam(skip, u, valid, clip, &ohp, &ctr, w, m, v);
    if (!skip) orc_cast(ZERO_F16, w, valid, o16);

    /* device: the step through the C ABI, the other rank's values as arguments */
    const void* ranks[2] = {d_g[0], d_g[1]};
    ZCHECK(zero_reduce_grads(h, ranks, 2, inv, NULL));
    int32_t gflag = -1;
    ZCHECK(zero_check_overflow(h, flag[0], &gflag, NULL));
    double dnorm = 0.0;
    if (step != 3) /* the global sum of squares, added once in rank order and given to every rank */
      ZCHECK(zero_grad_norm_global(h, local[0] + local[1], max_norm, &dnorm, NULL));
    else /* the other rank's sum; this rank's own is added on the device */
      ZCHECK(zero_grad_norm(h, local[0], max_norm, &dnorm, NULL));
    ZCHECK(zero_adam_step(h, &hp, 1, NULL));
    int64_t t;
    int32_t skipped;
    double qnorm;
    float qclip;
    ZCHECK(zero_shard_query(h, &t, &skipped, &qnorm, &qclip, NULL));
    if (gflag != skip || skipped != skip || t != ctr.t || (!skip && qclip != clip)) {
      printf("FAIL step %d: flag %d/%d skipped %d t %lld/%lld clip %.9g/%.9g\n", step, gflag, skip, skipped,
             (long long)t, (long long)ctr.t, qclip, clip);
      fflush(stdout);
      return 1;
    }
    if (!skip && fabs(dnorm - norm) > 1e-9 * norm) {
      printf("FAIL step %d: norm %.17g against %.17g\n", step, dnorm, norm);
      fflush(stdout);
      return 1;
    }
    printf("ok step %d: skipped %d, t %lld, clip %.9g\n", step, skip, (long long)t, qclip);
  }

  /* every element of the state and of this rank's 16-bit slice; nothing outside it moved */
  const float* exp[3] = {w, m, v};
  const char* names[3] = {"master", "m", "v"};
  float* got = malloc(sizeof(float) * valid);
  for (int k = 0; k < 3; ++k) {
    ZCHECK(zero_export_state(h, k, d_out, NULL));
    HIPCHECK(hipDeviceSynchronize());
    HIPCHECK(hipMemcpy(got, d_out, sizeof(float) * valid, hipMemcpyDeviceToHost));
    if (memcmp(got, exp[k], sizeof(float) * valid) != 0) {
      printf("FAIL %s differs from the oracle\n", names[k]);
      fflush(stdout);
      return 1;
    }
    printf("ok %s: %lld elements bit-exact\n", names[k], (long long)valid);
  }
  uint16_t* dev16 = malloc(2 * psi);
  HIPCHECK(hipMemcpy(dev16, d_p16, 2 * psi, hipMemcpyDeviceToHost));
  if (memcmp(dev16 + b, o16, 2 * valid) != 0 || memcmp(dev16, p16, 2 * b) != 0) {
    printf("FAIL 16-bit parameters\n");
    fflush(stdout);
    return 1;
  }
  printf("ok p16: slice bit-exact, the rest untouched\n");
  ZCHECK(zero_shard_destroy(h));
  for (int k = 0; k < 4; ++k) HIPCHECK(hipFree(d_state[k]));
  HIPCHECK(hipFree(d_ws));
  HIPCHECK(hipFree(d_master0));
  HIPCHECK(hipFree(d_out));
  HIPCHECK(hipFree(d_p16));
  HIPCHECK(hipFree(d_g[0]));
  HIPCHECK(hipFree(d_g[1]));
  free(master), free(p16), free(g[0]), free(g[1]), free(w), free(m), free(v), free(u), free(o16), free(got);
  free(dev16);
  fflush(stdout);
  return 0;
}
