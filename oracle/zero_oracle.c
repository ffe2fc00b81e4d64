/* Oracle for one data-parallel rank's partitioned mixed-precision optimizer step.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, single-threaded CPU
 * statement of what the step computes.  Only the test-suite, the smoke check
 * and the benchmark's CPU-baseline leg may load it; the product path never does.
 * It shares no code with the HIP library.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no -march, no fast-math), so
 * every float operation is one IEEE binary32 operation rounded to nearest even,
 * with no fused multiply-add and with subnormals kept.
 *
 * Sources (the pages on DeepSpeed ZeRO):
 *  - fp16/bf16 parameters and gradients with fp32 master, momentum and variance:
 *    "ZeRO 技术原理" section 3; "DeepSpeed ZeRO" (formulaic) 表格计算.
 *  - the rank keeps a 1/N_d slice of the flattened, padded state and updates
 *    only that slice: "ZeRO 技术原理" 3.1.1 and 3.3.1 (param.partition());
 *    "DeepSpeed ZeRO" ZeRO Stage 3 基本流程 (flatten, pad, [start, end)).
 *  - the slice's gradient is the reduce-scatter of the ranks' gradients:
 *    "DeepSpeed ZeRO" ZeRO Stage 2 基本思想.
 *  - nan/inf gradients trigger no update, leave the moments uninitialised and do
 *    not copy fp32 into fp16: "DeepSpeed ZeRO" 权重更新的触发条件.
 *  - the Adam formulas m, v, W: "DeepSpeed ZeRO" ZeRO Stage 1, "以 AdaW 为例".
 *  - the in-place 16-bit copy of the updated fp32 slice: same page, step 4 text.
 * Where the pages are silent (bias correction, decoupled weight decay, clipping,
 * the reduce order, the partition rule, the NaN encoding), the reading taken is
 * stated at each function below.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORC_F16 1
#define ORC_BF16 2

/* ------------------------------------------------------------------------ */
/* Partition: flatten the tensor list, pad to N_d equal shards whose length is
 * a multiple of `align` elements; rank r owns [r*S, r*S + S) clipped to [0, psi).
 * The pages pad so that the flat length divides by N_d ("DeepSpeed ZeRO",
 * ZeRO Stage 3 基本流程) and give start = partition_size * rank
 * ("ZeRO 技术原理" 3.3.1).  Returns 0, or -1 on bad arguments. */
int orc_plan(const int64_t* numel, int64_t num_tensors, int32_t nd, int32_t rank, int32_t align,
             int64_t* psi_out, int64_t* shard_out, int64_t* begin_out, int64_t* valid_out) {
  if (nd < 1 || rank < 0 || rank >= nd || align < 1 || num_tensors < 0) return -1;
  int64_t psi = 0;
  for (int64_t k = 0; k < num_tensors; ++k) {
    if (numel[k] < 0) return -1;
    psi += numel[k];
  }
  int64_t per_rank = (psi + nd - 1) / nd;                 /* ceil(psi / nd) */
  int64_t shard = (per_rank + align - 1) / align * align; /* round up to align */
  int64_t begin = (int64_t)rank * shard;
  int64_t valid = psi - begin;
  if (valid < 0) valid = 0;
  if (valid > shard) valid = shard;
  *psi_out = psi;
  *shard_out = shard;
  *begin_out = begin;
  *valid_out = valid;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* 16-bit formats, written from their definitions.
 * binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits; subnormals m*2^-24.
 * bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits; subnormals m*2^-133. */

float orc_f16_to_f32(uint16_t h) {
  int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 31) v = m ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)m, -24);
  else v = ldexp((double)(1024 + m), e - 25);
  return (float)(sign ? -v : v);
}

float orc_bf16_to_f32(uint16_t h) {
  int sign = h >> 15, e = (h >> 7) & 255, m = h & 127;
  double v;
  if (e == 255) v = m ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)m, -133);
  else v = ldexp((double)(128 + m), e - 134);
  return (float)(sign ? -v : v);
}

/* Round |x| to the nearest multiple of the format's spacing, ties to even.
 * p = fraction bits, emin = smallest normal exponent.  Returns the rounded
 * magnitude as a double (exact). */
static double round_to_format(double a, int p, int emin) {
  int e;
  if (a == 0.0) return 0.0;
  frexp(a, &e); /* a = f * 2^e with f in [0.5, 1) */
  e -= 1;       /* now 2^e <= a < 2^(e+1) */
  if (e < emin) e = emin;
  double q = ldexp(1.0, e - p); /* spacing of representable values at this exponent */
  return nearbyint(a / q) * q;  /* a / q is exact; nearbyint rounds half to even */
}

static uint16_t encode_format(double r, int p, int emin, int bias) {
  int e;
  if (r == 0.0) return 0;
  frexp(r, &e);
  e -= 1;
  if (e < emin) return (uint16_t)(r / ldexp(1.0, emin - p)); /* subnormal: fraction only */
  return (uint16_t)(((e + bias) << p) | (uint16_t)(r / ldexp(1.0, e - p) - ldexp(1.0, p)));
}

/* NaN rule of the write-back (the pages are silent on it): every NaN becomes the
 * format's positive canonical quiet NaN (binary16 0x7E00, bfloat16 0x7FC0),
 * whatever its sign and payload.  IEEE 754 leaves the sign and payload of a NaN
 * produced by arithmetic unspecified, and hosts differ (an invalid operation such
 * as inf - inf gives a negative NaN on x86 and a positive one on the GPU), so a
 * rule that kept them would make the written bits depend on the machine. */
uint16_t orc_f32_to_f16(float x) {
  if (isnan(x)) return 0x7E00;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs((double)x);
  /* the largest finite binary16 is 65504; halfway to 65536 is 65520, which rounds to even (65536): overflow */
  if (a >= 65520.0) return sign | 0x7C00;
  return sign | encode_format(round_to_format(a, 10, -14), 10, -14, 15);
}

uint16_t orc_f32_to_bf16(float x) {
  if (isnan(x)) return 0x7FC0; /* the NaN rule above */
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs((double)x);
  /* the largest finite bfloat16 is (2 - 2^-7) * 2^127; from (2 - 2^-8) * 2^127 on it rounds to infinity */
  if (a >= ldexp(2.0 - ldexp(1.0, -8), 127)) return sign | 0x7F80;
  return sign | encode_format(round_to_format(a, 7, -126), 7, -126, 127);
}

static float dec16(int dtype, uint16_t h) { return dtype == ORC_BF16 ? orc_bf16_to_f32(h) : orc_f16_to_f32(h); }
static uint16_t enc16(int dtype, float x) { return dtype == ORC_BF16 ? orc_f32_to_bf16(x) : orc_f32_to_f16(x); }

/* ------------------------------------------------------------------------ */
/* Gradient intake for this rank's slice of n elements.
 *   n_src == 1: src[0] is the already-reduced 16-bit gradient slice (the ZeRO-1
 *               path, where the gradient was all-reduced).
 *   n_src >= 2: src[q] is rank q's 16-bit gradient at this rank's slice; the
 *               slice is their sum (the local half of the reduce-scatter), added
 *               in fp32 in rank order: red = g_0 + g_1 + ... + g_{n_src-1}.
 * Then u = red * inv_loss_scale (unscale), flag = any u not finite, and
 * *sumsq_acc += u^2 in fp64, element by element in index order (each term is
 * exact in fp64).  Writes u[0..n).  Returns the flag. */
int orc_grad_stats(int dtype, const uint16_t* const* src, int n_src, int64_t n, float inv_loss_scale,
                   float* u, double* sumsq_acc) {
  int flag = 0;
  double acc = *sumsq_acc;
  for (int64_t i = 0; i < n; ++i) {
    float red = dec16(dtype, src[0][i]);
    for (int q = 1; q < n_src; ++q) red = red + dec16(dtype, src[q][i]);
    float ui = red * inv_loss_scale;
    if (!isfinite(ui)) flag = 1;
    acc = acc + (double)ui * (double)ui;
    u[i] = ui;
  }
  *sumsq_acc = acc;
  return flag;
}

/* 16-bit output of the local reduce.  "DeepSpeed ZeRO", ZeRO Stage 2 基本思想: the
 * rank's fp32 gradient shard is taken from the reduce-scatter's bf16 result.  The
 * reduction is the rank-order fp32 sum of orc_grad_stats; its result is delivered in
 * the 16-bit type, rounded once to nearest even:
 *   out16[i] = RNE16(g_0[i] + g_1[i] + ... + g_{n_src-1}[i]).
 * The step then takes this 16-bit slice in as an already-reduced gradient. */
void orc_reduce_to16(int dtype, const uint16_t* const* src, int n_src, int64_t n, uint16_t* out16) {
  for (int64_t i = 0; i < n; ++i) {
    float s = dec16(dtype, src[0][i]);
    for (int q = 1; q < n_src; ++q) s = s + dec16(dtype, src[q][i]);
    out16[i] = enc16(dtype, s);
  }
}

/* Gradient accumulation over micro-steps ("DeepSpeed ZeRO", ZeRO Stage 2: with
 * gradient accumulation every backward reduce-scatters and the rank adds its
 * 1/N_d slice to what it has accumulated).  s = g_0 + g_1 + ... in fp32 rank
 * order (one source = already reduced); acc = s on the first micro-step, else
 * acc = acc + s. */
void orc_accumulate(int dtype, const uint16_t* const* src, int n_src, int64_t n, float* acc, int first) {
  for (int64_t i = 0; i < n; ++i) {
    float s = dec16(dtype, src[0][i]);
    for (int q = 1; q < n_src; ++q) s = s + dec16(dtype, src[q][i]);
    acc[i] = first ? s : acc[i] + s;
  }
}

/* Intake of an accumulated fp32 gradient: u = acc * inv_loss_scale, flag = any u
 * not finite, *sumsq_acc += u^2 in fp64 in index order.  Returns the flag. */
int orc_stats_f32(const float* acc, int64_t n, float inv_loss_scale, float* u, double* sumsq_acc) {
  int flag = 0;
  double a = *sumsq_acc;
  for (int64_t i = 0; i < n; ++i) {
    float ui = acc[i] * inv_loss_scale;
    if (!isfinite(ui)) flag = 1;
    a = a + (double)ui * (double)ui;
    u[i] = ui;
  }
  *sumsq_acc = a;
  return flag;
}

/* Global-norm clipping coefficient.  norm = sqrt(global sum of squares);
 * coefficient = max_norm / (norm + 1e-6) when that is below 1, else 1; a
 * non-positive max_norm disables clipping. */
float orc_clip_coef(double global_sumsq, float max_norm, double* norm_out) {
  double norm = sqrt(global_sumsq);
  if (norm_out) *norm_out = norm;
  if (!(max_norm > 0.0f)) return 1.0f;
  double c = (double)max_norm / (norm + 1e-6);
  return c < 1.0 ? (float)c : 1.0f;
}

typedef struct {
  float lr, beta1, beta2, eps, weight_decay;
} orc_hparams;

typedef struct {
  int64_t t;     /* applied steps so far */
  double p1, p2; /* beta1^t and beta2^t as running fp64 products */
} orc_counters;

/* Bias-correction scalars of the next applied step (t+1), without committing them. */
void orc_next_scalars(const orc_hparams* hp, const orc_counters* c, float* bc1, float* bc2) {
  double p1 = c->p1 * (double)hp->beta1, p2 = c->p2 * (double)hp->beta2;
  *bc1 = (float)(1.0 - p1);
  *bc2 = (float)(1.0 - p2);
}

/* One Adam update with bias correction and decoupled weight decay on n elements.
 * If skip is set nothing at all changes: not the counters, not w, m or v.
 * Otherwise t += 1, beta^t are advanced, and for every element:
 *   g  = u * clip
 *   m  = beta1 * m + (1 - beta1) * g
 *   v  = beta2 * v + (1 - beta2) * g * g
 *   mh = m / (1 - beta1^t),  vh = v / (1 - beta2^t)
 *   w  = w - lr * (mh / (sqrt(vh) + eps) + wd * w)      (wd * w uses the old w)
 * which is the pages' m, v, W recurrence with the textbook bias correction and
 * a decoupled weight-decay term added. */
void orc_adam(int skip, const float* u, int64_t n, float clip, const orc_hparams* hp, orc_counters* c,
              float* w, float* m, float* v) {
  if (skip) return;
  float bc1, bc2;
  orc_next_scalars(hp, c, &bc1, &bc2);
  c->t += 1;
  c->p1 = c->p1 * (double)hp->beta1;
  c->p2 = c->p2 * (double)hp->beta2;
  const float b1 = hp->beta1, b2 = hp->beta2;
  const float omb1 = 1.0f - b1, omb2 = 1.0f - b2;
  for (int64_t i = 0; i < n; ++i) {
    float g = u[i] * clip;
    float mi = b1 * m[i] + omb1 * g;
    float vi = b2 * v[i] + omb2 * (g * g);
    float mh = mi / bc1;
    float vh = vi / bc2;
    float den = sqrtf(vh) + hp->eps;
    float upd = mh / den;
    float wi = w[i];
    w[i] = wi - hp->lr * (upd + hp->weight_decay * wi);
    m[i] = mi;
    v[i] = vi;
  }
}

/* Per-element form of orc_adam for sampled checks: the caller supplies the
 * bias-correction scalars of the step (from orc_next_scalars). */
void orc_adam_elems(const float* u, int64_t n, float clip, const orc_hparams* hp, float bc1, float bc2, float* w,
                    float* m, float* v) {
  const float b1 = hp->beta1, b2 = hp->beta2;
  const float omb1 = 1.0f - b1, omb2 = 1.0f - b2;
  for (int64_t i = 0; i < n; ++i) {
    float g = u[i] * clip;
    float mi = b1 * m[i] + omb1 * g;
    float vi = b2 * v[i] + omb2 * (g * g);
    float mh = mi / bc1;
    float vh = vi / bc2;
    float den = sqrtf(vh) + hp->eps;
    float upd = mh / den;
    float wi = w[i];
    w[i] = wi - hp->lr * (upd + hp->weight_decay * wi);
    m[i] = mi;
    v[i] = vi;
  }
}

/* Dynamic loss scale ("DeepSpeed ZeRO" 配置说明: fp16.loss_scale = 0 selects dynamic
 * scaling, starting at 2^initial_scale_power).  The pages give no update rule; the
 * rule taken is the standard one: after a step with an overflow the scale is
 * multiplied by `backoff` (not below min_scale) and the count of good steps is
 * reset; after `interval` consecutive good steps it is multiplied by `growth`
 * when that product is finite (a scale that grew to infinity would skip every
 * later step for good) and the count is reset.  The intake then unscales by
 * inv = 1 / scale (fp32). */
void orc_loss_scale_update(int skipped, float growth, float backoff, int interval, float min_scale, float* scale,
                           int* good) {
  if (skipped) {
    float s = *scale * backoff;
    *scale = s < min_scale ? min_scale : s;
    *good = 0;
  } else {
    *good += 1;
    if (*good == interval) {
      float grown = *scale * growth;
      if (isfinite(grown)) *scale = grown;
      *good = 0;
    }
  }
}

float orc_inv_scale(float scale) { return 1.0f / scale; }

/* In-place 16-bit write-back of the updated fp32 slice: p16[i] = RNE(w[i]). */
void orc_cast(int dtype, const float* w, int64_t n, uint16_t* p16) {
  for (int64_t i = 0; i < n; ++i) p16[i] = enc16(dtype, w[i]);
}

/* Master initialisation from the 16-bit slice (partition_fp16.copy().float()). */
void orc_upcast(int dtype, const uint16_t* p16, int64_t n, float* w) {
  for (int64_t i = 0; i < n; ++i) w[i] = dec16(dtype, p16[i]);
}

void orc_encode_many(int dtype, const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = enc16(dtype, x[i]);
}

void orc_decode_many(int dtype, const uint16_t* h, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = dec16(dtype, h[i]);
}
