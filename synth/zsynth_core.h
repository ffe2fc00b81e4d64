/* Counter-based synthetic input generator shared by the CPU and GPU fillers.
 *
 * Every value is a pure function of (seed, stream, index), so any slice of a
 * multi-billion-element input can be regenerated independently, on the host
 * or on the device, with identical bits.  The generator holds none of the
 * optimizer's arithmetic: it only produces test and benchmark inputs.
 *
 * Bits: SplitMix64 (Steele, Lea and Flood, "Fast Splittable Pseudorandom
 * Number Generators", OOPSLA 2014) -- the published finaliser applied to a
 * Weyl sequence with the golden-ratio increment.
 *
 * Approximately normal values: Irwin-Hall sum of eight independent uniform
 * 16-bit integers (taken from two 64-bit words), centred and divided by its
 * exact standard deviation sqrt(8*(65536^2-1)/12).  Tails stop at about
 * +-4.9 sigma.  Integer work is exact; the two double multiplies and the final
 * double->float conversion are IEEE round-to-nearest-even on both sides, so
 * host and device agree bit for bit.
 */
#ifndef ZSYNTH_CORE_H
#define ZSYNTH_CORE_H
#include <stdint.h>

#if defined(__HIPCC__)
#define ZS_FN static inline __host__ __device__
#else
#define ZS_FN static inline
#endif

#define ZS_GAMMA 0x9E3779B97F4A7C15ULL
/* 1 / sqrt(8 * (65536^2 - 1) / 12), correctly rounded to double */
#define ZS_INV_SD8 0x1.3988e1412ed76p-16

ZS_FN uint64_t zs_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

ZS_FN uint64_t zs_key(uint64_t seed, uint64_t stream) {
  return zs_mix64(zs_mix64(seed) ^ (stream * 0xD1B54A32D192ED03ULL));
}

ZS_FN uint64_t zs_word(uint64_t key, uint64_t j) { return zs_mix64(key + (j + 1) * ZS_GAMMA); }

/* Standardised value (mean 0, variance 1) for element idx of (key). */
ZS_FN double zs_std(uint64_t key, uint64_t idx) {
  uint64_t a = zs_word(key, 2 * idx), b = zs_word(key, 2 * idx + 1);
  int64_t s = (int64_t)((a & 0xFFFF) + ((a >> 16) & 0xFFFF) + ((a >> 32) & 0xFFFF) + (a >> 48) +
                        (b & 0xFFFF) + ((b >> 16) & 0xFFFF) + ((b >> 32) & 0xFFFF) + (b >> 48));
  return (double)(s - 262140) * ZS_INV_SD8;
}

/* True when element idx is forced to an exact +0 (about one in `mod`). */
ZS_FN int zs_is_zero(uint64_t zero_key, uint64_t idx, uint32_t mod) {
  return mod != 0 && (zs_mix64(zero_key + (idx + 1) * ZS_GAMMA) % mod) == 0;
}

ZS_FN uint32_t zs_f32_bits(float f) {
  union { float f; uint32_t u; } c;
  c.f = f;
  return c.u;
}

/* float -> IEEE binary16 bits, round to nearest even (input values are finite). */
ZS_FN uint16_t zs_f16_bits(float f) {
  uint32_t x = zs_f32_bits(f);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t ax = x & 0x7FFFFFFFu;
  if (ax > 0x7F800000u) return (uint16_t)(sign | 0x7E00u);
  if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u); /* |f| >= 65520 overflows */
  if (ax >= 0x38800000u) {                                   /* normal binary16 */
    uint32_t r = ax - 0x38000000u;
    r += 0x0FFFu + ((r >> 13) & 1u);
    return (uint16_t)(sign | (r >> 13));
  }
  if (ax <= 0x33000000u) return (uint16_t)sign; /* |f| <= 2^-25 rounds to zero */
  {
    uint32_t e = ax >> 23; /* 102..112 */
    uint32_t mant = (ax & 0x7FFFFFu) | 0x800000u;
    uint32_t shift = 126u - e; /* 14..24 */
    uint32_t q = mant >> shift, rem = mant & ((1u << shift) - 1u), half = 1u << (shift - 1u);
    if (rem > half || (rem == half && (q & 1u))) q += 1u;
    return (uint16_t)(sign | q);
  }
}

/* float -> bfloat16 bits, round to nearest even (finite inputs). */
ZS_FN uint16_t zs_bf16_bits(float f) {
  uint32_t x = zs_f32_bits(f);
  return (uint16_t)((x + 0x7FFFu + ((x >> 16) & 1u)) >> 16);
}

/* dtype codes shared with the library's public header: 1 = fp16, 2 = bf16 */
ZS_FN uint16_t zs_value16(uint64_t key, uint64_t idx, double sigma, int dtype) {
  float x = (float)(zs_std(key, idx) * sigma);
  return dtype == 2 ? zs_bf16_bits(x) : zs_f16_bits(x);
}

#endif
