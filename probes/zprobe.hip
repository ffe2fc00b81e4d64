// Bandwidth probes: streaming kernels with the memory-access patterns of the
// optimizer step's kernels and none of the method's arithmetic.  The benchmark
// runs them on the same GPU as the step to measure what HBM delivers to each
// pattern -- the ceiling the step's kernels are judged against, besides the
// published peak.  Not part of the optimizer library.
//
// Layout of every probe: a one-dimensional grid of short-lived blocks, block b
// covering elements [b*epb, min((b+1)*epb, n)) of each stream; each lane moves
// 4-element quads (8-byte accesses of 16-bit data, 16-byte accesses of fp32
// data), a block of BS lanes covering 4*BS consecutive elements per quad slot,
// U slots loaded before any is stored.  With epb = 2048, BS = 256, U = 2 and
// non-temporal state accesses this is exactly the Adam pass's pattern; with
// the other parameters it explores nearby ones.  n must be a multiple of 4.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool NT, class T>
__device__ __forceinline__ T ld(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT, class T>
__device__ __forceinline__ void st(T* p, T v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}
// 16-bit quad -> fp32 quad by placing each half in the top of a word (a bit move, no rounding)
__device__ __forceinline__ f32x4 widen(u32x2 r) {
  return f32x4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u), __uint_as_float(r.y << 16),
               __uint_as_float(r.y & 0xFFFF0000u)};
}
__device__ __forceinline__ u32x2 narrow(f32x4 a) {
  return u32x2{(__float_as_uint(a.x) >> 16) | (__float_as_uint(a.y) & 0xFFFF0000u),
               (__float_as_uint(a.z) >> 16) | (__float_as_uint(a.w) & 0xFFFF0000u)};
}

struct Span {
  int64_t q0, q1;  // quads of this block
};
__device__ __forceinline__ Span span(int64_t nq, int64_t qpb) {
  const int64_t q0 = (int64_t)blockIdx.x * qpb;
  return Span{q0, q0 + qpb < nq ? q0 + qpb : nq};
}

// Adam pass mix: read g (2 B, or 4 B with G32), w, m, v (4 B each); write w, m, v and p16.
// 28 B per element (30 B with an fp32 gradient, the Adam pass after a local reduce).
template <int U, int BS, bool NTL, bool NTS, bool G32>
__global__ void __launch_bounds__(BS) adam_mix(const void* gp, f32x4* w, f32x4* m, f32x4* v, u32x2* p, int64_t nq,
                                               int64_t qpb) {
  const Span s = span(nq, qpb);
  for (int64_t q = s.q0 + threadIdx.x; q < s.q1; q += U * BS) {
    f32x4 G[U], W[U], M[U], V[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int64_t i = q + k * BS;
      if (i < s.q1) {
        if constexpr (G32) G[k] = ld<NTL>(static_cast<const f32x4*>(gp) + i);
        else G[k] = widen(ld<false>(static_cast<const u32x2*>(gp) + i));
        W[k] = ld<NTL>(w + i);
        M[k] = ld<NTL>(m + i);
        V[k] = ld<NTL>(v + i);
      }
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int64_t i = q + k * BS;
      if (i < s.q1) {
        const f32x4 a = W[k] + G[k];
        st<NTS>(w + i, a);
        st<NTS>(m + i, M[k] + G[k]);
        st<NTS>(v + i, V[k] + G[k]);
        st<NTS>(p + i, narrow(a));
      }
    }
  }
}

// Pure read of fp32 (the block's sum goes to sink[block], so nothing is optimised away).
template <int U, int BS, bool NT>
__global__ void __launch_bounds__(BS) read32(const f32x4* src, float* sink, int64_t nq, int64_t qpb) {
  const Span s = span(nq, qpb);
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t q = s.q0 + threadIdx.x; q < s.q1; q += U * BS) {
    f32x4 X[U];
#pragma unroll
    for (int k = 0; k < U; ++k) X[k] = q + k * BS < s.q1 ? ld<NT>(src + q + k * BS) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < U; ++k) acc += X[k];
  }
  float t = acc.x + acc.y + acc.z + acc.w;
  for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off, 64);
  if (threadIdx.x == 0) sink[blockIdx.x] = t;  // one wave's sum stands for the block's
}

// Pure read of 16-bit data (the statistics pass's stream).
template <int U, int BS, bool NT>
__global__ void __launch_bounds__(BS) read16(const u32x2* src, float* sink, int64_t nq, int64_t qpb) {
  const Span s = span(nq, qpb);
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t q = s.q0 + threadIdx.x; q < s.q1; q += U * BS) {
    u32x2 X[U];
#pragma unroll
    for (int k = 0; k < U; ++k) X[k] = q + k * BS < s.q1 ? ld<NT>(src + q + k * BS) : u32x2{0u, 0u};
#pragma unroll
    for (int k = 0; k < U; ++k) acc += widen(X[k]);
  }
  float t = acc.x + acc.y + acc.z + acc.w;
  for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off, 64);
  if (threadIdx.x == 0) sink[blockIdx.x] = t;
}

// Pure write of fp32.
template <int U, int BS, bool NT>
__global__ void __launch_bounds__(BS) write32(f32x4* dst, int64_t nq, int64_t qpb) {
  const Span s = span(nq, qpb);
  const float b = (float)blockIdx.x;
  for (int64_t q = s.q0 + threadIdx.x; q < s.q1; q += U * BS) {
#pragma unroll
    for (int k = 0; k < U; ++k)
      if (q + k * BS < s.q1) st<NT>(dst + q + k * BS, f32x4{b, b, b, b});
  }
}

// fp32 copy (one read and one write stream).
template <int U, int BS, bool NT>
__global__ void __launch_bounds__(BS) copy32(const f32x4* src, f32x4* dst, int64_t nq, int64_t qpb) {
  const Span s = span(nq, qpb);
  for (int64_t q = s.q0 + threadIdx.x; q < s.q1; q += U * BS) {
    f32x4 X[U];
#pragma unroll
    for (int k = 0; k < U; ++k)
      if (q + k * BS < s.q1) X[k] = ld<NT>(src + q + k * BS);
#pragma unroll
    for (int k = 0; k < U; ++k)
      if (q + k * BS < s.q1) st<NT>(dst + q + k * BS, X[k]);
  }
}

// The local reduce's mix: read NR 16-bit streams, write one fp32 stream.
constexpr int kMaxSrc = 8;
struct Srcs {
  const u32x2* s[kMaxSrc];
};
template <int NR, int U, int BS, bool NT>
__global__ void __launch_bounds__(BS) reduce_mix(Srcs src, f32x4* out, int64_t nq, int64_t qpb) {
  const Span s = span(nq, qpb);
  for (int64_t q = s.q0 + threadIdx.x; q < s.q1; q += U * BS) {
    u32x2 R[NR][U];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int k = 0; k < U; ++k)
        if (q + k * BS < s.q1) R[r][k] = ld<NT>(src.s[r] + q + k * BS);
#pragma unroll
    for (int k = 0; k < U; ++k) {
      if (q + k * BS >= s.q1) continue;
      f32x4 a = widen(R[0][k]);
#pragma unroll
      for (int r = 1; r < NR; ++r) a += widen(R[r][k]);
      st<NT>(out + q + k * BS, a);
    }
  }
}

struct Grid {
  unsigned blocks;
  int64_t nq, qpb;
};

// epb: elements per block, a positive multiple of 4 * bs.
bool grid_of(int64_t n, int32_t epb, int32_t bs, Grid* g) {
  if (n < 0 || (n & 3) != 0 || epb <= 0 || epb % (4 * bs) != 0) return false;
  g->nq = n / 4;
  g->qpb = epb / 4;
  const int64_t blocks = (g->nq + g->qpb - 1) / g->qpb;
  if (blocks > 0x7FFFFFFF) return false;
  g->blocks = (unsigned)(blocks < 1 ? 1 : blocks);
  return true;
}

#define ZP_BS_SWITCH(BSV, ...)                                     \
  switch (BSV) {                                                   \
    case 256: { constexpr int BS = 256; __VA_ARGS__; break; }      \
    case 512: { constexpr int BS = 512; __VA_ARGS__; break; }      \
    default: return (int)hipErrorInvalidValue;                     \
  }
#define ZP_U_SWITCH(UV, ...)                                       \
  switch (UV) {                                                    \
    case 1: { constexpr int U = 1; __VA_ARGS__; break; }           \
    case 2: { constexpr int U = 2; __VA_ARGS__; break; }           \
    case 4: { constexpr int U = 4; __VA_ARGS__; break; }           \
    default: return (int)hipErrorInvalidValue;                     \
  }
#define ZP_NT_SWITCH(NAME, V, ...)                                 \
  if (V) { constexpr bool NAME = true; __VA_ARGS__; }              \
  else { constexpr bool NAME = false; __VA_ARGS__; }

}  // namespace

extern "C" {

// Every call enqueues one kernel on `stream` and returns a hipError_t code (0 = success).
// epb: elements per block (a multiple of 4 * bs); u: quads per lane in flight (1, 2, 4);
// bs: threads per block (256, 512); nt*: non-temporal accesses.

// g: n 16-bit values (g32 = 0) or n floats (g32 = 1).
int zprobe_adam_mix(const void* g, int32_t g32, float* w, float* m, float* v, void* p16, int64_t n, int32_t epb,
                    int32_t u, int32_t bs, int32_t nt_load, int32_t nt_store, void* stream) {
  Grid gr;
  if (!grid_of(n, epb, bs, &gr)) return (int)hipErrorInvalidValue;
  if (n == 0) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  ZP_NT_SWITCH(G32, g32, ZP_BS_SWITCH(bs, ZP_U_SWITCH(u, ZP_NT_SWITCH(NTL, nt_load, ZP_NT_SWITCH(NTS, nt_store,
      hipLaunchKernelGGL((adam_mix<U, BS, NTL, NTS, G32>), dim3(gr.blocks), dim3(BS), 0, st, g,
                         reinterpret_cast<f32x4*>(w), reinterpret_cast<f32x4*>(m), reinterpret_cast<f32x4*>(v),
                         static_cast<u32x2*>(p16), gr.nq, gr.qpb))))));
  return (int)hipGetLastError();
}

// sink: at least ceil(n / epb) floats.
int zprobe_read32(const float* src, int64_t n, float* sink, int32_t epb, int32_t u, int32_t bs, int32_t nt,
                  void* stream) {
  Grid gr;
  if (!grid_of(n, epb, bs, &gr)) return (int)hipErrorInvalidValue;
  if (n == 0) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  ZP_BS_SWITCH(bs, ZP_U_SWITCH(u, ZP_NT_SWITCH(NT, nt,
      hipLaunchKernelGGL((read32<U, BS, NT>), dim3(gr.blocks), dim3(BS), 0, st,
                         reinterpret_cast<const f32x4*>(src), sink, gr.nq, gr.qpb))));
  return (int)hipGetLastError();
}

int zprobe_read16(const void* src, int64_t n, float* sink, int32_t epb, int32_t u, int32_t bs, int32_t nt,
                  void* stream) {
  Grid gr;
  if (!grid_of(n, epb, bs, &gr)) return (int)hipErrorInvalidValue;
  if (n == 0) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  ZP_BS_SWITCH(bs, ZP_U_SWITCH(u, ZP_NT_SWITCH(NT, nt,
      hipLaunchKernelGGL((read16<U, BS, NT>), dim3(gr.blocks), dim3(BS), 0, st,
                         static_cast<const u32x2*>(src), sink, gr.nq, gr.qpb))));
  return (int)hipGetLastError();
}

int zprobe_write32(float* dst, int64_t n, int32_t epb, int32_t u, int32_t bs, int32_t nt, void* stream) {
  Grid gr;
  if (!grid_of(n, epb, bs, &gr)) return (int)hipErrorInvalidValue;
  if (n == 0) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  ZP_BS_SWITCH(bs, ZP_U_SWITCH(u, ZP_NT_SWITCH(NT, nt,
      hipLaunchKernelGGL((write32<U, BS, NT>), dim3(gr.blocks), dim3(BS), 0, st,
                         reinterpret_cast<f32x4*>(dst), gr.nq, gr.qpb))));
  return (int)hipGetLastError();
}

int zprobe_copy32(const float* src, float* dst, int64_t n, int32_t epb, int32_t u, int32_t bs, int32_t nt,
                  void* stream) {
  Grid gr;
  if (!grid_of(n, epb, bs, &gr)) return (int)hipErrorInvalidValue;
  if (n == 0) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  ZP_BS_SWITCH(bs, ZP_U_SWITCH(u, ZP_NT_SWITCH(NT, nt,
      hipLaunchKernelGGL((copy32<U, BS, NT>), dim3(gr.blocks), dim3(BS), 0, st,
                         reinterpret_cast<const f32x4*>(src), reinterpret_cast<f32x4*>(dst), gr.nq, gr.qpb))));
  return (int)hipGetLastError();
}

// srcs: host array of nsrc (2, 4 or 8) device pointers to 16-bit streams of n elements.
int zprobe_reduce_mix(const void* const* srcs, int32_t nsrc, float* out, int64_t n, int32_t epb, int32_t u,
                      int32_t bs, int32_t nt, void* stream) {
  Grid gr;
  if (!grid_of(n, epb, bs, &gr) || !srcs) return (int)hipErrorInvalidValue;
  if (n == 0) return 0;
  Srcs s{};
  for (int r = 0; r < nsrc && r < kMaxSrc; ++r) s.s[r] = static_cast<const u32x2*>(srcs[r]);
  hipStream_t st = static_cast<hipStream_t>(stream);
  f32x4* o = reinterpret_cast<f32x4*>(out);
  switch (nsrc) {
    case 2:
      ZP_BS_SWITCH(bs, ZP_U_SWITCH(u, ZP_NT_SWITCH(NT, nt,
          hipLaunchKernelGGL((reduce_mix<2, U, BS, NT>), dim3(gr.blocks), dim3(BS), 0, st, s, o, gr.nq, gr.qpb))));
      break;
    case 4:
      ZP_BS_SWITCH(bs, ZP_U_SWITCH(u, ZP_NT_SWITCH(NT, nt,
          hipLaunchKernelGGL((reduce_mix<4, U, BS, NT>), dim3(gr.blocks), dim3(BS), 0, st, s, o, gr.nq, gr.qpb))));
      break;
    case 8:
      ZP_BS_SWITCH(bs, ZP_U_SWITCH(u, ZP_NT_SWITCH(NT, nt,
          hipLaunchKernelGGL((reduce_mix<8, U, BS, NT>), dim3(gr.blocks), dim3(BS), 0, st, s, o, gr.nq, gr.qpb))));
      break;
    default:
      return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // extern "C"
