// gfx950 kernels of the partitioned mixed-precision optimizer step.
//
// The kernels walk the shard's chunk table (chunks of at most kChunk elements
// inside one tensor piece).  The statistics pass launches one short-lived block
// per chunk (or per run of a few consecutive chunks on small shards), the local
// reduce one per part of a chunk; both combine their sums of squares in a fixed
// two-level order without float atomics (see finish_stats).  The Adam pass
// launches one short-lived block per part of a chunk.  The hardware dispatcher
// balances the load in all of them.
// Inside a run of elements a block peels at most 3 leading elements, streams
// the body as 4-element quads -- 8-byte loads and stores of 16-bit data,
// 16-byte loads and stores of fp32 data, each wave covering 256 consecutive
// elements per quad slot so every memory instruction is fully coalesced --
// with U quads per lane in flight, then finishes a tail of at most 3 elements.
// Runs whose streams are not co-aligned fall back to one element per lane.
// Per-element arithmetic is plain fp32 (compiled with -ffp-contract=off and
// the default correctly rounded division and square root), identical in the
// vector and scalar paths.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zs_internal.h"

// Tuning knobs (each set to the value measured fastest on MI355X):
//   ZS_ADAM_U   quads per lane in flight in the Adam pass
//   ZS_STATS_U  quads per lane in flight in the statistics pass
//   ZS_STATS_NT_BYTES  a statistics pass over a gradient slice of more bytes than this (the
//                      Infinity Cache, 256 MiB) reads it with non-temporal loads
//   ZS_STATS_TAIL_BYTES  ... except for its last ZS_STATS_TAIL_BYTES, read with plain loads so
//                      they stay in the Infinity Cache; the Adam pass then walks the shard from
//                      its end and re-reads them from there (256 MiB measured 3.8% faster on
//                      the 389 MB GPT-2 slice than none, 240 and 320 MiB in between); not for
//                      slices beyond 16 times this, where the gain is within the noise
//   ZS_REDUCE_TAIL_BYTES  the local reduce stores the last this many bytes of its output (all of
//                      it if smaller) with plain stores, which stay in the Infinity Cache for
//                      the Adam pass, the rest non-temporally (128-192 MiB measured 2.7% faster
//                      with the 16-bit output of the 8-way reduce, 0.6% with fp32 u; the plain
//                      stores slow the reduce pass itself, so more is not better)
//   ZS_STATS_SMALL  a statistics pass over fewer chunks than this takes ZS_STATS_SMALL_CPB
//                   consecutive chunks per block (else one); the reduce passes take one chunk,
//                   or one part of it (ZS_REDUCE_PARTS, over several rank slices)
//   ZS_REDUCE_U quads per lane in flight in the local-reduce pass
//   ZS_REDUCE_NT non-temporal loads of the local reduce's and accumulation's sources
//   ZS_STATS_PF request the next chunk's table entry before streaming the current chunk
//               (intake blocks that cover several chunks)
//   ZS_NT_LOAD  non-temporal loads of the fp32 state (read once per step)
//   ZS_NT_STORE non-temporal stores of the fp32 state and 16-bit parameters
//   ZS_ADAM_SPLIT    parts per chunk in the Adam pass (one block per part)
//   ZS_ADAM_SPLIT_RED  the same when the gradient is the fp32 u of a local reduce (30 B per
//                      element): 1024-element parts measured 3.5% faster there, and slower
//                      for the 16-bit gradient sources (re-measured later: 3.7% faster on one
//                      box, 1.1% slower on another)
//   ZS_ADAM_BLOCK    threads per block of the Adam pass
#ifndef ZS_ADAM_U
#define ZS_ADAM_U 2
#endif
#ifndef ZS_STATS_U
#define ZS_STATS_U 8
#endif
#ifndef ZS_STATS_NT_BYTES
#define ZS_STATS_NT_BYTES (256ll << 20)
#endif
#ifndef ZS_STATS_TAIL_BYTES
#define ZS_STATS_TAIL_BYTES (256ll << 20)
#endif
#ifndef ZS_REDUCE_TAIL_BYTES
#define ZS_REDUCE_TAIL_BYTES (192ll << 20)
#endif
#ifndef ZS_STATS_SMALL
#define ZS_STATS_SMALL 32768
#endif
#ifndef ZS_STATS_SMALL_CPB
#define ZS_STATS_SMALL_CPB 4
#endif
#ifndef ZS_REDUCE_U
#define ZS_REDUCE_U 2
#endif
#ifndef ZS_REDUCE_NT
#define ZS_REDUCE_NT 1
#endif
#ifndef ZS_STATS_PF
#define ZS_STATS_PF 1
#endif
#ifndef ZS_ADAM_BLOCK
#define ZS_ADAM_BLOCK 256
#endif
#ifndef ZS_ADAM_SPLIT
#define ZS_ADAM_SPLIT 4
#endif
#ifndef ZS_ADAM_SPLIT_RED
#define ZS_ADAM_SPLIT_RED 8
#endif
#ifndef ZS_NT_LOAD
#define ZS_NT_LOAD 1
#endif
#ifndef ZS_NT_STORE
#define ZS_NT_STORE 1
#endif

namespace zs {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// 16-bit formats

template <int DT>
__device__ __forceinline__ float dec16(uint32_t h) {
  if constexpr (DT == ZERO_BF16) {
    return __uint_as_float(h << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  }
}

// Round to nearest even into the 16-bit format.  Every NaN, whatever its sign and
// payload, becomes the format's positive canonical quiet NaN (0x7FC0, 0x7E00): the
// sign and payload of an arithmetic NaN are not fixed by IEEE 754 and differ
// between machines, so keeping them would make the written bits machine-dependent.
template <int DT>
__device__ __forceinline__ uint32_t enc16(float x) {
  if constexpr (DT == ZERO_BF16) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;           // canonical quiet NaN
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;                   // round to nearest even
  } else {
    const uint32_t h = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);  // v_cvt_f16_f32, RNE
    return __builtin_isnan(x) ? 0x7E00u : h;                         // canonical quiet NaN
  }
}

template <int DT>
__device__ __forceinline__ f32x4 dec16x4(u32x2 r) {
  f32x4 o;
  o.x = dec16<DT>(r.x & 0xFFFFu);
  o.y = dec16<DT>(r.x >> 16);
  o.z = dec16<DT>(r.y & 0xFFFFu);
  o.w = dec16<DT>(r.y >> 16);
  return o;
}

template <int DT>
__device__ __forceinline__ u32x2 enc16x4(f32x4 w) {
  u32x2 r;
  r.x = enc16<DT>(w.x) | (enc16<DT>(w.y) << 16);
  r.y = enc16<DT>(w.z) | (enc16<DT>(w.w) << 16);
  return r;
}

__device__ __forceinline__ u32x2 ld16x4(const uint16_t* p) { return *reinterpret_cast<const u32x2*>(p); }
// Gradient loads of the statistics pass.  A slice that fits in the Infinity Cache is
// read with plain loads, so the Adam pass finds it there; a larger one cannot stay
// cached until then, and non-temporal loads stream it faster (full state 2.40 ->
// 2.24 ms, GPT-2 shard 78 -> 67 us).
template <bool NT>
__device__ __forceinline__ u32x2 ld16x4_stats(const uint16_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  else return *reinterpret_cast<const u32x2*>(p);
}
// Vector loads of the sources of a local reduce or accumulation.  Each element is
// read once per step (the Adam pass reads the reduce's output instead), so they
// are marked non-temporal.
__device__ __forceinline__ u32x2 ld16x4_src(const uint16_t* p) {
#if ZS_REDUCE_NT
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
#else
  return *reinterpret_cast<const u32x2*>(p);
#endif
}
__device__ __forceinline__ void st16x4(uint16_t* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }
__device__ __forceinline__ void st16x4_nt(uint16_t* p, u32x2 v) {
#if ZS_NT_STORE
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
#else
  *reinterpret_cast<u32x2*>(p) = v;
#endif
}
// Device-scope stores of the 16-bit slice, used while segments are tracked: they
// are written through the XCD's L2, so once complete they are visible to every
// XCD without an L2 write-back.
__device__ __forceinline__ void st16x4_dev(uint16_t* p, u32x2 v) {
  const uint64_t bits = ((uint64_t)v[1] << 32) | (uint64_t)v[0];
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st16_dev(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4 ld32x4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 ld32x4_nt(const float* p) {
#if ZS_NT_LOAD
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
#else
  return *reinterpret_cast<const f32x4*>(p);
#endif
}
__device__ __forceinline__ void st32x4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ void st32x4_nt(float* p, f32x4 v) {
#if ZS_NT_STORE
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
#else
  *reinterpret_cast<f32x4*>(p) = v;
#endif
}

__device__ __forceinline__ bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Leading elements before a 16-bit pointer reaches an 8-byte boundary (0..3).
__device__ __forceinline__ int head16(const uint16_t* p) { return (int)(((8u - ((uintptr_t)p & 7u)) & 7u) >> 1); }

// ---------------------------------------------------------------------------
// chunk driver

// A chunk of `len` elements: `head` leading elements one per lane, then groups of
// V consecutive elements per lane (U groups in flight, each wave covering 64*V
// consecutive elements per group slot), then a tail of fewer than V elements.
// When the streams are not co-aligned (vec_ok false) every element goes one per lane.
template <int U, int V, class Op, int BS = kBlock>
__device__ __forceinline__ void run_chunk(Op& op, int64_t len, int head, bool vec_ok) {
  const int64_t tid = threadIdx.x;
  if (!vec_ok) {
    for (int64_t j = tid; j < len; j += BS) op.elem(j);
    return;
  }
  if (head > len) head = (int)len;
  if (tid < head) op.elem(tid);
  const int64_t ng = (len - head) / V;  // whole groups in the body
  int64_t q = tid;
  for (; q + (U - 1) * BS < ng; q += U * BS) op.template groups<U>(head + V * q, V * BS);
  for (; q < ng; q += BS) op.template groups<1>(head + V * q, 0);
  const int64_t t0 = head + V * ng;
  if (tid < len - t0) op.elem(t0 + tid);
}

// ---------------------------------------------------------------------------
// deterministic block reductions (fixed butterfly, fixed cross-wave order)

__device__ __forceinline__ double block_sum(double x, double* lds) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) lds[wave] = x;
  __syncthreads();
  double r = lds[0];
  for (int w = 1; w < kBlock / 64; ++w) r += lds[w];
  return r;
}

__device__ __forceinline__ void store_part(uint64_t* p, double v) {
  __hip_atomic_store(p, (uint64_t)__double_as_longlong(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double load_part(const uint64_t* p) {
  return __longlong_as_double((long long)__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
// Waits until this thread's device-scope stores have reached the device's coherence
// point, so that an arrival counted after it finds them there.
__device__ __forceinline__ void stores_complete() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Called by every block of an intake pass with its partial sum of squares: a
// deterministic two-level combine without float atomics or cache-wide fences.
// Block b stores its partial (device scope), waits for the store to complete and
// arrives on the counter of its group of kGroup blocks.  The group's last block
// adds the group's partials in block order (one per lane, fixed butterfly),
// stores the group sum and arrives on the pass counter; the last group's block
// adds the group sums in group order and publishes this rank's sum of squares and
// non-finite flag (the sum is non-finite exactly when some u is, see SumSq).
// Counters are re-armed by their last arrival.
__device__ void finish_stats(double acc, DevScalars* sc, const IntakeParts& p, int32_t flip) {
  __shared__ double lds[kBlock / 64];
  __shared__ int is_last;
  const double bsum = block_sum(acc, lds);
  const uint32_t b = blockIdx.x, nb = gridDim.x;
  const uint32_t g = b / kGroup, g0 = g * kGroup;
  const uint32_t gsize = nb - g0 < (uint32_t)kGroup ? nb - g0 : (uint32_t)kGroup;
  const uint32_t ngroups = (nb + kGroup - 1) / kGroup;
  if (threadIdx.x == 0) {
    store_part(p.part + b, bsum);
    stores_complete();
    const uint32_t prev = __hip_atomic_fetch_add(&p.gcount[g].count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = prev + 1 == gsize;
  }
  __syncthreads();
  if (!is_last) return;
  const double gsum = block_sum(threadIdx.x < gsize ? load_part(p.part + g0 + threadIdx.x) : 0.0, lds);
  if (threadIdx.x == 0) {
    __hip_atomic_store(&p.gcount[g].count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    store_part(p.gpart + g, gsum);
    stores_complete();
    const uint32_t prev = __hip_atomic_fetch_add(&sc->counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = prev + 1 == ngroups;
  }
  __syncthreads();
  if (!is_last) return;
  double s = 0.0;
  for (uint32_t i = threadIdx.x; i < ngroups; i += kBlock) s += load_part(p.gpart + i);
  const double total = block_sum(s, lds);
  if (threadIdx.x == 0) {
    sc->local_sumsq = total;
    sc->local_flag = !__builtin_isfinite(total);
    if (flip) sc->cur_slot ^= 1u;  // every block of the pass has read it by now
    __hip_atomic_store(&sc->counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// statistics pass over an already-reduced 16-bit gradient

// Sum of squares in fp64.  The square of a float is exact in fp64 (at most 48
// significant bits), so fma(d, d, acc) rounds exactly like acc + d * d.  One
// accumulator per group slot keeps the dependency chains short; they are added
// in a fixed order at the end.  No separate non-finite test is needed: a finite
// float squared is at most 1.2e77, so a sum of fewer than 2^63 of them stays
// finite, and the sum is non-finite exactly when some u is (squares are >= 0,
// so no inf - inf can occur).
struct SumSq {
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  __device__ __forceinline__ void add(int k, float u) {
    const double d = (double)u;
    acc[k & 3] = __builtin_fma(d, d, acc[k & 3]);
  }
  __device__ __forceinline__ double total() const { return ((acc[0] + acc[1]) + acc[2]) + acc[3]; }
};

template <int DT, bool NT>
struct Stats16Op {
  const uint16_t* g;
  float inv;
  SumSq& ss;
  __device__ __forceinline__ void elem(int64_t j) { ss.add(0, dec16<DT>(g[j]) * inv); }
  template <int U>
  __device__ __forceinline__ void groups(int64_t j, int64_t stride) {
    u32x2 r[U];  // 4 elements per group: 8-byte loads
#pragma unroll
    for (int k = 0; k < U; ++k) r[k] = ld16x4_stats<NT>(g + j + k * stride);
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const f32x4 x = dec16x4<DT>(r[k]);
#pragma unroll
      for (int e = 0; e < 4; ++e) ss.add(k, x[e] * inv);
    }
  }
};

struct StatsArgs {
  const Chunk* chunks;
  int64_t n_chunks;
  const uint16_t* flat_g;  // flat [psi] gradient, or null to use chunk.g16
  float inv;
  int32_t dyn;             // 1: unscale by 1 / the device-resident loss scale instead of inv
  int32_t cpb;             // consecutive chunks per block
  int32_t flip;            // 1: the step's first intake (its last block flips sc->cur_slot)
  DevScalars* sc;
  IntakeParts parts;
  int64_t plain_from;      // NT passes: chunks from this state offset on are read with plain loads
                           // (the slice's tail, left in the Infinity Cache for the Adam pass)
};

// The unscale factor of an intake pass: the call's inv, or 1 / the device-resident
// dynamic loss scale (fp32, correctly rounded) of the latest counters: slot
// cur_slot ^ 1 before the step's first intake flips cur_slot, slot cur_slot after.
__device__ __forceinline__ float intake_inv(float inv, int32_t dyn, int32_t flip, const DevScalars* sc) {
  return dyn ? 1.0f / sc->slot[flip ? sc->cur_slot ^ 1u : sc->cur_slot].scale : inv;
}

// The table fields an intake pass needs, held in scalar registers.
struct ChunkRef {
  int64_t state_off, flat_off;
  uint64_t g16;
  int64_t len;
};
__device__ __forceinline__ ChunkRef chunk_ref(const Chunk* c) { return ChunkRef{c->state_off, c->flat_off, c->g16, c->len}; }

// Walks block b's run of `cpb` consecutive chunks, calling body(ref).  The blocks
// are short-lived and dispatched in order, so the pass streams a compact window of
// the shard.  With ZS_STATS_PF and more than one chunk per block the next chunk's
// table entry is requested before the current chunk is streamed.
template <class Body>
__device__ __forceinline__ void walk_chunks(const Chunk* chunks, int64_t n_chunks, int32_t cpb, Body body) {
  const int64_t c0 = (int64_t)blockIdx.x * cpb;
  const int64_t c1 = c0 + cpb < n_chunks ? c0 + cpb : n_chunks;
  if (c0 >= c1) return;
#if ZS_STATS_PF
  if (cpb > 1) {
    ChunkRef ch = chunk_ref(chunks + c0);
    for (int64_t c = c0;;) {
      const int64_t cn = c + 1;
      const ChunkRef nx = chunk_ref(chunks + (cn < c1 ? cn : c));  // unconditional: nothing waits for it here
      body(ch);
      if (cn >= c1) break;
      ch = nx;
      c = cn;
    }
    return;
  }
#endif
  for (int64_t c = c0; c < c1; ++c) body(chunk_ref(chunks + c));
}

// Part `part` of `n_parts` of a chunk of `chunk_len` elements: [lo, lo + len), every
// part but the last of a length that is a multiple of 8, so the parts keep the chunk's
// alignment.  Trailing parts of a short chunk are empty (len <= 0).
struct Part {
  int64_t lo, len;
};
__device__ __forceinline__ Part chunk_part(int64_t chunk_len, int64_t part, int64_t n_parts) {
  const int64_t sub = ((chunk_len + n_parts - 1) / n_parts + 7) & ~(int64_t)7;
  const int64_t lo = part * sub;
  return Part{lo, (lo + sub < chunk_len ? lo + sub : chunk_len) - lo};
}

// Walks block b's part (b % ppc) of chunk b / ppc.  ppc == 1 walks one whole chunk per block.
template <class Body>
__device__ __forceinline__ void walk_parts(const Chunk* chunks, int64_t n_chunks, int32_t ppc, Body body) {
  const int64_t c = (int64_t)blockIdx.x / ppc;
  if (c >= n_chunks) return;
  ChunkRef ch = chunk_ref(chunks + c);
  if (ppc > 1) {
    const Part p = chunk_part(ch.len, (int64_t)blockIdx.x % ppc, ppc);
    if (p.lo >= ch.len) return;
    ch.len = p.len;
    ch.state_off += p.lo;
    ch.flat_off += p.lo;
    if (ch.g16) ch.g16 += 2 * (uint64_t)p.lo;
  }
  body(ch);
}

// TAIL (with NT): chunks from a.plain_from on are read with plain loads.
template <int DT, bool NT, bool TAIL>
__global__ void __launch_bounds__(kBlock) stats16_kernel(StatsArgs a) {
  SumSq ss;
  Stats16Op<DT, NT> op{nullptr, intake_inv(a.inv, a.dyn, a.flip, a.sc), ss};
  Stats16Op<DT, false> op_plain{nullptr, op.inv, ss};
  walk_chunks(a.chunks, a.n_chunks, a.cpb, [&](const ChunkRef ch) {
    const uint16_t* g = a.flat_g ? a.flat_g + ch.flat_off : reinterpret_cast<const uint16_t*>(ch.g16);
    if (TAIL && ch.state_off >= a.plain_from) {
      op_plain.g = g;
      run_chunk<ZS_STATS_U, 4>(op_plain, ch.len, head16(g), true);
    } else {
      op.g = g;
      run_chunk<ZS_STATS_U, 4>(op, ch.len, head16(g), true);
    }
  });
  finish_stats(ss.total(), a.sc, a.parts, a.flip);
}

// ---------------------------------------------------------------------------
// local reduce of N rank buffers (rank order, fp32) + unscale + statistics

struct ReduceArgs {
  const Chunk* chunks;
  int64_t n_chunks;
  const uint16_t* ranks[kMaxRanks];
  int32_t n_ranks;
  float inv;
  int32_t dyn;             // as in StatsArgs
  float* red;
  int32_t ppc;             // parts per chunk of the local-reduce intake passes
  int32_t flip;            // as in StatsArgs
  DevScalars* sc;
  IntakeParts parts;
  int64_t keep_from;       // outputs from this state offset on are stored with plain stores
};

// Gradient sources of the intake passes.  NR > 0: that many rank buffers
// (specialised fan-in); kSrcRanksN: a runtime number of rank buffers (>= 1);
// kSrcChunk: the gradient registered at init (one already-reduced source per
// chunk); kSrcNone: no new gradient (the accumulated one alone).
enum { kSrcRanksN = 0, kSrcChunk = -1, kSrcNone = -2 };

// The 16-bit output of the local reduce: the fp32 sum rounded once to the 16-bit
// type (nearest even), as the step then takes it in.
template <int DT>
__device__ __forceinline__ float round16(float s) { return dec16<DT>(enc16<DT>(s)); }
template <int DT>
__device__ __forceinline__ f32x4 round16x4(f32x4 s) { return dec16x4<DT>(enc16x4<DT>(s)); }

// s = the rank-order fp32 sum of this element's sources (g_0 + g_1 + ...).
template <int DT, int NR>
struct GradSum {
  const ReduceArgs* a;
  const uint16_t* src0;  // registered chunk source (kSrcChunk)
  int64_t flat_off;      // rank buffers are flat
  __device__ __forceinline__ int nranks() const { return NR > 0 ? NR : a->n_ranks; }
  __device__ __forceinline__ const uint16_t* src(int q) const {
    return NR == kSrcChunk ? src0 : a->ranks[q] + flat_off;
  }
  __device__ __forceinline__ float one(int64_t j) const {
    float r = dec16<DT>(src(0)[j]);
    if constexpr (NR != kSrcChunk)
      for (int q = 1; q < nranks(); ++q) r = r + dec16<DT>(src(q)[j]);
    return r;
  }
  template <int U>
  __device__ __forceinline__ void quads(int64_t j, int64_t stride, f32x4 (&s)[U]) const {
    if constexpr (NR > 0) {
      u32x2 raw[NR][U];
#pragma unroll
      for (int q = 0; q < NR; ++q)
#pragma unroll
        for (int k = 0; k < U; ++k) raw[q][k] = ld16x4_src(src(q) + j + k * stride);
#pragma unroll
      for (int k = 0; k < U; ++k) {
        s[k] = dec16x4<DT>(raw[0][k]);
#pragma unroll
        for (int q = 1; q < NR; ++q) s[k] = s[k] + dec16x4<DT>(raw[q][k]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < U; ++k) s[k] = dec16x4<DT>(ld16x4_src(src(0) + j + k * stride));
      if constexpr (NR != kSrcChunk)
        for (int q = 1; q < nranks(); ++q)
#pragma unroll
          for (int k = 0; k < U; ++k) s[k] = s[k] + dec16x4<DT>(ld16x4_src(src(q) + j + k * stride));
    }
  }
  // leading elements to peel, and co-alignment of every source with the fp32 buffer after them
  __device__ __forceinline__ int head(const float* red) const {
    if constexpr (NR == kSrcNone) return (int)(((16u - ((uintptr_t)red & 15u)) & 15u) >> 2);
    else return head16(src(0));
  }
  __device__ __forceinline__ bool aligned_at(int h, const float* red) const {
    bool ok = aligned(red + h, 16);
    if constexpr (NR != kSrcNone)
      for (int q = 0; q < (NR == kSrcChunk ? 1 : nranks()); ++q) ok = ok && aligned(src(q) + h, 8);
    return ok;
  }
};

// Intake with statistics: u = (ACC ? red + s : s) * inv stored in red, plus the
// fp64 sum of squares.  With kSrcNone, u = red * inv.  R16: the new sources' sum s
// arrives as a 16-bit reduce output (rounded once) before it is added.  !STORE:
// statistics only; red keeps the accumulator and the Adam pass recomputes u.
template <int DT, int NR, bool ACC, bool R16 = false, bool STORE = true>
struct ReduceOp {
  GradSum<DT, NR> gs;
  float* red;
  float inv;
  SumSq ss;
  int32_t keep;  // plain stores: the output stays in the Infinity Cache
  __device__ __forceinline__ void elem(int64_t j) {
    float r;
    if constexpr (NR == kSrcNone) r = red[j];
    else if constexpr (ACC) r = red[j] + (R16 ? round16<DT>(gs.one(j)) : gs.one(j));
    else r = R16 ? round16<DT>(gs.one(j)) : gs.one(j);
    const float u = r * inv;
    ss.add(0, u);
    if constexpr (STORE) red[j] = u;
  }
  template <int U>
  __device__ __forceinline__ void groups(int64_t j, int64_t stride) {
    f32x4 s[U];
    if constexpr (NR != kSrcNone) gs.template quads<U>(j, stride, s);
    if constexpr (R16 && NR != kSrcNone)
#pragma unroll
      for (int k = 0; k < U; ++k) s[k] = round16x4<DT>(s[k]);
    if constexpr (ACC || NR == kSrcNone) {
      f32x4 acc[U];
#pragma unroll
      for (int k = 0; k < U; ++k) acc[k] = ld32x4_nt(red + j + k * stride);
#pragma unroll
      for (int k = 0; k < U; ++k) {
        if constexpr (NR == kSrcNone) s[k] = acc[k];
        else s[k] = acc[k] + s[k];
      }
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const f32x4 u = s[k] * inv;
#pragma unroll
      for (int e = 0; e < 4; ++e) ss.add(k, u[e]);
      if constexpr (STORE) {
        if (keep) st32x4(red + j + k * stride, u);
        else st32x4_nt(red + j + k * stride, u);
      }
    }
  }
};

template <int DT, int NR, bool ACC, bool R16 = false, bool STORE = true>
__global__ void __launch_bounds__(kBlock) reduce_kernel(ReduceArgs a) {
  ReduceOp<DT, NR, ACC, R16, STORE> op{GradSum<DT, NR>{&a, nullptr, 0}, nullptr, intake_inv(a.inv, a.dyn, a.flip, a.sc),
                                SumSq{}, 0};
  walk_parts(a.chunks, a.n_chunks, a.ppc, [&](const ChunkRef ch) {
    op.keep = ch.state_off >= a.keep_from;
    op.gs.flat_off = ch.flat_off;
    op.gs.src0 = reinterpret_cast<const uint16_t*>(ch.g16);
    op.red = a.red + ch.state_off;
    const int head = op.gs.head(op.red);
    run_chunk<ZS_REDUCE_U, 4>(op, ch.len, head, op.gs.aligned_at(head, op.red));
  });
  finish_stats(op.ss.total(), a.sc, a.parts, a.flip);
}

// Intake with a 16-bit reduce output: h = RNE16(s) is stored in red16 (this rank's
// reduce-scatter result, in the state layout), then u = f32(h) * inv and the fp64
// sum of squares of u.  The Adam pass re-reads h.
template <int DT, int NR>
struct Reduce16Op {
  GradSum<DT, NR> gs;
  uint16_t* red16;
  float inv;
  SumSq ss;
  int32_t keep;  // plain stores: the output stays in the Infinity Cache
  __device__ __forceinline__ void elem(int64_t j) {
    const uint32_t h = enc16<DT>(gs.one(j));
    red16[j] = (uint16_t)h;
    ss.add(0, dec16<DT>(h) * inv);
  }
  template <int U>
  __device__ __forceinline__ void groups(int64_t j, int64_t stride) {
    f32x4 s[U];
    gs.template quads<U>(j, stride, s);
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const u32x2 h = enc16x4<DT>(s[k]);
      if (keep) st16x4(red16 + j + k * stride, h);
      else st16x4_nt(red16 + j + k * stride, h);
      const f32x4 u = dec16x4<DT>(h) * inv;
#pragma unroll
      for (int e = 0; e < 4; ++e) ss.add(k, u[e]);
    }
  }
};

template <int DT, int NR>
__global__ void __launch_bounds__(kBlock) reduce16_kernel(ReduceArgs a) {
  Reduce16Op<DT, NR> op{GradSum<DT, NR>{&a, nullptr, 0}, nullptr, intake_inv(a.inv, a.dyn, a.flip, a.sc), SumSq{},
                        0};
  walk_parts(a.chunks, a.n_chunks, a.ppc, [&](const ChunkRef ch) {
    op.keep = ch.state_off >= a.keep_from;
    op.gs.flat_off = ch.flat_off;
    op.red16 = reinterpret_cast<uint16_t*>(a.red) + ch.state_off;
    const int head = head16(op.gs.src(0));
    bool ok = aligned(op.red16 + head, 8);
    for (int q = 0; q < op.gs.nranks(); ++q) ok = ok && aligned(op.gs.src(q) + head, 8);
    run_chunk<ZS_REDUCE_U, 4>(op, ch.len, head, ok);
  });
  finish_stats(op.ss.total(), a.sc, a.parts, a.flip);
}

// One micro-step into the accumulator, no statistics: red = FIRST ? s : red + s.
// R16: s arrives as a 16-bit reduce output (rounded once) before it is added.
template <int DT, int NR, bool FIRST, bool R16 = false>
struct AccumOp {
  GradSum<DT, NR> gs;
  float* red;
  __device__ __forceinline__ void elem(int64_t j) {
    const float s = R16 ? round16<DT>(gs.one(j)) : gs.one(j);
    red[j] = FIRST ? s : red[j] + s;
  }
  template <int U>
  __device__ __forceinline__ void groups(int64_t j, int64_t stride) {
    f32x4 s[U];
    gs.template quads<U>(j, stride, s);
    if constexpr (R16)
#pragma unroll
      for (int k = 0; k < U; ++k) s[k] = round16x4<DT>(s[k]);
    if constexpr (!FIRST) {
      f32x4 acc[U];
#pragma unroll
      for (int k = 0; k < U; ++k) acc[k] = ld32x4_nt(red + j + k * stride);
#pragma unroll
      for (int k = 0; k < U; ++k) s[k] = acc[k] + s[k];
    }
#pragma unroll
    for (int k = 0; k < U; ++k) st32x4_nt(red + j + k * stride, s[k]);
  }
};

// One short-lived block per part of a chunk, as in the Adam pass.
template <int DT, int NR, bool FIRST, bool R16 = false>
__global__ void __launch_bounds__(kBlock) accum_kernel(ReduceArgs a) {
  AccumOp<DT, NR, FIRST, R16> op{GradSum<DT, NR>{&a, nullptr, 0}, nullptr};
  const int64_t n_items = a.n_chunks * ZS_ADAM_SPLIT;
  for (int64_t i = blockIdx.x; i < n_items; i += gridDim.x) {
    const Chunk ch = a.chunks[i / ZS_ADAM_SPLIT];
    const Part p = chunk_part(ch.len, i % ZS_ADAM_SPLIT, ZS_ADAM_SPLIT);
    if (p.lo >= ch.len) continue;
    op.gs.flat_off = ch.flat_off + p.lo;
    op.gs.src0 = reinterpret_cast<const uint16_t*>(ch.g16) + p.lo;
    op.red = a.red + ch.state_off + p.lo;
    const int head = op.gs.head(op.red);
    run_chunk<ZS_REDUCE_U, 4>(op, p.len, head, op.gs.aligned_at(head, op.red));
  }
}

// ---------------------------------------------------------------------------
// Adam with bias correction, decoupled weight decay, clip; optional fused cast

struct AdamScalars {
  float inv, clip, b1, b2, omb1, omb2, bc1, bc2, lr, eps, wd;
};

__device__ __forceinline__ void adam_elem(float u, float& w, float& m, float& v, const AdamScalars& s) {
  const float g = u * s.clip;
  const float mi = s.b1 * m + s.omb1 * g;
  const float vi = s.b2 * v + s.omb2 * (g * g);
  const float mh = mi / s.bc1;
  const float vh = vi / s.bc2;
  const float den = __builtin_sqrtf(vh) + s.eps;
  const float upd = mh / den;
  w = w - s.lr * (upd + s.wd * w);
  m = mi;
  v = vi;
}

// Gradient sources of the Adam pass (GradSource): the flat or registered 16-bit
// gradient, the fp32 u of a reduce, the 16-bit reduce output (in red, state layout),
// or, after an intake on top of an accumulation from one source or none, u
// recomputed from the accumulator with the intake's own operations.
template <int GS>
constexpr bool grad_from_acc() { return GS == kGradAcc || GS == kGradAccFlat16 || GS == kGradAccChunk16; }
template <int GS>
constexpr bool grad_acc16() { return GS == kGradAccFlat16 || GS == kGradAccChunk16; }

template <int DT, int GS, bool CAST, bool WT>
struct AdamOp {
  const uint16_t* g16;
  const float* gred;
  float* w;
  float* m;
  float* v;
  uint16_t* p16;
  AdamScalars s;
  __device__ __forceinline__ float grad(int64_t j) const {
    if constexpr (GS == kGradRed) return gred[j];
    else if constexpr (GS == kGradAcc) return gred[j] * s.inv;
    else if constexpr (grad_acc16<GS>()) return (gred[j] + dec16<DT>(g16[j])) * s.inv;
    else return dec16<DT>(g16[j]) * s.inv;
  }
  __device__ __forceinline__ void elem(int64_t j) {
    float wj = w[j], mj = m[j], vj = v[j];
    adam_elem(grad(j), wj, mj, vj, s);
    w[j] = wj;
    m[j] = mj;
    v[j] = vj;
    if constexpr (CAST) {
      if constexpr (WT) st16_dev(p16 + j, (uint16_t)enc16<DT>(wj));
      else p16[j] = (uint16_t)enc16<DT>(wj);
    }
  }
  template <int U>
  __device__ __forceinline__ void groups(int64_t j, int64_t stride) {
    f32x4 G[U], W[U], M[U], V[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int64_t o = j + k * stride;
      if constexpr (GS == kGradRed) {
        G[k] = ld32x4_nt(gred + o);
      } else if constexpr (GS == kGradAcc) {
        G[k] = ld32x4_nt(gred + o) * s.inv;
      } else if constexpr (grad_acc16<GS>()) {
        G[k] = (ld32x4_nt(gred + o) + dec16x4<DT>(ld16x4(g16 + o))) * s.inv;
      } else {
        G[k] = dec16x4<DT>(ld16x4(g16 + o)) * s.inv;
      }
      W[k] = ld32x4_nt(w + o);
      M[k] = ld32x4_nt(m + o);
      V[k] = ld32x4_nt(v + o);
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float we = W[k][e], me = M[k][e], ve = V[k][e];
        adam_elem(G[k][e], we, me, ve, s);
        W[k][e] = we;
        M[k][e] = me;
        V[k][e] = ve;
      }
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int64_t o = j + k * stride;
      st32x4_nt(w + o, W[k]);
      st32x4_nt(m + o, M[k]);
      st32x4_nt(v + o, V[k]);
      if constexpr (CAST) {
        if constexpr (WT) st16x4_dev(p16 + o, enc16x4<DT>(W[k]));
        else st16x4_nt(p16 + o, enc16x4<DT>(W[k]));
      }
    }
  }
};

struct AdamArgs {
  const Chunk* chunks;
  int64_t n_chunks;
  const uint16_t* flat_g;  // kGradFlat16 source
  const float* red;        // kGradRed source (kGradRed16: 16-bit values in the same buffer)
  float* master;
  float* m;
  float* v;
  DevScalars* sc;
  int32_t other_flag;
  double other_sumsq;      // the other ranks' sum of squares, or (sumsq_global) the global sum
  int32_t sumsq_global;
  float max_norm;
  float inv;
  float lr, beta1, beta2, eps, wd;
  int32_t dyn;             // dynamic loss scale: unscale by 1 / slot.scale and update it
  float growth, backoff, min_scale;
  int32_t interval;
  SegArgs seg;             // segment completion flags (seg.seg null: none)
  int32_t reverse;         // walk the work items from the last (the cached tail of the gradient first)
};

// ---------------------------------------------------------------------------
// segment completion (chunk-pipelined step)

// Called by every thread of a block after it has written work item `i` (of
// `items_per_chunk` per chunk) of chunk `c` of the 16-bit slice, with
// device-scope stores; uniform over the block.  Each wave waits until its
// stores are complete -- written through to the device's coherence point --
// and after the barrier one thread arrives.  Whoever completes a sub-counter
// arrives on the segment's counter, and whoever completes that publishes the
// epoch, so once a consumer reads epoch >= e, every element of the segment as
// written by step e is in device-coherent memory.  (An agent-scope release
// fence here would write back the XCD's whole L2 for every work item: measured
// about 20x slower than the Adam pass itself.  One counter per segment instead
// of sub-counters serialises the atomics: +15% on the Adam pass at 64
// segments, +35% at 8.)
__device__ __forceinline__ void seg_arrive(const SegArgs& g, int64_t i, int64_t c, int items_per_chunk) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t k = c / g.per_seg;
    const int64_t c_end = (k + 1) * g.per_seg < g.n_chunks ? (k + 1) * g.per_seg : g.n_chunks;
    const int64_t i0 = k * g.per_seg * items_per_chunk, i1 = c_end * items_per_chunk;
    const int64_t j = i % kSegSubs;
    // items of [i0, i1) that fall on sub-counter j: count of x < bound with x % kSegSubs == j
    auto below = [j](int64_t bound) { return bound > j ? (bound - j - 1) / kSegSubs + 1 : (int64_t)0; };
    const uint32_t sub_target = (uint32_t)(below(i1) - below(i0));
    const uint32_t top_target = (uint32_t)(i1 - i0 < kSegSubs ? i1 - i0 : kSegSubs);
    SegState* s = g.seg + k;
    const uint32_t old = __hip_atomic_fetch_add(&s->sub[j].count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 == sub_target) {
      __hip_atomic_store(&s->sub[j].count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t top = __hip_atomic_fetch_add(&s->count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (top + 1 == top_target) {
        __hip_atomic_store(&s->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&s->epoch, g.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// A skipped step writes nothing: every segment is complete at once.
__device__ __forceinline__ void seg_publish_all(const SegArgs& g) {
  for (int k = 0; k < g.n_seg; ++k)
    __hip_atomic_store(&g.seg[k].epoch, g.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// One lane polls segment k until step `epoch` has published it, sleeping
// between polls; after max_polls it gives up and counts a timeout, so the
// wait always ends.  Every wait polls on its own: an earlier timeout does not
// shorten a later wait.
__global__ void seg_wait_kernel(const SegState* seg, int32_t k, uint64_t epoch, int64_t max_polls,
                                DevScalars* sc) {
  if (threadIdx.x != 0) return;
  for (int64_t n = 0;; ++n) {
    // relaxed polls (device scope, no cache invalidation each time); one acquire at the end
    const uint64_t e = __hip_atomic_load(&seg[k].epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (e >= epoch) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      return;
    }
    if (n >= max_polls) {
      __hip_atomic_fetch_add(&sc->wait_timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(32);
  }
}

// Step scalars, computed identically by every block from the device scalar
// block and the call's arguments.  Returns the skip decision.
__device__ __forceinline__ int step_scalars(const AdamArgs& a, AdamScalars& s, Slot& next, double& norm) {
  const DevScalars* sc = a.sc;
  const int skip = (sc->local_flag | a.other_flag) != 0;
  norm = sqrt(a.sumsq_global ? a.other_sumsq : sc->local_sumsq + a.other_sumsq);
  float clip = 1.0f;
  if (a.max_norm > 0.0f) {
    const double c = (double)a.max_norm / (norm + 1e-6);
    if (c < 1.0) clip = (float)c;
  }
  const Slot cur = sc->slot[sc->cur_slot];
  next = cur;
  if (!skip) {
    next.t = cur.t + 1;
    next.p1 = cur.p1 * (double)a.beta1;
    next.p2 = cur.p2 * (double)a.beta2;
  }
  if (a.dyn) {
    // backoff on an overflow step (not below the floor), growth after `interval` good steps
    if (skip) {
      const float b = cur.scale * a.backoff;
      next.scale = b < a.min_scale ? a.min_scale : b;
      next.good = 0;
    } else {
      next.good = cur.good + 1;
      if (next.good == a.interval) {
        const float grown = cur.scale * a.growth;
        if (__builtin_isfinite(grown)) next.scale = grown;  // never grow to infinity
        next.good = 0;
      }
    }
  }
  s.inv = a.dyn ? 1.0f / cur.scale : a.inv;
  s.clip = clip;
  s.b1 = a.beta1;
  s.b2 = a.beta2;
  s.omb1 = 1.0f - a.beta1;
  s.omb2 = 1.0f - a.beta2;
  s.bc1 = (float)(1.0 - next.p1);
  s.bc2 = (float)(1.0 - next.p2);
  s.lr = a.lr;
  s.eps = a.eps;
  s.wd = a.wd;
  return skip;
}

// Parts per chunk of the Adam pass for a gradient source.
__host__ __device__ constexpr int adam_split(int gs) { return gs == kGradRed ? ZS_ADAM_SPLIT_RED : ZS_ADAM_SPLIT; }

template <int DT, int GS, bool CAST, bool SEG>
__global__ void __launch_bounds__(ZS_ADAM_BLOCK) adam_kernel(AdamArgs a) {
  constexpr int64_t kSplit = adam_split(GS);
  AdamScalars s;
  Slot next;
  double norm;
  const int skip = step_scalars(a, s, next, norm);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.sc->slot[a.sc->cur_slot ^ 1u] = next;
    a.sc->norm = norm;
    a.sc->clip = s.clip;
    a.sc->skipped = skip;
    a.sc->report_t = next.t;
    if (SEG && skip) seg_publish_all(a.seg);
  }
  if (skip) return;
  AdamOp<DT, GS, CAST, SEG> op{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, s};
  // Work item i is part i % kSplit of chunk i / kSplit: one short-lived block per part,
  // scheduled by the hardware dispatcher (measured faster than a persistent grid here).
  const int64_t n_items = a.n_chunks * kSplit;
  for (int64_t i0 = blockIdx.x; i0 < n_items; i0 += gridDim.x) {
    const int64_t i = a.reverse ? n_items - 1 - i0 : i0;
    const Chunk ch = a.chunks[i / kSplit];
    const Part p = chunk_part(ch.len, i % kSplit, kSplit);
    if (p.lo < ch.len) {
      const int64_t lo = p.lo;
      op.w = a.master + ch.state_off + lo;
      op.m = a.m + ch.state_off + lo;
      op.v = a.v + ch.state_off + lo;
      op.p16 = reinterpret_cast<uint16_t*>(ch.p16) + lo;
      int head;
      bool ok;
      if constexpr (GS == kGradRed || GS == kGradAcc) {
        op.gred = a.red + ch.state_off + lo;
        head = head16(op.p16);
        ok = aligned(op.w + head, 16) && aligned(op.gred + head, 16);
      } else {
        op.g16 = (GS == kGradFlat16 || GS == kGradAccFlat16 ? a.flat_g + ch.flat_off
                  : GS == kGradRed16 ? reinterpret_cast<const uint16_t*>(a.red) + ch.state_off
                                     : reinterpret_cast<const uint16_t*>(ch.g16)) +
                 lo;
        head = head16(op.g16);
        ok = aligned(op.w + head, 16) && aligned(op.g16 + head, 8);
        if constexpr (grad_acc16<GS>()) {
          op.gred = a.red + ch.state_off + lo;
          ok = ok && aligned(op.gred + head, 16);
        }
      }
      if constexpr (CAST) ok = ok && aligned(op.p16 + head, 8);
      ok = ok && aligned(op.m + head, 16) && aligned(op.v + head, 16);
      run_chunk<ZS_ADAM_U, 4, AdamOp<DT, GS, CAST, SEG>, ZS_ADAM_BLOCK>(op, p.len, head, ok);
    }
    if constexpr (SEG) seg_arrive(a.seg, i, i / kSplit, (int)kSplit);
  }
}

// ---------------------------------------------------------------------------
// standalone write-back, init, export, fill

template <int DT, bool WT>
struct CastOp {
  const float* w;
  uint16_t* p16;
  __device__ __forceinline__ void elem(int64_t j) {
    if constexpr (WT) st16_dev(p16 + j, (uint16_t)enc16<DT>(w[j]));
    else p16[j] = (uint16_t)enc16<DT>(w[j]);
  }
  template <int U>
  __device__ __forceinline__ void groups(int64_t j, int64_t stride) {
    f32x4 W[U];
#pragma unroll
    for (int k = 0; k < U; ++k) W[k] = ld32x4_nt(w + j + k * stride);
#pragma unroll
    for (int k = 0; k < U; ++k) {
      if constexpr (WT) st16x4_dev(p16 + j + k * stride, enc16x4<DT>(W[k]));
      else st16x4_nt(p16 + j + k * stride, enc16x4<DT>(W[k]));
    }
  }
};

template <int DT, bool SEG>
__global__ void __launch_bounds__(kBlock) cast_kernel(const Chunk* chunks, int64_t n_chunks, const float* master,
                                                      const DevScalars* sc, SegArgs seg) {
  if (sc->skipped) {
    if (SEG && blockIdx.x == 0 && threadIdx.x == 0) seg_publish_all(seg);
    return;
  }
  CastOp<DT, SEG> op{nullptr, nullptr};
  for (int64_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
    const Chunk ch = chunks[c];
    op.w = master + ch.state_off;
    op.p16 = reinterpret_cast<uint16_t*>(ch.p16);
    const int head = head16(op.p16);
    run_chunk<4, 4>(op, ch.len, head, aligned(op.w + head, 16));
    if constexpr (SEG) seg_arrive(seg, c, c, 1);
  }
}

template <int DT>
__global__ void __launch_bounds__(kBlock) init_kernel(const Chunk* chunks, int64_t n_chunks, float* master,
                                                      const float* master_init) {
  for (int64_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
    const Chunk ch = chunks[c];
    const uint16_t* p = reinterpret_cast<const uint16_t*>(ch.p16);
    float* w = master + ch.state_off;
    for (int64_t j = threadIdx.x; j < ch.len; j += kBlock)
      w[j] = master_init ? master_init[ch.shard_off + j] : dec16<DT>(p[j]);
  }
}

__global__ void __launch_bounds__(kBlock) export_kernel(const Chunk* chunks, int64_t n_chunks, const float* src,
                                                        float* dst) {
  for (int64_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
    const Chunk ch = chunks[c];
    for (int64_t j = threadIdx.x; j < ch.len; j += kBlock) dst[ch.shard_off + j] = src[ch.state_off + j];
  }
}

__global__ void __launch_bounds__(kBlock) fill_zero_kernel(float* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x; j < n; j += stride) p[j] = 0.0f;
}

__global__ void empty_stats_kernel(DevScalars* sc, int32_t flip) {
  sc->local_sumsq = 0.0;
  sc->local_flag = 0;
  if (flip) sc->cur_slot ^= 1u;
}

// ---------------------------------------------------------------------------
// launchers (host)

struct Launch {
  hipStream_t stream;
  unsigned grid;
};

static unsigned clamp_grid(int64_t n_chunks, int64_t cap) {
  int64_t g = n_chunks < cap ? n_chunks : cap;
  return (unsigned)(g < 1 ? 1 : g);
}

// Grid of an intake pass: one short-lived block per run of cpb chunks.
static unsigned intake_grid(int64_t n_chunks, int32_t cpb) {
  return clamp_grid((n_chunks + cpb - 1) / cpb, n_chunks);
}

// Whether the statistics pass over a 16-bit slice of slice_elems elements reads its tail with
// plain loads: a slice too large for the Infinity Cache (read non-temporally otherwise) but
// not so large that the tail's share of the re-read is negligible (beyond 16 times the tail
// the statistics kernel's extra load path costs about what the tail saves).
static bool stats_tail_cached(int64_t slice_elems) {
  return 2 * slice_elems > (int64_t)ZS_STATS_NT_BYTES && ZS_STATS_TAIL_BYTES > 0 &&
         2 * slice_elems <= 16 * (int64_t)ZS_STATS_TAIL_BYTES;
}

// The local reduce stores its output of `bytes` per element with plain stores from this
// state offset on (the last ZS_REDUCE_TAIL_BYTES of it, or all of it when it fits), so
// that part stays in the Infinity Cache for the Adam pass.
static int64_t reduce_keep_from(int64_t slice_elems, int bytes) {
  if (ZS_REDUCE_TAIL_BYTES <= 0) return INT64_MAX;
  const int64_t keep = (int64_t)ZS_REDUCE_TAIL_BYTES / bytes;
  return slice_elems > keep ? slice_elems - keep : 0;
}
// Whether only a tail of that output is cached (so the Adam pass should start at the end).
static bool reduce_tail_cached(int64_t slice_elems, int bytes) {
  const int64_t from = reduce_keep_from(slice_elems, bytes);
  return from > 0 && from != INT64_MAX;
}

hipError_t launch_stats16(int dtype, const Chunk* chunks, int64_t n_chunks, int64_t slice_elems,
                          const uint16_t* flat_g, float inv, bool dyn, bool flip, DevScalars* sc,
                          const IntakeParts& parts, hipStream_t st) {
  if (n_chunks == 0) {
    hipLaunchKernelGGL(empty_stats_kernel, dim3(1), dim3(1), 0, st, sc, (int32_t)flip);
    return hipGetLastError();
  }
  const int32_t cpb = n_chunks < ZS_STATS_SMALL ? ZS_STATS_SMALL_CPB : 1;
  const bool nt = 2 * slice_elems > (int64_t)ZS_STATS_NT_BYTES;
  const bool tail = stats_tail_cached(slice_elems);
  const int64_t plain_from = tail ? slice_elems - (int64_t)ZS_STATS_TAIL_BYTES / 2 : INT64_MAX;
  StatsArgs a{chunks, n_chunks, flat_g, inv, (int32_t)dyn, cpb, (int32_t)flip, sc, parts, plain_from};
  const unsigned g = intake_grid(n_chunks, cpb);
  if (dtype == ZERO_BF16) {
    if (tail) hipLaunchKernelGGL((stats16_kernel<ZERO_BF16, true, true>), dim3(g), dim3(kBlock), 0, st, a);
    else if (nt) hipLaunchKernelGGL((stats16_kernel<ZERO_BF16, true, false>), dim3(g), dim3(kBlock), 0, st, a);
    else hipLaunchKernelGGL((stats16_kernel<ZERO_BF16, false, false>), dim3(g), dim3(kBlock), 0, st, a);
  } else {
    if (tail) hipLaunchKernelGGL((stats16_kernel<ZERO_F16, true, true>), dim3(g), dim3(kBlock), 0, st, a);
    else if (nt) hipLaunchKernelGGL((stats16_kernel<ZERO_F16, true, false>), dim3(g), dim3(kBlock), 0, st, a);
    else hipLaunchKernelGGL((stats16_kernel<ZERO_F16, false, false>), dim3(g), dim3(kBlock), 0, st, a);
  }
  return hipGetLastError();
}

// Rank-buffer reduces whose micro-step sum arrives as a 16-bit reduce output (R16);
// a single source needs no rounding (a 16-bit value rounds to itself).
template <int DT>
static void launch_reduce_acc_r16(const ReduceArgs& a, int src, unsigned g, hipStream_t st) {
  switch (src) {
    case 2: hipLaunchKernelGGL((reduce_kernel<DT, 2, true, true>), dim3(g), dim3(kBlock), 0, st, a); break;
    case 4: hipLaunchKernelGGL((reduce_kernel<DT, 4, true, true>), dim3(g), dim3(kBlock), 0, st, a); break;
    case 8: hipLaunchKernelGGL((reduce_kernel<DT, 8, true, true>), dim3(g), dim3(kBlock), 0, st, a); break;
    default: hipLaunchKernelGGL((reduce_kernel<DT, kSrcRanksN, true, true>), dim3(g), dim3(kBlock), 0, st, a); break;
  }
}

template <int DT>
static void launch_reduce16_src(const ReduceArgs& a, int src, unsigned g, hipStream_t st) {
  switch (src) {
    case 2: hipLaunchKernelGGL((reduce16_kernel<DT, 2>), dim3(g), dim3(kBlock), 0, st, a); break;
    case 4: hipLaunchKernelGGL((reduce16_kernel<DT, 4>), dim3(g), dim3(kBlock), 0, st, a); break;
    case 8: hipLaunchKernelGGL((reduce16_kernel<DT, 8>), dim3(g), dim3(kBlock), 0, st, a); break;
    default: hipLaunchKernelGGL((reduce16_kernel<DT, kSrcRanksN>), dim3(g), dim3(kBlock), 0, st, a); break;
  }
}

template <int DT, bool FIRST>
static void launch_accum_r16(const ReduceArgs& a, int src, unsigned g, hipStream_t st) {
  switch (src) {
    case 2: hipLaunchKernelGGL((accum_kernel<DT, 2, FIRST, true>), dim3(g), dim3(kBlock), 0, st, a); break;
    case 4: hipLaunchKernelGGL((accum_kernel<DT, 4, FIRST, true>), dim3(g), dim3(kBlock), 0, st, a); break;
    case 8: hipLaunchKernelGGL((accum_kernel<DT, 8, FIRST, true>), dim3(g), dim3(kBlock), 0, st, a); break;
    default: hipLaunchKernelGGL((accum_kernel<DT, kSrcRanksN, FIRST, true>), dim3(g), dim3(kBlock), 0, st, a); break;
  }
}

static bool is_rank_reduce(int src) { return src == 2 || src == 4 || src == 8 || src == kSrcRanksN; }

template <int DT, bool ACC>
static void launch_reduce_acc(const ReduceArgs& a, int src, unsigned g, hipStream_t st) {
  switch (src) {
    case 1: hipLaunchKernelGGL((reduce_kernel<DT, 1, ACC>), dim3(g), dim3(kBlock), 0, st, a); break;
    case 2: hipLaunchKernelGGL((reduce_kernel<DT, 2, ACC>), dim3(g), dim3(kBlock), 0, st, a); break;
    case 4: hipLaunchKernelGGL((reduce_kernel<DT, 4, ACC>), dim3(g), dim3(kBlock), 0, st, a); break;
    case 8: hipLaunchKernelGGL((reduce_kernel<DT, 8, ACC>), dim3(g), dim3(kBlock), 0, st, a); break;
    case kSrcChunk: hipLaunchKernelGGL((reduce_kernel<DT, kSrcChunk, ACC>), dim3(g), dim3(kBlock), 0, st, a); break;
    case kSrcNone: hipLaunchKernelGGL((reduce_kernel<DT, kSrcNone, true>), dim3(g), dim3(kBlock), 0, st, a); break;
    default: hipLaunchKernelGGL((reduce_kernel<DT, kSrcRanksN, ACC>), dim3(g), dim3(kBlock), 0, st, a); break;
  }
}

// Statistics-only intake on top of an accumulation from one source or none: red keeps
// the accumulator, the Adam pass recomputes u from it.
template <int DT>
static void launch_acc_stats(const ReduceArgs& a, int src, unsigned g, hipStream_t st) {
  switch (src) {
    case 1: hipLaunchKernelGGL((reduce_kernel<DT, 1, true, false, false>), dim3(g), dim3(kBlock), 0, st, a); break;
    case kSrcChunk:
      hipLaunchKernelGGL((reduce_kernel<DT, kSrcChunk, true, false, false>), dim3(g), dim3(kBlock), 0, st, a);
      break;
    default:
      hipLaunchKernelGGL((reduce_kernel<DT, kSrcNone, true, false, false>), dim3(g), dim3(kBlock), 0, st, a);
      break;
  }
}

template <int DT, bool FIRST>
static void launch_accum_first(const ReduceArgs& a, int src, unsigned g, hipStream_t st) {
  switch (src) {
    case 1: hipLaunchKernelGGL((accum_kernel<DT, 1, FIRST>), dim3(g), dim3(kBlock), 0, st, a); break;
    case 2: hipLaunchKernelGGL((accum_kernel<DT, 2, FIRST>), dim3(g), dim3(kBlock), 0, st, a); break;
    case 4: hipLaunchKernelGGL((accum_kernel<DT, 4, FIRST>), dim3(g), dim3(kBlock), 0, st, a); break;
    case 8: hipLaunchKernelGGL((accum_kernel<DT, 8, FIRST>), dim3(g), dim3(kBlock), 0, st, a); break;
    case kSrcChunk: hipLaunchKernelGGL((accum_kernel<DT, kSrcChunk, FIRST>), dim3(g), dim3(kBlock), 0, st, a); break;
    default: hipLaunchKernelGGL((accum_kernel<DT, kSrcRanksN, FIRST>), dim3(g), dim3(kBlock), 0, st, a); break;
  }
}

static ReduceArgs make_reduce_args(const Chunk* chunks, int64_t n_chunks, const void* const* ranks, int32_t n_ranks,
                                   float inv, bool dyn, bool flip, float* red, DevScalars* sc,
                                   const IntakeParts& parts) {
  ReduceArgs a;
  a.chunks = chunks;
  a.n_chunks = n_chunks;
  for (int q = 0; q < kMaxRanks; ++q)
    a.ranks[q] = (ranks && q < n_ranks) ? static_cast<const uint16_t*>(ranks[q]) : nullptr;
  a.n_ranks = n_ranks > 0 ? n_ranks : 1;
  a.inv = inv;
  a.dyn = dyn;
  a.red = red;
  a.ppc = 1;
  a.flip = flip;
  a.sc = sc;
  a.parts = parts;
  a.keep_from = INT64_MAX;
  return a;
}

// Source code of the template switch: n_ranks >= 1 rank buffers (1, 2, 4, 8 are
// specialised), 0 -> the registered gradient, -1 -> none (the accumulated one alone).
static int src_code(int32_t n_ranks) {
  if (n_ranks == 0) return kSrcChunk;
  if (n_ranks < 0) return kSrcNone;
  if (n_ranks == 1 || n_ranks == 2 || n_ranks == 4 || n_ranks == 8) return n_ranks;
  return kSrcRanksN;
}

// Intake with statistics into red: u = (accumulate ? red + s : s) * inv, or red * inv
// when n_ranks < 0; the local flag and sum of squares go to the scalar block.
//
// r16: the rank buffers' sum arrives as a 16-bit reduce output.  Without
// accumulation the 16-bit result itself is stored, in red (state layout, 2 bytes
// per element), and u is taken from it; with accumulation the rounded sum is added.
// keep_acc (with accumulation from one source or none, n_ranks 0, 1 or < 0):
// statistics only, red keeps the accumulator.
hipError_t launch_reduce(int dtype, const Chunk* chunks, int64_t n_chunks, int64_t slice_elems, const void* const* ranks,
                         int32_t n_ranks, bool accumulate, bool r16, bool keep_acc, float inv, bool dyn, bool flip,
                         float* red, DevScalars* sc, const IntakeParts& parts, hipStream_t st) {
  if (n_chunks == 0) {
    hipLaunchKernelGGL(empty_stats_kernel, dim3(1), dim3(1), 0, st, sc, (int32_t)flip);
    return hipGetLastError();
  }
  const int src = src_code(n_ranks);
  ReduceArgs a = make_reduce_args(chunks, n_chunks, ranks, n_ranks, inv, dyn, flip, red, sc, parts);
  // Parts of a chunk pay off where a block reads several rank slices; over one
  // 16-bit source (and the accumulator) whole chunks per block measured faster.
  a.ppc = is_rank_reduce(src) ? kIntakeParts : 1;
  a.keep_from = reduce_keep_from(slice_elems, r16 && !accumulate && is_rank_reduce(src) ? 2 : 4);
  const unsigned g = clamp_grid(n_chunks * a.ppc, n_chunks * a.ppc);
  if (keep_acc) {
    if (!accumulate || !(src == 1 || src == kSrcChunk || src == kSrcNone)) return hipErrorInvalidValue;
    if (dtype == ZERO_BF16) launch_acc_stats<ZERO_BF16>(a, src, g, st);
    else launch_acc_stats<ZERO_F16>(a, src, g, st);
    return hipGetLastError();
  }
  if (r16 && is_rank_reduce(src)) {
    if (dtype == ZERO_BF16) {
      if (accumulate) launch_reduce_acc_r16<ZERO_BF16>(a, src, g, st);
      else launch_reduce16_src<ZERO_BF16>(a, src, g, st);
    } else {
      if (accumulate) launch_reduce_acc_r16<ZERO_F16>(a, src, g, st);
      else launch_reduce16_src<ZERO_F16>(a, src, g, st);
    }
    return hipGetLastError();
  }
  if (dtype == ZERO_BF16) {
    if (accumulate) launch_reduce_acc<ZERO_BF16, true>(a, src, g, st);
    else launch_reduce_acc<ZERO_BF16, false>(a, src, g, st);
  } else {
    if (accumulate) launch_reduce_acc<ZERO_F16, true>(a, src, g, st);
    else launch_reduce_acc<ZERO_F16, false>(a, src, g, st);
  }
  return hipGetLastError();
}

// One micro-step into the accumulator: red = first ? s : red + s (r16: s rounded to
// the 16-bit type first, the reduce-scatter's 16-bit result).
hipError_t launch_accumulate(int dtype, const Chunk* chunks, int64_t n_chunks, const void* const* ranks,
                             int32_t n_ranks, bool first, bool r16, float* red, int64_t grid_cap, hipStream_t st) {
  if (n_chunks == 0) return hipSuccess;
  const ReduceArgs a = make_reduce_args(chunks, n_chunks, ranks, n_ranks, 1.0f, false, false, red, nullptr,
                                        IntakeParts{});
  const unsigned g = clamp_grid(n_chunks * ZS_ADAM_SPLIT, grid_cap);
  const int src = src_code(n_ranks);
  if (r16 && is_rank_reduce(src)) {
    if (dtype == ZERO_BF16) {
      if (first) launch_accum_r16<ZERO_BF16, true>(a, src, g, st);
      else launch_accum_r16<ZERO_BF16, false>(a, src, g, st);
    } else {
      if (first) launch_accum_r16<ZERO_F16, true>(a, src, g, st);
      else launch_accum_r16<ZERO_F16, false>(a, src, g, st);
    }
    return hipGetLastError();
  }
  if (dtype == ZERO_BF16) {
    if (first) launch_accum_first<ZERO_BF16, true>(a, src, g, st);
    else launch_accum_first<ZERO_BF16, false>(a, src, g, st);
  } else {
    if (first) launch_accum_first<ZERO_F16, true>(a, src, g, st);
    else launch_accum_first<ZERO_F16, false>(a, src, g, st);
  }
  return hipGetLastError();
}

template <int DT, int GS>
static void launch_adam_gs(const AdamArgs& a, bool cast, unsigned g, hipStream_t st) {
  if (cast && a.seg.seg)
    hipLaunchKernelGGL((adam_kernel<DT, GS, true, true>), dim3(g), dim3(ZS_ADAM_BLOCK), 0, st, a);
  else if (cast)
    hipLaunchKernelGGL((adam_kernel<DT, GS, true, false>), dim3(g), dim3(ZS_ADAM_BLOCK), 0, st, a);
  else
    hipLaunchKernelGGL((adam_kernel<DT, GS, false, false>), dim3(g), dim3(ZS_ADAM_BLOCK), 0, st, a);
}

template <int DT>
static void launch_adam_dt(const AdamArgs& a, int gs, bool cast, unsigned g, hipStream_t st) {
  switch (gs) {
    case kGradFlat16: launch_adam_gs<DT, kGradFlat16>(a, cast, g, st); break;
    case kGradChunk16: launch_adam_gs<DT, kGradChunk16>(a, cast, g, st); break;
    case kGradRed: launch_adam_gs<DT, kGradRed>(a, cast, g, st); break;
    case kGradRed16: launch_adam_gs<DT, kGradRed16>(a, cast, g, st); break;
    case kGradAccFlat16: launch_adam_gs<DT, kGradAccFlat16>(a, cast, g, st); break;
    case kGradAccChunk16: launch_adam_gs<DT, kGradAccChunk16>(a, cast, g, st); break;
    default: launch_adam_gs<DT, kGradAcc>(a, cast, g, st); break;
  }
}

hipError_t launch_adam(int dtype, int grad_source, bool cast, const AdamArgs& a, int64_t grid_cap, hipStream_t st) {
  const unsigned g = clamp_grid(a.n_chunks * adam_split(grad_source), grid_cap);
  if (dtype == ZERO_BF16)
    launch_adam_dt<ZERO_BF16>(a, grad_source, cast, g, st);
  else
    launch_adam_dt<ZERO_F16>(a, grad_source, cast, g, st);
  return hipGetLastError();
}

hipError_t launch_adam_step(int dtype, int grad_source, bool cast, const Chunk* chunks, int64_t n_chunks,
                            int64_t slice_elems, const uint16_t* flat_g, const float* red, float* master, float* m,
                            float* v, DevScalars* sc, int32_t other_flag, double other_sumsq, bool sumsq_global,
                            float max_norm, float inv, const zero_adam_hparams_t* hp, const zero_loss_scaler_t* dyn,
                            const SegArgs* seg, int64_t grid_cap, hipStream_t st) {
  AdamArgs a;
  a.chunks = chunks;
  a.n_chunks = n_chunks;
  a.flat_g = flat_g;
  a.red = red;
  a.master = master;
  a.m = m;
  a.v = v;
  a.sc = sc;
  a.other_flag = other_flag;
  a.other_sumsq = other_sumsq;
  a.sumsq_global = sumsq_global ? 1 : 0;
  a.max_norm = max_norm;
  a.inv = inv;
  a.lr = hp->lr;
  a.beta1 = hp->beta1;
  a.beta2 = hp->beta2;
  a.eps = hp->eps;
  a.wd = hp->weight_decay;
  a.dyn = dyn != nullptr;
  a.growth = dyn ? dyn->growth_factor : 1.0f;
  a.backoff = dyn ? dyn->backoff_factor : 1.0f;
  a.min_scale = dyn ? dyn->min_scale : 1.0f;
  a.interval = dyn ? dyn->growth_interval : 1;
  a.seg = seg ? *seg : SegArgs{nullptr, 1, 0, 0, 0};
  // After an intake that left the tail of the Adam pass's gradient source in the cache, start
  // where it ended -- unless the write-back reports segments, whose consumers wait in order.
  const bool tail = (grad_source == kGradFlat16 || grad_source == kGradChunk16) ? stats_tail_cached(slice_elems)
                    : grad_source == kGradRed                                    ? reduce_tail_cached(slice_elems, 4)
                    : grad_source == kGradRed16                                  ? reduce_tail_cached(slice_elems, 2)
                                                                                 : false;
  a.reverse = tail && !(cast && seg);
  return launch_adam(dtype, grad_source, cast, a, grid_cap, st);
}

hipError_t launch_cast(int dtype, const Chunk* chunks, int64_t n_chunks, const float* master,
                       const DevScalars* sc, const SegArgs* seg, int64_t grid_cap, hipStream_t st) {
  if (n_chunks == 0) return hipSuccess;
  const unsigned g = clamp_grid(n_chunks, grid_cap);
  const SegArgs sa = seg ? *seg : SegArgs{nullptr, 1, 0, 0, 0};
  if (dtype == ZERO_BF16) {
    if (sa.seg)
      hipLaunchKernelGGL((cast_kernel<ZERO_BF16, true>), dim3(g), dim3(kBlock), 0, st, chunks, n_chunks, master, sc,
                         sa);
    else
      hipLaunchKernelGGL((cast_kernel<ZERO_BF16, false>), dim3(g), dim3(kBlock), 0, st, chunks, n_chunks, master,
                         sc, sa);
  } else {
    if (sa.seg)
      hipLaunchKernelGGL((cast_kernel<ZERO_F16, true>), dim3(g), dim3(kBlock), 0, st, chunks, n_chunks, master, sc,
                         sa);
    else
      hipLaunchKernelGGL((cast_kernel<ZERO_F16, false>), dim3(g), dim3(kBlock), 0, st, chunks, n_chunks, master,
                         sc, sa);
  }
  return hipGetLastError();
}

hipError_t launch_seg_wait(const SegState* seg, int32_t k, uint64_t epoch, int64_t max_polls, DevScalars* sc,
                           hipStream_t st) {
  hipLaunchKernelGGL(seg_wait_kernel, dim3(1), dim3(64), 0, st, seg, k, epoch, max_polls, sc);
  return hipGetLastError();
}

hipError_t launch_init(int dtype, const Chunk* chunks, int64_t n_chunks, float* master, float* m, float* v,
                       int64_t state_elems, const float* master_init, int64_t grid_cap, hipStream_t st) {
  const unsigned gz = clamp_grid((state_elems + kBlock - 1) / kBlock, 4096);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(gz), dim3(kBlock), 0, st, master, state_elems);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(gz), dim3(kBlock), 0, st, m, state_elems);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(gz), dim3(kBlock), 0, st, v, state_elems);
  if (n_chunks > 0) {
    const unsigned g = clamp_grid(n_chunks, grid_cap);
    if (dtype == ZERO_BF16)
      hipLaunchKernelGGL(init_kernel<ZERO_BF16>, dim3(g), dim3(kBlock), 0, st, chunks, n_chunks, master,
                         master_init);
    else
      hipLaunchKernelGGL(init_kernel<ZERO_F16>, dim3(g), dim3(kBlock), 0, st, chunks, n_chunks, master,
                         master_init);
  }
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const unsigned gz = clamp_grid((n + kBlock - 1) / kBlock, 4096);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(gz), dim3(kBlock), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_export(const Chunk* chunks, int64_t n_chunks, const float* src, float* dst, int64_t grid_cap,
                         hipStream_t st) {
  if (n_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(export_kernel, dim3(clamp_grid(n_chunks, grid_cap)), dim3(kBlock), 0, st, chunks, n_chunks,
                     src, dst);
  return hipGetLastError();
}

}  // namespace zs
