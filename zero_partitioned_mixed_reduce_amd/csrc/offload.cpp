// Offloaded optimizer step (ZeRO-Offload): host runtime and AVX-512 loops.
//
// The pages keep the fp32 master, momentum, variance and the 16-bit gradients
// in host memory and let the host cores run the update, copying only the
// 16-bit weights back to the GPU ("DeepSpeed ZeRO", ZeRO-Offload;
// "千亿参数模型如何塞进有限显卡", ZeRO-Offload：利用CPU内存).  Here:
//   - the shard is cut into tiles of kTile elements, the unit of host work, and
//     copy blocks of kBlockTiles tiles, the unit of device<->host transfer;
//   - a fixed pool of worker threads takes tiles in order from an atomic
//     counter; each tile runs one AVX-512 loop (16 elements per instruction);
//   - with a device workspace, the flag and sum of squares are taken on the GPU
//     (the statistics kernel of the device step, over the gradient still in
//     HBM) while the gradient slice is copied to the host, and the Adam pass
//     starts on each copy block as soon as it lands; without one, a host
//     statistics pass consumes the blocks as they land and the Adam pass
//     follows;
//   - the Adam pass hands each finished block to the calling thread, which
//     enqueues its host-to-device copy while the workers go on with the next
//     blocks;
//   - the per-element arithmetic is the step's fp32 sequence, every operation
//     one IEEE binary32 operation rounded to nearest even (this file is built
//     with -ffp-contract=off; division and square root are the correctly
//     rounded vdivps / vsqrtps), and each worker runs with MXCSR at its IEEE
//     default (no flush-to-zero, no denormals-are-zero);
//   - the fp64 sum of squares is formed per tile (fixed lane and accumulator
//     order) and the tile sums are added in tile order, so results do not
//     depend on the number of threads.
#include <hip/hip_runtime_api.h>
#include <immintrin.h>
#include <math.h>
#include <string.h>

#include <atomic>
#include <cstddef>
#include <cmath>
#include <condition_variable>
#include <functional>
#include <memory>
#include <mutex>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "zero_offload.h"
#include "zs_host.h"
#include "zs_internal.h"

#define ZO_AVX512 __attribute__((target("avx512f,avx512bw,avx512vl")))

namespace {

constexpr int64_t kTile = 1 << 14;        // elements per unit of host work
constexpr int64_t kBlockTiles = 256;      // tiles per copy block
constexpr int64_t kBlock = kTile * kBlockTiles;
constexpr int kMaxThreads = 256;

zero_status_t fail(zero_status_t s, const std::string& msg) { return zs::set_error(s, msg); }
zero_status_t hip_fail(const char* what, hipError_t e) {
  return zs::set_error(ZERO_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool host_has_avx512() {
  __builtin_cpu_init();
  return __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
         __builtin_cpu_supports("avx512vl");
}

// ---------------------------------------------------------------------------
// worker pool

class Pool {
 public:
  // Throws when a thread cannot be started, after stopping the ones already running.
  explicit Pool(int n) : n_(n) {
    try {
      for (int i = 0; i < n; ++i) threads_.emplace_back([this, i] { loop(i); });
    } catch (...) {
      stop_all();
      throw;
    }
  }
  ~Pool() { stop_all(); }
  int size() const { return n_; }
  // Runs fn(worker) once on every worker; wait() returns when all have returned.
  void start(std::function<void(int)> fn) {
    {
      std::lock_guard<std::mutex> l(mu_);
      job_ = std::move(fn);
      busy_ = n_;
      ++gen_;
    }
    wake_.notify_all();
  }
  void wait() {
    std::unique_lock<std::mutex> l(mu_);
    done_.wait(l, [this] { return busy_ == 0; });
  }
  void run(std::function<void(int)> fn) {
    start(std::move(fn));
    wait();
  }

 private:
  void stop_all() {
    {
      std::lock_guard<std::mutex> l(mu_);
      stop_ = true;
      ++gen_;
    }
    wake_.notify_all();
    for (auto& t : threads_) t.join();
  }
  void loop(int i) {
    _mm_setcsr(0x1F80);  // round to nearest even, all exceptions masked, no FTZ, no DAZ
    uint64_t seen = 0;
    for (;;) {
      std::function<void(int)> fn;
      {
        std::unique_lock<std::mutex> l(mu_);
        wake_.wait(l, [&] { return gen_ != seen; });
        seen = gen_;
        if (stop_) return;
        fn = job_;
      }
      fn(i);
      {
        std::lock_guard<std::mutex> l(mu_);
        if (--busy_ == 0) done_.notify_all();
      }
    }
  }
  int n_;
  std::vector<std::thread> threads_;
  std::mutex mu_;
  std::condition_variable wake_, done_;
  std::function<void(int)> job_;
  uint64_t gen_ = 0;
  int busy_ = 0;
  bool stop_ = false;
};

inline void spin_pause(int& n) {
  if (++n < 64) _mm_pause();
  else {
    n = 0;
    std::this_thread::yield();
  }
}

// ---------------------------------------------------------------------------
// AVX-512 loops

template <int DT>
ZO_AVX512 inline __m512 dec16(__m256i h) {
  if constexpr (DT == ZERO_BF16) return _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(h), 16));
  else return _mm512_cvtph_ps(h);
}

// Round to nearest even into the 16-bit format; every NaN becomes the format's
// positive canonical quiet NaN (0x7FC0, 0x7E00), whatever its sign and payload, as
// on the device.
template <int DT>
ZO_AVX512 inline __m256i enc16(__m512 w) {
  const __m512i u = _mm512_castps_si512(w);
  const __mmask16 nan = _mm512_cmp_ps_mask(w, w, _CMP_UNORD_Q);
  if constexpr (DT == ZERO_BF16) {
    const __m512i lsb = _mm512_and_si512(_mm512_srli_epi32(u, 16), _mm512_set1_epi32(1));
    __m512i r = _mm512_srli_epi32(_mm512_add_epi32(_mm512_add_epi32(u, _mm512_set1_epi32(0x7FFF)), lsb), 16);
    r = _mm512_mask_mov_epi32(r, nan, _mm512_set1_epi32(0x7FC0));
    return _mm512_cvtepi32_epi16(r);
  } else {
    const __m256i h = _mm512_cvtps_ph(w, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
    return _mm256_mask_mov_epi16(h, nan, _mm256_set1_epi16(0x7E00));
  }
}

ZO_AVX512 inline __mmask16 tail_mask(int64_t left) {
  return left >= 16 ? (__mmask16)0xFFFF : (__mmask16)((1u << left) - 1u);
}

// Sum of (double)u * (double)u over one tile, u = g * inv.  The square of a
// float is exact in fp64, so fma(d, d, acc) rounds exactly like acc + d * d.
template <int DT>
ZO_AVX512 double sumsq_tile(const uint16_t* g, int64_t n, float inv) {
  const __m512 vinv = _mm512_set1_ps(inv);
  __m512d a0 = _mm512_setzero_pd(), a1 = a0, a2 = a0, a3 = a0;
  int64_t i = 0;
  for (; i + 32 <= n; i += 32) {
    const __m512 x = _mm512_mul_ps(dec16<DT>(_mm256_loadu_si256(reinterpret_cast<const __m256i*>(g + i))), vinv);
    const __m512 y =
        _mm512_mul_ps(dec16<DT>(_mm256_loadu_si256(reinterpret_cast<const __m256i*>(g + i + 16))), vinv);
    const __m512d x0 = _mm512_cvtps_pd(_mm512_castps512_ps256(x));
    const __m512d x1 = _mm512_cvtps_pd(_mm256_castpd_ps(_mm512_extractf64x4_pd(_mm512_castps_pd(x), 1)));
    const __m512d y0 = _mm512_cvtps_pd(_mm512_castps512_ps256(y));
    const __m512d y1 = _mm512_cvtps_pd(_mm256_castpd_ps(_mm512_extractf64x4_pd(_mm512_castps_pd(y), 1)));
    a0 = _mm512_fmadd_pd(x0, x0, a0);
    a1 = _mm512_fmadd_pd(x1, x1, a1);
    a2 = _mm512_fmadd_pd(y0, y0, a2);
    a3 = _mm512_fmadd_pd(y1, y1, a3);
  }
  for (; i < n; i += 16) {
    const __mmask16 k = tail_mask(n - i);
    const __m512 x = _mm512_mul_ps(dec16<DT>(_mm256_maskz_loadu_epi16(k, g + i)), vinv);
    const __m512d x0 = _mm512_cvtps_pd(_mm512_castps512_ps256(x));
    const __m512d x1 = _mm512_cvtps_pd(_mm256_castpd_ps(_mm512_extractf64x4_pd(_mm512_castps_pd(x), 1)));
    a0 = _mm512_fmadd_pd(x0, x0, a0);
    a1 = _mm512_fmadd_pd(x1, x1, a1);
  }
  alignas(64) double lane[8];
  _mm512_store_pd(lane, _mm512_add_pd(_mm512_add_pd(a0, a1), _mm512_add_pd(a2, a3)));
  double s = 0.0;
  for (int j = 0; j < 8; ++j) s += lane[j];
  return s;
}

struct StepScalars {
  float inv, clip, b1, b2, omb1, omb2, bc1, bc2, lr, eps, wd;
};

template <int DT>
ZO_AVX512 void adam_tile(const uint16_t* g, float* w, float* m, float* v, uint16_t* p16, int64_t n,
                         const StepScalars& s) {
  const __m512 inv = _mm512_set1_ps(s.inv), clip = _mm512_set1_ps(s.clip);
  const __m512 b1 = _mm512_set1_ps(s.b1), b2 = _mm512_set1_ps(s.b2);
  const __m512 omb1 = _mm512_set1_ps(s.omb1), omb2 = _mm512_set1_ps(s.omb2);
  const __m512 bc1 = _mm512_set1_ps(s.bc1), bc2 = _mm512_set1_ps(s.bc2);
  const __m512 lr = _mm512_set1_ps(s.lr), eps = _mm512_set1_ps(s.eps), wd = _mm512_set1_ps(s.wd);
  for (int64_t i = 0; i < n; i += 16) {
    const __mmask16 k = tail_mask(n - i);
    const __m512 u = _mm512_mul_ps(dec16<DT>(_mm256_maskz_loadu_epi16(k, g + i)), inv);
    const __m512 W = _mm512_maskz_loadu_ps(k, w + i);
    const __m512 M = _mm512_maskz_loadu_ps(k, m + i);
    const __m512 V = _mm512_maskz_loadu_ps(k, v + i);
    const __m512 gc = _mm512_mul_ps(u, clip);
    const __m512 mi = _mm512_add_ps(_mm512_mul_ps(b1, M), _mm512_mul_ps(omb1, gc));
    const __m512 vi = _mm512_add_ps(_mm512_mul_ps(b2, V), _mm512_mul_ps(omb2, _mm512_mul_ps(gc, gc)));
    const __m512 mh = _mm512_div_ps(mi, bc1);
    const __m512 vh = _mm512_div_ps(vi, bc2);
    const __m512 den = _mm512_add_ps(_mm512_sqrt_ps(vh), eps);
    const __m512 upd = _mm512_div_ps(mh, den);
    const __m512 wn = _mm512_sub_ps(W, _mm512_mul_ps(lr, _mm512_add_ps(upd, _mm512_mul_ps(wd, W))));
    _mm512_mask_storeu_ps(w + i, k, wn);
    _mm512_mask_storeu_ps(m + i, k, mi);
    _mm512_mask_storeu_ps(v + i, k, vi);
    _mm256_mask_storeu_epi16(p16 + i, k, enc16<DT>(wn));
  }
}

template <int DT>
ZO_AVX512 void upcast_tile(const uint16_t* p16, float* w, int64_t n) {
  for (int64_t i = 0; i < n; i += 16) {
    const __mmask16 k = tail_mask(n - i);
    _mm512_mask_storeu_ps(w + i, k, dec16<DT>(_mm256_maskz_loadu_epi16(k, p16 + i)));
  }
}

ZO_AVX512 void zero_tile(float* p, int64_t n) {
  for (int64_t i = 0; i < n; i += 16) _mm512_mask_storeu_ps(p + i, tail_mask(n - i), _mm512_setzero_ps());
}

enum Phase { kReady, kFetched, kStats, kStepped };

}  // namespace

struct zero_offload {
  zero_shard_info_t info;
  std::vector<zs::Piece> pieces;
  std::vector<uint64_t> piece_p16;  // device address of each piece's first 16-bit parameter (0: host-only)
  std::vector<uint64_t> piece_g16;  // device address of each piece's first registered gradient (0: none)
  int dtype;
  int device;
  bool has_device;
  bool has_registered_grads;
  float *master, *m, *v;
  uint16_t *g16, *p16;
  std::unique_ptr<Pool> pool;
  int64_t n_tiles, n_blocks;
  std::vector<hipEvent_t> fetch_ev;  // one per copy block
  hipEvent_t push_ev;
  bool fetch_pending, push_pending, pushed;
  // device statistics (optional workspace): scalar block, chunk table, partial sums
  bool dev_stats;
  zs::DevScalars* sc;
  zs::Chunk* chunks;
  int64_t n_chunks;
  zs::IntakeParts parts;
  hipStream_t aux;       // non-blocking stream that reads the statistics back
  hipEvent_t stats_ev;   // recorded after the statistics kernel
  bool stats_pending;
  float stats_inv;
  Phase phase;
  // step state
  float inv;
  int32_t local_flag;
  double local_sumsq;
  std::vector<double> partials;
  int64_t t;
  double p1, p2;
  int32_t skipped;
  double norm;
  float clip;
};

namespace {

// Makes the handle's device current for the call; does nothing for a host-only handle
// (which never calls the HIP runtime).
struct DeviceGuard {
  int prev = -1;
  bool changed = false;
  DeviceGuard(int dev, bool active) {
    if (active && hipGetDevice(&prev) == hipSuccess && prev != dev) changed = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    if (changed) (void)hipSetDevice(prev);
  }
};

int64_t tile_len(const zero_offload* h, int64_t t) {
  const int64_t lo = t * kTile;
  return (h->info.valid_elems - lo) < kTile ? (h->info.valid_elems - lo) : kTile;
}

int64_t block_tiles(const zero_offload* h, int64_t k) {
  const int64_t lo = k * kBlockTiles;
  return (h->n_tiles - lo) < kBlockTiles ? (h->n_tiles - lo) : kBlockTiles;
}

// Calls fn(piece, lo, hi) for every piece intersecting copy block k, with
// [lo, hi) the intersection in logical shard offsets.
template <class Fn>
zero_status_t for_block_pieces(const zero_offload* h, int64_t k, Fn fn) {
  const int64_t b0 = k * kBlock;
  const int64_t b1 = (b0 + kBlock) < h->info.valid_elems ? (b0 + kBlock) : h->info.valid_elems;
  // pieces are sorted by shard offset and tile the shard; binary search the first one
  size_t lo = 0, hi = h->pieces.size();
  while (lo + 1 < hi) {
    const size_t mid = (lo + hi) / 2;
    if (h->pieces[mid].shard_off <= b0) lo = mid;
    else hi = mid;
  }
  for (size_t p = lo; p < h->pieces.size(); ++p) {
    const zs::Piece& pc = h->pieces[p];
    if (pc.shard_off >= b1) break;
    const int64_t a = pc.shard_off > b0 ? pc.shard_off : b0;
    const int64_t e = (pc.shard_off + pc.len) < b1 ? (pc.shard_off + pc.len) : b1;
    if (a < e) {
      zero_status_t s = fn(p, a, e);
      if (s != ZERO_OK) return s;
    }
  }
  return ZERO_OK;
}

zero_status_t enqueue_push_block(zero_offload* h, int64_t k, hipStream_t st) {
  return for_block_pieces(h, k, [&](size_t p, int64_t a, int64_t e) -> zero_status_t {
    void* dst = reinterpret_cast<void*>(h->piece_p16[p] + 2 * (uint64_t)(a - h->pieces[p].shard_off));
    hipError_t err = hipMemcpyAsync(dst, h->p16 + a, 2 * (size_t)(e - a), hipMemcpyHostToDevice, st);
    return err == hipSuccess ? ZERO_OK : hip_fail("hipMemcpyAsync(host to device)", err);
  });
}

zero_status_t wait_push(zero_offload* h) {
  if (!h->push_pending) return ZERO_OK;
  hipError_t e = hipEventSynchronize(h->push_ev);
  h->push_pending = false;
  return e == hipSuccess ? ZERO_OK : hip_fail("hipEventSynchronize(push)", e);
}

template <int DT>
void run_upcast(zero_offload* h) {
  std::atomic<int64_t> next{0};
  h->pool->run([&](int) {
    for (;;) {
      const int64_t t = next.fetch_add(1, std::memory_order_relaxed);
      if (t >= h->n_tiles) break;
      upcast_tile<DT>(h->p16 + t * kTile, h->master + t * kTile, tile_len(h, t));
    }
  });
}

}  // namespace

namespace {

zero_status_t offload_init(const zero_shard_desc_t* desc, const zero_offload_bufs_t* bufs, const float* master_init,
                           int32_t num_threads, void* stream, zero_offload_t* out) {
  if (!desc || !bufs || !out) return fail(ZERO_EINVAL, "null description, buffers or output handle");
  *out = nullptr;
  if (!host_has_avx512()) return fail(ZERO_EINVAL, "the offloaded step needs host AVX-512 (F, BW, VL)");
  const bool has_device = desc->param16 || desc->flat_param16;
  zero_shard_desc_t d = *desc;
  if (!has_device) d.flat_param16 = reinterpret_cast<void*>(uintptr_t{256});  // partition only: never accessed
  zs::Plan p;
  std::string err;
  zero_status_t s = zs::build_plan(&d, &p, &err);
  if (s != ZERO_OK) return fail(s, err);
  if (!bufs->master || !bufs->m || !bufs->v || !bufs->grad16 || !bufs->param16)
    return fail(ZERO_EINVAL, "master, m, v, grad16 and param16 must be non-null");
  if (bufs->capacity < p.info.valid_elems)
    return fail(ZERO_EINVAL, "capacity " + std::to_string(bufs->capacity) + " < valid_elems " +
                                 std::to_string(p.info.valid_elems));
  if (((uintptr_t)bufs->master | (uintptr_t)bufs->m | (uintptr_t)bufs->v) & 3u)
    return fail(ZERO_EINVAL, "fp32 host arrays must be 4-byte aligned");
  if (((uintptr_t)bufs->grad16 | (uintptr_t)bufs->param16) & 1u)
    return fail(ZERO_EINVAL, "16-bit host arrays must be 2-byte aligned");
  if (num_threads > kMaxThreads) return fail(ZERO_EINVAL, "num_threads must be at most 256");
  if (bufs->workspace) {
    if (!has_device) return fail(ZERO_EINVAL, "a device workspace needs device parameters");
    if (((uintptr_t)bufs->workspace & 255u) != 0) return fail(ZERO_EINVAL, "workspace must be 256-byte aligned");
    if (bufs->workspace_capacity < p.info.workspace_bytes)
      return fail(ZERO_EINVAL, "workspace_capacity " + std::to_string(bufs->workspace_capacity) +
                                   " < workspace_bytes " + std::to_string(p.info.workspace_bytes));
  }
  int threads = num_threads > 0 ? num_threads : (int)std::thread::hardware_concurrency();
  if (threads < 1) threads = 1;
  if (threads > kMaxThreads) threads = kMaxThreads;

  std::unique_ptr<zero_offload> h(new (std::nothrow) zero_offload());
  if (!h) return fail(ZERO_ENOMEM, "out of host memory");
  h->info = p.info;
  h->pieces = std::move(p.pieces);
  h->dtype = desc->dtype;
  h->has_device = has_device;
  h->has_registered_grads = has_device && (desc->grad16 || desc->flat_grad16);
  h->piece_p16.assign(h->pieces.size(), 0);
  h->piece_g16.assign(h->pieces.size(), 0);
  const int64_t begin = p.info.shard_begin;
  for (size_t q = 0; q < h->pieces.size(); ++q) {
    const zs::Piece& pc = h->pieces[q];
    if (!has_device) continue;
    h->piece_p16[q] = desc->param16 ? (uint64_t)(uintptr_t)desc->param16[pc.tensor] + 2 * (uint64_t)pc.tensor_off
                                    : (uint64_t)(uintptr_t)desc->flat_param16 + 2 * (uint64_t)(begin + pc.shard_off);
    if (desc->grad16)
      h->piece_g16[q] = (uint64_t)(uintptr_t)desc->grad16[pc.tensor] + 2 * (uint64_t)pc.tensor_off;
    else if (desc->flat_grad16)
      h->piece_g16[q] = (uint64_t)(uintptr_t)desc->flat_grad16 + 2 * (uint64_t)(begin + pc.shard_off);
  }
  h->master = bufs->master;
  h->m = bufs->m;
  h->v = bufs->v;
  h->g16 = static_cast<uint16_t*>(bufs->grad16);
  h->p16 = static_cast<uint16_t*>(bufs->param16);
  const int64_t valid = p.info.valid_elems;
  h->n_tiles = (valid + kTile - 1) / kTile;
  h->n_blocks = (h->n_tiles + kBlockTiles - 1) / kBlockTiles;
  h->partials.assign(h->n_tiles, 0.0);
  h->push_ev = nullptr;
  h->fetch_pending = h->push_pending = h->pushed = false;
  h->phase = kReady;
  h->inv = 1.0f;
  h->local_flag = 0;
  h->local_sumsq = 0.0;
  h->t = 0;
  h->p1 = h->p2 = 1.0;
  h->skipped = 0;
  h->norm = 0.0;
  h->clip = 1.0f;
  h->device = 0;
  h->dev_stats = bufs->workspace != nullptr;
  h->sc = nullptr;
  h->chunks = nullptr;
  h->n_chunks = (int64_t)p.chunks.size();
  h->aux = nullptr;
  h->stats_ev = nullptr;
  h->stats_pending = false;
  h->stats_inv = 0.0f;

  auto cleanup_events = [&]() {
    // copies already enqueued on the caller's stream may still read the set-up's host tables
    if (has_device) (void)hipStreamSynchronize(static_cast<hipStream_t>(stream));
    for (hipEvent_t e : h->fetch_ev)
      if (e) (void)hipEventDestroy(e);
    h->fetch_ev.clear();
    if (h->push_ev) (void)hipEventDestroy(h->push_ev);
    h->push_ev = nullptr;
    if (h->stats_ev) (void)hipEventDestroy(h->stats_ev);
    h->stats_ev = nullptr;
    if (h->aux) (void)hipStreamDestroy(h->aux);
    h->aux = nullptr;
  };
  if (has_device) {
    hipError_t e = hipGetDevice(&h->device);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    h->fetch_ev.assign(h->n_blocks, nullptr);
    for (auto& ev : h->fetch_ev)
      if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) {
        cleanup_events();
        return hip_fail("hipEventCreateWithFlags", e);
      }
    if ((e = hipEventCreateWithFlags(&h->push_ev, hipEventDisableTiming)) != hipSuccess) {
      cleanup_events();
      return hip_fail("hipEventCreateWithFlags", e);
    }
  }
  if (h->dev_stats) {
    // the device step's intake layout: scalar block, chunk table, group counters at zero
    char* ws = static_cast<char*>(bufs->workspace);
    const zs::IntakeLayout il = zs::intake_layout(h->n_chunks);
    h->sc = reinterpret_cast<zs::DevScalars*>(ws);
    h->chunks = reinterpret_cast<zs::Chunk*>(ws + zs::kChunksOff);
    h->parts.part = reinterpret_cast<uint64_t*>(ws + il.part_off);
    h->parts.gcount = reinterpret_cast<zs::GroupCount*>(ws + il.gcount_off);
    h->parts.gpart = reinterpret_cast<uint64_t*>(ws + il.gpart_off);
    hipStream_t st = static_cast<hipStream_t>(stream);
    zs::DevScalars init_sc;
    memset(&init_sc, 0, sizeof(init_sc));
    const int64_t n_groups = zs::intake_groups(h->n_chunks);
    hipError_t e;
    if ((e = hipStreamCreateWithFlags(&h->aux, hipStreamNonBlocking)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&h->stats_ev, hipEventDisableTiming)) != hipSuccess ||
        (e = hipMemcpyAsync(h->sc, &init_sc, sizeof(init_sc), hipMemcpyHostToDevice, st)) != hipSuccess ||
        (h->n_chunks && (e = hipMemcpyAsync(h->chunks, p.chunks.data(), p.chunks.size() * sizeof(zs::Chunk),
                                             hipMemcpyHostToDevice, st)) != hipSuccess) ||
        (e = zs::launch_fill_zero(reinterpret_cast<float*>(h->parts.gcount),
                                  n_groups * (int64_t)(sizeof(zs::GroupCount) / sizeof(float)), st)) != hipSuccess ||
        (e = hipStreamSynchronize(st)) != hipSuccess) {
      cleanup_events();
      return hip_fail("device statistics set-up", e);
    }
  }
  h->pool.reset(new (std::nothrow) Pool(threads));
  if (!h->pool) {
    cleanup_events();
    return fail(ZERO_ENOMEM, "out of host memory");
  }

  // state: m = v = 0; master given, or the exact upcast of the 16-bit slice
  {
    std::atomic<int64_t> next{0};
    zero_offload* hp = h.get();
    hp->pool->run([&](int) {
      for (;;) {
        const int64_t t = next.fetch_add(1, std::memory_order_relaxed);
        if (t >= hp->n_tiles) break;
        zero_tile(hp->m + t * kTile, tile_len(hp, t));
        zero_tile(hp->v + t * kTile, tile_len(hp, t));
      }
    });
  }
  if (master_init) {
    memcpy(h->master, master_init, sizeof(float) * (size_t)valid);
  } else {
    if (has_device) {
      hipStream_t st = static_cast<hipStream_t>(stream);
      zero_offload* hp = h.get();
      for (int64_t k = 0; k < h->n_blocks; ++k) {
        zero_status_t cs = for_block_pieces(hp, k, [&](size_t q, int64_t a, int64_t e) -> zero_status_t {
          const void* src = reinterpret_cast<const void*>(hp->piece_p16[q] + 2 * (uint64_t)(a - hp->pieces[q].shard_off));
          hipError_t he = hipMemcpyAsync(hp->p16 + a, src, 2 * (size_t)(e - a), hipMemcpyDeviceToHost, st);
          return he == hipSuccess ? ZERO_OK : hip_fail("hipMemcpyAsync(parameters to host)", he);
        });
        if (cs != ZERO_OK) {
          cleanup_events();
          return cs;
        }
      }
      hipError_t e = hipStreamSynchronize(st);
      if (e != hipSuccess) {
        cleanup_events();
        return hip_fail("hipStreamSynchronize(init)", e);
      }
    }
    if (h->dtype == ZERO_BF16) run_upcast<ZERO_BF16>(h.get());
    else run_upcast<ZERO_F16>(h.get());
  }
  *out = h.release();
  return ZERO_OK;
}

}  // namespace

extern "C" {

// Host allocations and thread creation may throw; no exception leaves the C ABI.
zero_status_t zero_offload_init(const zero_shard_desc_t* desc, const zero_offload_bufs_t* bufs,
                                const float* master_init, int32_t num_threads, void* stream, zero_offload_t* out) {
  try {
    return offload_init(desc, bufs, master_init, num_threads, stream, out);
  } catch (const std::exception& e) {
    return fail(ZERO_ENOMEM, std::string("host resources: ") + e.what());
  }
}

zero_status_t zero_offload_fetch_grads(zero_offload_t h, const void* flat_grad16, float inv_loss_scale,
                                       void* stream) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  if (!h->has_device) return fail(ZERO_EINVAL, "host-only handle: no device gradient to fetch");
  if (!flat_grad16 && !h->has_registered_grads)
    return fail(ZERO_EINVAL, "no flat_grad16 given and no gradient registered at init");
  if (h->phase == kStats) return fail(ZERO_ESTATE, "the gradient of this step was already taken in");
  if (!(inv_loss_scale > 0.0f) || !std::isfinite(inv_loss_scale))
    return fail(ZERO_EINVAL, "inv_loss_scale must be finite and positive");
  hipStream_t st = static_cast<hipStream_t>(stream);
  DeviceGuard dg(h->device, h->has_device);
  if (h->dev_stats) {
    // flag and sum of squares on the device, from the gradient still in HBM; the copies follow
    hipError_t he = zs::launch_stats16(h->dtype, h->chunks, h->n_chunks, h->info.valid_elems,
                                       static_cast<const uint16_t*>(flat_grad16),
                                       inv_loss_scale, false, false, h->sc, h->parts, st);
    if (he == hipSuccess) he = hipEventRecord(h->stats_ev, st);
    if (he != hipSuccess) return hip_fail("device statistics", he);
    h->stats_pending = true;
    h->stats_inv = inv_loss_scale;
  }
  const int64_t begin = h->info.shard_begin;
  for (int64_t k = 0; k < h->n_blocks; ++k) {
    zero_status_t s = for_block_pieces(h, k, [&](size_t p, int64_t a, int64_t e) -> zero_status_t {
      const uint64_t src = flat_grad16 ? (uint64_t)(uintptr_t)flat_grad16 + 2 * (uint64_t)(begin + a)
                                       : h->piece_g16[p] + 2 * (uint64_t)(a - h->pieces[p].shard_off);
      hipError_t he = hipMemcpyAsync(h->g16 + a, reinterpret_cast<const void*>(src), 2 * (size_t)(e - a),
                                     hipMemcpyDeviceToHost, st);
      return he == hipSuccess ? ZERO_OK : hip_fail("hipMemcpyAsync(gradient to host)", he);
    });
    if (s != ZERO_OK) return s;
    hipError_t he = hipEventRecord(h->fetch_ev[k], st);
    if (he != hipSuccess) return hip_fail("hipEventRecord", he);
  }
  h->fetch_pending = true;
  h->phase = kFetched;
  return ZERO_OK;
}

zero_status_t zero_offload_grad_stats(zero_offload_t h, float inv_loss_scale, int32_t* found_inf, double* sumsq) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  if (!(inv_loss_scale > 0.0f) || !std::isfinite(inv_loss_scale))
    return fail(ZERO_EINVAL, "inv_loss_scale must be finite and positive");
  if (h->stats_pending) {
    // the device computed them: read the two scalars back on the non-blocking stream, without
    // waiting for the gradient copies, which the Adam pass consumes block by block
    if (inv_loss_scale != h->stats_inv)
      return fail(ZERO_EINVAL, "inv_loss_scale differs from the one given to zero_offload_fetch_grads");
    DeviceGuard dg(h->device, h->has_device);
    struct {
      double sumsq;
      int32_t flag;
    } v;
    static_assert(offsetof(zs::DevScalars, local_flag) == sizeof(double), "scalar block layout");
    hipError_t e = hipStreamWaitEvent(h->aux, h->stats_ev, 0);
    if (e == hipSuccess) e = hipMemcpyAsync(&v, h->sc, sizeof(double) + sizeof(int32_t), hipMemcpyDeviceToHost, h->aux);
    if (e == hipSuccess) e = hipStreamSynchronize(h->aux);
    if (e != hipSuccess) return hip_fail("reading the device statistics", e);
    h->stats_pending = false;
    h->inv = inv_loss_scale;
    h->local_sumsq = v.sumsq;
    h->local_flag = v.flag;
    h->phase = kStats;
    if (found_inf) *found_inf = h->local_flag;
    if (sumsq) *sumsq = v.sumsq;
    return ZERO_OK;
  }
  std::atomic<int64_t> next{0};
  std::atomic<int64_t> landed{h->fetch_pending ? -1 : h->n_blocks};
  const int dt = h->dtype;
  h->pool->start([&](int) {
    int spins = 0;
    for (;;) {
      const int64_t t = next.fetch_add(1, std::memory_order_relaxed);
      if (t >= h->n_tiles) break;
      const int64_t blk = t / kBlockTiles;
      while (landed.load(std::memory_order_acquire) < blk) spin_pause(spins);
      const uint16_t* g = h->g16 + t * kTile;
      h->partials[t] = dt == ZERO_BF16 ? sumsq_tile<ZERO_BF16>(g, tile_len(h, t), inv_loss_scale)
                                       : sumsq_tile<ZERO_F16>(g, tile_len(h, t), inv_loss_scale);
    }
  });
  zero_status_t rs = ZERO_OK;
  if (h->fetch_pending) {
    for (int64_t k = 0; k < h->n_blocks; ++k) {
      hipError_t e = hipEventSynchronize(h->fetch_ev[k]);
      if (e != hipSuccess) {
        rs = hip_fail("hipEventSynchronize(gradient copy)", e);
        landed.store(h->n_blocks, std::memory_order_release);  // release the workers; the result is void
        break;
      }
      landed.store(k, std::memory_order_release);
    }
  }
  h->pool->wait();
  h->fetch_pending = false;
  if (rs != ZERO_OK) {
    h->phase = kReady;
    return rs;
  }
  double total = 0.0;
  for (int64_t t = 0; t < h->n_tiles; ++t) total += h->partials[t];
  h->inv = inv_loss_scale;
  h->local_sumsq = total;
  h->local_flag = !std::isfinite(total);  // a finite float squared is finite in fp64, so this is "some u non-finite"
  h->phase = kStats;
  if (found_inf) *found_inf = h->local_flag;
  if (sumsq) *sumsq = total;
  return ZERO_OK;
}

namespace {
// The step of zero_offload_adam_step / zero_offload_adam_step_global: sumsq is the other
// ranks' sum of squares (global false) or the global sum.
zero_status_t offload_adam_step(zero_offload_t h, const zero_adam_hparams_t* hp, int32_t other_ranks_found_inf,
                                double sumsq, bool global, float max_norm, int32_t push, void* stream) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  if (global && sumsq < 0.0) return fail(ZERO_EINVAL, "global_sumsq must not be negative");
  if (!hp) return fail(ZERO_EINVAL, "null hparams");
  if (push && !h->has_device) return fail(ZERO_EINVAL, "push needs device parameters (host-only handle)");
  if (h->phase != kStats) return fail(ZERO_ESTATE, "zero_offload_adam_step needs zero_offload_grad_stats first");
  // per copy block: tiles finished (allocated before any state changes)
  std::unique_ptr<std::atomic<int64_t>[]> done(new (std::nothrow) std::atomic<int64_t>[h->n_blocks > 0 ? h->n_blocks : 1]);
  if (!done) return fail(ZERO_ENOMEM, "out of host memory");
  DeviceGuard dg(h->device, h->has_device);
  zero_status_t rs = wait_push(h);
  if (rs != ZERO_OK) return rs;
  const int skip = (h->local_flag | (other_ranks_found_inf != 0)) != 0;
  const double norm = sqrt(global ? sumsq : h->local_sumsq + sumsq);
  float clip = 1.0f;
  if (max_norm > 0.0f) {
    const double c = (double)max_norm / (norm + 1e-6);
    if (c < 1.0) clip = (float)c;
  }
  h->norm = norm;
  h->clip = clip;
  h->skipped = skip;
  h->phase = kStepped;
  h->pushed = false;
  if (skip) {
    // nothing is updated; let a gradient copy still in flight land before returning
    if (h->fetch_pending) {
      for (int64_t k = 0; k < h->n_blocks; ++k) {
        hipError_t e = hipEventSynchronize(h->fetch_ev[k]);
        if (e != hipSuccess && rs == ZERO_OK) rs = hip_fail("hipEventSynchronize(gradient copy)", e);
      }
      h->fetch_pending = false;
    }
    return rs;
  }
  h->t += 1;
  h->p1 = h->p1 * (double)hp->beta1;
  h->p2 = h->p2 * (double)hp->beta2;
  StepScalars s;
  s.inv = h->inv;
  s.clip = clip;
  s.b1 = hp->beta1;
  s.b2 = hp->beta2;
  s.omb1 = 1.0f - hp->beta1;
  s.omb2 = 1.0f - hp->beta2;
  s.bc1 = (float)(1.0 - h->p1);
  s.bc2 = (float)(1.0 - h->p2);
  s.lr = hp->lr;
  s.eps = hp->eps;
  s.wd = hp->weight_decay;

  std::atomic<int64_t> next{0};
  // copy blocks of the gradient that have landed (all of them unless a fetch is still in flight)
  std::atomic<int64_t> landed{h->fetch_pending ? -1 : h->n_blocks};
  for (int64_t k = 0; k < h->n_blocks; ++k) done[k].store(0, std::memory_order_relaxed);
  const int dt = h->dtype;
  h->pool->start([&](int) {
    int spins = 0;
    for (;;) {
      const int64_t t = next.fetch_add(1, std::memory_order_relaxed);
      if (t >= h->n_tiles) break;
      while (landed.load(std::memory_order_acquire) < t / kBlockTiles) spin_pause(spins);
      const int64_t o = t * kTile, n = tile_len(h, t);
      if (dt == ZERO_BF16) adam_tile<ZERO_BF16>(h->g16 + o, h->master + o, h->m + o, h->v + o, h->p16 + o, n, s);
      else adam_tile<ZERO_F16>(h->g16 + o, h->master + o, h->m + o, h->v + o, h->p16 + o, n, s);
      done[t / kBlockTiles].fetch_add(1, std::memory_order_release);
    }
  });
  hipStream_t st = static_cast<hipStream_t>(stream);
  // The calling thread releases each gradient block to the workers as its copy lands, and
  // hands each finished block of the 16-bit slice to the DMA engine.
  int64_t next_push = 0;
  auto push_finished = [&](bool wait) {
    while (next_push < h->n_blocks) {
      const int64_t want = block_tiles(h, next_push);
      if (done[next_push].load(std::memory_order_acquire) < want) {
        if (!wait) return;
        int spins = 0;
        while (done[next_push].load(std::memory_order_acquire) < want) spin_pause(spins);
      }
      if (push && rs == ZERO_OK) rs = enqueue_push_block(h, next_push, st);
      ++next_push;
    }
  };
  if (h->fetch_pending) {
    for (int64_t k = 0; k < h->n_blocks; ++k) {
      hipError_t e = hipEventSynchronize(h->fetch_ev[k]);
      if (e != hipSuccess) {
        if (rs == ZERO_OK) rs = hip_fail("hipEventSynchronize(gradient copy)", e);
        landed.store(h->n_blocks, std::memory_order_release);  // release the workers; the result is void
        break;
      }
      landed.store(k, std::memory_order_release);
      push_finished(false);
    }
    h->fetch_pending = false;
  }
  push_finished(true);
  h->pool->wait();
  if (push && rs == ZERO_OK) {
    hipError_t e = hipEventRecord(h->push_ev, st);
    if (e != hipSuccess) rs = hip_fail("hipEventRecord(push)", e);
    else h->push_pending = true;
  }
  h->pushed = push && rs == ZERO_OK;
  return rs;
}
}  // namespace

zero_status_t zero_offload_adam_step(zero_offload_t h, const zero_adam_hparams_t* hp, int32_t other_ranks_found_inf,
                                     double other_ranks_sumsq, float max_norm, int32_t push, void* stream) {
  return offload_adam_step(h, hp, other_ranks_found_inf, other_ranks_sumsq, false, max_norm, push, stream);
}

zero_status_t zero_offload_adam_step_global(zero_offload_t h, const zero_adam_hparams_t* hp,
                                            int32_t other_ranks_found_inf, double global_sumsq, float max_norm,
                                            int32_t push, void* stream) {
  return offload_adam_step(h, hp, other_ranks_found_inf, global_sumsq, true, max_norm, push, stream);
}

zero_status_t zero_offload_push_params(zero_offload_t h, void* stream) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  if (!h->has_device) return fail(ZERO_EINVAL, "host-only handle: no device parameters");
  if (h->phase != kStepped) return fail(ZERO_ESTATE, "zero_offload_push_params follows zero_offload_adam_step");
  if (h->skipped || h->pushed) return ZERO_OK;
  DeviceGuard dg(h->device, h->has_device);
  zero_status_t rs = wait_push(h);
  if (rs != ZERO_OK) return rs;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int64_t k = 0; k < h->n_blocks; ++k) {
    rs = enqueue_push_block(h, k, st);
    if (rs != ZERO_OK) return rs;
  }
  hipError_t e = hipEventRecord(h->push_ev, st);
  if (e != hipSuccess) return hip_fail("hipEventRecord(push)", e);
  h->push_pending = true;
  h->pushed = true;
  return ZERO_OK;
}

zero_status_t zero_offload_query(zero_offload_t h, int64_t* t, int32_t* last_skipped, double* last_norm,
                                 float* last_clip) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  if (t) *t = h->t;
  if (last_skipped) *last_skipped = h->skipped;
  if (last_norm) *last_norm = h->norm;
  if (last_clip) *last_clip = h->clip;
  return ZERO_OK;
}

zero_status_t zero_offload_destroy(zero_offload_t h) {
  if (!h) return fail(ZERO_EINVAL, "null handle");
  zero_status_t rs = ZERO_OK;
  if (h->has_device) {
    DeviceGuard dg(h->device, h->has_device);
    rs = wait_push(h);
    for (size_t k = 0; k < h->fetch_ev.size(); ++k) {
      if (h->fetch_pending) (void)hipEventSynchronize(h->fetch_ev[k]);
      (void)hipEventDestroy(h->fetch_ev[k]);
    }
    if (h->push_ev) (void)hipEventDestroy(h->push_ev);
    if (h->stats_ev) (void)hipEventDestroy(h->stats_ev);
    if (h->aux) {
      hipError_t e = hipStreamSynchronize(h->aux);
      if (e != hipSuccess && rs == ZERO_OK) rs = hip_fail("hipStreamSynchronize(statistics read-back)", e);
      (void)hipStreamDestroy(h->aux);
    }
  }
  delete h;
  return rs;
}

}  // extern "C"
