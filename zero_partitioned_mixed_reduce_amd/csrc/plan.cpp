// Host-side partition and work table of one rank's shard.
//
// Partition: flatten the tensor list, pad it to N_d equal shards whose length
// is a multiple of `align` elements, rank r owning flat [r*S, r*S + S) clipped
// to [0, psi) -- the flatten/pad/[start, end) rule of "DeepSpeed ZeRO", ZeRO
// Stage 3 基本流程, with start = partition size * rank as in "ZeRO 技术原理"
// 3.3.1.
//
// State layout (this library's choice): the shard is cut at tensor
// boundaries into pieces; each piece's fp32 state starts at an element offset
// congruent, modulo 8, to its 16-bit parameters' element address, so a piece's
// 16-bit and fp32 streams reach their 8- and 16-byte boundaries together and
// the kernels can use vector loads on both after peeling at most 3 elements.
// Pieces are cut into chunks of at most kChunk elements whose starts (after
// the first) are 8-element aligned in the 16-bit data.
#include <stdint.h>
#include <string.h>

#include "zs_internal.h"

namespace zs {

static int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Largest model: every byte count and flat byte offset derived from psi stays far
// inside int64 (the model-state count is about 16 psi).
static constexpr int64_t kMaxPsi = int64_t{1} << 60;

zero_status_t build_plan(const zero_shard_desc_t* d, Plan* out, std::string* err) {
  if (!d || !out) {
    *err = "null description or output";
    return ZERO_EINVAL;
  }
  if (d->dp_size < 1 || d->dp_rank < 0 || d->dp_rank >= d->dp_size) {
    *err = "need dp_size >= 1 and 0 <= dp_rank < dp_size";
    return ZERO_EINVAL;
  }
  if (d->dtype != ZERO_F16 && d->dtype != ZERO_BF16) {
    *err = "dtype must be ZERO_F16 or ZERO_BF16";
    return ZERO_EINVAL;
  }
  const int64_t align = d->align == 0 ? 64 : d->align;
  if (align < 8 || align % 8 != 0) {
    *err = "align must be a positive multiple of 8";
    return ZERO_EINVAL;
  }
  if (d->num_tensors < 1 || d->num_tensors > INT32_MAX || !d->numel) {
    *err = "need 1 <= num_tensors <= 2^31 - 1 and a numel array";
    return ZERO_EINVAL;
  }
  if ((d->param16 == nullptr) == (d->flat_param16 == nullptr)) {
    *err = "give exactly one of param16 (per tensor) or flat_param16";
    return ZERO_EINVAL;
  }
  if (d->grad16 && d->flat_grad16) {
    *err = "give at most one of grad16 (per tensor) or flat_grad16";
    return ZERO_EINVAL;
  }
  const int64_t T = d->num_tensors;
  int64_t psi = 0;
  for (int64_t k = 0; k < T; ++k) {
    if (d->numel[k] < 0) {
      *err = "numel must be >= 0";
      return ZERO_EINVAL;
    }
    if (d->numel[k] > kMaxPsi - psi) {
      *err = "the model exceeds 2^60 elements";
      return ZERO_EINVAL;
    }
    if (d->numel[k] > 0 && d->param16 && !d->param16[k]) {
      *err = "param16 pointer of a non-empty tensor is null";
      return ZERO_EINVAL;
    }
    if (d->numel[k] > 0 && d->grad16 && !d->grad16[k]) {
      *err = "grad16 pointer of a non-empty tensor is null";
      return ZERO_EINVAL;
    }
    psi += d->numel[k];
  }
  const int64_t nd = d->dp_size;
  const int64_t per_rank = (psi + nd - 1) / nd;
  const int64_t S = round_up(per_rank, align);
  const int64_t begin = (int64_t)d->dp_rank * S;
  int64_t valid = psi - begin;
  if (valid < 0) valid = 0;
  if (valid > S) valid = S;

  Plan p;
  memset(&p.info, 0, sizeof(p.info));
  const int64_t end = begin + valid;
  int64_t start = 0, cursor = 0;
  for (int64_t k = 0; k < T; ++k) {
    const int64_t n = d->numel[k];
    const int64_t lo = start > begin ? start : begin;
    const int64_t hi = (start + n) < end ? (start + n) : end;
    if (lo < hi) {
      Piece pc;
      pc.tensor = k;
      pc.tensor_off = lo - start;
      pc.shard_off = lo - begin;
      pc.len = hi - lo;
      const uint64_t paddr = d->param16 ? (uint64_t)(uintptr_t)d->param16[k] + 2 * (uint64_t)pc.tensor_off
                                        : (uint64_t)(uintptr_t)d->flat_param16 + 2 * (uint64_t)lo;
      const int64_t res = (int64_t)((paddr >> 1) & 7);
      pc.state_off = cursor + (((res - cursor) % 8) + 8) % 8;
      cursor = pc.state_off + pc.len;
      p.pieces.push_back(pc);
      // chunks: the first ends where the 16-bit element address is next 8-aligned
      int64_t off = 0;
      while (off < pc.len) {
        int64_t room = kChunk;
        if (off == 0 && res != 0) room = kChunk - res;
        const int64_t len = (pc.len - off) < room ? (pc.len - off) : room;
        Chunk c;
        c.state_off = pc.state_off + off;
        c.flat_off = lo + off;
        c.shard_off = pc.shard_off + off;
        c.p16 = paddr + 2 * (uint64_t)off;
        if (d->grad16)
          c.g16 = (uint64_t)(uintptr_t)d->grad16[k] + 2 * (uint64_t)(pc.tensor_off + off);
        else if (d->flat_grad16)
          c.g16 = (uint64_t)(uintptr_t)d->flat_grad16 + 2 * (uint64_t)(lo + off);
        else
          c.g16 = 0;
        c.len = (int32_t)len;
        c.tensor = (int32_t)k;
        p.chunks.push_back(c);
        off += len;
      }
    }
    start += n;
  }
  int64_t state_elems = round_up(cursor, 64);
  if (state_elems < 64) state_elems = 64;
  p.info.psi = psi;
  p.info.shard_elems = S;
  p.info.shard_begin = begin;
  p.info.valid_elems = valid;
  p.info.state_elems = state_elems;
  p.info.num_pieces = (int64_t)p.pieces.size();
  p.info.num_chunks = (int64_t)p.chunks.size();
  p.info.workspace_bytes = intake_layout((int64_t)p.chunks.size()).end;
  p.info.model_state_bytes = 2 * psi + 2 * psi + 12 * state_elems;
  *out = std::move(p);
  return ZERO_OK;
}

}  // namespace zs
