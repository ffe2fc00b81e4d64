// Internal layout shared by the host plan and the gfx950 kernels.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "zero_shard.h"

namespace zs {

// Elements per work item.  A multiple of 8, so that every chunk after the
// first of a tensor piece starts on a 16-byte boundary of the 16-bit data.
#ifndef ZS_CHUNK
#define ZS_CHUNK 8192
#endif
constexpr int64_t kChunk = ZS_CHUNK;
// Local-reduce fan-in limit (rank pointers travel as kernel arguments).
constexpr int kMaxRanks = 64;
// Parts per chunk of the local-reduce intake passes over several rank slices (one
// block per part, one partial sum per part): 2048-element parts measured 5-6% faster
// than whole chunks for the local reduce of 8 ranks, 1024-element parts slower.
#ifndef ZS_REDUCE_PARTS
#define ZS_REDUCE_PARTS 4
#endif
constexpr int kIntakeParts = ZS_REDUCE_PARTS;
constexpr int kBlock = 256;
// Blocks of an intake pass whose partial sums one group combines (a group's last
// block adds them; the last group adds the group sums).
constexpr int kGroup = 256;
static_assert(kGroup == kBlock, "a group's partials are read one per thread");

// One work item: a run of `len` consecutive shard elements inside one tensor.
struct alignas(16) Chunk {
  int64_t state_off;  // offset in master / m / v / red
  int64_t flat_off;   // flat model index of the first element (rank buffers are flat)
  int64_t shard_off;  // logical offset inside the shard
  uint64_t p16;       // device address of the first 16-bit parameter
  uint64_t g16;       // device address of the first registered gradient element, or 0
  int32_t len;
  int32_t tensor;
};
static_assert(sizeof(Chunk) == 48, "chunk layout");

struct Slot {
  int64_t t;      // applied steps
  double p1, p2;  // beta1^t, beta2^t (fp64 running products)
  float scale;    // dynamic loss scale
  int32_t good;   // consecutive steps without overflow since the last scale change
};
static_assert(sizeof(Slot) == 32, "slot layout");

// Device-resident scalars of the step (first 256 bytes of the workspace).
//
// Step counters live in two slots, selected on the device, so that a step needs no
// host state and can be replayed from a captured graph.  Between steps the latest
// counters are in slot[cur_slot ^ 1].  The first intake pass of a step reads its
// loss scale there and its last block flips cur_slot; the Adam pass then reads
// slot[cur_slot] (the latest) and writes the next counters to slot[cur_slot ^ 1].
// A repeated intake in the same step does not flip and reads slot[cur_slot].
struct alignas(256) DevScalars {
  double local_sumsq;  // this rank's sum of u^2 (statistics pass)
  int32_t local_flag;  // this rank's non-finite flag
  uint32_t counter;    // groups of an intake pass that have completed (reset by the last one)
  Slot slot[2];        // step counters (see above)
  double norm;         // report of the last zero_adam_step
  float clip;
  int32_t skipped;
  int64_t report_t;
  uint32_t wait_timeouts;  // segment waits that gave up (see SegState)
  uint32_t cur_slot;       // 0 or 1 (see above)
};
static_assert(sizeof(DevScalars) == 256, "scalar block");

// Completion of one segment of the 16-bit write-back (chunk-pipelined step).
// A segment is a run of consecutive chunks.  Work item i of the kernel that
// writes the 16-bit slice arrives, once its stores are complete, on sub-counter
// i % kSegSubs of its segment (spreading the atomics over several addresses);
// the last arrival on a sub-counter re-arms it and arrives on `count`, and the
// last of those re-arms `count` and publishes the step's number in `epoch`.
constexpr int kMaxSegments = 256;
constexpr int kSegSubs = 16;
struct alignas(64) SegSub {
  uint32_t count;  // work items of this sub-counter that have arrived
};
struct alignas(64) SegState {
  uint64_t epoch;  // 1-based zero_adam_step call whose write-back of this segment is complete
  uint32_t count;  // sub-counters of the current write-back that have completed
  SegSub sub[kSegSubs];
};
static_assert(sizeof(SegSub) == 64 && sizeof(SegState) == 64 * (kSegSubs + 1), "segment layout");

// Segment configuration passed to the kernel that writes the 16-bit slice.
struct SegArgs {
  SegState* seg;       // null: no completion tracking
  int64_t per_seg;     // chunks per segment (the last one may hold fewer)
  int64_t n_chunks;
  int32_t n_seg;
  uint64_t epoch;      // number of this zero_adam_step call (1-based)
};

// Completion counter of one group of intake blocks, on its own 64-byte line.
struct alignas(64) GroupCount {
  uint32_t count;  // blocks of the group that have stored their partial (re-armed by the last)
};
static_assert(sizeof(GroupCount) == 64, "group counter layout");

// Where an intake pass leaves its partial sums of squares (fp64, as bits).
struct IntakeParts {
  uint64_t* part;      // one per block
  GroupCount* gcount;  // one per group of kGroup blocks
  uint64_t* gpart;     // one per group: the sum of its blocks' partials
};

// Gradient source of the Adam pass, fixed by the step's intake.
enum GradSource : int {
  kGradFlat16 = 0,      // the flat already-reduced 16-bit gradient given to the intake
  kGradChunk16 = 1,     // the already-reduced 16-bit gradient registered at init
  kGradRed = 2,         // fp32 u, stored in red by the intake
  kGradRed16 = 3,       // the 16-bit reduce output, stored in red by the intake
  kGradAccFlat16 = 4,   // u = (accumulator in red + the flat 16-bit gradient) * inv, recomputed
  kGradAccChunk16 = 5,  // u = (accumulator in red + the registered 16-bit gradient) * inv, recomputed
  kGradAcc = 6,         // u = accumulator in red * inv, recomputed
};

constexpr int64_t kSegOff = sizeof(DevScalars);
constexpr int64_t kChunksOff = kSegOff + kMaxSegments * (int64_t)sizeof(SegState);

// Workspace after the chunk table: per-block partials, group counters and group
// sums, sized for the largest intake grid (one block per part of a chunk).
struct IntakeLayout {
  int64_t part_off, gcount_off, gpart_off, end;
};
inline int64_t intake_groups(int64_t n_chunks) { return (n_chunks * kIntakeParts + kGroup - 1) / kGroup; }
inline IntakeLayout intake_layout(int64_t n_chunks) {
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  const int64_t n_groups = intake_groups(n_chunks);
  IntakeLayout l;
  l.part_off = up(kChunksOff + n_chunks * (int64_t)sizeof(Chunk));
  l.gcount_off = up(l.part_off + 8 * n_chunks * kIntakeParts);
  l.gpart_off = up(l.gcount_off + n_groups * (int64_t)sizeof(GroupCount));
  l.end = up(l.gpart_off + 8 * n_groups);
  return l;
}

struct Piece {
  int64_t tensor, tensor_off, shard_off, state_off, len;
};

struct Plan {
  zero_shard_info_t info;
  std::vector<Piece> pieces;
  std::vector<Chunk> chunks;
};

// Validates the description and lays out pieces and chunks.  Returns
// ZERO_OK or ZERO_EINVAL with *err set.
zero_status_t build_plan(const zero_shard_desc_t* d, Plan* out, std::string* err);

}  // namespace zs
