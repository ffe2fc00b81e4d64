/* The C ABI used from plain C (C99): both headers compile as C, and the
 * host-only calls of the library answer as documented.  Prints one line per
 * check; exits non-zero on the first failure.  No GPU call is made: the
 * device addresses in the description are never dereferenced by
 * zero_shard_plan. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "zero_offload.h"
#include "zero_shard.h"

#define CHECK(cond, what)                                     \
  do {                                                        \
    if (!(cond)) {                                            \
      printf("FAIL %s (last error: %s)\n", what, zero_last_error()); \
      return 1;                                               \
    }                                                         \
    printf("ok %s\n", what);                                  \
  } while (0)

int main(void) {
  /* three tensors, 4 ranks, rank 3: psi = 1000 + 37 + 64000 = 65037, S = 64 * ceil(ceil(65037 / 4) / 64) */
  const int64_t numel[3] = {1000, 37, 64000};
  zero_shard_desc_t d;
  memset(&d, 0, sizeof d);
  d.dp_size = 4;
  d.dp_rank = 3;
  d.dtype = ZERO_BF16;
  d.num_tensors = 3;
  d.numel = numel;
  d.flat_param16 = (void*)(uintptr_t)(1u << 20);
  zero_shard_info_t info;
  CHECK(zero_shard_plan(&d, &info) == ZERO_OK, "plan");
  CHECK(info.psi == 65037, "psi");
  CHECK(info.shard_elems == 16320, "shard length");
  CHECK(info.shard_begin == 3 * 16320, "shard begin");
  CHECK(info.valid_elems == 65037 - 3 * 16320, "valid elements");
  CHECK(info.state_elems >= info.valid_elems && info.workspace_bytes > 0, "state and workspace sizes");

  d.dp_rank = 4; /* out of range */
  CHECK(zero_shard_plan(&d, &info) == ZERO_EINVAL, "bad rank is EINVAL");
  CHECK(strlen(zero_last_error()) > 0, "error message");
  CHECK(zero_shard_plan(NULL, &info) == ZERO_EINVAL, "null description is EINVAL");
  CHECK(zero_adam_step(NULL, NULL, 1, NULL) == ZERO_EINVAL, "null handle is EINVAL");
  CHECK(zero_offload_query(NULL, NULL, NULL, NULL, NULL) == ZERO_EINVAL, "null offload handle is EINVAL");
  CHECK(ZERO_DEVICE_LOSS_SCALE == 0.0f && ZERO_ACCUMULATED == -1, "constants");
  return 0;
}
