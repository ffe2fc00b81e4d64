"""The host planner built alone with AddressSanitizer and UndefinedBehaviorSanitizer
(g++, no HIP code) and driven over many descriptions on the CPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = r'''
#include <stdio.h>
#include <string>
#include <vector>
#include "zs_internal.h"
int main() {
  unsigned long long seed = 12345;
  auto rnd = [&]() { seed = seed * 6364136223846793005ULL + 1442695040888963407ULL; return (unsigned)(seed >> 33); };
  long checked = 0;
  for (int it = 0; it < 3000; ++it) {
    int T = 1 + rnd() % 9;
    std::vector<int64_t> numel(T);
    std::vector<void*> ptrs(T), gptrs(T);
    int64_t psi = 0;
    for (int k = 0; k < T; ++k) {
      numel[k] = (rnd() % 4 == 0) ? 0 : (rnd() % 50000);
      psi += numel[k];
      ptrs[k] = (void*)(uintptr_t)(0x100000 + 256ull * k * 1000 + 2 * (rnd() % 8));
      gptrs[k] = (void*)(uintptr_t)(0x9000000 + 256ull * k * 1000 + 2 * (rnd() % 8));
    }
    zero_shard_desc_t d = {};
    d.dp_size = 1 + rnd() % 70;
    d.dp_rank = rnd() % d.dp_size;
    d.dtype = 1 + rnd() % 2;
    d.align = (rnd() % 3 == 0) ? 8 * (1 + rnd() % 16) : 0;
    d.num_tensors = T;
    d.numel = numel.data();
    if (rnd() % 2) d.param16 = ptrs.data(); else d.flat_param16 = (void*)0x100000;
    if (rnd() % 2) d.grad16 = (const void* const*)gptrs.data();
    zs::Plan p;
    std::string err;
    if (zs::build_plan(&d, &p, &err) != ZERO_OK) { printf("unexpected error: %s\n", err.c_str()); return 1; }
    int64_t covered = 0, last_state_end = 0;
    for (const auto& pc : p.pieces) {
      if (pc.state_off < last_state_end || pc.len <= 0) { printf("bad piece\n"); return 1; }
      last_state_end = pc.state_off + pc.len;
      covered += pc.len;
    }
    if (covered != p.info.valid_elems || last_state_end > p.info.state_elems) { printf("bad cover\n"); return 1; }
    int64_t sum = 0;
    for (const auto& c : p.chunks) {
      if (c.len <= 0 || c.len > zs::kChunk) { printf("bad chunk\n"); return 1; }
      sum += c.len;
    }
    if (sum != covered) { printf("bad chunks\n"); return 1; }
    ++checked;
  }
  // invalid descriptions are rejected, not crashed on
  zero_shard_desc_t d = {};
  zs::Plan p;
  std::string err;
  if (zs::build_plan(&d, &p, &err) == ZERO_OK) return 1;
  if (zs::build_plan(nullptr, &p, &err) == ZERO_OK) return 1;
  printf("ok %ld\n", checked);
  return 0;
}
'''


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_under_asan_ubsan(tmp_path):
    src = tmp_path / "driver.cpp"
    src.write_text(DRIVER)
    exe = tmp_path / "driver"
    csrc = os.path.join(ROOT, "zero_partitioned_mixed_reduce_amd", "csrc")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", csrc, str(src), os.path.join(csrc, "plan.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok 3000")
