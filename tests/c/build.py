"""Builds the C test programs of the ABI (test infrastructure, not the product):
libstep_from_c.so, the step driven from plain C, linked against the library,
the C oracle and the HIP runtime.  Called by __graft_entry__.build() after the
library and the oracle are built."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
LIB = os.path.join(HERE, "libstep_from_c.so")


def build(verbose=False):
    lib_dir = os.path.join(ROOT, "zero_partitioned_mixed_reduce_amd", "lib")
    orc_dir = os.path.join(ROOT, "oracle")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "step_from_c.c"), "-o", LIB + ".tmp",
           "-L", lib_dir, "-lzero_shard", "-L", orc_dir, "-lzero_oracle", "-L", os.path.join(ROCM, "lib"),
           "-lamdhip64", "-lm", "-Wl,-rpath," + ":".join([lib_dir, orc_dir, os.path.join(ROCM, "lib")])]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)


if __name__ == "__main__":
    build(verbose=True)
