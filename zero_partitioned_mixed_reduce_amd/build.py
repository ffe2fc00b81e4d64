"""Build libzero_shard.so (gfx950) in-tree.

hipcc flags: -O3, no fused multiply-add contraction (-ffp-contract=off) so
every float operation rounds once as the method's fp32 arithmetic specifies,
the default correctly rounded fp32 division and square root, IEEE denormals,
and packed-fp32 instructions disabled.

The offloaded (host) step is plain C++ built by g++ with the same
floating-point rules (-ffp-contract=off, no fast-math); its AVX-512 loops
carry their own target attributes, so the rest of the object is baseline
x86-64.  It is linked into the same library.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_DIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIB_DIR, "libzero_shard.so")
SOURCES = ["plan.cpp", "zero_shard_api.cpp", "kernels.hip"]
HOST_SOURCES = ["offload.cpp"]
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-result"]
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
              "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]


def host_objects(verbose: bool = False, extra_flags=()):
    """Compiles the host-only sources; returns the object paths."""
    objs = []
    for s in HOST_SOURCES:
        obj = os.path.join(LIB_DIR, os.path.splitext(s)[0] + ".o")
        cmd = ["g++", *HOST_FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
               os.path.join(CSRC, s), "-o", obj + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(obj + ".tmp", obj)
        objs.append(obj)
    return objs


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    objs = host_objects(verbose)
    cmd = ["hipcc", *HIP_FLAGS, *extra_flags, "-shared", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", LIB + ".tmp"]
    for s in SOURCES:
        path = os.path.join(CSRC, s)
        cmd += (["-x", "hip", path, "-x", "none"] if s.endswith(".cpp") else [path])
    cmd += [*objs, "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
