"""Build the synthetic-input fillers: libzsynth.so (host, OpenMP) and
libzsynth_gpu.so (gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(HERE, "libzsynth.so")
GPU_LIB = os.path.join(HERE, "libzsynth_gpu.so")
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False):
    cmds = [
        (HOST_LIB, ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-Wall",
                    "-o", HOST_LIB + ".tmp", os.path.join(HERE, "zsynth.c")]),
        (GPU_LIB, ["hipcc", *HIP_FLAGS, "-o", GPU_LIB + ".tmp", os.path.join(HERE, "zsynth_gpu.hip")]),
    ]
    for out, cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)
    return HOST_LIB, GPU_LIB


if __name__ == "__main__":
    print(build(verbose=True))
