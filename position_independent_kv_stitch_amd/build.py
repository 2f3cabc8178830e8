"""Build libpic_stitch.so (HIP, gfx950) in-tree, next to this file."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libpic_stitch.so")
SOURCES = [os.path.join(CSRC, "stitch.hip"), os.path.join(CSRC, "attend.hip"),
           os.path.join(CSRC, "attend_mla.hip"), os.path.join(CSRC, "attend_boundary.hip"),
           os.path.join(CSRC, "attend_gqa.hip"),
           os.path.join(CSRC, "cdc.hip"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(CSRC, "attend_plan.cpp")]

# Packed-fp32 instructions are kept out of the device code on purpose.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False, extra=()) -> str:
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    tmp = LIBRARY + ".tmp"
    cmd = [hipcc, *HIP_FLAGS, *extra, "-shared", "-I", INCLUDE, "-I", CSRC, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
