"""Build libpic_stitch.so (HIP, gfx950) in-tree, next to this file.  Each
source is compiled to an object of its own under _build/ (in parallel), then
the objects are linked."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libpic_stitch.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = [os.path.join(CSRC, "stitch.hip"), os.path.join(CSRC, "attend.hip"),
           os.path.join(CSRC, "attend_mla.hip"), os.path.join(CSRC, "attend_boundary.hip"),
           os.path.join(CSRC, "attend_gqa.hip"),
           os.path.join(CSRC, "cdc.hip"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(CSRC, "attend_plan.cpp")]

# Packed-fp32 instructions are kept out of the device code on purpose.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

# Flags of single sources.  The GQA tile kernel's matrix-core instructions
# take their accumulators in VGPRs: with them in AGPRs the compiler copied all
# 32 out and back at every step (its register budget has room for them).  The
# latent kernel's one- and two-wave workgroups need the AGPRs and keep the
# default.
SOURCE_FLAGS = {"attend_gqa.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def build(verbose: bool = False, extra=()) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs, objects = [], []
    for src in SOURCES:
        name = os.path.basename(src)
        obj = os.path.join(BUILD_DIR, name + ".o")
        cmd = [hipcc, *HIP_FLAGS, *SOURCE_FLAGS.get(name, []), *extra, "-c", "-I", INCLUDE,
               "-I", CSRC, "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((cmd, subprocess.Popen(cmd)))
        objects.append(obj)
    failed = [cmd for cmd, p in jobs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    tmp = LIBRARY + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-fPIC", "-shared", "-o", tmp, *objects]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
