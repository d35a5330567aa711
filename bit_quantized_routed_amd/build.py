"""Build the HIP library libmoe_q2.so in-tree for gfx950 (hipcc)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmoe_q2.so")
SOURCES = ["moe_q2.cpp", "setup.hip", "route.hip", "prep.hip", "ffn_dec.hip", "ffn_mma.hip", "combine.hip", "gemm.hip",
           "cache.hip"]

# Packed fp32 VALU ops are switched off for all device code.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-munsafe-fp-atomics", "-Wno-unused-command-line-argument"]
# Matrix-core kernels keep their accumulators in ordinary VGPRs (no copies out of
# the accumulation registers in the per-block fold).
FILE_FLAGS = {"ffn_mma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose=False, jobs=8):
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"]
        cmd = ["hipcc", *lang, *DEVICE_FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd))
        procs.append(subprocess.Popen(cmd))
        if len(procs) >= jobs:
            _wait(procs)
    _wait(procs)
    tmp = OUT + ".tmp"
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(tmp, OUT)
    return OUT


def _wait(procs):
    while procs:
        p = procs.pop(0)
        if p.wait() != 0:
            raise RuntimeError("hipcc failed: %s" % (p.args,))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
