"""Build the HIP library libmoe_q2.so in-tree for gfx950 (hipcc), and its diagnostic
variant libmoe_q2_timeline.so (the same sources with -DMQ_WG_TIMELINE: per-work-group
timestamps of the decode launches, read by bit_quantized_routed_amd.timeline)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmoe_q2.so")
OUT_TIMELINE = os.path.join(HERE, "libmoe_q2_timeline.so")
SOURCES = ["moe_q2.cpp", "setup.hip", "route.hip", "prep.hip", "ffn_dec.hip", "ffn_mma.hip", "combine.hip", "gemm.hip",
           "cache.hip"]

# Packed fp32 VALU ops are switched off for all device code.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-munsafe-fp-atomics", "-Wno-unused-command-line-argument"]
# Matrix-core kernels keep their accumulators in ordinary VGPRs (no copies out of
# the accumulation registers in the per-block fold).
FILE_FLAGS = {"ffn_mma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose=False, jobs=8, timeline=False):
    out = OUT_TIMELINE if timeline else OUT
    objdir = os.path.join(HERE, "_build_timeline" if timeline else "_build")
    extra = ["-DMQ_WG_TIMELINE"] if timeline else []
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"]
        cmd = ["hipcc", *lang, *DEVICE_FLAGS, *extra, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o",
               obj]
        if verbose:
            print(" ".join(cmd))
        procs.append(subprocess.Popen(cmd))
        if len(procs) >= jobs:
            _wait(procs)
    _wait(procs)
    tmp = out + ".tmp"
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def _wait(procs):
    while procs:
        p = procs.pop(0)
        if p.wait() != 0:
            raise RuntimeError("hipcc failed: %s" % (p.args,))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, timeline="--timeline" in sys.argv))
