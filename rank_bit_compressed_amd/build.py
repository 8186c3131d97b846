"""Build librbc_kvc.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librbc_kvc.so")
SOURCES = ["api.cpp", "decode_head.hip", "decode_int4.hip", "decode_res.hip", "decode_shared.hip", "compress.hip", "dense.hip", "fit.hip", "alloc.hip", "plan.cpp", "tucker.hip", "evict.hip", "check.hip", "noalloc.hip", "peaks.hip", "tfit.hip"]
# -packed-fp32-ops: no packed fp32 VALU instructions are generated (fp16 packed math is unaffected)
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared", "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics",
         "-mllvm", "-amdgpu-mfma-vgpr-form"]  # MFMA results in VGPRs: no accumulator copies


def build(verbose: bool = False, extra=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *FLAGS, *extra, *srcs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed")
    if verbose:
        sys.stderr.write(r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
