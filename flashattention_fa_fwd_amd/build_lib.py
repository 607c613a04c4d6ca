"""Build libattn.so (the HIP kernels + C ABI) for gfx950 with hipcc.

Compiles every translation unit under csrc/ in one hipcc invocation into a
shared library next to this file.  Packed-fp32 instructions are disabled
(-packed-fp32-ops).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn.so")
SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_fwd_block.hip", "attn_bwd.hip"]


def hipcc_cmd(out: str) -> list:
    return [
        "hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # keep matrix-instruction accumulators in ordinary VGPRs: the softmax
        # and rescale work on them every step, and AGPRs would need copies
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = hipcc_cmd(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature: that warning is harmless
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
