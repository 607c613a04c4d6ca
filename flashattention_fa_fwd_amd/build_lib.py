"""Build libattn.so (the HIP kernels + C ABI) for gfx950 with hipcc.

Compiles every translation unit under csrc/ to an object (in parallel) and
links them into a shared library next to this file.  Packed-fp32
instructions are disabled (-packed-fp32-ops).  The dK/dV kernel's unit is
scheduled with LLVM's iterative-ILP strategy (measured faster for that
kernel, with bitwise-equal results; the other kernels are faster with the
default).
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn.so")
SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_fwd_block.hip", "attn_bwd_dq.hip", "attn_bwd_dkdv.hip"]
EXTRA_FLAGS = {"attn_bwd_dkdv.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}

COMMON = [
    "hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep matrix-instruction accumulators in ordinary VGPRs: the softmax
    # and rescale work on them every step, and AGPRs would need copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def compile_cmd(src: str, obj: str) -> list:
    return [*COMMON, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature, nor the
    # device-only scheduler option: those warnings are harmless
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and "argument unused during compilation" not in l)
    return r.returncode, errs


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="attn_build_") as tmpd:
        objs = [os.path.join(tmpd, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [compile_cmd(s, o) for s, o in zip(SOURCES, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
            results = list(ex.map(_run, cmds))
        for (rc, errs), src in zip(results, SOURCES):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {src} ({rc}):\n{errs}")
            if verbose and errs.strip():
                print(errs)
        tmp = LIB + ".tmp"
        link = ["hipcc", "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        rc, errs = _run(link)
        if rc != 0:
            raise RuntimeError(f"hipcc link failed ({rc}):\n{errs}")
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
