"""Build tests/probes/libisa_probe.so (test infrastructure, gfx950): the
single-instruction probes and the shader-clock monitor."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libisa_probe.so")


def build(verbose: bool = False) -> str:
    cmd = ["hipcc", "--offload-arch=gfx950", "-O2", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(HERE, "isa_probe.hip"), os.path.join(HERE, "clock_probe.hip"), "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{r.stdout}{r.stderr}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
