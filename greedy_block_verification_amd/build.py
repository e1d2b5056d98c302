"""Build libsv.so (HIP kernels + host runtime) for gfx950 with hipcc, in-tree."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsv.so")
SOURCES = ["sv_kernels.hip", "sv_runtime.cpp"]

# -ffp-contract=off: no fused multiply-adds the source does not spell out, so
# every instantiation of a kernel rounds identically.  Packed-fp32 VALU ops
# are disabled for all device code.
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
    "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    # the first 14 dwords of a kernel's arguments (pointers and scalars) go
    # into SGPRs before its waves start
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *FLAGS, "-I", os.path.join(ROOT, "include"), "-o", LIB + ".tmp"]
    cmd += ["-x", "hip"] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libsv.so")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
