"""Build libmxgemm.so, the gfx950 MX GEMM library, with hipcc (in-tree)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmxgemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = [os.path.join(CSRC, "mxgemm.hip")]
HEADERS = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")] + \
          [os.path.join(ROOT, "include", "mxgemm.h")]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Keep packed-FP32 VALU instructions out of the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout)
        raise RuntimeError("hipcc failed building libmxgemm.so")
    if verbose and proc.stdout.strip():
        # hipcc's host pass warns that it does not know the packed-fp32 feature.
        lines = [l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            print("\n".join(lines))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
