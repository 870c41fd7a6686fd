"""Build libmxgemm.so, the gfx950 MX GEMM library, with hipcc (in-tree)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmxgemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Translation units compiled side by side, then linked.
SOURCES = [os.path.join(CSRC, f) for f in ("mxgemm.hip", "mxgrouped.hip", "mxfp6pairs.hip",
                                               "mxgrouped_fp6.hip", "mxdecode.hip")]
HEADERS = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")] + \
          [os.path.join(ROOT, "include", "mxgemm.h")]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Keep packed-FP32 VALU instructions out of the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _run(cmd):
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def _finish(procs, what):
    for proc in procs:
        out, _ = proc.communicate()
        if proc.returncode != 0:
            sys.stderr.write(out)
            raise RuntimeError("hipcc failed building %s" % what)
        yield out


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    objs = [LIB + ".%d.o" % i for i in range(len(SOURCES))]
    cmds = [[HIPCC] + [f for f in FLAGS if f != "-shared"] + ["-c", src, "-o", obj]
            for src, obj in zip(SOURCES, objs)]
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        for cmd in cmds + [link]:
            print(" ".join(cmd), flush=True)
    outs = list(_finish([_run(c) for c in cmds], "libmxgemm.so"))
    outs += list(_finish([_run(link)], "libmxgemm.so"))
    for obj in objs:
        os.remove(obj)
    if verbose:
        # hipcc's host pass warns that it does not know the packed-fp32 feature.
        lines = [l for out in outs for l in out.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            print("\n".join(lines))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
