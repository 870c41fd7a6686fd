"""The CPU oracle and the GPU library's host logic under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, no GPU).

* The oracle: tests/sanitize/oracle_checks.c includes oracle/mx_oracle.c
  and runs every entry point on small ragged shapes, arbitrary bytes,
  non-finite quantizer inputs and the argument errors (gcc).
* The host logic: the library's four translation units are compiled for the
  host only (no device code) with both sanitizers and linked with
  tests/sanitize/host_checks.cpp and a stand-in HIP runtime that has no
  device (tests/sanitize/hip_stub.cpp).  The driver calls every entry point
  of include/mxgemm.h on paths that end before a kernel could launch: the
  plans over shapes up to the ABI's limits, the tile table, the error
  strings, every argument error, and valid calls that stop at the device
  check.
A sanitizer report aborts the program, and the test fails with its output.
"""
import glob
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_DIR = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "microscaled_block_scaled_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert p.returncode == 0, "%s\n%s" % (" ".join(cmd), p.stdout[-4000:])
    return p.stdout


def test_oracle_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_checks")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall", "-Wextra",
          os.path.join(SAN_DIR, "oracle_checks.c"), "-o", exe, "-lm"])
    out = _run([exe], env=dict(ENV, OMP_NUM_THREADS="2"), timeout=300)
    assert "oracle checks passed" in out


def test_host_logic_under_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not available")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    san_host = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer"):
        san_host += ["-Xarch_host", f]
    objs, procs = [], []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen(
            [HIPCC, "--offload-host-only", "-O1", "-g", "-std=c++17"] + san_host + inc
            + ["-c", src, "-o", obj], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
            text=True))
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out[-4000:]
    # The host objects name the device code bundles they would register; the
    # stand-in runtime never reads them, so empty definitions satisfy the link.
    names = set()
    for obj in objs:
        names |= set(re.findall(r"\b(__hip_fatbin_[0-9a-f]+)\b", _run(["nm", "-u", obj])))
    fat = tmp_path / "fatbins.cpp"
    fat.write_text("".join('extern "C" { extern const unsigned char %s[16]; '
                           'const unsigned char %s[16] = {0}; }\n' % (n, n) for n in sorted(names)))
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    for src, obj in ((os.path.join(SAN_DIR, "host_checks.cpp"), "host_checks.o"),
                     (os.path.join(SAN_DIR, "hip_stub.cpp"), "hip_stub.o"),
                     (str(fat), "fatbins.o")):
        _run([CLANG, "-O1", "-g", "-std=c++17"] + san + inc + ["-c", src, "-o",
                                                             str(tmp_path / obj)])
        objs.append(str(tmp_path / obj))
    exe = str(tmp_path / "host_checks")
    _run([CLANG] + san + objs + ["-o", exe])
    out = _run([exe], env=ENV, timeout=300)
    assert "host checks passed" in out
