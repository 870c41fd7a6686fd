"""Register use of the built kernels (CPU only: reads the gfx950 code objects'
metadata notes out of libmxgemm.so with the ROCm LLVM tools).

A GEMM kernel that spills in its main loop is still correct -- every parity
test passes -- but it moves its spills through scratch memory on every slab
(a change that formed the copy limits per slab once pushed the mixed-format
kernels to hundreds of spilled registers and 30 times the GEMM's own HBM
traffic).  So the register budget is checked on the build itself: every
kernel within the VGPRs its launch shape allows (two waves per SIMD for the
512-thread workgroups), and no kernel spilling more than a few registers."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "microscaled_block_scaled_amd", "libmxgemm.so")
LLVM = "/opt/rocm/llvm/bin"
MAX_SPILLED_VGPRS = 16


def _kernels(tmp_path):
    fatbin = str(tmp_path / "fatbin.bin")
    subprocess.run([LLVM + "/llvm-objcopy", "--dump-section", ".hip_fatbin=" + fatbin, LIB],
                   check=True)
    data = open(fatbin, "rb").read()
    starts = [m.start() for m in re.finditer(re.escape(b"__CLANG_OFFLOAD_BUNDLE__"), data)]
    assert starts, "no offload bundle in the library"
    res = {}
    for j, st in enumerate(starts):
        end = starts[j + 1] if j + 1 < len(starts) else len(data)
        bundle = str(tmp_path / ("b%d.bin" % j))
        with open(bundle, "wb") as f:
            f.write(data[st:end])
        co = str(tmp_path / ("co%d.o" % j))
        r = subprocess.run([LLVM + "/clang-offload-bundler", "--unbundle", "--type=o",
                            "--input=" + bundle, "--output=" + co,
                            "--targets=hipv4-amdgcn-amd-amdhsa--gfx950"],
                           capture_output=True, text=True)
        if r.returncode != 0:
            continue
        notes = subprocess.run([LLVM + "/llvm-readelf", "--notes", co], capture_output=True,
                               text=True, check=True).stdout
        # one YAML list entry per kernel, fields in alphabetical order
        for block in re.split(r"\n\s*- \.", notes)[1:]:
            fields = dict(re.findall(r"^\s*\.?([a-z_]+):\s+(\S+)\s*$", "." + block, re.M))
            if "symbol" not in fields or "name" not in fields:
                continue
            res[fields["name"]] = {k: int(fields[k]) for k in
                                   ("vgpr_count", "vgpr_spill_count", "max_flat_workgroup_size",
                                    "group_segment_fixed_size")
                                   if k in fields and fields[k].isdigit()}
    return res


def test_kernels_fit_their_register_budget(tmp_path):
    if not os.path.exists(LIB):
        pytest.skip("libmxgemm.so is not built")
    for tool in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf"):
        if not os.path.exists(os.path.join(LLVM, tool)):
            pytest.skip("ROCm LLVM tools not available")
    ks = _kernels(tmp_path)
    tiles = {k: v for k, v in ks.items() if "tile_kernel" in k}
    assert len(tiles) > 100, len(tiles)
    over = [(k, v) for k, v in tiles.items() if v.get("vgpr_spill_count", 0) > MAX_SPILLED_VGPRS]
    assert not over, over[:5]
    # 512-thread workgroups run two waves per SIMD: at most 256 VGPRs each
    wide = [(k, v) for k, v in tiles.items()
            if v.get("max_flat_workgroup_size", 0) >= 512 and v.get("vgpr_count", 0) > 256]
    assert not wide, wide[:5]
    # the decode kernels: the 7 pairs of E2M1 / E4M3 / E5M2 other than an
    # 8-bit A with an E2M1 B, and the wide slabs (8, 16 and 32 A rows) of
    # those two pairs, x 2 output types, none spilling at all
    dec = {k: v for k, v in ks.items() if "decode_kernel" in k}
    assert len(dec) == 26, sorted(dec)
    assert not [(k, v) for k, v in dec.items() if v.get("vgpr_spill_count", 0) > 0]


def test_decode_kernel_lds_matches_the_copy_model(tmp_path):
    """The decode kernels' LDS (from the code objects) is what the copy
    model's geometry implies: 4 waves x (S slabs + R period buffers of 1 KB)
    plus the 4 slot offsets of the partial tiles, so the model checks the
    ring the kernel really has."""
    if not os.path.exists(LIB):
        pytest.skip("libmxgemm.so is not built")
    for tool in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf"):
        if not os.path.exists(os.path.join(LLVM, tool)):
            pytest.skip("ROCm LLVM tools not available")
    import sys
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import test_copy_bounds_cpu as cb
    seen = 0
    for name, v in _kernels(tmp_path).items():
        m = re.search(r"decode_kernelILi(\d)ELi(\d)ELi(\d)ELi(\d+)E", name)
        if not m:
            continue
        fa, fb, wide = int(m.group(1)), int(m.group(2)), int(m.group(4))
        kv, RA, RB, MA, ncopy, S, R = cb.decode_geo(fa, fb, wide)
        want = (cb.DECODE_WAVES * (S * (MA * RA + cb.DECODE_ROWS * RB) + R * 1024)
                + cb.DECODE_OFFS)
        assert v.get("group_segment_fixed_size") == want, (name, v, want)
        seen += 1
    assert seen == 26
