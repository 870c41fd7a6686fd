"""The C-ABI library without a GPU: it loads, exports every function the
header declares, and rejects bad arguments before touching HIP."""
import ctypes
import os
import re

import pytest

import microscaled_block_scaled_amd as mxg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxgemm.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert {"mx_gemm", "mx_strerror", "mx_gemm_plan"} <= set(names)
    L = mxg.lib()
    for n in names:
        assert hasattr(L, n), n


def test_header_constants_match_binding():
    src = open(HEADER).read()
    consts = dict((k, int(v)) for k, v in re.findall(r"\b(MX_[A-Z0-9_]+)\s*=\s*(-?\d+)", src))
    for k, v in consts.items():
        short = k[3:]
        if hasattr(mxg, short):
            assert getattr(mxg, short) == v, k
        elif hasattr(mxg, k):
            assert getattr(mxg, k) == v, k
    assert consts["MX_FMT_E2M1"] == mxg.FMT_E2M1 and consts["MX_OUT_BF16"] == mxg.OUT_BF16
    limits = dict((k, 1 << int(v)) for k, v in
                  re.findall(r"#define (MX_MAX_[A-Z]+) \(\(int64_t\)1 << (\d+)\)", src))
    assert limits == {"MX_MAX_DIM": mxg.MAX_DIM, "MX_MAX_K": mxg.MAX_K}
    assert int(re.search(r"#define MX_MAX_K_BF16 \(\(int64_t\)1 << (\d+)\)", src).group(1)) \
        == mxg.MAX_K_BF16.bit_length() - 1
    assert int(re.search(r"#define MX_MAX_SPLIT_K (\d+)", src).group(1)) == mxg.MAX_SPLIT_K
    assert int(re.search(r"#define MX_MAX_GROUPS (\d+)", src).group(1)) == mxg.MAX_GROUPS
    assert int(re.search(r"#define MX_DECODE_TILE (\d+)", src).group(1)) == mxg.DECODE_TILE
    assert consts["MX_VARIANT_DECODE"] == mxg.VARIANT_DECODE


def test_strerror_covers_codes():
    for code in range(-11, 1):
        s = mxg.strerror(code)
        assert s and s != "unknown error code", code
    assert mxg.strerror(5) == "unknown error code"


@pytest.mark.parametrize("fmt,M,N,K,out,code", [
    (0, 16, 16, 128, 1, mxg.MX_ERR_FORMAT),
    (6, 16, 16, 128, 1, mxg.MX_ERR_FORMAT),
    (1, 16, 16, 128, 0, mxg.MX_ERR_OUT_DTYPE),
    (2, 16, 16, 128, 7, mxg.MX_ERR_OUT_DTYPE),
    (1, 0, 16, 128, 1, mxg.MX_ERR_SHAPE),
    (1, 16, 0, 128, 1, mxg.MX_ERR_SHAPE),
    (1, 16, 16, 0, 1, mxg.MX_ERR_SHAPE),
    (1, 16, 16, 64, 1, mxg.MX_ERR_SHAPE),
    (2, 16, 16, 100, 1, mxg.MX_ERR_SHAPE),
    (2, 16, 16, 192, 2, mxg.MX_ERR_SHAPE),
    (2, 16, 16, -128, 2, mxg.MX_ERR_SHAPE),
    (2, (1 << 30) + 1, 16, 128, 2, mxg.MX_ERR_SHAPE),
    (2, 16, (1 << 30) + 1, 128, 2, mxg.MX_ERR_SHAPE),
    (2, 16, 16, (1 << 24) + 128, 2, mxg.MX_ERR_SHAPE),
])
def test_argument_errors(fmt, M, N, K, out, code):
    L = mxg.lib()
    p = mxg.MxPlan()
    assert L.mx_gemm_plan(fmt, M, N, K, out, ctypes.byref(p)) == code
    # Same code from mx_gemm, before any pointer is looked at or HIP called.
    assert L.mx_gemm(fmt, M, N, K, None, None, None, None, None, out, None) == code


def test_largest_shapes_accepted():
    p = mxg.MxPlan()
    L = mxg.lib()
    assert L.mx_gemm_plan(2, 1 << 30, 16, 1 << 24, 2, ctypes.byref(p)) == mxg.MX_OK
    assert L.mx_gemm_plan(1, 16, 1 << 30, 1 << 24, 1, ctypes.byref(p)) == mxg.MX_OK


def test_null_and_alignment_errors():
    L = mxg.lib()
    good = 1 << 20            # never dereferenced: checks fail first
    args = [good, good, good, good, good]
    for i in range(5):
        a = list(args)
        a[i] = None
        assert L.mx_gemm(1, 16, 16, 128, *a[:4], a[4], 1, None) == mxg.MX_ERR_NULL
    for i, mis in ((0, 8), (2, 4), (4, 2), (1, 2), (3, 1)):
        a = list(args)
        a[i] = good + mis
        assert L.mx_gemm(1, 16, 16, 128, *a[:4], a[4], 1, None) == mxg.MX_ERR_ALIGN, i
    assert L.mx_gemm_plan(1, 16, 16, 128, 1, None) == mxg.MX_ERR_NULL


def test_no_device_reported():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible here")
    good = 1 << 20
    rc = mxg.lib().mx_gemm(2, 16, 16, 128, good, good, good, good, good, 2, None)
    assert rc == mxg.MX_ERR_NO_DEVICE


def test_tile_shapes_and_forced_tile_errors():
    shapes = mxg.tile_shapes()
    assert (256, 192) in shapes and len(shapes) == len(set(shapes))
    for bm, bn in shapes:
        assert bm % 32 == 0 and bn % 32 == 0
    p = mxg.plan(mxg.FMT_E4M3, 2048, 6144, 4096)
    assert (p["tile_m"], p["tile_n"]) in shapes
    L = mxg.lib()
    good = 1 << 20
    # An unknown tile, a bad split or a bad shape is rejected before any HIP call.
    assert L.mx_gemm_tile(2, 64, 64, 128, good, good, good, good, good, 2, 100, 64, 0,
                          None) == mxg.MX_ERR_SHAPE
    assert L.mx_gemm_tile(2, 64, 64, 100, good, good, good, good, good, 2, 256, 192, 0,
                          None) == mxg.MX_ERR_SHAPE
    assert L.mx_gemm_tile(2, 64, 64, 128, good, good, good, good, good, 2, 256, 192, -1,
                          None) == mxg.MX_ERR_SHAPE
    assert L.mx_gemm_tile(2, 64, 64, 128, good, good, good, good, good, 2, 256, 192,
                          mxg.MAX_SPLIT_K + 1, None) == mxg.MX_ERR_SHAPE
    assert L.mx_gemm_tile(9, 64, 64, 128, good, good, good, good, good, 2, 256, 192, 0,
                          None) == mxg.MX_ERR_FORMAT
    assert L.mx_gemm_tile(2, 64, 64, 128, None, good, good, good, good, 2, 256, 192, 0,
                          None) == mxg.MX_ERR_NULL


def test_plan_shapes():
    p = mxg.plan(mxg.FMT_E4M3, 2048, 6144, 4096, mxg.OUT_BF16)
    assert p["workgroups"] >= 1 and p["threads"] % 64 == 0
    assert p["tile_m"] % 16 == 0 and p["tile_n"] % 16 == 0
    tiles = -(-2048 // p["tile_m"]) * -(-6144 // p["tile_n"]) * p["split_k"]
    assert p["workgroups"] == tiles
    with pytest.raises(ValueError):
        mxg.plan(mxg.FMT_E4M3, 16, 16, 100)


@pytest.mark.parametrize("M,N,K", [(1, 4096, 28672), (32, 100, 16384), (64, 8192, 28672),
                                   (33, 28672, 4096), (8, 28672, 512)])
def test_plan_small_m_uses_short_tile(M, N, K):
    for fmt in (mxg.FMT_E2M1, mxg.FMT_E4M3):
        p = mxg.plan(fmt, M, N, K)
        assert p["variant"] == mxg.VARIANT_TILE
        # HBM-bound: a short tile (64 or 128 rows), whatever its padding
        assert (p["tile_m"], p["tile_n"]) in ((64, 256), (128, 128))
        tiles = -(-N // p["tile_n"])
        assert p["workgroups"] == tiles * p["split_k"]
        # split only up to one wave of workgroups (half of one for 64 rows)
        cap = 256 if p["tile_m"] == 128 else 128
        assert p["workgroups"] <= cap or p["split_k"] == 1
        if tiles <= 64 and K >= 8192:
            assert p["split_k"] > 1 and p["workspace_bytes"] > 0


@pytest.mark.parametrize("M,N,K", [(1, 8192, 28672), (8, 8192, 28672), (32, 8192, 4096),
                                   (16, 14336, 4096), (5, 8161, 2048), (8, 6144, 28672),
                                   (32, 100, 512), (1, 16384, 8192), (8, 28672, 28672),
                                   (16, 3072, 14336), (1, 12288, 1024), (8, 28672, 4096),
                                   (16, 8192, 28672), (1, 32768, 2048), (32, 20480, 8192),
                                   (8, 57344, 8192), (1, 40960, 28672), (1, 24608, 1024),
                                   (1, 16385, 896), (32, 57344, 4096)])
def test_plan_decode(M, N, K):
    """M <= 32 and K >= 512 within the measured limits (rounds of 256
    decode workgroups, K, M): the decode variant, for each of E2M1, E4M3
    and E5M2."""
    for fmt in (mxg.FMT_E2M1, mxg.FMT_E4M3, mxg.FMT_E5M2):
        p = mxg.plan(fmt, M, N, K)
        assert p["variant"] == mxg.VARIANT_DECODE, (fmt, p)
        assert (p["tile_m"], p["tile_n"]) == (mxg.DECODE_TILE, mxg.DECODE_TILE)
        assert p["split_k"] == 1 and p["workspace_bytes"] == 0 and p["threads"] == 256
        # at most one workgroup per CU, each taking every grid-th column group
        assert p["workgroups"] == min(-(-N // mxg.DECODE_TILE), 256)
    # FP6 has no decode kernel: the tiled one
    for fmt in (mxg.FMT_E2M3, mxg.FMT_E3M2):
        assert mxg.plan(fmt, M, N, K)["variant"] == mxg.VARIANT_TILE


@pytest.mark.parametrize("M,N,K", [(33, 8192, 28672), (8, 4096, 28672), (17, 8192, 28672),
                                   (1, 24577, 896), (8, 8192, 384), (32, 57344, 28672),
                                   (24, 12288, 14336), (1, 32768, 512), (1, 5088, 16384)])
def test_plan_decode_not_taken(M, N, K):
    """M > 32; K >= 16384 with fewer than 160 column groups (N <= 5088);
    more than 3 column groups per workgroup at K < 1024 (N > 24576); M > 16
    with K > 14336, or with more than one group per workgroup at
    K = 14336; K < 512: the tiled kernel."""
    assert mxg.plan(mxg.FMT_E4M3, M, N, K)["variant"] == mxg.VARIANT_TILE


def test_forced_decode_tile_errors():
    """The decode tile forced through mx_gemm_tile / mx_gemm_mixed /
    mx_gemm_bf16: refused (before any HIP call) for FP6, BF16, M > 32,
    K < 512 or a split; accepted otherwise (then stopped by a NULL pointer,
    or by the missing device)."""
    L = mxg.lib()
    good = 1 << 20
    D = mxg.DECODE_TILE
    for fmt in (mxg.FMT_E2M3, mxg.FMT_E3M2):
        assert L.mx_gemm_tile(fmt, 8, 64, 512, good, good, good, good, good, 2, D, D, 0,
                              None) == mxg.MX_ERR_SHAPE
    for M, K, split in ((33, 512, 0), (8, 384, 0), (8, 128, 1), (8, 512, 2)):
        assert L.mx_gemm_tile(2, M, 64, K, good, good, good, good, good, 2, D, D, split,
                              None) == mxg.MX_ERR_SHAPE, (M, K, split)
    for fa, fb in ((mxg.FMT_E4M3, mxg.FMT_E2M3), (mxg.FMT_E3M2, mxg.FMT_E2M1)):
        assert L.mx_gemm_mixed(fa, fb, 8, 64, 512, good, good, good, good, good, 2, D, D, 0,
                               None) == mxg.MX_ERR_SHAPE
    assert L.mx_gemm_bf16(8, 64, 512, good, good, good, 2, D, D, 0, None) == mxg.MX_ERR_SHAPE
    for fmt in (mxg.FMT_E2M1, mxg.FMT_E4M3, mxg.FMT_E5M2):
        for split in (0, 1):
            assert L.mx_gemm_tile(fmt, 32, 64, 512, None, good, good, good, good, 2, D, D,
                                  split, None) == mxg.MX_ERR_NULL
    for fa, fb in ((mxg.FMT_E4M3, mxg.FMT_E2M1), (mxg.FMT_E2M1, mxg.FMT_E5M2)):
        assert L.mx_gemm_mixed(fa, fb, 1, 1, 640, good, good, None, good, good, 2, D, D, 0,
                               None) == mxg.MX_ERR_NULL
    import torch
    if torch.cuda.device_count() == 0:
        assert L.mx_gemm_tile(2, 8, 64, 512, good, good, good, good, good, 2, D, D, 0,
                              None) == mxg.MX_ERR_NO_DEVICE


def test_plan_split_k():
    # Too few tiles for the GPU and a long K: K is split into whole 512-K
    # periods, a workspace of one FP32 plane per slice is reported.
    p = mxg.plan(mxg.FMT_E4M3, 256, 8192, 28672)
    assert p["variant"] == mxg.VARIANT_TILE and p["split_k"] > 1
    slice_k = -(-(-(-28672 // p["split_k"])) // 512) * 512
    assert -(-28672 // slice_k) == p["split_k"]
    tiles = -(-256 // p["tile_m"]) * -(-8192 // p["tile_n"])
    assert p["workgroups"] == tiles * p["split_k"] <= 256
    assert p["workspace_bytes"] >= p["split_k"] * 256 * 8192 * 4
    # Enough tiles, or a short K: no split, no workspace.
    for M, N, K in ((2048, 6144, 4096), (256, 8192, 2048)):
        p = mxg.plan(mxg.FMT_E4M3, M, N, K)
        assert p["split_k"] == 1 and p["workspace_bytes"] == 0


def test_plan_larger_m_uses_taller_tiles():
    for M in (65, 256, 2048):
        p = mxg.plan(mxg.FMT_E4M3, M, 8192, 4096)
        assert p["variant"] == mxg.VARIANT_TILE and p["tile_m"] >= 128


def test_python_shim_rejects_bad_tensors():
    import torch
    a = torch.zeros((16, 64), dtype=torch.uint8)
    s = torch.zeros((16, 4), dtype=torch.uint8)
    with pytest.raises(ValueError):
        mxg.mx_gemm(a, s, a, s, fmt=7)
    with pytest.raises(ValueError):          # not on the GPU
        mxg.mx_gemm(a, s, a, s, fmt=mxg.FMT_E2M1)
    with pytest.raises(ValueError):          # float32 is not a byte type
        mxg.mx_gemm(a.float(), s, a, s, fmt=mxg.FMT_E2M1)
    with pytest.raises(ValueError):          # non-contiguous
        mxg.mx_gemm(torch.zeros((16, 128), dtype=torch.uint8)[:, ::2], s, a, s,
                    fmt=mxg.FMT_E2M1)


@pytest.mark.parametrize("fmt,ind,rows,K,code", [
    (6, 1, 4, 64, mxg.MX_ERR_FORMAT),
    (1, 3, 4, 64, mxg.MX_ERR_IN_DTYPE),
    (2, 0, 4, 64, mxg.MX_ERR_IN_DTYPE),
    (1, 1, 0, 64, mxg.MX_ERR_SHAPE),
    (1, 1, 4, 0, mxg.MX_ERR_SHAPE),
    (2, 2, 4, 48, mxg.MX_ERR_SHAPE),
    (2, 2, 4, 16, mxg.MX_ERR_SHAPE),
    (2, 1, (1 << 30) + 1, 32, mxg.MX_ERR_SHAPE),
])
def test_quantize_argument_errors(fmt, ind, rows, K, code):
    good = 1 << 20            # never dereferenced: the checks fail first
    assert mxg.lib().mx_quantize(fmt, ind, rows, K, good, good, good, None) == code


def test_quantize_null_and_alignment_errors():
    L = mxg.lib()
    good = 1 << 20
    assert L.mx_quantize(1, 1, 4, 64, None, good, good, None) == mxg.MX_ERR_NULL
    assert L.mx_quantize(1, 1, 4, 64, good, good, None, None) == mxg.MX_ERR_NULL
    assert L.mx_quantize(1, 1, 4, 64, good + 8, good, good, None) == mxg.MX_ERR_ALIGN
    assert L.mx_quantize(2, 2, 4, 64, good, good + 4, good, None) == mxg.MX_ERR_ALIGN


def _grouped(fmt, rows, N, K, ptrs=(1 << 20,) * 5, out=2):
    arr = None if rows is None else (ctypes.c_int64 * max(len(rows), 1))(*rows)
    G = 1 if rows is None else len(rows)
    return mxg.lib().mx_gemm_grouped(fmt, G, arr, N, K, *ptrs, out, None)


@pytest.mark.parametrize("fmt,rows,N,K,out,code", [
    (0, [4], 16, 128, 2, mxg.MX_ERR_FORMAT),
    (2, [4], 16, 128, 5, mxg.MX_ERR_OUT_DTYPE),
    (2, [4], 0, 128, 2, mxg.MX_ERR_SHAPE),
    (2, [4], 16, 96, 2, mxg.MX_ERR_SHAPE),
    (2, [4, -1], 16, 128, 2, mxg.MX_ERR_SHAPE),
    (1, [4] * 257, 16, 128, 2, mxg.MX_ERR_SHAPE),
    (1, [1 << 29, 1 << 29, 1], 16, 128, 2, mxg.MX_ERR_SHAPE),   # rows above MX_MAX_DIM
    (1, [4, 4], 1 << 29 | 1, 128, 2, mxg.MX_ERR_SHAPE),         # G * N above MX_MAX_DIM
])
def test_grouped_argument_errors(fmt, rows, N, K, out, code):
    assert _grouped(fmt, rows, N, K, out=out) == code


def test_grouped_null_alignment_and_empty():
    L = mxg.lib()
    good = 1 << 20
    assert L.mx_gemm_grouped(2, 0, None, 16, 128, good, good, good, good, good, 2, None) \
        == mxg.MX_ERR_SHAPE
    assert _grouped(2, None, 16, 128) == mxg.MX_ERR_NULL
    for i in range(5):
        ptrs = [good] * 5
        ptrs[i] = None
        assert _grouped(2, [3, 0, 5], 16, 128, ptrs) == mxg.MX_ERR_NULL, i
    for i, mis in ((0, 8), (2, 4), (4, 2), (1, 2), (3, 1)):
        ptrs = [good] * 5
        ptrs[i] = good + mis
        assert _grouped(1, [3, 0, 5], 16, 128, ptrs) == mxg.MX_ERR_ALIGN, i
    # no rows at all: success without looking at a pointer or the device
    assert _grouped(1, [0, 0, 0], 16, 128, (None,) * 5) == mxg.MX_OK
    assert _grouped(2, [0] * mxg.MAX_GROUPS, 16, 128, (None,) * 5) == mxg.MX_OK


def test_grouped_no_device_reported():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible here")
    assert _grouped(2, [3, 0, 5], 16, 128) == mxg.MX_ERR_NO_DEVICE


def test_grouped_python_shim_checks():
    import torch
    a = torch.zeros((10, 64), dtype=torch.uint8)
    s = torch.zeros((10, 2), dtype=torch.uint8)
    b = torch.zeros((8, 64), dtype=torch.uint8)
    bs = torch.zeros((8, 2), dtype=torch.uint8)
    with pytest.raises(ValueError):          # group rows do not sum to a's rows
        mxg.mx_gemm_grouped(a, s, b, bs, [3, 3], fmt=mxg.FMT_E4M3)
    with pytest.raises(ValueError):          # b's rows not a multiple of the groups
        mxg.mx_gemm_grouped(a, s, b, bs, [3, 3, 4], fmt=mxg.FMT_E4M3)
    with pytest.raises(ValueError):          # negative count
        mxg.mx_gemm_grouped(a, s, b, bs, [12, -2], fmt=mxg.FMT_E4M3)
    with pytest.raises(ValueError):          # not on the GPU
        mxg.mx_gemm_grouped(a, s, b, bs, [6, 4], fmt=mxg.FMT_E4M3)


def test_grouped_plan():
    rows = [704, 320, 512, 896, 128, 640, 448, 448]
    p = mxg.grouped_plan(mxg.FMT_E4M3, rows, 4096, 2048)
    assert p["split_k"] == 1 and p["workspace_bytes"] == 0
    assert (p["tile_m"], p["tile_n"]) in mxg.tile_shapes() and p["tile_m"] == 256
    tiles = sum(-(-r // p["tile_m"]) for r in rows) * -(-4096 // p["tile_n"])
    assert p["workgroups"] == tiles
    # every group short: the 64-row tile; no rows: an empty grid
    p = mxg.grouped_plan(mxg.FMT_E2M1, [8, 1, 0, 33], 4096, 2048)
    assert (p["tile_m"], p["tile_n"]) == (64, 256) and p["workgroups"] == 3 * 16
    assert mxg.grouped_plan(mxg.FMT_E2M1, [0, 0], 64, 128)["workgroups"] == 0
    with pytest.raises(ValueError):
        mxg.grouped_plan(mxg.FMT_E2M1, [1] * (mxg.MAX_GROUPS + 1), 64, 128)
    arr = (ctypes.c_int64 * 1)(4)
    assert mxg.lib().mx_gemm_grouped_plan(1, 1, arr, 64, 128, 2, None) == mxg.MX_ERR_NULL


def test_mixed_argument_errors():
    L = mxg.lib()
    good = 1 << 20
    args = (good,) * 5
    # format of A, then of B; output type; shapes; tile and split
    assert L.mx_gemm_mixed(0, 1, 16, 16, 128, *args, 2, 0, 0, 0, None) == mxg.MX_ERR_FORMAT
    assert L.mx_gemm_mixed(2, 0, 16, 16, 128, *args, 2, 0, 0, 0, None) == mxg.MX_ERR_FORMAT
    assert L.mx_gemm_mixed(2, 1, 16, 16, 128, *args, 9, 0, 0, 0, None) == mxg.MX_ERR_OUT_DTYPE
    assert L.mx_gemm_mixed(2, 1, 16, 16, 96, *args, 2, 0, 0, 0, None) == mxg.MX_ERR_SHAPE
    assert L.mx_gemm_mixed(2, 1, 16, 16, 128, *args, 2, 100, 64, 0, None) == mxg.MX_ERR_SHAPE
    assert L.mx_gemm_mixed(2, 1, 16, 16, 128, *args, 2, 0, 0, -1, None) == mxg.MX_ERR_SHAPE
    assert L.mx_gemm_mixed(2, 1, 16, 16, 128, *args, 2, 0, 0, mxg.MAX_SPLIT_K + 1,
                           None) == mxg.MX_ERR_SHAPE
    assert L.mx_gemm_mixed(2, 1, 16, 16, 128, None, good, good, good, good, 2, 0, 0, 0,
                           None) == mxg.MX_ERR_NULL
    assert L.mx_gemm_mixed(1, 2, 16, 16, 128, good, good, good + 8, good, good, 2, 256, 192, 0,
                           None) == mxg.MX_ERR_ALIGN


def test_mixed_shim_checks_k_per_operand():
    import torch
    a8 = torch.zeros((16, 128), dtype=torch.uint8)     # E4M3: K = 128
    b4 = torch.zeros((8, 64), dtype=torch.uint8)       # E2M1: K = 128
    b4_bad = torch.zeros((8, 128), dtype=torch.uint8)  # E2M1: K = 256
    sa = torch.zeros((16, 4), dtype=torch.uint8)
    sb = torch.zeros((8, 4), dtype=torch.uint8)
    with pytest.raises(ValueError):                    # K mismatch
        mxg.mx_gemm(a8, sa, b4_bad, sb, fmt=mxg.FMT_E4M3, fmt_b=mxg.FMT_E2M1)
    with pytest.raises(ValueError):                    # shapes fine, but not on the GPU
        mxg.mx_gemm(a8, sa, b4, sb, fmt=mxg.FMT_E4M3, fmt_b=mxg.FMT_E2M1)
    with pytest.raises(ValueError):
        mxg.mx_gemm(a8, sa, b4, sb, fmt=mxg.FMT_E4M3, fmt_b=5)


def test_e5m2_accepted_where_documented():
    L = mxg.lib()
    good = 1 << 20
    args = (good,) * 5
    p = mxg.MxPlan()
    assert L.mx_gemm_plan(mxg.FMT_E5M2, 64, 64, 256, 2, ctypes.byref(p)) == mxg.MX_OK
    # E5M2 pairs with any format (only argument checks run here: no device)
    for fa, fb in ((3, 2), (2, 3), (3, 1), (1, 3)):
        assert L.mx_gemm_mixed(fa, fb, 16, 16, 128, *args, 2, 0, 0, 0, None) \
            == mxg.MX_ERR_NO_DEVICE, (fa, fb)
    assert L.mx_gemm_mixed(3, 6, 16, 16, 128, *args, 2, 0, 0, 0, None) == mxg.MX_ERR_FORMAT
    # the grouped GEMMs take every MX format and every pair of them
    for f in (3, 4, 5):
        assert _grouped(f, [4], 16, 128) == mxg.MX_ERR_NO_DEVICE, f
    arr = (ctypes.c_int64 * 2)(4, 0)
    for fa, fb in ((3, 2), (2, 3), (3, 1), (1, 3), (3, 3), (4, 2), (1, 5), (4, 5), (5, 4)):
        assert L.mx_gemm_grouped_mixed(fa, fb, 2, arr, 16, 128, *args, 2, None) \
            == mxg.MX_ERR_NO_DEVICE, (fa, fb)
    for fa, fb in ((3, 6), (0, 1), (6, 4)):
        assert L.mx_gemm_grouped_mixed(fa, fb, 2, arr, 16, 128, *args, 2, None) \
            == mxg.MX_ERR_FORMAT, (fa, fb)
    # the quantizer takes E5M2 too
    assert L.mx_quantize(3, 1, 4, 64, good, good, good, None) == mxg.MX_ERR_NO_DEVICE \
        or __import__("torch").cuda.device_count() > 0
    assert L.mx_quantize(6, 1, 4, 64, good, good, good, None) == mxg.MX_ERR_FORMAT


def test_bf16_argument_errors():
    L = mxg.lib()
    good = 1 << 20
    p = mxg.MxPlan()
    # output type; K from one 16-K step up, a multiple of 16, at most MAX_K_BF16
    assert L.mx_gemm_bf16(16, 16, 64, good, good, good, 0, 0, 0, 0, None) == mxg.MX_ERR_OUT_DTYPE
    for M, N, K in ((0, 16, 64), (16, 0, 64), (16, 16, 0), (16, 16, 8), (16, 16, 40),
                    (mxg.MAX_DIM + 1, 16, 64), (16, 16, mxg.MAX_K_BF16 + 16)):
        assert L.mx_gemm_bf16(M, N, K, good, good, good, 2, 0, 0, 0, None) == mxg.MX_ERR_SHAPE
        assert L.mx_gemm_bf16_plan(M, N, K, 2, ctypes.byref(p)) == mxg.MX_ERR_SHAPE
    assert L.mx_gemm_bf16_plan(16, 16, mxg.MAX_K_BF16, 2, ctypes.byref(p)) == mxg.MX_OK
    # forced tile and split
    assert L.mx_gemm_bf16(16, 16, 64, good, good, good, 2, 100, 64, 0, None) == mxg.MX_ERR_SHAPE
    assert L.mx_gemm_bf16(16, 16, 64, good, good, good, 2, 0, 0, -1, None) == mxg.MX_ERR_SHAPE
    assert L.mx_gemm_bf16(16, 16, 64, good, good, good, 2, 0, 0, mxg.MAX_SPLIT_K + 1,
                          None) == mxg.MX_ERR_SHAPE
    # pointers: no scales to pass; A, B and C must be non-null and 16-byte aligned
    assert L.mx_gemm_bf16(16, 16, 64, None, good, good, 2, 0, 0, 0, None) == mxg.MX_ERR_NULL
    assert L.mx_gemm_bf16(16, 16, 64, good, good, None, 2, 0, 0, 0, None) == mxg.MX_ERR_NULL
    assert L.mx_gemm_bf16(16, 16, 64, good, good + 8, good, 2, 0, 0, 0, None) == mxg.MX_ERR_ALIGN
    assert L.mx_gemm_bf16(16, 16, 64, good, good, good + 4, 2, 256, 128, 2,
                          None) == mxg.MX_ERR_ALIGN
    assert L.mx_gemm_bf16_plan(16, 16, 64, 2, None) == mxg.MX_ERR_NULL


def test_bf16_plan_matches_mx_plan():
    """The BF16 GEMM runs on the tile kernels with the MX GEMM's tile and
    split choice (both depend on M, N and K only), as the FP6 formats do;
    where the MX plan takes the decode kernel, which has no BF16 form, BF16
    stays on the tiled kernel."""
    for M, N, K in ((2048, 6144, 4096), (8, 8192, 28672), (256, 28672, 4096),
                    (2048, 5120, 25600), (1, 1, 128)):
        assert mxg.plan_bf16(M, N, K) == mxg.plan(mxg.FMT_E2M3, M, N, K)
    assert mxg.plan(mxg.FMT_E4M3, 8, 8192, 28672)["variant"] == mxg.VARIANT_DECODE
    assert mxg.plan_bf16(8, 8192, 28672)["variant"] == mxg.VARIANT_TILE
    p = mxg.plan_bf16(5, 7, 48)
    assert p["split_k"] == 1 and p["workgroups"] >= 1


def test_bf16_shim_checks():
    import torch
    a = torch.zeros((16, 64), dtype=torch.bfloat16)
    b = torch.zeros((8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):                    # K mismatch
        mxg.mx_gemm_bf16(a, torch.zeros((8, 32), dtype=torch.bfloat16))
    with pytest.raises(ValueError):                    # wrong element type
        mxg.mx_gemm_bf16(a.float(), b)
    with pytest.raises(ValueError):                    # not contiguous
        mxg.mx_gemm_bf16(torch.zeros((64, 16), dtype=torch.bfloat16).t(), b)
    with pytest.raises(ValueError):                    # shapes fine, but not on the GPU
        mxg.mx_gemm_bf16(a, b)


def test_bf16_no_device_reported():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible here")
    good = 1 << 20
    rc = mxg.lib().mx_gemm_bf16(16, 16, 64, good, good, good, 2, 0, 0, 0, None)
    assert rc == mxg.MX_ERR_NO_DEVICE


def _grouped_bf16(rows, N, K, ptrs=(1 << 20,) * 3, out=2):
    arr = (ctypes.c_int64 * max(len(rows), 1))(*rows)
    return mxg.lib().mx_gemm_grouped_bf16(len(rows), arr, N, K, *ptrs, out, None)


def test_grouped_bf16_argument_errors():
    good = 1 << 20
    assert _grouped_bf16([4], 16, 64, out=7) == mxg.MX_ERR_OUT_DTYPE
    for rows, N, K in (([4], 16, 40), ([4], 16, 0), ([4], 0, 64), ([-1], 16, 64),
                       ([1] * (mxg.MAX_GROUPS + 1), 16, 64), ([4], 16, mxg.MAX_K_BF16 + 16)):
        assert _grouped_bf16(rows, N, K) == mxg.MX_ERR_SHAPE, (rows, N, K)
    assert _grouped_bf16([4], 16, 64, ptrs=(None, good, good)) == mxg.MX_ERR_NULL
    assert _grouped_bf16([4], 16, 64, ptrs=(good, good + 8, good)) == mxg.MX_ERR_ALIGN
    assert _grouped_bf16([0, 0], 16, 64, ptrs=(None, None, None)) == mxg.MX_OK   # no rows
    # the MX entry points do not take the BF16 marker as a format
    arr = (ctypes.c_int64 * 1)(4)
    p = mxg.MxPlan()
    assert mxg.lib().mx_gemm_grouped_plan(0x100, 1, arr, 16, 128, 2, ctypes.byref(p)) \
        == mxg.MX_ERR_FORMAT
    assert _grouped(0x100, [4], 16, 128) == mxg.MX_ERR_FORMAT


def test_grouped_bf16_plan_matches_mx_plan():
    """The grouped BF16 GEMM picks its tile like the MX grouped GEMM."""
    for rows, N, K in (([704, 320, 512, 896, 128, 640, 448, 448], 4096, 2048),
                       ([8, 1, 0, 33], 4096, 2048), ([0, 0], 64, 128)):
        assert mxg.grouped_bf16_plan(rows, N, K) == mxg.grouped_plan(mxg.FMT_E4M3, rows, N, K)
    assert mxg.grouped_bf16_plan([5, 3], 64, 48)["workgroups"] >= 2


def test_grouped_mixed_argument_errors():
    good = 1 << 20
    arr = (ctypes.c_int64 * 2)(4, 3)
    L = mxg.lib()
    call = lambda fa, fb, K=128, ptrs=(good,) * 5: L.mx_gemm_grouped_mixed(
        fa, fb, 2, arr, 16, K, *ptrs, 2, None)
    for fa, fb in ((2, 6), (6, 1), (0, 1), (2, 9), (0x100, 0x100)):
        assert call(fa, fb) == mxg.MX_ERR_FORMAT, (fa, fb)
    assert call(2, 1, K=96) == mxg.MX_ERR_SHAPE
    assert call(2, 1, ptrs=(good, None, good, good, good)) == mxg.MX_ERR_NULL
    assert call(1, 2, ptrs=(good, good, good + 8, good, good)) == mxg.MX_ERR_ALIGN
    assert call(2, 1) == mxg.MX_ERR_NO_DEVICE or __import__("torch").cuda.device_count() > 0


def test_fp6_accepted_where_documented():
    L = mxg.lib()
    good = 1 << 20
    args = (good,) * 5
    p = mxg.MxPlan()
    for f in (mxg.FMT_E2M3, mxg.FMT_E3M2):
        assert L.mx_gemm_plan(f, 64, 64, 256, 2, ctypes.byref(p)) == mxg.MX_OK
        # FP6 pairs with every MX format (argument checks pass: no device here)
        for g in (1, 2, 3, 4, 5):
            assert L.mx_gemm_mixed(f, g, 16, 16, 128, *args, 2, 0, 0, 0, None) \
                == mxg.MX_ERR_NO_DEVICE, (f, g)
            assert L.mx_gemm_mixed(g, f, 16, 16, 128, *args, 2, 0, 0, 0, None) \
                == mxg.MX_ERR_NO_DEVICE, (g, f)
        for g in (0, 6):
            assert L.mx_gemm_mixed(f, g, 16, 16, 128, *args, 2, 0, 0, 0, None) == mxg.MX_ERR_FORMAT
        # in the grouped GEMM and the quantizer (argument checks pass: no device here)
        assert _grouped(f, [4], 16, 128) == mxg.MX_ERR_NO_DEVICE
        assert L.mx_quantize(f, 1, 4, 64, good, good, good, None) == mxg.MX_ERR_NO_DEVICE
    # the shim derives K from 3K/4-byte rows
    import torch
    a = torch.zeros((4, 96), dtype=torch.uint8)
    s = torch.zeros((4, 4), dtype=torch.uint8)
    with pytest.raises(ValueError):          # shapes fine (K = 128), but not on the GPU
        mxg.mx_gemm(a, s, a, s, mxg.FMT_E2M3)
    with pytest.raises(ValueError):          # K mismatch against a 128-byte E4M3 row
        mxg.mx_gemm(a, s, torch.zeros((4, 128), dtype=torch.uint8), s, mxg.FMT_E2M3,
                    fmt_b=mxg.FMT_E4M3)


@pytest.mark.parametrize("fmt,M,N,K,out,code", [
    (0, 16, 16, 128, 1, mxg.MX_ERR_FORMAT),
    (1, 16, 16, 128, 0, mxg.MX_ERR_OUT_DTYPE),
    (1, 16, 16, 64, 1, mxg.MX_ERR_SHAPE),
    (2, 16, 16, (1 << 24) + 128, 2, mxg.MX_ERR_SHAPE),
])
def test_noalloc_argument_errors(fmt, M, N, K, out, code):
    """mx_gemm_noalloc checks its arguments as mx_gemm does, before any HIP call."""
    L = mxg.lib()
    assert L.mx_gemm_noalloc(fmt, M, N, K, None, None, None, None, None, out, None) == code


def test_noalloc_rejects_workspace_beyond_scratch():
    """A problem whose split-K planes exceed the fixed scratch is refused with
    MX_ERR_SCRATCH before any HIP call (the pointers are never touched: any
    16-byte aligned values will do); one that fits, or needs no split, is
    not refused for its size."""
    L = mxg.lib()
    big = (2, 512, 6144, 28672)             # 256x192 tiles, split 4: 4 planes of 12 MiB
    p = mxg.plan(*big, out_dtype=2)
    assert p["workspace_bytes"] > mxg.NOALLOC_SCRATCH_BYTES, p
    fake = 1 << 20
    assert L.mx_gemm_noalloc(big[0], big[1], big[2], big[3], fake, fake, fake, fake, fake, 2,
                             None) == mxg.MX_ERR_SCRATCH
    fits = mxg.plan(2, 256, 8192, 28672, out_dtype=2)
    assert 0 < fits["workspace_bytes"] <= mxg.NOALLOC_SCRATCH_BYTES, fits
    assert "scratch" in mxg.strerror(mxg.MX_ERR_SCRATCH)


def test_operand_row_length_must_hold_whole_elements():
    """K is inferred from an operand's row length: an FP6 row must be exactly
    3*K/4 bytes (97 bytes is refused, not read as K = 128)."""
    assert mxg._k_of(mxg.FMT_E2M3, 96) == 128
    assert mxg._k_of(mxg.FMT_E3M2, 3 * 1024 // 4) == 1024
    assert mxg._k_of(mxg.FMT_E2M1, 64) == 128 and mxg._k_of(mxg.FMT_E4M3, 128) == 128
    for fmt in (mxg.FMT_E2M3, mxg.FMT_E3M2):
        for rb in (97, 98, 1):
            with pytest.raises(ValueError):
                mxg._k_of(fmt, rb)


def test_hbm_read_ceiling_argument_errors():
    """mx_hbm_read_ceiling checks its arguments before any HIP call."""
    L = mxg.lib()
    fake = 1 << 20
    assert L.mx_hbm_read_ceiling(None, 1024, fake, None) == mxg.MX_ERR_NULL
    assert L.mx_hbm_read_ceiling(fake, 1024, None, None) == mxg.MX_ERR_NULL
    for nbytes in (-16, 0, 8, 1000):
        assert L.mx_hbm_read_ceiling(fake, nbytes, fake, None) == mxg.MX_ERR_SHAPE
    assert L.mx_hbm_read_ceiling(fake + 8, 1024, fake, None) == mxg.MX_ERR_ALIGN
    assert L.mx_hbm_read_ceiling(fake, 1024, fake + 2, None) == mxg.MX_ERR_ALIGN
