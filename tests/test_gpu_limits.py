"""GPU parity at the size limits of the C ABI: the largest K (MX_MAX_K = 2^24)
with 256-row tiles, where a lane's 32-bit copy offset (row within the tile
times the row pitch) comes within 2^24 of 2^32, for MXFP8 (K bytes per row)
and MXFP4; the same K on the decode kernel; and the largest dense-BF16 K
(2^23, 2K bytes per row).  Checked on sampled rows against the oracle."""
import numpy as np
import pytest

import microscaled_block_scaled_amd as mxg
import mxinputs
import oracle
from gpu_util import acceptance, host64, log

pytestmark = pytest.mark.gpu

E2M1, E4M3 = mxinputs.FMT_E2M1, mxinputs.FMT_E4M3
F32 = mxinputs.OUT_FP32


def _codes(rng, fmt, rows, K):
    if fmt == E2M1:
        return rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    c = rng.integers(0, 256, size=(rows, K), dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0                  # no E4M3 NaN codes
    return c


@pytest.mark.parametrize("fmt", [E4M3, E2M1], ids=["e4m3", "e2m1"])
def test_largest_k(fmt):
    import torch
    M, N, K = 260, 40, mxg.MAX_K
    p = mxg.plan(fmt, M, N, K, F32)
    log("largest K fmt=%d M=%d N=%d K=%d plan=%s" % (fmt, M, N, K, p))
    assert p["tile_m"] == 256
    rng = np.random.default_rng(2024 + fmt)
    A, B = _codes(rng, fmt, M, K), _codes(rng, fmt, N, K)
    As = rng.integers(120, 135, size=(M, K // 32), dtype=np.uint8)
    Bs = rng.integers(120, 135, size=(N, K // 32), dtype=np.uint8)
    d = [torch.from_numpy(x).cuda() for x in (A, As, B, Bs)]
    C = mxg.mx_gemm(d[0], d[1], d[2], d[3], fmt, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = [0, 1, 130, 255, 256, 259]
    Cref, T, E = oracle.gemm(fmt, A, As, B, Bs, K, rows=rows, group_bound=True)
    r = acceptance(host64(C)[rows], Cref, T, False, E, what="largest K")
    assert r["n_bad"] == 0, r


def test_largest_k_bf16():
    import torch
    M, N, K = 260, 24, mxg.MAX_K_BF16
    p = mxg.plan_bf16(M, N, K, F32)
    log("largest BF16 K M=%d N=%d K=%d plan=%s" % (M, N, K, p))
    rng = np.random.default_rng(7)
    # small integer values: every product and partial sum is exact in FP32
    ia = rng.integers(-2, 3, size=(M, K), dtype=np.int8)
    ib = rng.integers(-2, 3, size=(N, K), dtype=np.int8)
    A = torch.from_numpy(ia).cuda().to(torch.bfloat16)
    B = torch.from_numpy(ib).cuda().to(torch.bfloat16)
    C = mxg.mx_gemm_bf16(A, B, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = [0, 1, 255, 256, 259]
    want = (ia[rows].astype(np.int64) @ ib.astype(np.int64).T).astype(np.float64)
    got = host64(C)[rows]
    log("  max |diff| %g" % np.max(np.abs(got - want)))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt", [E4M3, E2M1], ids=["e4m3", "e2m1"])
def test_largest_k_decode(fmt):
    """The decode kernel (forced tile 32 x 32) at the largest K: 32 rows of
    A, so its copy extents reach 32 rows of 2^24 (E4M3) bytes, each wave's
    K-range is 2^22 values long, and N = 40 gives a ragged second column
    group; sampled rows against the oracle."""
    import torch
    M, N, K = 32, 40, mxg.MAX_K
    log("largest K decode fmt=%d M=%d N=%d K=%d" % (fmt, M, N, K))
    rng = np.random.default_rng(4048 + fmt)
    A, B = _codes(rng, fmt, M, K), _codes(rng, fmt, N, K)
    As = rng.integers(120, 135, size=(M, K // 32), dtype=np.uint8)
    Bs = rng.integers(120, 135, size=(N, K // 32), dtype=np.uint8)
    d = [torch.from_numpy(x).cuda() for x in (A, As, B, Bs)]
    C = mxg.mx_gemm(d[0], d[1], d[2], d[3], fmt, out_dtype=torch.float32,
                    tile=(mxg.DECODE_TILE, mxg.DECODE_TILE))
    torch.cuda.synchronize()
    rows = [0, 17, 31]
    Cref, T, E = oracle.gemm(fmt, A, As, B, Bs, K, rows=rows, group_bound=True)
    r = acceptance(host64(C)[rows], Cref, T, False, E, what="largest K decode")
    assert r["n_bad"] == 0, r
