"""GPU parity of E5M2 MX GEMMs (both operands E5M2, the wider-range MXFP8
encoding) against the oracle through the C ABI: ragged shapes, every tile
with and without a K split, small M, a full-size shape on sampled rows, and
where infinities and NaNs land.

Acceptance as for E4M3: |gpu - C| <= 1e-5 * T (+ one bf16 ulp of C for BF16
output) + E, the oracle's 8-product group-alignment term; the log says how
many elements need E."""
import numpy as np
import pytest

import microscaled_block_scaled_amd as mxg
import mxinputs
import oracle
from gpu_util import acceptance, host64, log, sample_rows

pytestmark = pytest.mark.gpu

E5M2 = mxinputs.FMT_E5M2
F32, BF16 = mxinputs.OUT_FP32, mxinputs.OUT_BF16


def _run(case, out, tile=None, split_k=0):
    import torch
    d = [torch.from_numpy(np.ascontiguousarray(case[k])).cuda()
         for k in ("A", "A_scale", "B", "B_scale")]
    tdt = torch.float32 if out == F32 else torch.bfloat16
    C = mxg.mx_gemm(d[0], d[1], d[2], d[3], E5M2, out_dtype=tdt, tile=tile, split_k=split_k)
    torch.cuda.synchronize()
    return C


def _check(case, out, C, rows=None, what="", group_term=False):
    Cref, T, E = oracle.gemm(E5M2, case["A"], case["A_scale"], case["B"], case["B_scale"],
                             case["K"], rows=rows, group_bound=True)
    g = host64(C)
    if rows is not None:
        g = g[np.asarray(rows)]
    r = acceptance(g, Cref, T, out == BF16, E, group_term, what)
    assert r["n_bad"] == 0, "%s: %d bad, worst ratio %.3g at %s" % (
        what, r["n_bad"], r["max_ratio"], r["first_bad"])


TAIL_SHAPES = [(1, 1, 128), (7, 33, 256), (33, 255, 128), (255, 257, 384),
               (257, 129, 512), (130, 7, 640), (64, 300, 1152)]


@pytest.mark.parametrize("out", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", TAIL_SHAPES)
def test_e5m2_tails(out, M, N, K):
    log("e5m2 tails out=%d M=%d N=%d K=%d" % (out, M, N, K))
    case = mxinputs.make_random(E5M2, M, N, K, seed=M * 3 + N + K)
    _check(case, out, _run(case, out), what="tails")


def _tile_ids():
    return ["%dx%d" % t for t in mxg.tile_shapes()]


@pytest.mark.parametrize("split", [1, 3], ids=["nosplit", "split3"])
@pytest.mark.parametrize("tile", mxg.tile_shapes(), ids=_tile_ids())
def test_e5m2_every_tile(tile, split):
    bm, bn = tile
    M, N, K = 2 * bm + 19, 2 * bn + 24, 3584
    log("e5m2 tile %dx%d split %d" % (bm, bn, split))
    case = mxinputs.make_random(E5M2, M, N, K, seed=bm + bn + split)
    C = _run(case, BF16, tile=tile, split_k=split)
    _check(case, BF16, C, rows=sample_rows(M, tile=bm), what="tile")


def test_e5m2_wide_scales():
    """Scale bytes drawn over a wide range, so blocks of very different
    magnitude meet in one sum.  One block then dominates most outputs, so
    the error of its groups of 8 is not averaged over many blocks: the bound
    adds the oracle's group term (deliberately wide-range input)."""
    case = mxinputs.make_random(E5M2, 96, 80, 1024, seed=8, scale_lo=90, scale_hi=160)
    log("e5m2 wide scales")
    for out in (F32, BF16):
        _check(case, out, _run(case, out), what="wide scales", group_term=True)


@pytest.mark.parametrize("M,N,K", [(1, 1000, 8192), (8, 8192, 4096)])
def test_e5m2_small_m(M, N, K):
    log("e5m2 small M M=%d N=%d K=%d plan=%s" % (M, N, K, mxg.plan(E5M2, M, N, K)))
    case = mxinputs.make_random(E5M2, M, N, K, seed=M + N)
    _check(case, BF16, _run(case, BF16), what="small M")


def test_e5m2_full_size():
    """The fused-QKV projection shape in the plan's configuration, sampled
    rows; a rerun is bit for bit the same."""
    import torch
    M, N, K = 2048, 6144, 4096
    log("e5m2 full size")
    case = mxinputs.make_random(E5M2, M, N, K, seed=12)
    C = _run(case, BF16)
    assert torch.equal(C, _run(case, BF16))
    _check(case, BF16, C, rows=sample_rows(M, n=24), what="full size")


def test_e5m2_infinities_and_nans():
    """E5M2 has infinities and NaNs.  An infinity times a non-zero value
    makes its output row infinite, an infinity times zero or a NaN makes
    NaN; the GPU's pattern of infinite and NaN outputs is the oracle's."""
    K = 128
    case = mxinputs.make_random(E5M2, 4, 6, K, seed=3)
    A, B = case["A"].copy(), case["B"].copy()
    A[0, 5] = 0x7C                       # +inf in row 0
    A[1, 40] = 0x7F                      # NaN in row 1
    B[2, 70] = 0xFC                      # -inf in B row 2
    A[3, 70] = 0x00                      # ... times zero in A row 3: NaN at (3, 2)
    case = dict(case, A=A, B=B)
    C = host64(_run(case, F32))
    Cref, _ = oracle.gemm(E5M2, A, case["A_scale"], B, case["B_scale"], K)
    log("e5m2 specials: gpu inf %s nan %s / oracle inf %s nan %s" % (
        np.isinf(C).sum(), np.isnan(C).sum(), np.isinf(Cref).sum(), np.isnan(Cref).sum()))
    assert np.array_equal(np.isnan(C), np.isnan(Cref))
    assert np.array_equal(np.isinf(C), np.isinf(Cref))
    fin = np.isfinite(Cref)
    assert np.array_equal(np.sign(C[np.isinf(C)]), np.sign(Cref[np.isinf(Cref)]))
    assert np.all(np.abs(C[fin] - Cref[fin]) <= 1e-4 * np.abs(Cref[fin]) + 1e-30)
