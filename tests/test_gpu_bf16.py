"""GPU parity of the dense BF16 NT GEMM (mx_gemm_bf16) against the oracle
through the C ABI: ragged shapes, every tile with and without a K split,
small M, exact integer results, BF16 output as the rounding of FP32 output,
and a full-size shape on sampled rows.

Acceptance is the MX GEMM's: |gpu - C| <= 1e-5 * T, plus one BF16 ulp of C
for BF16 output, with T = sum_k |a_k * b_k|.  Products of two BF16 values are
exact in FP32; the only error is the FP32 accumulation."""
import numpy as np
import pytest

import microscaled_block_scaled_amd as mxg
import mxinputs
import oracle
from gpu_util import acceptance, host64, log, sample_rows

pytestmark = pytest.mark.gpu

F32, BF16 = mxinputs.OUT_FP32, mxinputs.OUT_BF16


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def _run(A, B, out, tile=None, split_k=0, dA=None, dB=None):
    import torch
    tdt = torch.float32 if out == F32 else torch.bfloat16
    dA = _dev(A) if dA is None else dA
    dB = _dev(B) if dB is None else dB
    C = mxg.mx_gemm_bf16(dA, dB, out_dtype=tdt, tile=tile, split_k=split_k)
    torch.cuda.synchronize()
    return C


def _check(A, B, out, C, rows=None, what=""):
    Cref, T = oracle.gemm_bf16(A, B, rows=rows)
    g = host64(C)
    if rows is not None:
        g = g[np.asarray(rows)]
    r = acceptance(g, Cref, T, out == BF16, what=what)
    assert r["n_bad"] == 0, "%s: %d bad, worst ratio %.3g at %s" % (
        what, r["n_bad"], r["max_ratio"], r["first_bad"])


def _case(M, N, K, seed):
    return (mxinputs.make_bf16(M, K, seed=seed, tensor=0),
            mxinputs.make_bf16(N, K, seed=seed, tensor=1))


# K from one instruction step (16) through partial 64-K slabs to several
# main-loop trips with a partial last slab.
TAIL_SHAPES = [(1, 1, 16), (7, 33, 48), (33, 255, 80), (255, 257, 208),
               (257, 129, 512), (130, 7, 640), (64, 300, 1168)]


@pytest.mark.parametrize("out", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", TAIL_SHAPES)
def test_bf16_tails(out, M, N, K):
    log("bf16 tails out=%d M=%d N=%d K=%d plan=%s" % (out, M, N, K, mxg.plan_bf16(M, N, K)))
    A, B = _case(M, N, K, seed=M * 3 + N + K)
    _check(A, B, out, _run(A, B, out), what="tails")


def _tile_ids():
    return ["%dx%d" % t for t in mxg.tile_shapes()]


@pytest.mark.parametrize("split", [1, 3], ids=["nosplit", "split3"])
@pytest.mark.parametrize("tile", mxg.tile_shapes(), ids=_tile_ids())
def test_bf16_every_tile(tile, split):
    bm, bn = tile
    M, N, K = 2 * bm + 19, 2 * bn + 24, 3584 + 48
    log("bf16 tile %dx%d split %d" % (bm, bn, split))
    A, B = _case(M, N, K, seed=bm + bn + split)
    for out in (F32, BF16):
        C = _run(A, B, out, tile=tile, split_k=split)
        _check(A, B, out, C, rows=sample_rows(M, tile=bm), what="tile")


@pytest.mark.parametrize("M,N,K", [(1, 1000, 8192), (8, 8192, 4096), (64, 2048, 2048),
                                   (100, 4000, 1040)])
def test_bf16_small_m(M, N, K):
    log("bf16 small M M=%d N=%d K=%d plan=%s" % (M, N, K, mxg.plan_bf16(M, N, K)))
    A, B = _case(M, N, K, seed=M + N)
    _check(A, B, BF16, _run(A, B, BF16), what="small M")


def test_bf16_exact_integers():
    """Small integer values: every product and partial sum is an integer
    below 2^24, so FP32 accumulation is exact in any order and the GPU must
    equal numpy's int64 matmul bit for bit, with and without a K split."""
    import torch
    rng = np.random.default_rng(5)
    M, N, K = 200, 300, 2048
    ia = rng.integers(-4, 5, (M, K))
    ib = rng.integers(-4, 5, (N, K))

    def bits(x):
        return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16) \
            .numpy().view(np.uint16)

    A, B = bits(ia), bits(ib)
    want = (ia @ ib.T).astype(np.float64)
    for split in (0, 4):
        g = host64(_run(A, B, F32, tile=(256, 128) if split else None, split_k=split))
        log("bf16 exact integers split %d: max |diff| %g" % (split, np.max(np.abs(g - want))))
        assert np.array_equal(g, want)


def test_bf16_output_is_rounded_fp32():
    """With the same plan, BF16 output is the round-to-nearest-even of the
    FP32 output (checked with torch's conversion), bit for bit."""
    import torch
    A, B = _case(300, 520, 1024, seed=9)
    dA, dB = _dev(A), _dev(B)
    for split in (0, 2):
        tile = (256, 128) if split else None
        c32 = _run(A, B, F32, tile=tile, split_k=split, dA=dA, dB=dB)
        c16 = _run(A, B, BF16, tile=tile, split_k=split, dA=dA, dB=dB)
        assert torch.equal(c32.to(torch.bfloat16).view(torch.int16), c16.view(torch.int16))


def test_bf16_zero_and_one_hot():
    """All-zero operands give exact zeros; one non-zero pair gives exactly
    its product at its (row, column) and zero elsewhere."""
    M, N, K = 70, 90, 256
    A = np.zeros((M, K), np.uint16)
    B = np.zeros((N, K), np.uint16)
    assert not host64(_run(A, B, F32)).any()
    A[13, 200] = 0x4040                  # 3.0
    B[77, 200] = 0xC0A0                  # -5.0
    g = host64(_run(A, B, F32))
    want = np.zeros((M, N))
    want[13, 77] = -15.0
    assert np.array_equal(g, want)


def test_bf16_full_size():
    """The fused-QKV projection shape (2048 x 6144 x 4096) in the plan's
    configuration, sampled rows; a rerun is bit for bit the same."""
    import torch
    M, N, K = 2048, 6144, 4096
    log("bf16 full size plan=%s" % mxg.plan_bf16(M, N, K))
    A, B = _case(M, N, K, seed=12)
    dA, dB = _dev(A), _dev(B)
    C = _run(A, B, BF16, dA=dA, dB=dB)
    assert torch.equal(C, _run(A, B, BF16, dA=dA, dB=dB))
    _check(A, B, BF16, C, rows=sample_rows(M, n=24), what="full size")


@pytest.mark.parametrize("M,N,K", [(2048, 8192, 28672), (8, 8192, 28672)],
                         ids=["llama70b_down_m2048", "llama70b_down_m8"])
def test_bf16_bench_workloads(M, N, K):
    """The 70B down-projection shapes bench.py times, in the plan's
    configuration (256x256 tiles; 128x128 with a 4-way K split at M = 8),
    checked on sampled rows."""
    log("bf16 bench workload M=%d N=%d K=%d plan=%s" % (M, N, K, mxg.plan_bf16(M, N, K)))
    A, B = _case(M, N, K, seed=40 + M)
    C = _run(A, B, BF16)
    _check(A, B, BF16, C, rows=sample_rows(M, n=32), what="bench workload")
