"""GPU parity of FP6 MX GEMMs (E2M3 and E3M2 elements, both operands in one
format, packed four per three bytes) against the oracle through the C ABI:
ragged shapes, every tile with and without a K split, small M, a full-size
shape on sampled rows, exact integer results and wide scales.

Acceptance as for the other MX formats: |gpu - C| <= 1e-5 * T (+ one bf16
ulp of C for BF16 output) + E, the oracle's 8-product group-alignment term
(E3M2 products span enough binades for the hardware's alignment to round)."""
import numpy as np
import pytest

import microscaled_block_scaled_amd as mxg
import mxinputs
import oracle
from gpu_util import acceptance, host64, log, sample_rows

pytestmark = pytest.mark.gpu

E2M3, E3M2 = mxinputs.FMT_E2M3, mxinputs.FMT_E3M2
F32, BF16 = mxinputs.OUT_FP32, mxinputs.OUT_BF16
FMTS, IDS = [E2M3, E3M2], ["e2m3", "e3m2"]


def _run(case, out, tile=None, split_k=0):
    import torch
    d = [torch.from_numpy(np.ascontiguousarray(case[k])).cuda()
         for k in ("A", "A_scale", "B", "B_scale")]
    tdt = torch.float32 if out == F32 else torch.bfloat16
    C = mxg.mx_gemm(d[0], d[1], d[2], d[3], case["fmt"], out_dtype=tdt, tile=tile,
                    split_k=split_k)
    torch.cuda.synchronize()
    return C


def _check(case, out, C, rows=None, what="", group_term=False):
    Cref, T, E = oracle.gemm(case["fmt"], case["A"], case["A_scale"], case["B"],
                             case["B_scale"], case["K"], rows=rows, group_bound=True)
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
@pytest.mark.parametrize("fmt", FMTS, ids=IDS)
def test_fp6_tails(fmt, M, N, K, out):
    log("fp6 fmt=%d out=%d M=%d N=%d K=%d" % (fmt, out, M, N, K))
    case = mxinputs.make_random(fmt, M, N, K, seed=M * 3 + N + K + fmt)
    _check(case, out, _run(case, out), what="tails")


@pytest.mark.parametrize("split", [1, 3], ids=["nosplit", "split3"])
@pytest.mark.parametrize("tile", mxg.tile_shapes(), ids=["%dx%d" % t for t in mxg.tile_shapes()])
@pytest.mark.parametrize("fmt", FMTS, ids=IDS)
def test_fp6_every_tile(fmt, tile, split):
    bm, bn = tile
    M, N, K = 2 * bm + 19, 2 * bn + 24, 3584
    log("fp6 fmt=%d tile %dx%d split %d" % (fmt, bm, bn, split))
    case = mxinputs.make_random(fmt, M, N, K, seed=bm + bn + split + fmt)
    C = _run(case, BF16, tile=tile, split_k=split)
    _check(case, BF16, C, rows=sample_rows(M, tile=bm), what="tile")


@pytest.mark.parametrize("fmt", FMTS, ids=IDS)
def test_fp6_small_m_full_size_and_scales(fmt):
    """8 rows in the split-K plan; the fused-QKV shape on sampled rows,
    bit-identical on a rerun; scale bytes drawn over a wide range."""
    import torch
    case = mxinputs.make_random(fmt, 8, 8192, 4096, seed=70 + fmt)
    _check(case, BF16, _run(case, BF16), what="small M")
    case = mxinputs.make_random(fmt, 2048, 6144, 4096, seed=80 + fmt)
    C = _run(case, BF16)
    assert torch.equal(C, _run(case, BF16))
    _check(case, BF16, C, rows=sample_rows(2048, n=32), what="full size")
    # deliberately wide-range scales: one block dominates most outputs, so
    # the bound adds the oracle's group term
    case = mxinputs.make_random(fmt, 96, 80, 1024, seed=8, scale_lo=90, scale_hi=160)
    for out in (F32, BF16):
        _check(case, out, _run(case, out), what="wide scales", group_term=True)


@pytest.mark.parametrize("fmt", FMTS, ids=IDS)
def test_fp6_exact_integers(fmt):
    """Integer-valued FP6 codes with every scale 127: each block sum is an
    integer, so the GPU must equal an int64 matmul bit for bit."""
    g = np.array([oracle.default().gemm(fmt, mxinputs.pack_fp6(np.array([[c] + [0] * 31])),
                                        np.full((1, 1), 127, np.uint8),
                                        mxinputs.pack_fp6(np.array([[8 if fmt == E2M3 else 12] + [0] * 31])),
                                        np.full((1, 1), 127, np.uint8), 32)[0][0, 0]
                  for c in range(64)])
    ints = [c for c in range(64) if g[c] == np.round(g[c]) and abs(g[c]) <= 4]
    rng = np.random.default_rng(11)
    M, N, K = 130, 200, 1024
    ia, ib = rng.choice(ints, size=(M, K)), rng.choice(ints, size=(N, K))
    case = dict(fmt=fmt, M=M, N=N, K=K, A=mxinputs.pack_fp6(ia), B=mxinputs.pack_fp6(ib),
                A_scale=np.full((M, K // 32), 127, np.uint8),
                B_scale=np.full((N, K // 32), 127, np.uint8))
    want = (g[ia].astype(np.int64) @ g[ib].astype(np.int64).T).astype(np.float64)
    got = host64(_run(case, F32))
    log("fp6 exact integers fmt=%d max |diff| %g" % (fmt, np.max(np.abs(got - want))))
    assert np.array_equal(got, want)
