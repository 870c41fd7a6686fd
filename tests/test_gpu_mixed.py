"""GPU parity of mixed-format MX GEMMs (A E4M3 x B E2M1, "W4A8", and A E2M1
x B E4M3) against the oracle, through the C ABI (mx_gemm_mixed): ragged
shapes, every tile with and without a K split, small M, full-size shapes on
sampled rows, and equal formats through mx_gemm_mixed matching mx_gemm bit
for bit.

Acceptance as for one format: |gpu - C| <= 1e-5 * T (+ one bf16 ulp of C for
BF16 output) + E, the oracle's 8-product group-alignment term; the log says
how many elements need E."""

import numpy as np
import pytest

import microscaled_block_scaled_amd as mxg
import mxinputs
import oracle
from gpu_util import acceptance, host64, log, sample_rows

pytestmark = pytest.mark.gpu

E2M1, E4M3 = mxinputs.FMT_E2M1, mxinputs.FMT_E4M3
F32, BF16 = mxinputs.OUT_FP32, mxinputs.OUT_BF16
PAIRS = [(E4M3, E2M1), (E2M1, E4M3)]
PAIR_IDS = ["a8w4", "a4w8"]


def _case(fa, fb, M, N, K, seed):
    ca = mxinputs.make_random(fa, M, 1, K, seed=seed)
    cb = mxinputs.make_random(fb, 1, N, K, seed=seed + 1)
    return dict(fa=fa, fb=fb, M=M, N=N, K=K, A=ca["A"], A_scale=ca["A_scale"],
                B=cb["B"], B_scale=cb["B_scale"])


def _run(case, out, tile=None, split_k=0):
    import torch
    d = [torch.from_numpy(np.ascontiguousarray(case[k])).cuda()
         for k in ("A", "A_scale", "B", "B_scale")]
    tdt = torch.float32 if out == F32 else torch.bfloat16
    C = mxg.mx_gemm(d[0], d[1], d[2], d[3], case["fa"], out_dtype=tdt, tile=tile,
                    split_k=split_k, fmt_b=case["fb"])
    torch.cuda.synchronize()
    return C


def _check(case, out, C, rows=None, what=""):
    Cref, T, E = oracle.gemm(case["fa"], case["A"], case["A_scale"], case["B"],
                             case["B_scale"], case["K"], rows=rows, group_bound=True,
                             fmt_b=case["fb"])
    g = host64(C)
    if rows is not None:
        g = g[np.asarray(rows)]
    r = acceptance(g, Cref, T, out == BF16, E, what=what)
    assert r["n_bad"] == 0, "%s: %d bad, worst ratio %.3g at %s" % (
        what, r["n_bad"], r["max_ratio"], r["first_bad"])


TAIL_SHAPES = [(1, 1, 128), (7, 33, 256), (33, 255, 128), (255, 257, 384),
               (257, 129, 512), (130, 7, 640), (64, 300, 1152)]


@pytest.mark.parametrize("fa,fb", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("out", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", TAIL_SHAPES)
def test_mixed_tails(fa, fb, out, M, N, K):
    log("mixed tails fa=%d fb=%d out=%d M=%d N=%d K=%d" % (fa, fb, out, M, N, K))
    case = _case(fa, fb, M, N, K, seed=M * 5 + N + K)
    _check(case, out, _run(case, out), what="tails")


def _tile_ids():
    return ["%dx%d" % t for t in mxg.tile_shapes()]


@pytest.mark.parametrize("split", [1, 3], ids=["nosplit", "split3"])
@pytest.mark.parametrize("tile", mxg.tile_shapes(), ids=_tile_ids())
@pytest.mark.parametrize("fa,fb", PAIRS, ids=PAIR_IDS)
def test_mixed_every_tile(fa, fb, tile, split):
    """Each tile forced on a problem two tiles (plus a ragged part) in each
    direction, K spanning several scale periods and a partial main-loop
    trip; with 3 K slices the split-K path and its reduction run too."""
    bm, bn = tile
    M, N, K = 2 * bm + 19, 2 * bn + 24, 3584
    log("mixed tile %dx%d split %d fa=%d fb=%d" % (bm, bn, split, fa, fb))
    case = _case(fa, fb, M, N, K, seed=bm + bn + split)
    C = _run(case, BF16, tile=tile, split_k=split)
    _check(case, BF16, C, rows=sample_rows(M, tile=bm), what="tile")


@pytest.mark.parametrize("fa,fb", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("M,N,K", [(1, 1000, 8192), (8, 8192, 4096), (64, 640, 3968)])
def test_mixed_small_m(fa, fb, M, N, K):
    log("mixed small M fa=%d fb=%d M=%d N=%d K=%d plan=%s" % (fa, fb, M, N, K,
                                                             mxg.plan(fa, M, N, K)))
    case = _case(fa, fb, M, N, K, seed=M + N)
    _check(case, BF16, _run(case, BF16), what="small M")


@pytest.mark.parametrize("fa,fb", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("M,N,K", [(2048, 6144, 4096), (8, 8192, 28672)])
def test_mixed_full_size(fa, fb, M, N, K):
    """Serving shapes (fused QKV projection; 70B down projection at batch 8)
    in the plan's launch configuration, on sampled rows; a second run is bit
    for bit the same."""
    import torch
    log("mixed full size fa=%d fb=%d M=%d N=%d K=%d" % (fa, fb, M, N, K))
    case = _case(fa, fb, M, N, K, seed=7)
    C = _run(case, BF16)
    assert torch.equal(C, _run(case, BF16))
    rows = sample_rows(M, n=24)
    _check(case, BF16, C, rows=rows, what="full size")


@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
def test_mixed_entry_with_equal_formats_is_mx_gemm(fmt):
    import torch
    M, N, K = 300, 260, 1536
    case = mxinputs.make_random(fmt, M, N, K, seed=21)
    d = [torch.from_numpy(np.ascontiguousarray(case[k])).cuda()
         for k in ("A", "A_scale", "B", "B_scale")]
    C1 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    C2 = torch.empty_like(C1)
    st = torch.cuda.current_stream().cuda_stream
    ptrs = [t.data_ptr() for t in d]
    assert mxg.lib().mx_gemm(fmt, M, N, K, *ptrs, C1.data_ptr(), BF16, st) == 0
    assert mxg.lib().mx_gemm_mixed(fmt, fmt, M, N, K, *ptrs, C2.data_ptr(), BF16, 0, 0, 0,
                                   st) == 0
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
