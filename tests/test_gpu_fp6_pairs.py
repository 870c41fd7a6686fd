"""GPU parity of MX GEMMs pairing an FP6 format (E2M3, E3M2) with another
element format -- E2M1, E4M3, E5M2 or the other FP6 format, either way round
-- against the oracle, through the C ABI (mx_gemm_mixed): ragged shapes,
every tile with and without a K split, and the fused-QKV shape on sampled
rows.  Each operand keeps its own row layout (K/2, 3K/4 or K bytes) and
MFMA format selector.

Acceptance as for the other MX formats: |gpu - C| <= 1e-5 * T (+ one bf16
ulp of C for BF16 output) + E, the oracle's 8-product group-alignment
term."""
import numpy as np
import pytest

import microscaled_block_scaled_amd as mxg
import mxinputs
import oracle
from gpu_util import acceptance, host64, log, sample_rows

pytestmark = pytest.mark.gpu

E2M1, E4M3, E5M2 = mxinputs.FMT_E2M1, mxinputs.FMT_E4M3, mxinputs.FMT_E5M2
E2M3, E3M2 = mxinputs.FMT_E2M3, mxinputs.FMT_E3M2
F32, BF16 = mxinputs.OUT_FP32, mxinputs.OUT_BF16
PAIRS = ([(f6, g) for f6 in (E2M3, E3M2) for g in (E2M1, E4M3, E5M2)] +
         [(g, f6) for f6 in (E2M3, E3M2) for g in (E2M1, E4M3, E5M2)] +
         [(E2M3, E3M2), (E3M2, E2M3)])
PAIR_IDS = ["%s_x_%s" % (mxinputs.fmt_name(a), mxinputs.fmt_name(b)) for a, b in PAIRS]


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


TAIL_SHAPES = [(1, 1, 128), (33, 255, 384), (130, 7, 640), (64, 300, 1152)]


@pytest.mark.parametrize("out", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", TAIL_SHAPES)
@pytest.mark.parametrize("fa,fb", PAIRS, ids=PAIR_IDS)
def test_fp6_pair_tails(fa, fb, M, N, K, out):
    log("fp6 pair %d x %d out=%d M=%d N=%d K=%d" % (fa, fb, out, M, N, K))
    case = _case(fa, fb, M, N, K, seed=M + 2 * N + K + 7 * fa + fb)
    _check(case, out, _run(case, out), what="tails")


@pytest.mark.parametrize("split", [1, 3], ids=["nosplit", "split3"])
@pytest.mark.parametrize("tile", mxg.tile_shapes(), ids=["%dx%d" % t for t in mxg.tile_shapes()])
@pytest.mark.parametrize("fa,fb", PAIRS, ids=PAIR_IDS)
def test_fp6_pair_every_tile(fa, fb, tile, split):
    bm, bn = tile
    M, N, K = 2 * bm + 19, 2 * bn + 24, 3584
    log("fp6 pair %d x %d tile %dx%d split %d" % (fa, fb, bm, bn, split))
    case = _case(fa, fb, M, N, K, seed=bm + bn + split + 7 * fa + fb)
    C = _run(case, BF16, tile=tile, split_k=split)
    _check(case, BF16, C, rows=sample_rows(M, tile=bm, n=32), what="tile")


@pytest.mark.parametrize("fa,fb", PAIRS, ids=PAIR_IDS)
def test_fp6_pair_full_size(fa, fb):
    """The fused-QKV shape (2048 x 6144 x 4096) in the plan's configuration,
    sampled rows; a rerun is bit for bit the same."""
    import torch
    M, N, K = 2048, 6144, 4096
    case = _case(fa, fb, M, N, K, seed=90 + 7 * fa + fb)
    log("fp6 pair %d x %d full size plan %s" % (fa, fb, mxg.plan(fa, M, N, K)))
    C = _run(case, BF16)
    assert torch.equal(C, _run(case, BF16))
    _check(case, BF16, C, rows=sample_rows(M, n=24), what="full size")
