"""GPU parity of MX GEMMs pairing E5M2 with another element format (A E4M3
x B E5M2 and the reverse, E5M2 x E2M1 and the reverse) against the oracle,
through the C ABI (mx_gemm_mixed): ragged shapes, every tile with and
without a K split, small M, a full-size shape on sampled rows, and
infinities and NaNs from the E5M2 operand.

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
F32, BF16 = mxinputs.OUT_FP32, mxinputs.OUT_BF16
PAIRS = [(E4M3, E5M2), (E5M2, E4M3), (E5M2, E2M1), (E2M1, E5M2)]
PAIR_IDS = ["e4m3_e5m2", "e5m2_e4m3", "e5m2_e2m1", "e2m1_e5m2"]


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


def _check(case, out, C, rows=None, what="", group_term=False):
    Cref, T, E = oracle.gemm(case["fa"], case["A"], case["A_scale"], case["B"],
                             case["B_scale"], case["K"], rows=rows, group_bound=True,
                             fmt_b=case["fb"])
    g = host64(C)
    if rows is not None:
        g = g[np.asarray(rows)]
    r = acceptance(g, Cref, T, out == BF16, E, group_term, what)
    assert r["n_bad"] == 0, "%s: %d bad, worst ratio %.3g at %s" % (
        what, r["n_bad"], r["max_ratio"], r["first_bad"])


TAIL_SHAPES = [(1, 1, 128), (33, 255, 128), (255, 257, 384), (130, 7, 640), (64, 300, 1152)]


@pytest.mark.parametrize("out", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", TAIL_SHAPES)
@pytest.mark.parametrize("fa,fb", PAIRS, ids=PAIR_IDS)
def test_e5m2_pair_tails(fa, fb, M, N, K, out):
    log("e5m2 pair %d x %d out=%d M=%d N=%d K=%d" % (fa, fb, out, M, N, K))
    case = _case(fa, fb, M, N, K, seed=M + 2 * N + K + fa)
    # K = 128 is four blocks: the group error of an 8-bit operand is then not
    # averaged over many blocks (the only shape here that needs the group term)
    _check(case, out, _run(case, out), what="tails", group_term=K == 128)


@pytest.mark.parametrize("split", [1, 3], ids=["nosplit", "split3"])
@pytest.mark.parametrize("tile", mxg.tile_shapes(), ids=["%dx%d" % t for t in mxg.tile_shapes()])
@pytest.mark.parametrize("fa,fb", [(E4M3, E5M2), (E5M2, E2M1)], ids=["e4m3_e5m2", "e5m2_e2m1"])
def test_e5m2_pair_every_tile(fa, fb, tile, split):
    bm, bn = tile
    M, N, K = 2 * bm + 19, 2 * bn + 24, 3584
    log("e5m2 pair %d x %d tile %dx%d split %d" % (fa, fb, bm, bn, split))
    case = _case(fa, fb, M, N, K, seed=bm + bn + split + fa)
    C = _run(case, BF16, tile=tile, split_k=split)
    _check(case, BF16, C, rows=sample_rows(M, tile=bm), what="tile")


@pytest.mark.parametrize("fa,fb", PAIRS, ids=PAIR_IDS)
def test_e5m2_pair_small_m_and_full_size(fa, fb):
    """8 rows against a 70B-down-shaped weight (the decode kernel), and the
    fused-QKV shape on sampled rows, bit-identical on a rerun."""
    import torch
    case = _case(fa, fb, 8, 8192, 4096, seed=70 + fa)
    _check(case, BF16, _run(case, BF16), what="small M")
    case = _case(fa, fb, 2048, 6144, 4096, seed=80 + fa)
    C = _run(case, BF16)
    assert torch.equal(C, _run(case, BF16))
    _check(case, BF16, C, rows=sample_rows(2048, n=32), what="full size")


def test_e5m2_pair_infinities_and_nans():
    """An E5M2 infinity times a non-zero E4M3 value makes its output infinite,
    times zero makes NaN, and an E5M2 NaN makes NaN; the GPU's pattern of
    infinite and NaN outputs is the oracle's."""
    K = 128
    case = _case(E5M2, E4M3, 4, 6, K, seed=3)
    A, B = case["A"].copy(), case["B"].copy()
    A[0, 5] = 0x7C                       # +inf in A row 0
    A[1, 40] = 0x7F                      # NaN in A row 1
    A[2, 70] = 0xFC                      # -inf in A row 2 ...
    B[3, 70] = 0x00                      # ... times zero in B row 3: NaN at (2, 3)
    case = dict(case, A=A, B=B)
    C = host64(_run(case, F32))
    Cref, _ = oracle.gemm(E5M2, A, case["A_scale"], B, case["B_scale"], K, fmt_b=E4M3)
    log("e5m2 pair specials: gpu inf %s nan %s / oracle inf %s nan %s" % (
        np.isinf(C).sum(), np.isnan(C).sum(), np.isinf(Cref).sum(), np.isnan(Cref).sum()))
    assert np.array_equal(np.isnan(C), np.isnan(Cref))
    assert np.array_equal(np.isinf(C), np.isinf(Cref))
    assert np.array_equal(np.sign(C[np.isinf(C)]), np.sign(Cref[np.isinf(Cref)]))
    fin = np.isfinite(Cref)
    assert np.all(np.abs(C[fin] - Cref[fin]) <= 1e-4 * np.abs(Cref[fin]) + 1e-30)
