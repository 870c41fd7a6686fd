"""GPU parity of the grouped MX GEMM with the expert weights in their own
format (mx_gemm_grouped_mixed): E4M3 activations with E2M1 weights, the
usual mixture-of-experts serving layout, and the reverse, against the
oracle's grouped GEMM, through the C ABI: uneven, empty and single-row
groups, ragged N and K, both output types, equal formats matching
mx_gemm_grouped bit for bit, and a full-size expert layer on sampled rows.

Acceptance as for the other MX GEMMs: |gpu - C| <= 1e-5 * T (+ one bf16 ulp
of C for BF16 output) + E, the oracle's 8-product group-alignment term."""
import numpy as np
import pytest

import microscaled_block_scaled_amd as mxg
import mxinputs
import oracle
from gpu_util import acceptance, host64, log

pytestmark = pytest.mark.gpu

E2M1, E4M3 = mxinputs.FMT_E2M1, mxinputs.FMT_E4M3
F32, BF16 = mxinputs.OUT_FP32, mxinputs.OUT_BF16
PAIRS = [(E4M3, E2M1), (E2M1, E4M3)]
PAIR_IDS = ["a8w4", "a4w8"]
EXPERT_ROWS = [704, 320, 512, 896, 128, 640, 448, 448]


def _case(fa, fb, rows, N, K, seed):
    ca = mxinputs.make_random(fa, sum(rows), 1, K, seed=seed)
    cb = mxinputs.make_random(fb, 1, len(rows) * N, K, seed=seed + 1)
    return dict(fa=fa, fb=fb, rows=list(rows), N=N, K=K, A=ca["A"], A_scale=ca["A_scale"],
                B=cb["B"], B_scale=cb["B_scale"])


def _run(case, out, fb=None):
    import torch
    d = [torch.from_numpy(np.ascontiguousarray(case[k])).cuda()
         for k in ("A", "A_scale", "B", "B_scale")]
    tdt = torch.float32 if out == F32 else torch.bfloat16
    C = mxg.mx_gemm_grouped(d[0], d[1], d[2], d[3], case["rows"], case["fa"], out_dtype=tdt,
                            fmt_b=case["fb"] if fb is None else fb)
    torch.cuda.synchronize()
    return C


def _check(case, out, C, pick=None):
    Cref, T, E = oracle.gemm_grouped(case["fa"], case["A"], case["A_scale"], case["B"],
                                     case["B_scale"], case["K"], case["rows"], rows=pick,
                                     group_bound=True, fmt_b=case["fb"])
    g = host64(C)
    if pick is not None:
        g = g[np.asarray(pick)]
    r = acceptance(g, Cref, T, out == BF16, E, what="grouped mixed")
    assert r["n_bad"] == 0, "%d bad, worst ratio %.3g at %s" % (
        r["n_bad"], r["max_ratio"], r["first_bad"])


GROUP_SHAPES = [
    ([70, 0, 200], 130, 384),
    ([1], 33, 128),
    ([0, 0, 5], 256, 256),
    ([300, 1, 0, 64, 257], 96, 640),
    ([17, 64, 0, 300, 1, 129, 256, 33], 200, 1152),
]


@pytest.mark.parametrize("out", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("rows,N,K", GROUP_SHAPES)
@pytest.mark.parametrize("fa,fb", PAIRS, ids=PAIR_IDS)
def test_grouped_mixed_shapes(fa, fb, rows, N, K, out):
    log("grouped mixed %d x %d out=%d rows=%s N=%d K=%d" % (fa, fb, out, rows, N, K))
    case = _case(fa, fb, rows, N, K, seed=sum(rows) + N + K + fa)
    _check(case, out, _run(case, out))


def test_grouped_mixed_equal_formats_is_grouped():
    """fmt_a == fmt_b through the mixed entry point is mx_gemm_grouped, bit for
    bit (the binding routes equal formats there, so call the C ABI)."""
    import torch
    case = _case(E4M3, E4M3, [100, 0, 300], 192, 512, seed=3)
    d = [torch.from_numpy(np.ascontiguousarray(case[k])).cuda()
         for k in ("A", "A_scale", "B", "B_scale")]
    C1 = torch.empty((400, 192), dtype=torch.bfloat16, device="cuda")
    C2 = torch.empty_like(C1)
    import ctypes
    arr = (ctypes.c_int64 * 3)(100, 0, 300)
    L = mxg.lib()
    s = torch.cuda.current_stream().cuda_stream
    ptr = [t.data_ptr() for t in d]
    assert L.mx_gemm_grouped_mixed(E4M3, E4M3, 3, arr, 192, 512, *ptr, C1.data_ptr(), 2, s) == 0
    assert L.mx_gemm_grouped(E4M3, 3, arr, 192, 512, *ptr, C2.data_ptr(), 2, s) == 0
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)


@pytest.mark.parametrize("fa,fb", PAIRS, ids=PAIR_IDS)
def test_grouped_mixed_expert_layer(fa, fb):
    """Eight uneven experts, N = 4096, K = 2048: every group's first, middle
    and last rows; bit-identical on a rerun."""
    import torch
    case = _case(fa, fb, EXPERT_ROWS, 4096, 2048, seed=60 + fa)
    C = _run(case, BF16)
    assert torch.equal(C, _run(case, BF16))
    pick, r0 = [], 0
    for m in EXPERT_ROWS:
        pick += [r0, r0 + m // 2, r0 + m - 1]
        r0 += m
    _check(case, BF16, C, pick=pick)
