"""GPU parity of the grouped MX GEMM in the formats beyond E2M1 / E4M3: E5M2
with itself and paired with E4M3 or E2M1 either way round, and each FP6
format (E2M3, E3M2) with itself, the other FP6 format, E2M1, E4M3 or E5M2
either way round, against the oracle's grouped GEMM, through
the C ABI: uneven, empty and single-row groups, ragged N and K, both output
types, a full-size expert layer on sampled rows, and one group equal bit for
bit to the dense GEMM on the same tile.

Acceptance as for the other MX GEMMs: |gpu - C| <= 1e-5 * T (+ one bf16 ulp
of C for BF16 output) + E, the oracle's group-alignment term."""
import numpy as np
import pytest

import microscaled_block_scaled_amd as mxg
import mxinputs
import oracle
from gpu_util import acceptance, host64, log

pytestmark = pytest.mark.gpu

E2M1, E4M3, E5M2 = mxinputs.FMT_E2M1, mxinputs.FMT_E4M3, mxinputs.FMT_E5M2
E2M3, E3M2 = mxinputs.FMT_E2M3, mxinputs.FMT_E3M2
F32, BF16 = mxinputs.OUT_FP32, mxinputs.OUT_BF16
PAIRS = ([(E5M2, E5M2), (E4M3, E5M2), (E5M2, E4M3), (E2M1, E5M2), (E5M2, E2M1),
          (E2M3, E2M3), (E3M2, E3M2), (E2M3, E3M2), (E3M2, E2M3)] +
         [(f6, g) for f6 in (E2M3, E3M2) for g in (E2M1, E4M3, E5M2)] +
         [(g, f6) for f6 in (E2M3, E3M2) for g in (E2M1, E4M3, E5M2)])
PAIR_IDS = ["%s_x_%s" % (mxinputs.fmt_name(a), mxinputs.fmt_name(b)) for a, b in PAIRS]
EXPERT_ROWS = [704, 320, 512, 896, 128, 640, 448, 448]


def _case(fa, fb, rows, N, K, seed):
    ca = mxinputs.make_random(fa, sum(rows), 1, K, seed=seed)
    cb = mxinputs.make_random(fb, 1, len(rows) * N, K, seed=seed + 1)
    return dict(fa=fa, fb=fb, rows=list(rows), N=N, K=K, A=ca["A"], A_scale=ca["A_scale"],
                B=cb["B"], B_scale=cb["B_scale"])


def _dev(case):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(case[k])).cuda()
            for k in ("A", "A_scale", "B", "B_scale")]


def _run(case, out, d=None):
    import torch
    d = _dev(case) if d is None else d
    tdt = torch.float32 if out == F32 else torch.bfloat16
    C = mxg.mx_gemm_grouped(d[0], d[1], d[2], d[3], case["rows"], case["fa"], out_dtype=tdt,
                            fmt_b=case["fb"])
    torch.cuda.synchronize()
    return C


def _check(case, out, C, pick=None):
    Cref, T, E = oracle.gemm_grouped(case["fa"], case["A"], case["A_scale"], case["B"],
                                     case["B_scale"], case["K"], case["rows"], rows=pick,
                                     group_bound=True, fmt_b=case["fb"])
    g = host64(C)
    if pick is not None:
        g = g[np.asarray(pick)]
    r = acceptance(g, Cref, T, out == BF16, E, what="grouped formats")
    assert r["n_bad"] == 0, "%d bad, worst ratio %.3g at %s" % (
        r["n_bad"], r["max_ratio"], r["first_bad"])


GROUP_SHAPES = [
    ([70, 0, 200], 130, 384),
    ([1], 33, 128),
    ([300, 1, 0, 64, 257], 96, 640),
    ([17, 64, 0, 300, 1, 129, 256, 33], 200, 1152),
]


@pytest.mark.parametrize("out", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("rows,N,K", GROUP_SHAPES)
@pytest.mark.parametrize("fa,fb", PAIRS, ids=PAIR_IDS)
def test_grouped_formats_shapes(fa, fb, rows, N, K, out):
    log("grouped %d x %d out=%d rows=%s N=%d K=%d" % (fa, fb, out, rows, N, K))
    case = _case(fa, fb, rows, N, K, seed=sum(rows) + N + K + 7 * fa + fb)
    _check(case, out, _run(case, out))


@pytest.mark.parametrize("fa,fb", PAIRS, ids=PAIR_IDS)
def test_grouped_formats_one_group_is_dense(fa, fb):
    """One group is the dense GEMM: mx_gemm on the grouped plan's tile with
    no K split gives the same bits (same kernel body, same K order)."""
    import torch
    M, N, K = 300, 520, 1024
    case = _case(fa, fb, [M], N, K, seed=11 + fa + 3 * fb)
    d = _dev(case)
    plan = mxg.grouped_plan(fa, [M], N, K)
    tile = (plan["tile_m"], plan["tile_n"])
    log("one group %d x %d tile %s" % (fa, fb, tile))
    Cg = _run(case, BF16, d)
    Cd = mxg.mx_gemm(d[0], d[1], d[2], d[3], fa, out_dtype=torch.bfloat16, tile=tile,
                     split_k=1, fmt_b=fb)
    torch.cuda.synchronize()
    assert torch.equal(Cg.view(torch.int16), Cd.view(torch.int16))


@pytest.mark.parametrize("fa,fb", PAIRS, ids=PAIR_IDS)
def test_grouped_formats_expert_layer(fa, fb):
    """Eight uneven experts, N = 4096, K = 2048 (the 8-expert layer the
    bench times): every group's first, middle and last rows; bit-identical
    on a rerun."""
    import torch
    case = _case(fa, fb, EXPERT_ROWS, 4096, 2048, seed=80 + 7 * fa + fb)
    log("expert layer %d x %d plan %s" % (fa, fb, mxg.grouped_plan(fa, EXPERT_ROWS, 4096, 2048)))
    d = _dev(case)
    C = _run(case, BF16, d)
    assert torch.equal(C, _run(case, BF16, d))
    pick, r0 = [], 0
    for m in EXPERT_ROWS:
        pick += [r0, r0 + m // 2, r0 + m - 1]
        r0 += m
    _check(case, BF16, C, pick=pick)
