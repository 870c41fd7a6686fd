"""GPU parity of the grouped dense BF16 GEMM (one BF16 weight per group, as
in a mixture-of-experts layer) against the oracle's grouped BF16 GEMM,
through the C ABI: uneven, empty, single-row and many tiny groups, ragged N
and K tails, both output types, one group against mx_gemm_bf16, and a
full-size expert layer checked on sampled rows of every group.

Acceptance as for the dense BF16 GEMM: |gpu - C| <= 1e-5 * T (+ one BF16
ulp of C for BF16 output)."""
import numpy as np
import pytest

import microscaled_block_scaled_amd as mxg
import mxinputs
import oracle
from gpu_util import acceptance, host64, log

pytestmark = pytest.mark.gpu

F32, BF16 = mxinputs.OUT_FP32, mxinputs.OUT_BF16

# Eight experts' token counts of one 4096-token batch (uneven load).
EXPERT_ROWS = [704, 320, 512, 896, 128, 640, 448, 448]


def _case(rows, N, K, seed):
    return (mxinputs.make_bf16(sum(rows), K, seed=seed, tensor=0),
            mxinputs.make_bf16(len(rows) * N, K, seed=seed, tensor=1))


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def _run(A, B, rows, out, dA=None, dB=None):
    import torch
    tdt = torch.float32 if out == F32 else torch.bfloat16
    C = mxg.mx_gemm_grouped_bf16(_dev(A) if dA is None else dA, _dev(B) if dB is None else dB,
                                 rows, out_dtype=tdt)
    torch.cuda.synchronize()
    return C


def _check(A, B, rows, out, C, pick=None):
    Cref, T = oracle.gemm_grouped_bf16(A, B, rows, rows=pick)
    g = host64(C)
    if pick is not None:
        g = g[np.asarray(pick)]
    r = acceptance(g, Cref, T, out == BF16, what="grouped bf16")
    assert r["n_bad"] == 0, "%d bad, worst ratio %.3g at %s" % (
        r["n_bad"], r["max_ratio"], r["first_bad"])


GROUP_SHAPES = [
    ([70, 0, 200], 130, 384),            # an empty group, ragged rows and N
    ([1], 33, 128),                       # one row, one group
    ([0, 0, 5], 256, 256),                # leading empty groups
    ([300, 1, 0, 64, 257], 96, 656),      # single-row and empty groups between; K % 64 != 0
    ([17, 64, 0, 300, 1, 129, 256, 33], 200, 1104),
]


@pytest.mark.parametrize("out", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("rows,N,K", GROUP_SHAPES)
def test_grouped_bf16_shapes(out, rows, N, K):
    log("grouped bf16 out=%d rows=%s N=%d K=%d plan=%s"
        % (out, rows, N, K, mxg.grouped_bf16_plan(rows, N, K, out)))
    A, B = _case(rows, N, K, seed=sum(rows) + N + K)
    _check(A, B, rows, out, _run(A, B, rows, out))


def test_grouped_bf16_most_groups():
    """256 groups of 0 to 5 rows: the group table at its largest."""
    rows = [int(x) for x in np.random.default_rng(4).integers(0, 6, mxg.MAX_GROUPS)]
    A, B = _case(rows, 48, 128, seed=99)
    _check(A, B, rows, F32, _run(A, B, rows, F32))


def test_grouped_bf16_no_rows():
    """Every group empty: nothing is launched and C has no rows."""
    import torch
    A = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((3 * 64, 128), dtype=torch.bfloat16, device="cuda")
    C = mxg.mx_gemm_grouped_bf16(A, B, [0, 0, 0])
    assert tuple(C.shape) == (0, 64)


def test_grouped_bf16_one_group_equals_plain():
    """One group is the plain BF16 GEMM with the same tile, bit for bit."""
    import torch
    M, N, K = 600, 520, 1024
    A, B = _case([M], N, K, seed=7)
    dA, dB = _dev(A), _dev(B)
    p = mxg.grouped_bf16_plan([M], N, K)
    C1 = _run(A, B, [M], BF16, dA, dB)
    C2 = mxg.mx_gemm_bf16(dA, dB, tile=(p["tile_m"], p["tile_n"]), split_k=1)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)


def test_grouped_bf16_expert_layer():
    """Eight uneven experts, N = 4096, K = 2048: the first, last and a middle
    row of every group, bit-identical on a rerun."""
    import torch
    rows, N, K = EXPERT_ROWS, 4096, 2048
    log("grouped bf16 expert layer plan=%s" % mxg.grouped_bf16_plan(rows, N, K))
    A, B = _case(rows, N, K, seed=5)
    dA, dB = _dev(A), _dev(B)
    C = _run(A, B, rows, BF16, dA, dB)
    assert torch.equal(C, _run(A, B, rows, BF16, dA, dB))
    pick, r0 = [], 0
    for m in rows:
        pick += [r0, r0 + m // 2, r0 + m - 1]
        r0 += m
    _check(A, B, rows, BF16, C, pick=pick)
