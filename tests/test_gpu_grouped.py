"""GPU parity of the grouped MX GEMM (one weight per group, as in a
mixture-of-experts layer) against the oracle's grouped GEMM, through the C
ABI: uneven, empty, single-row and many tiny groups, ragged N and K tails,
both element formats and both output types, the largest group count, and a
full-size expert layer checked on sampled rows."""
import numpy as np
import pytest

import microscaled_block_scaled_amd as mxg
import mxinputs
import oracle
from gpu_util import acceptance, host64, log

pytestmark = pytest.mark.gpu

E2M1, E4M3 = mxinputs.FMT_E2M1, mxinputs.FMT_E4M3
F32, BF16 = mxinputs.OUT_FP32, mxinputs.OUT_BF16

# Eight experts' token counts of one 4096-token batch (uneven load).
EXPERT_ROWS = [704, 320, 512, 896, 128, 640, 448, 448]


def _case(fmt, rows, N, K, seed):
    G = len(rows)
    case = mxinputs.make_random(fmt, sum(rows), G * N, K, seed=seed)
    case["rows"], case["N"] = list(rows), N
    return case


def _dev(case):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(case[k])).cuda()
            for k in ("A", "A_scale", "B", "B_scale")]


def _run(case, out, dev=None):
    import torch
    a, s, b, bs = dev or _dev(case)
    tdt = torch.float32 if out == F32 else torch.bfloat16
    C = mxg.mx_gemm_grouped(a, s, b, bs, case["rows"], case["fmt"], out_dtype=tdt)
    torch.cuda.synchronize()
    return C


def _check(case, out, C, rows=None):
    e4m3 = case["fmt"] == E4M3
    res = oracle.gemm_grouped(case["fmt"], case["A"], case["A_scale"], case["B"],
                              case["B_scale"], case["K"], case["rows"], rows=rows,
                              group_bound=e4m3)
    g = host64(C)
    if rows is not None:
        g = g[np.asarray(rows)]
    r = acceptance(g, res[0], res[1], out == BF16, res[2] if e4m3 else None, what="grouped")
    assert r["n_bad"] == 0, "%d bad, worst ratio %.3g at %s" % (
        r["n_bad"], r["max_ratio"], r["first_bad"])


GROUP_SHAPES = [
    ([70, 0, 200], 130, 384),            # an empty group, ragged rows and N
    ([1], 33, 128),                       # one row, one group
    ([0, 0, 5], 256, 256),                # leading empty groups
    ([300, 1, 0, 64, 257], 96, 640),      # single-row and empty groups between
    ([17, 64, 0, 300, 1, 129, 256, 33], 200, 1152),
]


@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
@pytest.mark.parametrize("out", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("rows,N,K", GROUP_SHAPES)
def test_grouped_shapes(fmt, out, rows, N, K):
    log("grouped fmt=%d out=%d rows=%s N=%d K=%d" % (fmt, out, rows, N, K))
    case = _case(fmt, rows, N, K, seed=sum(rows) + N + K)
    _check(case, out, _run(case, out))


@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
def test_grouped_most_groups(fmt):
    """256 groups of 0 to 5 rows: the group table at its largest."""
    rng = np.random.default_rng(3)
    rows = [int(r) for r in rng.integers(0, 6, mxg.MAX_GROUPS)]
    log("grouped fmt=%d G=%d total=%d" % (fmt, len(rows), sum(rows)))
    case = _case(fmt, rows, 64, 128, seed=77)
    _check(case, BF16, _run(case, BF16))


def test_grouped_small_m_groups():
    """Every group shorter than 64 rows (decode-like expert loads): the short
    tile runs."""
    rows = [8, 1, 33, 64, 0, 17]
    log("grouped small groups %s" % rows)
    case = _case(E4M3, rows, 1000, 2048, seed=5)
    _check(case, BF16, _run(case, BF16))


def test_grouped_no_rows_launches_nothing():
    import torch
    rows = [0, 0, 0]
    K, N = 256, 64
    a = torch.zeros((0, K), dtype=torch.uint8, device="cuda")
    s = torch.zeros((0, K // 32), dtype=torch.uint8, device="cuda")
    b = torch.zeros((3 * N, K), dtype=torch.uint8, device="cuda")
    bs = torch.zeros((3 * N, K // 32), dtype=torch.uint8, device="cuda")
    C = mxg.mx_gemm_grouped(a, s, b, bs, rows, E4M3)
    torch.cuda.synchronize()
    assert tuple(C.shape) == (0, N)


def test_grouped_single_group_matches_plain_gemm():
    """One group is a plain GEMM: same values as mx_gemm at the tile the
    grouped launch uses, with no K split (same accumulation order)."""
    import torch
    M, N, K = 300, 520, 1024
    case = _case(E2M1, [M], N, K, seed=9)
    dev = _dev(case)
    Cg = _run(case, F32, dev)
    # The grouped launch never splits K; compare against each unsplit tile
    # mx_gemm offers: one of them is the grouped launch's tile.
    same = False
    for tile in mxg.tile_shapes():
        if tile[0] < 256 and M > tile[0]:
            continue
        Cp = mxg.mx_gemm(*dev, E2M1, out_dtype=torch.float32, tile=tile, split_k=1)
        torch.cuda.synchronize()
        same |= bool(torch.equal(Cp, Cg))
    assert same
    _check(case, F32, Cg)


@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
def test_grouped_expert_layer_full_size(fmt):
    """Eight uneven experts, 4096 tokens, N = 4096, K = 2048 (the size the
    benchmark times): sampled rows of every group, including each group's
    first and last rows, against the oracle; two runs are bit-identical."""
    import torch
    rows, N, K = EXPERT_ROWS, 4096, 2048
    log("grouped full size fmt=%d" % fmt)
    case = _case(fmt, rows, N, K, seed=2024 + fmt)
    dev = _dev(case)
    C = _run(case, BF16, dev)
    C2 = _run(case, BF16, dev)
    assert torch.equal(C, C2)
    starts = np.cumsum([0] + rows)
    pick = set()
    for g in range(len(rows)):
        lo, hi = starts[g], starts[g + 1]
        pick |= {lo, lo + 1, hi - 2, hi - 1, (lo + hi) // 2}
    pick = sorted(int(r) for r in pick)
    _check(case, BF16, C, rows=pick)


def test_grouped_out_argument_and_stream():
    import torch
    rows, N, K = [40, 0, 90], 128, 512
    case = _case(E4M3, rows, N, K, seed=12)
    dev = _dev(case)
    ref = _run(case, BF16, dev)
    out = torch.full((sum(rows), N), float("nan"), dtype=torch.bfloat16, device="cuda")
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        mxg.mx_gemm_grouped(*dev, rows, E4M3, out=out)
    st.synchronize()
    assert torch.equal(out, ref)
