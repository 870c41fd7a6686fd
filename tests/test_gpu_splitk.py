"""The split-K path through the C ABI: every K-slice of a tile writes its
FP32 partial sums to a plane of the stream's workspace, and a second kernel
adds the planes in slice order.  The result must not depend on the order
in which the slices ran, on what an earlier call left in the workspace, or
on whether the grid's slices fit on the GPU at once."""
import numpy as np
import pytest

import microscaled_block_scaled_amd as mxg
import mxinputs
import oracle
from gpu_util import acceptance, host64, log, run_gpu, to_dev

pytestmark = pytest.mark.gpu

E2M1, E4M3 = mxinputs.FMT_E2M1, mxinputs.FMT_E4M3
F32, BF16 = mxinputs.OUT_FP32, mxinputs.OUT_BF16


def _case(fmt, M, N, K, seed):
    case = mxinputs.make_random(fmt, M, N, K, seed=seed)
    case["fmt"] = fmt
    return case


def _check(case, C, out, what):
    Cref, T = oracle.gemm(case["fmt"], case["A"], case["A_scale"], case["B"], case["B_scale"],
                          case["K"])[:2]
    res = acceptance(host64(C), Cref, T, out == BF16, what=what)
    assert res["n_bad"] == 0, (what, res)


def _bits(C):
    import torch
    return C.view(torch.int16 if C.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
def test_split_result_is_the_same_every_call(fmt):
    """The order in which a tile's slices run changes from call to call; the
    sum does not (planes added in slice order): ten calls, one result, bit
    for bit."""
    M, N, K = 256, 1024, 8192
    case = _case(fmt, M, N, K, seed=4100 + fmt)
    dev = to_dev(case)
    log("split repeat fmt=%d M=%d N=%d K=%d tile 256x128 split 8" % (fmt, M, N, K))
    first = run_gpu(case, BF16, dev=dev, tile=(256, 128), split_k=8)
    _check(case, first, BF16, "split repeat first")
    want = _bits(first)
    for i in range(9):
        again = run_gpu(case, BF16, dev=dev, tile=(256, 128), split_k=8)
        assert np.array_equal(_bits(again), want), "call %d differs" % (i + 1)


def test_split_sequence_reuses_the_workspace():
    """Split calls of different grids back to back on one stream: larger
    planes than before (the workspace grows), smaller ones (it is reused
    with stale planes beyond the new ones), other splits, ragged N and both
    output types.  Every result is checked, and the first shape, run again
    at the end, must repeat its first result bit for bit."""
    seq = [
        (E2M1, 64, 520, 4096, (128, 128), 4, BF16),
        (E4M3, 300, 2000, 4096, (128, 128), 2, F32),      # larger planes: workspace grows
        (E2M1, 40, 203, 6144, (128, 128), 3, F32),        # N % 4 != 0
        (E4M3, 40, 203, 3072, (64, 256), 6, BF16),
        (E2M1, 512, 768, 2048, (256, 256), 4, BF16),
        (E2M1, 64, 520, 4096, (128, 128), 4, BF16),       # the first call again
    ]
    import torch
    results = []
    for i, (fmt, M, N, K, tile, split, out) in enumerate(seq):
        case = _case(fmt, M, N, K, seed=4200 if i in (0, len(seq) - 1) else 4200 + i)
        log("split sequence %d fmt=%d M=%d N=%d K=%d tile %s split %d out %d"
            % (i, fmt, M, N, K, tile, split, out))
        C = run_gpu(case, out, tile=tile, split_k=split)
        torch.cuda.synchronize()
        _check(case, C, out, "split sequence %d" % i)
        results.append(_bits(C))
    assert np.array_equal(results[0], results[-1])


@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
def test_split_grid_larger_than_the_gpu(fmt):
    """256 tiles x 4 slices = 1024 workgroups, four per CU: the slices of a
    tile run in different waves of workgroups."""
    M, N, K = 2048, 2048, 4096
    case = _case(fmt, M, N, K, seed=4300 + fmt)
    p = mxg.plan(fmt, M, N, K, BF16)
    log("split large grid fmt=%d M=%d N=%d K=%d tile 128x128 split 4 (plan: %s)"
        % (fmt, M, N, K, p))
    C = run_gpu(case, BF16, tile=(128, 128), split_k=4)
    rows = np.unique(np.r_[0:8, 120:136, np.linspace(0, M - 1, 64).astype(int), M - 8:M])
    Cref, T = oracle.gemm(fmt, case["A"][rows], case["A_scale"][rows], case["B"],
                          case["B_scale"], K)[:2]
    res = acceptance(host64(C)[rows], Cref, T, True, what="split large grid")
    assert res["n_bad"] == 0, res


def test_split_and_unsplit_exact_on_integers():
    """On integer inputs every partial sum is an exact FP32 integer, so the
    order of the K-sum does not matter: the unsplit kernel and an 8-way
    split both equal numpy's int64 product bit for bit."""
    M, N, K = 96, 640, 8192
    rng = np.random.default_rng(4400)
    # E4M3 integers 0..4 with scale 2^0: every partial sum is an exact FP32 integer
    case = _case(E4M3, M, N, K, seed=4400)
    vals = np.array([0x00, 0x38, 0x40, 0x44, 0x48], np.uint8)      # 0, 1, 2, 3, 4
    case["A"] = vals[rng.integers(0, 5, size=(M, K))]
    case["B"] = vals[rng.integers(0, 5, size=(N, K))]
    case["A_scale"] = np.full((M, K // 32), 127, np.uint8)
    case["B_scale"] = np.full((N, K // 32), 127, np.uint8)
    unsplit = run_gpu(case, F32, tile=(128, 128), split_k=1)
    split = run_gpu(case, F32, tile=(128, 128), split_k=8)
    ia = np.select([case["A"] == v for v in vals], np.arange(5)).astype(np.int64)
    ib = np.select([case["B"] == v for v in vals], np.arange(5)).astype(np.int64)
    want = ia @ ib.T
    assert np.array_equal(host64(unsplit), want.astype(np.float64))
    assert np.array_equal(host64(split), want.astype(np.float64))
