"""mx_gemm_noalloc (no allocation: split-K planes in the library's fixed
per-device scratch) against mx_gemm, through the C ABI: the same plan and
kernels, so the results must be identical bit for bit.  Two calls in a row,
the second smaller, so the second reads a scratch the first has written."""
import numpy as np
import pytest

import microscaled_block_scaled_amd as mxg
import mxinputs
import oracle
from gpu_util import acceptance, host64, log

pytestmark = pytest.mark.gpu

E2M1, E4M3 = mxinputs.FMT_E2M1, mxinputs.FMT_E4M3


def _dev(case):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(case[k])).cuda()
            for k in ("A", "A_scale", "B", "B_scale")]


def _both(case, out):
    """C from mx_gemm and from mx_gemm_noalloc on the same device inputs."""
    import torch
    A, As, B, Bs = _dev(case)
    M, N, K, fmt = case["M"], case["N"], case["K"], case["fmt"]
    tdt = torch.float32 if out == mxinputs.OUT_FP32 else torch.bfloat16
    s = torch.cuda.current_stream().cuda_stream
    res = []
    for fn in (mxg.gemm_ptr, mxg.gemm_noalloc_ptr):
        C = torch.full((M, N), float("nan"), dtype=tdt, device="cuda")
        rc = fn(fmt, M, N, K, A.data_ptr(), As.data_ptr(), B.data_ptr(), Bs.data_ptr(),
                C.data_ptr(), out, s)
        assert rc == 0, mxg.strerror(rc)
        torch.cuda.synchronize()
        res.append(C)
    return res


@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
def test_noalloc_matches_mx_gemm_twice(fmt):
    """A split-K shape and then a smaller one (fewer planes, a smaller plane):
    each equals mx_gemm bit for bit and meets the oracle's bound."""
    for i, (M, N, K, out) in enumerate([(130, 520, 8192, mxinputs.OUT_BF16),
                                        (40, 200, 4608, mxinputs.OUT_FP32)]):
        p = mxg.plan(fmt, M, N, K, out)
        assert p["split_k"] > 1 and 0 < p["workspace_bytes"] <= mxg.NOALLOC_SCRATCH_BYTES, p
        case = mxinputs.make_random(fmt, M, N, K, seed=900 + 10 * i + fmt)
        case["fmt"] = fmt
        log("noalloc call %d fmt=%d M=%d N=%d K=%d split=%d" % (i, fmt, M, N, K, p["split_k"]))
        c_ref, c_na = _both(case, out)
        assert _bits_equal(c_ref, c_na)
        Cref, T = oracle.gemm(fmt, case["A"], case["A_scale"], case["B"], case["B_scale"], K)[:2]
        res = acceptance(host64(c_na), Cref, T, out == mxinputs.OUT_BF16,
                         what="noalloc call %d" % i)
        assert res["n_bad"] == 0, res


def _bits_equal(a, b):
    import torch
    it = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return bool(torch.equal(a.view(it), b.view(it)))


def test_noalloc_unsplit_problem():
    """A problem the plan does not split uses no scratch at all."""
    M, N, K = 512, 512, 1024
    p = mxg.plan(E2M1, M, N, K, mxinputs.OUT_FP32)
    assert p["split_k"] == 1, p
    case = mxinputs.make_random(E2M1, M, N, K, seed=77)
    case["fmt"] = E2M1
    c_ref, c_na = _both(case, mxinputs.OUT_FP32)
    assert _bits_equal(c_ref, c_na)
