"""The split-K workspace path of mx_gemm on the GPU: an allocation failure
(forced through the library's test hook) is reported as MX_ERR_ALLOC with
nothing launched, and the next call works."""
import numpy as np
import pytest

import microscaled_block_scaled_amd as mxg
import mxinputs
import oracle
from gpu_util import acceptance, host64, log

pytestmark = pytest.mark.gpu


def test_allocation_failure_reports_alloc_error():
    import torch
    M, N, K, fmt, out = 64, 256, 8192, mxinputs.FMT_E2M1, mxinputs.OUT_FP32
    assert mxg.plan(fmt, M, N, K, out)["split_k"] > 1
    case = mxinputs.make_random(fmt, M, N, K, seed=5)
    A, As, B, Bs = (torch.from_numpy(np.ascontiguousarray(case[k])).cuda()
                    for k in ("A", "A_scale", "B", "B_scale"))
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    args = (fmt, M, N, K, A.data_ptr(), As.data_ptr(), B.data_ptr(), Bs.data_ptr(),
            C.data_ptr(), out, s)
    mxg.debug_fail_allocations(1)
    try:
        assert mxg.gemm_ptr(*args) == mxg.MX_ERR_ALLOC
        torch.cuda.synchronize()
        assert torch.isnan(C).all(), "a failed call launched a kernel"
        assert mxg.gemm_ptr(*args) == 0
    finally:
        mxg.debug_fail_allocations(0)
    torch.cuda.synchronize()
    Cref, T = oracle.gemm(fmt, case["A"], case["A_scale"], case["B"], case["B_scale"], K)[:2]
    res = acceptance(host64(C), Cref, T, False, what="after an allocation failure")
    log("allocation failure then success: %s" % res)
    assert res["n_bad"] == 0, res
