"""GPU parity of mx_quantize (through the C ABI) against the CPU oracle's
quantizer: every code byte and every scale byte equal."""
import numpy as np
import pytest

import microscaled_block_scaled_amd as mxg
import mxinputs
import oracle
from gpu_util import log

pytestmark = pytest.mark.gpu

E2M1, E4M3, E5M2 = mxinputs.FMT_E2M1, mxinputs.FMT_E4M3, mxinputs.FMT_E5M2
E2M3, E3M2 = mxinputs.FMT_E2M3, mxinputs.FMT_E3M2
FMTS = [E2M1, E4M3, E5M2, E2M3, E3M2]
FMT_IDS = ["e2m1", "e4m3", "e5m2", "e2m3", "e3m2"]


def _gpu(x, fmt):
    import torch
    q, qs = mxg.mx_quantize(x, fmt)
    torch.cuda.synchronize()
    return q.cpu().numpy(), qs.cpu().numpy()


def _check(x, fmt, what):
    q, qs = _gpu(x, fmt)
    rq, rs = oracle.quantize(fmt, x.float().cpu().numpy().astype(np.float64))
    bad_s = np.argwhere(qs != rs)
    bad_q = np.argwhere(q != rq)
    assert len(bad_s) == 0, "%s: %d scale bytes differ, first at %s (gpu %d, oracle %d)" % (
        what, len(bad_s), bad_s[0], qs[tuple(bad_s[0])], rs[tuple(bad_s[0])])
    assert len(bad_q) == 0, "%s: %d code bytes differ, first at %s (gpu %#x, oracle %#x)" % (
        what, len(bad_q), bad_q[0], q[tuple(bad_q[0])], rq[tuple(bad_q[0])])


def _random(rows, K, seed, dtype):
    import torch
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, K)) * np.exp2(rng.integers(-40, 40, (rows, 1)))
    x[:, :32] *= (rng.random((rows, 1)) < 0.2)          # some all-zero blocks
    t = torch.from_numpy(x.astype(np.float32))
    return t.to(dtype).cuda()


SHAPES = [(1, 32), (3, 96), (17, 4128), (256, 4096), (1000, 128)]


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
@pytest.mark.parametrize("rows,K", SHAPES)
def test_quantize_random(fmt, dtype, rows, K):
    import torch
    x = _random(rows, K, rows * 31 + K, getattr(torch, dtype))
    log("quantize fmt=%d %s rows=%d K=%d" % (fmt, dtype, rows, K))
    _check(x, fmt, "random")


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_quantize_edge_values(fmt, dtype):
    """Ties after scaling, saturation, negative zero, values rounding to zero
    with either sign, FP32 and BF16 subnormal and huge block maxima, and
    blocks holding a NaN or an infinity."""
    import torch
    top = {E2M1: 6.0, E4M3: 448.0, E5M2: 57344.0, E2M3: 7.5, E3M2: 28.0}[fmt]
    if fmt in (E2M3, E3M2):                 # the 32 FP6 magnitudes by code
        grid = np.asarray(mxinputs._fp6_magnitudes(fmt), np.float64)
    elif fmt == E2M1:
        grid = oracle.tables()[0][:8]
    elif fmt == E4M3:
        grid = np.abs(oracle.tables()[1][:127])
    else:                                   # E5M2 codes 0 .. 123 are the finite magnitudes
        grid = np.array([oracle.default().e5m2_value(c) for c in range(124)])
    g = np.unique(np.abs(grid[np.isfinite(grid)]))
    mids = (g[1:] + g[:-1]) / 2
    vals = np.concatenate([g, mids, -mids, [-0.0, -1e-3, 1e-3, top * 1.06, -top * 1.12]])
    rows = []
    for block_max in (top, top * 2.0 ** -100, top * 2.0 ** 60, top * 2.0 ** -140):
        v = np.concatenate([vals, np.zeros(-len(vals) % 31)]).reshape(-1, 31)
        blocks = np.concatenate([np.full((len(v), 1), block_max), v * (block_max / top)], axis=1)
        rows.append(blocks.reshape(-1))
    n = max(128, max(len(r) for r in rows))
    n += -n % 32
    X = np.zeros((len(rows) + 3, n))
    for i, r in enumerate(rows):
        X[i, :len(r)] = r
    X[-3, 40] = np.nan
    X[-2, 70] = np.inf
    X[-1, 5] = -np.inf
    X[-1, 33] = 2.0 ** -133            # a subnormal block maximum (exact in FP32 and BF16)
    x = torch.from_numpy(X.astype(np.float32)).to(getattr(torch, dtype)).cuda()
    log("quantize edge values fmt=%d %s" % (fmt, dtype))
    _check(x, fmt, "edge values")


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_quantize_full_size(fmt):
    """The 8B-Llama fused-QKV operands (2048 + 6144 rows, K = 4096) from FP32.
    The FP6 formats store 3 (FP32 input) or 6 (BF16 input) bytes per lane;
    both are run here at full size."""
    import torch
    x = _random(8192, 4096, 99 + fmt, torch.float32)
    log("quantize full size fmt=%d" % fmt)
    _check(x, fmt, "full size")
    if fmt in (E2M3, E3M2):
        _check(x.to(torch.bfloat16), fmt, "full size bf16")


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_quantize_then_gemm(fmt):
    """Operands quantized on the GPU feed mx_gemm directly."""
    import torch
    from gpu_util import acceptance, check_against_oracle
    a = _random(300, 1024, 5, torch.float32)
    b = _random(200, 1024, 6, torch.bfloat16)
    qa, sa = mxg.mx_quantize(a, fmt)
    qb, sb = mxg.mx_quantize(b, fmt)
    C = mxg.mx_gemm(qa, sa, qb, sb, fmt, out_dtype=torch.float32)
    torch.cuda.synchronize()
    case = dict(fmt=fmt, M=300, N=200, K=1024, A=qa.cpu().numpy(), A_scale=sa.cpu().numpy(),
                B=qb.cpu().numpy(), B_scale=sb.cpu().numpy())
    if fmt in (E2M3, E3M2):
        # FP6: judged with the oracle's group term E, as the FP6 GEMM tests do
        Cref, T, E = oracle.gemm(fmt, case["A"], case["A_scale"], case["B"], case["B_scale"],
                                 1024, group_bound=True)
        res = acceptance(C.double().cpu().numpy(), Cref, T, False, E, what="quantize then gemm")
    else:
        res, *_ = check_against_oracle(case, mxinputs.OUT_FP32, C=C)
    assert res["n_bad"] == 0, res
