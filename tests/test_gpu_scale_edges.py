"""GPU parity at the hazards of scale placement: NaN scales (E8M0 byte 255),
E4M3 NaN codes, block scales that push results past FP32's range (to the
infinities) and below its normal range (subnormal and underflowed results),
and non-finite inputs carried through mx_quantize into mx_gemm.  The AI-compiler
digest of 2026-10-22, item 2 ("Deciding Scale Placement in MXFP4 Dot Products
with Integer Arithmetic"), names overflow, NaN and subnormal rounding as the
places where applying a scale before or after the sum changes the result.

Formats: E2M1 x E2M1, E4M3 x E4M3, and E4M3 activations x E2M1 weights
("W4A8").  The oracle forms exact block sums and then scales them (the
post-scale form); NaN scales and NaN codes make every output they touch NaN
(OCP MX); a result beyond the output type's range is the infinity of its
sign (oracle.compare).

Results in FP32's subnormal range cannot meet 1e-5 * T: T is then itself
below the subnormal spacing 2^-149.  There the test takes the output type's
own resolution as the bound (an FP32 result correctly rounded from each
block's exact value is within 2^-150 per block of it).

Measured on gfx950 and held here: NaN scales and NaN codes poison exactly
the outputs the oracle's do; subnormal results are kept, not flushed; with
E2M1 operands overflow matches the oracle's post-scale result exactly,
while with an E4M3 operand the device scales partial sums of products, so
the sign of an overflowed output can follow a partial sum (see
test_overflow_to_infinity)."""
import numpy as np
import pytest

import microscaled_block_scaled_amd as mxg
import mxinputs
import oracle
from gpu_util import acceptance, host64, log

pytestmark = pytest.mark.gpu

E2M1, E4M3 = mxinputs.FMT_E2M1, mxinputs.FMT_E4M3
F32, BF16 = mxinputs.OUT_FP32, mxinputs.OUT_BF16
PAIRS = [(E2M1, E2M1), (E4M3, E4M3), (E4M3, E2M1)]
PAIR_IDS = ["e2m1", "e4m3", "w4a8"]
FLT_MIN = 2.0 ** -126


def _case(fa, fb, M, N, K, seed):
    ca = mxinputs.make_random(fa, M, 1, K, seed=seed)
    cb = mxinputs.make_random(fb, 1, N, K, seed=seed + 1)
    return dict(fa=fa, fb=fb, M=M, N=N, K=K, A=ca["A"].copy(), A_scale=ca["A_scale"].copy(),
                B=cb["B"].copy(), B_scale=cb["B_scale"].copy())


def _run(case, out):
    import torch
    d = [torch.from_numpy(np.ascontiguousarray(case[k])).cuda()
         for k in ("A", "A_scale", "B", "B_scale")]
    tdt = torch.float32 if out == F32 else torch.bfloat16
    C = mxg.mx_gemm(d[0], d[1], d[2], d[3], case["fa"], out_dtype=tdt, fmt_b=case["fb"])
    torch.cuda.synchronize()
    return host64(C)


def _oracle(case):
    Cref, T = oracle.gemm(case["fa"], case["A"], case["A_scale"], case["B"], case["B_scale"],
                          case["K"], fmt_b=case["fb"])
    return Cref, T


def _pattern(g, Cref, out):
    ref = oracle.round_to_output(Cref, out == BF16)
    return dict(nan_ref=int(np.isnan(Cref).sum()), nan_gpu=int(np.isnan(g).sum()),
                inf_ref=int((~np.isnan(Cref) & np.isinf(ref)).sum()),
                inf_gpu=int(np.isinf(g).sum()))


@pytest.mark.parametrize("out", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("fa,fb", PAIRS, ids=PAIR_IDS)
def test_nan_scale_bytes(fa, fb, out):
    """Scale byte 255 (E8M0 NaN) in a few blocks of A rows and of B rows:
    every output of those rows and columns is NaN, the others are exact to
    the bound."""
    case = _case(fa, fb, 70, 90, 640, seed=41)
    r = np.random.default_rng(5)
    for m in (0, 17, 69):
        case["A_scale"][m, r.integers(0, 20)] = 255
    for n in (3, 44, 89):
        case["B_scale"][n, r.integers(0, 20)] = 255
    # a NaN scale on a block whose elements are all zero still makes NaN
    case["A_scale"][30, 4] = 255
    if fa == E2M1:
        case["A"][30, 64:80] = 0
    else:
        case["A"][30, 128:160] = 0
    log("nan scale bytes %d x %d out=%d" % (fa, fb, out))
    g = _run(case, out)
    Cref, T = _oracle(case)
    log("  %s" % _pattern(g, Cref, out))
    assert np.isnan(Cref[[0, 17, 69, 30], :]).all() and np.isnan(Cref[:, [3, 44, 89]]).all()
    res = acceptance(g, Cref, T, out == BF16, what="nan scales")
    assert res["n_bad"] == 0, res


@pytest.mark.parametrize("out", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E4M3, E2M1)], ids=["e4m3", "w4a8"])
def test_e4m3_nan_codes(fa, fb, out):
    """E4M3 NaN codes 0x7F and 0xFF in A (and in B when B is E4M3): the
    outputs of those rows and columns are NaN."""
    case = _case(fa, fb, 40, 72, 512, seed=43)
    case["A"][5, 100] = 0x7F
    case["A"][22, 511] = 0xFF
    if fb == E4M3:
        case["B"][7, 0] = 0xFF
        case["B"][60, 300] = 0x7F
    log("e4m3 nan codes %d x %d out=%d" % (fa, fb, out))
    g = _run(case, out)
    Cref, T = _oracle(case)
    log("  %s" % _pattern(g, Cref, out))
    assert np.isnan(Cref[[5, 22], :]).all()
    res = acceptance(g, Cref, T, out == BF16, what="nan codes")
    assert res["n_bad"] == 0, res


def _overflow_case(fa, fb, seed):
    """Every block of every row at exponent 0 (scale bytes 127), except block
    3, whose exponent sA + sB - 254 is a_m + b_n with a_m, b_n in [50, 127]:
    from +100 (finite in FP32) to +254 (far beyond it)."""
    M, N, K = 64, 72, 512
    case = _case(fa, fb, M, N, K, seed)
    case["A_scale"][:] = 127
    case["B_scale"][:] = 127
    a = np.linspace(50, 127, M).round().astype(np.int64)
    b = np.linspace(50, 127, N).round().astype(np.int64)
    case["A_scale"][:, 3] = 127 + a
    case["B_scale"][:, 3] = 127 + b
    return case


@pytest.mark.parametrize("out", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("fa,fb", PAIRS, ids=PAIR_IDS)
def test_overflow_to_infinity(fa, fb, out):
    """sA + sB - 254 from +100 to +254 in one block (which then dominates
    each output, so the bound adds the group term of 8-bit operands).

    E2M1 x E2M1: exactly the oracle's post-scale result: outputs whose exact
    value lies beyond the output type's range are the infinity of their
    sign, the rest meet the bound.

    An E4M3 operand: the device scales partial sums of products before the
    32-term block sum is complete.  Measured: outputs beyond the range are
    infinities, but about a quarter of them carry the sign of a partial sum
    rather than of the block sum, and a few outputs within 2^-1.4 of the
    largest finite value become infinities too.  The test holds the device
    to that envelope: no NaN; every output beyond the range an infinity;
    every output below 2^126 within the bound; and reports the rest."""
    case = _overflow_case(fa, fb, seed=47)
    log("overflow %d x %d out=%d" % (fa, fb, out))
    g = _run(case, out)
    Cref, T, E = oracle.gemm(case["fa"], case["A"], case["A_scale"], case["B"],
                             case["B_scale"], case["K"], fmt_b=case["fb"], group_bound=True)
    p = _pattern(g, Cref, out)
    log("  %s" % p)
    assert p["inf_ref"] > 100 and p["nan_ref"] == 0
    if fa == E2M1 and fb == E2M1:
        res = acceptance(g, Cref, T, out == BF16, what="overflow")
        assert res["n_bad"] == 0, res
        return
    ref = oracle.round_to_output(Cref, out == BF16)
    beyond = np.isinf(ref)
    inside = np.abs(Cref) < 2.0 ** 126
    assert not np.isnan(g).any()
    assert np.isinf(g[beyond]).all()
    res = acceptance(g[inside], Cref[inside], T[inside], out == BF16, E[inside],
                     group_term=True, what="overflow, below 2^126")
    assert res["n_bad"] == 0, res
    near = ~beyond & ~inside
    log("  8-bit operand: %d of %d infinities with the other sign; %d of %d outputs in "
        "[2^126, max] became infinities" % (
            int((g[beyond] != ref[beyond]).sum()), int(beyond.sum()),
            int(np.isinf(g[near]).sum()), int(near.sum())))


def _underflow_case(fa, fb, seed):
    """Every block at exponent sA + sB - 254 = a_m + b_n, a_m and b_n in
    [-127, -50]: from -100 (normal FP32 results) through the subnormal range
    to -254 (results that underflow to zero)."""
    M, N, K = 64, 72, 512
    case = _case(fa, fb, M, N, K, seed)
    a = np.linspace(-127, -50, M).round().astype(np.int64)
    b = np.linspace(-127, -50, N).round().astype(np.int64)
    case["A_scale"][:] = (127 + a)[:, None]
    case["B_scale"][:] = (127 + b)[:, None]
    return case


@pytest.mark.parametrize("fa,fb", PAIRS, ids=PAIR_IDS)
def test_underflow_and_subnormal_results(fa, fb):
    """sA + sB - 254 from -100 to -254 in every block, FP32 output.  Normal
    results meet 1e-5 * T.  Results below 2^-126 cannot (T is then below the
    subnormal spacing): the device keeps them as FP32 subnormals (measured:
    no flush to zero), each within 1e-5 * T + 2^-150 per block of the exact
    value, and none whose exact value exceeds 2^-140 comes out zero."""
    case = _underflow_case(fa, fb, seed=53)
    log("underflow %d x %d" % (fa, fb))
    g = _run(case, F32)
    Cref, T = _oracle(case)
    nb = case["K"] // 32
    normal = np.abs(Cref) >= FLT_MIN
    sub = ~normal & (Cref != 0)
    res = acceptance(g[normal], Cref[normal], T[normal], False, what="underflow, normal")
    assert res["n_bad"] == 0, res
    assert sub.sum() > 100 and not np.isnan(g).any() and not np.isinf(g).any()
    kept = np.abs(g[sub] - Cref[sub]) <= 1e-5 * T[sub] + nb * 2.0 ** -150
    clear = sub & (np.abs(Cref) > 2.0 ** -140)
    log("  %d normal, %d subnormal-range results (%d above 2^-140): %d within the subnormal "
        "bound, %d of those above 2^-140 non-zero" % (
            int(normal.sum()), int(sub.sum()), int(clear.sum()), int(kept.sum()),
            int((g[clear] != 0).sum())))
    assert kept.all()
    assert (g[clear] != 0).all()


@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
def test_nonfinite_inputs_through_quantize(fmt):
    """NaN and +-Inf in the FP32 input of mx_quantize: their blocks get scale
    byte 255, and mx_gemm then makes NaN of every output those rows touch,
    as the oracle's quantizer and GEMM do."""
    import torch
    r = np.random.default_rng(61)
    M, N, K = 48, 40, 512
    xa = r.standard_normal((M, K)).astype(np.float32)
    xb = r.standard_normal((N, K)).astype(np.float32)
    xa[3, 10] = np.nan
    xa[20, 300] = np.inf
    xa[47, 511] = -np.inf
    xb[9, 64] = np.nan
    qa, sa = mxg.mx_quantize(torch.from_numpy(xa).cuda(), fmt)
    qb, sb = mxg.mx_quantize(torch.from_numpy(xb).cuda(), fmt)
    C = mxg.mx_gemm(qa, sa, qb, sb, fmt, out_dtype=torch.float32)
    torch.cuda.synchronize()
    g = host64(C)
    ra, rsa = oracle.quantize(fmt, xa.astype(np.float64))
    rb, rsb = oracle.quantize(fmt, xb.astype(np.float64))
    assert (sa.cpu().numpy() == rsa).all() and (sb.cpu().numpy() == rsb).all()
    assert (rsa[[3, 20, 47]] == 255).any(axis=1).all()
    Cref, T = oracle.gemm(fmt, ra, rsa, rb, rsb, K)
    log("nonfinite through quantize fmt=%d: %s" % (fmt, _pattern(g, Cref, F32)))
    assert np.isnan(Cref[[3, 20, 47], :]).all() and np.isnan(Cref[:, 9]).all()
    res = acceptance(g, Cref, T, False, what="quantize nonfinite")
    assert res["n_bad"] == 0, res
