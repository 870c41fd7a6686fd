"""GPU parity of the decode kernel (M <= 32 rows; one workgroup per 32
columns of C, its four waves on four K-ranges, partial tiles added in LDS)
against the oracle, through the C ABI: every pair of E2M1, E4M3 and E5M2
on ragged shapes (short last periods, half E2M1 slabs, waves with empty
K-ranges, N tails), every M from 1 to 32 (also for the 8-bit x E2M1 pairs,
whose M <= 16 runs the wide slabs), more column groups than workgroups,
exact integers, NaN rows,
stores confined to C, the plan's shapes equal to the forced kernel bit for
bit, repeatability, and the no-allocation entry point.

Acceptance as for the other formats: |gpu - C| <= 1e-5 * T (+ one bf16 ulp
of C for BF16 output) + E, the oracle's 8-product group-alignment term
(non-zero only for E5M2 and mixed pairs)."""
import ctypes

import numpy as np
import pytest

import microscaled_block_scaled_amd as mxg
import mxinputs
import oracle
from gpu_util import acceptance, host64, log

pytestmark = pytest.mark.gpu

E2M1, E4M3, E5M2 = mxinputs.FMT_E2M1, mxinputs.FMT_E4M3, mxinputs.FMT_E5M2
F32, BF16 = mxinputs.OUT_FP32, mxinputs.OUT_BF16
FORMATS = [E2M1, E4M3, E5M2]
NAMES = {E2M1: "e2m1", E4M3: "e4m3", E5M2: "e5m2"}
PAIRS = [(a, b) for a in FORMATS for b in FORMATS]
PAIR_IDS = ["%s_%s" % (NAMES[a], NAMES[b]) for a, b in PAIRS]
DECODE = (mxg.DECODE_TILE, mxg.DECODE_TILE)


def _case(fa, fb, M, N, K, seed):
    ca = mxinputs.make_random(fa, M, 1, K, seed=seed)
    cb = mxinputs.make_random(fb, 1, N, K, seed=seed + 1)
    return dict(fa=fa, fb=fb, M=M, N=N, K=K, A=ca["A"], A_scale=ca["A_scale"],
                B=cb["B"], B_scale=cb["B_scale"])


def _dev(case):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(case[k])).cuda()
            for k in ("A", "A_scale", "B", "B_scale")]


def _run(case, out, tile=DECODE, d=None, stream=None):
    import torch
    d = d or _dev(case)
    tdt = torch.float32 if out == F32 else torch.bfloat16
    C = mxg.mx_gemm(d[0], d[1], d[2], d[3], case["fa"], out_dtype=tdt, tile=tile,
                    fmt_b=case["fb"], stream=stream)
    torch.cuda.synchronize()
    return C


def _check(case, out, C, what=""):
    Cref, T, E = oracle.gemm(case["fa"], case["A"], case["A_scale"], case["B"],
                             case["B_scale"], case["K"], group_bound=True, fmt_b=case["fb"])
    r = acceptance(host64(C), Cref, T, out == BF16, E, what=what)
    assert r["n_bad"] == 0, "%s: %d bad, worst ratio %.3g at %s" % (
        what, r["n_bad"], r["max_ratio"], r["first_bad"])


# K: one period, a short second period in wave 1 (waves 2 and 3 empty), 13
# periods of 128 with a half E2M1 slab and a short last period, 25 with one,
# a ragged 9 + 3 split, and ranges of several periods per wave with a short
# tail of 128 or 384.
SHAPES = [(1, 1, 512), (32, 203, 640), (5, 100, 1664), (17, 64, 3200), (3, 40, 1152),
          (32, 96, 8192 + 384), (2, 33, 4096 + 128)]


@pytest.mark.parametrize("fa,fb", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("out", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_decode_pairs(fa, fb, out, M, N, K):
    log("decode pair fa=%d fb=%d out=%d M=%d N=%d K=%d" % (fa, fb, out, M, N, K))
    case = _case(fa, fb, M, N, K, seed=M * 7 + N + K + 10 * fa + fb)
    _check(case, out, _run(case, out), what="decode pair")


@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
def test_decode_every_m(fmt):
    """Every row count 1 .. 32: rows past M are neither fetched nor stored,
    and each row's result lands in its own row of C."""
    N, K = 300, 2560
    for M in range(1, 33):
        log("decode every M fmt=%d M=%d N=%d K=%d" % (fmt, M, N, K))
        case = _case(fmt, fmt, M, N, K, seed=500 + M)
        _check(case, F32, _run(case, F32), what="every M, M=%d" % M)


@pytest.mark.parametrize("fa", [E4M3, E5M2], ids=["e4m3", "e5m2"])
def test_decode_w4a8_every_m(fa):
    """An 8-bit A with an E2M1 B, every row count 1 .. 32: M <= 16 runs the
    wide slabs (256 K-values, 8 or 16 A rows staged), larger M the 128-K slabs.
    K = 3200: a short last period and a half wide slab in the last wave."""
    N, K = 140, 3200
    for M in range(1, 33):
        log("decode w4a8 every M fa=%d M=%d N=%d K=%d" % (fa, M, N, K))
        case = _case(fa, E2M1, M, N, K, seed=550 + M)
        _check(case, BF16, _run(case, BF16), what="w4a8 every M, M=%d" % M)


@pytest.mark.parametrize("fa,fb", [(E2M1, E2M1), (E4M3, E4M3), (E4M3, E2M1)],
                         ids=["e2m1", "e4m3", "w4a8"])
@pytest.mark.parametrize("M,N,K", [(5, 20000, 1664), (32, 9000, 640), (8, 16417, 4224),
                                   (13, 16417, 3200)])
def test_decode_many_groups(fa, fb, M, N, K):
    """More column groups than workgroups (at most 256): each workgroup's
    copy stream runs on from one group into the next (2 to 3 groups each
    here, the last one ragged), and every element matches the oracle."""
    log("decode many groups fa=%d fb=%d M=%d N=%d K=%d" % (fa, fb, M, N, K))
    case = _case(fa, fb, M, N, K, seed=M + N + K + fa)
    _check(case, BF16, _run(case, BF16), what="many groups")


@pytest.mark.parametrize("fmt", FORMATS, ids=[NAMES[f] for f in FORMATS])
def test_decode_exact_integers(fmt):
    """Small integer elements with scale 2^0: every partial sum is an exact
    FP32 integer, so the kernel's four K-ranges and their sum in LDS equal
    numpy's int64 product bit for bit."""
    M, N, K = 32, 200, 8192
    rng = np.random.default_rng(600 + fmt)
    case = _case(fmt, fmt, M, N, K, seed=600 + fmt)
    if fmt == E2M1:
        codes = np.array([0x0, 0x2, 0x4, 0x5, 0x6], np.uint8)            # 0, 1, 2, 3, 4
        ia = rng.integers(0, 5, size=(M, K))
        ib = rng.integers(0, 5, size=(N, K))
        pack = lambda x: (codes[x[:, 0::2]] | (codes[x[:, 1::2]] << 4)).astype(np.uint8)
        case["A"], case["B"] = pack(ia), pack(ib)
    else:
        codes = (np.array([0x00, 0x38, 0x40, 0x44, 0x48], np.uint8) if fmt == E4M3 else
                 np.array([0x00, 0x3C, 0x40, 0x42, 0x44], np.uint8))     # 0, 1, 2, 3, 4
        ia = rng.integers(0, 5, size=(M, K))
        ib = rng.integers(0, 5, size=(N, K))
        case["A"], case["B"] = codes[ia], codes[ib]
    case["A_scale"] = np.full((M, K // 32), 127, np.uint8)
    case["B_scale"] = np.full((N, K // 32), 127, np.uint8)
    want = (ia.astype(np.int64) @ ib.astype(np.int64).T).astype(np.float64)
    _check(case, F32, _run(case, F32), what="exact integers")
    assert np.array_equal(host64(_run(case, F32)), want)


def test_decode_nan_scale_poisons_its_row_only():
    """A scale byte of 255 (NaN) in one block of A row 3 makes row 3 of C
    NaN and nothing else; in B row 70, column 70 only."""
    M, N, K = 8, 130, 4096
    case = _case(E4M3, E4M3, M, N, K, seed=700)
    case["A_scale"] = case["A_scale"].copy()
    case["B_scale"] = case["B_scale"].copy()
    case["A_scale"][3, 77] = 255
    case["B_scale"][70, 120] = 255
    C = host64(_run(case, F32))
    nan = np.isnan(C)
    assert nan[3].all() and nan[:, 70].all()
    assert nan.sum() == N + M - 1
    _check(case, F32, _run(case, F32), what="NaN scale")


@pytest.mark.parametrize("out", [F32, BF16], ids=["f32", "bf16"])
def test_decode_stores_only_into_c(out):
    """C handed over inside a larger buffer filled with a marker: every
    element of C is written, and nothing beyond it (N = 203: the last
    workgroup has 11 columns; M = 7)."""
    import torch
    M, N, K = 7, 203, 1024
    case = _case(E2M1, E2M1, M, N, K, seed=800)
    d = _dev(case)
    tdt = torch.float32 if out == F32 else torch.bfloat16
    buf = torch.full((M * N + 4096,), -12288.0, dtype=tdt, device="cuda")
    rc = mxg.gemm_ptr(E2M1, M, N, K, d[0].data_ptr(), d[1].data_ptr(), d[2].data_ptr(),
                      d[3].data_ptr(), buf.data_ptr(), out, 0, DECODE, 0, E2M1)
    torch.cuda.synchronize()
    assert rc == mxg.MX_OK
    assert bool((buf[M * N:] == -12288.0).all())
    C = buf[:M * N].view(M, N)
    assert not bool((C == -12288.0).any())
    _check(case, out, C, what="stores")


@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
def test_decode_plan_is_the_decode_kernel(fmt):
    """The 70B down projection at batch 8: the plan runs the decode kernel
    (mx_gemm equals the forced decode tile bit for bit), ten calls give one
    result, on the default and on a side stream, and sampled columns match
    the oracle."""
    import torch
    M, N, K = 8, 8192, 28672
    p = mxg.plan(fmt, M, N, K)
    assert p["variant"] == mxg.VARIANT_DECODE, p
    case = _case(fmt, fmt, M, N, K, seed=900 + fmt)
    d = _dev(case)
    log("decode plan fmt=%d M=%d N=%d K=%d plan=%s" % (fmt, M, N, K, p))
    first = _run(case, BF16, tile=None, d=d)
    assert torch.equal(first, _run(case, BF16, tile=DECODE, d=d))
    for _ in range(9):
        assert torch.equal(first, _run(case, BF16, tile=None, d=d))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        C2 = _run(case, BF16, tile=None, d=d, stream=s.cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(first, C2)
    cols = np.unique(np.r_[0:40, 4090:4110, np.linspace(0, N - 1, 200).astype(int), N - 40:N])
    sub = dict(case, B=case["B"][cols], B_scale=case["B_scale"][cols], N=len(cols))
    _check(sub, BF16, first[:, torch.from_numpy(cols).cuda()], what="plan columns")


@pytest.mark.parametrize("fa,fb", [(E4M3, E2M1), (E2M1, E2M1)], ids=["w4a8", "e2m1"])
def test_decode_gateup_full_size(fa, fb):
    """The 70B gate and up projections at batch 8 (8 x 57344 x 8192): 1792
    column groups, 7 per workgroup, so every wave's copy stream runs through
    seven groups.  The plan runs the decode kernel; the columns of the first,
    second and last group of the first and last workgroup, and 200 spread
    over the rest, match the oracle; a second call is bit-identical."""
    import torch
    M, N, K = 8, 57344, 8192
    p = mxg.plan(fa, M, N, K)
    assert p["variant"] == mxg.VARIANT_DECODE and p["workgroups"] == 256, p
    case = _case(fa, fb, M, N, K, seed=1200 + fa)
    d = _dev(case)
    log("decode gate-up fa=%d fb=%d M=%d N=%d K=%d plan=%s" % (fa, fb, M, N, K, p))
    first = _run(case, BF16, tile=None, d=d)
    assert torch.equal(first, _run(case, BF16, tile=None, d=d))
    groups = [0, 256, 1536, 255, 511, 1791]
    cols = np.unique(np.r_[np.concatenate([np.arange(32 * g, 32 * g + 32) for g in groups]),
                           np.linspace(0, N - 1, 200).astype(int)])
    sub = dict(case, B=case["B"][cols], B_scale=case["B_scale"][cols], N=len(cols))
    _check(sub, BF16, first[:, torch.from_numpy(cols).cuda()], what="gate-up columns")


@pytest.mark.parametrize("fa", [E4M3, E5M2], ids=["e4m3", "e5m2"])
def test_decode_w4a8_plan_at_m32(fa):
    """An 8-bit A with an E2M1 B at 32 rows and long K: the plan takes the
    decode kernel's 32-row wide slabs (the M > 16 limit of the other pairs
    does not apply), equal to the forced decode tile bit for bit, and
    sampled columns match the oracle."""
    import torch
    M, N, K = 32, 8192, 28672
    case = _case(fa, E2M1, M, N, K, seed=1300 + fa)
    d = _dev(case)
    log("decode w4a8 plan fa=%d M=%d N=%d K=%d" % (fa, M, N, K))
    planned = _run(case, BF16, tile=None, d=d)
    assert torch.equal(planned, _run(case, BF16, tile=DECODE, d=d))
    cols = np.unique(np.r_[0:40, np.linspace(0, N - 1, 120).astype(int), N - 40:N])
    sub = dict(case, B=case["B"][cols], B_scale=case["B_scale"][cols], N=len(cols))
    _check(sub, BF16, planned[:, torch.from_numpy(cols).cuda()], what="w4a8 plan columns")


def test_decode_noalloc_entry_matches():
    """mx_gemm_noalloc on a decode-planned shape (no scratch needed) equals
    mx_gemm bit for bit, twice, the second call smaller."""
    import torch
    L = mxg.lib()
    for M, N, K in ((16, 8192, 4096), (3, 8192, 2048)):
        assert mxg.plan(E4M3, M, N, K)["variant"] == mxg.VARIANT_DECODE
        case = _case(E4M3, E4M3, M, N, K, seed=1000 + M)
        d = _dev(case)
        C1 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        C2 = torch.empty_like(C1)
        args = [d[0].data_ptr(), d[1].data_ptr(), d[2].data_ptr(), d[3].data_ptr()]
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        assert L.mx_gemm(E4M3, M, N, K, *args, C1.data_ptr(), BF16, s) == mxg.MX_OK
        assert L.mx_gemm_noalloc(E4M3, M, N, K, *args, C2.data_ptr(), BF16, s) == mxg.MX_OK
        torch.cuda.synchronize()
        assert torch.equal(C1, C2)
