"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Acceptance per element: |gpu - C| <= 1e-5 * T for FP32 output, plus one bf16
ulp of C for BF16 output, with C and T from the oracle (T = sum |a_k b_k|).
One test only, built so that a large product shares its group of 8 with
small ones, adds the oracle's group-alignment term E: gfx950's block-scaled
MFMA adds each group of 8 E4M3 products after aligning them to the largest,
dropping bits more than 13 binades below it."""
import zlib

import numpy as np
import pytest

import microscaled_block_scaled_amd as mxg
import mxinputs
import oracle
from gpu_util import check_against_oracle, host64, log, run_gpu, sample_rows, to_dev

pytestmark = pytest.mark.gpu

E2M1, E4M3 = mxinputs.FMT_E2M1, mxinputs.FMT_E4M3
F32, BF16 = mxinputs.OUT_FP32, mxinputs.OUT_BF16


def _assert_ok(res, what):
    assert res["n_bad"] == 0, "%s: %d bad, worst ratio %.3g at %s" % (
        what, res["n_bad"], res["max_ratio"], res["first_bad"])


def test_small_workload_full():
    case = mxinputs.make_case("mxfp4_256")
    log("mxfp4_256 full")
    res, *_ = check_against_oracle(case, case["out"])
    _assert_ok(res, "mxfp4_256")


TAIL_SHAPES = [(1, 1, 128), (7, 33, 256), (16, 16, 384), (33, 255, 128),
               (255, 257, 384), (257, 129, 512), (130, 7, 640), (64, 300, 1152)]


@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
@pytest.mark.parametrize("out", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", TAIL_SHAPES)
def test_tails(fmt, out, M, N, K):
    case = mxinputs.make_random(fmt, M, N, K, seed=M * 7 + N + K)
    log("tails fmt=%d out=%d M=%d N=%d K=%d" % (fmt, out, M, N, K))
    # K = 128 is four blocks: the E4M3 group error is then not averaged over
    # many blocks, and the bound adds the oracle's group term (the only shape
    # of this test that needs it; logged per file at the end of the run)
    res, *_ = check_against_oracle(case, out, group_term=(fmt == E4M3 and K == 128),
                                   what="tails")
    _assert_ok(res, "tails")


SMALL_M_SHAPES = [(1, 32, 128), (8, 97, 1152), (32, 64, 3968), (33, 40, 640),
                  (64, 129, 2560), (17, 1000, 384), (8, 300, 9216)]


@pytest.mark.parametrize("tile", [None, (64, 256), (128, 128)], ids=["plan", "64x256", "128x128"])
@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
@pytest.mark.parametrize("out", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", SMALL_M_SHAPES)
def test_small_m(tile, fmt, out, M, N, K):
    """Small M runs the decode kernel (M <= 32, K >= 512, and for K > 8192
    also M <= 8 and enough columns) or a short tile, 128x128 or 64x256 (rows
    past M not fetched, never stored), with split-K when the grid is small
    and K long (the last shape): the plan's pick and each short tile forced,
    at its planned split."""
    p = mxg.plan(fmt, M, N, K, out)
    if p["variant"] == mxg.VARIANT_DECODE:
        assert M <= mxg.DECODE_TILE and K >= 512, p
    else:
        assert p["tile_m"] in (64, 128), p
    case = mxinputs.make_random(fmt, M, N, K, seed=1000 + M * 3 + N + K)
    log("small M fmt=%d out=%d M=%d N=%d K=%d tile=%s plan split=%d"
        % (fmt, out, M, N, K, tile, p["split_k"]))
    res, *_ = check_against_oracle(case, out, tile=tile)
    _assert_ok(res, "small M")


@pytest.mark.parametrize("tile", [(256, 256), (128, 128)], ids=["256x256", "128x128"])
@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
def test_tile_kernel_small_m(tile, fmt):
    """The tile kernel, forced, on a problem much shorter than one tile."""
    case = mxinputs.make_random(fmt, 5, 70, 640, seed=77 + fmt)
    log("tile kernel small M tile=%s fmt=%d" % (tile, fmt))
    res, *_ = check_against_oracle(case, BF16, tile=tile)
    _assert_ok(res, "tile kernel small M")


def _tile_ids():
    return ["%dx%d" % t for t in mxg.tile_shapes()]


@pytest.mark.parametrize("tile", mxg.tile_shapes(), ids=_tile_ids())
@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
@pytest.mark.parametrize("out", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("split", [1, 3], ids=["nosplit", "split3"])
def test_every_tile(tile, fmt, out, split):
    """Each kernel configuration, forced, on a ragged problem two tiles high
    and wide whose K walks several full main-loop trips and a partial one.
    E2M1 cases use an odd N (rows of C not 16-byte multiples: element-wise
    output stores), E4M3 cases an N that is a multiple of 8 (16-byte stores,
    with a partial last tile).  With split 3, K is cut into 3 slices of whole
    512-K periods, the last one short: E2M1 K = 4736 -> 2048 + 2048 + 640
    (ending in half a slab), E4M3 K = 2432 -> 1024 + 1024 + 384 (fewer than
    16 scale bytes per row)."""
    M, N = tile[0] + 37, tile[1] + (19 if fmt == E2M1 else 24)
    K = 4736 if fmt == E2M1 else 2432           # 37 / 19 x 128
    case = mxinputs.make_random(fmt, M, N, K, seed=tile[0] + tile[1] + fmt)
    log("every tile %s split=%d fmt=%d out=%d M=%d N=%d K=%d" % (tile, split, fmt, out, M, N, K))
    res, *_ = check_against_oracle(case, out, tile=tile, split_k=split)
    _assert_ok(res, "tile %s split %d" % (tile, split))


@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
@pytest.mark.parametrize("out", [F32, BF16], ids=["f32", "bf16"])
def test_split_k_planned(fmt, out):
    """A grid too small for the GPU with a long K: the plan splits K itself
    (4 slices of 2560 here, the last one 1152; ragged M and N)."""
    M, N, K = 130, 250, 8192 + 640
    p = mxg.plan(fmt, M, N, K, out)
    assert p["variant"] == mxg.VARIANT_TILE and p["split_k"] > 1, p
    case = mxinputs.make_random(fmt, M, N, K, seed=555 + fmt)
    log("split-K planned fmt=%d out=%d split=%d" % (fmt, out, p["split_k"]))
    res, *_ = check_against_oracle(case, out)
    _assert_ok(res, "split-K planned")


@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
def test_scale_extremes(fmt):
    # sa + sb - 254 spans [-100, 100]: every block result stays an FP32
    # normal.  Deliberately wide-range scales: one block dominates most
    # outputs, so for E4M3 the bound adds the oracle's group term.
    case = mxinputs.make_random(fmt, 70, 90, 512, seed=31, scale_lo=77, scale_hi=177)
    log("scale extremes fmt=%d" % fmt)
    res, *_ = check_against_oracle(case, F32, group_term=fmt == E4M3, what="scale extremes")
    _assert_ok(res, "scale extremes")


def _integer_pool(fmt, vmax):
    import oracle_pins
    t = oracle_pins.golden_e2m1()[:8] if fmt == E2M1 else oracle_pins.torch_e4m3()[:127]
    return [c for c in range(len(t)) if float(t[c]).is_integer() and t[c] <= vmax]


@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
def test_exact_integers(fmt):
    """All scales 2^0, integer elements, every partial sum an integer below
    2^24: FP32 accumulation is exact in any order, so the GPU must match the
    integer matmul bit for bit."""
    import oracle_pins
    K = 1024 if fmt == E2M1 else 512
    pool = _integer_pool(fmt, 6 if fmt == E2M1 else 16)
    A, As = mxinputs.random_codes(fmt, 96, K, 5, pool, tensor=0)
    B, Bs = mxinputs.random_codes(fmt, 80, K, 5, pool, tensor=1)
    case = dict(fmt=fmt, M=96, N=80, K=K, A=A, A_scale=As, B=B, B_scale=Bs)
    ia = oracle_pins.decode_rows(fmt, A).astype(np.int64)
    ib = oracle_pins.decode_rows(fmt, B).astype(np.int64)
    ref = (ia @ ib.T).astype(np.float64)
    log("exact integers fmt=%d" % fmt)
    g = host64(run_gpu(case, F32))
    assert np.array_equal(g, ref)


@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
def test_zero_and_onehot(fmt):
    K = 256
    rb = K // 2 if fmt == E2M1 else K
    A = np.zeros((20, rb), np.uint8)
    B = np.zeros((24, rb), np.uint8)
    As = np.full((20, K // 32), 140, np.uint8)
    Bs = np.full((24, K // 32), 90, np.uint8)
    case = dict(fmt=fmt, M=20, N=24, K=K, A=A, A_scale=As, B=B, B_scale=Bs)
    log("zeros fmt=%d" % fmt)
    assert not host64(run_gpu(case, F32)).any()
    k = 141
    if fmt == E2M1:
        A[17, k // 2] = 0x7 << 4          # odd k: high nibble; 6.0
        B[22, k // 2] = 0xB << 4          # -1.5
        va, vb = 6.0, -1.5
    else:
        A[17, k] = 0x7E                   # 448
        B[22, k] = 0x81                   # -2^-9
        va, vb = 448.0, -(2.0 ** -9)
    As[17, k // 32], Bs[22, k // 32] = 150, 60
    g = host64(run_gpu(case, F32))
    expect = np.zeros((20, 24))
    expect[17, 22] = va * vb * 2.0 ** (150 + 60 - 254)
    assert np.array_equal(g, expect)


def test_e4m3_group_alignment_is_bounded():
    """Rows built so that a large product shares its 8-group with many small
    ones: the GPU result may drop the small ones, and must stay within
    1e-5 * T + E of the exact result."""
    import oracle_pins
    K, M, N = 512, 48, 40
    r = np.random.default_rng(17)
    A = np.full((M, K), 0x38, np.uint8)                    # 1.0
    B = np.zeros((N, K), np.uint8)
    small = np.array([0x01, 0x08, 0x10, 0x20, 0x28, 0x81, 0x88], np.uint8)
    B[:] = small[r.integers(0, len(small), size=(N, K))]
    for g in range(K // 8):
        A[r.integers(0, M), 8 * g + r.integers(0, 8)] = 0x7E   # 448
        B[r.integers(0, N), 8 * g + r.integers(0, 8)] = 0x7E
    As = r.integers(120, 135, size=(M, K // 32)).astype(np.uint8)
    Bs = r.integers(120, 135, size=(N, K // 32)).astype(np.uint8)
    case = dict(fmt=E4M3, M=M, N=N, K=K, A=A, A_scale=As, B=B, B_scale=Bs)
    log("e4m3 group alignment")
    res, g, Cref, T, E = check_against_oracle(case, F32, group_term=True,
                                              what="e4m3 group alignment")
    _assert_ok(res, "e4m3 group alignment")
    # E models the hardware, it is not slack: somewhere the device's error
    # reaches at least half of it.
    err = np.abs(g - Cref)
    assert np.any((E > 0) & (err >= 0.5 * E)), "E is loose: max err/E %.3g" % float(
        np.max(np.where(E > 0, err / np.where(E > 0, E, 1.0), 0.0)))


@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
def test_bf16_is_rounded_fp32(fmt):
    """The BF16 output is the FP32 result rounded to nearest even."""
    import torch
    case = mxinputs.make_random(fmt, 200, 136, 768, seed=8)
    dev = to_dev(case)
    c32 = run_gpu(case, F32, dev)
    c16 = run_gpu(case, BF16, dev)
    assert torch.equal(c32.to(torch.bfloat16).view(torch.int16), c16.view(torch.int16))


@pytest.mark.parametrize("M", [300, 40], ids=["tall", "short"])
def test_deterministic_and_stream(M):
    import torch
    case = mxinputs.make_random(E4M3, M, 260, 4096, seed=12)
    dev = to_dev(case)
    c1 = run_gpu(case, F32, dev)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for _ in range(3):
            c2 = mxg.mx_gemm(dev["A"], dev["A_scale"], dev["B"], dev["B_scale"], E4M3,
                             out_dtype=torch.float32)
            s.synchronize()
            assert torch.equal(c1.view(torch.int32), c2.view(torch.int32))


FULL = ["mxfp8_llama8b_qkv", "mxfp4_llama8b_gateup_decode", "mxfp4_qwen32b_down",
        "mxfp8_llama70b_down_m8", "mxfp8_llama70b_down_m64",
        "mxfp8_llama70b_down_m256", "mxfp8_llama70b_down_m2048",
        "mxfp4_llama70b_down_m8", "mxfp4_llama70b_down_m64",
        "mxfp4_llama70b_down_m256", "mxfp4_llama70b_down_m2048"]


@pytest.mark.parametrize("name", FULL)
def test_full_workload_sampled(name):
    """Full-size workloads in the benchmark's launch configuration; the oracle
    checks a deterministic sample of rows (all columns)."""
    log("full workload %s: generating" % name)
    case = mxinputs.make_case(name)
    log("full workload %s: running" % name)
    rows = sample_rows(case["M"])
    res, *_ = check_against_oracle(case, case["out"], rows=rows, what=name)
    _assert_ok(res, name)


def _dequant(fmt, codes, scales):
    """float64 values of MX rows (E2M1 or E4M3), scale applied, from the
    oracle's pinned decode tables; element 2i of an E2M1 row in the low
    nibble of byte i."""
    t4, t8 = oracle.tables()
    if fmt == E2M1:
        v = np.empty((codes.shape[0], codes.shape[1] * 2), np.float64)
        v[:, 0::2] = t4[codes & 15]
        v[:, 1::2] = t4[codes >> 4]
    else:
        v = t8[codes]
    return v * np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)


def _projections(fmt, X, Xs, z, chunk=512):
    """(X^T z, |X|^T |z|) over the dequantized rows of X, in row chunks."""
    K = Xs.shape[1] * 32
    p, q = np.zeros(K), np.zeros(K)
    for r in range(0, X.shape[0], chunk):
        d = _dequant(fmt, X[r:r + chunk], Xs[r:r + chunk])
        p += d.T @ z[r:r + chunk]
        q += np.abs(d).T @ np.abs(z[r:r + chunk])
    return p, q


def _rows_times(fmt, X, Xs, v, chunk=512):
    """(X v, |X| v) over the dequantized rows of X."""
    out, outa = np.zeros(X.shape[0]), np.zeros(X.shape[0])
    for r in range(0, X.shape[0], chunk):
        d = _dequant(fmt, X[r:r + chunk], Xs[r:r + chunk])
        out[r:r + chunk] = d @ v[0]
        outa[r:r + chunk] = np.abs(d) @ v[1]
    return out, outa


@pytest.mark.parametrize("name", FULL)
def test_full_workload_projections(name):
    """Every element of a full-size result, in aggregate: for random x and y,
    C x and y^T C from the GPU against A (B^T x) and (y^T A) B^T from the
    dequantized operands in float64.  If every element meets its bound
    1e-5 * T (+ one BF16 ulp), then |(C_gpu x - C x)_m| <= sum_n (1e-5 T_mn
    + ulp_mn) |x_n|, and sum_n T_mn |x_n| = (|A| (|B|^T |x|))_m exactly, so
    each of the M + N projections is held to that bound.  A wrong tile, row,
    column or slice anywhere shows up, whichever rows the sampled test
    looked at."""
    case = mxinputs.make_case(name)
    fmt, M, N, out = case["fmt"], case["M"], case["N"], case["out"]
    log("projections %s: running" % name)
    g = host64(run_gpu(case, out))
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    x, y = rng.standard_normal(N), rng.standard_normal(M)
    bf16 = out == mxinputs.OUT_BF16
    ulp = oracle.bf16_ulp(g) if bf16 else np.zeros_like(g)
    # C x: A (B^T x), bound 1e-5 |A| (|B|^T |x|) + ulp |x|
    ref, lim = _rows_times(fmt, case["A"], case["A_scale"],
                           _projections(fmt, case["B"], case["B_scale"], x))
    got = g @ x
    bound = 1e-5 * lim + ulp @ np.abs(x) + 1e-12 * lim
    worst_rows = float(np.max(np.abs(got - ref) / np.maximum(bound, 1e-300)))
    # y^T C: B (A^T y), bound 1e-5 |B| (|A|^T |y|) + |y|^T ulp
    refc, limc = _rows_times(fmt, case["B"], case["B_scale"],
                             _projections(fmt, case["A"], case["A_scale"], y))
    gotc = y @ g
    boundc = 1e-5 * limc + np.abs(y) @ ulp + 1e-12 * limc
    worst_cols = float(np.max(np.abs(gotc - refc) / np.maximum(boundc, 1e-300)))
    log("  %s: worst |C x - ref| / bound %.3g over %d rows, columns %.3g over %d"
        % (name, worst_rows, M, worst_cols, N))
    assert worst_rows <= 1.0 and worst_cols <= 1.0, (worst_rows, worst_cols)
