"""Checks that pin the CPU oracle to facts outside itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with:
  * library routines: torch's float8_e4m3fn / float8_e8m0fnu decodings, and a
    numpy float64 matmul of dequantized operands;
  * hand-computed worked examples and the OCP E2M1 value list (tests/golden);
  * exact rational arithmetic (fractions.Fraction) on tiny inputs;
  * exact integer matmul when every scale is 2^0 and every element an integer;
  * invariants: a scale byte +k multiplies exactly its block's contribution
    by 2^k; swapping the operands transposes C bit for bit; zeros give zero;
    NaN scales and NaN elements poison exactly the outputs they touch.
The decode tables used here come from torch and the golden file, never from
the oracle.  tests/test_oracle_mutants.py plants mistakes in copies of the
oracle and checks that these pins catch each one.
"""
import math
import os
from fractions import Fraction

import numpy as np

import mxinputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
E2M1, E4M3, E5M2 = mxinputs.FMT_E2M1, mxinputs.FMT_E4M3, mxinputs.FMT_E5M2
E2M3, E3M2 = mxinputs.FMT_E2M3, mxinputs.FMT_E3M2


# --------------------------------------------------------------------------
# Independent decode tables (not the oracle's).

def golden_e2m1():
    vals = np.zeros(16, np.float64)
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                c, v = line.split()
                vals[int(c)] = float(v)
    return vals


def torch_e4m3():
    import torch
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def torch_e5m2():
    import torch
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).double().numpy()


def torch_e8m0():
    import torch
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()


def golden_fp6(fmt):
    """The 64 FP6 values by code, from the OCP value list (codes 0..31) and
    the sign bit (code | 32)."""
    name = "e2m3" if fmt == E2M3 else "e3m2"
    vals = np.zeros(64, np.float64)
    with open(os.path.join(GOLDEN, "%s_values.txt" % name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                c, v = line.split()
                vals[int(c)] = float(v)
                vals[int(c) | 32] = -float(v)
    return vals


def decode_rows(fmt, packed):
    """uint8 operand rows -> float64 values with the independent tables."""
    if fmt == E2M1:
        return golden_e2m1()[mxinputs.unpack_e2m1(packed)]
    if fmt in (E2M3, E3M2):
        return golden_fp6(fmt)[mxinputs.unpack_fp6(packed)]
    if fmt == E5M2:
        return torch_e5m2()[np.asarray(packed, np.uint8)]
    return torch_e4m3()[np.asarray(packed, np.uint8)]


def dequant(fmt, packed, scales):
    v = decode_rows(fmt, packed)
    e = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    return np.ldexp(v, e)


# --------------------------------------------------------------------------
def _same(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return a.shape == b.shape and bool(np.all((a == b) | (np.isnan(a) & np.isnan(b))))


def pin_e4m3_table(orc):
    _, t8 = orc.tables()
    assert _same(t8, torch_e4m3()), "E4M3 table differs from torch.float8_e4m3fn"
    for c in (0x01, 0x38, 0x7E, 0x7F, 0xFE, 0x80):
        v = orc.e4m3_value(c)
        assert _same(v, torch_e4m3()[c])


def pin_e2m1_table(orc):
    t4, _ = orc.tables()
    g = golden_e2m1()
    assert np.array_equal(t4, g), "E2M1 table differs from the OCP value list"
    assert all(np.signbit(t4[8:]))


def pin_e8m0(orc):
    ref = torch_e8m0()
    got = np.array([orc.e8m0_value(b) for b in range(256)])
    assert _same(got, ref), "E8M0 decode differs from torch.float8_e8m0fnu"


def _parse_bytes(tokens):
    out = []
    for t in tokens:
        if "*" in t:
            v, n = t.split("*")
            out += [int(v, 16)] * int(n)
        else:
            out.append(int(t, 16))
    return np.array(out, np.uint8)


def load_worked_example(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, *v = line.split()
                d[k] = v
    fmt = {"e2m1": E2M1, "e4m3": E4M3}[d["fmt"][0]]
    K = int(d["K"][0])
    A = _parse_bytes(d["a_row"])[None, :]
    B = _parse_bytes(d["b_row"])[None, :]
    As = np.array([int(x) for x in d["a_scale"]], np.uint8)[None, :]
    Bs = np.array([int(x) for x in d["b_scale"]], np.uint8)[None, :]
    assert A.shape[1] == (K // 2 if fmt == E2M1 else K)
    return fmt, K, A, As, B, Bs, Fraction(d["C"][0]), Fraction(d["T"][0])


def pin_worked_examples(orc):
    for name in ("worked_example_e2m1.txt", "worked_example_e4m3.txt"):
        fmt, K, A, As, B, Bs, Cx, Tx = load_worked_example(name)
        C, T = orc.gemm(fmt, A, As, B, Bs, K)
        assert C[0, 0] == float(Cx), (name, C[0, 0], float(Cx))
        assert T[0, 0] == float(Tx), (name, T[0, 0], float(Tx))


def _exact(fmt, A, As, B, Bs, K):
    """C and T as Fractions, from the definition, with independent tables."""
    va, vb = decode_rows(fmt, A), decode_rows(fmt, B)
    M, N, nb = A.shape[0], B.shape[0], K // 32
    C = [[Fraction(0)] * N for _ in range(M)]
    T = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            for b in range(nb):
                w = Fraction(2) ** (int(As[m, b]) + int(Bs[n, b]) - 254)
                p = sum(Fraction(float(va[m, j])) * Fraction(float(vb[n, j]))
                        for j in range(32 * b, 32 * b + 32))
                q = sum(abs(Fraction(float(va[m, j])) * Fraction(float(vb[n, j])))
                        for j in range(32 * b, 32 * b + 32))
                C[m][n] += w * p
                T[m][n] += w * q
    return C, T


def pin_bruteforce(orc):
    for fmt in (E2M1, E4M3):
        for seed, (M, N, K) in enumerate([(2, 3, 128), (3, 2, 256), (1, 4, 128)]):
            pool = range(8) if fmt == E2M1 else range(127)
            A, _ = mxinputs.random_codes(fmt, M, K, seed, pool, tensor=0)
            B, _ = mxinputs.random_codes(fmt, N, K, seed, pool, tensor=1)
            r = np.random.default_rng([7, seed, fmt])
            As = r.integers(100, 155, size=(M, K // 32)).astype(np.uint8)
            Bs = r.integers(100, 155, size=(N, K // 32)).astype(np.uint8)
            C, T = orc.gemm(fmt, A, As, B, Bs, K)
            Cx, Tx = _exact(fmt, A, As, B, Bs, K)
            nb = K // 32
            for m in range(M):
                for n in range(N):
                    tol = nb * 2.0 ** -52 * float(Tx[m][n])
                    assert abs(C[m, n] - float(Cx[m][n])) <= tol, (fmt, m, n)
                    assert abs(T[m, n] - float(Tx[m][n])) <= tol, (fmt, m, n)


def _integer_pool(fmt):
    """Magnitude codes whose value is an integer (found from the independent
    tables)."""
    t = golden_e2m1()[:8] if fmt == E2M1 else torch_e4m3()[:127]
    return [c for c in range(len(t)) if float(t[c]).is_integer()]


def pin_integer_exact(orc):
    for fmt, K in ((E2M1, 256), (E4M3, 384)):
        pool = _integer_pool(fmt)
        A, As = mxinputs.random_codes(fmt, 9, K, 11, pool, tensor=0)
        B, Bs = mxinputs.random_codes(fmt, 7, K, 11, pool, tensor=1)
        ia = decode_rows(fmt, A).astype(np.int64)
        ib = decode_rows(fmt, B).astype(np.int64)
        ref = ia @ ib.T
        C, T = orc.gemm(fmt, A, As, B, Bs, K)
        assert np.array_equal(C, ref.astype(np.float64)), fmt
        assert np.array_equal(T, (np.abs(ia) @ np.abs(ib).T).astype(np.float64)), fmt


def pin_scale_shift(orc):
    for fmt in (E2M1, E4M3):
        case = mxinputs.make_random(fmt, 3, 4, 256, seed=3)
        A, As, B, Bs, K = case["A"], case["A_scale"], case["B"], case["B_scale"], 256
        base = {(m, n, b): orc.block_contrib(fmt, A, As, B, Bs, K, m, n, b)
                for m in range(3) for n in range(4) for b in range(K // 32)}
        for (side, row, blk, k) in (("a", 1, 2, 5), ("b", 3, 7, -9), ("a", 0, 0, 1)):
            As2, Bs2 = As.copy(), Bs.copy()
            if side == "a":
                As2[row, blk] = int(As2[row, blk]) + k
            else:
                Bs2[row, blk] = int(Bs2[row, blk]) + k
            for key, (c0, t0) in base.items():
                c1, t1 = orc.block_contrib(fmt, A, As2, B, Bs2, K, *key)
                m, n, b = key
                hit = b == blk and ((side == "a" and m == row) or (side == "b" and n == row))
                f = 2.0 ** k if hit else 1.0
                assert c1 == c0 * f and t1 == t0 * f, (fmt, side, key)
            # The whole sum moves by exactly (2^k - 1) * that block's term, up to
            # the final double rounding of the block sum.
            C0, T0 = orc.gemm(fmt, A, As, B, Bs, K)
            C1, _ = orc.gemm(fmt, A, As2, B, Bs2, K)
            if side == "a":
                delta = np.array([[base[(row, n, blk)][0] * (2.0 ** k - 1) for n in range(4)]])
                got = C1[row:row + 1] - C0[row:row + 1]
                tol = 1e-14 * (T0[row:row + 1] * max(1.0, 2.0 ** k))
            else:
                delta = np.array([[base[(m, row, blk)][0] * (2.0 ** k - 1)] for m in range(3)])
                got = C1[:, row:row + 1] - C0[:, row:row + 1]
                tol = 1e-14 * (T0[:, row:row + 1] * max(1.0, 2.0 ** k))
            assert np.all(np.abs(got - delta) <= tol), (fmt, side)


def pin_numpy_matmul(orc):
    for fmt in (E2M1, E4M3):
        case = mxinputs.make_random(fmt, 64, 48, 512, seed=5)
        A, As, B, Bs = case["A"], case["A_scale"], case["B"], case["B_scale"]
        ref = dequant(fmt, A, As) @ dequant(fmt, B, Bs).T
        C, T = orc.gemm(fmt, A, As, B, Bs, 512)
        assert np.all(np.abs(C - ref) <= 1e-12 * T), fmt
        tref = np.abs(dequant(fmt, A, As)) @ np.abs(dequant(fmt, B, Bs)).T
        assert np.all(np.abs(T - tref) <= 1e-12 * T), fmt


def pin_symmetry(orc):
    for fmt in (E2M1, E4M3):
        case = mxinputs.make_random(fmt, 5, 7, 256, seed=9, scale_lo=90, scale_hi=160)
        A, As, B, Bs = case["A"], case["A_scale"], case["B"], case["B_scale"]
        C, T = orc.gemm(fmt, A, As, B, Bs, 256)
        Ct, Tt = orc.gemm(fmt, B, Bs, A, As, 256)
        assert np.array_equal(C, Ct.T) and np.array_equal(T, Tt.T), fmt


def pin_zero_and_onehot(orc):
    for fmt in (E2M1, E4M3):
        K = 256
        rb = K // 2 if fmt == E2M1 else K
        A = np.zeros((2, rb), np.uint8)
        B = np.zeros((3, rb), np.uint8)
        As = np.full((2, K // 32), 140, np.uint8)
        Bs = np.full((3, K // 32), 90, np.uint8)
        C, T = orc.gemm(fmt, A, As, B, Bs, K)
        assert not C.any() and not T.any()
        # one nonzero element in A[1] and B[2] at the same k = 77 (block 2)
        k = 77
        if fmt == E2M1:
            A[1, k // 2] = 0x7 << 4          # odd k -> high nibble, 6.0
            B[2, k // 2] = 0xB << 4          # -1.5
            va, vb = 6.0, -1.5
        else:
            A[1, k] = 0x7E                   # 448
            B[2, k] = 0x81                   # -2^-9
            va, vb = 448.0, -(2.0 ** -9)
        As[1, 2], Bs[2, 2] = 150, 60
        C, T = orc.gemm(fmt, A, As, B, Bs, K)
        expect = np.zeros((2, 3))
        expect[1, 2] = va * vb * 2.0 ** (150 + 60 - 254)
        assert np.array_equal(C, expect), fmt
        assert np.array_equal(T, np.abs(expect)), fmt


def pin_nan(orc):
    for fmt in (E2M1, E4M3):
        case = mxinputs.make_random(fmt, 3, 3, 128, seed=2)
        A, As, B, Bs = case["A"], case["A_scale"], case["B"], case["B_scale"]
        As = As.copy()
        As[1, 3] = 255
        C, _ = orc.gemm(fmt, A, As, B, Bs, 128)
        assert np.all(np.isnan(C[1])) and not np.isnan(C[[0, 2]]).any(), fmt
        c, t = orc.block_contrib(fmt, A, As, B, Bs, 128, 1, 0, 3)
        assert np.isnan(c) and np.isnan(t), fmt
        c, t = orc.block_contrib(fmt, A, As, B, Bs, 128, 1, 0, 2)
        assert not np.isnan(c) and not np.isnan(t), fmt
    A = np.zeros((2, 128), np.uint8)
    A[0, 5] = 0x7F
    B = np.full((2, 128), 0x38, np.uint8)
    s = np.full((2, 4), 127, np.uint8)
    C, _ = orc.gemm(E4M3, A, s, B, s, 128)
    assert np.all(np.isnan(C[0])) and np.all(C[1] == 0)


def pin_row_subset(orc):
    case = mxinputs.make_random(E2M1, 40, 6, 128, seed=4)
    A, As, B, Bs = case["A"], case["A_scale"], case["B"], case["B_scale"]
    C, T = orc.gemm(E2M1, A, As, B, Bs, 128)
    rows = [39, 0, 17, 17]
    Cs, Ts = orc.gemm(E2M1, A, As, B, Bs, 128, rows=rows)
    assert np.array_equal(Cs, C[rows]) and np.array_equal(Ts, T[rows])


def _group_bound_numpy(fmt, A, As, B, Bs, K):
    """E recomputed from its definition with numpy and the independent
    tables: per aligned group of 8 K-values, the scaled sum of |p| mod
    2^(floor(log2 max|p|) - 12)."""
    va, vb = decode_rows(fmt, A), decode_rows(fmt, B)
    M, N = va.shape[0], vb.shape[0]
    E = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            p = (va[m] * vb[n]).reshape(-1, 8)
            w = np.repeat(np.ldexp(1.0, As[m].astype(np.int64) + Bs[n].astype(np.int64) - 254), 4)
            mx = np.abs(p).max(axis=1)
            tot = 0.0
            for gi in range(p.shape[0]):
                if mx[gi] == 0:
                    continue
                grid = 2.0 ** (math.floor(math.log2(mx[gi])) - 12)
                tot += w[gi] * float(np.sum(np.fmod(np.abs(p[gi]), grid)))
            E[m, n] = tot
    return E


def pin_group_bound(orc):
    # Closed forms: products {2^8, 7 x 2^-6} in one group: grid 2^-4, each
    # 2^-6 lies wholly below it -> E = 7 * 2^-6.  With every small product a
    # multiple of the grid (2^-4), E = 0.  Scale 2^(sA+sB-254) multiplies E.
    K = 128
    A = np.zeros((1, K), np.uint8)
    B = np.zeros((1, K), np.uint8)
    A[0, 8] = 0x78                        # 2^8 (E4M3 e=15, m=0)
    B[0, 8:16] = 0x38                     # 1.0
    for code, val, expect_mult in ((0x08, 2.0 ** -6, 7), (0x18, 2.0 ** -4, 0)):
        A[0, 9:16] = code                 # 0x08 = 2^-6, 0x18 = 2^-4
        for sa, sb in ((127, 127), (130, 120)):
            As = np.full((1, 4), sa, np.uint8)
            Bs = np.full((1, 4), sb, np.uint8)
            C, T, E = orc.gemm(E4M3, A, As, B, Bs, K, group_bound=True)
            assert E[0, 0] == expect_mult * val * 2.0 ** (sa + sb - 254), (code, sa, sb, E[0, 0])
    # E2M1: every product is a multiple of 1/4 and the grid is at most 2^-7.
    case = mxinputs.make_random(E2M1, 6, 5, 512, seed=21)
    _, _, E = orc.gemm(E2M1, case["A"], case["A_scale"], case["B"], case["B_scale"], 512,
                       group_bound=True)
    assert not E.any()
    # Random E4M3 with wide exponents: equal to the numpy recomputation.
    for seed in (1, 2):
        pool = range(127)
        A, _ = mxinputs.random_codes(E4M3, 3, 256, 40 + seed, pool, tensor=0)
        B, _ = mxinputs.random_codes(E4M3, 4, 256, 40 + seed, pool, tensor=1)
        r = np.random.default_rng([9, seed])
        As = r.integers(110, 145, size=(3, 8)).astype(np.uint8)
        Bs = r.integers(110, 145, size=(4, 8)).astype(np.uint8)
        _, T, E = orc.gemm(E4M3, A, As, B, Bs, 256, group_bound=True)
        ref = _group_bound_numpy(E4M3, A, As, B, Bs, 256)
        assert np.all(np.abs(E - ref) <= 1e-12 * T), seed
        assert E.any()


# --------------------------------------------------------------------------
# The quantizer (mxo_quantize): OCP MX conversion of wider values.

def _sweep_values(vmax, positive_grid):
    """Values in [-vmax, vmax]: every grid point, every midpoint between
    neighbours (the ties), points just beside each midpoint, and a random
    sample; as float32 (all exact in float64)."""
    g = np.asarray(sorted(set(positive_grid)), np.float64)
    mids = (g[1:] + g[:-1]) / 2
    eps = np.float32(1e-6)
    extra = np.concatenate([mids * (1 - eps), mids * (1 + eps)])
    rng = np.random.default_rng(7)
    rnd = rng.uniform(0, vmax, 4000)
    v = np.concatenate([g, mids, extra, rnd]).astype(np.float32).astype(np.float64)
    v = v[v <= vmax]
    return np.concatenate([v, -v])


def _blocks_with_amax(vals, amax):
    """Pack values into blocks of 31 plus one element equal to amax, so that
    every block's shared exponent is floor(log2 amax) - emax."""
    n = -(-len(vals) // 31)
    vals = np.concatenate([vals, np.zeros(n * 31 - len(vals))])
    blocks = np.concatenate([np.full((n, 1), amax), vals.reshape(n, 31)], axis=1)
    return blocks.reshape(1, -1)


def pin_quantize_e4m3_vs_torch(orc):
    """Elements: with amax = 448 the shared exponent is 0 (byte 127), so each
    code must equal torch's float8_e4m3fn conversion (round to nearest even)
    of the value itself."""
    import torch
    t8 = torch_e4m3()
    grid = [abs(x) for x in t8[np.isfinite(t8)]]
    vals = _sweep_values(448.0, grid)
    X = _blocks_with_amax(vals, 448.0)
    Q, S = orc.quantize(E4M3, X)
    assert (S == 127).all(), "E4M3 scale byte for amax 448 must be 127"
    ref = torch.from_numpy(X.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (Q == ref).all(), "E4M3 codes differ from torch's conversion at %s" % (
        X[Q != ref][:5],)
    # Saturation: above 448 (torch would give NaN past 464) the code is +-448.
    X = _blocks_with_amax(np.array([449.0, 460.0, 479.0, -470.0]), 479.0)
    Q, S = orc.quantize(E4M3, X)
    assert S[0, 0] == 127 and (Q[0, :5] == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]).all(), Q[0, :5]


def pin_quantize_e5m2_vs_torch(orc):
    """E5M2 elements: with amax = 57344 the shared exponent is 0 (byte 127),
    so each code must equal torch's float8_e5m2 conversion (round to nearest
    even, subnormals down to 2^-16) of the value itself; above 57344 the code
    saturates, where torch's conversion would overflow to infinity."""
    import torch
    t = torch_e5m2()
    grid = [abs(x) for x in t[np.isfinite(t)]]
    vals = _sweep_values(57344.0, grid)
    X = _blocks_with_amax(vals, 57344.0)
    Q, S = orc.quantize(E5M2, X)
    assert (S == 127).all(), "E5M2 scale byte for amax 57344 must be 127"
    ref = torch.from_numpy(X.astype(np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert (Q == ref).all(), "E5M2 codes differ from torch's conversion at %s" % (
        X[Q != ref][:5],)
    X = _blocks_with_amax(np.array([57345.0, 61440.0, 65000.0, -62000.0]), 65000.0)
    Q, S = orc.quantize(E5M2, X)
    assert S[0, 0] == 127 and (Q[0, :5] == [0x7B, 0x7B, 0x7B, 0x7B, 0xFB]).all(), Q[0, :5]
    # the scale rule with emax 15: amax 1.0 -> byte 112, amax 2^-20 -> 92
    X = _blocks_with_amax(np.array([0.5]), 1.0)
    assert orc.quantize(E5M2, X)[1][0, 0] == 127 - 15
    X = _blocks_with_amax(np.array([2.0 ** -21]), 2.0 ** -20)
    assert orc.quantize(E5M2, X)[1][0, 0] == 127 - 20 - 15


def pin_quantize_e2m1_bruteforce(orc):
    """Elements: with amax = 6 the shared exponent is 0, so each code must be
    the nearest E2M1 value (independent golden table), ties to the code with
    an even last bit, sign from the value."""
    g = golden_e2m1()
    vals = _sweep_values(6.0, [abs(x) for x in g])
    X = _blocks_with_amax(vals, 6.0)
    Q, S = orc.quantize(E2M1, X)
    assert (S == 127).all(), "E2M1 scale byte for amax 6 must be 127"
    codes = mxinputs.unpack_e2m1(Q)[0]
    mags = np.abs(g[:8])
    for x, c in zip(X[0], codes):
        d = np.abs(mags - abs(x))
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        want |= 8 if np.signbit(x) else 0
        assert c == want, "E2M1 code for %r: got %d want %d" % (x, c, want)


def pin_quantize_fp6_bruteforce(orc):
    """FP6 elements (E2M3, E3M2): with amax equal to the format's largest
    value (7.5, 28) the shared exponent is 0, so each code must be the
    nearest value of the OCP list (tests/golden), ties to the code with an
    even last bit, sign from the value, unpacked by the input generator's
    own FP6 unpacking.  Above the largest value within the top binade the
    code saturates, and the scale byte follows emax 2 / 4."""
    for fmt, maxv, top in ((E2M3, 7.5, 7.9), (E3M2, 28.0, 31.5)):
        g = golden_fp6(fmt)
        mags = g[:32]
        vals = _sweep_values(maxv, [abs(x) for x in mags])
        X = _blocks_with_amax(vals, maxv)
        Q, S = orc.quantize(fmt, X)
        assert Q.shape == (1, X.shape[1] // 4 * 3)
        assert (S == 127).all(), "fmt %d scale byte for amax %g must be 127" % (fmt, maxv)
        codes = mxinputs.unpack_fp6(Q)[0]
        for x, c in zip(X[0], codes):
            d = np.abs(mags - abs(x))
            best = np.flatnonzero(d == d.min())
            want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
            want |= 32 if np.signbit(x) else 0
            assert c == want, "fmt %d code for %r: got %d want %d" % (fmt, x, c, want)
        # saturation in the top binade, both signs
        X = _blocks_with_amax(np.array([top, (maxv + top) / 2, -top]), top)
        Q, S = orc.quantize(fmt, X)
        assert S[0, 0] == 127, S[0, 0]
        assert list(mxinputs.unpack_fp6(Q)[0][:4]) == [31, 31, 31, 63]
        # emax: amax 1.0 gives byte 127 - emax
        X = _blocks_with_amax(np.array([0.25]), 1.0)
        assert orc.quantize(fmt, X)[1][0, 0] == 127 - (2 if fmt == E2M3 else 4)


def pin_quantize_scale_rule(orc):
    """Scale bytes: floor(log2 amax) from Python's frexp, minus emax, plus
    127, clamped to [0, 254]; 0 for an all-zero block.  amax ranges over
    FP32 subnormals, exact powers of two and the values just below them."""
    amaxes = [0.0, 2.0 ** -149, 2.0 ** -140, 2.0 ** -126, 3.0 * 2 ** -130, 1.0, 6.0, 7.99,
              8.0, 448.0, 512.0, 1e30, 2.0 ** 127, 3.4e38]
    for e in range(-120, 120, 7):
        amaxes += [2.0 ** e, float(np.nextafter(np.float32(2.0 ** e), np.float32(0)))]
    for fmt, emax in ((E2M1, 2), (E4M3, 8)):
        X = np.zeros((len(amaxes), 32))
        X[:, 5] = amaxes
        X[:, 9] = -np.asarray(amaxes) / 3.0          # smaller magnitude, other sign
        _, S = orc.quantize(fmt, X)
        for a, s in zip(amaxes, S[:, 0]):
            want = 0 if a == 0 else min(254, max(0, math.frexp(a)[1] - 1 - emax + 127))
            assert s == want, "fmt %d amax %r: scale %d want %d" % (fmt, a, s, want)


def pin_quantize_nonfinite(orc):
    """A block holding a NaN or an infinity gets scale byte 255 and zero codes;
    its neighbours are unaffected."""
    for fmt in (E2M1, E4M3):
        X = np.ones((3, 64))
        X[0, 3] = np.nan
        X[1, 40] = np.inf
        X[2, 0] = -np.inf
        Q, S = orc.quantize(fmt, X)
        assert S[0, 0] == 255 and S[1, 1] == 255 and S[2, 0] == 255
        assert S[0, 1] != 255 and S[1, 0] != 255 and S[2, 1] != 255
        codes = Q if fmt == E4M3 else mxinputs.unpack_e2m1(Q)
        assert (codes[0, :32] == 0).all() and (codes[1, 32:] == 0).all()
        assert (codes[0, 32:] != 0).all()


def pin_quantize_roundtrip(orc):
    """Decoding (independent tables) the quantized values of random data gives
    back each value to within half the element spacing times 2^X, except
    where it saturated; and each nonzero block's largest value lands in the
    format's top binade (the definition of the shared exponent)."""
    rng = np.random.default_rng(11)
    X = rng.standard_normal((40, 256)) * np.exp2(rng.integers(-30, 30, (40, 1)))
    X = X.astype(np.float32).astype(np.float64)
    for fmt, man, top in ((E2M1, 1, 4.0), (E4M3, 3, 256.0)):
        Q, S = orc.quantize(fmt, X)
        deq = dequant(fmt, Q, S)
        scale = np.repeat(np.exp2(S.astype(np.int64) - 127.0), 32, axis=1)
        mag = np.abs(X) / scale
        _, e = np.frexp(np.maximum(mag, 2.0 ** -60))
        spacing = np.exp2(np.maximum(e - 1, 1 - (1 if fmt == E2M1 else 7)) - man) * scale
        sat = mag > (6.0 if fmt == E2M1 else 448.0)
        err = np.abs(deq - X)
        assert (err[~sat] <= spacing[~sat] / 2 * (1 + 1e-12)).all(), fmt
        bmax = np.abs(deq).reshape(40, -1, 32).max(axis=2) / scale[:, ::32]
        assert (bmax >= top).all(), fmt


def pin_grouped(orc):
    """Grouped GEMM: each group's rows equal a numpy matmul of the dequantized
    group rows against that group's weight (independent tables), and the
    whole result is the block diagonal of one plain GEMM of A against every
    weight; empty groups take no rows."""
    for fmt in (E2M1, E4M3):
        rows, N, K = [5, 0, 9, 1, 0, 6], 7, 256
        G = len(rows)
        case = mxinputs.make_random(fmt, sum(rows), G * N, K, seed=11)
        A, As, B, Bs = case["A"], case["A_scale"], case["B"], case["B_scale"]
        C, T = orc.gemm_grouped(fmt, A, As, B, Bs, K, rows)
        Cf, Tf = orc.gemm(fmt, A, As, B, Bs, K)
        dA, dB = dequant(fmt, A, As), dequant(fmt, B, Bs)
        r0 = 0
        for g, m in enumerate(rows):
            sl = slice(r0, r0 + m)
            wl = slice(g * N, (g + 1) * N)
            assert np.array_equal(C[sl], Cf[sl, wl]) and np.array_equal(T[sl], Tf[sl, wl])
            ref = dA[sl] @ dB[wl].T
            assert np.all(np.abs(C[sl] - ref) <= 1e-12 * T[sl]), (fmt, g)
            r0 += m
        # a row subset, in any order, picks the same values
        pick = [20, 0, 14, 5, 5]
        Cs, Ts, Es = orc.gemm_grouped(fmt, A, As, B, Bs, K, rows, rows=pick, group_bound=True)
        assert np.array_equal(Cs, C[pick]) and np.array_equal(Ts, T[pick])
        _, _, Ef = orc.gemm(fmt, A, As, B, Bs, K, group_bound=True)
        assert np.array_equal(Es[1], Ef[0, :N]) and np.array_equal(Es[0], Ef[20, 5 * N:])
    # E4M3 activations with E2M1 weights, and the reverse
    for fa, fb in ((E4M3, E2M1), (E2M1, E4M3)):
        rows, N, K = [3, 0, 6, 1], 5, 256
        G = len(rows)
        ca = mxinputs.make_random(fa, sum(rows), 1, K, seed=13)
        cb = mxinputs.make_random(fb, 1, G * N, K, seed=14)
        A, As, B, Bs = ca["A"], ca["A_scale"], cb["B"], cb["B_scale"]
        C, T = orc.gemm_grouped(fa, A, As, B, Bs, K, rows, fmt_b=fb)
        Cf, Tf = orc.gemm(fa, A, As, B, Bs, K, fmt_b=fb)
        dA, dB = dequant(fa, A, As), dequant(fb, B, Bs)
        r0 = 0
        for g, m in enumerate(rows):
            sl, wl = slice(r0, r0 + m), slice(g * N, (g + 1) * N)
            assert np.array_equal(C[sl], Cf[sl, wl]) and np.array_equal(T[sl], Tf[sl, wl])
            assert np.all(np.abs(C[sl] - dA[sl] @ dB[wl].T) <= 1e-12 * T[sl]), (fa, fb, g)
            r0 += m


def pin_mixed_formats(orc):
    """A and B in different formats (E4M3 x E2M1 and the reverse): a numpy
    matmul of the dequantized operands (independent tables), exact rationals
    on a tiny case, and the transpose symmetry across the two directions."""
    for fa, fb in ((E4M3, E2M1), (E2M1, E4M3)):
        ca = mxinputs.make_random(fa, 24, 3, 512, seed=31)
        cb = mxinputs.make_random(fb, 3, 20, 512, seed=32)
        A, As, B, Bs = ca["A"], ca["A_scale"], cb["B"], cb["B_scale"]
        C, T = orc.gemm(fa, A, As, B, Bs, 512, fmt_b=fb)
        ref = dequant(fa, A, As) @ dequant(fb, B, Bs).T
        tref = np.abs(dequant(fa, A, As)) @ np.abs(dequant(fb, B, Bs)).T
        assert np.all(np.abs(C - ref) <= 1e-12 * T), (fa, fb)
        assert np.all(np.abs(T - tref) <= 1e-12 * T), (fa, fb)
        Ct, Tt = orc.gemm(fb, B, Bs, A, As, 512, fmt_b=fa)
        assert np.array_equal(C, Ct.T) and np.array_equal(T, Tt.T), (fa, fb)
        # exact rationals on 2 x 2 outputs, one 128-K block row each
        ca = mxinputs.make_random(fa, 2, 2, 128, seed=33, scale_lo=110, scale_hi=140)
        cb = mxinputs.make_random(fb, 2, 2, 128, seed=34, scale_lo=110, scale_hi=140)
        va, vb = decode_rows(fa, ca["A"]), decode_rows(fb, cb["B"])
        C, _ = orc.gemm(fa, ca["A"], ca["A_scale"], cb["B"], cb["B_scale"], 128, fmt_b=fb)
        for m in range(2):
            for n in range(2):
                tot = Fraction(0)
                for k in range(128):
                    w = Fraction(2) ** (int(ca["A_scale"][m, k // 32]) + int(cb["B_scale"][n, k // 32]) - 254)
                    tot += Fraction(va[m, k]) * Fraction(vb[n, k]) * w
                assert C[m, n] == float(tot), (fa, fb, m, n)


def pin_e5m2(orc):
    """E5M2 (both operands): the decode table against torch's float8_e5m2
    (infinities and NaNs included); a numpy matmul of dequantized operands;
    exact rationals over a wide exponent spread; and a block whose exact sum
    is a tiny remainder between two products 63 binades larger, which a
    double-precision running sum would lose."""
    ref = torch_e5m2()
    got = np.array([orc.e5m2_value(c) for c in range(256)])
    assert _same(got, ref)
    case = mxinputs.make_random(E5M2, 40, 24, 512, seed=41)
    A, As, B, Bs = case["A"], case["A_scale"], case["B"], case["B_scale"]
    C, T = orc.gemm(E5M2, A, As, B, Bs, 512)
    refc = dequant(E5M2, A, As) @ dequant(E5M2, B, Bs).T
    assert np.all(np.abs(C - refc) <= 1e-12 * T)
    # exact rationals: random finite codes over the whole exponent range
    rng = np.random.default_rng(5)
    finite = np.array([c for c in range(256) if np.isfinite(ref[c])], np.uint8)
    A = rng.choice(finite, size=(3, 64)).astype(np.uint8)
    B = rng.choice(finite, size=(2, 64)).astype(np.uint8)
    As = rng.integers(100, 150, size=(3, 2)).astype(np.uint8)
    Bs = rng.integers(100, 150, size=(2, 2)).astype(np.uint8)
    C, _ = orc.gemm(E5M2, A, As, B, Bs, 64)
    for m in range(3):
        for n in range(2):
            blocks = []
            for b in range(2):
                w = Fraction(2) ** (int(As[m, b]) + int(Bs[n, b]) - 254)
                blocks.append(float(sum(Fraction(ref[A[m, k]]) * Fraction(ref[B[n, k]])
                                        for k in range(32 * b, 32 * b + 32)) * w))
            assert C[m, n] == blocks[0] + blocks[1], (m, n)
    # cancellation: 57344 * 57344 - 57344 * 57344 + 2^-16 * 2^-16 = 2^-32
    code_max, code_min = 0x7B, 0x01            # 57344 and 2^-16
    A = np.zeros((1, 32), np.uint8)
    B = np.zeros((1, 32), np.uint8)
    A[0, :3] = [code_max, code_min, code_max | 0x80]
    B[0, :3] = [code_max, code_min, code_max]
    s = np.full((1, 1), 127, np.uint8)
    C, T = orc.gemm(E5M2, A, s, B, s, 32)
    assert C[0, 0] == 2.0 ** -32, C[0, 0]
    assert T[0, 0] == 2 * 57344.0 ** 2 + 2.0 ** -32 or T[0, 0] == 2 * 57344.0 ** 2


def pin_e5m2_pairs(orc):
    """E5M2 paired with E4M3 or E2M1, in both directions: a numpy matmul of
    the dequantized operands (torch's tables); the transpose symmetry
    between the two directions; and a block whose exact sum is 2^-25, the
    smallest E4M3 x E5M2 product, left over after fifteen products of
    448 * 57344 cancel, which a double-precision running sum rounds away."""
    for fa, fb in ((E4M3, E5M2), (E5M2, E2M1)):
        ca = mxinputs.make_random(fa, 20, 3, 256, seed=51)
        cb = mxinputs.make_random(fb, 3, 14, 256, seed=52)
        A, As, B, Bs = ca["A"], ca["A_scale"], cb["B"], cb["B_scale"]
        C, T = orc.gemm(fa, A, As, B, Bs, 256, fmt_b=fb)
        ref = dequant(fa, A, As) @ dequant(fb, B, Bs).T
        assert np.all(np.abs(C - ref) <= 1e-12 * T), (fa, fb)
        Ct, Tt = orc.gemm(fb, B, Bs, A, As, 256, fmt_b=fa)
        assert np.array_equal(C, Ct.T) and np.array_equal(T, Tt.T), (fa, fb)
    A = np.zeros((1, 32), np.uint8)            # E4M3
    B = np.zeros((1, 32), np.uint8)            # E5M2
    A[0, :15] = 0x7E                           # 448
    A[0, 15] = 0x01                            # 2^-9
    A[0, 16:31] = 0xFE                         # -448
    B[0, :31] = 0x7B                           # 57344
    B[0, 15] = 0x01                            # 2^-16
    s = np.full((1, 1), 127, np.uint8)
    C, T = orc.gemm(E4M3, A, s, B, s, 32, fmt_b=E5M2)
    assert C[0, 0] == 2.0 ** -25, C[0, 0]


def pin_fp6(orc):
    """FP6 (E2M3, E3M2): every code's value against the OCP value lists; a
    numpy matmul of operands decoded with those lists and the generator's own
    unpacking; the bit position of every element of a 4-element, 3-byte
    group (one-hot products at each k of a block); exact integers; and the
    transpose symmetry."""
    for fmt in (E2M3, E3M2):
        g = golden_fp6(fmt)
        got = np.array([orc.gemm(fmt, *_fp6_onehot(fmt, c, g), 32)[0][0, 0] for c in range(64)])
        assert np.array_equal(got, g), (fmt, np.flatnonzero(got != g)[:5])
        case = mxinputs.make_random(fmt, 24, 18, 512, seed=61)
        A, As, B, Bs = case["A"], case["A_scale"], case["B"], case["B_scale"]
        C, T = orc.gemm(fmt, A, As, B, Bs, 512)
        assert np.all(np.abs(C - dequant(fmt, A, As) @ dequant(fmt, B, Bs).T) <= 1e-12 * T), fmt
        Ct, Tt = orc.gemm(fmt, B, Bs, A, As, 512)
        assert np.array_equal(C, Ct.T) and np.array_equal(T, Tt.T)
        # one-hot at every position k of the first block: A_k = 1, B_k = 2
        one, two = int(np.flatnonzero(g == 1.0)[0]), int(np.flatnonzero(g == 2.0)[0])
        s = np.full((1, 1), 127, np.uint8)
        for k in range(32):
            ca = np.zeros((1, 32), np.uint8)
            cb = np.zeros((1, 32), np.uint8)
            ca[0, k], cb[0, k] = one, two
            ca[0, (k + 1) % 32] = one                  # neighbour: A only, B zero there
            C1, _ = orc.gemm(fmt, mxinputs.pack_fp6(ca), s, mxinputs.pack_fp6(cb), s, 32)
            assert C1[0, 0] == 2.0, (fmt, k, C1[0, 0])
            # the same against an E4M3 operand (2.0 = code 0x40), which fixes
            # the FP6 element position on its own (a permutation applied to
            # both FP6 operands would leave every block sum unchanged)
            c8 = np.zeros((1, 32), np.uint8)
            c8[0, k] = 0x40
            C2, _ = orc.gemm(fmt, mxinputs.pack_fp6(ca), s, c8, s, 32, fmt_b=E4M3)
            assert C2[0, 0] == 2.0, (fmt, k, C2[0, 0])
        # integer-valued codes, scales 127: exact
        ints = [c for c in range(64) if g[c] == np.round(g[c])]
        rng = np.random.default_rng(7)
        ia = rng.choice(ints, size=(6, 256))
        ib = rng.choice(ints, size=(5, 256))
        s = np.full((6, 8), 127, np.uint8)
        Ci, _ = orc.gemm(fmt, mxinputs.pack_fp6(ia), s, mxinputs.pack_fp6(ib), s[:5], 256)
        want = g[ia].astype(np.int64) @ g[ib].astype(np.int64).T
        assert np.array_equal(Ci, want.astype(np.float64)), fmt


def _fp6_onehot(fmt, code, g):
    """A = [code, 0, ...], B = [1.0, 0, ...] (one 32-block, scale 127): C is
    the value of the code."""
    one = int(np.flatnonzero(g == 1.0)[0])
    ca = np.zeros((1, 32), np.uint8)
    cb = np.zeros((1, 32), np.uint8)
    ca[0, 0], cb[0, 0] = code, one
    s = np.full((1, 1), 127, np.uint8)
    return mxinputs.pack_fp6(ca), s, mxinputs.pack_fp6(cb), s


def pin_bf16(orc):
    """BF16 dense GEMM: the decode against torch's bfloat16 (every pattern);
    a numpy matmul of torch-decoded values; exact rationals on a tiny case;
    exact integers (small integer values make every sum exact); and the
    transpose symmetry."""
    import torch
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([orc.bf16_value(int(b)) for b in bits[::97]])
    assert _same(got, ref[::97])
    A = mxinputs.make_bf16(20, 256, seed=1)
    B = mxinputs.make_bf16(12, 256, seed=1, tensor=1)
    dA = torch.from_numpy(A.view(np.int16)).view(torch.bfloat16).double().numpy()
    dB = torch.from_numpy(B.view(np.int16)).view(torch.bfloat16).double().numpy()
    C, T = orc.gemm_bf16(A, B)
    assert np.all(np.abs(C - dA @ dB.T) <= 1e-12 * T)
    assert np.all(np.abs(T - np.abs(dA) @ np.abs(dB).T) <= 1e-12 * T)
    Ct, Tt = orc.gemm_bf16(B, A)
    assert np.array_equal(C, Ct.T) and np.array_equal(T, Tt.T)
    Cs, _ = orc.gemm_bf16(A[:2, :8], B[:2, :8])
    for m in range(2):
        for n in range(2):
            exact = sum(Fraction(dA[m, k]) * Fraction(dB[n, k]) for k in range(8))
            assert Cs[m, n] == float(exact)
    rng = np.random.default_rng(2)
    ia = rng.integers(-8, 9, size=(5, 64)).astype(np.float32)
    ib = rng.integers(-8, 9, size=(4, 64)).astype(np.float32)
    to_bits = lambda x: torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    Ci, _ = orc.gemm_bf16(to_bits(ia), to_bits(ib))
    assert np.array_equal(Ci, ia.astype(np.int64) @ ib.astype(np.int64).T)


def pin_grouped_bf16(orc):
    """Grouped dense BF16 GEMM: each group's rows equal a numpy matmul of
    the torch-decoded group rows against that group's weight, and the whole
    result is the block diagonal of one plain BF16 GEMM of A against every
    weight; empty groups take no rows; a row subset picks the same values."""
    import torch
    rows, N, K = [4, 0, 7, 1, 0, 3], 5, 96
    G = len(rows)
    A = mxinputs.make_bf16(sum(rows), K, seed=21)
    B = mxinputs.make_bf16(G * N, K, seed=21, tensor=1)
    dA = torch.from_numpy(A.view(np.int16)).view(torch.bfloat16).double().numpy()
    dB = torch.from_numpy(B.view(np.int16)).view(torch.bfloat16).double().numpy()
    C, T = orc.gemm_grouped_bf16(A, B, rows)
    Cf, Tf = orc.gemm_bf16(A, B)
    r0 = 0
    for g, m in enumerate(rows):
        sl = slice(r0, r0 + m)
        wl = slice(g * N, (g + 1) * N)
        assert np.array_equal(C[sl], Cf[sl, wl]) and np.array_equal(T[sl], Tf[sl, wl])
        assert np.all(np.abs(C[sl] - dA[sl] @ dB[wl].T) <= 1e-12 * T[sl]), g
        r0 += m
    pick = [14, 0, 11, 4, 4]
    Cs, Ts = orc.gemm_grouped_bf16(A, B, rows, rows=pick)
    assert np.array_equal(Cs, C[pick]) and np.array_equal(Ts, T[pick])


ALL_PINS = [pin_e4m3_table, pin_e2m1_table, pin_e8m0, pin_worked_examples,
            pin_bruteforce, pin_integer_exact, pin_scale_shift, pin_numpy_matmul,
            pin_symmetry, pin_zero_and_onehot, pin_nan, pin_row_subset,
            pin_group_bound, pin_quantize_e4m3_vs_torch, pin_quantize_e5m2_vs_torch,
            pin_quantize_e2m1_bruteforce, pin_quantize_fp6_bruteforce,
            pin_quantize_scale_rule, pin_quantize_nonfinite, pin_quantize_roundtrip,
            pin_grouped, pin_mixed_formats, pin_e5m2, pin_e5m2_pairs, pin_fp6, pin_bf16,
            pin_grouped_bf16]


# --------------------------------------------------------------------------
# The acceptance helpers: oracle.bf16_ulp, bound, round_to_output and compare.
# Each pin takes a namespace holding those four functions (the oracle module,
# or a copy with a planted mistake) and checks them against torch's bfloat16
# and float32 conversions and against cases worked out by hand.

def _torch_bf16_values(bits):
    import torch
    return torch.from_numpy(np.asarray(bits, np.int16)).view(torch.bfloat16).double().numpy()


def pin_bf16_ulp(h):
    """bf16_ulp(x) is the spacing to the next bfloat16 number up, for every
    positive finite bfloat16 value below the largest (subnormals included),
    for its negation, and for values between two bfloat16 numbers."""
    bits = np.arange(1, 0x7F7F, dtype=np.int64)
    v = _torch_bf16_values(bits)
    spacing = _torch_bf16_values(bits + 1) - v
    assert np.array_equal(h.bf16_ulp(v), spacing)
    assert np.array_equal(h.bf16_ulp(-v), spacing)
    assert np.array_equal(h.bf16_ulp((v + (v + spacing)) / 2), spacing)
    assert h.bf16_ulp(np.array([0.0]))[0] == spacing[0] == 2.0 ** -133
    # the largest finite bfloat16, (2 - 2^-7) * 2^127, is in the binade of 2^127
    assert h.bf16_ulp(np.array([_torch_bf16_values([0x7F7F])[0]]))[0] == 2.0 ** 120


def pin_round_to_output(h):
    """round_to_output equals torch's float64 -> float32 conversion, and for
    BF16 output torch's float32 -> bfloat16 conversion of that, over
    magnitudes from below the bfloat16 subnormals to beyond float32's range,
    exact ties, the bfloat16 overflow threshold and NaN."""
    import torch
    r = np.random.default_rng(7)
    x = np.ldexp(r.uniform(1.0, 2.0, 4000), r.integers(-150, 130, 4000))
    x *= np.where(r.random(4000) < 0.5, -1.0, 1.0)
    ties = np.ldexp(1.0 + (2 * r.integers(0, 128, 200) + 1) / 256.0, r.integers(-120, 120, 200))
    big = np.array([3.3895313892515355e+38, 3.3961775292304740e+38, 3.39617753e38,
                    3.4e38, 3.5e38, 1e39, -1e39, 2.0 ** -149, 2.0 ** -150, 0.0, -0.0])
    x = np.concatenate([x, ties, -ties, big])
    t32 = torch.from_numpy(x).to(torch.float32)
    assert np.array_equal(h.round_to_output(x, False), t32.double().numpy())
    assert np.array_equal(h.round_to_output(x, True), t32.to(torch.bfloat16).double().numpy())
    assert np.isnan(h.round_to_output(np.array([np.nan]), True)).all()
    assert np.isnan(h.round_to_output(np.array([np.nan]), False)).all()


def pin_bound(h):
    """bound = 1e-5 * T (FP32 out), + E when given, + one bfloat16 ulp of C
    for BF16 out; ulps from hand: 0 -> 2^-133, 1 -> 2^-7, -3 -> 2^-6,
    2^-130 -> 2^-133 (subnormal), 1e30 (2^99.66) -> 2^92."""
    C = np.array([0.0, 1.0, -3.0, 2.0 ** -130, 1e30])
    T = np.array([0.0, 1.0, 5.0, 2.0 ** -130, 2e30])
    E = np.array([0.5, 0.0, 2.0, 0.0, 1e20])
    ulp = np.array([2.0 ** -133, 2.0 ** -7, 2.0 ** -6, 2.0 ** -133, 2.0 ** 92])
    assert np.array_equal(h.bound(C, T, False), 1e-5 * T)
    assert np.array_equal(h.bound(C, T, False, E), 1e-5 * T + E)
    assert np.array_equal(h.bound(C, T, True), 1e-5 * T + ulp)
    assert np.array_equal(h.bound(C, T, True, E), 1e-5 * T + E + ulp)


def pin_compare(h):
    """compare() on cases worked out by hand: errors exactly at the bound
    pass and the next double above it fails; T = 0 demands an exact zero
    (FP32) or at most the bfloat16 subnormal spacing (BF16); +0 equals -0; E
    counts only when given, and n_plain_bad counts what passes only thanks
    to it; NaN must meet NaN; a value beyond the output type's range must
    meet the infinity of its sign; the worst ratio and the first failing
    index are reported."""
    def one(g, c, t, bf16, e=None):
        return h.compare(np.array([g]), np.array([c]), np.array([t]), bf16,
                         None if e is None else np.array([e]))
    lim = 1e-5 * 2.0 ** 20                       # exact: a power-of-two multiple
    assert one(lim, 0.0, 2.0 ** 20, False)["n_bad"] == 0
    assert one(np.nextafter(lim, np.inf), 0.0, 2.0 ** 20, False)["n_bad"] == 1
    assert one(-lim, 0.0, 2.0 ** 20, False)["n_bad"] == 0
    assert one(0.0, 0.0, 0.0, False)["n_bad"] == 0
    assert one(-0.0, 0.0, 0.0, False)["n_bad"] == 0
    r = one(2.0 ** -149, 0.0, 0.0, False)
    assert r["n_bad"] == 1 and r["max_ratio"] == float("inf")
    assert one(2.0 ** -133, 0.0, 0.0, True)["n_bad"] == 0
    assert one(2.0 ** -132, 0.0, 0.0, True)["n_bad"] == 1
    assert one(1.0 + 2.0 ** -7, 1.0, 0.0, True)["n_bad"] == 0
    assert one(1.0 + 2.0 ** -6, 1.0, 0.0, True)["n_bad"] == 1
    assert one(1.0 + 2.0 ** -7, 1.0, 0.0, False)["n_bad"] == 1
    r = one(0.5, 0.0, 0.0, False, 0.5)
    assert r["n_bad"] == 0 and r["n_plain_bad"] == 1
    assert one(0.5, 0.0, 0.0, False)["n_bad"] == 1
    assert one(0.5, 0.0, 0.0, False, 0.25)["n_bad"] == 1
    nan, inf = float("nan"), float("inf")
    assert one(nan, nan, 1.0, False)["n_bad"] == 0
    assert one(nan, nan, 1.0, True)["n_bad"] == 0
    assert one(1.0, nan, 1.0, False)["n_bad"] == 1
    assert one(nan, 1.0, 1.0, False)["n_bad"] == 1
    assert one(inf, 1e39, 1e39, False)["n_bad"] == 0
    assert one(-inf, -1e39, 1e39, False)["n_bad"] == 0
    assert one(-inf, 1e39, 1e39, False)["n_bad"] == 1
    assert one(3.4028234663852886e38, 1e39, 1e39, False)["n_bad"] == 1
    assert one(inf, 1.0, 1.0, False)["n_bad"] == 1
    assert one(inf, 3.4e38, 3.4e38, True)["n_bad"] == 0     # above bfloat16's largest
    assert one(inf, 3.4e38, 3.4e38, False)["n_bad"] == 1    # float32 still holds it
    g = np.array([1.0, 2.0, 3.0, 4.0 + 1e-3, 5.0])
    C = np.array([1.0, 2.0 + 0.5e-5, 3.0, 4.0, 5.0])
    r = h.compare(g, C, np.ones(5), False)
    assert r["n_bad"] == 1 and r["first_bad"] == (3,)
    assert abs(r["max_ratio"] - 100.0) < 1e-6
    r = h.compare(g[:3], C[:3], np.ones(3), False)
    assert r["n_bad"] == 0 and abs(r["max_ratio"] - 0.5) < 1e-6


HELPER_PINS = [pin_bf16_ulp, pin_round_to_output, pin_bound, pin_compare]
