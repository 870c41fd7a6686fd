"""CPU oracle for the MX block-scaled NT GEMM -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  It wraps ``liboracle.so`` (plain C, ``mx_oracle.c``), which
shares no code with the GPU library.

What the oracle computes, and where it comes from, is stated in
``mx_oracle.c``: exact per-32 block dot products of table-decoded E2M1/E4M3
elements, each scaled by 2^(sA+sB-254), summed over blocks in double; and the
OCP MX quantization of a matrix (``quantize``).

The acceptance rule lives here too:
  FP32 output: |gpu - C| <= 1e-5 * T
  BF16 output: |gpu - C| <= 1e-5 * T + ulp_bf16(C)
where T = sum over k of |a_k * b_k| (scaled) and ulp_bf16(x) is the spacing
of bfloat16 numbers in x's binade (2^(max(floor(log2|x|), -126) - 7)); for
x = 0 it is the smallest subnormal spacing, 2^-133.  NaN results are not
graded by this rule.

For E4M3 operands the rule may add E, the oracle's bound on what an 8-product
group adder loses when it aligns every product to the group's largest one
(see mx_oracle.c).  gfx950's block-scaled MFMA adds E4M3 products that way,
so an E4M3 result can miss 1e-5 * T by at most E; ``compare`` reports the
elements that pass only thanks to E separately (``n_plain_bad``).
"""
import ctypes
import os

import numpy as np

FMT_E2M1 = 1
FMT_E4M3 = 2
FMT_E5M2 = 3
FMT_E2M3 = 4
FMT_E3M2 = 5
_FORMATS = (FMT_E2M1, FMT_E4M3, FMT_E5M2, FMT_E2M3, FMT_E3M2)


def _row_bytes(fmt, K):
    if fmt == FMT_E2M1:
        return K // 2
    if fmt in (FMT_E2M3, FMT_E3M2):
        return K // 4 * 3
    return K

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

REL_TOL = 1e-5


def _bind(lib):
    u8p = ctypes.POINTER(ctypes.c_uint8)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.mxo_e2m1_value.restype = ctypes.c_double
    lib.mxo_e2m1_value.argtypes = [ctypes.c_uint]
    lib.mxo_e4m3_value.restype = ctypes.c_double
    lib.mxo_e4m3_value.argtypes = [ctypes.c_uint]
    lib.mxo_e5m2_value.restype = ctypes.c_double
    lib.mxo_e5m2_value.argtypes = [ctypes.c_uint]
    lib.mxo_e8m0_value.restype = ctypes.c_double
    lib.mxo_e8m0_value.argtypes = [ctypes.c_uint]
    lib.mxo_tables.restype = None
    lib.mxo_tables.argtypes = [dp, dp]
    lib.mxo_block_contrib.restype = ctypes.c_double
    lib.mxo_block_contrib.argtypes = [ctypes.c_int, i64, u8p, u8p, u8p, u8p,
                                      i64, i64, i64, dp]
    lib.mxo_bf16_value.restype = ctypes.c_double
    lib.mxo_bf16_value.argtypes = [ctypes.c_uint]
    u16p = ctypes.POINTER(ctypes.c_uint16)
    lib.mxo_gemm_bf16.restype = ctypes.c_int
    lib.mxo_gemm_bf16.argtypes = [i64, i64, i64, u16p, u16p, ctypes.POINTER(ctypes.c_int64), i64,
                                  dp, dp, ctypes.c_int]
    lib.mxo_quantize.restype = ctypes.c_int
    lib.mxo_quantize.argtypes = [ctypes.c_int, i64, i64, dp, u8p, u8p]
    lib.mxo_gemm.restype = ctypes.c_int
    lib.mxo_gemm.argtypes = [ctypes.c_int, i64, i64, i64, u8p, u8p, u8p, u8p,
                             ctypes.POINTER(ctypes.c_int64), i64, dp, dp, dp,
                             ctypes.c_int]
    lib.mxo_gemm_ab.restype = ctypes.c_int
    lib.mxo_gemm_ab.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, u8p, u8p, u8p, u8p,
                                ctypes.POINTER(ctypes.c_int64), i64, dp, dp, dp,
                                ctypes.c_int]
    return lib


def _u8(a):
    a = np.ascontiguousarray(a, dtype=np.uint8)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def _check_shapes(fmt, A, As, B, Bs, K, fmt_b=None):
    fmt_b = fmt if fmt_b is None else fmt_b
    if fmt not in _FORMATS or fmt_b not in _FORMATS:
        raise ValueError("formats must be E2M1, E4M3 or E5M2 (any pair)")
    rba, rbb = _row_bytes(fmt, K), _row_bytes(fmt_b, K)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != rba or B.shape[1] != rbb:
        raise ValueError("A and B must be 2-D with %d and %d bytes per row" % (rba, rbb))
    if As.shape != (A.shape[0], K // 32) or Bs.shape != (B.shape[0], K // 32):
        raise ValueError("scale arrays must be rows x K/32")


class Oracle:
    """The oracle's entry points, bound to one build of ``mx_oracle.c``."""

    def __init__(self, path=LIB_PATH):
        if not os.path.exists(path):
            raise FileNotFoundError(
                "%s is not built (run oracle/build.py or __graft_entry__.build())" % path)
        self.lib = _bind(ctypes.CDLL(path))

    def e2m1_value(self, code):
        return self.lib.mxo_e2m1_value(int(code))

    def e4m3_value(self, code):
        return self.lib.mxo_e4m3_value(int(code))

    def e5m2_value(self, code):
        return self.lib.mxo_e5m2_value(int(code))

    def e8m0_value(self, byte):
        return self.lib.mxo_e8m0_value(int(byte))

    def tables(self):
        """(e2m1[16], e4m3[256]) decode tables as float64 arrays."""
        t4 = np.zeros(16, np.float64)
        t8 = np.zeros(256, np.float64)
        dp = ctypes.POINTER(ctypes.c_double)
        self.lib.mxo_tables(t4.ctypes.data_as(dp), t8.ctypes.data_as(dp))
        return t4, t8

    def gemm(self, fmt, A, A_scale, B, B_scale, K, rows=None, threads=0,
             group_bound=False, fmt_b=None):
        """Return (C, T), or (C, T, E) with ``group_bound``, as float64 arrays
        of shape (len(rows) or M, N).

        A: uint8 M x (K/2 or K); B: uint8 N x (K/2 or K); scales uint8
        rows x K/32.  ``fmt`` is A's element format, and B's too unless
        ``fmt_b`` names another (mixed formats).  ``rows`` selects a subset of
        A's rows; ``threads`` <= 0 lets OpenMP choose."""
        fmt_b = fmt if fmt_b is None else fmt_b
        A, pa = _u8(A)
        As, pas = _u8(A_scale)
        B, pb = _u8(B)
        Bs, pbs = _u8(B_scale)
        _check_shapes(fmt, A, As, B, Bs, K, fmt_b)
        M, N = A.shape[0], B.shape[0]
        if rows is None:
            nrows, prow = M, None
        else:
            rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
            nrows = rows_arr.shape[0]
            prow = rows_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        C = np.zeros((nrows, N), np.float64)
        T = np.zeros((nrows, N), np.float64)
        E = np.zeros((nrows, N), np.float64) if group_bound else None
        dp = ctypes.POINTER(ctypes.c_double)
        if fmt_b == fmt:
            rc = self.lib.mxo_gemm(fmt, M, N, K, pa, pas, pb, pbs, prow, nrows,
                                   C.ctypes.data_as(dp), T.ctypes.data_as(dp),
                                   E.ctypes.data_as(dp) if group_bound else None,
                                   int(threads))
        else:
            rc = self.lib.mxo_gemm_ab(fmt, fmt_b, M, N, K, pa, pas, pb, pbs, prow, nrows,
                                      C.ctypes.data_as(dp), T.ctypes.data_as(dp),
                                      E.ctypes.data_as(dp) if group_bound else None,
                                      int(threads))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return (C, T, E) if group_bound else (C, T)

    def gemm_grouped(self, fmt, A, A_scale, B, B_scale, K, group_rows, rows=None,
                     threads=0, group_bound=False, fmt_b=None):
        """Grouped GEMM of a mixture-of-experts layer, by its definition: A's
        rows come in consecutive groups of ``group_rows[g]`` rows, B holds G
        weights of N rows each (weight g = rows g*N .. g*N+N-1), and group g's
        rows of C are A_g * B_g^T, each an ordinary ``gemm`` (with B in
        ``fmt_b`` when given).  ``rows`` selects A rows by their index in A.
        Returns (C, T) or (C, T, E), with the rows in A's (or ``rows``')
        order."""
        group_rows = [int(r) for r in group_rows]
        G = len(group_rows)
        if G < 1 or min(group_rows) < 0 or sum(group_rows) != A.shape[0]:
            raise ValueError("group_rows must be >= 0 and sum to A's row count")
        if B.shape[0] % G or B_scale.shape[0] != B.shape[0]:
            raise ValueError("B must hold G weights of equal row count")
        N = B.shape[0] // G
        want = np.arange(A.shape[0]) if rows is None else np.asarray(rows, np.int64)
        nout = 3 if group_bound else 2
        out = [np.zeros((want.shape[0], N), np.float64) for _ in range(nout)]
        r0 = 0
        for g, m in enumerate(group_rows):
            pos = np.nonzero((want >= r0) & (want < r0 + m))[0]
            if pos.size:
                res = self.gemm(fmt, A[r0:r0 + m], A_scale[r0:r0 + m], B[g * N:(g + 1) * N],
                                B_scale[g * N:(g + 1) * N], K, rows=want[pos] - r0,
                                threads=threads, group_bound=group_bound, fmt_b=fmt_b)
                for o, r in zip(out, res):
                    o[pos] = r
            r0 += m
        return tuple(out)

    def gemm_grouped_bf16(self, A, B, group_rows, rows=None, threads=0):
        """Grouped dense BF16 GEMM, by its definition: A's rows come in
        consecutive groups of ``group_rows[g]`` rows, B holds G weights of N
        rows each (weight g = rows g*N .. g*N+N-1), and group g's rows of C
        are A_g * B_g^T, each an ordinary ``gemm_bf16``.  ``rows`` selects A
        rows by their index in A.  Returns (C, T) with the rows in A's (or
        ``rows``') order."""
        group_rows = [int(r) for r in group_rows]
        G = len(group_rows)
        if G < 1 or min(group_rows) < 0 or sum(group_rows) != A.shape[0]:
            raise ValueError("group_rows must be >= 0 and sum to A's row count")
        if B.shape[0] % G:
            raise ValueError("B must hold G weights of equal row count")
        N = B.shape[0] // G
        want = np.arange(A.shape[0]) if rows is None else np.asarray(rows, np.int64)
        C = np.zeros((want.shape[0], N), np.float64)
        T = np.zeros((want.shape[0], N), np.float64)
        r0 = 0
        for g, m in enumerate(group_rows):
            pos = np.nonzero((want >= r0) & (want < r0 + m))[0]
            if pos.size:
                Cg, Tg = self.gemm_bf16(A[r0:r0 + m], B[g * N:(g + 1) * N], rows=want[pos] - r0,
                                        threads=threads)
                C[pos] = Cg
                T[pos] = Tg
            r0 += m
        return C, T

    def bf16_value(self, bits):
        return self.lib.mxo_bf16_value(int(bits))

    def gemm_bf16(self, A, B, rows=None, threads=0):
        """BF16 dense NT GEMM: A (M x K) and B (N x K) uint16 arrays of BF16
        bit patterns -> (C, T) float64, rows of A as in ``gemm``."""
        A = np.ascontiguousarray(A, dtype=np.uint16)
        B = np.ascontiguousarray(B, dtype=np.uint16)
        if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[1]:
            raise ValueError("A and B must be 2-D with the same K")
        M, K = A.shape
        N = B.shape[0]
        if rows is None:
            nrows, prow = M, None
        else:
            rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
            nrows = rows_arr.shape[0]
            prow = rows_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        C = np.zeros((nrows, N), np.float64)
        T = np.zeros((nrows, N), np.float64)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        dp = ctypes.POINTER(ctypes.c_double)
        rc = self.lib.mxo_gemm_bf16(M, N, K, A.ctypes.data_as(u16p), B.ctypes.data_as(u16p),
                                    prow, nrows, C.ctypes.data_as(dp), T.ctypes.data_as(dp),
                                    int(threads))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return C, T

    def quantize(self, fmt, X):
        """MX-quantize X (rows x K, values exactly representable in float64,
        K a multiple of 32) -> (codes, scales) uint8 arrays: codes rows x K
        (E4M3, E5M2), rows x K/2 (E2M1) or rows x 3K/4 (E2M3, E3M2), scales
        rows x K/32."""
        X = np.ascontiguousarray(X, dtype=np.float64)
        if X.ndim != 2 or X.shape[1] % 32:
            raise ValueError("X must be 2-D with a multiple of 32 columns")
        rows, K = X.shape
        Q = np.zeros((rows, _row_bytes(fmt, K)), np.uint8)
        S = np.zeros((rows, K // 32), np.uint8)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        rc = self.lib.mxo_quantize(int(fmt), rows, K, X.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                   Q.ctypes.data_as(u8p), S.ctypes.data_as(u8p))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return Q, S

    def block_contrib(self, fmt, A, A_scale, B, B_scale, K, m, n, b):
        """(contribution, magnitude) of block b to C[m][n]."""
        A, pa = _u8(A)
        As, pas = _u8(A_scale)
        B, pb = _u8(B)
        Bs, pbs = _u8(B_scale)
        _check_shapes(fmt, A, As, B, Bs, K)
        t = ctypes.c_double(0.0)
        c = self.lib.mxo_block_contrib(fmt, K, pa, pas, pb, pbs, int(m), int(n),
                                       int(b), ctypes.byref(t))
        return c, t.value


_default = None


def default():
    """The oracle built from this directory's ``mx_oracle.c``."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def gemm(*args, **kw):
    return default().gemm(*args, **kw)


def gemm_grouped(*args, **kw):
    return default().gemm_grouped(*args, **kw)


def block_contrib(*args, **kw):
    return default().block_contrib(*args, **kw)


def quantize(*args, **kw):
    return default().quantize(*args, **kw)


def gemm_bf16(*args, **kw):
    return default().gemm_bf16(*args, **kw)


def gemm_grouped_bf16(*args, **kw):
    return default().gemm_grouped_bf16(*args, **kw)


def tables():
    return default().tables()


def bf16_ulp(x):
    """Spacing of bfloat16 numbers in the binade of each |x| (float64 array):
    2^(max(floor(log2|x|), -126) - 7), and 2^-133 (the subnormal spacing)
    for x = 0."""
    x = np.abs(np.asarray(x, np.float64))
    _, e = np.frexp(x)                       # x = f * 2^e, f in [0.5, 1)
    expo = np.maximum(e - 1, -126)           # floor(log2 |x|), clamped
    ulp = np.ldexp(1.0, expo - 7)
    return np.where(x == 0, np.ldexp(1.0, -133), ulp)


def bound(C, T, out_is_bf16, E=None):
    """Allowed |gpu - C| per element: 1e-5 * T, plus one bfloat16 ulp of C
    for BF16 output, plus E when given."""
    b = REL_TOL * np.asarray(T, np.float64)
    if E is not None:
        b = b + np.asarray(E, np.float64)
    if out_is_bf16:
        b = b + bf16_ulp(C)
    return b


def round_to_output(C, out_is_bf16):
    """C (float64) as the output type holds it: rounded to float32 (nearest
    even), then for BF16 output to bfloat16 (nearest even, from the float32
    bits, as the device converts its FP32 accumulator).  Values beyond the
    type's range become infinities; NaN stays NaN.  Returned as float64."""
    C = np.asarray(C, np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        c32 = C.astype(np.float32)
    if out_is_bf16:
        bits = c32.view(np.uint32).astype(np.uint64)
        rnd = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
        finite = np.isfinite(c32)
        bits = np.where(finite, rnd, bits & 0xFFFF0000).astype(np.uint32)
        c32 = bits.view(np.float32)
    return c32.astype(np.float64)


def compare(gpu, C, T, out_is_bf16, E=None):
    """Per-element acceptance.

    An element whose oracle value is NaN must be NaN on the GPU, and one
    whose value the output type cannot hold (it rounds to an infinity) must
    be that infinity; every other element must be finite and meet
    |gpu - C| <= bound(C, T, out_is_bf16, E) (with T == 0 and FP32 output
    that is an exact zero; +0 and -0 are equal).  Returns a dict with the
    worst error/bound ratio over the finite elements, the number of failing
    elements and the first failing index (or None); when E is given, also how
    many elements fail the plain bound (without E) and the worst ratio
    against it."""
    g = np.asarray(gpu, np.float64)
    C = np.asarray(C, np.float64)
    if g.shape != C.shape:
        raise ValueError("shape mismatch %s vs %s" % (g.shape, C.shape))
    ref = round_to_output(C, out_is_bf16)
    cnan = np.isnan(C)
    cinf = ~cnan & np.isinf(ref)
    special = cnan | cinf
    special_bad = special & ~np.where(cnan, np.isnan(g), g == ref)
    with np.errstate(invalid="ignore"):
        err = np.where(special, 0.0, np.abs(g - np.where(special, 0.0, C)))

    def judge(lim):
        lim = np.where(special, 0.0, lim)
        # A zero limit (T == 0, FP32 output) demands an exact zero.
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = np.where(lim > 0, err / lim, np.where(err == 0, 0.0, np.inf))
        bad = special_bad | (~special & ~(err <= lim))
        finite = ratio[~special]
        return (float(np.max(finite)) if finite.size else 0.0), bad

    worst, bad = judge(bound(C, T, out_is_bf16, E))
    nbad = int(bad.sum())
    first = tuple(int(i) for i in np.argwhere(bad)[0]) if nbad else None
    res = {"max_ratio": worst, "n_bad": nbad, "first_bad": first}
    if E is not None:
        pw, pbad = judge(bound(C, T, out_is_bf16))
        res["plain_max_ratio"] = pw
        res["n_plain_bad"] = int(pbad.sum())
    return res
