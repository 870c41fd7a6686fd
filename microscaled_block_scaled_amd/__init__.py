"""Python binding of libmxgemm.so, the gfx950 MX block-scaled NT GEMM.

Argument marshalling only: every step of the GEMM runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  There is no
fallback: if the library is missing, or the device is not a gfx950, calls
raise.

    C = mx_gemm(a, a_scale, b, b_scale, fmt, out_dtype=torch.bfloat16)

a: (M, K/2) uint8 for MXFP4 (E2M1, two elements per byte, element 2i in the
   low nibble), (M, K) uint8 / float8_e4m3fn for MXFP8 (E4M3; or E5M2,
   FMT_E5M2, as uint8 / float8_e5m2), or (M, 3K/4) uint8 for MXFP6 (FMT_E2M3,
   FMT_E3M2; element k in bits 6k .. 6k+5 of the row); ``fmt_b`` gives B its
   own format;
b: (N, ...) likewise; a_scale: (M, K/32) uint8 E8M0; b_scale: (N, K/32).
Returns C = A * B^T, (M, N), float32 or bfloat16.

    q, q_scale = mx_quantize(x, fmt)

quantizes a float32 / bfloat16 matrix into that operand layout (OCP MX rule).

    C = mx_gemm_grouped(a, a_scale, b, b_scale, group_rows, fmt)

multiplies consecutive row groups of a by their own weights: b is
(G*N, ...), rows g*N .. g*N+N-1 being group g's weight.

    C = mx_gemm_bf16(a, b, out_dtype=torch.bfloat16)

is the dense BF16 GEMM on the same tile kernels: a (M, K) and b (N, K)
bfloat16, no scales, K a multiple of 16.
"""
import ctypes
import os

FMT_E2M1 = 1
FMT_E4M3 = 2
FMT_E5M2 = 3
FMT_E2M3 = 4          # MXFP6, packed 4 elements per 3 bytes
FMT_E3M2 = 5
OUT_FP32 = 1
OUT_BF16 = 2
MAX_DIM = 1 << 30     # largest M or N
MAX_K = 1 << 24       # largest K
MAX_K_BF16 = 1 << 23  # largest K of the dense BF16 GEMM
MAX_SPLIT_K = 8       # largest forced K split (mx_gemm_tile)
MAX_GROUPS = 256      # most groups of mx_gemm_grouped
VARIANT_TILE = 1
VARIANT_DECODE = 2    # the decode kernel: M <= DECODE_TILE rows, E2M1 / E4M3 / E5M2
DECODE_TILE = 32      # its tile: DECODE_TILE columns of C (all M rows) per workgroup

MX_OK = 0
MX_ERR_FORMAT = -1
MX_ERR_OUT_DTYPE = -2
MX_ERR_SHAPE = -3
MX_ERR_NULL = -4
MX_ERR_ALIGN = -5
MX_ERR_NO_DEVICE = -6
MX_ERR_ARCH = -7
MX_ERR_ALLOC = -8
MX_ERR_LAUNCH = -9
MX_ERR_IN_DTYPE = -10
MX_ERR_SCRATCH = -11
NOALLOC_SCRATCH_BYTES = 32 << 20   # mx_gemm_noalloc's fixed split-K scratch per device

IN_FP32 = 1
IN_BF16 = 2

_VALUE_ERRORS = (MX_ERR_FORMAT, MX_ERR_OUT_DTYPE, MX_ERR_SHAPE, MX_ERR_NULL, MX_ERR_ALIGN,
                 MX_ERR_IN_DTYPE, MX_ERR_SCRATCH)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxgemm.so")
_lib = None


class MxPlan(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int), ("tile_m", ctypes.c_int),
                ("tile_n", ctypes.c_int), ("split_k", ctypes.c_int),
                ("threads", ctypes.c_int), ("lds_bytes", ctypes.c_int),
                ("workgroups", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


def lib():
    """The loaded libmxgemm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libmxgemm.so is not built; run microscaled_block_scaled_amd/build.py "
            "(or __graft_entry__.build())")
    # torch ships its own HIP runtime.  Load it first, so the library's
    # libamdhip64.so.7 dependency resolves to that same runtime: two HIP (and
    # HSA) runtimes in one process would not share devices, streams or memory.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    L.mx_gemm.restype = ctypes.c_int
    L.mx_gemm.argtypes = [ctypes.c_int, i64, i64, i64, vp, vp, vp, vp, vp,
                          ctypes.c_int, vp]
    L.mx_strerror.restype = ctypes.c_char_p
    L.mx_strerror.argtypes = [ctypes.c_int]
    L.mx_gemm_plan.restype = ctypes.c_int
    L.mx_gemm_plan.argtypes = [ctypes.c_int, i64, i64, i64, ctypes.c_int,
                               ctypes.POINTER(MxPlan)]
    L.mx_tile_shapes.restype = ctypes.c_int
    L.mx_tile_shapes.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int]
    L.mx_gemm_tile.restype = ctypes.c_int
    L.mx_gemm_tile.argtypes = [ctypes.c_int, i64, i64, i64, vp, vp, vp, vp, vp,
                               ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    L.mx_quantize.restype = ctypes.c_int
    L.mx_quantize.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, vp, vp, vp, vp]
    L.mx_gemm_mixed.restype = ctypes.c_int
    L.mx_gemm_mixed.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, vp, vp, vp, vp, vp,
                                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    L.mx_gemm_grouped_plan.restype = ctypes.c_int
    L.mx_gemm_grouped_plan.argtypes = [ctypes.c_int, i64, ctypes.POINTER(i64), i64, i64,
                                       ctypes.c_int, ctypes.POINTER(MxPlan)]
    L.mx_gemm_bf16.restype = ctypes.c_int
    L.mx_gemm_bf16.argtypes = [i64, i64, i64, vp, vp, vp, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, ctypes.c_int, vp]
    L.mx_gemm_bf16_plan.restype = ctypes.c_int
    L.mx_gemm_bf16_plan.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.POINTER(MxPlan)]
    L.mx_gemm_grouped_bf16.restype = ctypes.c_int
    L.mx_gemm_grouped_bf16.argtypes = [i64, ctypes.POINTER(i64), i64, i64, vp, vp, vp,
                                       ctypes.c_int, vp]
    L.mx_gemm_grouped_bf16_plan.restype = ctypes.c_int
    L.mx_gemm_grouped_bf16_plan.argtypes = [i64, ctypes.POINTER(i64), i64, i64, ctypes.c_int,
                                            ctypes.POINTER(MxPlan)]
    L.mx_gemm_grouped_mixed.restype = ctypes.c_int
    L.mx_gemm_grouped_mixed.argtypes = [ctypes.c_int, ctypes.c_int, i64, ctypes.POINTER(i64), i64,
                                        i64, vp, vp, vp, vp, vp, ctypes.c_int, vp]
    L.mx_gemm_grouped.restype = ctypes.c_int
    L.mx_gemm_grouped.argtypes = [ctypes.c_int, i64, ctypes.POINTER(i64), i64, i64, vp, vp,
                                  vp, vp, vp, ctypes.c_int, vp]
    L.mx_gemm_noalloc.restype = ctypes.c_int
    L.mx_gemm_noalloc.argtypes = [ctypes.c_int, i64, i64, i64, vp, vp, vp, vp, vp,
                                  ctypes.c_int, vp]
    L.mx_debug_fail_allocations.restype = None
    L.mx_debug_fail_allocations.argtypes = [ctypes.c_int]
    L.mx_mfma_ceiling.restype = ctypes.c_int
    L.mx_mfma_ceiling.argtypes = [ctypes.c_int, i64, ctypes.c_int, vp, vp]
    L.mx_hbm_read_ceiling.restype = ctypes.c_int
    L.mx_hbm_read_ceiling.argtypes = [vp, i64, vp, vp]
    _lib = L
    return L


def strerror(code):
    return lib().mx_strerror(int(code)).decode()


def _raise(code):
    msg = "mx_gemm: %s (code %d)" % (strerror(code), code)
    if code in _VALUE_ERRORS:
        raise ValueError(msg)
    raise RuntimeError(msg)


def plan(fmt, M, N, K, out_dtype=OUT_BF16):
    """How the library would run this problem (a dict); host logic only."""
    p = MxPlan()
    rc = lib().mx_gemm_plan(int(fmt), int(M), int(N), int(K), int(out_dtype),
                            ctypes.byref(p))
    if rc != MX_OK:
        _raise(rc)
    return p.as_dict()


def tile_shapes():
    """[(tile_m, tile_n), ...] the library has kernels for."""
    n = lib().mx_tile_shapes(None, 0)
    buf = (ctypes.c_int * (2 * n))()
    lib().mx_tile_shapes(buf, n)
    return [(buf[2 * i], buf[2 * i + 1]) for i in range(n)]


def gemm_ptr(fmt, M, N, K, A, A_scale, B, B_scale, C, out_dtype, stream=0, tile=None,
             split_k=0, fmt_b=None):
    """Raw entry point: integer device addresses, returns the status code.
    ``tile=(tile_m, tile_n)`` forces a tile shape, and ``split_k`` (with a
    tile) the number of K slices, 0 meaning the plan's choice (mx_gemm_tile).
    ``fmt_b`` other than ``fmt`` gives B its own format (mx_gemm_mixed)."""
    if fmt_b is not None and fmt_b != fmt:
        tm, tn = tile if tile is not None else (0, 0)
        return lib().mx_gemm_mixed(int(fmt), int(fmt_b), int(M), int(N), int(K), A, A_scale,
                                   B, B_scale, C, int(out_dtype), int(tm), int(tn),
                                   int(split_k), stream or None)
    if tile is not None:
        return lib().mx_gemm_tile(int(fmt), int(M), int(N), int(K), A, A_scale, B,
                                  B_scale, C, int(out_dtype), int(tile[0]), int(tile[1]),
                                  int(split_k), stream or None)
    return lib().mx_gemm(int(fmt), int(M), int(N), int(K), A, A_scale, B,
                         B_scale, C, int(out_dtype), stream or None)


def _out_code(out_dtype):
    import torch
    if out_dtype in (torch.float32, OUT_FP32):
        return OUT_FP32, torch.float32
    if out_dtype in (torch.bfloat16, OUT_BF16):
        return OUT_BF16, torch.bfloat16
    raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")


def _as_u8(t, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn, torch.float8_e5m2, torch.float8_e8m0fnu,
                       getattr(torch, "float4_e2m1fn_x2", torch.uint8)):
        raise ValueError("%s must hold bytes (uint8 or an 8-bit float view), got %s"
                         % (name, t.dtype))
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous (no stride arguments; copy first)" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    return t


def _row_bytes(fmt, K):
    """Bytes of an operand row of K values in format fmt."""
    if fmt == FMT_E2M1:
        return K // 2
    if fmt in (FMT_E2M3, FMT_E3M2):
        return K // 4 * 3
    return K


def _k_of(fmt, row_bytes):
    """K-values in an operand row of row_bytes bytes; raises ValueError when
    no K has rows of exactly that length (an FP6 row must be a multiple of 3
    bytes, an E2M1 row any length)."""
    if fmt == FMT_E2M1:
        K = row_bytes * 2
    elif fmt in (FMT_E2M3, FMT_E3M2):
        K = row_bytes // 3 * 4
    else:
        K = row_bytes
    if _row_bytes(fmt, K) != row_bytes:
        raise ValueError("a row of %d bytes holds no whole number of format-%d elements "
                         "(FP6 rows are 3*K/4 bytes)" % (row_bytes, fmt))
    return K


def mx_gemm(a, a_scale, b, b_scale, fmt, out_dtype=None, out=None, stream=None,
            tile=None, split_k=0, fmt_b=None):
    """C = A * B^T for MX-quantized A (M x K) and B (N x K); see module doc.
    ``fmt`` is the element format of A, and of B unless ``fmt_b`` gives B
    another one (E4M3 x E2M1 and the reverse).  ``tile=(tile_m, tile_n)``
    forces one of ``tile_shapes()``, and with it ``split_k`` the number of K
    slices (0: the plan's choice); ``tile=(DECODE_TILE, DECODE_TILE)`` forces
    the decode kernel (M <= DECODE_TILE, E2M1 / E4M3 / E5M2, K >= 512, no
    split)."""
    import torch
    if out_dtype is None:
        out_dtype = torch.bfloat16
    fmt_b = fmt if fmt_b is None else fmt_b
    fmts = (FMT_E2M1, FMT_E4M3, FMT_E5M2, FMT_E2M3, FMT_E3M2)
    if fmt not in fmts or fmt_b not in fmts:
        raise ValueError("fmt and fmt_b must be one of the MX element formats")
    code, tdt = _out_code(out_dtype)
    a, b = _as_u8(a, "a"), _as_u8(b, "b")
    a_scale, b_scale = _as_u8(a_scale, "a_scale"), _as_u8(b_scale, "b_scale")
    M, N = a.shape[0], b.shape[0]
    K = _k_of(fmt, a.shape[1])
    if _k_of(fmt_b, b.shape[1]) != K:
        raise ValueError("a and b disagree on K")
    if tuple(a_scale.shape) != (M, K // 32) or tuple(b_scale.shape) != (N, K // 32):
        raise ValueError("scales must be (rows, K/32) = (%d, %d) and (%d, %d)"
                         % (M, K // 32, N, K // 32))
    dev = a.device
    for t in (b, a_scale, b_scale):
        if t.device != dev:
            raise ValueError("all operands must be on the same device")
    if out is None:
        out = torch.empty((M, N), dtype=tdt, device=dev)
    elif out.dtype != tdt or tuple(out.shape) != (M, N) or not out.is_contiguous() \
            or out.device != dev:
        raise ValueError("out must be a contiguous (M, N) %s tensor on %s" % (tdt, dev))
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        rc = gemm_ptr(fmt, M, N, K, a.data_ptr(), a_scale.data_ptr(), b.data_ptr(),
                      b_scale.data_ptr(), out.data_ptr(), code, stream, tile, split_k, fmt_b)
    if rc != MX_OK:
        _raise(rc)
    return out


def plan_bf16(M, N, K, out_dtype=OUT_BF16):
    """How mx_gemm_bf16 would run this problem (a dict); host logic only."""
    p = MxPlan()
    rc = lib().mx_gemm_bf16_plan(int(M), int(N), int(K), int(out_dtype), ctypes.byref(p))
    if rc != MX_OK:
        _raise(rc)
    return p.as_dict()


def gemm_bf16_ptr(M, N, K, A, B, C, out_dtype, stream=0, tile=None, split_k=0):
    """Raw dense BF16 entry point (mx_gemm_bf16): integer device addresses,
    returns the status code.  ``tile=None`` and ``split_k=0`` take the plan's
    choice."""
    tm, tn = tile if tile is not None else (0, 0)
    return lib().mx_gemm_bf16(int(M), int(N), int(K), A, B, C, int(out_dtype), int(tm),
                              int(tn), int(split_k), stream or None)


def _as_bf16(t, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError("%s must hold bfloat16 values (bfloat16, or int16 / uint16 bit "
                         "patterns), got %s" % (name, t.dtype))
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous (no stride arguments; copy first)" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    return t


def mx_gemm_bf16(a, b, out_dtype=None, out=None, stream=None, tile=None, split_k=0):
    """Dense C = A * B^T for BF16 A (M x K) and B (N x K), FP32 accumulation,
    C in ``out_dtype`` (torch.bfloat16 by default, or torch.float32).
    ``tile=(tile_m, tile_n)`` forces one of ``tile_shapes()``, ``split_k``
    the number of K slices (0: the plan's choice)."""
    import torch
    if out_dtype is None:
        out_dtype = torch.bfloat16
    code, tdt = _out_code(out_dtype)
    a, b = _as_bf16(a, "a"), _as_bf16(b, "b")
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b disagree on K")
    if b.device != a.device:
        raise ValueError("all operands must be on the same device")
    dev = a.device
    if out is None:
        out = torch.empty((M, N), dtype=tdt, device=dev)
    elif out.dtype != tdt or tuple(out.shape) != (M, N) or not out.is_contiguous() \
            or out.device != dev:
        raise ValueError("out must be a contiguous (M, N) %s tensor on %s" % (tdt, dev))
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        rc = gemm_bf16_ptr(M, N, K, a.data_ptr(), b.data_ptr(), out.data_ptr(), code, stream,
                           tile, split_k)
    if rc != MX_OK:
        _raise(rc)
    return out


def gemm_noalloc_ptr(fmt, M, N, K, A, A_scale, B, B_scale, C, out_dtype, stream=0):
    """Raw entry point of mx_gemm_noalloc (no allocation: split-K planes in
    the library's fixed per-device scratch): integer device addresses,
    returns the status code."""
    return lib().mx_gemm_noalloc(int(fmt), int(M), int(N), int(K), A, A_scale, B, B_scale, C,
                                 int(out_dtype), stream or None)


def debug_fail_allocations(count):
    """Test hook: the next `count` split-K workspace allocations fail."""
    lib().mx_debug_fail_allocations(int(count))


# Launch shape and work of mx_mfma_ceiling (include/mxgemm.h).
CEILING_WORKGROUPS = 256
CEILING_THREADS = 512


def ceiling_flops(steps):
    """FLOPs of one mx_mfma_ceiling launch of `steps` K-steps."""
    return CEILING_WORKGROUPS * CEILING_THREADS // 64 * steps * 8 * 2 * 32 * 32 * 64


def ceiling_ptr(fmt, steps, random_data, out, stream=0):
    """Raw entry point of mx_mfma_ceiling (a measurement kernel): status code."""
    return lib().mx_mfma_ceiling(int(fmt), int(steps), int(bool(random_data)), out,
                                 stream or None)


# Launch shape of mx_hbm_read_ceiling (include/mxgemm.h).
HBM_CEILING_WORKGROUPS = 512
HBM_CEILING_THREADS = 256


def hbm_ceiling_ptr(src, nbytes, out, stream=0):
    """Raw entry point of mx_hbm_read_ceiling (a measurement kernel): status code."""
    return lib().mx_hbm_read_ceiling(src, int(nbytes), out, stream or None)


def quantize_ptr(fmt, in_dtype, rows, K, X, Q, Q_scale, stream=0):
    """Raw entry point of mx_quantize: integer device addresses, status code."""
    return lib().mx_quantize(int(fmt), int(in_dtype), int(rows), int(K), X, Q, Q_scale,
                             stream or None)


def mx_quantize(x, fmt, stream=None):
    """MX-quantize x (rows x K float32 or bfloat16 on the GPU, K a multiple of
    32) -> (q, q_scale) uint8 tensors in mx_gemm's operand layout: q is
    rows x K (E4M3, E5M2), rows x K/2 (E2M1) or rows x 3K/4 (E2M3, E3M2),
    q_scale rows x K/32."""
    import torch
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D torch.Tensor")
    if x.dtype == torch.float32:
        code = IN_FP32
    elif x.dtype == torch.bfloat16:
        code = IN_BF16
    else:
        raise ValueError("x must be float32 or bfloat16")
    if not x.is_contiguous() or not x.is_cuda:
        raise ValueError("x must be a contiguous GPU tensor")
    if fmt not in (FMT_E2M1, FMT_E4M3, FMT_E5M2, FMT_E2M3, FMT_E3M2):
        raise ValueError("fmt must be one of the MX element formats")
    rows, K = x.shape
    rb = K // 2 if fmt == FMT_E2M1 else K // 4 * 3 if fmt in (FMT_E2M3, FMT_E3M2) else K
    q = torch.empty((rows, rb), dtype=torch.uint8, device=x.device)
    qs = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    with torch.cuda.device(x.device):
        rc = quantize_ptr(fmt, code, rows, K, x.data_ptr(), q.data_ptr(), qs.data_ptr(), stream)
    if rc != MX_OK:
        _raise(rc)
    return q, qs


def grouped_plan(fmt, group_rows, N, K, out_dtype=OUT_BF16):
    """How mx_gemm_grouped would run these groups (a dict); host logic only."""
    rows = [int(r) for r in group_rows]
    arr = (ctypes.c_int64 * max(len(rows), 1))(*rows)
    p = MxPlan()
    rc = lib().mx_gemm_grouped_plan(int(fmt), len(rows), arr, int(N), int(K), int(out_dtype),
                                    ctypes.byref(p))
    if rc != MX_OK:
        _raise(rc)
    return p.as_dict()


def grouped_ptr(fmt, group_rows, N, K, A, A_scale, B, B_scale, C, out_dtype, stream=0,
                fmt_b=None):
    """Raw entry point of mx_gemm_grouped (mx_gemm_grouped_mixed when
    ``fmt_b`` differs from ``fmt``): a list of row counts, integer device
    addresses; returns the status code."""
    rows = list(group_rows)
    arr = (ctypes.c_int64 * max(len(rows), 1))(*rows)
    if fmt_b is not None and fmt_b != fmt:
        return lib().mx_gemm_grouped_mixed(int(fmt), int(fmt_b), len(rows), arr, int(N), int(K),
                                           A, A_scale, B, B_scale, C, int(out_dtype),
                                           stream or None)
    return lib().mx_gemm_grouped(int(fmt), len(rows), arr, int(N), int(K), A, A_scale, B,
                                 B_scale, C, int(out_dtype), stream or None)


def mx_gemm_grouped(a, a_scale, b, b_scale, group_rows, fmt, out_dtype=None, out=None,
                    stream=None, fmt_b=None):
    """C_g = A_g * B_g^T for consecutive row groups of a (group_rows[g] rows
    each, summing to a's row count; zeros allowed) and the G = len(group_rows)
    weights stacked in b, (G*N, K) in mx_gemm's operand layout.  ``fmt_b``
    gives the weights their own format (the pairs mx_gemm accepts).
    Returns (sum(group_rows), N)."""
    import torch
    if out_dtype is None:
        out_dtype = torch.bfloat16
    fmt_b = fmt if fmt_b is None else fmt_b
    fmts = (FMT_E2M1, FMT_E4M3, FMT_E5M2, FMT_E2M3, FMT_E3M2)
    if fmt not in fmts or fmt_b not in fmts:
        raise ValueError("fmt and fmt_b must be one of the MX element formats")
    code, tdt = _out_code(out_dtype)
    rows = [int(r) for r in group_rows]
    G = len(rows)
    if not 1 <= G <= MAX_GROUPS or min(rows) < 0:
        raise ValueError("group_rows: 1 .. %d non-negative row counts" % MAX_GROUPS)
    a, b = _as_u8(a, "a"), _as_u8(b, "b")
    a_scale, b_scale = _as_u8(a_scale, "a_scale"), _as_u8(b_scale, "b_scale")
    M = a.shape[0]
    if sum(rows) != M:
        raise ValueError("group_rows sum to %d, a has %d rows" % (sum(rows), M))
    if b.shape[0] % G != 0:
        raise ValueError("b's rows are not a multiple of the group count")
    N = b.shape[0] // G
    K = _k_of(fmt, a.shape[1])
    if _k_of(fmt_b, b.shape[1]) != K:
        raise ValueError("a and b disagree on K")
    if tuple(a_scale.shape) != (M, K // 32) or tuple(b_scale.shape) != (G * N, K // 32):
        raise ValueError("scales must be (rows, K/32)")
    dev = a.device
    for t in (b, a_scale, b_scale):
        if t.device != dev:
            raise ValueError("all operands must be on the same device")
    if out is None:
        out = torch.empty((M, N), dtype=tdt, device=dev)
    elif out.dtype != tdt or tuple(out.shape) != (M, N) or not out.is_contiguous() \
            or out.device != dev:
        raise ValueError("out must be a contiguous (M, N) %s tensor on %s" % (tdt, dev))
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        rc = grouped_ptr(fmt, rows, N, K, a.data_ptr(), a_scale.data_ptr(), b.data_ptr(),
                         b_scale.data_ptr(), out.data_ptr(), code, stream, fmt_b)
    if rc != MX_OK:
        _raise(rc)
    return out


def grouped_bf16_plan(group_rows, N, K, out_dtype=OUT_BF16):
    """How mx_gemm_grouped_bf16 would run these groups (a dict); host logic
    only."""
    rows = [int(r) for r in group_rows]
    arr = (ctypes.c_int64 * max(len(rows), 1))(*rows)
    p = MxPlan()
    rc = lib().mx_gemm_grouped_bf16_plan(len(rows), arr, int(N), int(K), int(out_dtype),
                                         ctypes.byref(p))
    if rc != MX_OK:
        _raise(rc)
    return p.as_dict()


def grouped_bf16_ptr(group_rows, N, K, A, B, C, out_dtype, stream=0):
    """Raw entry point of mx_gemm_grouped_bf16; returns the status code."""
    rows = list(group_rows)
    arr = (ctypes.c_int64 * max(len(rows), 1))(*rows)
    return lib().mx_gemm_grouped_bf16(len(rows), arr, int(N), int(K), A, B, C, int(out_dtype),
                                      stream or None)


def mx_gemm_grouped_bf16(a, b, group_rows, out_dtype=None, out=None, stream=None):
    """C_g = A_g * B_g^T for consecutive row groups of BF16 a (group_rows[g]
    rows each) and the G = len(group_rows) BF16 weights stacked in b,
    (G*N, K).  Returns (sum(group_rows), N)."""
    import torch
    if out_dtype is None:
        out_dtype = torch.bfloat16
    code, tdt = _out_code(out_dtype)
    rows = [int(r) for r in group_rows]
    G = len(rows)
    if not 1 <= G <= MAX_GROUPS or min(rows) < 0:
        raise ValueError("group_rows: 1 .. %d non-negative row counts" % MAX_GROUPS)
    a, b = _as_bf16(a, "a"), _as_bf16(b, "b")
    M, K = a.shape
    if sum(rows) != M:
        raise ValueError("group_rows sum to %d, a has %d rows" % (sum(rows), M))
    if b.shape[0] % G != 0:
        raise ValueError("b's rows are not a multiple of the group count")
    N = b.shape[0] // G
    if b.shape[1] != K:
        raise ValueError("a and b disagree on K")
    if b.device != a.device:
        raise ValueError("all operands must be on the same device")
    dev = a.device
    if out is None:
        out = torch.empty((M, N), dtype=tdt, device=dev)
    elif out.dtype != tdt or tuple(out.shape) != (M, N) or not out.is_contiguous() \
            or out.device != dev:
        raise ValueError("out must be a contiguous (M, N) %s tensor on %s" % (tdt, dev))
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        rc = grouped_bf16_ptr(rows, N, K, a.data_ptr(), b.data_ptr(), out.data_ptr(), code,
                              stream)
    if rc != MX_OK:
        _raise(rc)
    return out
