"""Seeded synthetic inputs for the MX block-scaled NT GEMM.

Both the CPU oracle and the GPU library consume what this module produces;
it holds none of the GEMM's arithmetic (no decoding, no dot products, no
scale application).  It draws Gaussian values with numpy and turns them into
MX operands by the OCP Microscaling v1.0 conversion rule:

  * per block of 32 consecutive values along K, shared exponent
    X = floor(log2(max |v|)) - emax_elem  (emax_elem = 2 for E2M1, 8 for E4M3,
    15 for E5M2),
    stored as the E8M0 byte X + 127, clamped to [0, 254] (an all-zero block
    gets byte 0; its elements are zero whatever the byte);
  * each element v / 2^X rounded to nearest, ties to even, saturated at the
    format's largest magnitude (6 for E2M1, 448 for E4M3, 57344 for E5M2).

The pages fix the block size (32 along K), the scale type (E8M0) and that the
measured kernels start from already-quantized inputs (FlyDSL summary page,
sections "Performance numbers need their baselines" and "API compatibility is
not universal input coverage").  They give no quantizer; the OCP rule above
is the plain reading.

Layouts produced (all row-major, dense):
  E4M3 / E5M2   rows x K     uint8, element k in byte k
  E2M1 operand  rows x K/2   uint8, element 2i in the low nibble of byte i
  scales        rows x K/32  uint8, byte b covers K-values 32b .. 32b+31
"""
import numpy as np

FMT_E2M1 = 1
FMT_E4M3 = 2
FMT_E5M2 = 3
FMT_E2M3 = 4
FMT_E3M2 = 5
OUT_FP32 = 1
OUT_BF16 = 2

_EMAX = {FMT_E2M1: 2, FMT_E4M3: 8, FMT_E5M2: 15, FMT_E2M3: 2, FMT_E3M2: 4}
_CHUNK_ROWS = 256

# The workloads.  Shapes come from the serving models the pages measure
# (Llama-3.1-8B, Qwen3-32B, Llama-3.3-70B; FlyDSL summary page, section
# "Whole-request experiments are closer to serving").
CONFIGS = {
    "mxfp4_256": dict(index=0, fmt=FMT_E2M1, M=256, N=256, K=256, out=OUT_FP32,
                      kind="gauss"),
    "mxfp8_llama8b_qkv": dict(index=1, fmt=FMT_E4M3, M=2048, N=6144, K=4096,
                              out=OUT_BF16, kind="gauss"),
    "mxfp4_llama8b_gateup_decode": dict(index=2, fmt=FMT_E2M1, M=256, N=28672,
                                        K=4096, out=OUT_BF16, kind="decode_rowstd"),
    "mxfp4_qwen32b_down": dict(index=3, fmt=FMT_E2M1, M=2048, N=5120, K=25600,
                               out=OUT_FP32, kind="gauss"),
}
for _fmt, _fname in ((FMT_E4M3, "mxfp8"), (FMT_E2M1, "mxfp4")):
    for _m in (8, 64, 256, 2048):
        CONFIGS["%s_llama70b_down_m%d" % (_fname, _m)] = dict(
            index=4, fmt=_fmt, M=_m, N=8192, K=28672, out=OUT_BF16, kind="outlier")


def fmt_name(fmt):
    return {FMT_E2M1: "mxfp4", FMT_E4M3: "mxfp8", FMT_E5M2: "mxfp8_e5m2",
            FMT_E2M3: "mxfp6_e2m3", FMT_E3M2: "mxfp6_e3m2"}[fmt]


def row_bytes(fmt, K):
    if fmt == FMT_E2M1:
        return K // 2
    if fmt in (FMT_E2M3, FMT_E3M2):
        return K // 4 * 3
    return K


# --------------------------------------------------------------------------
# Element encoders (value -> code).  Inputs are already divided by the block
# scale, so they lie in (-2^(emax+1), 2^(emax+1)).

# E2M1 magnitudes by code: 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Rounding up past the
# midpoint between code c and c+1 happens at v > mid when c+1 is odd and at
# v >= mid when c+1 is even (ties to the even code).
_E2M1_MIDS = ((0.25, False), (0.75, True), (1.25, False), (1.75, True),
              (2.5, False), (3.5, True), (5.0, False))


def encode_e2m1(v):
    """float array -> uint8 E2M1 codes (0..15), RNE, saturating at 6."""
    v = np.asarray(v, np.float32)
    mag = np.abs(v)
    code = np.zeros(v.shape, np.uint8)
    for mid, inclusive in _E2M1_MIDS:
        code += (mag >= mid) if inclusive else (mag > mid)
    code |= np.signbit(v).astype(np.uint8) << 3
    return code


def encode_e4m3(v):
    """float array -> uint8 E4M3 codes, RNE, saturating at 448 (torch's
    float8_e4m3fn conversion rounds to nearest even; clamping first keeps
    out-of-range values off its NaN path)."""
    import torch
    v = np.clip(np.asarray(v, np.float32), -448.0, 448.0)
    t = torch.from_numpy(np.ascontiguousarray(v)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def encode_e5m2(v):
    """float array -> uint8 E5M2 codes, RNE, saturating at 57344 (torch's
    float8_e5m2 conversion rounds to nearest even; clamping first keeps
    out-of-range values off its infinity path)."""
    import torch
    v = np.clip(np.asarray(v, np.float32), -57344.0, 57344.0)
    t = torch.from_numpy(np.ascontiguousarray(v)).to(torch.float8_e5m2)
    return t.view(torch.uint8).numpy().copy()


def _fp6_magnitudes(fmt):
    """The 32 non-negative FP6 magnitudes by code (E2M3: 2 exponent bits,
    bias 1, 3 mantissa bits; E3M2: 3 exponent bits, bias 3, 2 mantissa bits;
    exponent field 0 subnormal)."""
    mb = 3 if fmt == FMT_E2M3 else 2
    bias = 1 if fmt == FMT_E2M3 else 3
    out = []
    for c in range(32):
        e, m = c >> mb, c & ((1 << mb) - 1)
        frac = m / float(1 << mb)
        out.append(np.ldexp(frac, 1 - bias) if e == 0 else np.ldexp(1.0 + frac, e - bias))
    return np.array(out)


def encode_fp6(v, fmt):
    """float array -> FP6 codes (0..63, sign bit 5): nearest magnitude, ties
    to the even code, saturating at the largest magnitude."""
    v = np.asarray(v, np.float64)
    mags = _fp6_magnitudes(fmt)
    a = np.minimum(np.abs(v), mags[-1])
    hi = np.clip(np.searchsorted(mags, a), 1, 31)
    lo = hi - 1
    dlo, dhi = a - mags[lo], mags[hi] - a
    code = np.where(dhi < dlo, hi, np.where(dlo < dhi, lo, np.where(hi % 2 == 0, hi, lo)))
    return (code | (np.signbit(v).astype(np.int64) << 5)).astype(np.uint8)


def pack_fp6(codes):
    """rows x K codes -> rows x 3K/4 bytes: element k in bits 6k .. 6k+5 of
    the row's little-endian bit string."""
    c = np.asarray(codes, np.uint32)
    w = c[:, 0::4] | (c[:, 1::4] << 6) | (c[:, 2::4] << 12) | (c[:, 3::4] << 18)
    out = np.empty((c.shape[0], w.shape[1] * 3), np.uint8)
    out[:, 0::3] = w & 255
    out[:, 1::3] = (w >> 8) & 255
    out[:, 2::3] = w >> 16
    return out


def unpack_fp6(packed):
    p = np.asarray(packed, np.uint32)
    w = p[:, 0::3] | (p[:, 1::3] << 8) | (p[:, 2::3] << 16)
    out = np.empty((p.shape[0], w.shape[1] * 4), np.uint8)
    for i in range(4):
        out[:, i::4] = (w >> (6 * i)) & 63
    return out


def quantize(x, fmt):
    """float32 rows x K -> (codes, scales) per the OCP MX conversion rule."""
    x = np.asarray(x, np.float32)
    rows, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    blocks = x.reshape(rows, K // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    _, e = np.frexp(amax)                     # amax = f * 2^e, f in [0.5, 1)
    xexp = e.astype(np.int32) - 1 - _EMAX[fmt]   # floor(log2 amax) - emax
    sbyte = np.clip(xexp + 127, 0, 254)
    sbyte = np.where(amax > 0, sbyte, 0).astype(np.uint8)
    shift = -(sbyte.astype(np.int32) - 127)
    scaled = np.ldexp(blocks, shift[:, :, None]).astype(np.float32)
    scaled = scaled.reshape(rows, K)
    if fmt == FMT_E4M3:
        codes = encode_e4m3(scaled)
    elif fmt == FMT_E5M2:
        codes = encode_e5m2(scaled)
    elif fmt in (FMT_E2M3, FMT_E3M2):
        codes = pack_fp6(encode_fp6(scaled, fmt))
    else:
        c = encode_e2m1(scaled)
        codes = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    return np.ascontiguousarray(codes), np.ascontiguousarray(sbyte)


def pack_e2m1(codes):
    """rows x K nibble codes -> rows x K/2 bytes (element 2i in the low nibble)."""
    codes = np.asarray(codes, np.uint8)
    return np.ascontiguousarray(codes[:, 0::2] | (codes[:, 1::2] << 4))


def unpack_e2m1(packed):
    packed = np.asarray(packed, np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), np.uint8)
    out[:, 0::2] = packed & 15
    out[:, 1::2] = packed >> 4
    return out


# --------------------------------------------------------------------------
# Seeded value sources.  Every matrix has its own numpy Generator seeded with
# (config index, tensor id, stream id); values are drawn row by row in order,
# so a row-chunked draw equals a one-shot draw, and the first m rows of a
# matrix do not depend on how many rows are drawn.

def _rng(cfg_index, tensor, stream):
    return np.random.default_rng([cfg_index, tensor, stream])


def _gen_quantized(rows, K, fmt, cfg_index, tensor, kind):
    vals = _rng(cfg_index, tensor, 0)
    rowstd = None
    if kind == "decode_rowstd" and tensor == 1:
        rowstd = _rng(cfg_index, tensor, 2).uniform(0.5, 2.0, size=rows).astype(np.float32)
    outl = _rng(cfg_index, tensor, 1) if kind == "outlier" else None
    codes = np.empty((rows, row_bytes(fmt, K)), np.uint8)
    scales = np.empty((rows, K // 32), np.uint8)
    for r0 in range(0, rows, _CHUNK_ROWS):
        r1 = min(rows, r0 + _CHUNK_ROWS)
        x = vals.standard_normal((r1 - r0, K), dtype=np.float32)
        if kind == "decode_rowstd":
            if tensor == 0:
                x *= np.float32(0.02)
            else:
                x *= rowstd[r0:r1, None]
        if outl is not None:
            mask = outl.random((r1 - r0, K), dtype=np.float32) < np.float32(0.001)
            x[mask] *= np.float32(50.0)
        codes[r0:r1], scales[r0:r1] = quantize(x, fmt)
    return codes, scales


def make_case(name, M=None):
    """Quantized operands for a named workload.

    Returns dict(fmt, M, N, K, out, A, A_scale, B, B_scale) with numpy uint8
    arrays.  ``M`` may override the row count of A (A's rows are a prefix of
    the workload's A, so a smaller M is a row subset)."""
    cfg = CONFIGS[name]
    fmt, K, N = cfg["fmt"], cfg["K"], cfg["N"]
    M = cfg["M"] if M is None else M
    A, As = _gen_quantized(M, K, fmt, cfg["index"], 0, cfg["kind"])
    B, Bs = _gen_quantized(N, K, fmt, cfg["index"], 1, cfg["kind"])
    return dict(name=name, fmt=fmt, M=M, N=N, K=K, out=cfg["out"],
                A=A, A_scale=As, B=B, B_scale=Bs)


def make_bf16(rows, K, seed, tensor=0):
    """Seeded Gaussian rows x K matrix rounded to BF16 (torch's
    round-to-nearest-even conversion), returned as uint16 bit patterns."""
    import torch
    x = _rng(200 + seed, tensor, 0).standard_normal((rows, K), dtype=np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def make_random(fmt, M, N, K, seed, kind="gauss", scale_lo=None, scale_hi=None):
    """Small seeded Gaussian case of any shape (K a multiple of 32).  With
    scale_lo/scale_hi set, scale bytes are replaced by uniform draws in that
    closed range (to sweep exponents)."""
    A, As = _gen_quantized(M, K, fmt, 100 + seed, 0, kind)
    B, Bs = _gen_quantized(N, K, fmt, 100 + seed, 1, kind)
    if scale_lo is not None:
        r = _rng(100 + seed, 2, 0)
        As = r.integers(scale_lo, scale_hi + 1, size=As.shape).astype(np.uint8)
        Bs = r.integers(scale_lo, scale_hi + 1, size=Bs.shape).astype(np.uint8)
    return dict(name="random", fmt=fmt, M=M, N=N, K=K, A=A, A_scale=As, B=B,
                B_scale=Bs)


def random_codes(fmt, rows, K, seed, pool, tensor=0):
    """Element codes drawn uniformly from ``pool`` (magnitude codes without
    the sign bit) with a random sign each, and scale byte 127 everywhere."""
    r = _rng(200 + seed, tensor, 0)
    pool = np.asarray(pool, np.uint8)
    mag = pool[r.integers(0, len(pool), size=(rows, K))]
    if fmt == FMT_E2M1:
        sign = r.integers(0, 2, size=(rows, K)).astype(np.uint8) << 3
        codes = pack_e2m1(mag | sign)
    else:
        sign = r.integers(0, 2, size=(rows, K)).astype(np.uint8) << 7
        codes = np.ascontiguousarray(mag | sign)
    scales = np.full((rows, K // 32), 127, np.uint8)
    return codes, scales
