// mx_quant.h -- gfx950 device code for MX quantization: FP32 or BF16 values
// -> MXFP4 (E2M1) or MXFP8 (E4M3 or E5M2) elements plus one E8M0 scale per
// 32 values along K, by the OCP Microscaling v1.0 conversion rule (the
// operands the MX scaled GEMM of the FlyDSL article starts from; section
// "Performance numbers need their baselines"):
//   per block of 32 values: X = floor(log2 max|x|) - emax (emax 2 for E2M1,
//   8 for E4M3, 15 for E5M2), scale byte s = X + 127 clamped to [0, 254] (0
//   for an all-zero block), element = x * 2^(127 - s) rounded to the nearest
//   element value, ties to the even code, saturating at 6 / 448 / 57344, sign
//   kept; a block with a NaN or an infinity gets s = 255 and zero codes.
//
// Rows are dense and K is a multiple of 32, so the matrix is a flat sequence
// of 32-value blocks: block b is input values 32b .. 32b+31, scale byte b,
// and output bytes 32b .. (E4M3, E5M2) or 16b .. (E2M1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

enum { IN_F32 = 1, IN_BF16 = 2 };   // equal to MX_IN_FP32 / MX_IN_BF16

// floor(log2 a) for a finite a > 0, from its bits (FP32 subnormals included).
__device__ __forceinline__ int floor_log2(float a)
{
    const uint32_t u = __float_as_uint(a);
    const int field = (int)(u >> 23);
    if (field > 0) return field - 127;
    return (31 - __clz((int)(u & 0x7fffffu))) - 149;
}

// Two E2M1 codes in one byte (low nibble: a, high nibble: b): gfx950's
// v_cvt_scalef32_pk_fp4_f32 with scale 1 rounds to nearest, ties to the even
// code, saturates at +-6 and keeps the sign (also of zero).
__device__ __forceinline__ uint32_t e2m1_pair(float a, float b)
{
    return (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xffu;
}

// Two E4M3 codes (low byte: a, high byte: b), round to nearest even, values
// clamped to +-448 first so nothing overflows to NaN (gfx950 converts to the
// OCP E4M3 format).
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b)
{
    a = fminf(fmaxf(a, -448.f), 448.f);
    b = fminf(fmaxf(b, -448.f), 448.f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// Two E5M2 codes (low byte: a, high byte: b), round to nearest even, values
// clamped to +-57344 first so nothing rounds to an infinity (gfx950 converts
// to the OCP E5M2 format).
__device__ __forceinline__ uint32_t e5m2_pair(float a, float b)
{
    a = fminf(fmaxf(a, -57344.f), 57344.f);
    b = fminf(fmaxf(b, -57344.f), 57344.f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false) & 0xffffu;
}

// Maximum over each group of LPB (4 or 8) consecutive lanes, by DPP moves
// within registers: swap neighbours, swap pairs, then (groups of 8) mirror
// each half-row of 8 lanes, which pairs every lane with one of the other
// quad of its group.
template <int LPB>
__device__ __forceinline__ float group_max(float v)
{
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
    if (LPB == 8)
        v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
    return v;
}

// One lane holds V = 4 (FP32 input) or 8 (BF16 input) consecutive values of
// a block, so LPB = 32 / V lanes share a block; a workgroup of 256 threads
// covers 256 / LPB blocks per pass, UNR passes per loop trip (their loads
// issued together), walking the blocks grid-stride.
template <int FMT, int IN>
__global__ void __launch_bounds__(256)
quantize_kernel(const void *__restrict__ X, uint8_t *__restrict__ Q, uint8_t *__restrict__ S,
                int64_t nblocks)
{
    constexpr int V = (IN == IN_F32) ? 4 : 8;
    constexpr int LPB = 32 / V;
    constexpr int EMAX = (FMT == FP4) ? 2 : (FMT == BF8) ? 15 : 8;
    constexpr int UNR = 2;
    const int sub = threadIdx.x % LPB;
    const int64_t first = (int64_t)blockIdx.x * (256 / LPB) + threadIdx.x / LPB;
    const int64_t stride = (int64_t)gridDim.x * (256 / LPB);
    for (int64_t b0 = first; b0 < nblocks; b0 += UNR * stride) {
        v4i raw[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int64_t b = min(b0 + u * stride, nblocks - 1);   // a repeat past the end is not stored
            raw[u] = (IN == IN_F32) ? *(const v4i *)((const float *)X + b * 32 + sub * V)
                                    : *(const v4i *)((const uint16_t *)X + b * 32 + sub * V);
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
        const int64_t b = b0 + u * stride;
        if (b >= nblocks) break;
        float v[V];
        const int64_t e0 = b * 32 + sub * V;          // first value of the lane
        if (IN == IN_F32) {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = __int_as_float(raw[u][i]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = __uint_as_float((uint32_t)raw[u][i] << 16);
                v[2 * i + 1] = __uint_as_float((uint32_t)raw[u][i] & 0xffff0000u);
            }
        }
        // A non-finite value makes the lane's maximum +inf, which no finite
        // block reaches: after the group maximum, amax == inf marks the block.
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < V; ++i)
            amax = fmaxf(amax, isfinite(v[i]) ? fabsf(v[i]) : __builtin_inff());
        amax = group_max<LPB>(amax);
        const bool bad = amax == __builtin_inff();
        int s = 0;
        if (bad) s = 255;
        else if (amax > 0.f) s = min(254, max(0, floor_log2(amax) - EMAX + 127));
        if (sub == 0) S[b] = (uint8_t)s;
        float y[V];
#pragma unroll
        for (int i = 0; i < V; ++i) y[i] = bad ? 0.f : ldexpf(v[i], 127 - s);
        if (FMT != FP4) {
            uint32_t w[V / 4];
#pragma unroll
            for (int i = 0; i < V / 4; ++i)
                w[i] = (FMT == BF8) ? e5m2_pair(y[4 * i], y[4 * i + 1]) |
                                          (e5m2_pair(y[4 * i + 2], y[4 * i + 3]) << 16)
                                    : e4m3_pair(y[4 * i], y[4 * i + 1]) |
                                          (e4m3_pair(y[4 * i + 2], y[4 * i + 3]) << 16);
            if (bad) {
#pragma unroll
                for (int i = 0; i < V / 4; ++i) w[i] = 0;
            }
            if (V == 4) *(uint32_t *)(Q + e0) = w[0];
            else *(uint2 *)(Q + e0) = make_uint2(w[0], w[V / 4 - 1]);
        } else {
            uint32_t w = 0;
#pragma unroll
            for (int i = 0; i < V / 2; ++i) w |= e2m1_pair(y[2 * i], y[2 * i + 1]) << (8 * i);
            if (bad) w = 0;
            if (V == 4) *(uint16_t *)(Q + e0 / 2) = (uint16_t)w;
            else *(uint32_t *)(Q + e0 / 2) = w;
        }
        }
    }
}

}  // namespace mx
