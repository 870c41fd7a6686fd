// mx_quant.h -- gfx950 device code for MX quantization: FP32 or BF16 values
// -> MXFP4 (E2M1) or MXFP8 (E4M3) elements plus one E8M0 scale per 32 values
// along K, by the OCP Microscaling v1.0 conversion rule (the operands the MX
// scaled GEMM of the FlyDSL article starts from; section "Performance numbers
// need their baselines"):
//   per block of 32 values: X = floor(log2 max|x|) - emax (emax 2 for E2M1,
//   8 for E4M3), scale byte s = X + 127 clamped to [0, 254] (0 for an
//   all-zero block), element = x * 2^(127 - s) rounded to the nearest element
//   value, ties to the even code, saturating at 6 / 448, sign kept; a block
//   with a NaN or an infinity gets s = 255 and zero codes.
//
// Rows are dense and K is a multiple of 32, so the matrix is a flat sequence
// of 32-value blocks: block b is input values 32b .. 32b+31, scale byte b,
// and output bytes 32b .. (E4M3) or 16b .. (E2M1).
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

// E2M1 code of y (|y| already at most a little above 6): the number of
// midpoints between neighbouring values that |y| lies above, where a tie
// goes to the even code (0.75, 1.75 and 3.5 round up; 0.25, 1.25, 2.5 and 5
// round down), plus the sign bit.
__device__ __forceinline__ uint32_t e2m1_code(float y)
{
    const float a = fabsf(y);
    uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                 (a >= 3.5f) + (a > 5.0f);
    return c | ((__float_as_uint(y) >> 28) & 8u);
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

// One lane holds V = 4 (FP32 input) or 8 (BF16 input) consecutive values of
// a block, so LPB = 32 / V lanes share a block; a workgroup of 256 threads
// covers 256 / LPB blocks per pass and walks the blocks grid-stride.
template <int FMT, int IN>
__global__ void __launch_bounds__(256)
quantize_kernel(const void *__restrict__ X, uint8_t *__restrict__ Q, uint8_t *__restrict__ S,
                int64_t nblocks)
{
    constexpr int V = (IN == IN_F32) ? 4 : 8;
    constexpr int LPB = 32 / V;
    constexpr int EMAX = (FMT == FP4) ? 2 : 8;
    const int sub = threadIdx.x % LPB;
    const int64_t first = (int64_t)blockIdx.x * (256 / LPB) + threadIdx.x / LPB;
    const int64_t stride = (int64_t)gridDim.x * (256 / LPB);
    for (int64_t b = first; b < nblocks; b += stride) {
        float v[V];
        const int64_t e0 = b * 32 + sub * V;          // first value of the lane
        if (IN == IN_F32) {
            const v4f x = *(const v4f *)((const float *)X + e0);
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = x[i];
        } else {
            const v4i x = *(const v4i *)((const uint16_t *)X + e0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = __uint_as_float((uint32_t)x[i] << 16);
                v[2 * i + 1] = __uint_as_float((uint32_t)x[i] & 0xffff0000u);
            }
        }
        float amax = 0.f;
        int bad = 0;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            bad |= !isfinite(v[i]);
            amax = fmaxf(amax, fabsf(v[i]));
        }
#pragma unroll
        for (int m = 1; m < LPB; m <<= 1) {
            amax = fmaxf(amax, __shfl_xor(amax, m));
            bad |= __shfl_xor(bad, m);
        }
        int s = 0;
        if (bad) s = 255;
        else if (amax > 0.f) s = min(254, max(0, floor_log2(amax) - EMAX + 127));
        if (sub == 0) S[b] = (uint8_t)s;
        float y[V];
#pragma unroll
        for (int i = 0; i < V; ++i) y[i] = bad ? 0.f : ldexpf(v[i], 127 - s);
        if (FMT == FP8) {
            uint32_t w[V / 4];
#pragma unroll
            for (int i = 0; i < V / 4; ++i)
                w[i] = e4m3_pair(y[4 * i], y[4 * i + 1]) |
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
            for (int i = 0; i < V; ++i) w |= e2m1_code(y[i]) << (4 * i);
            if (bad) w = 0;
            if (V == 4) *(uint16_t *)(Q + e0 / 2) = (uint16_t)w;
            else *(uint32_t *)(Q + e0 / 2) = w;
        }
    }
}

}  // namespace mx
