// mx_quant6.h -- gfx950 device code for MX quantization to MXFP6: FP32 or
// BF16 values -> E2M3 or E3M2 elements plus one E8M0 scale per 32 values
// along K, by the OCP Microscaling v1.0 conversion rule (as mx_quant.h, with
// emax 2 for E2M3 and 4 for E3M2, saturation at 7.5 / 28, sign kept, a
// block with a NaN or an infinity getting s = 255 and zero codes).
//
// Output rows are bit strings: element k of a row is bits 6k .. 6k+5, little
// endian, so block b of the flat matrix is output bytes 24b .. 24b+23 and a
// lane's 16 values are 12 whole bytes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_quant.h"

namespace mx {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// FP6 code of y (finite) without a NaN path: the nearest element value,
// ties to the even code, saturating, sign bit 5 from y.  With a = |y|
// clamped to the largest value and bias 1 - emin:
//  * a >= 2^emin (normal): the FP32 significand rounded to MAN bits, ties
//    to even, by adding 2^(SH-1) - 1 plus the lowest kept bit (SH = 23 -
//    MAN), with the exponent rebased from 127 to the FP6 bias; the code is
//    the rounded bits from bit SH up, and a carry out of the significand
//    moves to the next exponent as it should;
//  * a < 2^emin (subnormal): n = rint(a * 2^(MAN - emin)), the step count,
//    by one FP32 add of 2^(SH + emin), whose binade has that step as its
//    ulp (rounded half to even by the add), less that constant's bits; n up
//    to 2^MAN is also the code of the smallest normal.
// This equals ((e - emin) << MAN) + rint(a * 2^(MAN - e)) with
// e = max(floor(log2 a), emin) for every FP32 a in [0, the largest value]
// (checked exhaustively on the host for both formats) in fewer operations.
template <int F>
__device__ __forceinline__ uint32_t fp6_code(float y)
{
    constexpr int MAN = (F == F6E2) ? 3 : 2;
    constexpr int EMIN = (F == F6E2) ? 0 : -2;            // 1 - bias
    constexpr int SH = 23 - MAN;
    constexpr uint32_t REBIAS = (uint32_t)(127 - (1 - EMIN)) << 23;
    constexpr float MAXV = (F == F6E2) ? 7.5f : 28.f;
    constexpr float MAGIC = (float)(1u << (SH + EMIN));   // 2^20 (E2M3) or 2^19 (E3M2)
    constexpr float SMALLEST_NORMAL = (F == F6E2) ? 1.f : 0.25f;
    const float a = fminf(fabsf(y), MAXV);
    const uint32_t u = __float_as_uint(a);
    const uint32_t nrm = (u + ((1u << (SH - 1)) - 1u) + ((u >> SH) & 1u) - REBIAS) >> SH;
    const uint32_t sub = __float_as_uint(a + MAGIC) - __float_as_uint(MAGIC);
    const uint32_t code = a < SMALLEST_NORMAL ? sub : nrm;
    return code | ((__float_as_uint(y) >> 26) & 32u);
}

// One lane holds 16 consecutive values of a block (two lanes per block,
// lanes 2k and 2k + 1, which always run the same loop trips), grid-stride
// over blocks as quantize_kernel.  The lane's 16 codes are 96 bits, three
// whole dwords, which it stores itself: block b's 24 output bytes are lane
// 0's 12 then lane 1's.
template <int F, int IN>
__global__ void __launch_bounds__(256)
quantize6_kernel(const void *__restrict__ X, uint8_t *__restrict__ Q, uint8_t *__restrict__ S,
                 int64_t nblocks)
{
    constexpr int EMAX = (F == F6E2) ? 2 : 4;
    constexpr int NLD = (IN == IN_F32) ? 4 : 2;            // 16-byte loads per lane
    const int sub = threadIdx.x & 1;
    const int64_t first = (int64_t)blockIdx.x * 128 + threadIdx.x / 2;
    const int64_t stride = (int64_t)gridDim.x * 128;
    for (int64_t b = first; b < nblocks; b += stride) {
        v4i raw[NLD];
#pragma unroll
        for (int r = 0; r < NLD; ++r)
            raw[r] = (IN == IN_F32) ? *(const v4i *)((const float *)X + b * 32 + sub * 16 + 4 * r)
                                    : *(const v4i *)((const uint16_t *)X + b * 32 + sub * 16 + 8 * r);
        float v[16];
#pragma unroll
        for (int r = 0; r < NLD; ++r) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (IN == IN_F32) {
                    v[4 * r + i] = __int_as_float(raw[r][i]);
                } else {
                    v[8 * r + 2 * i] = __uint_as_float((uint32_t)raw[r][i] << 16);
                    v[8 * r + 2 * i + 1] = __uint_as_float((uint32_t)raw[r][i] & 0xffff0000u);
                }
            }
        }
        // The largest magnitude, as the largest sign-cleared bit pattern (the
        // patterns of finite values order as their magnitudes; a NaN or an
        // infinity is at least the infinity pattern, which then stands for
        // it, so a non-finite value makes the block's maximum +inf, as in
        // quantize_kernel).  BF16 pairs are compared two at a time.
        uint32_t mb = 0;
        if constexpr (IN == IN_F32) {
#pragma unroll
            for (int r = 0; r < NLD; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) mb = max(mb, (uint32_t)raw[r][i] & 0x7fffffffu);
        } else {
            u16x2 m2 = {0, 0};
#pragma unroll
            for (int r = 0; r < NLD; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    m2 = __builtin_elementwise_max(
                        m2, __builtin_bit_cast(u16x2, (uint32_t)raw[r][i] & 0x7fff7fffu));
            mb = (uint32_t)max(m2.x, m2.y) << 16;
        }
        float amax = __uint_as_float(min(mb, 0x7f800000u));
        // with the other lane of the block (quad_perm 1,0,3,2)
        amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(
                               0, __float_as_int(amax), 0xB1, 0xF, 0xF, false)));
        const bool bad = amax == __builtin_inff();
        int s = 0;
        if (bad) s = 255;
        else if (amax > 0.f) s = min(254, max(0, floor_log2(amax) - EMAX + 127));
        if (sub == 0) S[b] = (uint8_t)s;
        // four 24-bit groups of four codes, then the 96-bit string's dwords
        uint32_t g[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            g[j] = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                g[j] |= fp6_code<F>(ldexpf(v[4 * j + i], 127 - s)) << (6 * i);
        }
        uint32_t *const q32 = (uint32_t *)(Q + b * 24 + sub * 12);
        q32[0] = bad ? 0u : g[0] | (g[1] << 24);
        q32[1] = bad ? 0u : (g[1] >> 8) | (g[2] << 16);
        q32[2] = bad ? 0u : (g[2] >> 16) | (g[3] << 8);
    }
}

}  // namespace mx
