// mx_quant6.h -- gfx950 device code for MX quantization to MXFP6: FP32 or
// BF16 values -> E2M3 or E3M2 elements plus one E8M0 scale per 32 values
// along K, by the OCP Microscaling v1.0 conversion rule (as mx_quant.h, with
// emax 2 for E2M3 and 4 for E3M2, saturation at 7.5 / 28, sign kept, a
// block with a NaN or an infinity getting s = 255 and zero codes).
//
// Output rows are bit strings: element k of a row is bits 6k .. 6k+5, little
// endian, so block b of the flat matrix is output bytes 24b .. 24b+23 and a
// lane's 4 (FP32 input) or 8 (BF16 input) values are 3 or 6 whole bytes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_quant.h"

namespace mx {

// FP6 code of y (finite) without a NaN path: the nearest element value,
// ties to the even code, saturating, sign bit 5 from y.  With
// e = max(floor(log2 |y|), emin) the magnitude is n * 2^(e - MAN) for the
// integer n = rint(|y| * 2^(MAN - e)), exact in FP32 (a power-of-two scaling
// of a value below 2^5) and rounded half to even by rintf; the code is then
// ((e - emin) << MAN) + n, which also covers subnormals (e = emin, n below
// 2^MAN) and n rounding up into the next binade (n = 2^(MAN+1)).
template <int F>
__device__ __forceinline__ uint32_t fp6_code(float y)
{
    constexpr int MAN = (F == F6E2) ? 3 : 2;
    constexpr int EMIN = (F == F6E2) ? 0 : -2;            // 1 - bias
    constexpr float MAXV = (F == F6E2) ? 7.5f : 28.f;
    const float a = fminf(fabsf(y), MAXV);
    const int e = a > 0.f ? max(floor_log2(a), EMIN) : EMIN;
    const uint32_t n = (uint32_t)rintf(ldexpf(a, MAN - e));
    const uint32_t code = ((uint32_t)(e - EMIN) << MAN) + n;
    return code | ((__float_as_uint(y) >> 26) & 32u);
}

// One lane holds V = 4 (FP32 input) or 8 (BF16 input) consecutive values of
// a block, LPB = 32 / V lanes per block, grid-stride over blocks as
// quantize_kernel.  A lane's codes are 3 (V = 4) or 6 (V = 8) bytes, so 4 or
// 2 lanes make 12 bytes, three whole dwords, which those lanes store after
// one DPP move brings each the neighbour's bits it needs.  The lanes of a
// hardware quad always hold one block (LPB is 8 or 4, blocks start at lane
// multiples of LPB), so they run the same loop trips and the DPP sources
// are active.
template <int F, int IN>
__global__ void __launch_bounds__(256)
quantize6_kernel(const void *__restrict__ X, uint8_t *__restrict__ Q, uint8_t *__restrict__ S,
                 int64_t nblocks)
{
    constexpr int V = (IN == IN_F32) ? 4 : 8;
    constexpr int LPB = 32 / V;
    constexpr int EMAX = (F == F6E2) ? 2 : 4;
    const int sub = threadIdx.x % LPB;
    const int64_t first = (int64_t)blockIdx.x * (256 / LPB) + threadIdx.x / LPB;
    const int64_t stride = (int64_t)gridDim.x * (256 / LPB);
    for (int64_t b = first; b < nblocks; b += stride) {
        const v4i raw = (IN == IN_F32) ? *(const v4i *)((const float *)X + b * 32 + sub * V)
                                       : *(const v4i *)((const uint16_t *)X + b * 32 + sub * V);
        float v[V];
        if (IN == IN_F32) {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = __int_as_float(raw[i]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = __uint_as_float((uint32_t)raw[i] << 16);
                v[2 * i + 1] = __uint_as_float((uint32_t)raw[i] & 0xffff0000u);
            }
        }
        // a non-finite value makes the block's maximum +inf (see quantize_kernel)
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
        uint32_t w[V / 4];                                 // 24 bits per 4 values
#pragma unroll
        for (int j = 0; j < V / 4; ++j) {
            w[j] = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                w[j] |= fp6_code<F>(ldexpf(v[4 * j + i], 127 - s)) << (6 * i);
            if (bad) w[j] = 0;
        }
        if (V == 4) {
            // quad lane r < 3 stores dword r of the quad's 12 bytes: its own
            // bytes from byte r on, then the next lane's (quad_perm 1,2,3,3)
            const int r = sub & 3;
            const uint32_t nb = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w[0], 0xF9, 0xF, 0xF, false);
            if (r < 3)
                *(uint32_t *)(Q + b * 24 + (sub >> 2) * 12 + 4 * r) =
                    (w[0] >> (8 * r)) | (nb << (24 - 8 * r));
        } else {
            // lane pair (A0 A1 | B0 B1, 3 bytes each): the even lane stores
            // A0 A1[0] and A1[1..2] B0[0..1], the odd lane B0[2] B1; the even
            // lane takes B0 from its neighbour (quad_perm 1,1,3,3)
            const uint32_t w1 = w[V / 4 - 1];
            const uint32_t nb = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w[0], 0xF5, 0xF, 0xF, false);
            uint32_t *q32 = (uint32_t *)(Q + b * 24 + (sub >> 1) * 12);
            if ((sub & 1) == 0) {
                q32[0] = w[0] | (w1 << 24);
                q32[1] = (w1 >> 8) | (nb << 16);
            } else {
                q32[2] = (w[0] >> 16) | (w1 << 8);
            }
        }
    }
}

}  // namespace mx
