// mx_ceiling.h -- measurement kernels, not part of the GEMM.
//   * mfma_ceiling_kernel: the rate at which this device sustains the
//     block-scaled MFMA with no memory traffic at all, in the tile kernel's
//     launch shape (one 512-thread workgroup per CU, two waves per SIMD).  It
//     bounds what any GEMM kernel can reach on the same data: the datasheet
//     peak assumes the matrix units run at the top clock, which the power
//     limit does not allow when the operands are random.
//   * hbm_read_kernel: the rate at which this device streams a buffer from
//     HBM into the CUs, the practical bound of the memory-bound shapes (the
//     datasheet's 8 TB/s is the interface's raw rate).
#pragma once

#include "mx_kernels.h"

namespace mx {

// 32-bit integer mix (the finaliser of MurmurHash3), for operand bytes that
// look random to the matrix unit.
__device__ __forceinline__ uint32_t mix32(uint32_t h)
{
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

// Each wave keeps the 256x256 tile's wave tile, a 2 x 4 grid of 32x32 FP32
// accumulators, and issues the 8 MFMAs of one K-step per step on
// register-resident operands.  Two operand sets alternate step by step, so
// the matrix unit sees new data on every step, as in a K loop.  Operand bytes
// are hashed from (workgroup, lane, register) when `random` is set (E4M3
// NaN codes are replaced by 448), else they are the constant 0x22 (E2M1 and
// E4M3 values of magnitude near 1); scale bytes are hashed into [120, 135].
// Each lane writes the sum of its accumulators to out[global thread index],
// so no MFMA is dead code.
template <int F>
__global__ void __launch_bounds__(512) mfma_ceiling_kernel(float *out, int steps, int random)
{
    constexpr int FMv = 2, FNv = 4;
    constexpr int NW = (F == FP4) ? 4 : 8;                 // operand dwords in use
    const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
    v8i a[2][FMv], b[2][FNv];
    int sa[2][FMv], sb[2][FNv];
    uint32_t h = mix32(gid * 0x9e3779b9u + 1u);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < FMv + FNv; ++i) {
            v8i v = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                h = mix32(h + 0x632be5abu);
                uint32_t x = random ? h : 0x22222222u;
                if (F != FP4) {   // E4M3: no NaN codes (S.1111.111)
                    uint32_t nan = ((x & 0x7f7f7f7fu) + 0x01010101u) & 0x80808080u;
                    x &= ~(nan >> 7);                  // 0x7f -> 0x7e in each NaN byte
                }
                v[w] = (int)x;
            }
            h = mix32(h + 0x1b873593u);
            const int sc = 120 + (h & 15);
            if (i < FMv) { a[s][i] = v; sa[s][i] = sc; }
            else { b[s][i - FMv] = v; sb[s][i - FMv] = sc; }
        }
    }
    v16f acc[FMv][FNv];
#pragma unroll
    for (int i = 0; i < FMv; ++i)
#pragma unroll
        for (int j = 0; j < FNv; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    for (int t = 0; t < steps; t += 2) {
        static_for<2>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
#pragma unroll
            for (int j = 0; j < FNv; ++j)
#pragma unroll
                for (int i = 0; i < FMv; ++i)
                    acc[i][j] = mma<F, F, 0>(a[s][i], b[s][j], acc[i][j], sa[s][i], sb[s][j]);
        });
    }
    float r = 0.f;
#pragma unroll
    for (int i = 0; i < FMv; ++i)
#pragma unroll
        for (int j = 0; j < FNv; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) r += acc[i][j][e];
    out[gid] = r;
}

// Workgroup w reads the w-th of gridDim.x contiguous ranges of the buffer
// (ceil(n / gridDim.x) 16-byte chunks each, the last ones shorter or empty):
// its 256 threads read 256 consecutive chunks per step, eight steps' loads in
// flight, with the nontemporal hint (measured on MI355X: about 6.9 TB/s with
// it over 1 GiB, 6.1 without, 5.3 for a grid-strided walk).  Thread t folds
// (XOR) the chunks it read, those at t, t + 256, ... from the range's start,
// and writes the fold to out[global thread index], so no load is dead code.
__global__ void __launch_bounds__(256) hbm_read_kernel(const v4i *__restrict__ src, int64_t n,
                                                       uint32_t *__restrict__ out)
{
    constexpr int U = 8;
    const int64_t per = (n + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = min((int64_t)blockIdx.x * per, n), b1 = min(b0 + per, n);
    v4i x = {0, 0, 0, 0};
    int64_t i = b0 + threadIdx.x;
    for (; i + (U - 1) * 256 < b1; i += U * 256) {
        v4i v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
        for (int u = 0; u < U; ++u) x ^= v[u];
    }
    for (; i < b1; i += 256) x ^= __builtin_nontemporal_load(src + i);
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = (uint32_t)(x[0] ^ x[1] ^ x[2] ^ x[3]);
}

}  // namespace mx
