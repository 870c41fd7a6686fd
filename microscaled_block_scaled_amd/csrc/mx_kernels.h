// mx_kernels.h -- gfx950 device code for the MX block-scaled NT GEMM.
//
// C[m][n] = sum_b 2^(sA[m][b]+sB[n][b]-254) * sum_{j<32} A[m][32b+j]*B[n][32b+j]
// with FP32 accumulation (the MX scaled GEMM of the FlyDSL article: E8M0 scale
// per 32 K-values, FP32 accumulation, K a multiple of 128; digest 2026-10-22,
// item 1).  Every product block is computed by the CDNA4 block-scaled matrix
// instruction v_mfma_scale_f32_16x16x128_f8f6f4, which applies the two E8M0
// scales itself.
//
// Operand placement of that instruction on gfx950, as measured on the device
// with one-hot inputs (lane l, row r = l % 16, lane group g = l / 16):
//   * E2M1: lane (r, g) holds K-values 32g .. 32g+31 of row r as 16 bytes,
//     element 2i in the low nibble of byte i;
//   * E4M3: lane (r, g) holds K-values 16g .. 16g+15 in bytes 0..15 and
//     64+16g .. 64+16g+15 in bytes 16..31;
//   * in both formats, lane (r, g) supplies the scale byte of K-block g
//     (K-values 32g .. 32g+31) of row r, at the byte op_sel selects;
//   * B uses the same placement with r the column index;
//   * the 16x16 FP32 result: lane (c, g) holds rows 4g .. 4g+3 of column c.
// So with a row's K-values staged as 16-byte chunks (chunk c = bytes
// 16c .. 16c+15 of a 128-byte row segment), lane group g reads chunks g and
// 4+g: for E4M3 both feed one instruction (128 K-values); for E2M1 a 128-byte
// segment holds 256 K-values and chunk g feeds the first instruction, chunk
// 4+g the second.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

enum { FP4 = 1, FP8 = 2 };      // equal to MX_FMT_E2M1 / MX_FMT_E4M3
enum { OF32 = 1, OBF16 = 2 };   // equal to MX_OUT_FP32 / MX_OUT_BF16

// Format selector of the scaled MFMA (cbsz for A, blgp for B).
template <int FMT> struct mfma_fmt { static constexpr int sel = (FMT == FP4) ? 4 : 0; };

// K-values held by one 128-byte row segment, and E8M0 bytes covering it.
template <int FMT> struct seg {
    static constexpr int kvals = (FMT == FP4) ? 256 : 128;
    static constexpr int sbytes = kvals / 32;        // 8 (E2M1) or 4 (E4M3)
    static constexpr int mfmas = (FMT == FP4) ? 2 : 1;
};

// FP32 -> BF16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// LDS row swizzle: chunk c of staged row r lives at chunk c ^ swz(r).  Any 8
// consecutive rows, and the even (or odd) rows of any 16 aligned rows, then
// hit 8 distinct 16-byte bank groups, so the lane groups' 16-byte reads are
// free of bank conflicts.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int FMT>
__device__ __forceinline__ v4f mma(const v8i &a, const v8i &b, v4f acc, int sa, int sb)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        a, b, acc, mfma_fmt<FMT>::sel, mfma_fmt<FMT>::sel, 0, sa, 0, sb);
}

// --------------------------------------------------------------------------
// Tiled kernel: one workgroup computes a BM x BN tile of C; WGM x WGN waves
// each own a (BM/WGM) x (BN/WGN) sub-tile of 16x16 accumulator fragments.
// K is walked in 128-byte row segments, staged HBM -> registers -> LDS with
// two LDS buffers: the global loads of segment s+1 are in flight while the
// waves run the MFMAs of segment s.
template <int FMT, int OUT, int BM, int BN, int WGM, int WGN>
__global__ void __launch_bounds__(WGM * WGN * 64)
tile_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
            const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
            void *__restrict__ C, int M, int N, int K, int tiles_n)
{
    constexpr int NT = WGM * WGN * 64;
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int KV = seg<FMT>::kvals, SBY = seg<FMT>::sbytes;
    constexpr int CA = BM * 8 / NT, CB = BN * 8 / NT;        // 16-B chunks per thread
    constexpr int SDW = SBY / 4;                              // scale dwords per row
    constexpr int SQ = (BM + BN) * SDW;                       // scale dwords per segment
    constexpr int SQT = (SQ + NT - 1) / NT;
    static_assert(CA * NT == BM * 8 && CB * NT == BN * 8, "tile / thread mismatch");
    static_assert(FM * 16 == WTM && FN * 16 == WTN, "wave tile must be 16-aligned");

    __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * 128];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * 128];
    __shared__ __attribute__((aligned(16))) uint8_t sS[2][(BM + BN) * 8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const int64_t rowb = (FMT == FP4) ? (int64_t)K / 2 : (int64_t)K;
    const int sp = K / 32;
    const int nseg = (K + KV - 1) / KV;

    v4i ra[CA], rbv[CB];
    uint32_t rs[SQT];

    auto gload = [&](int s) {
        const int64_t koff = (int64_t)s * 128;
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            int q = tid + i * NT, r = q >> 3, c = q & 7;
            int row = min(m0 + r, M - 1);
            int64_t off = koff + c * 16;
            ra[i] = (off < rowb) ? *(const v4i *)(A + (int64_t)row * rowb + off) : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            int q = tid + i * NT, r = q >> 3, c = q & 7;
            int row = min(n0 + r, N - 1);
            int64_t off = koff + c * 16;
            rbv[i] = (off < rowb) ? *(const v4i *)(B + (int64_t)row * rowb + off) : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < SQT; ++i) {
            int q = tid + i * NT;
            uint32_t v = 0x7f7f7f7fu;
            if (q < SQ) {
                int r = q / SDW, part = q % SDW;
                int soff = s * SBY + part * 4;
                if (soff < sp) {
                    if (r < BM) v = *(const uint32_t *)(As + (int64_t)min(m0 + r, M - 1) * sp + soff);
                    else v = *(const uint32_t *)(Bs + (int64_t)min(n0 + r - BM, N - 1) * sp + soff);
                }
            }
            rs[i] = v;
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            int q = tid + i * NT, r = q >> 3, c = q & 7;
            *(v4i *)(&sA[buf][r * 128 + ((c ^ swz(r)) << 4)]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            int q = tid + i * NT, r = q >> 3, c = q & 7;
            *(v4i *)(&sB[buf][r * 128 + ((c ^ swz(r)) << 4)]) = rbv[i];
        }
#pragma unroll
        for (int i = 0; i < SQT; ++i) {
            int q = tid + i * NT;
            if (q < SQ) {
                int r = q / SDW, part = q % SDW;
                *(uint32_t *)(&sS[buf][r * 8 + part * 4]) = rs[i];
            }
        }
    };

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int lr = lane & 15, g = lane >> 4;

    gload(0);
    lstore(0);
    __syncthreads();

    for (int s = 0; s < nseg; ++s) {
        const int buf = s & 1;
        if (s + 1 < nseg) gload(s + 1);
        // E2M1 with K % 256 == 128: the last segment holds one instruction's worth.
        const int nh = (FMT == FP4 && (s + 1) * KV > K) ? 1 : seg<FMT>::mfmas;
#pragma unroll
        for (int h = 0; h < seg<FMT>::mfmas; ++h) {
            if (h >= nh) break;
            v8i af[FM], bf[FN];
            int sa[FM], sb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                int r = wm * WTM + i * 16 + lr;
                const uint8_t *rowp = &sA[buf][r * 128];
                if (FMT == FP8) {
                    v4i lo = *(const v4i *)(rowp + ((g ^ swz(r)) << 4));
                    v4i hi = *(const v4i *)(rowp + (((4 + g) ^ swz(r)) << 4));
                    af[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    sa[i] = sS[buf][r * 8 + g];
                } else {
                    v4i v = *(const v4i *)(rowp + (((4 * h + g) ^ swz(r)) << 4));
                    af[i] = v8i{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
                    sa[i] = sS[buf][r * 8 + 4 * h + g];
                }
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                int r = wn * WTN + j * 16 + lr;
                const uint8_t *rowp = &sB[buf][r * 128];
                if (FMT == FP8) {
                    v4i lo = *(const v4i *)(rowp + ((g ^ swz(r)) << 4));
                    v4i hi = *(const v4i *)(rowp + (((4 + g) ^ swz(r)) << 4));
                    bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    sb[j] = sS[buf][(BM + r) * 8 + g];
                } else {
                    v4i v = *(const v4i *)(rowp + (((4 * h + g) ^ swz(r)) << 4));
                    bf[j] = v8i{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
                    sb[j] = sS[buf][(BM + r) * 8 + 4 * h + g];
                }
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = mma<FMT>(af[i], bf[j], acc[i][j], sa[i], sb[j]);
        }
        if (s + 1 < nseg) lstore(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: lane (c, g) of fragment (i, j) holds rows 4g..4g+3, column c.
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * WTN + j * 16 + lr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + wm * WTM + i * 16 + 4 * g + e;
                if (row < M && col < N) {
                    if (OUT == OF32)
                        ((float *)C)[(int64_t)row * N + col] = acc[i][j][e];
                    else
                        ((uint16_t *)C)[(int64_t)row * N + col] = f32_to_bf16(acc[i][j][e]);
                }
            }
        }
    }
}

}  // namespace mx
