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

// Direct HBM -> LDS copies (gfx950 global_load_lds): lane l of the wave
// writes its `size` bytes to lds + l * size; `lds` must be wave-uniform.
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void g2l_16(const void *src, void *lds)
{
    __builtin_amdgcn_global_load_lds(src, (lds_void *)lds, 16, 0, 0);
}
__device__ __forceinline__ void g2l_4(const void *src, void *lds)
{
    __builtin_amdgcn_global_load_lds(src, (lds_void *)lds, 4, 0, 0);
}
__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Tile order: workgroups are dispatched round-robin over the 8 XCDs (bid % 8).
// Give each XCD a contiguous run of tiles, walked in groups of `gm` M-tiles,
// so the workgroups sharing an XCD's L2 also share A and B panels.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int gm,
                                        int &tm, int &tn)
{
    const int ntiles = tiles_m * tiles_n;
    int t = bid;
    if ((ntiles & 7) == 0) t = (bid & 7) * (ntiles >> 3) + (bid >> 3);
    const int per_group = gm * tiles_n;
    const int grp = t / per_group, first_m = grp * gm;
    const int gsz = min(tiles_m - first_m, gm);
    const int w = t - grp * per_group;
    tm = first_m + w % gsz;
    tn = w / gsz;
}

// --------------------------------------------------------------------------
// Tiled kernel: one workgroup computes a BM x BN tile of C with WGM x WGN
// waves, each owning a (BM/WGM) x (BN/WGN) block of 16x16 FP32 accumulators.
// K is walked in 128-byte row segments (128 E4M3 or 256 E2M1 K-values).
// Each segment of A, B and their scale bytes is copied HBM -> LDS directly
// (no register staging) into one of two LDS stages; the copy of segment s+1
// is in flight while the waves run segment s's MFMAs.  Rows are swizzled in
// LDS (chunk c of row r stored at chunk c ^ swz(r)); the swizzle is applied
// on the global side, since each lane's LDS slot is fixed by its lane id.
template <int FMT, int OUT, int BM, int BN, int WGM, int WGN>
__global__ void __launch_bounds__(WGM * WGN * 64)
tile_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
            const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
            void *__restrict__ C, int M, int N, int K, int tiles_m, int tiles_n, int gm)
{
    constexpr int NW = WGM * WGN;
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int KV = seg<FMT>::kvals, SBY = seg<FMT>::sbytes, SDW = SBY / 4;
    constexpr int DATA = (BM + BN) * 128;                  // element bytes per stage
    constexpr int SCALE_DW = (BM + BN) * SDW;              // scale dwords per stage
    // Scale copies write whole 64-lane instructions (256 bytes each).
    constexpr int STAGE = DATA + (SCALE_DW + 63) / 64 * 256;
    static_assert(BM % 8 == 0 && BN % 8 == 0, "rows per copy instruction");
    static_assert(FM * 16 == WTM && FN * 16 == WTN, "wave tile must be 16-aligned");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, gm, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int64_t rowb = (FMT == FP4) ? (int64_t)K / 2 : (int64_t)K;
    const int sp = K / 32;
    const int nseg = (K + KV - 1) / KV;

    // Per-lane constant parts of the copy addresses.
    const int crow = lane >> 3, cpc = lane & 7;   // row within an 8-row copy, LDS chunk

    auto issue = [&](int s, int stage) {
        uint8_t *base = smem + stage * STAGE;
        const int64_t koff = (int64_t)s * 128;
#pragma unroll
        for (int i = wave; i < BM / 8; i += NW) {
            const int r = i * 8 + crow;
            const int row = min(m0 + r, M - 1);
            int64_t off = koff + ((cpc ^ swz(r)) << 4);
            off = min(off, rowb - 16);                 // E2M1 half segment: unused data
            g2l_16(A + (int64_t)row * rowb + off, base + i * 1024);
        }
#pragma unroll
        for (int i = wave; i < BN / 8; i += NW) {
            const int r = i * 8 + crow;
            const int row = min(n0 + r, N - 1);
            int64_t off = koff + ((cpc ^ swz(r)) << 4);
            off = min(off, rowb - 16);
            g2l_16(B + (int64_t)row * rowb + off, base + BM * 128 + i * 1024);
        }
#pragma unroll
        for (int i = wave; i < (SCALE_DW + 63) / 64; i += NW) {
            const int q = min(i * 64 + lane, SCALE_DW - 1);
            const int r = q / SDW, part = q % SDW;
            const int soff = min(s * SBY + part * 4, sp - 4);
            const uint8_t *src = (r < BM) ? As + (int64_t)min(m0 + r, M - 1) * sp + soff
                                          : Bs + (int64_t)min(n0 + r - BM, N - 1) * sp + soff;
            g2l_4(src, base + DATA + i * 256);
        }
    };

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int lr = lane & 15, g = lane >> 4;

    issue(0, 0);
    for (int s = 0; s < nseg; ++s) {
        const int stage = s & 1;
        wait_vm0();            // this wave's copies of segment s have landed
        __syncthreads();       // ... and everyone's; stage s+1 is no longer read
        if (s + 1 < nseg) issue(s + 1, stage ^ 1);

        const uint8_t *sA = smem + stage * STAGE;
        const uint8_t *sB = sA + BM * 128;
        const uint8_t *sS = sA + DATA;
        // E2M1 with K % 256 == 128: the last segment holds one instruction's worth.
        const int nh = (FMT == FP4 && (s + 1) * KV > K) ? 1 : seg<FMT>::mfmas;
        // One pass per instruction-sized K slice; kept rolled so only one
        // pass's fragments are live.
#pragma unroll 1
        for (int h = 0; h < nh; ++h) {
            const int cl = (FMT == FP8) ? g : 4 * h + g;      // chunk (E4M3: also 4+g)
            const int sbyte = (FMT == FP8) ? g : 4 * h + g;   // scale byte in the segment
            v8i bf[FN];
            int sb[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int r = wn * WTN + j * 16 + lr;
                const uint8_t *rp = sB + r * 128;
                const v4i lo = *(const v4i *)(rp + ((cl ^ swz(r)) << 4));
                if (FMT == FP8) {
                    const v4i hi = *(const v4i *)(rp + (((4 + g) ^ swz(r)) << 4));
                    bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                } else {
                    bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
                }
                sb[j] = sS[(BM + r) * SBY + sbyte];
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = wm * WTM + i * 16 + lr;
                const uint8_t *rp = sA + r * 128;
                const v4i lo = *(const v4i *)(rp + ((cl ^ swz(r)) << 4));
                v8i af;
                if (FMT == FP8) {
                    const v4i hi = *(const v4i *)(rp + (((4 + g) ^ swz(r)) << 4));
                    af = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                } else {
                    af = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
                }
                const int sa = sS[r * SBY + sbyte];
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = mma<FMT>(af, bf[j], acc[i][j], sa, sb[j]);
            }
        }
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
