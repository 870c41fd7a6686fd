// mx_launch.h -- launches of the tile kernel for one format pair: the tile
// shape from the plan, the split-K slices and their in-order reduction, and
// the grouped launches.  Shared by mxgemm.hip, mxgrouped.hip and the units
// that hold the pairs of an FP6 format with another format (mxfp6pairs.hip,
// mxgrouped_fp6.hip), compiled as translation units of their own.
#pragma once
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "mxgemm.h"
#include "mx_kernels.h"
#include "mx_host.h"

namespace mxhost {

// Split-K slices are whole 512-K scale periods.
inline constexpr int64_t kPeriodK = 512;

inline int64_t slice_k(int64_t K, int split) { return cdiv(cdiv(K, split), kPeriodK) * kPeriodK; }

// FP32 elements per split-K plane (a multiple of 4 keeps planes 16-byte aligned).
inline int64_t plane_of(int64_t M, int64_t N) { return cdiv(M * N, 64) * 64; }

inline bool is_fp6_fmt(int fmt) { return fmt == MX_FMT_E2M3 || fmt == MX_FMT_E3M2; }

template <int FA, int FB, int OUT, int BM, int BN, int WGM, int WGN, int S>
void launch_cfg(const void *A, const void *As, const void *B, const void *Bs, void *C,
                int64_t M, int64_t N, int64_t K, int split, float *W, hipStream_t stream)
{
    const int tiles_m = (int)cdiv(M, BM), tiles_n = (int)cdiv(N, BN);
    const int gm = 4;
    const unsigned grid = (unsigned)(tiles_m * tiles_n * split);
    if (split == 1) {
        hipLaunchKernelGGL((mx::tile_kernel<FA, FB, OUT, BM, BN, WGM, WGN, S>), dim3(grid),
                           dim3(WGM * WGN * 64), 0, stream, (const uint8_t *)A,
                           (const uint8_t *)As, (const uint8_t *)B, (const uint8_t *)Bs, C,
                           (int)M, (int)N, (int)K, tiles_m, tiles_n, gm, (int)K, (int64_t)0);
        return;
    }
    const int64_t plane = plane_of(M, N);
    hipLaunchKernelGGL((mx::tile_kernel<FA, FB, mx::OF32, BM, BN, WGM, WGN, S>), dim3(grid),
                       dim3(WGM * WGN * 64), 0, stream, (const uint8_t *)A,
                       (const uint8_t *)As, (const uint8_t *)B, (const uint8_t *)Bs, (void *)W,
                       (int)M, (int)N, (int)K, tiles_m, tiles_n, gm, (int)slice_k(K, split),
                       plane);
    hipLaunchKernelGGL((mx::splitk_reduce<OUT>), dim3((unsigned)cdiv(M * N, 1024)), dim3(256),
                       0, stream, (const float *)W, C, M * N, plane, split);
}

template <int FA, int FB, int OUT>
bool launch_tile(const mx_plan_t &p, const void *A, const void *As, const void *B,
                 const void *Bs, void *C, int64_t M, int64_t N, int64_t K, float *W,
                 hipStream_t stream)
{
#define MX_CFG(BM_, BN_, WM_, WN_, S_)                                                    \
    if (p.tile_m == BM_ && p.tile_n == BN_ && p.threads == WM_ * WN_ * 64) {             \
        launch_cfg<FA, FB, OUT, BM_, BN_, WM_, WN_, S_>(A, As, B, Bs, C, M, N, K,          \
                                                        p.split_k, W, stream);             \
        return true;                                                                      \
    }
    MX_CFG(256, 256, 4, 2, 2)
    MX_CFG(256, 192, 4, 2, 2)
    MX_CFG(256, 160, 4, 1, 2)
    MX_CFG(256, 128, 4, 2, 3)
    MX_CFG(128, 128, 2, 2, 3)
    MX_CFG(64, 256, 1, 8, 3)
#undef MX_CFG
    return false;
}

// Dispatch on the output type for formats (FA, FB).
template <int FA, int FB>
bool launch(const mx_plan_t &p, int out_dtype, const void *A, const void *As, const void *B,
            const void *Bs, void *C, int64_t M, int64_t N, int64_t K, float *W,
            hipStream_t stream)
{
    return out_dtype == MX_OUT_FP32
        ? launch_tile<FA, FB, mx::OF32>(p, A, As, B, Bs, C, M, N, K, W, stream)
        : launch_tile<FA, FB, mx::OBF16>(p, A, As, B, Bs, C, M, N, K, W, stream);
}

// The tile kernel for fmt_a x fmt_b where one is an FP6 format and the pair
// is not one FP6 format twice (defined in mxfp6pairs.hip).  W is the split-K
// workspace of the plan.  Returns false if the plan's tile is not compiled.
bool launch_fp6_pair(int fmt_a, int fmt_b, const mx_plan_t &p, int out_dtype, const void *A,
                     const void *As, const void *B, const void *Bs, void *C, int64_t M,
                     int64_t N, int64_t K, float *W, hipStream_t stream);

// The decode kernel's problems: both operands E2M1, E4M3 or E5M2, M <= 32
// rows, and K >= 512 and a multiple of 128 (whole slabs of the 8-bit
// operands; the shapes it is tested and timed on -- shorter K is a GEMM
// the tiled kernel runs in a few microseconds).
inline bool decode_fits(int fmt_a, int fmt_b, int64_t M, int64_t N, int64_t K)
{
    auto mx8 = [](int f) { return f == MX_FMT_E2M1 || f == MX_FMT_E4M3 || f == MX_FMT_E5M2; };
    return mx8(fmt_a) && mx8(fmt_b) && M >= 1 && M <= MX_DECODE_TILE && N >= 1 &&
           K >= kPeriodK && K % 128 == 0;
}

// The decode kernel for fmt_a x fmt_b (defined in mxdecode.hip): one
// workgroup per MX_DECODE_TILE columns of C.  Returns false if the problem
// is not one decode_fits accepts.
bool launch_decode(int fmt_a, int fmt_b, int out_dtype, const void *A, const void *As,
                   const void *B, const void *Bs, void *C, int64_t M, int64_t N, int64_t K,
                   hipStream_t s);

// Grouped launches: one tile shape (kTiles[t]) for every group, the group
// table in the kernel arguments, no K split.
template <int FA, int FB, int OUT, int BM, int BN, int WGM, int WGN, int S>
void launch_grouped_cfg(const void *A, const void *As, const void *B, const void *Bs, void *C,
                        int64_t N, int64_t K, const mx::GroupTable &gt, hipStream_t stream)
{
    const int tiles_n = (int)cdiv(N, BN);
    hipLaunchKernelGGL((mx::tile_kernel<FA, FB, OUT, BM, BN, WGM, WGN, S, mx::GroupTable>),
                       dim3((unsigned)gt.tile_start[gt.n]), dim3(WGM * WGN * 64), 0, stream,
                       (const uint8_t *)A, (const uint8_t *)As, (const uint8_t *)B,
                       (const uint8_t *)Bs, C, 0, (int)N, (int)K, 0, tiles_n, 4, (int)K,
                       (int64_t)0, gt);
}

template <int FA, int FB, int OUT>
bool launch_grouped(int t, const void *A, const void *As, const void *B, const void *Bs,
                    void *C, int64_t N, int64_t K, const mx::GroupTable &gt, hipStream_t s)
{
    const TileCfg &c = kTiles[t];
#define MX_GCFG(BM_, BN_, WM_, WN_, S_)                                                   \
    if (c.bm == BM_ && c.bn == BN_ && c.wgm == WM_ && c.wgn == WN_) {                    \
        launch_grouped_cfg<FA, FB, OUT, BM_, BN_, WM_, WN_, S_>(A, As, B, Bs, C, N, K, gt, s); \
        return true;                                                                      \
    }
    MX_GCFG(256, 256, 4, 2, 2)
    MX_GCFG(256, 192, 4, 2, 2)
    MX_GCFG(256, 160, 4, 1, 2)
    MX_GCFG(256, 128, 4, 2, 3)
    MX_GCFG(128, 128, 2, 2, 3)
    MX_GCFG(64, 256, 1, 8, 3)
#undef MX_GCFG
    return false;
}

// The grouped tile kernel for fmt_a x fmt_b where one is an FP6 format and
// the pair is not one FP6 format twice (defined in mxgrouped_fp6.hip).
// Returns false if tile t is not compiled.
bool launch_grouped_fp6_pair(int fmt_a, int fmt_b, int t, bool f32, const void *A,
                             const void *As, const void *B, const void *Bs, void *C, int64_t N,
                             int64_t K, const mx::GroupTable &gt, hipStream_t stream);

}  // namespace mxhost
