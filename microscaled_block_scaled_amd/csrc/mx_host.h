// mx_host.h -- host-side helpers shared by the GEMM entry points
// (mxgemm.hip) and the grouped entry points (mxgrouped.hip): argument
// checks, the tile table, and the one-time per-device check.
#pragma once
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>
#include <string.h>

#include "mxgemm.h"

namespace mxhost {

inline constexpr int kMaxDevices = 64;

inline int check_args(int fmt, int64_t M, int64_t N, int64_t K, int out_dtype)
{
    if (fmt < MX_FMT_E2M1 || fmt > MX_FMT_E3M2) return MX_ERR_FORMAT;
    if (out_dtype != MX_OUT_FP32 && out_dtype != MX_OUT_BF16) return MX_ERR_OUT_DTYPE;
    // K a multiple of 128 (FlyDSL article, "API compatibility is not
    // universal input coverage").
    if (M < 1 || N < 1 || K < 128 || K % 128 != 0) return MX_ERR_SHAPE;
    if (M > MX_MAX_DIM || N > MX_MAX_DIM || K > MX_MAX_K) return MX_ERR_SHAPE;
    return MX_OK;
}

// Dense BF16 GEMM: K a multiple of 16 (one BF16 MFMA step), rows of at most
// MX_MAX_K bytes (the same 32-bit copy offsets as the MX formats).
inline int check_args_bf16(int64_t M, int64_t N, int64_t K, int out_dtype)
{
    if (out_dtype != MX_OUT_FP32 && out_dtype != MX_OUT_BF16) return MX_ERR_OUT_DTYPE;
    if (M < 1 || N < 1 || K < 16 || K % 16 != 0) return MX_ERR_SHAPE;
    if (M > MX_MAX_DIM || N > MX_MAX_DIM || K > MX_MAX_K_BF16) return MX_ERR_SHAPE;
    return MX_OK;
}

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Tile shapes of the tiled kernel: {BM, BN, waves along M, waves along N,
// LDS ring depth in slabs} (deeper rings where the LDS footprint allows).
struct TileCfg { int bm, bn, wgm, wgn, stages; };
inline constexpr TileCfg kTiles[] = {
    {256, 256, 4, 2, 2}, {256, 192, 4, 2, 2}, {256, 160, 4, 1, 2}, {256, 128, 4, 2, 3},
    {128, 128, 2, 2, 3}, {64, 256, 1, 8, 3},
};
inline constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

// Relative speed per CU of a tile shape on MFMA-bound work, for the plans.
// The 256-row tile with four waves (one per SIMD) leaves each SIMD's LDS and
// barrier latency uncovered: measured on MI355X, 2048 x 5120 x 25600 MXFP4
// took 192 us on 256x160 tiles (256 workgroups) and 170 us on 256x192 tiles
// with 40 of 256 CUs idle, i.e. 0.73 of the 8-wave tile's rate per CU.
inline double tile_speed(const TileCfg &c) { return c.bm == 256 && c.wgm * c.wgn == 4 ? 0.73 : 1.0; }
inline constexpr int kCUs = 256;   // MI355X compute units: one 256-row tile per CU per wave

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The kernels number workgroups (tile, slice) with a 32-bit int.
inline constexpr int64_t kMaxGrid = 0x7fffffff;

// Per-device one-time check: the device must be a gfx950.
inline std::once_flag g_dev_once[kMaxDevices];
inline int g_dev_status[kMaxDevices];

inline int device_ready(int *dev_out)
{
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count < 1) return MX_ERR_NO_DEVICE;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MX_ERR_NO_DEVICE;
    if (dev >= kMaxDevices) return MX_ERR_ARCH;
    std::call_once(g_dev_once[dev], [dev]() {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            g_dev_status[dev] = MX_ERR_NO_DEVICE;
            return;
        }
        g_dev_status[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? MX_OK : MX_ERR_ARCH;
    });
    *dev_out = dev;
    return g_dev_status[dev];
}

// One tile-kernel launch; with split > 1 it writes FP32 planes to the

// Formats as run_plan sees them: the MX_FMT_* codes, and dense BF16 (no
// scales), which has no format code of its own in the ABI.
inline constexpr int kFmtBF16 = 0x100;

}  // namespace mxhost
