// mxgrouped.hip -- host side of the grouped GEMM entry points declared in
// include/mxgemm.h: one weight per group of rows in one launch.  Built as
// its own translation unit beside mxgemm.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdint.h>
#include <string.h>

#include "mxgemm.h"
#include "mx_kernels.h"
#include "mx_host.h"
#include "mx_launch.h"

using namespace mxhost;

static_assert(MX_MAX_GROUPS == mx::kMaxGroups, "group table size");

namespace {

// Grouped GEMM: one tile shape for every group, chosen like choose_tile over
// the whole grid of the groups' tiles (no K split: the groups supply the
// parallelism).  Measured on 8 uneven experts (4096 x 4096 x 2048, MXFP8 /
// MXFP4, every tile forced): 256x192 60.1 / 39.9 us, 256x160 60.8 / 40.7,
// 256x128 65.5 / 45.7, 256x256 68.7 / 45.2, 128x128 72.6 / 52.6, 64x256
// 76.4 / 50.5 -- the 8-wave 256x192 tile, which this choice takes.
int choose_tile_grouped(const int64_t *rows, int64_t groups, int64_t N, int64_t total,
                        int64_t maxm)
{
    int best = 0;
    double best_eff = -1.0;
    for (int t = 0; t < kNumTiles; ++t) {
        const TileCfg &c = kTiles[t];
        if (c.bm < 256 && maxm > c.bm) continue;
        int64_t tiles = 0;
        for (int64_t g = 0; g < groups; ++g) tiles += cdiv(rows[g], c.bm) * cdiv(N, c.bn);
        if (tiles == 0) return best;                          // no rows
        const int64_t target = c.bm >= 128 ? kCUs : kCUs / 2;
        const double fill = (double)tiles / (double)(cdiv(tiles, target) * target);
        const double useful = (double)(total * N) / (double)(tiles * c.bm * c.bn);
        const double eff = fill * useful * tile_speed(c);
        if (eff > best_eff + 1e-9) { best_eff = eff; best = t; }
    }
    return best;
}

}  // namespace

// Checks a grouped problem and plans it: the tile (plan->tile_m/tile_n),
// the grid and, when gt is given, the group table.  Host logic only.
// fmt is an MX_FMT_* code or kFmtBF16 (dense BF16, no scales).
int grouped_plan(int fmt, int64_t groups, const int64_t *group_rows, int64_t N, int64_t K,
                 int out_dtype, mx_plan_t *plan, int *tile, mx::GroupTable *gt)
{
    int rc = fmt == kFmtBF16 ? check_args_bf16(1, N, K, out_dtype)
                             : check_args(fmt, 1, N, K, out_dtype);   // format, output, N, K
    if (rc != MX_OK) return rc;
    if (groups < 1 || groups > MX_MAX_GROUPS || groups * N > MX_MAX_DIM) return MX_ERR_SHAPE;
    if (!group_rows || !plan) return MX_ERR_NULL;
    int64_t total = 0, maxm = 0;
    for (int64_t g = 0; g < groups; ++g) {
        if (group_rows[g] < 0 || group_rows[g] > MX_MAX_DIM) return MX_ERR_SHAPE;
        total += group_rows[g];
        maxm = std::max(maxm, group_rows[g]);
    }
    if (total > MX_MAX_DIM) return MX_ERR_SHAPE;
    const int t = choose_tile_grouped(group_rows, groups, N, total, maxm);
    const TileCfg &c = kTiles[t];
    int64_t tiles = 0;
    if (gt) {
        gt->n = (int)groups;
        gt->tile_start[0] = 0;
        gt->row_start[0] = 0;
    }
    for (int64_t g = 0; g < groups; ++g) {
        tiles += cdiv(group_rows[g], c.bm) * cdiv(N, c.bn);
        if (tiles > kMaxGrid) return MX_ERR_SHAPE;
        if (gt) {
            gt->tile_start[g + 1] = (int)tiles;
            gt->row_start[g + 1] = gt->row_start[g] + (int)group_rows[g];
        }
    }
    memset(plan, 0, sizeof(*plan));
    plan->variant = MX_VARIANT_TILE;
    plan->tile_m = c.bm;
    plan->tile_n = c.bn;
    plan->split_k = 1;
    plan->threads = c.wgm * c.wgn * 64;
    plan->workgroups = tiles;
    *tile = t;
    return MX_OK;
}

extern "C" int mx_gemm_grouped_plan(int fmt, int64_t groups, const int64_t *group_rows,
                                    int64_t N, int64_t K, int out_dtype, mx_plan_t *plan)
{
    if (fmt == kFmtBF16) return MX_ERR_FORMAT;
    int t = 0;
    return grouped_plan(fmt, groups, group_rows, N, K, out_dtype, plan, &t, nullptr);
}

namespace {

// Grouped GEMM with A in fmt and B in fmt_b: any pair of MX formats, or
// fmt = fmt_b = kFmtBF16 with no scale arrays.
int run_grouped(int fmt, int fmt_b, int64_t groups, const int64_t *group_rows, int64_t N,
                int64_t K, const void *A, const void *A_scale, const void *B,
                const void *B_scale, void *C, int out_dtype, void *stream)
{
    mx_plan_t plan;
    mx::GroupTable gt;
    int t = 0;
    int rc = grouped_plan(fmt, groups, group_rows, N, K, out_dtype, &plan, &t, &gt);
    if (rc != MX_OK) return rc;
    const bool fp6a = fmt == MX_FMT_E2M3 || fmt == MX_FMT_E3M2;
    const bool fp6b = fmt_b == MX_FMT_E2M3 || fmt_b == MX_FMT_E3M2;
    if ((fmt == kFmtBF16) != (fmt_b == kFmtBF16) ||
        (fmt_b != kFmtBF16 && check_args(fmt_b, 1, N, K, out_dtype) != MX_OK))
        return MX_ERR_FORMAT;
    if (plan.workgroups == 0) return MX_OK;                 // no rows: nothing to compute
    const bool scaled = fmt != kFmtBF16;
    if (!A || !B || !C || (scaled && (!A_scale || !B_scale))) return MX_ERR_NULL;
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16) ||
        (scaled && (!aligned(A_scale, 4) || !aligned(B_scale, 4))))
        return MX_ERR_ALIGN;
    int dev = -1;
    rc = device_ready(&dev);
    if (rc != MX_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    bool launched;
    const bool f32 = out_dtype == MX_OUT_FP32;
#define MX_GRUN(FA_, FB_)                                                                         \
    (f32 ? launch_grouped<FA_, FB_, mx::OF32>(t, A, A_scale, B, B_scale, C, N, K, gt, s)         \
         : launch_grouped<FA_, FB_, mx::OBF16>(t, A, A_scale, B, B_scale, C, N, K, gt, s))
    if (fmt == kFmtBF16)
        launched = MX_GRUN(mx::B16, mx::B16);
    else if (fmt == MX_FMT_E2M3 && fmt_b == MX_FMT_E2M3)
        launched = MX_GRUN(mx::F6E2, mx::F6E2);
    else if (fmt == MX_FMT_E3M2 && fmt_b == MX_FMT_E3M2)
        launched = MX_GRUN(mx::F6E3, mx::F6E3);
    else if (fp6a || fp6b)                                         // FP6 with another format
        launched = launch_grouped_fp6_pair(fmt, fmt_b, t, f32, A, A_scale, B, B_scale, C, N, K,
                                           gt, s);
    else if (fmt == MX_FMT_E2M1)
        launched = fmt_b == MX_FMT_E2M1 ? MX_GRUN(mx::FP4, mx::FP4)
                 : fmt_b == MX_FMT_E4M3 ? MX_GRUN(mx::FP4, mx::FP8)
                                        : MX_GRUN(mx::FP4, mx::BF8);
    else if (fmt == MX_FMT_E4M3)
        launched = fmt_b == MX_FMT_E2M1 ? MX_GRUN(mx::FP8, mx::FP4)
                 : fmt_b == MX_FMT_E4M3 ? MX_GRUN(mx::FP8, mx::FP8)
                                        : MX_GRUN(mx::FP8, mx::BF8);
    else                                                           // A E5M2
        launched = fmt_b == MX_FMT_E2M1 ? MX_GRUN(mx::BF8, mx::FP4)
                 : fmt_b == MX_FMT_E4M3 ? MX_GRUN(mx::BF8, mx::FP8)
                                        : MX_GRUN(mx::BF8, mx::BF8);
#undef MX_GRUN
    return (launched && hipGetLastError() == hipSuccess) ? MX_OK : MX_ERR_LAUNCH;
}

}  // namespace

extern "C" int mx_gemm_grouped(int fmt, int64_t groups, const int64_t *group_rows,
                               int64_t N, int64_t K, const void *A, const void *A_scale,
                               const void *B, const void *B_scale, void *C, int out_dtype,
                               void *stream)
{
    if (fmt == kFmtBF16) return MX_ERR_FORMAT;
    return run_grouped(fmt, fmt, groups, group_rows, N, K, A, A_scale, B, B_scale, C, out_dtype,
                       stream);
}

extern "C" int mx_gemm_grouped_mixed(int fmt_a, int fmt_b, int64_t groups,
                                     const int64_t *group_rows, int64_t N, int64_t K,
                                     const void *A, const void *A_scale, const void *B,
                                     const void *B_scale, void *C, int out_dtype, void *stream)
{
    if (fmt_a == kFmtBF16 || fmt_b == kFmtBF16) return MX_ERR_FORMAT;
    return run_grouped(fmt_a, fmt_b, groups, group_rows, N, K, A, A_scale, B, B_scale, C,
                       out_dtype, stream);
}

extern "C" int mx_gemm_grouped_bf16(int64_t groups, const int64_t *group_rows, int64_t N,
                                    int64_t K, const void *A, const void *B, void *C,
                                    int out_dtype, void *stream)
{
    return run_grouped(kFmtBF16, kFmtBF16, groups, group_rows, N, K, A, nullptr, B, nullptr, C,
                       out_dtype, stream);
}

extern "C" int mx_gemm_grouped_bf16_plan(int64_t groups, const int64_t *group_rows, int64_t N,
                                         int64_t K, int out_dtype, mx_plan_t *plan)
{
    int t = 0;
    return grouped_plan(kFmtBF16, groups, group_rows, N, K, out_dtype, plan, &t, nullptr);
}
