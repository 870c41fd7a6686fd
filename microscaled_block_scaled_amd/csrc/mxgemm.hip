// mxgemm.hip -- host side of the C ABI declared in include/mxgemm.h for the
// dense GEMMs and the quantizer: argument checks (all before any HIP call),
// the launch plan, and the kernel launches.  The grouped GEMMs are in
// mxgrouped.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <stdint.h>
#include <string.h>

#include "mxgemm.h"
#include "mx_kernels.h"
#include "mx_decode.h"
#include "mx_quant.h"
#include "mx_quant6.h"
#include "mx_ceiling.h"
#include "mx_host.h"
#include "mx_launch.h"

using namespace mxhost;

namespace {


// Split-K for grids too small to fill the chip: K is cut into slices of
// whole 512-K scale periods, each slice a workgroup of its own writing an
// FP32 plane of the workspace, and a second kernel adds the planes in order.
// Slices double while the grid still fits in one wave of CUs and each slice
// keeps at least kMinSliceK of K.
constexpr int kMaxSplit = MX_MAX_SPLIT_K;
constexpr int64_t kMinSliceK = 2048;

// Measured on MI355X: 256-row tiles split until the grid fills the CUs once;
// the 64-row tile (small M, B streamed from memory) is fastest at about half
// that many workgroups.
int choose_split(const TileCfg &c, int64_t tiles, int64_t K)
{
    const int64_t target = c.bm >= 128 ? kCUs : kCUs / 2;
    int s = 1;
    while (s < kMaxSplit && tiles * 2 * s <= target && K / (2 * s) >= kMinSliceK) s *= 2;
    return (int)cdiv(K, slice_k(K, s));        // slices actually needed
}

// Pick the tile (and split) whose grid fills whole waves of CUs best,
// weighting away the padding in partial tiles; ties go to the larger tile
// (more reuse per byte).
int choose_tile(int64_t M, int64_t N, int64_t K)
{
    int best = 0;
    double best_eff = -1.0;
    for (int t = 0; t < kNumTiles; ++t) {
        const TileCfg &c = kTiles[t];
        if (c.bm < 256 && M > c.bm) continue;      // short tiles only for short M
        const int64_t tiles = cdiv(M, c.bm) * cdiv(N, c.bn);
        const int64_t wgs = tiles * choose_split(c, tiles, K);
        const int64_t target = c.bm >= 128 ? kCUs : kCUs / 2;
        const double fill = (double)wgs / (double)(cdiv(wgs, target) * target);
        // With M <= 128 the GEMM is HBM-bound (under 2M FLOP per byte of B,
        // below either format's ridge), so the MFMA work wasted on padding rows
        // of a short tile costs nothing: only the fill counts.
        const double useful = (M <= 128 && c.bm < 256)
            ? 1.0 : (double)(M * N) / (double)(tiles * c.bm * c.bn);
        // A split costs a workspace round trip of one FP32 plane per slice:
        // on a tie, fewer slices win.
        const int64_t split = wgs / tiles;
        const double eff = fill * useful * tile_speed(c) *
                           (split > 1 ? 1.0 - 0.01 * (double)split : 1.0);
        if (eff > best_eff + 1e-9) { best_eff = eff; best = t; }
    }
    return best;
}

// Plan for tile t: which kernel, which tile and split, how many workgroups.
// split_req 0 lets the plan choose; otherwise K is cut into split_req
// slices of whole periods (fewer if K is short).
void fill_plan(int t, int64_t M, int64_t N, int64_t K, mx_plan_t *p, int split_req = 0)
{
    memset(p, 0, sizeof(*p));
    const TileCfg &c = kTiles[t];
    const int64_t tiles = cdiv(M, c.bm) * cdiv(N, c.bn);
    p->variant = MX_VARIANT_TILE;
    p->tile_m = c.bm;
    p->tile_n = c.bn;
    p->split_k = split_req > 0 ? (int)cdiv(K, slice_k(K, split_req)) : choose_split(c, tiles, K);
    p->threads = c.wgm * c.wgn * 64;
    p->lds_bytes = 0;
    p->workgroups = tiles * p->split_k;
    // Planes only for grids the kernels take (callers refuse larger ones):
    // with at most 2^31 workgroups of at most 256 x 256 outputs, M * N <= 2^47
    // and the byte count cannot overflow.
    p->workspace_bytes = p->split_k > 1 && p->workgroups <= kMaxGrid
        ? p->split_k * plane_of(M, N) * 4 : 0;
}

// Plan for the decode kernel: column groups of MX_DECODE_TILE columns, at
// most one workgroup per CU, each taking every gridDim-th group.
void fill_decode_plan(int64_t N, mx_plan_t *p)
{
    memset(p, 0, sizeof(*p));
    p->variant = MX_VARIANT_DECODE;
    p->tile_m = p->tile_n = MX_DECODE_TILE;
    p->split_k = 1;
    p->threads = mx::kDecodeWaves * 64;
    p->workgroups = std::min<int64_t>(cdiv(N, MX_DECODE_TILE), kCUs);
}

// Whether the plan takes the decode kernel for a problem it can run.  The
// decode kernel runs at most one workgroup per CU (it takes all of a CU's
// LDS), each streaming every 256th column group of 32 columns.  The
// thresholds were fitted to cold per-call times of both kernels on MI355X
// over 576 problems (M = 1 .. 32, N = 1024 .. 57344, K = 512 .. 28672,
// E2M1 and E4M3): with them the plan reaches 0.996 of the faster kernel's
// speed (geometric mean; worst 0.84), against 0.79 for the tiled kernel
// alone and 0.976 for the decode kernel alone.  The decode kernel loses
//   * at K < 1024 with more than 3 column groups per workgroup (N > 24576):
//     its per-group work is short (0.9 - 0.95x);
//   * at K >= 16384 with fewer than 160 column groups (N <= 5088), where
//     the tiled kernel's K split spreads B over more CUs (N = 4096,
//     K = 28672: 0.65 - 0.99x);
//   * for M > 16 at K > 14336, or with more than one group per workgroup
//     at K = 14336: every workgroup reads all of A (M = 32, N = 57344,
//     K = 28672: 0.85 - 0.95x).
// M = 8, N = 8192, K = 28672: 1.09x E4M3, 1.12x E2M1; M = 8, N = 57344,
// K = 8192: 1.26x, 1.30x.  `wide` is an E4M3 / E5M2 A with an E2M1 B, which
// the decode kernel runs on its wide slabs (whole-line E2M1 rows) for every
// M: for that pair the M > 16 limit does not hold.  Over 125 such problems
// (M = 9 .. 32, N = 4096 .. 57344, K = 2048 .. 28672) the rule without it
// reaches 0.999 of the faster kernel (worst 0.955), against 0.994 (worst
// 0.87) with it.
bool decode_preferred(int64_t M, int64_t N, int64_t K, bool wide)
{
    const int64_t wgs = cdiv(N, MX_DECODE_TILE);    // column groups
    if (K < 1024 && wgs > 3 * kCUs) return false;
    if (K >= 16384 && wgs < kCUs * 5 / 8) return false;
    if (!wide && M > 16 && K >= 14336 && (K > 14336 || wgs > kCUs)) return false;
    return true;
}

// The plan's choice of kernel, tile and split (split_req as for fill_plan;
// a requested split > 1 keeps the tiled kernel).
void plan_for(int fmt_a, int fmt_b, int64_t M, int64_t N, int64_t K, mx_plan_t *p,
              int split_req = 0)
{
    const bool wide = fmt_b == MX_FMT_E2M1 && (fmt_a == MX_FMT_E4M3 || fmt_a == MX_FMT_E5M2);
    if (split_req <= 1 && decode_fits(fmt_a, fmt_b, M, N, K) && decode_preferred(M, N, K, wide))
        fill_decode_plan(N, p);
    else
        fill_plan(choose_tile(M, N, K), M, N, K, p, split_req);
}

int make_plan(int fmt, int64_t M, int64_t N, int64_t K, int out_dtype, mx_plan_t *p)
{
    int rc = check_args(fmt, M, N, K, out_dtype);
    if (rc != MX_OK) return rc;
    plan_for(fmt, fmt, M, N, K, p);
    return p->workgroups > kMaxGrid ? MX_ERR_SHAPE : MX_OK;
}

int find_tile(int tile_m, int tile_n)
{
    for (int t = 0; t < kNumTiles; ++t)
        if (kTiles[t].bm == tile_m && kTiles[t].bn == tile_n) return t;
    return -1;
}

// The plan for a caller-chosen tile: one of kTiles (split_req as for
// fill_plan), or the decode tile, which takes no split and only the
// problems decode_fits accepts.
int forced_plan(int fmt_a, int fmt_b, int64_t M, int64_t N, int64_t K, int tile_m, int tile_n,
                int split_req, mx_plan_t *p)
{
    if (split_req < 0 || split_req > kMaxSplit) return MX_ERR_SHAPE;
    if (tile_m == MX_DECODE_TILE && tile_n == MX_DECODE_TILE) {
        if (split_req > 1 || !decode_fits(fmt_a, fmt_b, M, N, K)) return MX_ERR_SHAPE;
        fill_decode_plan(N, p);
        return MX_OK;
    }
    const int t = find_tile(tile_m, tile_n);
    if (t < 0) return MX_ERR_SHAPE;
    fill_plan(t, M, N, K, p, split_req);
    return p->workgroups > kMaxGrid ? MX_ERR_SHAPE : MX_OK;
}

// Split-K workspace: one per (device, stream), grown on demand with the
// stream-ordered allocator on that stream (the old buffer freed on it first)
// and kept until the process exits, so repeated calls neither allocate nor
// synchronise.  g_ws_mu is held from the lookup until both kernels of a call
// are enqueued, so host threads sharing a stream cannot interleave their use
// of its workspace.  Calls on one stream are ordered by the stream itself;
// calls on different streams use different buffers.  (A per-call allocation,
// or one buffer shared across streams behind an event chain, measured 5-20 %
// slower on split-K shapes: the extra stream packets.)
struct Workspace { void *ptr = nullptr; size_t bytes = 0; };
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

float *stream_workspace(int dev, hipStream_t s, size_t bytes)
{
    Workspace &w = g_ws[{dev, s}];
    if (w.bytes < bytes) {
        if (w.ptr) (void)hipFreeAsync(w.ptr, s);
        w = Workspace{};
        void *p = nullptr;
        if (hipMallocAsync(&p, bytes, s) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        w.ptr = p;
        w.bytes = bytes;
    }
    return (float *)w.ptr;
}

// Test hook (mx_debug_fail_allocations): the next n workspace allocations
// report failure without allocating.
std::atomic<int> g_fail_allocs{0};

bool fail_injected()
{
    int n = g_fail_allocs.load();
    while (n > 0)
        if (g_fail_allocs.compare_exchange_weak(n, n - 1)) return true;
    return false;
}

// The split-K scratch of mx_gemm_noalloc: a fixed array in device memory,
// one per device the library runs on, held until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: its device
// address on each device is looked up once, with that device current, and
// only that address is ever passed to kernels.
constexpr size_t kScratchBytes = (size_t)MX_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch[kMaxDevices];
int g_scratch_rc[kMaxDevices];

int device_scratch(int dev, void **ptr)
{
    std::call_once(g_scratch_once[dev], [dev]() {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            g_scratch_rc[dev] = MX_ERR_LAUNCH;
            return;
        }
        g_scratch[dev] = p;
        g_scratch_rc[dev] = MX_OK;
    });
    *ptr = g_scratch[dev];
    return g_scratch_rc[dev];
}

// Checks that need no device, then the device check, then the launch.  With
// noalloc the split-K workspace is the device's fixed scratch instead of a
// stream-ordered allocation.
int run_plan(const mx_plan_t &plan, int fmt_a, int fmt_b, int64_t M, int64_t N, int64_t K,
             const void *A, const void *A_scale, const void *B, const void *B_scale,
             void *C, int out_dtype, void *stream, bool noalloc = false)
{
    const bool scaled = fmt_a != kFmtBF16;
    if (!A || !B || !C || (scaled && (!A_scale || !B_scale))) return MX_ERR_NULL;
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16) ||
        (scaled && (!aligned(A_scale, 4) || !aligned(B_scale, 4))))
        return MX_ERR_ALIGN;
    if (noalloc && plan.workspace_bytes > (int64_t)kScratchBytes) return MX_ERR_SCRATCH;
    int dev = -1;
    int rc = device_ready(&dev);
    if (rc != MX_OK) return rc;

    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();  // clear any stale error so the checks below are ours
    float *W = nullptr;
    std::unique_lock<std::mutex> ws_lock(g_ws_mu, std::defer_lock);
    if (plan.workspace_bytes > 0) {
        if (noalloc) {
            void *p = nullptr;
            rc = device_scratch(dev, &p);
            if (rc != MX_OK) return rc;
            W = (float *)p;
        } else {
            ws_lock.lock();
            W = fail_injected() ? nullptr : stream_workspace(dev, s, (size_t)plan.workspace_bytes);
            if (!W) return MX_ERR_ALLOC;
        }
    }
    bool launched;
    const int o = out_dtype;
    if (plan.variant == MX_VARIANT_DECODE)
        launched = launch_decode(fmt_a, fmt_b, o, A, A_scale, B, B_scale, C, M, N, K, s);
    else if (!scaled)
        launched = launch<mx::B16, mx::B16>(plan, o, A, nullptr, B, nullptr, C, M, N, K, W, s);
    else if (fmt_a == MX_FMT_E2M3 && fmt_b == MX_FMT_E2M3)
        launched = launch<mx::F6E2, mx::F6E2>(plan, o, A, A_scale, B, B_scale, C, M, N, K, W, s);
    else if (fmt_a == MX_FMT_E3M2 && fmt_b == MX_FMT_E3M2)
        launched = launch<mx::F6E3, mx::F6E3>(plan, o, A, A_scale, B, B_scale, C, M, N, K, W, s);
    else if (is_fp6_fmt(fmt_a) || is_fp6_fmt(fmt_b))     // FP6 with another format
        launched = launch_fp6_pair(fmt_a, fmt_b, plan, o, A, A_scale, B, B_scale, C, M, N, K, W,
                                   s);
    else if (fmt_a == MX_FMT_E2M1 && fmt_b == MX_FMT_E2M1)
        launched = launch<mx::FP4, mx::FP4>(plan, o, A, A_scale, B, B_scale, C, M, N, K, W, s);
    else if (fmt_a == MX_FMT_E4M3 && fmt_b == MX_FMT_E4M3)
        launched = launch<mx::FP8, mx::FP8>(plan, o, A, A_scale, B, B_scale, C, M, N, K, W, s);
    else if (fmt_a == MX_FMT_E5M2 && fmt_b == MX_FMT_E5M2)
        launched = launch<mx::BF8, mx::BF8>(plan, o, A, A_scale, B, B_scale, C, M, N, K, W, s);
    else if (fmt_a == MX_FMT_E4M3 && fmt_b == MX_FMT_E2M1)
        launched = launch<mx::FP8, mx::FP4>(plan, o, A, A_scale, B, B_scale, C, M, N, K, W, s);
    else if (fmt_a == MX_FMT_E2M1 && fmt_b == MX_FMT_E4M3)
        launched = launch<mx::FP4, mx::FP8>(plan, o, A, A_scale, B, B_scale, C, M, N, K, W, s);
    else if (fmt_a == MX_FMT_E4M3 && fmt_b == MX_FMT_E5M2)
        launched = launch<mx::FP8, mx::BF8>(plan, o, A, A_scale, B, B_scale, C, M, N, K, W, s);
    else if (fmt_a == MX_FMT_E5M2 && fmt_b == MX_FMT_E4M3)
        launched = launch<mx::BF8, mx::FP8>(plan, o, A, A_scale, B, B_scale, C, M, N, K, W, s);
    else if (fmt_a == MX_FMT_E5M2)                       // checked: fmt_b is E2M1
        launched = launch<mx::BF8, mx::FP4>(plan, o, A, A_scale, B, B_scale, C, M, N, K, W, s);
    else                                                 // E2M1 x E5M2
        launched = launch<mx::FP4, mx::BF8>(plan, o, A, A_scale, B, B_scale, C, M, N, K, W, s);
    const bool launch_ok = launched && hipGetLastError() == hipSuccess;
    return launch_ok ? MX_OK : MX_ERR_LAUNCH;
}


}  // namespace

extern "C" const char *mx_strerror(int code)
{
    switch (code) {
    case MX_OK: return "success";
    case MX_ERR_FORMAT: return "unsupported element format or format pair";
    case MX_ERR_OUT_DTYPE: return "unsupported output type (expected MX_OUT_FP32 or MX_OUT_BF16)";
    case MX_ERR_SHAPE: return "bad shape (need M >= 1, N >= 1, K >= 128, K % 128 == 0, M and N <= 2^30, K <= 2^24)";
    case MX_ERR_NULL: return "null pointer argument";
    case MX_ERR_ALIGN: return "misaligned pointer (A, B, C need 16 bytes; scales need 4)";
    case MX_ERR_NO_DEVICE: return "no HIP device available";
    case MX_ERR_ARCH: return "current device is not gfx950";
    case MX_ERR_ALLOC: return "workspace allocation failed";
    case MX_ERR_LAUNCH: return "kernel launch failed";
    case MX_ERR_IN_DTYPE: return "unsupported input type (expected MX_IN_FP32 or MX_IN_BF16)";
    case MX_ERR_SCRATCH: return "split-K workspace larger than the fixed scratch of the "
                                "no-allocation entry point (MX_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown error code";
    }
}

extern "C" int mx_gemm_plan(int fmt, int64_t M, int64_t N, int64_t K, int out_dtype,
                            mx_plan_t *plan)
{
    if (!plan) return MX_ERR_NULL;
    return make_plan(fmt, M, N, K, out_dtype, plan);
}

extern "C" int mx_tile_shapes(int *pairs, int max_pairs)
{
    if (pairs)
        for (int t = 0; t < kNumTiles && t < max_pairs; ++t) {
            pairs[2 * t] = kTiles[t].bm;
            pairs[2 * t + 1] = kTiles[t].bn;
        }
    return kNumTiles;
}

extern "C" int mx_gemm(int fmt, int64_t M, int64_t N, int64_t K,
                       const void *A, const void *A_scale,
                       const void *B, const void *B_scale,
                       void *C, int out_dtype, void *stream)
{
    mx_plan_t plan;
    int rc = make_plan(fmt, M, N, K, out_dtype, &plan);
    if (rc != MX_OK) return rc;
    return run_plan(plan, fmt, fmt, M, N, K, A, A_scale, B, B_scale, C, out_dtype, stream);
}

extern "C" int mx_gemm_noalloc(int fmt, int64_t M, int64_t N, int64_t K,
                               const void *A, const void *A_scale,
                               const void *B, const void *B_scale,
                               void *C, int out_dtype, void *stream)
{
    mx_plan_t plan;
    int rc = make_plan(fmt, M, N, K, out_dtype, &plan);
    if (rc != MX_OK) return rc;
    return run_plan(plan, fmt, fmt, M, N, K, A, A_scale, B, B_scale, C, out_dtype, stream, true);
}

extern "C" void mx_debug_fail_allocations(int count)
{
    g_fail_allocs.store(count > 0 ? count : 0);
}

extern "C" int mx_gemm_tile(int fmt, int64_t M, int64_t N, int64_t K,
                            const void *A, const void *A_scale,
                            const void *B, const void *B_scale,
                            void *C, int out_dtype, int tile_m, int tile_n, int split_k,
                            void *stream)
{
    int rc = check_args(fmt, M, N, K, out_dtype);
    if (rc != MX_OK) return rc;
    mx_plan_t plan;
    rc = forced_plan(fmt, fmt, M, N, K, tile_m, tile_n, split_k, &plan);
    if (rc != MX_OK) return rc;
    return run_plan(plan, fmt, fmt, M, N, K, A, A_scale, B, B_scale, C, out_dtype, stream);
}

extern "C" int mx_gemm_mixed(int fmt_a, int fmt_b, int64_t M, int64_t N, int64_t K,
                             const void *A, const void *A_scale,
                             const void *B, const void *B_scale,
                             void *C, int out_dtype, int tile_m, int tile_n, int split_k,
                             void *stream)
{
    int rc = check_args(fmt_a, M, N, K, out_dtype);
    if (rc != MX_OK) return rc;
    if (fmt_b < MX_FMT_E2M1 || fmt_b > MX_FMT_E3M2) return MX_ERR_FORMAT;   // any pair
    if (split_k < 0 || split_k > kMaxSplit) return MX_ERR_SHAPE;
    mx_plan_t plan;
    if (tile_m == 0 && tile_n == 0) {
        plan_for(fmt_a, fmt_b, M, N, K, &plan, split_k);
        if (plan.workgroups > kMaxGrid) return MX_ERR_SHAPE;
    } else {
        rc = forced_plan(fmt_a, fmt_b, M, N, K, tile_m, tile_n, split_k, &plan);
        if (rc != MX_OK) return rc;
    }
    return run_plan(plan, fmt_a, fmt_b, M, N, K, A, A_scale, B, B_scale, C, out_dtype, stream);
}

extern "C" int mx_gemm_bf16_plan(int64_t M, int64_t N, int64_t K, int out_dtype,
                                 mx_plan_t *plan)
{
    if (!plan) return MX_ERR_NULL;
    const int rc = check_args_bf16(M, N, K, out_dtype);
    if (rc != MX_OK) return rc;
    fill_plan(choose_tile(M, N, K), M, N, K, plan);
    return plan->workgroups > kMaxGrid ? MX_ERR_SHAPE : MX_OK;
}

extern "C" int mx_gemm_bf16(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                            void *C, int out_dtype, int tile_m, int tile_n, int split_k,
                            void *stream)
{
    const int rc = check_args_bf16(M, N, K, out_dtype);
    if (rc != MX_OK) return rc;
    if (split_k < 0 || split_k > kMaxSplit) return MX_ERR_SHAPE;
    mx_plan_t plan;
    if (tile_m == 0 && tile_n == 0) {
        fill_plan(choose_tile(M, N, K), M, N, K, &plan, split_k);
        if (plan.workgroups > kMaxGrid) return MX_ERR_SHAPE;
    } else {
        const int rc2 = forced_plan(kFmtBF16, kFmtBF16, M, N, K, tile_m, tile_n, split_k, &plan);
        if (rc2 != MX_OK) return rc2;
    }
    return run_plan(plan, kFmtBF16, kFmtBF16, M, N, K, A, nullptr, B, nullptr, C, out_dtype,
                    stream);
}

extern "C" int mx_quantize(int fmt, int in_dtype, int64_t rows, int64_t K,
                           const void *X, void *Q, void *Q_scale, void *stream)
{
    if (fmt < MX_FMT_E2M1 || fmt > MX_FMT_E3M2) return MX_ERR_FORMAT;
    if (in_dtype != MX_IN_FP32 && in_dtype != MX_IN_BF16) return MX_ERR_IN_DTYPE;
    if (rows < 1 || K < 32 || K % 32 != 0 || rows > MX_MAX_DIM || K > MX_MAX_DIM)
        return MX_ERR_SHAPE;
    if (!X || !Q || !Q_scale) return MX_ERR_NULL;
    if (!aligned(X, 16) || !aligned(Q, 8)) return MX_ERR_ALIGN;
    int dev = -1;
    const int rc = device_ready(&dev);
    if (rc != MX_OK) return rc;
    const int64_t nblocks = rows * (K / 32);
    const bool fp6 = fmt == MX_FMT_E2M3 || fmt == MX_FMT_E3M2;
    const int lpb = fp6 ? 2 : in_dtype == MX_IN_FP32 ? 8 : 4;  // lanes per block
    const int64_t per_wg = 256 / lpb;                          // blocks per pass
    const unsigned grid = (unsigned)std::min<int64_t>(cdiv(nblocks, per_wg), 8 * kCUs);
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    uint8_t *q = (uint8_t *)Q, *qs = (uint8_t *)Q_scale;
    if (fmt == MX_FMT_E2M1) {
        if (in_dtype == MX_IN_FP32)
            hipLaunchKernelGGL((mx::quantize_kernel<mx::FP4, mx::IN_F32>), dim3(grid), dim3(256), 0, s, X, q, qs, nblocks);
        else
            hipLaunchKernelGGL((mx::quantize_kernel<mx::FP4, mx::IN_BF16>), dim3(grid), dim3(256), 0, s, X, q, qs, nblocks);
    } else if (fmt == MX_FMT_E4M3) {
        if (in_dtype == MX_IN_FP32)
            hipLaunchKernelGGL((mx::quantize_kernel<mx::FP8, mx::IN_F32>), dim3(grid), dim3(256), 0, s, X, q, qs, nblocks);
        else
            hipLaunchKernelGGL((mx::quantize_kernel<mx::FP8, mx::IN_BF16>), dim3(grid), dim3(256), 0, s, X, q, qs, nblocks);
    } else if (fmt == MX_FMT_E5M2) {
        if (in_dtype == MX_IN_FP32)
            hipLaunchKernelGGL((mx::quantize_kernel<mx::BF8, mx::IN_F32>), dim3(grid), dim3(256), 0, s, X, q, qs, nblocks);
        else
            hipLaunchKernelGGL((mx::quantize_kernel<mx::BF8, mx::IN_BF16>), dim3(grid), dim3(256), 0, s, X, q, qs, nblocks);
    } else if (fmt == MX_FMT_E2M3) {
        if (in_dtype == MX_IN_FP32)
            hipLaunchKernelGGL((mx::quantize6_kernel<mx::F6E2, mx::IN_F32>), dim3(grid), dim3(256), 0, s, X, q, qs, nblocks);
        else
            hipLaunchKernelGGL((mx::quantize6_kernel<mx::F6E2, mx::IN_BF16>), dim3(grid), dim3(256), 0, s, X, q, qs, nblocks);
    } else {
        if (in_dtype == MX_IN_FP32)
            hipLaunchKernelGGL((mx::quantize6_kernel<mx::F6E3, mx::IN_F32>), dim3(grid), dim3(256), 0, s, X, q, qs, nblocks);
        else
            hipLaunchKernelGGL((mx::quantize6_kernel<mx::F6E3, mx::IN_BF16>), dim3(grid), dim3(256), 0, s, X, q, qs, nblocks);
    }
    return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

extern "C" int mx_hbm_read_ceiling(const void *src, int64_t bytes, uint32_t *out, void *stream)
{
    if (!src || !out) return MX_ERR_NULL;
    if (bytes < 16 || bytes % 16 != 0) return MX_ERR_SHAPE;
    if (!aligned(src, 16) || !aligned(out, 4)) return MX_ERR_ALIGN;
    int dev = -1;
    const int rc = device_ready(&dev);
    if (rc != MX_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    hipLaunchKernelGGL(mx::hbm_read_kernel, dim3(MX_HBM_CEILING_WORKGROUPS),
                       dim3(MX_HBM_CEILING_THREADS), 0, s, (const mx::v4i *)src, bytes / 16, out);
    return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

extern "C" int mx_mfma_ceiling(int fmt, int64_t steps, int random_data, float *out,
                               void *stream)
{
    if (fmt != MX_FMT_E2M1 && fmt != MX_FMT_E4M3) return MX_ERR_FORMAT;
    if (steps < 2 || steps % 2 != 0 || steps > ((int64_t)1 << 30)) return MX_ERR_SHAPE;
    if (!out) return MX_ERR_NULL;
    if (!aligned(out, 4)) return MX_ERR_ALIGN;
    int dev = -1;
    const int rc = device_ready(&dev);
    if (rc != MX_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    if (fmt == MX_FMT_E2M1)
        hipLaunchKernelGGL(mx::mfma_ceiling_kernel<mx::FP4>, dim3(MX_CEILING_WORKGROUPS),
                           dim3(MX_CEILING_THREADS), 0, s, out, (int)steps, random_data);
    else
        hipLaunchKernelGGL(mx::mfma_ceiling_kernel<mx::FP8>, dim3(MX_CEILING_WORKGROUPS),
                           dim3(MX_CEILING_THREADS), 0, s, out, (int)steps, random_data);
    return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}
