// The GPU library's host logic under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Test infrastructure: tests/test_sanitize_cpu.py
// compiles the library's sources for the host only (no device code; the
// kernels are never launched) with both sanitizers and links this driver.
// It calls every entry point of include/mxgemm.h along paths that return
// before any HIP call: the plans over a grid of shapes up to the ABI's
// limits (checking each plan's arithmetic), the tile table, the error
// strings, and every argument error (null, misaligned, bad shape, format,
// output type, group table, scratch size).  The sanitizers abort on the
// first out-of-bounds access or undefined operation (signed overflow
// included).  Prints "host checks passed" and exits 0 otherwise.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <vector>

#include "mxgemm.h"

static int fails = 0;
#define CHECK(c)                                                                  \
    do {                                                                          \
        if (!(c)) {                                                               \
            std::fprintf(stderr, "check failed, line %d: %s\n", __LINE__, #c);    \
            ++fails;                                                              \
        }                                                                         \
    } while (0)

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

static const int64_t kDims[] = {-1, 0, 1, 7, 8, 31, 32, 64, 127, 128, 129, 160, 192, 255, 256,
                                257, 1000, 2048, 5120, 8192, 28672, 65535, (int64_t)1 << 30,
                                ((int64_t)1 << 30) + 1};
static const int64_t kKs[] = {-128, 0, 16, 64, 100, 128, 256, 384, 512, 640, 2048, 4096, 25600,
                              28672, (int64_t)1 << 23, ((int64_t)1 << 23) + 16, (int64_t)1 << 24,
                              ((int64_t)1 << 24) + 128};

// A plan's arithmetic: whole tiles, slices of whole 512-K periods covering K
// with none empty, workspace of split_k planes; or the decode kernel, only
// for M <= MX_DECODE_TILE, K >= 512 and formats other than FP6 (fp6 true).
static void check_plan(const mx_plan_t &p, int64_t M, int64_t N, int64_t K, bool fp6 = false)
{
    if (p.variant == MX_VARIANT_DECODE) {
        CHECK(!fp6 && M >= 1 && M <= MX_DECODE_TILE && K >= 512);
        CHECK(p.tile_m == MX_DECODE_TILE && p.tile_n == MX_DECODE_TILE && p.split_k == 1);
        CHECK(p.threads == 256 && p.workspace_bytes == 0);
        CHECK(p.workgroups == std::min<int64_t>(cdiv(N, MX_DECODE_TILE), 256));
        return;
    }
    CHECK(p.variant == MX_VARIANT_TILE);
    CHECK(p.tile_m > 0 && p.tile_n > 0 && p.threads > 0 && p.threads <= 1024);
    CHECK(p.split_k >= 1 && p.split_k <= MX_MAX_SPLIT_K);
    const int64_t tiles = cdiv(M, p.tile_m) * cdiv(N, p.tile_n);
    CHECK(p.workgroups == tiles * p.split_k);
    if (p.split_k > 1) {
        const int64_t slice = cdiv(cdiv(K, p.split_k), 512) * 512;
        CHECK(cdiv(K, slice) == p.split_k);
        CHECK(p.workspace_bytes == p.split_k * cdiv(M * N, 64) * 64 * 4);
    } else {
        CHECK(p.workspace_bytes == 0);
    }
}

int main()
{
    for (int c = -40; c <= 40; ++c) {
        const char *s = mx_strerror(c);
        CHECK(s && std::strlen(s) > 0);
    }

    const int nt = mx_tile_shapes(nullptr, 0);
    CHECK(nt > 0 && nt < 64);
    std::vector<int> pairs(2 * nt + 2, -7);
    CHECK(mx_tile_shapes(pairs.data(), nt) == nt);
    CHECK(pairs[2 * nt] == -7 && pairs[2 * nt + 1] == -7);
    CHECK(mx_tile_shapes(pairs.data(), 1) == nt);

    // Plans: MX formats (and codes around them), both output types (and bad
    // ones), every M, N, K of the grid.
    int planned = 0, decode = 0;
    for (int fmt = -1; fmt <= 7; ++fmt)
        for (int out = 0; out <= 3; ++out)
            for (int64_t M : kDims)
                for (int64_t N : kDims)
                    for (int64_t K : kKs) {
                        mx_plan_t p;
                        std::memset(&p, 0x5a, sizeof p);
                        const int rc = mx_gemm_plan(fmt, M, N, K, out, &p);
                        CHECK(rc <= 0 && rc >= MX_ERR_SCRATCH);
                        if (rc == MX_OK) {
                            check_plan(p, M, N, K, fmt == MX_FMT_E2M3 || fmt == MX_FMT_E3M2);
                            ++planned;
                            decode += p.variant == MX_VARIANT_DECODE;
                        }
                    }
    CHECK(planned > 1000 && decode > 100);
    CHECK(mx_gemm_plan(1, 8, 8, 128, 2, nullptr) == MX_ERR_NULL);

    for (int out = 0; out <= 3; ++out)
        for (int64_t M : kDims)
            for (int64_t N : kDims)
                for (int64_t K : kKs) {
                    mx_plan_t p;
                    const int rc = mx_gemm_bf16_plan(M, N, K, out, &p);
                    CHECK(rc <= 0);
                    if (rc == MX_OK) check_plan(p, M, N, K, true);
                }

    // Forced tiles and splits: every tile shape, the decode tile, the plan's
    // choice (0, 0) and an unknown tile, splits 0..MX_MAX_SPLIT_K and beyond,
    // on shapes up to the limits.  Null operands: the call returns after
    // planning, before any HIP call.
    const int extra[][2] = {{100, 100}, {MX_DECODE_TILE, MX_DECODE_TILE}, {0, 0}};
    for (int t = 0; t < nt + 3; ++t) {
        const int bm = t < nt ? pairs[2 * t] : extra[t - nt][0];
        const int bn = t < nt ? pairs[2 * t + 1] : extra[t - nt][1];
        for (int split = -1; split <= MX_MAX_SPLIT_K + 1; ++split)
            for (int64_t M : kDims)
                for (int64_t N : kDims)
                    for (int64_t K : kKs) {
                        int rc = mx_gemm_tile(1, M, N, K, nullptr, nullptr, nullptr, nullptr,
                                              nullptr, 2, bm, bn, split, nullptr);
                        CHECK(rc < 0);
                        rc = mx_gemm_mixed(2, 1, M, N, K, nullptr, nullptr, nullptr, nullptr,
                                           nullptr, 1, bm, bn, split, nullptr);
                        CHECK(rc < 0);
                        rc = mx_gemm_bf16(M, N, K, nullptr, nullptr, nullptr, 2, bm, bn, split,
                                          nullptr);
                        CHECK(rc < 0);
                    }
    }

    // Argument errors of the launching entry points, all before any HIP call:
    // null and misaligned pointers (never dereferenced), shapes, formats.
    uint8_t *const fake = reinterpret_cast<uint8_t *>((uintptr_t)1 << 20);
    CHECK(mx_gemm(1, 8, 8, 128, nullptr, fake, fake, fake, fake, 2, nullptr) == MX_ERR_NULL);
    CHECK(mx_gemm(1, 8, 8, 128, fake + 8, fake, fake, fake, fake, 2, nullptr) == MX_ERR_ALIGN);
    CHECK(mx_gemm(1, 8, 8, 128, fake, fake + 2, fake, fake, fake, 2, nullptr) == MX_ERR_ALIGN);
    CHECK(mx_gemm(1, 8, 8, 128, fake, fake, fake, fake, fake + 4, 2, nullptr) == MX_ERR_ALIGN);
    CHECK(mx_gemm(9, 8, 8, 128, fake, fake, fake, fake, fake, 2, nullptr) == MX_ERR_FORMAT);
    CHECK(mx_gemm(1, 8, 8, 128, fake, fake, fake, fake, fake, 5, nullptr) == MX_ERR_OUT_DTYPE);
    CHECK(mx_gemm(1, 8, 8, 100, fake, fake, fake, fake, fake, 2, nullptr) == MX_ERR_SHAPE);
    CHECK(mx_gemm_noalloc(2, 512, 6144, 28672, fake, fake, fake, fake, fake, 2, nullptr) ==
          MX_ERR_SCRATCH);
    CHECK(mx_gemm_noalloc(2, 8, 8, 128, nullptr, fake, fake, fake, fake, 2, nullptr) ==
          MX_ERR_NULL);
    CHECK(mx_gemm_noalloc(2, (int64_t)1 << 30, (int64_t)1 << 30, 128, fake, fake, fake, fake,
                          nullptr, 2, nullptr) == MX_ERR_SHAPE);
    for (int fmt = -1; fmt <= 7; ++fmt)
        for (int in = 0; in <= 3; ++in)
            for (int64_t rows : kDims)
                for (int64_t K : kKs) {
                    const int rc = mx_quantize(fmt, in, rows, K, nullptr, fake, fake, nullptr);
                    CHECK(rc < 0);
                }
    CHECK(mx_quantize(1, 1, 8, 64, fake + 4, fake, fake, nullptr) == MX_ERR_ALIGN);
    CHECK(mx_quantize(1, 1, 8, 64, fake, fake + 4, fake, nullptr) == MX_ERR_ALIGN);
    for (int fmt = -1; fmt <= 3; ++fmt)
        for (int64_t steps : {(int64_t)-2, (int64_t)0, (int64_t)1, (int64_t)2, (int64_t)3,
                              (int64_t)1 << 30, ((int64_t)1 << 30) + 2})
            CHECK(mx_mfma_ceiling(fmt, steps, 1, nullptr, nullptr) < 0);
    // Valid arguments reach the device check, which finds no device.
    CHECK(mx_gemm(1, 8, 8, 128, fake, fake, fake, fake, fake, 2, nullptr) == MX_ERR_NO_DEVICE);
    CHECK(mx_gemm(2, 256, 8192, 28672, fake, fake, fake, fake, fake, 2, nullptr) ==
          MX_ERR_NO_DEVICE);
    CHECK(mx_gemm_noalloc(2, 256, 8192, 28672, fake, fake, fake, fake, fake, 2, nullptr) ==
          MX_ERR_NO_DEVICE);
    CHECK(mx_gemm_bf16(8, 8, 16, fake, fake, fake, 1, 0, 0, 0, nullptr) == MX_ERR_NO_DEVICE);
    CHECK(mx_quantize(2, 1, 8, 64, fake, fake, fake, nullptr) == MX_ERR_NO_DEVICE);
    CHECK(mx_mfma_ceiling(1, 2, 1, reinterpret_cast<float *>(fake), nullptr) == MX_ERR_NO_DEVICE);
    {
        const int64_t g2[2] = {100, 0};
        CHECK(mx_gemm_grouped(1, 2, g2, 64, 128, fake, fake, fake, fake, fake, 2, nullptr) ==
              MX_ERR_NO_DEVICE);
        const int64_t g0[2] = {0, 0};
        CHECK(mx_gemm_grouped(1, 2, g0, 64, 128, nullptr, nullptr, nullptr, nullptr, nullptr, 2,
                              nullptr) == MX_OK);
    }
    CHECK(mx_hbm_read_ceiling(nullptr, 1024, reinterpret_cast<uint32_t *>(fake), nullptr) ==
          MX_ERR_NULL);
    for (int64_t bytes : {(int64_t)-16, (int64_t)0, (int64_t)8, (int64_t)1000})
        CHECK(mx_hbm_read_ceiling(fake, bytes, reinterpret_cast<uint32_t *>(fake), nullptr) ==
              MX_ERR_SHAPE);
    CHECK(mx_hbm_read_ceiling(fake + 8, 1024, reinterpret_cast<uint32_t *>(fake), nullptr) ==
          MX_ERR_ALIGN);
    CHECK(mx_hbm_read_ceiling(fake, 1024, reinterpret_cast<uint32_t *>(fake), nullptr) ==
          MX_ERR_NO_DEVICE);
    mx_debug_fail_allocations(-3);
    mx_debug_fail_allocations(2);
    mx_debug_fail_allocations(0);

    // Grouped plans and argument errors: group counts 0..MX_MAX_GROUPS+1,
    // empty groups, negative and oversized row counts, totals beyond the
    // limit, groups * N beyond it.
    std::vector<int64_t> rows(MX_MAX_GROUPS + 1);
    for (int64_t groups : {(int64_t)0, (int64_t)1, (int64_t)2, (int64_t)8, (int64_t)255,
                           (int64_t)MX_MAX_GROUPS, (int64_t)MX_MAX_GROUPS + 1})
        for (int pattern = 0; pattern < 6; ++pattern)
            for (int64_t N : {(int64_t)1, (int64_t)160, (int64_t)4096, (int64_t)1 << 22,
                              (int64_t)1 << 30})
                for (int64_t K : {(int64_t)64, (int64_t)128, (int64_t)2048, (int64_t)1 << 24}) {
                    for (int64_t g = 0; g <= MX_MAX_GROUPS; ++g) {
                        switch (pattern) {
                        case 0: rows[g] = 0; break;
                        case 1: rows[g] = g % 3 == 0 ? 0 : 100 + 37 * g; break;
                        case 2: rows[g] = 704; break;
                        case 3: rows[g] = g == 1 ? -1 : 64; break;
                        case 4: rows[g] = (int64_t)1 << 30; break;
                        default: rows[g] = ((int64_t)1 << 22) + g; break;
                        }
                    }
                    mx_plan_t p;
                    for (int fmt = 0; fmt <= 6; ++fmt) {
                        const int rc = mx_gemm_grouped_plan(fmt, groups, rows.data(), N, K, 2, &p);
                        CHECK(rc <= 0);
                        if (rc == MX_OK) {
                            CHECK(p.split_k == 1 && p.workspace_bytes == 0);
                            int64_t tiles = 0;
                            for (int64_t g = 0; g < groups; ++g)
                                tiles += cdiv(rows[g], p.tile_m) * cdiv(N, p.tile_n);
                            CHECK(p.workgroups == tiles);
                        }
                        CHECK(mx_gemm_grouped(fmt, groups, rows.data(), N, K, nullptr, fake,
                                              fake, fake, fake, 2, nullptr) <= 0);
                        CHECK(mx_gemm_grouped_mixed(fmt, 2, groups, rows.data(), N, K, fake,
                                                    fake, fake, fake, nullptr, 2, nullptr) <= 0);
                    }
                    const int rc = mx_gemm_grouped_bf16_plan(groups, rows.data(), N, K, 2, &p);
                    CHECK(rc <= 0);
                    CHECK(mx_gemm_grouped_bf16(groups, rows.data(), N, K, nullptr, fake, fake, 2,
                                               nullptr) <= 0);
                }
    CHECK(mx_gemm_grouped_plan(1, 2, nullptr, 64, 128, 2, nullptr) == MX_ERR_NULL);

    if (fails) {
        std::fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    std::printf("host checks passed (%d plans)\n", planned);
    return 0;
}
