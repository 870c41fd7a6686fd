// mxdecode.hip -- launches of the decode kernel (mx_decode.h) for every pair
// of the E2M1, E4M3 and E5M2 formats, in a translation unit of their own so
// that the library builds in parallel.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "mx_decode.h"
#include "mx_launch.h"

namespace mxhost {

namespace {

template <int FA, int FB>
void go(int out_dtype, const void *A, const void *As, const void *B, const void *Bs, void *C,
        int64_t M, int64_t N, int64_t K, hipStream_t s)
{
    // at most one workgroup per CU; each takes every gridDim-th column group
    const dim3 grid((unsigned)std::min<int64_t>(cdiv(N, MX_DECODE_TILE), kCUs));
    const dim3 block(mx::kDecodeWaves * 64);
    const uint8_t *a = (const uint8_t *)A, *as = (const uint8_t *)As;
    const uint8_t *b = (const uint8_t *)B, *bs = (const uint8_t *)Bs;
    const bool f32 = out_dtype == MX_OUT_FP32;
    // An 8-bit A with an E2M1 B: the wide slabs, with 8, 16 or 32 A rows
    // staged
    if constexpr (FB == mx::FP4 && FA != mx::FP4) {
        if (M <= 8) {
            if (f32)
                hipLaunchKernelGGL((mx::decode_kernel<FA, FB, mx::OF32, 8>), grid, block, 0, s,
                                   a, as, b, bs, C, (int)M, (int)N, (int)K);
            else
                hipLaunchKernelGGL((mx::decode_kernel<FA, FB, mx::OBF16, 8>), grid, block, 0, s,
                                   a, as, b, bs, C, (int)M, (int)N, (int)K);
            return;
        }
        if (M <= 16) {
            if (f32)
                hipLaunchKernelGGL((mx::decode_kernel<FA, FB, mx::OF32, 16>), grid, block, 0, s,
                                   a, as, b, bs, C, (int)M, (int)N, (int)K);
            else
                hipLaunchKernelGGL((mx::decode_kernel<FA, FB, mx::OBF16, 16>), grid, block, 0, s,
                                   a, as, b, bs, C, (int)M, (int)N, (int)K);
            return;
        }
        if (f32)
            hipLaunchKernelGGL((mx::decode_kernel<FA, FB, mx::OF32, 32>), grid, block, 0, s,
                               a, as, b, bs, C, (int)M, (int)N, (int)K);
        else
            hipLaunchKernelGGL((mx::decode_kernel<FA, FB, mx::OBF16, 32>), grid, block, 0, s,
                               a, as, b, bs, C, (int)M, (int)N, (int)K);
    } else {
        if (f32)
            hipLaunchKernelGGL((mx::decode_kernel<FA, FB, mx::OF32, 0>), grid, block, 0, s, a,
                               as, b, bs, C, (int)M, (int)N, (int)K);
        else
            hipLaunchKernelGGL((mx::decode_kernel<FA, FB, mx::OBF16, 0>), grid, block, 0, s, a,
                               as, b, bs, C, (int)M, (int)N, (int)K);
    }
}

int kernel_fmt(int fmt)
{
    return fmt == MX_FMT_E2M1 ? mx::FP4 : fmt == MX_FMT_E4M3 ? mx::FP8
         : fmt == MX_FMT_E5M2 ? mx::BF8 : 0;
}

}  // namespace

bool launch_decode(int fmt_a, int fmt_b, int out_dtype, const void *A, const void *As,
                   const void *B, const void *Bs, void *C, int64_t M, int64_t N, int64_t K,
                   hipStream_t s)
{
    if (!decode_fits(fmt_a, fmt_b, M, N, K)) return false;
    const int fa = kernel_fmt(fmt_a), fb = kernel_fmt(fmt_b);
#define MX_DEC(FA_, FB_)                                                                   \
    if (fa == FA_ && fb == FB_) {                                                          \
        go<FA_, FB_>(out_dtype, A, As, B, Bs, C, M, N, K, s);                              \
        return true;                                                                       \
    }
    MX_DEC(mx::FP4, mx::FP4)
    MX_DEC(mx::FP8, mx::FP8)
    MX_DEC(mx::BF8, mx::BF8)
    MX_DEC(mx::FP8, mx::FP4)
    MX_DEC(mx::FP4, mx::FP8)
    MX_DEC(mx::FP8, mx::BF8)
    MX_DEC(mx::BF8, mx::FP8)
    MX_DEC(mx::BF8, mx::FP4)
    MX_DEC(mx::FP4, mx::BF8)
#undef MX_DEC
    return false;
}

}  // namespace mxhost
