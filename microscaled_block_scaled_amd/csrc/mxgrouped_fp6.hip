// mxgrouped_fp6.hip -- the grouped tile kernel for an FP6 format (E2M3,
// E3M2) paired with another MX format (E2M1, E4M3, E5M2 or the other FP6
// format), compiled beside mxgrouped.hip so the two build in parallel.
#include "mx_launch.h"

namespace mxhost {

bool launch_grouped_fp6_pair(int fmt_a, int fmt_b, int t, bool f32, const void *A,
                             const void *As, const void *B, const void *Bs, void *C, int64_t N,
                             int64_t K, const mx::GroupTable &gt, hipStream_t s)
{
#define MX_P(FA_, FB_)                                                                   \
    (f32 ? launch_grouped<FA_, FB_, mx::OF32>(t, A, As, B, Bs, C, N, K, gt, s)          \
         : launch_grouped<FA_, FB_, mx::OBF16>(t, A, As, B, Bs, C, N, K, gt, s))
    if (fmt_a == MX_FMT_E2M3 || fmt_a == MX_FMT_E3M2) {
        const bool e2 = fmt_a == MX_FMT_E2M3;
        switch (fmt_b) {
        case MX_FMT_E2M1: return e2 ? MX_P(mx::F6E2, mx::FP4) : MX_P(mx::F6E3, mx::FP4);
        case MX_FMT_E4M3: return e2 ? MX_P(mx::F6E2, mx::FP8) : MX_P(mx::F6E3, mx::FP8);
        case MX_FMT_E5M2: return e2 ? MX_P(mx::F6E2, mx::BF8) : MX_P(mx::F6E3, mx::BF8);
        case MX_FMT_E2M3: return e2 ? false : MX_P(mx::F6E3, mx::F6E2);
        case MX_FMT_E3M2: return e2 ? MX_P(mx::F6E2, mx::F6E3) : false;
        default: return false;
        }
    }
    const bool e2 = fmt_b == MX_FMT_E2M3;
    if (fmt_b != MX_FMT_E2M3 && fmt_b != MX_FMT_E3M2) return false;
    switch (fmt_a) {
    case MX_FMT_E2M1: return e2 ? MX_P(mx::FP4, mx::F6E2) : MX_P(mx::FP4, mx::F6E3);
    case MX_FMT_E4M3: return e2 ? MX_P(mx::FP8, mx::F6E2) : MX_P(mx::FP8, mx::F6E3);
    case MX_FMT_E5M2: return e2 ? MX_P(mx::BF8, mx::F6E2) : MX_P(mx::BF8, mx::F6E3);
    default: return false;
    }
#undef MX_P
}

}  // namespace mxhost
