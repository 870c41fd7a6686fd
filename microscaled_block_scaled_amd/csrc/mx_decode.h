// mx_decode.h -- the decode kernel: the MX GEMM for M <= 32 rows, a batch
// of tokens against a weight matrix (the small-M case of the FlyDSL
// article's decode-shaped GEMMs; digest 2026-10-22, item 1).  Such a GEMM
// reads each weight byte once and does 2M FLOP per byte, far below the MFMA
// ridge: its time is the time to stream B from HBM.
//
// C is cut into column groups of 32 columns (all M rows).  A workgroup of
// four waves takes groups blockIdx.x, blockIdx.x + gridDim.x, ...; the grid
// is at most one workgroup per CU.  Its four waves take four consecutive
// K-ranges of whole 512-K scale periods, one each, and after each group add
// their 32 x 32 FP32 partial tiles in LDS in wave order (so the result does
// not depend on timing).  The tile kernel instead splits K across
// workgroups, writes FP32 planes to memory and adds them in a second
// kernel; here the only memory traffic is A, B, their scales and C.
//
// A wave works alone: a private ring of slabs in LDS (a slab holds 128 or
// 256 K-values of the staged A rows and 32 B rows, as in the tile kernel,
// with the same XOR swizzle), filled by 16-byte buffer copies straight from
// HBM and read back as MFMA fragments, with no workgroup barrier in the K
// loop.  Its copies form one stream over all its groups: the first slabs of
// the next group are in flight while a group's last slabs are multiplied
// and its partial tiles are added, so a workgroup with several groups does
// not refill its pipeline from empty for each.  Rows of A past M and of B
// past N lie past the copy descriptor's num_records and are not fetched
// (their results are never stored).  B is read once and carries the
// nontemporal hint.  Scale bytes are loaded into registers, a few periods
// ahead.
#pragma once

#include "mx_kernels.h"

namespace mx {

constexpr int kDecodeWaves = 4;      // waves per workgroup, one K-range each
constexpr int kDecodeRows = 32;      // columns of C per workgroup, and the most rows of A
constexpr int kDecodeLds = 163840;   // LDS per workgroup: all of a CU's 160 KB
// LDS for adding the waves' partial tiles: a 32 x 32 FP32 tile per wave.
constexpr int kDecodeRed = kDecodeWaves * kDecodeRows * kDecodeRows * 4;

// Wait until at most N of this wave's memory loads are outstanding and all
// of its LDS reads are done (the ring slot about to be refilled was read by
// the previous slab's fragments).
template <int N>
__device__ __forceinline__ void wait_vm_lds()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}

// Slab geometry of the decode kernel for formats (FA, FB): the tile
// kernel's slabs (128 K-values, 256 when both operands are E2M1), 32 rows
// of A and 32 of B.  WIDE is for an E4M3 / E5M2 A with an E2M1 B and M <= 8
// (8-bit activations, 4-bit weights): 256-K slabs, so that each B row of a
// slab is one whole 128-byte line (with 128-K slabs it is half of one,
// and the line's other half is fetched again), A rows of 256 bytes, and
// only the 8 A rows of two copy instructions staged, which keeps the ring
// 6 slabs deep.  (Staging 8 A rows in the other geometries too, for a ring
// of 8 slabs instead of 5, measured no faster on MI355X: at M = 8,
// N = 8192, K = 28672 the same time within 1 %, and up to 18 % slower for
// E2M1 with K <= 4096.)
template <int FA, int FB, bool WIDE = false>
struct decode_geo {
    using SL = slab<FA, FB>;
    static_assert(!WIDE || (FB == FP4 && FA != FP4), "the wide slabs pair an 8-bit A with an E2M1 B");
    static constexpr int KS = WIDE ? 256 : SL::kvals;          // K-values per slab
    static constexpr int RA = WIDE ? 256 : SL::template row_bytes<FA>;   // slab row bytes
    static constexpr int RB = WIDE ? 128 : SL::template row_bytes<FB>;
    static constexpr int MA = WIDE ? 8 : kDecodeRows;         // rows of A staged
    static constexpr int NCOPY = MA * RA / 1024 + kDecodeRows * RB / 1024;   // copies per slab
    static constexpr int SLOT = MA * RA + kDecodeRows * RB;   // LDS bytes per slab
    // ring depth: as many slabs as the LDS beside the partial-tile area
    // holds, within the wait's count field ((S - 2) * NCOPY loads
    // outstanding, at most 63)
    static constexpr int S_LDS = (kDecodeLds - kDecodeRed) / (kDecodeWaves * SLOT);
    static constexpr int S_CNT = 2 + 63 / NCOPY;
    static constexpr int S = S_LDS < S_CNT ? S_LDS : S_CNT;
    static constexpr int WAVE_LDS = S * SLOT;
    static constexpr int SMEM = kDecodeWaves * WAVE_LDS + kDecodeRed;
};

// LDS swizzle of a slab row of R bytes: the tile kernel's for 128- and
// 64-byte rows; for 256-byte rows (16 chunks) chunk c of row r is stored at
// chunk c ^ (r mod 16), so 16 rows reading one chunk touch 16 distinct
// 16-byte bank groups.
template <int R> __device__ __forceinline__ int decode_swz(int r)
{
    return R == 256 ? (r & 15) : swz_row<R>(r);
}

template <int FA, int FB, int OUT, bool WIDE>
__global__ void __launch_bounds__(kDecodeWaves * 64)
decode_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
              const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs, void *__restrict__ C,
              int M, int N, int K)
{
    using SL = slab<FA, FB>;
    using G = decode_geo<FA, FB, WIDE>;
    static_assert(SL::scaled && !is_fp6<FA>::value && !is_fp6<FB>::value,
                  "E2M1, E4M3 and E5M2 operands");
    constexpr int KS = G::KS;                        // K-values per slab: 128 or 256
    constexpr int HS = KS / 64;                      // 64-K MFMA steps per slab: 2 or 4
    constexpr int PS = 512 / KS;                     // slabs per scale period
    constexpr int RA = G::RA, RB = G::RB, MA = G::MA;
    constexpr int RPCA = 1024 / RA, RPCB = 1024 / RB;             // rows per copy instruction
    constexpr int CPA = MA / RPCA, CPB = kDecodeRows / RPCB;      // copies per slab
    constexpr int NCOPY = G::NCOPY;
    static_assert(NCOPY == CPA + CPB, "copies per slab");
    constexpr int S = G::S, SLOT = G::SLOT;
    static_assert(S >= 3 && (S - 2) * NCOPY <= 63, "ring depth and the vmcnt field");
    static_assert(G::SMEM <= kDecodeLds, "LDS budget");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[G::SMEM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, g = lane >> 5;
    uint8_t *const ring = smem + wave * G::WAVE_LDS;
    float *const red = (float *)(smem + kDecodeWaves * G::WAVE_LDS);

    // This workgroup's column groups: gi = 0 .. ng-1 is group
    // blockIdx.x + gi * gridDim.x, columns n0 .. n0+31 of it.
    const int ngroups = (N + kDecodeRows - 1) / kDecodeRows;
    const int ng = (int)blockIdx.x < ngroups ? (ngroups - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
    auto group_n0 = [&](int gi) { return ((int)blockIdx.x + gi * (int)gridDim.x) * kDecodeRows; };

    // This wave's K-range [kb, kb + klen), the same for every group: whole
    // 512-K periods, split as evenly as they go; the last wave's range ends
    // at K (and may be empty).
    const int per_w = (K / 128 + 4 * kDecodeWaves - 1) / (4 * kDecodeWaves);
    const int kb = min(wave * per_w * 512, K), klen = min(per_w * 512, K - kb);
    const int nslab = (klen + KS - 1) / KS, nsteps = klen / 64, nper = (klen + 511) / 512;
    const int64_t rowba = kbytes<FA>(K), rowbb = kbytes<FB>(K);
    const int64_t kboffa = kbytes<FA>(kb), kboffb = kbytes<FB>(kb);
    const int64_t rowla = kbytes<FA>(klen), rowlb = kbytes<FB>(klen);
    const int sps = K / 32;                          // scale bytes per row

    // Scale registers: period q's bytes in (sa, sb), and the raw loads of
    // the next L periods in a ring of L register sets, period q in set q % L.
    // L periods of slab copies (at least S - 1 slab positions) separate a
    // period's loads from their use, so waiting for them never stalls the
    // copies in flight.
    constexpr int L = (S - 1 + PS - 1) / PS;
    // The stream: each group takes ppq periods (its range's, rounded up to
    // whole trips of L) of PS slab positions; position j is slab j % ppg of
    // group j / ppg.  Positions past a group's slabs, and past its last
    // group, copy nothing and do no MFMA.
    const int ppq = nslab > 0 ? (nper + L - 1) / L * L : 0;
    const int ppg = ppq * PS;

    // Copy geometry (the tile kernel's): lane l copies chunk l % (R/16) of row
    // l / (R/16) of a block of rows into that chunk of the row's LDS copy,
    // which holds global chunk (chunk ^ swizzle(row)).
    const int crowa = lane / (RA / 16), cpca = lane % (RA / 16);
    const int crowb = lane / (RB / 16), cpcb = lane % (RB / 16);
    const uint8_t *const Ab = A + kboffa;
    // Extents from each copy base to the end of the last real row: copies of
    // rows at or past M (A) or N (B) are not fetched.  Under 2^32: at most 32
    // rows of at most 2^24 bytes.
    const uint32_t exta = (uint32_t)(M * rowba - kboffa);

    // Copy stream position j into ring slot j % S.  Every position issues
    // the same copies, also those with no slab (then with num_records 0:
    // nothing is fetched), so that the count of loads in flight is the same
    // on every path through the loop.  When both operands are E2M1 and
    // klen % 256 == 128 the last slab is half a slab: its chunk offsets are
    // clamped into the range (those chunks are never read).
    auto issue = [&](int j) {
        uint8_t *const dst = ring + (j % S) * SLOT;
        const int gj = j / ppg, k = j - gj * ppg;
        const bool live = gj < ng && k < nslab;
        const int kc = min(k, nslab - 1);
        const int n0 = group_n0(min(gj, ng - 1));
        const uint32_t extb = (uint32_t)(min(kDecodeRows, N - n0) * rowbb - kboffb);
        const uint8_t *const Bb = B + (int64_t)n0 * rowbb + kboffb;
        const uint32_t koffa = (uint32_t)kc * RA, koffb = (uint32_t)kc * RB;
        const uint32_t cmaxa = (uint32_t)(rowla - 16) - koffa, cmaxb = (uint32_t)(rowlb - 16) - koffb;
        const rsrc_t Ak = make_rsrc(Ab + koffa, live ? exta - koffa : 0u);
        const rsrc_t Bk = make_rsrc(Bb + koffb, live ? extb - koffb : 0u);
#pragma unroll
        for (int i = 0; i < CPA; ++i) {
            const int row = i * RPCA + crowa;
            const uint32_t ch = min((uint32_t)(cpca ^ decode_swz<RA>(row)) << 4, cmaxa);
            b2l_16(Ak, (uint32_t)row * (uint32_t)rowba + ch, dst + i * 1024);
        }
#pragma unroll
        for (int i = 0; i < CPB; ++i) {
            const int row = i * RPCB + crowb;
            const uint32_t ch = min((uint32_t)(cpcb ^ decode_swz<RB>(row)) << 4, cmaxb);
            b2l_16<kStream>(Bk, (uint32_t)row * (uint32_t)rowbb + ch,
                            dst + MA * RA + i * 1024);
        }
    };

    // Scale bytes of stream period qg (period qg % ppq of group qg / ppq).
    // load_scales fetches the 16 bytes of period q (blocks kb/32 + 16q ..)
    // of A row lr and B row n0 + lr; a short last period is fetched as the
    // 16 bytes that end at the row's end, so that no load crosses a row.
    // Rows past M (N) are past the descriptors' num_records: not fetched.
    // use_scales then rotates a short period back by whole dwords and shifts
    // each dword right by 8g bits, so that this lane group's byte of step s
    // (block 2s + g of the period) is byte 2(s % 2) of dword s / 2.  The
    // empty asm pins that work, and with it the wait for the loads, to where
    // use_scales is called (else the compiler may start it right after the
    // loads and wait for them there).
    const rsrc_t Asr = make_rsrc(As, (uint32_t)(M * sps));
    auto scale_at = [&](int q) { return min(kb / 32 + 16 * min(q, nper - 1), sps - 16); };
    auto load_scales = [&](int qg, v4i &ra, v4i &rb) {
        const int gq = qg / ppq, q = qg - gq * ppq;
        const int n0 = group_n0(min(gq, ng - 1));
        const rsrc_t Bsr = make_rsrc(Bs + (int64_t)n0 * sps,
                                     (uint32_t)(min(kDecodeRows, N - n0) * sps));
        const uint32_t off = (uint32_t)lr * (uint32_t)sps + (uint32_t)scale_at(q);
        ra = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(Asr, off, 0, 0));
        rb = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(Bsr, off, 0, 0));
    };
    auto use_scales = [&](int qg, v4i a, v4i b, v4i &sa, v4i &sb) {
        asm volatile("" : "+v"(a), "+v"(b));
        const int q = qg % ppq;
        const int rot = (kb / 32 + 16 * min(q, nper - 1) - scale_at(q)) >> 2;
        if (rot & 1) { a = v4i{a[1], a[2], a[3], a[0]}; b = v4i{b[1], b[2], b[3], b[0]}; }
        if (rot & 2) { a = v4i{a[2], a[3], a[0], a[1]}; b = v4i{b[2], b[3], b[0], b[1]}; }
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            sa[d] = (int)((uint32_t)a[d] >> (8 * g));
            sb[d] = (int)((uint32_t)b[d] >> (8 * g));
        }
    };

    // Fragment of step p of a slab for lane row lr, from NR staged rows of R
    // bytes at `rows` (with NR = 8, the A rows of the wide slabs, lane row lr
    // reads row lr % 8; only rows below M <= 8 are stored): E4M3 / E5M2
    // chunks 4p+g and 4p+2+g, E2M1 chunk 2p+g.
    auto frag = [&](auto fc, auto rc, auto nc, const uint8_t *rows, int p, v8i &v) {
        constexpr int F = decltype(fc)::value, R = decltype(rc)::value, NR = decltype(nc)::value;
        const int r = lr % NR;
        const int sw = decode_swz<R>(r);
        const uint8_t *rp = rows + r * R;
        const int c0 = F == FP4 ? 2 * p + g : 4 * p + g;
        const v4i lo = *(const v4i *)(rp + ((c0 ^ sw) << 4));
        if constexpr (F == FP4) {
            v = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
        } else {
            const v4i hi = *(const v4i *)(rp + (((c0 + 2) ^ sw) << 4));
            v = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    };
    static_assert(WIDE || (RA == (FA == FP4 && FB != FP4 ? 64 : 128) &&
                           RB == (FB == FP4 && FA != FP4 ? 64 : 128)),
                  "slab rows as the fragment reads assume");

    v16f acc;
    v4i sa, sb, ra[L], rb[L];

    // Stream period qg = gi * ppq + q (period q of group gi), whose scales
    // are set i = q % L: its slabs, the loads of period qg + L into set i
    // (free since period qg's scales were made current), and at its end
    // period qg + 1's scales made current.
    auto period = [&](auto ic, int gi, int q) {
        constexpr int i = decltype(ic)::value;
        const int qg = gi * ppq + q;
        load_scales(qg + L, ra[i], rb[i]);
        static_for<PS>([&](auto kc) {
            constexpr int kp = decltype(kc)::value;
            const int k = q * PS + kp, j = qg * PS + kp;
            // Position j is in once at most the copies of the S - 2
            // positions issued after it are outstanding (the scale loads
            // issued since only make the wait stricter).
            wait_vm_lds<(S - 2) * NCOPY>();
            issue(j + S - 1);                        // into the slot of position j - 1
            if (k < nslab) {
                const uint8_t *slot = ring + (j % S) * SLOT;
                static_for<HS>([&](auto pc) {
                    constexpr int p = decltype(pc)::value, s = kp * HS + p;
                    if (HS == 2 || k * HS + p < nsteps) {
                        v8i a, b;
                        frag(std::integral_constant<int, FA>{}, std::integral_constant<int, RA>{},
                             std::integral_constant<int, MA>{}, slot, p, a);
                        frag(std::integral_constant<int, FB>{}, std::integral_constant<int, RB>{},
                             std::integral_constant<int, kDecodeRows>{}, slot + MA * RA, p, b);
                        acc = mma<FA, FB, 2 * (s & 1)>(a, b, acc, sa[s >> 1], sb[s >> 1]);
                    }
                });
            }
        });
        use_scales(qg + 1, ra[(i + 1) % L], rb[(i + 1) % L], sa, sb);
    };

    // Add the waves' partial tiles of group gi in wave order and store them.
    // In the MFMA result lane (c, g) holds, in element e, row
    // 8(e/4) + 4g + e%4 of column c; element e of lane l is kept at
    // red[1024 w + 64 e + l].  The barriers order LDS only: the stream's
    // copies into the rings stay in flight.
    auto add_and_store = [&](int gi) {
        const int n0 = group_n0(gi), rows_b = min(kDecodeRows, N - n0);
#pragma unroll
        for (int e = 0; e < 16; ++e) red[wave * 1024 + e * 64 + lane] = acc[e];
        lds_barrier();
#pragma unroll
        for (int q = 0; q < kDecodeRows * kDecodeRows / (kDecodeWaves * 64); ++q) {
            const int m = q * 8 + (tid >> 5), c = tid & 31;
            if (m >= M || c >= rows_b) continue;
            const int at = ((m >> 3) * 4 + (m & 3)) * 64 + c + 32 * ((m >> 2) & 1);
            float v = red[at];
#pragma unroll
            for (int w = 1; w < kDecodeWaves; ++w) v += red[w * 1024 + at];
            if constexpr (OUT == OF32) ((float *)C)[(int64_t)m * N + n0 + c] = v;
            else ((uint16_t *)C)[(int64_t)m * N + n0 + c] = f32_to_bf16(v);
        }
        lds_barrier();
    };

    if (ppg > 0) {
        static_for<L>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            load_scales(i, ra[i], rb[i]);
        });
#pragma unroll
        for (int j = 0; j < S - 1; ++j) issue(j);
        use_scales(0, ra[0], rb[0], sa, sb);
        for (int gi = 0; gi < ng; ++gi) {
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[e] = 0.f;
            // L periods per trip, so that the register sets keep their
            // roles without a register move (a move of a load's result
            // waits for the load).
            for (int q = 0; q < ppq; q += L)
                static_for<L>([&](auto ic) { period(ic, gi, q + decltype(ic)::value); });
            add_and_store(gi);
        }
    } else {                                         // an empty K-range: zero partial tiles
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.f;
        for (int gi = 0; gi < ng; ++gi) add_and_store(gi);
    }
    wait_vm0();                                      // the copies past the last group
}

}  // namespace mx
