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
// with the same XOR swizzle) and a few buffers of those rows' scale bytes,
// one 512-K period each, filled by buffer copies straight from HBM and read
// back as MFMA operands, with no workgroup barrier in the K loop.  Its
// copies form one stream over all its groups: the first slabs of the next
// group are in flight while a group's last slabs are multiplied and its
// partial tiles are added, so a workgroup with several groups does not
// refill its pipeline from empty for each.  Every wait for memory is the one explicit
// wait per slab: no load writes a register, so the compiler has nothing of
// its own to wait for.  Rows of A past M and of B past N lie past the copy
// descriptor's num_records and are not fetched (their results are never
// stored).  B is read once and carries the nontemporal hint.
#pragma once

#include "mx_kernels.h"

namespace mx {

constexpr int kDecodeWaves = 4;      // waves per workgroup, one K-range each
constexpr int kDecodeRows = 32;      // columns of C per workgroup, and the most rows of A
constexpr int kDecodeLds = 163840;   // LDS per workgroup: all of a CU's 160 KB
// A wave's 32 x 32 FP32 partial tile, added in a ring slot (see add_and_store).
constexpr int kDecodeTileBytes = kDecodeRows * kDecodeRows * 4;
// Beside the rings: the byte offset of each wave's slot holding its partial tile.
constexpr int kDecodeOffs = kDecodeWaves * 4;
constexpr int kDecodeMaxRing = 5;    // the deepest ring (slabs per wave)

// Wait until at most N of this wave's memory loads are outstanding and all
// of its LDS reads are done (the ring slot about to be refilled was read by
// the previous slab's fragments).
template <int N>
__device__ __forceinline__ void wait_vm_lds()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}

// A buffer copy of 4 bytes per lane (b2l_16's form for dwords): lane l
// writes lds + l * 4.
__device__ __forceinline__ void b2l_4(rsrc_t src, uint32_t off, void *lds)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void *)lds, 4, off, 0, 0, 0);
}

// The 32-bit LDS address of a generic pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Slab geometry of the decode kernel for formats (FA, FB): the tile
// kernel's slabs (128 K-values, 256 when both operands are E2M1), 32 rows
// of A and 32 of B.  WA = 8, 16 or 32 is for an E4M3 / E5M2 A with an E2M1
// B and M <= WA (8-bit activations, 4-bit weights): 256-K slabs, so that
// each B row of a slab is one whole 128-byte line (with 128-K slabs it is
// half of one, and the line's other half is fetched again), A rows of 256
// bytes, and only WA A rows staged (2, 4 or 8 copy instructions).
// (Staging 8 A rows in the other geometries too, for a deeper ring,
// measured no faster on MI355X: at M = 8, N = 8192, K = 28672 the same time
// within 1 %, and up to 18 % slower for E2M1 with K <= 4096.)
//
// Scale bytes are staged once per 512-K period, beside the ring: a period's
// 16 bytes of each of the 32 A and 32 B rows (1 KB, four 4-byte copy
// instructions) in one of R period buffers, issued with the period's first
// slab.  They are read into registers when that slab is multiplied, and the
// buffer is refilled R periods later, which the ring's lead of S - 1 slabs
// must not reach: R * PS > S - 1, with PS slabs per period.
//
// The ring is at most 5 slabs deep: 6 slabs of the 6 KB geometries fit, but
// measured 4 % slower on MI355X with several column groups per workgroup
// (8 x 57344 x 8192, an 8-bit A with an E2M1 B).
template <int FA, int FB, int WA = 0>
struct decode_geo {
    static constexpr bool WIDE = WA != 0;
    using SL = slab<FA, FB>;
    static_assert(!WIDE || (FB == FP4 && FA != FP4), "the wide slabs pair an 8-bit A with an E2M1 B");
    static_assert(WA == 0 || WA == 8 || WA == 16 || WA == 32, "8, 16 or 32 staged A rows");
    static constexpr int KS = WIDE ? 256 : SL::kvals;          // K-values per slab
    static constexpr int PS = 512 / KS;                        // slabs per scale period
    static constexpr int RA = WIDE ? 256 : SL::template row_bytes<FA>;   // slab row bytes
    static constexpr int RB = WIDE ? 128 : SL::template row_bytes<FB>;
    static constexpr int MA = WIDE ? WA : kDecodeRows;        // rows of A staged
    static constexpr int SLOT = MA * RA + kDecodeRows * RB;   // LDS bytes per slab
    static constexpr int NCOPY = SLOT / 1024;                 // copies per slab
    static constexpr int NSC = 4;                             // scale copies per period
    static constexpr int SCP = 1024;                          // LDS bytes per period buffer
    static constexpr int bufs(int s) { return (s - 1) / PS + 1; }
    // loads a slab's wait leaves outstanding: the next S - 2 positions'
    // copies, the most scale copies among them
    static constexpr int lead(int s) { return (s - 2) * NCOPY + NSC * ((s - 3 + PS) / PS); }
    static constexpr int wave_lds(int s) { return s * SLOT + bufs(s) * SCP; }
    // ring depth: the most slabs (up to kDecodeMaxRing) that fit in the LDS,
    // with a wait count that fits the vmcnt field (at most 63)
    static constexpr int depth()
    {
        int s = 3;
        while (s < kDecodeMaxRing && kDecodeWaves * wave_lds(s + 1) + kDecodeOffs <= kDecodeLds &&
               lead(s + 1) <= 63)
            ++s;
        return s;
    }
    static constexpr int S = depth();
    static constexpr int R = bufs(S);
    static constexpr int WAVE_LDS = wave_lds(S);
    static constexpr int SMEM = kDecodeWaves * WAVE_LDS + kDecodeOffs;
    static_assert(SLOT >= kDecodeTileBytes, "a ring slot holds a partial tile");
};

// LDS swizzle of a slab row of R bytes: the tile kernel's for 128- and
// 64-byte rows; for 256-byte rows (16 chunks) chunk c of row r is stored at
// chunk c ^ (r mod 16), so 16 rows reading one chunk touch 16 distinct
// 16-byte bank groups.
template <int R> __device__ __forceinline__ int decode_swz(int r)
{
    return R == 256 ? (r & 15) : swz_row<R>(r);
}

template <int FA, int FB, int OUT, int WA>
__global__ void __launch_bounds__(kDecodeWaves * 64)
decode_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
              const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs, void *__restrict__ C,
              int M, int N, int K)
{
    using SL = slab<FA, FB>;
    using G = decode_geo<FA, FB, WA>;
    constexpr bool WIDE = G::WIDE;
    static_assert(SL::scaled && !is_fp6<FA>::value && !is_fp6<FB>::value,
                  "E2M1, E4M3 and E5M2 operands");
    constexpr int KS = G::KS;                        // K-values per slab: 128 or 256
    constexpr int HS = KS / 64;                      // 64-K MFMA steps per slab: 2 or 4
    constexpr int PS = G::PS;                        // slabs per scale period: 4 or 2
    constexpr int RA = G::RA, RB = G::RB, MA = G::MA;
    constexpr int RPCA = 1024 / RA, RPCB = 1024 / RB;             // rows per copy instruction
    constexpr int CPA = MA / RPCA, CPB = kDecodeRows / RPCB;      // copies per slab
    constexpr int NCOPY = G::NCOPY;
    static_assert(NCOPY == CPA + CPB, "copies per slab");
    constexpr int S = G::S, SLOT = G::SLOT, R = G::R;
    static_assert(S >= 3 && G::lead(S) <= 63, "ring depth and the vmcnt field");
    static_assert(R * PS > S - 1, "a period buffer outlives its period's slabs");
    static_assert(G::SMEM <= kDecodeLds, "LDS budget");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[G::SMEM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, g = lane >> 5;
    uint8_t *const ring = smem + wave * G::WAVE_LDS;
    uint8_t *const sring = ring + S * SLOT;          // the period buffers
    int *const tile_at = (int *)(smem + kDecodeWaves * G::WAVE_LDS);

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

    // Copy stream position (gj, k) -- slab position k of group gj -- into
    // ring slot `slot`.  Every position issues the same copies, also those
    // with no slab (then with num_records 0: nothing is fetched), so that
    // the count of loads in flight is the same on every path through the
    // loop.  When both operands are E2M1 and klen % 256 == 128 the last slab
    // is half a slab: its chunk offsets are clamped into the range (those
    // chunks are never read).
    auto issue = [&](int gj, int k, int slot) {
        uint8_t *const dst = ring + slot * SLOT;
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

    // Scale bytes of period q of group gj into period buffer `buf`: row r's
    // 16 bytes of the period (blocks kb/32 + 16q ..) at 16r, A rows first,
    // then B rows; lane l of copy i takes dword l % 4 of row 16i + l / 4.
    // Each dword is checked on its own against num_records, which ends at
    // the last real row: a short last period's dwords past the row are the
    // next row's bytes, or not fetched, and are never read.
    const uint32_t csoff = (uint32_t)(lane >> 2) * (uint32_t)sps + 4u * (uint32_t)(lane & 3);
    auto issue_scales = [&](int gj, int q, int buf) {
        uint8_t *const dst = sring + buf * G::SCP;
        const bool live = gj < ng;
        const int n0 = group_n0(min(gj, ng - 1));
        const int kbs = kb / 32 + 16 * q;
        const rsrc_t Ask = make_rsrc(As + kbs, live ? (uint32_t)(M * sps - kbs) : 0u);
        const rsrc_t Bsk = make_rsrc(Bs + (int64_t)n0 * sps + kbs,
                                     live ? (uint32_t)(min(kDecodeRows, N - n0) * sps - kbs) : 0u);
        b2l_4(Ask, csoff, dst);
        b2l_4(Ask, csoff + 16u * (uint32_t)sps, dst + 256);
        b2l_4(Bsk, csoff, dst + 512);
        b2l_4(Bsk, csoff + 16u * (uint32_t)sps, dst + 768);
    };

    // Operands of step p of a slab for lane row lr, from NR staged rows of R
    // bytes at `rows` (with NR = 8 or 16 A rows of the wide slabs, lane row
    // lr reads row lr % NR; only rows below M <= NR are stored): E4M3 / E5M2
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
    // A period's scale bytes from its buffer, A row lr % MA and B row lr:
    // step s of the period takes block 2s + g, byte 2(s % 2) + g of dword
    // s / 2; shifted right by 8g it is byte 2(s % 2), which the MFMA's op_sel
    // picks.  The two LDS reads are an asm block that waits for its own
    // results: the compiler cannot tell the bytes they read from the LDS that
    // the copies in flight are filling, and would wait for every one of those
    // copies first.
    auto scales = [&](const uint8_t *buf, v4i &sa, v4i &sb) {
        const uint32_t la = lds_addr(buf + 16 * (lr % MA)), lb = lds_addr(buf + 512 + 16 * lr);
        v4i x, y;
        asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(x), "=&v"(y) : "v"(la), "v"(lb) : "memory");
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            sa[d] = (int)((uint32_t)x[d] >> (8 * g));
            sb[d] = (int)((uint32_t)y[d] >> (8 * g));
        }
    };

    v16f acc;
    v4i sa, sb;
    // The stream: each group takes nper periods of PS slab positions;
    // positions past a group's slabs, and past its last group, copy nothing
    // and do no MFMA.  Its running position (uniform scalars, advanced by
    // one at a time rather than divided out of a flat index): the next
    // position to issue (group ig, position ik, ring slot islot, period
    // buffer ibuf) and the ring slot and period buffer being multiplied
    // (rslot, rbuf).
    const int ppg = nslab > 0 ? nper * PS : 0;
    int ig = 0, ik = 0, islot = 0, ibuf = 0, rslot = 0, rbuf = 0;
    // Issue the next position; `first` (a std::bool_constant) says whether it
    // starts a period and so also copies that period's scale bytes, which is
    // known at compile time: the loop below is unrolled by the PS positions
    // of a period.
    auto issue_next = [&](auto first) {
        issue(ig, ik, islot);
        if constexpr (decltype(first)::value) {
            issue_scales(ig, ik / PS, ibuf);
            if (++ibuf == R) ibuf = 0;
        }
        if (++ik == ppg) { ik = 0; ++ig; }
        if (++islot == S) islot = 0;
    };

    // Add the waves' partial tiles of group gi in wave order and store them.
    // Each wave keeps its tile in the ring slot of the last slab it
    // multiplied: the copies in flight fill the other S - 1 slots, and that
    // one is refilled only by the next issue, after the second barrier below.
    // In the MFMA result lane (c, g) holds, in element e, row
    // 8(e/4) + 4g + e%4 of column c; element e of lane l is kept at float
    // 64 e + l of the slot.  The barriers order LDS only: the stream's copies
    // into the rings stay in flight.
    auto add_and_store = [&](int gi) {
        const int n0 = group_n0(gi), rows_b = min(kDecodeRows, N - n0);
        const int at_slot = wave * G::WAVE_LDS + (rslot == 0 ? S - 1 : rslot - 1) * SLOT;
        float *const mine = (float *)(smem + at_slot);
#pragma unroll
        for (int e = 0; e < 16; ++e) mine[e * 64 + lane] = acc[e];
        if (lane == 0) tile_at[wave] = at_slot;
        lds_barrier();
        int from[kDecodeWaves];
#pragma unroll
        for (int w = 0; w < kDecodeWaves; ++w) from[w] = tile_at[w];
#pragma unroll
        for (int q = 0; q < kDecodeRows * kDecodeRows / (kDecodeWaves * 64); ++q) {
            const int m = q * 8 + (tid >> 5), c = tid & 31;
            if (m >= M || c >= rows_b) continue;
            const int at = (((m >> 3) * 4 + (m & 3)) * 64 + c + 32 * ((m >> 2) & 1)) * 4;
            float v = *(const float *)(smem + from[0] + at);
#pragma unroll
            for (int w = 1; w < kDecodeWaves; ++w) v += *(const float *)(smem + from[w] + at);
            if constexpr (OUT == OF32) ((float *)C)[(int64_t)m * N + n0 + c] = v;
            else ((uint16_t *)C)[(int64_t)m * N + n0 + c] = f32_to_bf16(v);
        }
        lds_barrier();
    };

#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    if (ppg > 0) {
        static_for<S - 1>([&](auto jc) {
            issue_next(std::bool_constant<decltype(jc)::value % PS == 0>{});
        });
        for (int gi = 0; gi < ng; ++gi) {
            for (int q = 0; q < nper; ++q) {
                static_for<PS>([&](auto kc) {
                    constexpr int kp = decltype(kc)::value;
                    // Slab q*PS + kp is in once at most the loads of the S - 2
                    // positions issued after it are outstanding: their slab
                    // copies and the scale copies of the periods among them
                    // that start (stores of C issued since only make the
                    // wait stricter).
                    wait_vm_lds<(S - 2) * NCOPY + G::NSC * ((kp + S - 2) / PS)>();
                    issue_next(std::bool_constant<(kp + S - 1) % PS == 0>{});
                    const uint8_t *const slot = ring + rslot * SLOT;
                    if (++rslot == S) rslot = 0;
                    if constexpr (kp == 0) {
                        scales(sring + rbuf * G::SCP, sa, sb);
                        if (++rbuf == R) rbuf = 0;
                    }
                    const int k = q * PS + kp;
                    if (k < nslab) {
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
            }
            add_and_store(gi);
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[e] = 0.f;
        }
    } else {                                         // an empty K-range: zero partial tiles
        for (int gi = 0; gi < ng; ++gi) add_and_store(gi);
    }
    wait_vm0();                                      // the copies past the last group
}

}  // namespace mx
