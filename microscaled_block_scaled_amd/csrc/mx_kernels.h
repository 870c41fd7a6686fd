// mx_kernels.h -- gfx950 device code for the MX block-scaled NT GEMM.
//
// C[m][n] = sum_b 2^(sA[m][b]+sB[n][b]-254) * sum_{j<32} A[m][32b+j]*B[n][32b+j]
// with FP32 accumulation (the MX scaled GEMM of the FlyDSL article: E8M0 scale
// per 32 K-values, FP32 accumulation, K a multiple of 128; digest 2026-10-22,
// item 1).  Every product block is computed by the CDNA4 block-scaled matrix
// instruction v_mfma_scale_f32_32x32x64_f8f6f4, which applies the two E8M0
// scales itself.
//
// Operand placement of that instruction on gfx950, as measured on the device
// with one-hot inputs (lane l, row r = l % 32, lane group g = l / 32):
//   * E2M1: lane (r, g) holds K-values 32g .. 32g+31 of the instruction's 64
//     as 16 bytes, element 2i in the low nibble of byte i;
//   * E4M3: lane (r, g) holds K-values 16g .. 16g+15 in bytes 0..15 and
//     32+16g .. 32+16g+15 in bytes 16..31;
//   * in both formats, lane (r, g) supplies the scale byte of the
//     instruction's K-block g (K-values 32g .. 32g+31) of row r, at the byte
//     op_sel selects;
//   * B uses the same placement with r the column index;
//   * the 32x32 FP32 result: lane (c, g) holds, in element e, row
//     8*(e/4) + 4g + e%4 of column c.
// (The 16x16x128 form, measured the same way, places E4M3 K-values 16g..+15
// and 64+16g..+15 in lane group g of four; it is not used here.)
// With a row's K-values staged as 16-byte chunks (chunk c = bytes 16c..16c+15
// of a 128-byte row segment), one instruction's K-step p of a segment reads:
//   * E4M3 (2 steps per segment): chunks 4p+g and 4p+2+g, scale block 2p+g;
//   * E2M1 (4 steps per segment): chunk 2p+g, scale block 2p+g.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

enum { FP4 = 1, FP8 = 2 };      // equal to MX_FMT_E2M1 / MX_FMT_E4M3
enum { OF32 = 1, OBF16 = 2 };   // equal to MX_OUT_FP32 / MX_OUT_BF16

// Format selector of the scaled MFMA (cbsz for A, blgp for B).
template <int FMT> struct mfma_fmt { static constexpr int sel = (FMT == FP4) ? 4 : 0; };

// A slab is SW = 128 bytes of every row of the A and B tiles: 256 E2M1 or
// 128 E4M3 K-values, i.e. four or two 64-K instruction steps, and their
// scale bytes (8 or 4 per row).  128-byte rows make every copy request a
// whole 128-byte line.
constexpr int SW = 128;
template <int FMT> struct slab {
    static constexpr int kvals = (FMT == FP4) ? 2 * SW : SW;
    static constexpr int steps = kvals / 64;         // 4 (E2M1) or 2 (E4M3)
    static constexpr int sbytes = kvals / 32;        // 8 (E2M1) or 4 (E4M3)
};

// FP32 -> BF16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// LDS row swizzle for 128-byte rows: chunk c of row r lives at chunk
// c ^ swz(r).  Any 8 aligned rows get 8 distinct values, and so do the even
// (or odd) rows of any 16 aligned rows, so a 16-byte read of one chunk by
// consecutive rows is free of bank conflicts whether the LDS serves 8 or 16
// lanes per cycle.  swz depends on r mod 16 only.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int FMT>
__device__ __forceinline__ v16f mma(const v8i &a, const v8i &b, v16f acc, int sa, int sb)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
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
// Wait until at most N of this wave's memory loads are outstanding (loads
// retire in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
// Workgroup barrier that orders LDS only: this wave's LDS reads complete,
// then all waves meet.  Unlike __syncthreads() it does not drain the wave's
// in-flight HBM -> LDS copies (their completion is awaited with wait_vm).
// The memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

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
// Instruction interleave: ask the scheduler for NMF MFMAs with the NDS LDS
// reads spread evenly between them (one scheduling region).  One wave per
// SIMD cannot hide LDS issue behind MFMAs if the reads come in one cluster.
template <int C>
__device__ __forceinline__ void ds_reads_group()
{
    if constexpr (C > 0) __builtin_amdgcn_sched_group_barrier(0x100, C, 0);
}
template <int NMF, int NDS, int... I>
__device__ __forceinline__ void interleave_impl(std::integer_sequence<int, I...>)
{
    ((__builtin_amdgcn_sched_group_barrier(0x008, 1, 0),
      ds_reads_group<(I + 1) * NDS / NMF - I * NDS / NMF>()), ...);
}
template <int NMF, int NDS>
__device__ __forceinline__ void interleave()
{
    interleave_impl<NMF, NDS>(std::make_integer_sequence<int, NMF>{});
}

// --------------------------------------------------------------------------
// Tiled kernel: one workgroup computes a BM x BN tile of C with WGM x WGN
// waves, each owning a (BM/WGM) x (BN/WGN) block of 32x32 FP32 accumulators.
//
// K is walked in slabs: 128 bytes of every A and B row.  The LDS holds a
// ring of S = 2 slabs and two scale buffers:
//   * slab k+S-1 is copied HBM -> LDS directly (global_load_lds, no register
//     staging) into the ring slot that slab k-1 has just vacated, so S-1
//     slabs of copies are in flight while slab k is multiplied -- the
//     consumed part of the LDS tile is refilled as soon as it is free;
//   * scale bytes travel 16 per row at a time (a "period": 16 K-blocks, i.e.
//     4 E4M3 or 2 E2M1 slabs), one period ahead, into the scale buffer the
//     period before last has vacated.  Row scales are K/32 bytes apart in
//     memory, so a per-slab copy would cost one memory request per row for
//     4-8 bytes; per period it is one request per row for 16;
//   * the operand fragments of step t+1 are read LDS -> registers (two
//     register sets) while the MFMAs of step t run, the reads spread between
//     the MFMAs;
//   * one barrier per slab, before its first fragment read; the wait before
//     it only drains this wave's copies of that slab, not the later ones.
// Rows are swizzled in LDS (chunk c of row r stored at chunk c ^ swz(r)); the
// swizzle is applied on the global side, since each lane's LDS slot is fixed
// by its lane id.  The main loop is one basic block (no data-dependent
// branches), so the compiler keeps the MFMAs where they are written.
template <int FMT, int OUT, int BM, int BN, int WGM, int WGN>
__global__ void __launch_bounds__(WGM * WGN * 64)
tile_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
            const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
            void *__restrict__ C, int M, int N, int K, int tiles_m, int tiles_n, int gm)
{
    constexpr int NW = WGM * WGN;
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int HS = slab<FMT>::steps;                   // MFMA steps per slab
    constexpr int SBS = slab<FMT>::sbytes;                 // scale bytes per row per slab
    constexpr int PS = 16 / SBS;                           // slabs per scale period
    constexpr int NR = (FMT == FP8) ? 2 : 1;               // 16-byte reads per fragment
    constexpr int ROWS = BM + BN;
    constexpr int DATA = ROWS * SW;                        // element bytes per slab
    constexpr int NSI = (ROWS + 63) / 64;                  // scale copy instructions
    constexpr int SBUF = NSI * 64 * 16;                    // one scale buffer
    constexpr int S = 2;                                   // ring depth
    constexpr int RPC = 1024 / SW;                         // rows per copy instruction
    static_assert(S * DATA + 2 * SBUF <= 163840, "LDS budget");
    static_assert(PS % S == 0 || S % PS == 0, "trip alignment");
    static_assert(BM % RPC == 0 && BN % RPC == 0, "rows per copy instruction");
    static_assert(FM * 32 == WTM && FN * 32 == WTN, "wave tile must be 32-aligned");
    constexpr int CPA = (BM / RPC + NW - 1) / NW;          // A copies per wave per slab
    constexpr int CPB = (BN / RPC + NW - 1) / NW;          // B copies per wave per slab
    constexpr int CPS = (NSI + NW - 1) / NW;               // scale copies per wave per period
    constexpr int NCOPY = CPA + CPB;
    static_assert(NCOPY * (S - 2) < 64, "vmcnt range");
    static_assert(S == 2 || S == 4, "ring depth");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[S * DATA + 2 * SBUF];
    uint8_t *const sbase = smem + S * DATA;                // scale buffers

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, gm, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int64_t rowb = (FMT == FP4) ? (int64_t)K / 2 : (int64_t)K;
    const int sp = K / 32;
    const int nslab = (int)((rowb + SW - 1) / SW);          // E2M1: the last may be half
    const int nper = (sp + 15) / 16;                       // scale periods
    const int nsteps = K / 64;

    const int crow = lane / (SW / 16), cpc = lane % (SW / 16);   // row in a copy, LDS chunk

    // Copy slab k into ring slot `slot`.  Branch-free: every wave issues the
    // same NCOPY instructions (a surplus one repeats the last row block,
    // writing the same bytes to the same place), and k is clamped to the
    // last slab (a repeat past the end lands in a slot nobody reads again).
    auto issue = [&](int k, int slot) {
        k = min(k, nslab - 1);
        uint8_t *base = smem + slot * DATA;
        const int64_t koff = (int64_t)k * SW;
#pragma unroll
        for (int u = 0; u < CPA; ++u) {
            const int i = min(wave + u * NW, BM / RPC - 1);
            const int r = i * RPC + crow;
            const int row = min(m0 + r, M - 1);
            // E2M1 with K % 256 == 128: the last slab is half a row segment;
            // its upper half is never read, so the copy stays inside the row.
            const int64_t off = min(koff + ((cpc ^ swz(r)) << 4), rowb - 16);
            g2l_16(A + (int64_t)row * rowb + off, base + i * 1024);
        }
#pragma unroll
        for (int u = 0; u < CPB; ++u) {
            const int i = min(wave + u * NW, BN / RPC - 1);
            const int r = i * RPC + crow;
            const int row = min(n0 + r, N - 1);
            const int64_t off = min(koff + ((cpc ^ swz(r)) << 4), rowb - 16);
            g2l_16(B + (int64_t)row * rowb + off, base + BM * SW + i * 1024);
        }
    };
    // Copy scale period p (16 bytes of every row) into scale buffer `buf`.
    // Needs rows of at least 16 scale bytes (K >= 512).  The last period of a
    // row may be short: its copy is shifted left to end at the row's end, and
    // readers shift their byte index to match.  Every byte read lies inside
    // its row.
    auto issue_scales = [&](int p, int buf) {
        p = min(p, nper - 1);
        const int soff = min(p * 16, sp - 16);
#pragma unroll
        for (int u = 0; u < CPS; ++u) {
            const int i = min(wave + u * NW, NSI - 1);
            const int r = min(i * 64 + lane, ROWS - 1);
            const uint8_t *src = (r < BM) ? As + (int64_t)min(m0 + r, M - 1) * sp
                                          : Bs + (int64_t)min(n0 + r - BM, N - 1) * sp;
            g2l_16(src + soff, sbase + buf * SBUF + i * 1024);
        }
    };

    const int lr = lane & 31, g = lane >> 5;
    // Per-lane LDS offsets.  A fragment row r = wm*WTM + 32i + lr has
    // swz(r) = swz(lr) (WTM and 32i are multiples of 16), so fragment i is the
    // lane's offset plus the constant 32*SW*i.
    const int swl = swz(lr);
    const int a_off = (wm * WTM + lr) * SW;
    const int b_off = BM * SW + (wn * WTN + lr) * SW;
    const int sa_off = (wm * WTM + lr) * 16;
    const int sb_off = (BM + wn * WTN + lr) * 16;

    // Operand registers: two sets (the step being multiplied, the next one).
    v8i fa[2][FM], fb[2][FN];
    int fsa[2][FM], fsb[2][FN];

    // Fragments of pass p of slab k (ring slot `slot`, scale buffer `sbuf`,
    // slab `kp` within its period) into register set `set`.  `shift` moves
    // the scale byte index when the period's copy was shifted (last period).
    // Every call sits in fully unrolled code, so set, slot, pass and kp fold
    // to constants and each data read is the lane's offset plus an immediate;
    // the scale buffer (the period's parity) and shift are runtime values.
    auto load = [&](int set, int slot, int p, int sbuf, int kp, int shift) {
        const uint8_t *base = smem + slot * DATA;
        const uint8_t *sc = sbase + sbuf * SBUF;
        // Step p of a slab: E4M3 chunks 4p+g and 4p+2+g, E2M1 chunk 2p+g;
        // in both, scale block 2p+g of the slab.
        const int c0 = (FMT == FP8) ? 4 * p + g : 2 * p + g;
        const int o0 = (c0 ^ swl) << 4, o1 = ((c0 + 2) ^ swl) << 4;
        const int sbyte = kp * SBS + 2 * p + g + shift;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const uint8_t *rp = base + a_off + i * 32 * SW;
            const v4i lo = *(const v4i *)(rp + o0);
            if (FMT == FP8) {
                const v4i hi = *(const v4i *)(rp + o1);
                fa[set][i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            } else {
                fa[set][i] = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
            }
            fsa[set][i] = sc[sa_off + i * 32 * 16 + sbyte];
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const uint8_t *rp = base + b_off + j * 32 * SW;
            const v4i lo = *(const v4i *)(rp + o0);
            if (FMT == FP8) {
                const v4i hi = *(const v4i *)(rp + o1);
                fb[set][j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            } else {
                fb[set][j] = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
            }
            fsb[set][j] = sc[sb_off + j * 32 * 16 + sbyte];
        }
    };

    v16f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    auto mfmas = [&](int set) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = mma<FMT>(fa[set][i], fb[set][j], acc[i][j], fsa[set][i], fsb[set][j]);
    };
    constexpr int NDS = (FM + FN) * (NR + 1);   // LDS reads per step (data + scale)

    // Before the first read of slab k1: wait for this wave's copies of it
    // (later slabs may stay in flight), sync (every wave holds the current
    // step's operands in registers, and slab k1-1 is fully read), refill the
    // slot slab k1-1 vacated with slab k1+S-1, and at a period start fetch
    // the next period's scales into the buffer the previous period vacated.
    auto open = [&](int k1, int slot_next, bool period_start, int pbuf_next) {
        wait_vm<NCOPY * (S - 2)>();
        lds_barrier();
        issue(k1 + S - 1, slot_next);
        if (period_start) issue_scales(k1 / PS + 1, pbuf_next);
    };
    // Rows shorter than one period (K < 512: a single period, and too few
    // steps for the main loop to run) get their scale bytes with ordinary
    // loads in the prologue, copied exactly; longer rows use period copies.
    const bool short_rows = sp < 16;
    auto open_guarded = [&](int k1, int slot_next, bool period_start, int pbuf_next) {
        wait_vm<NCOPY * (S - 2)>();
        lds_barrier();
        issue(k1 + S - 1, slot_next);
        if (period_start && !short_rows) issue_scales(k1 / PS + 1, pbuf_next);
    };
    // Scale byte shift for slabs of the last period when it was copied short.
    const int last_shift = short_rows ? 0 : nper * 16 - sp;
    auto shift_of = [&](int k) { return (k / PS == nper - 1) ? last_shift : 0; };

    // Prologue: scale period 0 (period 1 follows at slab 0's opening),
    // slabs 0..S-2 in flight, then open slab 0 and read step 0.
    if (short_rows) {
        for (int r = tid; r < ROWS; r += NW * 64) {
            const uint8_t *src = (r < BM) ? As + (int64_t)min(m0 + r, M - 1) * sp
                                          : Bs + (int64_t)min(n0 + r - BM, N - 1) * sp;
            for (int d = 0; d < sp; d += 4)
                *(uint32_t *)(sbase + r * 16 + d) = *(const uint32_t *)(src + d);
        }
    } else {
        issue_scales(0, 0);
    }
#pragma unroll
    for (int k = 0; k < S - 1; ++k) issue(k, k);
    wait_vm<NCOPY * (S - 2)>();      // scales of period 0 and slab 0 done
    lds_barrier();
    issue(S - 1, S - 1);
    if (!short_rows) issue_scales(1, 1);
    load(0, 0, 0, 0, 0, shift_of(0));

    // Main loop: one trip = TS slabs (a multiple of the ring depth and of
    // the scale period) = TS*HS steps, so register set, ring slot, pass and
    // scale slot of every step are constants after unrolling.  Step q of a
    // trip uses set q&1; step q+1 is in slab (q+1)/HS of the trip.  The loop
    // only runs when K spans more than one trip (K > 512), so its period
    // copies always have rows of at least 16 scale bytes.
    constexpr int TS = (PS > S) ? PS : S;      // k0 is a multiple of PS: kq % PS is global
    static_assert(TS % PS == 0 && TS % S == 0, "trip covers whole periods and rings");
    constexpr int TRIP = TS * HS;
    int t0 = 0;
    for (; t0 + TRIP < nsteps; t0 += TRIP) {
        const int k0 = t0 / HS;                       // first slab of the trip
#pragma unroll
        for (int q = 0; q < TRIP; ++q) {
            const int kq = (q + 1) / HS;              // slab of step q+1 within the trip
            const int per = (k0 + kq) / PS;           // its scale period
            if ((q + 1) % HS == 0)
                open(k0 + kq, (kq + S - 1) % S, kq % PS == 0, (per + 1) & 1);
            load((q + 1) & 1, kq % S, (q + 1) % HS, per & 1, kq % PS, shift_of(k0 + kq));
            mfmas(q & 1);
            interleave<FM * FN, NDS>();
        }
    }
    // Last trip: steps t0 .. nsteps-1 (1 to TRIP of them).
    {
        const int k0 = t0 / HS;
#pragma unroll
        for (int q = 0; q < TRIP; ++q) {
            if (t0 + q < nsteps) {
                const int kq = (q + 1) / HS;
                const int per = (k0 + kq) / PS;
                if (t0 + q + 1 < nsteps) {
                    if ((q + 1) % HS == 0)
                        open_guarded(k0 + kq, (kq + S - 1) % S, kq % PS == 0, (per + 1) & 1);
                    load((q + 1) & 1, kq % S, (q + 1) % HS, per & 1, kq % PS,
                         shift_of(k0 + kq));
                }
                mfmas(q & 1);
            }
        }
    }

    // No copy may still be writing this workgroup's LDS once its waves exit.
    wait_vm0();

    // Epilogue: lane (c, g) of fragment (i, j) holds, in element e, row
    // 8*(e/4) + 4g + e%4 of column c.
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * WTN + j * 32 + lr;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + wm * WTM + i * 32 + 8 * (e / 4) + 4 * g + (e % 4);
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
