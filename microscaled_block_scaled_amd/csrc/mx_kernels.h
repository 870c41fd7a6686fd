// mx_kernels.h -- gfx950 device code for the MX block-scaled NT GEMM (E2M1,
// E4M3, E5M2 and FP6 elements, one format per operand), the same tile kernel
// on dense BF16 operands, and the split-K reduction.
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
// Dense BF16 operands (no scales) use v_mfma_f32_32x32x16_bf16: lane (r, g)
// holds 8 K-values of row r, 16 bytes.  Which 8 of the 16 does not matter
// here: A and B fragments are read with the same lane-to-K map, and a dot
// product does not depend on the order of its terms.  The kernel hands
// lane group g the K-values 8g .. 8g+7.
// With a row's K-values staged as 16-byte chunks (chunk c = bytes 16c..16c+15
// of a 128-byte row segment), one instruction's K-step p of a segment reads:
//   * E4M3 (2 steps per segment): chunks 4p+g and 4p+2+g, scale block 2p+g;
//   * E2M1 (4 steps per segment): chunk 2p+g, scale block 2p+g;
//   * BF16 (4 steps of 16 K-values per segment): chunk 2p+g.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <numeric>
#include <type_traits>
#include <utility>


namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

enum { FP4 = 1, FP8 = 2, BF8 = 3 };   // equal to MX_FMT_E2M1 / MX_FMT_E4M3 / MX_FMT_E5M2
enum { B16 = 4 };                     // dense BF16 elements, no scales (B16 pairs with B16 only)
enum { F6E2 = 5, F6E3 = 6 };          // FP6 E2M3 / E3M2 (MX_FMT_E2M3 / MX_FMT_E3M2 on the host)
template <int F> struct is_fp6 { static constexpr bool value = F == F6E2 || F == F6E3; };
enum { OF32 = 1, OBF16 = 2 };   // equal to MX_OUT_FP32 / MX_OUT_BF16

// Format selector of the scaled MFMA (cbsz for A, blgp for B): 0 E4M3,
// 1 E5M2, 2 E2M3, 3 E3M2, 4 E2M1.  E4M3 and E5M2 share one byte-per-element
// layout.  FP6 operands, measured on the device like the others: lane
// (r, g) holds K-values 32g .. 32g+31 as a 192-bit string in its first six
// dwords, element i in bits 6i .. 6i+5.
template <int FMT> struct mfma_fmt {
    static constexpr int sel = (FMT == FP4) ? 4 : (FMT == BF8) ? 1 : (FMT == F6E2) ? 2
                             : (FMT == F6E3) ? 3 : 0;
};

// A slab is a run of K-values of every row of the A and B tiles: 256 when
// both operands are E2M1, 64 for BF16, else 128 -- four or two 64-K scaled
// instruction steps and their scale bytes (8 or 4 per row), or four 16-K
// BF16 steps.  An operand's slab row is 128 bytes (E4M3, E2M1 with E2M1, or
// BF16), which makes every copy request a whole 128-byte line, or 64 bytes
// (E2M1 beside E4M3, half a line).
constexpr int SW = 128;
template <int FA, int FB> struct slab {
    static_assert((FA == B16) == (FB == B16), "BF16 pairs with BF16 only");
    static constexpr bool scaled = FA != B16;
    static constexpr int kvals = (FA == B16) ? SW / 2 : (FA == FP4 && FB == FP4) ? 2 * SW : SW;
    static constexpr int kstep = scaled ? 64 : 16;   // K-values per MFMA
    static constexpr int steps = kvals / kstep;      // 4, 2 or 4
    static constexpr int sbytes = scaled ? kvals / 32 : 0;   // 8, 4 or none
    // bytes of one row of an operand of format F in a slab
    template <int F> static constexpr int row_bytes =
        (F == FP4) ? kvals / 2 : (F == B16) ? 2 * kvals : is_fp6<F>::value ? kvals / 4 * 3 : kvals;
};
// Bytes of k consecutive elements of format F.
template <int F> __device__ __forceinline__ int64_t kbytes(int64_t k)
{
    return (F == FP4) ? k / 2 : (F == B16) ? 2 * k : is_fp6<F>::value ? k / 4 * 3 : k;
}

// FP32 -> BF16 bits, round to nearest even (NaN stays NaN): one gfx950
// v_cvt_pk_bf16_f32, branch-free.
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// LDS row swizzle for 128-byte rows: chunk c of row r lives at chunk
// c ^ swz(r).  Any 8 aligned rows get 8 distinct values, and so do the even
// (or odd) rows of any 16 aligned rows, so a 16-byte read of one chunk by
// consecutive rows is free of bank conflicts whether the LDS serves 8 or 16
// lanes per cycle.  swz depends on r mod 16 only.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// The same for 64-byte rows (4 chunks): two rows share a 128-byte bank
// window, and the rows of one parity among 8 aligned rows, or of one residue
// mod 4 among 16, get 4 distinct values, so 8 or 16 consecutive rows reading
// one chunk again touch distinct banks.  Depends on r mod 16 only.
__device__ __forceinline__ int swz64(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
// FP6 slab rows (96 bytes) are not swizzled.
template <int RB> __device__ __forceinline__ int swz_row(int r)
{
    return RB == 128 ? swz(r) : RB == 64 ? swz64(r) : 0;
}
// Rows per copy instruction for slab rows of RB bytes: 1024 / RB for 128-
// and 64-byte rows (64 lanes x 16 bytes); 8 for 96-byte FP6 rows, copied by
// lanes 0..47 (6 chunks per row).  An FP6 group of 8 rows takes a 1040-byte
// LDS block: the rows, 96 bytes apart, then padding into which lanes 48..63
// copy duplicate chunks, so the copies need no branch (the K loop stays one
// basic block).  The 16 bytes beyond 1024 shift each group's rows by 16
// bytes of bank offset against the previous group's, so two groups read by
// the same 16 lanes use different banks (8 rows of one group, 96 bytes
// apart, already do).  An FP6 row takes 130 LDS bytes on average.
template <int RB> struct copy_rows { static constexpr int value = RB == 96 ? 8 : 1024 / RB; };
template <int RB> struct lds_pitch { static constexpr int value = RB == 96 ? 130 : RB; };
// LDS offset of row r of an operand tile with slab rows of RB bytes.
template <int RB> __device__ __forceinline__ int lds_row(int r)
{
    return RB == 96 ? (r >> 3) * 1040 + (r & 7) * 96 : r * RB;
}

// The scale operands are 32-bit registers holding four E8M0 bytes; op_sel
// OPS picks byte OPS of each (measured on the device: op_sel i applies byte i,
// for A and for B alike).
template <int FA, int FB, int OPS>
__device__ __forceinline__ v16f mma(const v8i &a, const v8i &b, v16f acc, int sa, int sb)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        a, b, acc, mfma_fmt<FA>::sel, mfma_fmt<FB>::sel, OPS, sa, OPS, sb);
}
// Dense BF16: 16 bytes (8 values) per lane and operand, no scales.
template <int FA, int FB, int OPS>
__device__ __forceinline__ v16f mma(const v4i &a, const v4i &b, v16f acc, int, int)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a),
                                                  __builtin_bit_cast(v8bf, b), acc, 0, 0, 0);
}

// An FP6 operand fragment: the 24 bytes (32 elements) read from LDS as three
// 8-byte words go to the first six dwords of the MFMA operand.
template <typename V>
__device__ __forceinline__ void fp6_frag(V &v, uint2 q0, uint2 q1, uint2 q2)
{
    if constexpr (sizeof(V) == 32)
        v = V{(int)q0.x, (int)q0.y, (int)q1.x, (int)q1.y, (int)q2.x, (int)q2.y, 0, 0};
}

// Direct HBM -> LDS copies: buffer_load_dwordx4 with the lds bit (the gfx950
// form moves 16 bytes per lane).  Lane l of the wave writes its 16 bytes to
// lds + l * 16; `lds` must be wave-uniform.  The source is a buffer resource
// (wave-uniform 64-bit base) plus a 32-bit per-lane byte offset.  The buffer
// form, rather than global_load_lds, matters for scheduling: the compiler
// counts a global (FLAT-encoded) LDS copy as both a memory and an LDS access
// and then waits for every outstanding LDS read (lgkmcnt(0)) before any use
// of one, while with buffer copies in flight it waits only for the read it
// needs.  The descriptor's num_records bounds the offsets: a copy at or past
// it is not fetched (the hardware's range check returns zeros), which is how
// the rows of a partial tile beyond the matrix's last row cost no memory
// traffic (their results are never stored).  num_records -1 checks nothing.
// AUX is the cache policy: 0 the default, kStream the nontemporal hint for
// data read once (measured: it raises a plain streaming read over 1 GiB from
// 6.1 to 6.9 TB/s on MI355X).
typedef __attribute__((address_space(3))) void lds_void;
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// Word 3 of a gfx9 buffer descriptor: 32-bit data format, no swizzle.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kStream = 2;   // the nt bit of the cache-policy operand

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t num_records)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)num_records,
                                             kRsrcWord3);
}
template <int AUX = 0>
__device__ __forceinline__ void b2l_16(rsrc_t src, uint32_t off, void *lds)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void *)lds, 16, off, 0, 0, AUX);
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

// Workgroups are dispatched round-robin over the 8 XCDs: workgroup b runs on
// XCD b % 8.  xcd_run(b, T) numbers T workgroups so that each XCD gets a
// contiguous run of indices: XCD x holds T/8 of them, one more if x < T % 8,
// starting after the runs of XCDs 0 .. x-1.
__device__ __forceinline__ int xcd_run(int b, int T)
{
    const int q = T >> 3, r = T & 7, x = b & 7;
    return x * q + min(x, r) + (b >> 3);
}

// Tile order: give each XCD a contiguous run of tiles (when the tile count is
// a multiple of 8; `remap` false when the caller has already ordered the
// grid), walked in groups of `gm` M-tiles, so the workgroups sharing an
// XCD's L2 also share A and B panels.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int gm,
                                        int &tm, int &tn, bool remap = true)
{
    const int ntiles = tiles_m * tiles_n;
    int t = bid;
    if (remap && (ntiles & 7) == 0) t = xcd_run(bid, ntiles);
    const int per_group = gm * tiles_n;
    const int grp = t / per_group, first_m = grp * gm;
    const int gsz = min(tiles_m - first_m, gm);
    const int w = t - grp * per_group;
    tm = first_m + w % gsz;
    tn = w / gsz;
}

// Grouped GEMM (one weight matrix per group, as in a mixture-of-experts
// layer): group g owns rows row_start[g] .. row_start[g+1]-1 of A and C,
// weight g of B (N rows each) and tiles tile_start[g] .. tile_start[g+1]-1 of
// the grid.  Passed by value in the kernel arguments.  NoGroups marks a
// plain GEMM.
constexpr int kMaxGroups = 256;
struct GroupTable {
    static constexpr bool grouped = true;
    int n;
    int tile_start[kMaxGroups + 1];
    int row_start[kMaxGroups + 1];
};
struct NoGroups {
    static constexpr bool grouped = false;
};

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// --------------------------------------------------------------------------
// Tiled kernel: one workgroup computes a BM x BN tile of C with WGM x WGN
// waves, each owning a (BM/WGM) x (BN/WGN) block of 32x32 FP32 accumulators.
//
// A's elements are in format FA and B's in FB (equal, or one E4M3 and one
// E2M1).  K is walked in slabs of 128 or 256 K-values of every A and B row
// (see slab<>).  The LDS holds a ring of S slabs (2 or 3, as the tile's LDS footprint allows) and two scale
// buffers:
//   * slab k+S-1 is copied HBM -> LDS directly (buffer loads into LDS, no register
//     staging) into the ring slot that slab k-1 has just vacated, so S-1
//     slabs of copies are in flight while slab k is multiplied -- the
//     consumed part of the LDS tile is refilled as soon as it is free;
//   * scale bytes travel 16 per row at a time (a "period": 16 K-blocks, i.e.
//     4 E4M3 or 2 E2M1 slabs), one period ahead, into the scale buffer the
//     period before last has vacated.  Row scales are K/32 bytes apart in
//     memory, so a per-slab copy would cost one memory request per row for
//     4-8 bytes; per period it is one request per row for 16.  A period's
//     scales are issued at the opening of the previous period's first slab,
//     before that opening's slab copies; with S-1 <= slabs per period, every
//     slab of the period is issued after them, so the in-order wait for a
//     slab's copies also covers its scales;
//   * the operand fragments of step t+1 are read LDS -> registers (two
//     register sets) while the MFMAs of step t run, the reads spread between
//     the MFMAs;
//   * one barrier per slab, before its first fragment read; the wait before
//     it only drains this wave's copies of that slab, not the later ones.
// Rows are swizzled in LDS (chunk c of row r stored at chunk c ^ swz(r)); the
// swizzle is applied on the global side, since each lane's LDS slot is fixed
// by its lane id.  The main loop is one basic block (no data-dependent
// branches), so the compiler keeps the MFMAs where they are written.
template <int FA, int FB, int OUT, int BM, int BN, int WGM, int WGN, int S, typename GT = NoGroups>
__global__ void __launch_bounds__(WGM * WGN * 64)
tile_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
            const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
            void *__restrict__ C, int M, int N, int K, int tiles_m, int tiles_n, int gm,
            int kchunk, int64_t cplane, GT groups = GT{})
{
    constexpr int NW = WGM * WGN;
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    using SL = slab<FA, FB>;
    constexpr int KS = SL::kvals;                          // K-values per slab
    constexpr int HS = SL::steps;                          // MFMA steps per slab
    constexpr bool SCALED = SL::scaled;                    // MX formats (BF16 has no scales)
    constexpr int SBS = SL::sbytes;                        // scale bytes per row per slab
    constexpr int PS = SCALED ? 16 / SBS : S;              // slabs per scale period
    constexpr int RA = SL::template row_bytes<FA>;         // slab row bytes, A and B
    constexpr int RB = SL::template row_bytes<FB>;
    constexpr int ROWS = BM + BN;
    constexpr int LA = lds_pitch<RA>::value, LB = lds_pitch<RB>::value;   // LDS bytes per row
    constexpr int DATA = BM * LA + BN * LB;                // LDS bytes per slab
    constexpr int NSI = SCALED ? (ROWS + 63) / 64 : 0;     // scale copy instructions
    constexpr int SBUF = NSI * 64 * 16;                    // one scale buffer
    constexpr int RPCA = copy_rows<RA>::value, RPCB = copy_rows<RB>::value;   // rows per copy instruction
    static_assert(S >= 2 && S - 1 <= PS, "one period of scale lookahead covers the ring");
    static_assert(BM % RPCA == 0 && BN % RPCB == 0, "rows per copy instruction");
    static_assert(FM * 32 == WTM && FN * 32 == WTN, "wave tile must be 32-aligned");
    constexpr int CPA = (BM / RPCA + NW - 1) / NW;         // A copies per wave per slab
    constexpr int CPB = (BN / RPCB + NW - 1) / NW;         // B copies per wave per slab
    constexpr int CPS = SCALED ? (NSI + NW - 1) / NW : 0;  // scale copies per wave per period
    constexpr int NCOPY = CPA + CPB;
    // The epilogue reuses the LDS to stage output bands (see below).
    typedef typename std::conditional<OUT == OF32, float, uint16_t>::type otype;
    constexpr int OS = sizeof(otype);
    constexpr int PITCH = WTN * OS + 16;                   // staging row pitch, bytes
    // (+16: a half-period read of the last row of a short, shifted last
    // period may run up to 12 bytes past its buffer; those bytes belong to
    // steps that do not exist)
    constexpr int RING = S * DATA + 2 * SBUF + 16;
    constexpr int SMEM = RING > NW * 32 * PITCH ? RING : NW * 32 * PITCH;
    static_assert(SMEM <= 163840, "LDS budget");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];
    uint8_t *const sbase = smem + S * DATA;                // scale buffers

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    // Split-K: workgroup b computes K-slice b / (tiles_m*tiles_n), K-values
    // [kb, kb + klen) with kb a multiple of kchunk (itself a multiple of 512,
    // i.e. of whole scale periods), into the FP32 plane C + slice*cplane.
    // Without split-K, kchunk == K and there is one slice.
    int bid = blockIdx.x;
    if constexpr (GT::grouped) {
        // The whole grid (every group's tiles) is ordered per XCD first, so
        // consecutive tiles of a group, which share its weight panels, run
        // on one XCD whatever the group sizes.
        bid = xcd_run(bid, groups.tile_start[groups.n]);
        // This workgroup's group: the last g with tile_start[g] <= bid (an
        // empty group shares its start with the next one, so g is never
        // empty).  Then rebase every operand on the group and make the rest
        // of the kernel see one plain GEMM of M_g rows.
        int lo = 0, hi = groups.n - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) / 2;
            if (groups.tile_start[mid] <= bid) lo = mid; else hi = mid - 1;
        }
        const int r0 = groups.row_start[lo];
        const int64_t rba = kbytes<FA>(K), rbb = kbytes<FB>(K);
        M = groups.row_start[lo + 1] - r0;
        tiles_m = (M + BM - 1) / BM;
        bid -= groups.tile_start[lo];
        A += (int64_t)r0 * rba;
        B += (int64_t)lo * N * rbb;
        if constexpr (SL::scaled) {
            As += (int64_t)r0 * (K / 32);
            Bs += (int64_t)lo * N * (K / 32);
        }
        C = (uint8_t *)C + (int64_t)r0 * N * (OUT == OF32 ? 4 : 2);
    }
    const int ntiles = tiles_m * tiles_n;
    const int slice = bid / ntiles;
    int tm, tn;
    tile_of(bid - slice * ntiles, tiles_m, tiles_n, gm, tm, tn, !GT::grouped);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kb = slice * kchunk, klen = min(kchunk, K - kb);
    // Row stride, slice bytes per row and slice offset of each operand.
    const int64_t rowba = kbytes<FA>(K), rowbb = kbytes<FB>(K);
    const int64_t rowla = kbytes<FA>(klen), rowlb = kbytes<FB>(klen);
    const int64_t kboffa = kbytes<FA>(kb), kboffb = kbytes<FB>(kb);
    const int sps = K / 32, sp = klen / 32;                  // scale row stride, slice extent
    const int nslab = (klen + KS - 1) / KS;                  // E2M1 x E2M1: the last may be half
    const int nper = (sp + 15) / 16;                       // scale periods
    const int nsteps = klen / SL::kstep;

    // Copy addresses are a wave-uniform base (scalar registers) plus a 32-bit
    // per-lane offset, which stays below 256 rows * rowb <= 2^32 for K <= 2^24.
    // In a tile that runs past the matrix's last row, the copies of the rows
    // beyond it fall outside their descriptor's num_records and are not
    // fetched (their results are never stored).
    static_assert(BM % 64 == 0, "copy geometry");
    const uint8_t *const At = A + (int64_t)m0 * rowba + kboffa;
    const uint8_t *const Bt = B + (int64_t)n0 * rowbb + kboffb;
    const uint8_t *const Ast = As + (int64_t)m0 * sps + kb / 32;
    const uint8_t *const Bst = Bs + (int64_t)n0 * sps + kb / 32;
    const int last_a = min(BM, M - m0) - 1, last_b = min(BN, N - n0) - 1;   // last row in the tile
    // num_records of the copies: a partial tile's rows counted from the
    // slice's first byte (below 2^32: at most 255 rows), less the slab's
    // offset in issue(); whole tiles are not range-checked.  (Computed once
    // here: forming the 64-bit product per slab raised the mixed-format
    // kernels from 192 VGPRs to 256 and spills.)
    const bool whole_a = last_a + 1 == BM, whole_b = last_b + 1 == BN;
    const uint32_t ext_a = whole_a ? 0xffffffffu : (uint32_t)((last_a + 1) * rowba - kboffa);
    const uint32_t ext_b = whole_b ? 0xffffffffu : (uint32_t)((last_b + 1) * rowbb - kboffb);
    // B is streamed once per tile when every tile column has a single row
    // tile (the short tiles serve M <= their height): it takes the
    // nontemporal hint there.
    constexpr int AUXB = BM <= 128 ? kStream : 0;
    // Per operand (slab row bytes R, rows per copy instruction 1024/R): lane
    // l copies chunk l % (R/16) of row l / (R/16) of a block of rows, into
    // LDS chunk cpc of that row, which holds global chunk cpc ^ swz(row).
    // For 128-byte rows swz(i*8 + crow) depends only on crow and i's parity
    // (ch0 / ch1); for 64-byte rows swz64(i*16 + crow) only on crow.
    struct CopyGeo { int crow; uint32_t lane_row, ch0, ch1, rowb32; };
    auto copy_geo = [&](auto rc, int64_t rowb) {
        constexpr int R = decltype(rc)::value;
        const int crow = lane / (R / 16), cpc = lane % (R / 16);
        const uint32_t rb32 = (uint32_t)rowb;
        return CopyGeo{crow, (uint32_t)crow * rb32,
                       (uint32_t)(cpc ^ swz_row<R>(crow)) << 4,
                       (uint32_t)(cpc ^ swz_row<R>(crow + copy_rows<R>::value)) << 4, rb32};
    };
    const CopyGeo ga = copy_geo(std::integral_constant<int, RA>{}, rowba);
    const CopyGeo gb = copy_geo(std::integral_constant<int, RB>{}, rowbb);
    // Byte offset of this lane's row in the block of rows starting at r0.
    // FP6 lanes 48..63 name rows 8..10 of their 8-row block (their chunks
    // land in padding nobody reads): in a tile's last block those rows lie
    // past the tile, so every row is clamped to the tile's last one
    // (`rows` - 1), which is inside the matrix when the tile is whole and
    // past num_records (not fetched) when it is not.
    auto row_off = [&](const CopyGeo &c, int r0, int rows) -> uint32_t {
        return (r0 + c.crow < rows) ? (uint32_t)r0 * c.rowb32 + c.lane_row
                                    : (uint32_t)(rows - 1) * c.rowb32;
    };

    // Copy slab k into ring slot `slot`.  Branch-free: every wave issues the
    // same NCOPY instructions (a surplus one repeats the last row block,
    // writing the same bytes to the same place), and k is clamped to the
    // last slab (a repeat past the end lands in a slot nobody reads again).
    auto issue = [&](int k, int slot) {
        k = min(k, nslab - 1);
        uint8_t *base = smem + slot * DATA;
        const int64_t koffa = (int64_t)k * RA, koffb = (int64_t)k * RB;
        // E2M1 x E2M1 with K % 256 == 128: the last slab is half a row
        // segment; its upper half is never read, and its chunks are clamped
        // into the row.  (With 64-byte slab rows every slab is whole.)
        const uint32_t cmaxa = (uint32_t)(rowla - 16 - koffa);
        const uint32_t cmaxb = (uint32_t)(rowlb - 16 - koffb);
        const rsrc_t Ak = make_rsrc(At + koffa, whole_a ? ext_a : ext_a - (uint32_t)koffa);
        const rsrc_t Bk = make_rsrc(Bt + koffb, whole_b ? ext_b : ext_b - (uint32_t)koffb);
#pragma unroll
        for (int u = 0; u < CPA; ++u) {
            const int i = min(wave + u * NW, BM / RPCA - 1);
            const uint32_t ch = min((RA == 128 && (i & 1)) ? ga.ch1 : ga.ch0, cmaxa);
            b2l_16(Ak, row_off(ga, i * RPCA, BM) + ch, base + i * RPCA * LA);
        }
#pragma unroll
        for (int u = 0; u < CPB; ++u) {
            const int i = min(wave + u * NW, BN / RPCB - 1);
            const uint32_t ch = min((RB == 128 && (i & 1)) ? gb.ch1 : gb.ch0, cmaxb);
            b2l_16<AUXB>(Bk, row_off(gb, i * RPCB, BN) + ch, base + BM * LA + i * RPCB * LB);
        }
    };
    // Copy scale period p (16 bytes of every row) into scale buffer `buf`;
    // lane l of copy instruction i fetches row 64i + l of the A rows then the
    // B rows (BM is a multiple of 64, so each instruction is all A or all B).
    // Needs rows of at least 16 scale bytes (K >= 512).  The last period of a
    // row may be short: its copy is shifted left to end at the row's end, and
    // readers shift their byte index to match.  Every byte read lies inside
    // its row.
    auto issue_scales = [&](int p, int buf) {
        if constexpr (!SCALED) return;
        p = min(p, nper - 1);
        const int soff = min(p * 16, sp - 16);
#pragma unroll
        for (int u = 0; u < CPS; ++u) {
            const int i = min(wave + u * NW, NSI - 1);
            const bool in_a = i * 64 < BM;
            const int row = i * 64 + lane - (in_a ? 0 : BM);
            // (exact extents even for whole tiles: the last instruction's B
            // rows may run past BN)
            const int last = in_a ? last_a : last_b;
            const rsrc_t src = make_rsrc((in_a ? Ast : Bst) + soff,
                                         (uint32_t)((last + 1) * sps - kb / 32 - soff));
            b2l_16(src, (uint32_t)row * (uint32_t)sps, sbase + buf * SBUF + i * 1024);
        }
    };

    const int lr = lane & 31, g = lane >> 5;
    // Per-lane LDS offsets.  A fragment row r = wm*WTM + 32i + lr has
    // swz(r) = swz(lr) (WTM and 32i are multiples of 16), so fragment i is the
    // lane's offset plus the constant 32*R*i.
    const int swla = swz_row<RA>(lr), swlb = swz_row<RB>(lr);
    const int a_off = wm * WTM * LA + lds_row<RA>(lr);
    const int b_off = BM * LA + wn * WTN * LB + lds_row<RB>(lr);
    const int sa_off = (wm * WTM + lr) * 16;
    const int sb_off = (BM + wn * WTN + lr) * 16;

    // Operand registers.  The operand with more fragments per wave (the
    // "rolled" one, R) has a single register set: each of its fragments is
    // reloaded for the next step as soon as the last MFMA of this step that
    // reads it has been issued.  The other operand (D) has two sets, the next
    // step's read while this step's are multiplied.  This keeps 2 waves per
    // SIMD within 256 registers.
    constexpr bool ROLL_A = FM >= FN;
    constexpr int FR = ROLL_A ? FM : FN, FD = ROLL_A ? FN : FM;
    const int r_off = ROLL_A ? a_off : b_off, d_off = ROLL_A ? b_off : a_off;
    const int rs_off = ROLL_A ? sa_off : sb_off, ds_off = ROLL_A ? sb_off : sa_off;
    // Fragment registers: 8 dwords for the scaled MFMA (E2M1 uses the low
    // 4), 4 for BF16.  When both operands are E2M1 (4-dword fragments) the
    // rolled operand is double-buffered too (R2): then every fragment of the
    // next step is read right after the step's first MFMAs, a whole step
    // ahead of its use, and the burst of reads that all waves issue at once
    // has a step to drain through the LDS.
    constexpr bool R2 = FA == FP4 && FB == FP4;
    typedef typename std::conditional<SCALED, v8i, v4i>::type fv;
    fv fr[R2 ? 2 : 1][FR], fd[2][FD];
    // Scale registers (unused for BF16).  A period's 8 steps fall in two
    // halves of 4; for each half a fragment's lane holds the 4 scale bytes of
    // its steps in one register, byte i for the half's step i, applied by
    // the MFMA's op_sel.  The rolled operand reloads its register with the
    // fragment that opens a half; the D operand keeps one register per half
    // parity, since its next half is read while the current one is in use.
    int fsr[R2 ? 2 : 1][FR] = {}, fsd[2][FD] = {};

    // Where one step's operands are: ring slot `slot`, pass p of the slab,
    // scale buffer `sbuf`, slab `kp` within its scale period, and the scale
    // byte shift of a short last period.  Data chunk offsets (per operand)
    // are per lane (they depend on the lane group g and the swizzle); the
    // scale offset is that of the step's half-period.
    struct Src { int data, scale, a0, a1, b0, b1; };
    auto chunk_offs = [&](auto fc, int p, int swl, int &o0, int &o1) {
        // Step p of a slab: E4M3 / E5M2 chunks 4p+g and 4p+2+g of a 128-byte
        // row, E2M1 chunk 2p+g (of a 128- or a 64-byte row), BF16 chunk 2p+g;
        // FP6: 24 bytes at byte 48p+24g of a 96-byte row.
        constexpr int F = decltype(fc)::value;
        if constexpr (is_fp6<F>::value) {
            o0 = 48 * p + 24 * g;
            o1 = 0;
            return;
        }
        const int c0 = (F == FP4 || F == B16) ? 2 * p + g : 4 * p + g;
        o0 = (c0 ^ swl) << 4;
        o1 = ((c0 + 2) ^ swl) << 4;
    };
    auto src_of = [&](int slot, int p, int sbuf, int kp, int shift) {
        Src r;
        r.data = slot * DATA;
        // Step j = kp*HS + p of the period (0..7) reads scale block 2j + g,
        // byte shift + 2j + g of its row in the buffer (the shift, a multiple
        // of 4, only in a short last period).  Its half j/4 starts at byte
        // shift + 8*(j/4), a 4-byte boundary.
        r.scale = S * DATA + sbuf * SBUF + shift + 8 * ((kp * HS + p) >> 2);
        chunk_offs(std::integral_constant<int, FA>{}, p, swla, r.a0, r.a1);
        chunk_offs(std::integral_constant<int, FB>{}, p, swlb, r.b0, r.b1);
        return r;
    };
    auto sel = [](bool c, const Src &x, const Src &y) {
        return Src{c ? x.data : y.data, c ? x.scale : y.scale, c ? x.a0 : y.a0,
                   c ? x.a1 : y.a1, c ? x.b0 : y.b0, c ? x.b1 : y.b1};
    };
    // Fragment f of operand A (ia true) or B, whose lane rows start at LDS
    // offset `off`: 16 (E2M1), 24 (FP6) or 32 (E4M3) bytes.
    auto frag = [&](auto ia, const Src &s, int off, int f, fv &v) {
        constexpr bool IA = decltype(ia)::value;
        constexpr int F = IA ? FA : FB, L = IA ? LA : LB;     // 32 rows take 32 * L LDS bytes
        const uint8_t *rp = smem + s.data + off + f * 32 * L;
        if constexpr (is_fp6<F>::value) {
            // three 8-byte reads (the 24 bytes are 8-byte aligned)
            const uint8_t *q = rp + (IA ? s.a0 : s.b0);
            fp6_frag(v, *(const uint2 *)q, *(const uint2 *)(q + 8), *(const uint2 *)(q + 16));
            return;
        }
        const v4i lo = *(const v4i *)(rp + (IA ? s.a0 : s.b0));
        if constexpr (!SCALED) {
            v = lo;
        } else if constexpr (F != FP4) {
            const v4i hi = *(const v4i *)(rp + (IA ? s.a1 : s.b1));
            v = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
            v = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
        }
    };
    // The scale register of fragment f (scale rows at LDS offset `soff`) for
    // the half-period at s.scale: the row's 8 bytes there (two 4-byte reads,
    // merged into one ds_read2_b32) hold blocks 2i + g' of steps i = 0..3 for
    // both lane groups g'; one v_perm_b32 keeps this lane group's four, in
    // step order.
    const uint32_t psel = g ? 0x07050301u : 0x06040200u;
    auto frag_scale = [&](const Src &s, int soff, int f, int &sv) {
        if constexpr (SCALED) {
            const uint8_t *q = smem + s.scale + soff + f * 32 * 16;
            const uint32_t w0 = *(const uint32_t *)q, w1 = *(const uint32_t *)(q + 4);
            sv = (int)__builtin_amdgcn_perm(w1, w0, psel);
        }
    };
    const std::integral_constant<bool, ROLL_A> is_r{};       // the rolled operand is A?
    const std::integral_constant<bool, !ROLL_A> is_d{};
    auto load_all = [&](const Src &s) {
#pragma unroll
        for (int f = 0; f < FR; ++f) {
            frag(is_r, s, r_off, f, fr[0][f]);
            frag_scale(s, rs_off, f, fsr[0][f]);
        }
#pragma unroll
        for (int f = 0; f < FD; ++f) {
            frag(is_d, s, d_off, f, fd[0][f]);
            frag_scale(s, ds_off, f, fsd[0][f]);
        }
    };

    v16f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // Multiply one step (operands fr and fd[cur]) and read the next step's
    // operands from `nx`: rolled fragment o right after its FD MFMAs, and
    // the D fragments spread over the first half of the groups.  The first
    // MFMAs of the next step then read registers loaded at least half a step
    // earlier, so the LDS latency stays hidden even when the wave runs alone
    // on its SIMD (its partner parked at the slab barrier).  (All D reads in
    // the first group would spill on the 256x256 E4M3 tile.)  The scheduling
    // groups keep each rolled reload behind the MFMAs that read the old
    // value.
    // Step q (a compile-time index: the steps of a trip are unrolled, and a
    // trip starts at a period start, so q % 8 is the step within its period)
    // multiplies with register set q & 1 and scale byte q % 4 of the
    // half-period q / 4; the next step opens a half when (q + 1) % 4 == 0,
    // and then its fragments bring their scale registers along.
    constexpr int DH = R2 ? 1 : (FR + 1) / 2;              // groups that read D
    auto step = [&](auto qc, const Src &nx) {
        constexpr int q = decltype(qc)::value;
        constexpr int cur = q & 1, OPS = SCALED ? q % 4 : 0;
        constexpr bool NEWHALF = SCALED && (q + 1) % 4 == 0;
        constexpr int hc = (q / 4) & 1, hn = ((q + 1) / 4) & 1;   // half parities
        constexpr int rc = R2 ? cur : 0, rn = R2 ? cur ^ 1 : 0;   // rolled register sets
        constexpr int sc = R2 ? hc : 0, sn = R2 ? hn : 0;         // rolled scale sets
        static_for<FR>([&](auto oc) {
            constexpr int o = decltype(oc)::value;
            constexpr int d0 = o < DH ? o * FD / DH : FD, d1 = o < DH ? (o + 1) * FD / DH : FD;
            // rolled fragments read after this group: fragment o (R2: all of
            // them after the first group)
            constexpr int r0 = R2 ? (o == 0 ? 0 : FR) : o, r1 = R2 ? (o == 0 ? FR : FR) : o + 1;
            // LDS reads per fragment: data (2 for E4M3 / E5M2, 3 for FP6, 1
            // for E2M1 and BF16), + 1 for a scale register
            constexpr int FRF = ROLL_A ? FA : FB, FDF = ROLL_A ? FB : FA;
            constexpr int NRR = (is_fp6<FRF>::value ? 3 : (FRF == FP4 || FRF == B16) ? 1 : 2) + NEWHALF;
            constexpr int NRD = (is_fp6<FDF>::value ? 3 : (FDF == FP4 || FDF == B16) ? 1 : 2) + NEWHALF;
#pragma unroll
            for (int d = 0; d < FD; ++d) {
                if constexpr (ROLL_A)
                    acc[o][d] = mma<FA, FB, OPS>(fr[rc][o], fd[cur][d], acc[o][d], fsr[sc][o],
                                                 fsd[hc][d]);
                else
                    acc[d][o] = mma<FA, FB, OPS>(fd[cur][d], fr[rc][o], acc[d][o], fsd[hc][d],
                                                 fsr[sc][o]);
            }
#pragma unroll
            for (int r = r0; r < r1; ++r) {
                frag(is_r, nx, r_off, r, fr[rn][r]);
                if constexpr (NEWHALF) frag_scale(nx, rs_off, r, fsr[sn][r]);
            }
#pragma unroll
            for (int d = d0; d < d1; ++d) {
                frag(is_d, nx, d_off, d, fd[cur ^ 1][d]);
                if constexpr (NEWHALF) frag_scale(nx, ds_off, d, fsd[hn][d]);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, FD, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, NRR * (r1 - r0) + NRD * (d1 - d0), 0);
        });
    };

    // Before the first read of slab k1: wait for this wave's copies of it
    // (later slabs may stay in flight), sync (every wave holds the current
    // step's operands in registers, and slab k1-1 is fully read), refill the
    // slot slab k1-1 vacated with slab k1+S-1, and at a period start fetch
    // the next period's scales into the buffer the previous period vacated.
    // In-order wait for slab k1: after its copies came S-2 openings of
    // (scales and) NCOPY copies.
    constexpr int VMW = (S - 2) * NCOPY;
    static_assert(VMW + NCOPY + CPS < 64, "vmcnt range");
    auto open = [&](int k1, int slot_next, bool period_start, int pbuf_next) {
        wait_vm<VMW>();
        lds_barrier();
        if (period_start) issue_scales(k1 / PS + 1, pbuf_next);
        issue(k1 + S - 1, slot_next);
    };
    // Rows shorter than one period (K < 512: a single period, and too few
    // steps for the main loop to run) get their scale bytes with ordinary
    // loads in the prologue, copied exactly; longer rows use period copies.
    const bool short_rows = sp < 16;
    auto open_guarded = [&](int k1, int slot_next, bool period_start, int pbuf_next) {
        wait_vm<VMW>();
        lds_barrier();
        if (period_start && !short_rows) issue_scales(k1 / PS + 1, pbuf_next);
        issue(k1 + S - 1, slot_next);
    };
    // Scale byte shift for slabs of the last period when it was copied short.
    const int last_shift = short_rows ? 0 : nper * 16 - sp;
    auto shift_of = [&](int k) { return (k / PS == nper - 1) ? last_shift : 0; };

    // Prologue: scale period 0 (period 1 follows at slab 0's opening),
    // slabs 0..S-2 in flight, then open slab 0 and read step 0.
    if (!SCALED) {
        // no scales
    } else if (short_rows) {
        for (int r = tid; r < ROWS; r += NW * 64) {
            const uint8_t *src = ((r < BM) ? As + (int64_t)min(m0 + r, M - 1) * sps
                                           : Bs + (int64_t)min(n0 + r - BM, N - 1) * sps) + kb / 32;
            for (int d = 0; d < sp; d += 4)
                *(uint32_t *)(sbase + r * 16 + d) = *(const uint32_t *)(src + d);
        }
    } else {
        issue_scales(0, 0);
    }
#pragma unroll
    for (int k = 0; k < S - 1; ++k) issue(k, k);
    wait_vm<VMW>();                  // scales of period 0 and slab 0 done
    lds_barrier();
    if (!short_rows) issue_scales(1, 1);
    issue(S - 1, S - 1);
    Src cur = src_of(0, 0, 0, 0, shift_of(0));
    load_all(cur);

    // Main loop: one trip = TS slabs (a multiple of the ring depth and of
    // the scale period) = TS*HS steps, so register set, ring slot, pass and
    // scale slot of every step are constants after unrolling.  Step q of a
    // trip uses set q&1; step q+1 is in slab (q+1)/HS of the trip.  The loop
    // only runs when K spans more than one trip (K > 512), so its period
    // copies always have rows of at least 16 scale bytes.
    constexpr int TS = std::lcm(PS, S);       // k0 is a multiple of PS: kq % PS is global
    static_assert(TS % PS == 0 && TS % S == 0, "trip covers whole periods and rings");
    constexpr int TRIP = TS * HS;
    static_assert(!SCALED || TRIP % 8 == 0, "a trip is whole scale periods of 8 steps");
    int t0 = 0;
    for (; t0 + TRIP < nsteps; t0 += TRIP) {
        const int k0 = t0 / HS;                       // first slab of the trip
        static_for<TRIP>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            constexpr int kq = (q + 1) / HS;          // slab of step q+1 within the trip
            const int per = (k0 + kq) / PS;           // its scale period
            if constexpr ((q + 1) % HS == 0)
                open(k0 + kq, (kq + S - 1) % S, kq % PS == 0, (per + 1) & 1);
            cur = src_of(kq % S, (q + 1) % HS, per & 1, kq % PS, shift_of(k0 + kq));
            step(qc, cur);
        });
    }
    // Last trip: steps t0 .. nsteps-1 (1 to TRIP of them).  After the last
    // step the "next" operands are re-read from the last step's place (in
    // range, never used), which keeps the step code free of branches.
    {
        const int k0 = t0 / HS;
        static_for<TRIP>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            if (t0 + q < nsteps) {
                constexpr int kq = (q + 1) / HS;
                const int per = (k0 + kq) / PS;
                const bool more = t0 + q + 1 < nsteps;
                if ((q + 1) % HS == 0 && more)
                    open_guarded(k0 + kq, (kq + S - 1) % S, kq % PS == 0, (per + 1) & 1);
                cur = sel(more, src_of(kq % S, (q + 1) % HS, per & 1, kq % PS, shift_of(k0 + kq)),
                          cur);
                step(qc, cur);
            }
        });
    }

    // No copy may still be in flight, and every wave must be done reading the
    // ring and scale buffers, before their LDS is reused for the output.
    wait_vm0();
    lds_barrier();

    // Epilogue, one 32-row band of the wave's sub-tile at a time: the band is
    // written to a wave-private LDS area (row pitch padded by 16 bytes so the
    // two lane groups hit different banks), then read back row-major and
    // stored with 16-byte writes (8 BF16 or 4 FP32 values per lane).  Lane
    // (c, g) of fragment (i, j) holds, in element e, row 8*(e/4) + 4g + e%4
    // of column c.  Chunks that cross the end of a row of C, or rows of C
    // whose byte pitch is not a multiple of 16, are stored element by element.
    constexpr int VE = 16 / OS;                        // values per 16-byte chunk
    constexpr int CPR = WTN / VE;                      // chunks per band row
    uint8_t *const stage = smem + wave * 32 * PITCH;
    const bool vec_ok = ((int64_t)N * OS) % 16 == 0;
    otype *const Cp = (otype *)C + (int64_t)slice * cplane;
    const int col0 = n0 + wn * WTN;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = 8 * (e / 4) + 4 * g + (e % 4);
                otype v;
                if constexpr (OUT == OF32) v = acc[i][j][e];
                else v = f32_to_bf16(acc[i][j][e]);
                *(otype *)(stage + r * PITCH + (j * 32 + lr) * OS) = v;
            }
        const int row0 = m0 + wm * WTM + i * 32;
        constexpr int NIT = (32 * CPR + 63) / 64;
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int t = it * 64 + lane;
            const int r = t / CPR, ch = t % CPR;
            const int row = row0 + r, col = col0 + ch * VE;
            if (t >= 32 * CPR || row >= M || col >= N) continue;
            const v4i v = *(const v4i *)(stage + r * PITCH + ch * 16);
            otype *dst = Cp + (int64_t)row * N + col;
            if (vec_ok) {
                *(v4i *)dst = v;
            } else {
#pragma unroll
                for (int q = 0; q < VE; ++q) {
                    if (col + q >= N) break;
                    if constexpr (OUT == OF32)
                        dst[q] = __int_as_float(v[q]);
                    else
                        dst[q] = (uint16_t)((uint32_t)v[q / 2] >> (16 * (q & 1)));
                }
            }
        }
    }
}


// --------------------------------------------------------------------------
// Split-K reduction: C[i] = sum over slices s = 0, 1, ... of W[s*plane + i],
// added in slice order (so the result does not depend on timing), converted
// to the output type.  plane is a multiple of 4 and W, C are 16-byte
// aligned, so every group of 4 elements is one aligned vector access.
template <int OUT>
__global__ void __launch_bounds__(256)
splitk_reduce(const float *__restrict__ W, void *__restrict__ C, int64_t mn, int64_t plane,
              int slices)
{
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= mn) return;
    v4f acc = *(const v4f *)(W + i);
    for (int s = 1; s < slices; ++s) acc += *(const v4f *)(W + s * plane + i);
    const int n = (int)min((int64_t)4, mn - i);
    if (OUT == OF32) {
        float *c = (float *)C + i;
        if (n == 4) *(v4f *)c = acc;
        else for (int q = 0; q < n; ++q) c[q] = acc[q];
    } else {
        uint16_t *c = (uint16_t *)C + i;
        if (n == 4) {
            const uint32_t lo = f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
            const uint32_t hi = f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
            *(uint2 *)c = make_uint2(lo, hi);
        } else {
            for (int q = 0; q < n; ++q) c[q] = f32_to_bf16(acc[q]);
        }
    }
}

}  // namespace mx
