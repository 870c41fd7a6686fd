/*
 * mxgemm.h -- C ABI of the MI355X (gfx950) MX block-scaled NT GEMM, its
 * grouped (mixture-of-experts) form, MX quantization, and a dense BF16 GEMM
 * on the same kernels.
 *
 * The operation (FlyDSL summary pages, section "API compatibility is not
 * universal input coverage"; AI-compiler digest 2026-10-22, item 1
 * "Accelerating PyTorch on AMD GPUs with FlyDSL": MXFP8 / MXFP4 scaled GEMM,
 * BlockWise1x32, E8M0 scale, FP32 accumulation, K a multiple of 128):
 *
 *   C[m][n] = sum_b 2^(sA[m][b] + sB[n][b] - 254)
 *                   * sum_{j<32} A[m][32b+j] * B[n][32b+j]
 *
 * for m < M, n < N, b < K/32, with A and B holding MXFP4 (E2M1) or MXFP8
 * (E4M3) elements and sA, sB their E8M0 scale bytes.  Products and sums are
 * accumulated in FP32; C is written as FP32 or as BF16 (round to nearest
 * even).  The element and scale encodings are those of the OCP Microscaling
 * (MX) v1.0 specification.
 *
 * Memory layout (all dense, row-major, device memory owned by the caller):
 *   A        M x K   elements, K-contiguous.  E4M3: M x K bytes, element k in
 *            byte k.  E2M1: M x K/2 bytes, element 2i in the low nibble of
 *            byte i, element 2i+1 in the high nibble.
 *   B        N x K   elements, K-contiguous, same encoding as A ("NT": C is
 *            A times B transposed).
 *   A_scale  M x K/32 bytes; byte [m][b] scales K-values 32b .. 32b+31 of row m.
 *   B_scale  N x K/32 bytes; likewise for B.
 *   C        M x N  float or bfloat16 (uint16 bit pattern), row pitch N.
 * There are no stride arguments: callers with other layouts must copy.
 *
 * Errors.  Every argument check runs before any HIP call; a failed check
 * returns a negative MX_ERR_* code and touches nothing.  Launch failures are
 * reported as MX_ERR_LAUNCH.  No function aborts or throws.
 *
 * Asynchrony.  mx_gemm enqueues its kernels on `stream` (a hipStream_t;
 * NULL means the device's null stream) and returns without synchronising:
 * C is ready when the stream reaches that point.  Inputs must stay alive and
 * unmodified until then.  C must not overlap any input.  Results are
 * bit-for-bit deterministic for a given (M, N, K, formats, device).
 *
 * Thread safety.  Calls may be made concurrently from several host threads
 * and streams.  The library keeps read-only per-device state, set up once per
 * device on first use, and, for split-K calls (see mx_plan_t), one workspace
 * per (device, stream handle).  Lifetime of a workspace: it is allocated on
 * that stream with hipMallocAsync the first time a call there needs one,
 * replaced (freed and reallocated on the stream) when a call needs more, and
 * otherwise held, at the largest size a call on that stream has needed,
 * until the process exits -- destroying the stream does not free it.  Calls
 * on one stream are ordered by the stream; calls on different streams use
 * different workspaces; split-K calls on one stream from several host threads
 * are serialised while they are enqueued.  One precondition follows: a
 * stream must have finished its split-K calls (hipStreamSynchronize) before
 * it is destroyed, because a stream created later may receive the same
 * handle and would then share that workspace with the still-running calls.
 */
#ifndef MXGEMM_H
#define MXGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element formats: MXFP4 = E2M1; MXFP8 = E4M3, or its other OCP encoding
 * E5M2 (wider range: 2^-16 .. 57344, with infinities and NaNs); MXFP6 =
 * E2M3 (largest 7.5) or E3M2 (largest 28), no infinities or NaNs.  E5M2 is
 * accepted, like the FP6 formats, by mx_gemm, mx_gemm_tile, mx_gemm_mixed
 * (paired with any format), the grouped GEMMs (any pair) and mx_quantize.
 * FP6 rows are K*3/4 bytes: a little-endian bit string with element k in
 * bits 6k .. 6k+5 (bit b is bit b % 8 of byte b / 8), four elements in
 * three bytes (OCP MX v1.0 fixes the element encoding; this packing is this
 * library's). */
enum { MX_FMT_E2M1 = 1, MX_FMT_E4M3 = 2, MX_FMT_E5M2 = 3, MX_FMT_E2M3 = 4, MX_FMT_E3M2 = 5 };

/* Output element types. */
enum { MX_OUT_FP32 = 1, MX_OUT_BF16 = 2 };

/* Return codes. */
enum {
    MX_OK = 0,
    MX_ERR_FORMAT = -1,     /* unknown format, or one this call does not take */
    MX_ERR_OUT_DTYPE = -2,  /* out_dtype is not MX_OUT_FP32 / MX_OUT_BF16     */
    MX_ERR_SHAPE = -3,      /* M < 1, N < 1, K < 128, K % 128 != 0, M or N
                               above MX_MAX_DIM, K above MX_MAX_K, or more
                               than 2^31 - 1 workgroups of tiles needed        */
    MX_ERR_NULL = -4,       /* a required pointer is NULL                     */
    MX_ERR_ALIGN = -5,      /* A, B or C not 16-byte aligned, or a scale
                               array not 4-byte aligned                        */
    MX_ERR_NO_DEVICE = -6,  /* no HIP device is visible                       */
    MX_ERR_ARCH = -7,       /* the current device is not gfx950               */
    MX_ERR_ALLOC = -8,      /* split-K workspace allocation failed            */
    MX_ERR_LAUNCH = -9,     /* a kernel launch failed                         */
    MX_ERR_IN_DTYPE = -10,  /* in_dtype is not MX_IN_FP32 / MX_IN_BF16       */
    MX_ERR_SCRATCH = -11    /* mx_gemm_noalloc: the problem's split-K workspace
                               exceeds MX_NOALLOC_SCRATCH_BYTES               */
};

/* Input element types of mx_quantize. */
enum { MX_IN_FP32 = 1, MX_IN_BF16 = 2 };

/* Largest M or N accepted (keeps every tile index in 32 bits). */
#define MX_MAX_DIM ((int64_t)1 << 30)
/* Largest K accepted (keeps a tile's per-lane copy offsets, up to 256 rows of
 * one operand, within 32 bits). */
#define MX_MAX_K ((int64_t)1 << 24)

/*
 * C = A * B^T with MX block scaling, enqueued on `stream`.
 *   fmt        any MX_FMT_* code (A and B share the format; mx_gemm_mixed
 *              takes one per operand)
 *   M, N, K    sizes; K a multiple of 128, at most MX_MAX_K
 *   A, B       packed elements (layout above), 16-byte aligned device pointers
 *   A_scale,
 *   B_scale    E8M0 scale bytes (layout above), 4-byte aligned
 *   C          output, 16-byte aligned; float if out_dtype == MX_OUT_FP32,
 *              bfloat16 bits if MX_OUT_BF16
 *   stream     hipStream_t, or NULL
 * Returns MX_OK or a negative MX_ERR_* code.
 */
int mx_gemm(int fmt, int64_t M, int64_t N, int64_t K,
            const void *A, const void *A_scale,
            const void *B, const void *B_scale,
            void *C, int out_dtype, void *stream);

/* Static, NUL-terminated description of a return code. */
const char *mx_strerror(int code);

/*
 * Kernel variants a plan can choose.
 * MX_VARIANT_TILE: the tiled kernel, in which each workgroup computes one
 *   tile_m x tile_n tile of C, staging A and B through LDS.  Small M uses a
 *   128- or 64-row tile.  When the tiles cannot fill the GPU and K is long,
 *   each workgroup takes one of split_k K-slices and writes FP32 partial
 *   results to a workspace that a second kernel adds in slice order
 *   (workspace_bytes of the stream's workspace, see "Thread safety" above;
 *   mx_gemm_noalloc uses a fixed scratch instead).
 * MX_VARIANT_DECODE: the decode kernel, for M <= MX_DECODE_TILE rows with
 *   both operands E2M1, E4M3 or E5M2 and K >= 512.  C is cut into groups
 *   of MX_DECODE_TILE columns (all M rows); workgroups = min(groups, 256),
 *   at most one per CU, and workgroup b computes groups b, b + workgroups,
 *   ...; its four waves take four K-ranges of whole 512-K periods and add
 *   their partial sums in LDS in a fixed order.  tile_m = tile_n =
 *   MX_DECODE_TILE, split_k = 1, no workspace.  The plan takes it where it streams B faster than the tiled
 *   kernel; mx_gemm_tile and mx_gemm_mixed run it when asked for the tile
 *   (MX_DECODE_TILE, MX_DECODE_TILE).
 */
enum { MX_VARIANT_TILE = 1, MX_VARIANT_DECODE = 2 };
#define MX_DECODE_TILE 32

/* How mx_gemm would run a problem (filled by mx_gemm_plan). */
typedef struct {
    int variant;            /* MX_VARIANT_*                                   */
    int tile_m, tile_n;     /* output tile of one workgroup                   */
    int split_k;            /* K slices per output tile (1 = none); they are
                               added in a fixed order, never with atomics       */
    int threads;            /* threads per workgroup                          */
    int lds_bytes;          /* dynamic LDS per workgroup                      */
    int64_t workgroups;     /* workgroups in the main launch                  */
    int64_t workspace_bytes;/* split-K workspace the call uses (0 = none)     */
} mx_plan_t;

/*
 * Fill *plan with the launch mx_gemm would make for these arguments.  Pure
 * host logic: it makes no HIP call and does not need a device.  Returns
 * MX_OK, or the same argument error mx_gemm would return.
 */
int mx_gemm_plan(int fmt, int64_t M, int64_t N, int64_t K, int out_dtype,
                 mx_plan_t *plan);

/*
 * mx_gemm for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, plan, kernels, errors and results (bit for bit) as mx_gemm;
 * the only difference is where a split-K call keeps its FP32 partial planes.
 * Instead of allocating them, it uses a fixed scratch array in device memory
 * of MX_NOALLOC_SCRATCH_BYTES, one per device, which the library holds from
 * its first call on that device until the process ends.  It calls no
 * allocator at all (no hipMalloc, hipMallocAsync, hipFree or library routine
 * that allocates).
 *   Returns MX_ERR_SCRATCH, before any HIP call, when the plan's
 *   workspace_bytes (mx_gemm_plan) exceeds MX_NOALLOC_SCRATCH_BYTES: e.g.
 *   M = 256, N = 8192, K = 28672 (4 K-slices) needs exactly 32 MiB and runs;
 *   M = 512, N = 6144, K = 28672 (4 slices of 12 MiB) is refused.  Problems
 *   the plan does not split need no scratch and have no limit.
 * Every call on one device shares that device's scratch, and it keeps what
 * the last call wrote (each split-K call writes every element it reads, so
 * nothing needs clearing): two calls that overlap in time on one device --
 * on different streams, or from different host threads without stream
 * ordering between them -- race on it and may return wrong results.
 */
#define MX_NOALLOC_SCRATCH_BYTES ((int64_t)32 << 20)
int mx_gemm_noalloc(int fmt, int64_t M, int64_t N, int64_t K,
                    const void *A, const void *A_scale,
                    const void *B, const void *B_scale,
                    void *C, int out_dtype, void *stream);

/*
 * Test hook: the next `count` calls of mx_gemm and its variants that need a
 * split-K workspace fail as if obtaining it had failed: they return
 * MX_ERR_ALLOC and launch nothing.  count <= 0 clears it.  For exercising
 * the MX_ERR_ALLOC path only.
 */
void mx_debug_fail_allocations(int count);

/*
 * The output tile shapes the library has kernels for.  Writes up to
 * max_pairs (tile_m, tile_n) pairs to pairs[2i], pairs[2i+1] (pairs may be
 * NULL) and returns how many shapes there are.  Host logic only.
 */
int mx_tile_shapes(int *pairs, int max_pairs);

/*
 * mx_gemm on the tile kernel with the output tile (and K split) chosen by the
 * caller instead of the plan: (tile_m, tile_n) must be one of the shapes
 * mx_tile_shapes lists, and split_k is 0 (the plan's choice) or 1 ..
 * MX_MAX_SPLIT_K (K is then cut into that many slices of whole 512-K
 * periods, or fewer when K is short); otherwise MX_ERR_SHAPE.  The tile
 * (MX_DECODE_TILE, MX_DECODE_TILE) runs the decode kernel (MX_VARIANT_DECODE)
 * instead: it needs fmt E2M1, E4M3 or E5M2, M <= MX_DECODE_TILE, K >= 512 and
 * split_k 0 or 1, else MX_ERR_SHAPE.  Everything else -- arguments, layouts,
 * errors, results -- is as for mx_gemm.  It exists so that every kernel
 * configuration can be exercised (and timed) on any problem size.
 */
#define MX_MAX_SPLIT_K 8
int mx_gemm_tile(int fmt, int64_t M, int64_t N, int64_t K,
                 const void *A, const void *A_scale,
                 const void *B, const void *B_scale,
                 void *C, int out_dtype, int tile_m, int tile_n, int split_k,
                 void *stream);

/*
 * MX quantization, the step that produces mx_gemm's operands: X (rows x K,
 * FP32 or BF16, K-contiguous) -> Q and Q_scale in the layouts described
 * above for A and A_scale.  The rule is the OCP Microscaling v1.0
 * conversion (the FlyDSL article times its scaled GEMMs from operands
 * already in this form, section "Performance numbers need their
 * baselines"); per block of 32 consecutive values x along K:
 *   X = floor(log2 max|x|) - emax      (emax = 2 for E2M1, 8 for E4M3,
 *                                       15 for E5M2, 2 for E2M3, 4 for E3M2)
 *   scale byte = X + 127, clamped to [0, 254]; 0 for an all-zero block
 *   element    = x * 2^(127 - scale byte) rounded to the nearest element
 *                value (ties to the code with an even last bit), magnitudes
 *                above 6 (E2M1) / 448 (E4M3) / 57344 (E5M2) / 7.5 (E2M3) /
 *                28 (E3M2) saturating,
 *                sign kept
 *   a block holding a NaN or an infinity: scale byte 255, element codes 0.
 *   fmt        any MX_FMT_* code
 *   in_dtype   MX_IN_FP32 or MX_IN_BF16
 *   rows, K    rows >= 1, K >= 32, K % 32 == 0, both <= MX_MAX_DIM
 *   X          device pointer, 16-byte aligned
 *   Q          device pointer, 8-byte aligned: rows x K bytes (E4M3, E5M2)
 *              or rows x K/2 bytes (E2M1, element 2i in the low nibble)
 *              or rows x 3K/4 bytes (E2M3, E3M2, the FP6 bit string)
 *   Q_scale    device pointer: rows x K/32 bytes
 *   stream     hipStream_t, or NULL
 * Returns MX_OK or a negative MX_ERR_* code; errors and asynchrony as for
 * mx_gemm.  Outputs must not overlap X.
 */
int mx_quantize(int fmt, int in_dtype, int64_t rows, int64_t K,
                const void *X, void *Q, void *Q_scale, void *stream);

/*
 * MX GEMM with A and B in different element formats: fmt_a for A, fmt_b for
 * B, each any MX_FMT_* code, in any pair (A E4M3 with B E2M1 is the usual
 * "W4A8" serving layout; E4M3 with E5M2 pairs the two MXFP8 encodings; FP6
 * pairs with the 4- and 8-bit formats and with the other FP6 format).  The
 * block dot product is the one of mx_gemm with
 * each operand decoded in its own format (the OCP MX v1.0 dot product does
 * not require equal formats; the pages' "broader low precision" outlook, and
 * gfx950's scaled MFMA takes a format per operand).  A is M x K in fmt_a's
 * layout (K, K/2 or 3K/4 bytes per row), B is N x K in fmt_b's; scales, C, the
 * output types, alignment, errors and asynchrony as for mx_gemm.
 * tile_m = tile_n = 0 takes the plan's tile (the plan depends on M, N and K,
 * and on whether both formats are E2M1, E4M3 or E5M2, which the decode
 * kernel needs: mx_gemm_plan with either format describes it when both are,
 * and with an FP6 format when one is); otherwise (tile_m, tile_n) must be
 * one of mx_tile_shapes, or the decode tile under mx_gemm_tile's conditions.
 * split_k as for mx_gemm_tile (0: the plan's).  With fmt_a == fmt_b the
 * result equals mx_gemm's / mx_gemm_tile's bit for bit.
 */
int mx_gemm_mixed(int fmt_a, int fmt_b, int64_t M, int64_t N, int64_t K,
                  const void *A, const void *A_scale,
                  const void *B, const void *B_scale,
                  void *C, int out_dtype, int tile_m, int tile_n, int split_k,
                  void *stream);

/*
 * Dense BF16 NT GEMM, C = A * B^T with no scales:
 *   C[m][n] = sum_{k<K} A[m][k] * B[n][k]
 * accumulated in FP32 -- the FlyDSL article's second GEMM workload (dense
 * BF16 GEMMs, section "Performance numbers need their baselines").  It runs
 * on the same tile kernels as mx_gemm, on gfx950's BF16 matrix instruction.
 *   M, N, K    M, N >= 1 and <= MX_MAX_DIM; K >= 16, K % 16 == 0,
 *              K <= MX_MAX_K_BF16
 *   A          M x K bfloat16 values (16-bit patterns), K-contiguous, row
 *              pitch K; 16-byte aligned device pointer
 *   B          N x K bfloat16 values, likewise ("NT": C is A times B
 *              transposed)
 *   C          output, 16-byte aligned; float if out_dtype == MX_OUT_FP32,
 *              bfloat16 bits (round to nearest even) if MX_OUT_BF16
 *   tile_m, tile_n, split_k  as for mx_gemm_mixed: 0, 0, 0 takes the plan's
 *              choice (mx_gemm_bf16_plan describes it), otherwise one of
 *              mx_tile_shapes and 0 .. MX_MAX_SPLIT_K slices of whole 512-K
 *              periods
 *   stream     hipStream_t, or NULL
 * Returns MX_OK or a negative MX_ERR_* code.  Errors, asynchrony, the
 * split-K workspace and determinism are as for mx_gemm; C must not overlap
 * A or B.
 */
#define MX_MAX_K_BF16 ((int64_t)1 << 23)
int mx_gemm_bf16(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                 void *C, int out_dtype, int tile_m, int tile_n, int split_k,
                 void *stream);

/*
 * The launch mx_gemm_bf16 would make with tile and split 0.  Host logic only:
 * no HIP call, no device needed.  Returns MX_OK or mx_gemm_bf16's argument
 * error (MX_ERR_NULL for a NULL plan).
 */
int mx_gemm_bf16_plan(int64_t M, int64_t N, int64_t K, int out_dtype, mx_plan_t *plan);

/* Largest number of groups of mx_gemm_grouped. */
#define MX_MAX_GROUPS 256

/*
 * Grouped MX GEMM, as in a mixture-of-experts layer (the FlyDSL article's
 * grouped-GEMM cases, section "Performance numbers need their baselines":
 * uniform groups, changing projection sizes, uneven expert loads): group g
 * multiplies its group_rows[g] rows of A by its own N x K weight B_g,
 *   C_g = A_g * B_g^T  for g = 0 .. groups-1,
 * each exactly as mx_gemm would.
 *   groups       1 .. MX_MAX_GROUPS
 *   group_rows   HOST array of `groups` row counts, each >= 0 (0 allowed)
 *   A, A_scale   the groups' rows stacked in group order: (sum of
 *                group_rows) rows, laid out as mx_gemm's A / A_scale
 *   B, B_scale   the groups' weights stacked: groups * N rows, laid out as
 *                mx_gemm's B / B_scale (weight g is rows g*N .. g*N+N-1)
 *   C            (sum of group_rows) x N, rows in the order of A's rows
 * N, K, formats, alignment, errors and asynchrony as for mx_gemm (checked
 * with M = the total row count); groups * N must not exceed MX_MAX_DIM.
 * With no rows at all it returns MX_OK at once: nothing is launched and no
 * pointer is looked at.  No workspace is used.
 */
int mx_gemm_grouped(int fmt, int64_t groups, const int64_t *group_rows,
                    int64_t N, int64_t K, const void *A, const void *A_scale,
                    const void *B, const void *B_scale, void *C, int out_dtype,
                    void *stream);

/*
 * mx_gemm_grouped with the weights in their own format: A (and A_scale) in
 * fmt_a, every B_g (and B_scale) in fmt_b: the pairs mx_gemm_mixed takes
 * (any two MX formats; E4M3
 * activations with E2M1 expert weights is the usual serving layout of a
 * mixture-of-experts layer; the block dot product is mx_gemm_mixed's).
 * A's rows are as long as fmt_a says, B's as fmt_b says; everything
 * else as for mx_gemm_grouped, whose plan (mx_gemm_grouped_plan with fmt_a)
 * describes the launch.  With fmt_a == fmt_b it is mx_gemm_grouped.
 */
int mx_gemm_grouped_mixed(int fmt_a, int fmt_b, int64_t groups, const int64_t *group_rows,
                          int64_t N, int64_t K, const void *A, const void *A_scale,
                          const void *B, const void *B_scale, void *C, int out_dtype,
                          void *stream);

/*
 * How mx_gemm_grouped would run a problem: one tile shape for all groups
 * (split_k is always 1, workspace_bytes 0; workgroups is the total number of
 * tiles over the groups, 0 when there are no rows).  Host logic only: no
 * HIP call, no device needed.  Returns MX_OK or mx_gemm_grouped's argument
 * error (MX_ERR_NULL also for a NULL plan).
 */
int mx_gemm_grouped_plan(int fmt, int64_t groups, const int64_t *group_rows,
                         int64_t N, int64_t K, int out_dtype, mx_plan_t *plan);

/*
 * Grouped dense BF16 GEMM (the FlyDSL article's grouped-GEMM cases, section
 * "Performance numbers need their baselines", with the dense BF16 GEMM's
 * element type): group g multiplies its group_rows[g] rows of A by its own
 * N x K weight B_g with no scales,
 *   C_g = A_g * B_g^T  for g = 0 .. groups-1,
 * each exactly as mx_gemm_bf16 would (with its plan's tile and no K split).
 *   groups       1 .. MX_MAX_GROUPS
 *   group_rows   HOST array of `groups` row counts, each >= 0
 *   A            (sum of group_rows) x K bfloat16 values, K-contiguous
 *   B            groups * N rows of K bfloat16 values (weight g is rows
 *                g*N .. g*N+N-1)
 *   C            (sum of group_rows) x N, rows in the order of A's rows
 * K, the output types, alignment (16 bytes for A, B and C), errors and
 * asynchrony as for mx_gemm_bf16; groups * N must not exceed MX_MAX_DIM.
 * With no rows at all it returns MX_OK at once.  No workspace is used.
 */
int mx_gemm_grouped_bf16(int64_t groups, const int64_t *group_rows, int64_t N, int64_t K,
                         const void *A, const void *B, void *C, int out_dtype, void *stream);

/*
 * How mx_gemm_grouped_bf16 would run a problem (as mx_gemm_grouped_plan
 * does for MX formats).  Host logic only.
 */
int mx_gemm_grouped_bf16_plan(int64_t groups, const int64_t *group_rows, int64_t N,
                              int64_t K, int out_dtype, mx_plan_t *plan);

/* Launch shape of mx_mfma_ceiling: the tile kernel's (one 512-thread
 * workgroup per compute unit of the MI355X). */
#define MX_CEILING_WORKGROUPS 256
#define MX_CEILING_THREADS 512

/*
 * Measurement, not part of the GEMM: the rate at which the current device
 * sustains the block-scaled matrix instruction with no memory traffic, to
 * set a GEMM's measured rate against (the datasheet peak assumes the top
 * clock, which the power limit may not allow).  Every wave of
 * MX_CEILING_WORKGROUPS x MX_CEILING_THREADS threads keeps a 2 x 4 grid of
 * 32x32 FP32 accumulators and runs `steps` K-steps of 8 instructions (K 64
 * each, 2*32*32*64 FLOPs each) on register-resident operands: two operand
 * sets alternating step by step, hashed ("random_data" non-zero; E4M3 NaN
 * codes replaced) or constant.  Total FLOPs =
 * MX_CEILING_WORKGROUPS * MX_CEILING_THREADS / 64 * steps * 8 * 131072.
 *   fmt     MX_FMT_E2M1 or MX_FMT_E4M3 (both operands)
 *   steps   even, 2 .. 2^30
 *   out     device memory for MX_CEILING_WORKGROUPS * MX_CEILING_THREADS
 *           floats, 4-byte aligned; receives each lane's accumulator sum (a
 *           value with no meaning, written so that no work is dead code)
 * Returns MX_OK or MX_ERR_FORMAT / MX_ERR_SHAPE / MX_ERR_NULL / MX_ERR_ALIGN
 * / a device error; asynchronous on `stream` like mx_gemm.
 */
int mx_mfma_ceiling(int fmt, int64_t steps, int random_data, float *out, void *stream);

/* Launch shape of mx_hbm_read_ceiling: two 256-thread workgroups per CU. */
#define MX_HBM_CEILING_WORKGROUPS 512
#define MX_HBM_CEILING_THREADS 256

/*
 * Measurement only, not part of the GEMM: reads `bytes` of device memory at
 * src once, as a plain streaming kernel does.  The buffer is cut into
 * MX_HBM_CEILING_WORKGROUPS contiguous ranges of ceil(bytes/16 /
 * MX_HBM_CEILING_WORKGROUPS) 16-byte chunks (the last ones shorter or
 * empty); thread t of workgroup w folds with XOR the chunks t, t + 256, ...
 * of range w, and writes its fold to out[256 w + t] (out holds
 * MX_HBM_CEILING_WORKGROUPS * MX_HBM_CEILING_THREADS 32-bit words,
 * caller-owned device memory).  Loads carry the nontemporal hint.  Timing
 * it over a buffer larger than the last-level cache gives the rate at which
 * this device actually delivers HBM data to the CUs, the practical bound of
 * the memory-bound GEMM shapes (the FlyDSL article, "Performance numbers need
 * their baselines": a rate means little without its baseline).  bytes is a
 * positive multiple of 16; src is 16-byte aligned, out 4-byte aligned.
 * Enqueued on `stream`, asynchronous.  Returns MX_OK, MX_ERR_NULL,
 * MX_ERR_SHAPE, MX_ERR_ALIGN, a device error or MX_ERR_LAUNCH.
 */
int mx_hbm_read_ceiling(const void *src, int64_t bytes, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MXGEMM_H */
