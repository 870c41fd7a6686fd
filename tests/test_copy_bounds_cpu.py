"""The tile kernel's HBM -> LDS copy addresses, modelled on the CPU (no GPU).

`tile_kernel` (csrc/mx_kernels.h) copies operand rows and scale periods
with 16-byte buffer loads: a wave-uniform descriptor (base, num_records)
plus a 32-bit lane offset.  A copy at or past num_records is not fetched;
whole tiles have no range check at all.  This model recomputes, for every
tile shape, format pair, partial and whole tile, first and last K-slice and
first and last slab, the byte range every lane of every copy instruction
reads, and checks that
  * every fetched range lies inside its operand (or its scale array), and
  * every byte a real row of the tile needs is fetched.
A kernel change to the copy geometry must be mirrored here.  (A first build
of the range-check change missed the clamp of FP6 padding lanes to the
tile, which this model reports as reads past B on whole tiles; that build
faulted the GPU.)"""
import itertools

import numpy as np
import pytest

FP4, FP8, BF8, B16, F6E2, F6E3 = 1, 2, 3, 4, 5, 6
# (BM, BN, waves along M, waves along N): the library's tile table
TILES = [(256, 256, 4, 2), (256, 192, 4, 2), (256, 160, 4, 1), (256, 128, 4, 2),
         (128, 128, 2, 2), (64, 256, 1, 8)]


def is6(f):
    return f in (F6E2, F6E3)


def kvals(fa, fb):                       # K-values per slab
    return 64 if fa == B16 else 256 if (fa == FP4 and fb == FP4) else 128


def slab_row_bytes(f, kv):
    return kv // 2 if f == FP4 else 2 * kv if f == B16 else kv // 4 * 3 if is6(f) else kv


def kbytes(f, k):
    return k // 2 if f == FP4 else 2 * k if f == B16 else k // 4 * 3 if is6(f) else k


def copy_rows(R):                        # rows per copy instruction
    return 8 if R == 96 else 1024 // R


def operand_copies(R, rows, NW, rowb, last, skip, cmax, size, base):
    """Lane byte ranges of one slab's copies of one operand: (fetched ok,
    needed rows fetched)."""
    RPC = copy_rows(R)
    CP = (rows // RPC + NW - 1) // NW
    wave, u, lane = np.meshgrid(np.arange(NW), np.arange(CP), np.arange(64), indexing="ij")
    i = np.minimum(wave + u * NW, rows // RPC - 1)
    crow, cpc = lane // (R // 16), lane % (R // 16)
    ch = np.minimum(cpc * 16, cmax)               # the swizzle permutes chunks within a row
    r0 = i * RPC
    row = np.where(r0 + crow < rows, r0 + crow, rows - 1)
    off = row * rowb + ch
    assert (off + 16 <= 2 ** 32).all()
    nrec = None if last + 1 == rows else (last + 1) * rowb - skip
    fetched = np.ones_like(off, bool) if nrec is None else off + 16 <= nrec
    inside = (base + off >= 0) & (base + off + 16 <= size)
    real = (r0 + crow < rows) & (r0 + crow <= last)
    return bool(inside[fetched].all()), bool(fetched[real].all())


def scale_copies(BM, BN, NW, sps, last_a, last_b, kb, soff, m0, n0, M, N):
    NSI = (BM + BN + 63) // 64
    CPS = (NSI + NW - 1) // NW
    wave, u, lane = np.meshgrid(np.arange(NW), np.arange(CPS), np.arange(64), indexing="ij")
    i = np.minimum(wave + u * NW, NSI - 1)
    in_a = i * 64 < BM
    row = i * 64 + lane - np.where(in_a, 0, BM)
    last = np.where(in_a, last_a, last_b)
    nrec = (last + 1) * sps - kb // 32 - soff
    base = np.where(in_a, m0, n0) * sps + kb // 32 + soff
    size = np.where(in_a, M, N) * sps
    off = row * sps
    fetched = off + 16 <= nrec
    ok = (base + off + 16 <= size)[fetched].all()
    need = fetched[row <= last].all()
    return bool(ok), bool(need)


def check(fa, fb, BM, BN, WGM, WGN, M, N, K, kchunk):
    NW = WGM * WGN
    kv = kvals(fa, fb)
    RA, RB = slab_row_bytes(fa, kv), slab_row_bytes(fb, kv)
    rowba, rowbb = kbytes(fa, K), kbytes(fb, K)
    sps = K // 32
    nslices = -(-K // kchunk)
    tiles_m, tiles_n = -(-M // BM), -(-N // BN)
    problems = []
    for tm, tn, sl in itertools.product(sorted({0, tiles_m - 1}), sorted({0, tiles_n - 1}),
                                        sorted({0, nslices - 1})):
        m0, n0 = tm * BM, tn * BN
        kb = sl * kchunk
        klen = min(kchunk, K - kb)
        kboffa, kboffb = kbytes(fa, kb), kbytes(fb, kb)
        rowla, rowlb = kbytes(fa, klen), kbytes(fb, klen)
        nslab = -(-klen // kv)
        last_a, last_b = min(BM, M - m0) - 1, min(BN, N - n0) - 1
        for k in sorted({0, nslab - 1}):
            koffa, koffb = k * RA, k * RB
            for name, args in (
                    ("A", (RA, BM, NW, rowba, last_a, kboffa + koffa, rowla - 16 - koffa,
                           M * rowba, m0 * rowba + kboffa + koffa)),
                    ("B", (RB, BN, NW, rowbb, last_b, kboffb + koffb, rowlb - 16 - koffb,
                           N * rowbb, n0 * rowbb + kboffb + koffb))):
                ok, need = operand_copies(*args)
                if not ok or not need:
                    problems.append((name, tm, tn, sl, k, ok, need))
        if fa != B16 and sps >= 16:
            sp = klen // 32
            nper = -(-sp // 16)
            for p in sorted({0, nper - 1}):
                soff = min(p * 16, sp - 16)
                ok, need = scale_copies(BM, BN, NW, sps, last_a, last_b, kb, soff, m0, n0, M, N)
                if not ok or not need:
                    problems.append(("scales", tm, tn, sl, p, ok, need))
    return problems


FORMATS = [FP4, FP8, BF8, F6E2, F6E3]
PAIRS = [(a, b) for a in FORMATS for b in FORMATS] + [(B16, B16)]


@pytest.mark.parametrize("tile", TILES, ids=["%dx%d" % t[:2] for t in TILES])
def test_copies_stay_inside_their_operands(tile):
    BM, BN, WGM, WGN = tile
    shapes = [(8, 8192, 4096), (1, 1, 512), (300, 200, 1536), (BM, BN, 2048),
              (BM + 5, 2 * BN - 3, 640), (40, 203, 3072), (BM, 3 * BN, 384)]
    bad = []
    for fa, fb in PAIRS:
        for M, N, K in shapes:
            if is6(fa) or is6(fb):
                K = K // 128 * 128
            for kchunk in sorted({K, max(512, -(-K // 3) // 512 * 512)}):
                for prob in check(fa, fb, BM, BN, WGM, WGN, M, N, K, kchunk):
                    bad.append(((fa, fb), (M, N, K), kchunk, prob))
    assert not bad, bad[:5]


def test_model_reports_unclamped_fp6_padding_lanes():
    """The model itself: without the clamp of FP6 padding lanes to the tile,
    a whole tile at the end of B reads past B (the fault of a first build)."""
    RB = slab_row_bytes(F6E2, 128)
    rowb = kbytes(F6E2, 4096)
    N, BN = 8192, 128
    n0 = N - BN
    RPC = copy_rows(RB)
    lane = np.arange(64)
    crow = lane // (RB // 16)
    r0 = (BN // RPC - 1) * RPC                      # the tile's last 8-row block
    unclamped = (r0 + crow) * rowb
    assert ((n0 * rowb + unclamped + 16) > N * rowb).any()
    assert not check(F6E2, F6E2, 128, 128, 2, 2, 8, N, 4096, 4096)


# --------------------------------------------------------------------------
# The decode kernel (csrc/mx_decode.h): a grid of at most 256 workgroups,
# workgroup b taking column groups b, b + grid, ...; 4 waves per workgroup,
# each a K-range of whole 512-K periods, a private ring of S slabs of the
# staged A rows and 32 B rows (a slot of which also holds the wave's
# partial tile after each group), and R period buffers of those rows' scale
# bytes; each wave's copies form one stream of slab positions over all its
# groups, nper * PS positions per group (positions past a group's slabs, or
# past its last group, copy with num_records 0), with four 4-byte scale
# copies at each period's first position.
DECODE_LDS, DECODE_ROWS, DECODE_WAVES, DECODE_CUS = 163840, 32, 4, 256
DECODE_OFFS = DECODE_WAVES * 4       # the waves' partial-tile slot offsets
DECODE_MAX_RING = 5


def decode_wide(fa, fb, M):
    """The A rows the wide slabs stage (0: not wide): an 8-bit A with an
    E2M1 B, 8 rows for M <= 8, 16 for M <= 16, else 32."""
    if fb != FP4 or fa == FP4:
        return 0
    return 8 if M <= 8 else 16 if M <= 16 else 32


def decode_geo(fa, fb, wide=0):
    """(K-values per slab, A and B slab row bytes, rows of A staged, copies
    per slab, ring depth, period buffers) of the decode kernel: the deepest
    ring (at most 5 slabs) whose slabs and period buffers fit in the LDS,
    with a wait count (the next S - 2 positions' loads) within 63; each
    wave's partial tile is added in one of its ring slots."""
    kv = 256 if wide else kvals(fa, fb)
    RA, RB = slab_row_bytes(fa, kv), slab_row_bytes(fb, kv)
    MA = wide if wide else DECODE_ROWS
    slot = MA * RA + DECODE_ROWS * RB
    ncopy = slot // 1024
    PS = 512 // kv
    bufs = lambda s: (s - 1) // PS + 1
    lead = lambda s: (s - 2) * ncopy + 4 * ((s - 3 + PS) // PS)
    S = 3
    while (S < DECODE_MAX_RING
           and DECODE_WAVES * ((S + 1) * slot + bufs(S + 1) * 1024) + DECODE_OFFS <= DECODE_LDS
           and lead(S + 1) <= 63):
        S += 1
    assert slot >= DECODE_ROWS * DECODE_ROWS * 4     # a slot holds a partial tile
    return kv, RA, RB, MA, ncopy, S, bufs(S)


def decode_operand(R, rowb, rows_real, cmax, records, size, base, live, need_bytes,
                   staged=DECODE_ROWS):
    """One slab position's copies of one operand (`staged` rows)."""
    RPC = 1024 // R
    i, lane = np.meshgrid(np.arange(staged // RPC), np.arange(64), indexing="ij")
    row = i * RPC + lane // (R // 16)
    cpc = lane % (R // 16)
    ch = np.minimum(cpc * 16, cmax)               # the swizzle permutes chunks within a row
    off = row * rowb + ch
    assert (off < 2 ** 32).all()
    fetched = off + 16 <= records
    inside = (base + off >= 0) & (base + off + 16 <= size)
    ok = bool(inside[fetched].all())
    if not live:
        return ok and not fetched.any(), True
    needed = (row < rows_real) & (cpc * 16 < need_bytes)
    return ok, bool(fetched[needed].all())


def decode_scales(sps, rows_real, kbs, records, size, base, live, nbytes):
    """One period's scale copies of one operand: lane l of copy i takes
    dword l % 4 of row 16i + l // 4, from the period's first scale byte
    kbs.  Returns (every fetched dword inside the operand's scale array,
    every dword the MFMAs read fetched)."""
    i, lane = np.meshgrid(np.arange(2), np.arange(64), indexing="ij")
    row, w = 16 * i + lane // 4, lane % 4
    off = row * sps + 4 * w
    fetched = off + 4 <= records
    inside = (base + kbs + off >= 0) & (base + kbs + off + 4 <= size)
    ok = bool(inside[fetched].all())
    if not live:
        return ok and not fetched.any(), True
    needed = (row < rows_real) & (4 * w < nbytes)
    return ok, bool(fetched[needed].all())


def decode_check(fa, fb, M, N, K, scale_records_from_period=True, idle_records=True):
    """Problems of the decode kernel's loads for one problem, for the first
    and the last workgroup; the two flags turn off the scale copies' extent
    counted from the period's first scale byte and the zero num_records of
    copies with no slab (for the model's own tests)."""
    kv, RA, RB, MA, ncopy, S, R = decode_geo(fa, fb, decode_wide(fa, fb, M))
    PS = 512 // kv
    assert S >= 3 and (S - 2) * ncopy + 4 * ((S - 3 + PS) // PS) <= 63 and R * PS > S - 1
    assert DECODE_WAVES * (S * (MA * RA + DECODE_ROWS * RB) + R * 1024) + DECODE_OFFS <= DECODE_LDS
    rowba, rowbb = kbytes(fa, K), kbytes(fb, K)
    sps = K // 32
    per_w = -(-(K // 128) // (4 * DECODE_WAVES))
    ngroups = -(-N // DECODE_ROWS)
    grid = min(ngroups, DECODE_CUS)
    problems = []
    for b in sorted({0, grid - 1}):
        ng = (ngroups - 1 - b) // grid + 1
        group_n0 = lambda gi: (b + min(gi, ng - 1) * grid) * DECODE_ROWS
        for wave in range(DECODE_WAVES):
            kb = min(wave * per_w * 512, K)
            klen = min(per_w * 512, K - kb)
            nslab = -(-klen // kv)
            if nslab == 0:
                continue
            nper = -(-klen // 512)
            ppg = nper * PS                             # slab positions per group
            kboffa, kboffb = kbytes(fa, kb), kbytes(fb, kb)
            rowla, rowlb = kbytes(fa, klen), kbytes(fb, klen)
            exta = M * rowba - kboffa
            # every position the stream issues: S - 1 ahead, then one per position
            for j in range(ng * ppg + S - 1):
                gj, k = divmod(j, ppg)
                live = gj < ng and k < nslab
                kc = min(k, nslab - 1)
                n0 = group_n0(gj)
                rows_b = min(DECODE_ROWS, N - n0)
                extb = rows_b * rowbb - kboffb
                koffa, koffb = kc * RA, kc * RB
                # positions whose slab is read must be the group's first or last
                # or a dummy one: check those (plus every dummy) to bound the work
                if live and k not in (0, 1, nslab - 1) and gj not in (0, ng - 1):
                    continue
                for name, args in (
                        ("A", (RA, rowba, M, rowla - 16 - koffa,
                               exta - koffa if live or not idle_records else 0, M * rowba,
                               kboffa + koffa, live, rowla - koffa, MA)),
                        ("B", (RB, rowbb, rows_b, rowlb - 16 - koffb,
                               extb - koffb if live or not idle_records else 0, N * rowbb,
                               n0 * rowbb + kboffb + koffb, live, rowlb - koffb))):
                    ok, need = decode_operand(*args)
                    if not ok or not need:
                        problems.append((name, b, wave, j, ok, need))
                if k % PS:
                    continue
                q = k // PS                               # the period this position starts
                slive = gj < ng
                kbs = kb // 32 + 16 * q
                nbytes = min(512, klen - 512 * q) // 32   # scale bytes the period's steps read
                for name, rows, base, size in (("As", M, 0, M * sps),
                                               ("Bs", rows_b, n0 * sps, N * sps)):
                    rec = rows * sps - (kbs if scale_records_from_period else 0)
                    ok, need = decode_scales(sps, rows, kbs,
                                             rec if slive or not idle_records else 0,
                                             size, base, slive, nbytes)
                    if not ok or not need:
                        problems.append((name, b, wave, j, ok, need))
    return problems


DECODE_FORMATS = [FP4, FP8, BF8]


@pytest.mark.parametrize("fa,fb", [(a, b) for a in DECODE_FORMATS for b in DECODE_FORMATS])
def test_decode_copies_stay_inside_their_operands(fa, fb):
    shapes = [(1, 1, 512), (8, 8192, 28672), (32, 203, 640), (5, 100, 1664), (17, 64, 3200),
              (32, 8161, 2048), (3, 40, 1152), (32, 96, 8192 + 384), (2, 33, 4096 + 128),
              (9, 40, 2560), (16, 70, 1152), (8, 28672, 4096), (4, 16417, 1664),
              (32, 24607, 640), (12, 8200, 3200), (16, 16417, 4224), (24, 9000, 1664),
              (32, 8192, 28672)]
    bad = []
    for M, N, K in shapes:
        bad += [((M, N, K), prob) for prob in decode_check(fa, fb, M, N, K)]
    assert not bad, bad[:5]


def test_decode_model_reports_planted_mistakes():
    """The model itself: scale copies whose extent is not counted from the
    period's first scale byte read past the scale array (the dwords past
    the last row's end in a short last period); copies past the range with
    a live num_records fetch what the kernel never reads."""
    assert not decode_check(FP4, FP4, 5, 100, 1664)
    assert any(p[0] in ("As", "Bs") for p in decode_check(FP4, FP4, 5, 100, 1664,
                                                          scale_records_from_period=False))
    assert any(p[0] in ("A", "B") for p in decode_check(FP8, FP8, 8, 64, 4096 + 128,
                                                        idle_records=False))
