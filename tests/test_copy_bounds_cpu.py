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
