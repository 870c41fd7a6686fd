"""Captured HIP graphs of the GEMM, through the C ABI: the decode plan and a
split-K plan (whose planes go to mx_gemm_noalloc's fixed scratch, so the
capture allocates nothing), and the decode plan through mx_gemm itself
(no workspace).  The library records no memset.  Each graph is replayed
several times, with eager work and synchronisations between the replays,
and every replay must equal an eager call on the same inputs bit for bit,
also after the inputs were overwritten in place."""
import numpy as np
import pytest

import microscaled_block_scaled_amd as mxg
import mxinputs
from gpu_util import log

pytestmark = pytest.mark.gpu

E2M1, E4M3 = mxinputs.FMT_E2M1, mxinputs.FMT_E4M3
BF16 = mxinputs.OUT_BF16


def _codes(rng, fmt, rows, K):
    if fmt == E2M1:
        return rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    c = rng.integers(0, 256, size=(rows, K), dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0                  # no E4M3 NaN codes
    return c


def _inputs(rng, fmt, M, N, K):
    return (_codes(rng, fmt, M, K), rng.integers(120, 135, size=(M, K // 32), dtype=np.uint8),
            _codes(rng, fmt, N, K), rng.integers(120, 135, size=(N, K // 32), dtype=np.uint8))


@pytest.mark.parametrize("name,fmt,M,N,K,noalloc,variant", [
    ("decode_noalloc", E4M3, 8, 4096, 4096, True, mxg.VARIANT_DECODE),
    ("splitk_noalloc", E2M1, 64, 2048, 16384, True, mxg.VARIANT_TILE),
    ("decode_gemm", E2M1, 5, 3000, 2560, False, mxg.VARIANT_DECODE),
])
def test_graph_replays_equal_eager(name, fmt, M, N, K, noalloc, variant):
    import torch
    p = mxg.plan(fmt, M, N, K, BF16)
    log("graph %s fmt=%d M=%d N=%d K=%d plan=%s" % (name, fmt, M, N, K, p))
    assert p["variant"] == variant
    if variant == mxg.VARIANT_TILE:
        assert p["split_k"] > 1 and p["workspace_bytes"] <= mxg.NOALLOC_SCRATCH_BYTES
    fn = mxg.gemm_noalloc_ptr if noalloc else mxg.gemm_ptr
    rng = np.random.default_rng(77 + M + fmt)
    dev = [torch.from_numpy(x).cuda() for x in _inputs(rng, fmt, M, N, K)]
    A, As, B, Bs = dev
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ref = torch.empty_like(C)

    def call(out, stream):
        rc = fn(fmt, M, N, K, A.data_ptr(), As.data_ptr(), B.data_ptr(), Bs.data_ptr(),
                out.data_ptr(), BF16, stream.cuda_stream)
        assert rc == 0, mxg.strerror(rc)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(C, side)                          # warm-up (and the scratch's address lookup)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call(C, side)
    torch.cuda.synchronize()

    cur = torch.cuda.current_stream()
    for rep in range(4):
        if rep == 3:                           # new contents, same buffers
            for d, x in zip(dev, _inputs(rng, fmt, M, N, K)):
                d.copy_(torch.from_numpy(x))
        call(ref, cur)                         # eager, on the current stream
        torch.cuda.synchronize()
        C.view(torch.int16).fill_(0x7FC1)      # a NaN pattern the GEMM never writes
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(C.view(torch.int16), ref.view(torch.int16))
        log("  replay %d: %s" % (rep, "bit-identical" if same else "DIFFERENT"))
        assert same, (name, rep)
