"""The two measurement kernels through the C ABI: mx_hbm_read_ceiling reads
every byte of its buffer exactly once (its per-thread XOR folds equal
numpy's over the chunk assignment the header states), and mx_mfma_ceiling
runs both formats on random and constant operands."""
import numpy as np
import pytest

import microscaled_block_scaled_amd as mxg
import mxinputs
from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 16 * 524288 + 48, 16 * 524288 * 4 + 16 * 1000,
                                    (64 << 20) + 160])
def test_hbm_read_ceiling_reads_every_chunk_once(nbytes):
    import torch
    T = mxg.HBM_CEILING_WORKGROUPS * mxg.HBM_CEILING_THREADS
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.full((T,), -1, dtype=torch.int32, device="cuda")
    log("hbm read ceiling %d bytes" % nbytes)
    rc = mxg.hbm_ceiling_ptr(src.data_ptr(), nbytes, out.data_ptr(),
                             torch.cuda.current_stream().cuda_stream)
    assert rc == 0, mxg.strerror(rc)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    # workgroup w reads the w-th of G contiguous ranges of ceil(n / G) chunks;
    # its thread t folds chunks t, t + 256, ... of the range, then the 4 words
    chunks = host.reshape(-1, 4)
    n, G = chunks.shape[0], mxg.HBM_CEILING_WORKGROUPS
    per = -(-n // G)
    want = np.zeros(T, np.uint32)
    for w in range(G):
        seg = chunks[min(w * per, n):min(w * per + per, n)]
        seg = np.concatenate([seg, np.zeros(((-len(seg)) % 256, 4), np.uint32)])
        fold = np.bitwise_xor.reduce(seg.reshape(-1, 256, 4), axis=0) if len(seg) else \
            np.zeros((256, 4), np.uint32)
        want[w * 256:(w + 1) * 256] = np.bitwise_xor.reduce(fold, axis=1)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt", [mxinputs.FMT_E2M1, mxinputs.FMT_E4M3], ids=["e2m1", "e4m3"])
def test_mfma_ceiling_runs(fmt):
    import torch
    out = torch.full((mxg.CEILING_WORKGROUPS * mxg.CEILING_THREADS,), float("nan"),
                     dtype=torch.float32, device="cuda")
    for random_data in (1, 0):
        log("mfma ceiling fmt=%d random=%d" % (fmt, random_data))
        rc = mxg.ceiling_ptr(fmt, 64, random_data, out.data_ptr(),
                             torch.cuda.current_stream().cuda_stream)
        assert rc == 0, mxg.strerror(rc)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out).all())
