"""Helpers shared by the GPU tests: move a case to the device, run the
library, and compare against the oracle."""
import sys

import numpy as np

import microscaled_block_scaled_amd as mxg
import mxinputs
import oracle


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(case):
    import torch
    d = {}
    for k in ("A", "A_scale", "B", "B_scale"):
        d[k] = torch.from_numpy(np.ascontiguousarray(case[k])).cuda()
    return d


def run_gpu(case, out_dtype, dev=None, stream=None, tile=None, split_k=0):
    import torch
    dev = dev or to_dev(case)
    tdt = torch.float32 if out_dtype == mxinputs.OUT_FP32 else torch.bfloat16
    C = mxg.mx_gemm(dev["A"], dev["A_scale"], dev["B"], dev["B_scale"], case["fmt"],
                    out_dtype=tdt, stream=stream, tile=tile, split_k=split_k)
    torch.cuda.synchronize()
    return C


def host64(C):
    return C.float().cpu().numpy().astype(np.float64)


# Per test file: elements judged, elements beyond the plain bound, the worst
# plain ratio, and whether the file's cases may add the group term E.
# Printed at the end of a session (tests/conftest.py).
PLAIN_STATS = {}


def _caller_file():
    import inspect
    import os
    for fr in inspect.stack()[1:]:
        base = os.path.basename(fr.filename)
        if base.startswith("test_"):
            return base
    return "?"


def acceptance(g, Cref, T, out_is_bf16, E=None, group_term=False, what=""):
    """The acceptance rule, element by element: |gpu - C| <= 1e-5 * T, plus
    one bfloat16 ulp of C for BF16 output (NaN and out-of-range values as
    oracle.compare says).

    group_term=True is for cases built on purpose so that a large product
    shares its group of 8 with small ones: there the bound adds the oracle's
    term E, the most that gfx950's block-scaled MFMA drops when it aligns a
    group of 8-bit products to the largest one.  Every call records, per
    test file, how many elements miss the plain bound (they must be none
    unless group_term is set) and the worst plain ratio."""
    plain = oracle.compare(g, Cref, T, out_is_bf16)
    res = dict(plain)
    res["n_plain_bad"] = plain["n_bad"]
    res["plain_max_ratio"] = plain["max_ratio"]
    if group_term:
        if E is None:
            raise ValueError("group_term needs the oracle's E")
        withe = oracle.compare(g, Cref, T, out_is_bf16, E)
        res.update(max_ratio=withe["max_ratio"], n_bad=withe["n_bad"],
                   first_bad=withe["first_bad"])
    st = PLAIN_STATS.setdefault(_caller_file(), {"elements": 0, "beyond_plain": 0,
                                                 "worst_plain_ratio": 0.0, "group_term": False})
    st["elements"] += int(np.asarray(g).size)
    st["beyond_plain"] += plain["n_bad"]
    st["worst_plain_ratio"] = max(st["worst_plain_ratio"], plain["max_ratio"])
    st["group_term"] |= bool(group_term)
    log("  %s: worst err/plain bound %.3g, %d elements beyond it%s" % (
        what, plain["max_ratio"], plain["n_bad"],
        (", worst with E %.3g" % res["max_ratio"]) if group_term else ""))
    return res


def check_against_oracle(case, out_dtype, rows=None, C=None, tile=None, split_k=0,
                         group_term=False, what=""):
    """Run (or take) the GPU result and compare rows with the oracle under
    acceptance() (the plain bound unless group_term)."""
    if C is None:
        C = run_gpu(case, out_dtype, tile=tile, split_k=split_k)
    g = host64(C)
    eight_bit = case["fmt"] in (mxinputs.FMT_E4M3, mxinputs.FMT_E5M2)
    out = oracle.gemm(case["fmt"], case["A"], case["A_scale"], case["B"],
                      case["B_scale"], case["K"], rows=rows, group_bound=eight_bit)
    Cref, T = out[0], out[1]
    E = out[2] if eight_bit else None
    if rows is not None:
        g = g[np.asarray(rows)]
    res = acceptance(g, Cref, T, out_dtype == mxinputs.OUT_BF16, E, group_term, what)
    return res, g, Cref, T, E


def sample_rows(M, tile=256, n=64):
    """Deterministic row sample: the first and last tile's edges and an even
    spread in between."""
    if M <= n:
        return list(range(M))
    rows = set(range(8)) | set(range(M - 8, M))
    last_tile = (M - 1) // tile * tile
    rows |= set(range(last_tile, min(M, last_tile + 8)))
    rows |= set(int(x) for x in np.linspace(0, M - 1, max(0, n - len(rows))))
    return sorted(rows)
