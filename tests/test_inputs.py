"""The seeded input generator and its OCP-MX quantizer (CPU only).

The encoders are checked against a brute-force nearest-value search over the
decode tables of torch (E4M3) and the golden E2M1 list, with ties going to
the code with an even least significant bit, and saturation at the largest
finite magnitude."""
import math

import numpy as np
import pytest

import mxinputs
import oracle_pins

E2M1, E4M3 = mxinputs.FMT_E2M1, mxinputs.FMT_E4M3


def _brute(v, table, sign_bit):
    finite = [c for c in range(sign_bit) if not math.isnan(table[c])]
    vmax = max(table[c] for c in finite)
    out = []
    for x in v:
        mag = min(abs(float(x)), vmax)
        best = None
        for c in finite:
            d = abs(mag - table[c])
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
                best = (d, c)
        out.append(best[1] | (sign_bit if np.signbit(x) else 0))
    return np.array(out, np.uint8)


def _sweep(table, sign_bit):
    mags = sorted(set(table[c] for c in range(sign_bit) if not math.isnan(table[c])))
    pts = set(mags)
    for a, b in zip(mags, mags[1:]):
        mid = (a + b) / 2
        pts |= {mid, np.nextafter(mid, 0), np.nextafter(mid, 1e9), (a + mid) / 2}
    top = mags[-1]
    pts |= {top * 1.03, top * 1.2, top * 4}
    v = np.array(sorted(pts), np.float32)
    return np.concatenate([v, -v])


def test_encode_e2m1_bruteforce():
    t = oracle_pins.golden_e2m1()
    v = _sweep(t, 8)
    v = np.concatenate([v, np.random.default_rng(0).uniform(-8, 8, 2000).astype(np.float32)])
    assert np.array_equal(mxinputs.encode_e2m1(v), _brute(v, t, 8))


def test_encode_e2m1_ties():
    v = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0], np.float32)
    t = oracle_pins.golden_e2m1()
    got = t[mxinputs.encode_e2m1(v)]
    assert list(got) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0]


def test_encode_e4m3_bruteforce():
    t = oracle_pins.torch_e4m3()
    v = _sweep(t, 128)
    v = np.concatenate([v, np.random.default_rng(1).uniform(-500, 500, 3000).astype(np.float32),
                        np.random.default_rng(2).uniform(-0.02, 0.02, 3000).astype(np.float32)])
    assert np.array_equal(mxinputs.encode_e4m3(v), _brute(v, t, 128))


@pytest.mark.parametrize("fmt", [E2M1, E4M3])
def test_quantize_scale_rule(fmt):
    emax = 2 if fmt == E2M1 else 8
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, 32 * 7)).astype(np.float32)
    x[0, :32] = 0.0                       # all-zero block
    x[1, 32:64] = 0.0
    x[1, 40] = 4.0                        # amax exactly a power of two
    x[2, 64:96] *= 1e-30                  # tiny block
    x[3, 96:128] *= 1e30                  # huge block
    codes, s = mxinputs.quantize(x, fmt)
    for r in range(6):
        for b in range(7):
            amax = float(np.abs(x[r, 32 * b:32 * b + 32]).max())
            if amax == 0:
                assert s[r, b] == 0
            else:
                want = math.floor(math.log2(amax)) - emax + 127
                assert s[r, b] == max(0, min(254, want)), (r, b)
    assert s[1, 1] == 2 - emax + 127


@pytest.mark.parametrize("fmt", [E2M1, E4M3])
def test_quantize_roundtrip_error(fmt):
    """Dequantized values are within half a code spacing of the input, or
    within the saturation gap (2^(emax+1) minus the largest magnitude) where
    the block maximum rounds past the largest code."""
    x = np.random.default_rng(4).standard_normal((8, 256)).astype(np.float32)
    codes, s = mxinputs.quantize(x, fmt)
    deq = oracle_pins.dequant(fmt, codes, s)
    scale = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1)
    top, half_gap, sat = (6.0, 1.0, 2.0) if fmt == E2M1 else (448.0, 16.0, 64.0)
    err = np.abs(deq - x)
    inside = np.abs(x) <= top * scale
    assert np.all(err[inside] <= half_gap * scale[inside])
    assert np.all(err[~inside] <= sat * scale[~inside])


def test_prefix_and_chunk_independence():
    a = mxinputs._gen_quantized(300, 256, E2M1, 9, 0, "outlier")
    b = mxinputs._gen_quantized(40, 256, E2M1, 9, 0, "outlier")
    assert np.array_equal(a[0][:40], b[0]) and np.array_equal(a[1][:40], b[1])


def test_case_shapes():
    c = mxinputs.make_case("mxfp4_256")
    assert c["A"].shape == (256, 128) and c["A_scale"].shape == (256, 8)
    assert c["B"].shape == (256, 128) and c["B_scale"].shape == (256, 8)
    c2 = mxinputs.make_random(E4M3, 3, 5, 128, seed=1)
    assert c2["A"].shape == (3, 128) and c2["B_scale"].shape == (5, 4)


@pytest.mark.parametrize("fmt", [mxinputs.FMT_E2M1, mxinputs.FMT_E4M3, mxinputs.FMT_E5M2],
                         ids=["e2m1", "e4m3", "e5m2"])
def test_generator_quantizer_matches_oracle(orc, fmt):
    """The input generator's numpy quantizer and the oracle's C quantizer are
    two implementations of the same OCP rule: they agree on every byte."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 512)) * np.exp2(rng.integers(-20, 20, (64, 1)))).astype(np.float32)
    x[3, :32] = 0.0
    codes, scales = mxinputs.quantize(x, fmt)
    q, s = orc.quantize(fmt, x.astype(np.float64))
    assert (scales == s).all()
    assert (codes == q).all()
