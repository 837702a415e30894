"""Pins for the underflow-map oracle (CPU only): the E4M3 magnitudes against torch's own float8
decoding, NVFP4 at B = 32 against a brute-force nearest search over exact rationals, the zero
thresholds of each format worked out by hand on a block with maximum 1, and invariances."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.mx import E2M1_GRID
from oracle.underflow import KINDS, e4m3_magnitudes, nvfp4_dequantize, nvfp4_quantize, underflow_map


def test_e4m3_magnitudes_match_torch_float8_decode():
    mags = e4m3_magnitudes()
    ref = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(mags, ref)
    assert mags[-1] == 448.0 and mags[1] == 2.0**-9 and np.all(np.diff(mags) > 0)


def _nearest(t, grid, ties_even=True):
    """Index of the nearest grid value to the rational t; ties to the even index."""
    d = [abs(t - Fraction(g)) for g in grid]
    best = min(d)
    idx = [i for i, v in enumerate(d) if v == best]
    return idx[0] if len(idx) == 1 else [i for i in idx if i % 2 == 0][0]


def test_nvfp4_b32_bruteforce():
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((6, 128)) * np.exp2(rng.integers(-14, 3, (6, 128)))).astype(np.float32)
    x[2, 32:64] *= np.float32(2.0**-20)        # a block whose scale underflows E4M3
    x[4, 64:96] = 0.0                          # an all-zero block
    codes, sc, amax_t = nvfp4_quantize(x)
    T = Fraction(float(np.abs(x).max()))
    assert Fraction(float(amax_t)) == T
    mags = [float(v) for v in e4m3_magnitudes()]
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 32):
            blk = x[r, 32 * b:32 * b + 32]
            amax_b = Fraction(float(np.abs(blk).max()))
            s_idx = _nearest(448 * amax_b / T, mags)
            assert sc[r, b] == s_idx, (r, b)
            s = Fraction(mags[s_idx])
            for i in range(32):
                v = Fraction(float(blk[i]))
                nib = int(codes[r, (32 * b + i) // 2]) >> (4 * ((32 * b + i) & 1)) & 15
                want = 0 if s == 0 else _nearest(abs(v) * 2688 / (s * T), E2M1_GRID)
                assert nib & 7 == want, (r, b, i)
                if want:
                    assert nib >> 3 == (1 if blk[i] < 0 else 0)
    dq = nvfp4_dequantize(codes, sc, amax_t)
    assert np.all(dq[4, 64:96] == 0) and np.all(dq[2, 32:64] == 0)
    # the tensor's largest element is represented exactly (s = 448, element 6)
    r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert dq[r, c] == float(x[r, c])


def _hand_block_rows():
    """One row of blocks with maximum exactly 1 (at elements 0, 8, 16, 24, so every MiX-4.5b
    sub-block has mantissa 0) and probe values around each format's zero threshold."""
    probes = [2.0**-3, np.nextafter(np.float32(2.0**-3), np.float32(1)), 2.0**-4,
              np.nextafter(np.float32(2.0**-4), np.float32(1)), 0.0416, 0.0417, 2.0**-7,
              np.nextafter(np.float32(2.0**-7), np.float32(1)), 2.0**-8,
              np.nextafter(np.float32(2.0**-8), np.float32(1)), 2.0**-9, 2.0**-6]
    vals = [np.float32(p) for p in probes] + [np.float32(-p) for p in probes]
    blocks = []
    for i in range(0, len(vals), 28):
        chunk = vals[i:i + 28]
        chunk += [np.float32(0.5)] * (28 - len(chunk))
        blk, it = [], iter(chunk)
        for e in range(32):
            blk.append(np.float32(1.0) if e % 8 == 0 else next(it))
        blocks += blk
    return np.array([blocks], np.float32), vals


def test_zero_thresholds_worked_by_hand():
    # block max 1: MXINT4 X = 0, zero iff |x| <= 2^-3 (q = RNE(4|x|) = 0); MXFP4 X = -2 under both
    # rules, zero iff |x| <= 0.25 * 2^-2; NVFP4 with amax_T = 1: s = 448, zero iff
    # 2688 |x| <= 0.25 * 448, i.e. |x| <= 1/24; MiX with Emax = 0, M = 1: positives are zero iff
    # |x| <= 2^-8 (half the reclaimed step 2^-7), negatives iff |x| <= 2^-7 (half of 2^-6)
    x, vals = _hand_block_rows()
    got = underflow_map(x).sum(axis=1)

    def count(pred):
        return sum(1 for v in vals if v != 0 and pred(float(v)))

    want = [count(lambda v: abs(v) <= 2.0**-3), count(lambda v: abs(v) <= 2.0**-4),
            count(lambda v: abs(v) <= 2.0**-4), count(lambda v: Fraction(abs(v)) <= Fraction(1, 24)),
            count(lambda v: abs(v) <= (2.0**-8 if v > 0 else 2.0**-7)),
            count(lambda v: abs(v) <= (2.0**-8 if v > 0 else 2.0**-7))]
    assert list(got[:len(KINDS)]) == want
    assert got[-1] == np.count_nonzero(x)


def test_counts_invariant_under_power_of_two_scaling_and_ordered():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-6, 1, (64, 256)))).astype(np.float32)
    x[:, 5] *= 30.0                            # an outlier channel: its blocks turn into dead zones
    base = underflow_map(x)
    for k in (-3, 2):
        assert np.array_equal(underflow_map((x * np.float32(2.0**k)).astype(np.float32)), base)
    tot = base.sum(axis=1)
    # floor exponents are never larger than ceil ones, so the floor rule zeros a subset
    assert tot[1] <= tot[2]
    # a MiX zero is an MXINT4 zero (thresholds M 2^(Emax-8) and M 2^(Emax-7) lie below 2^(Emax-3))
    assert tot[4] <= tot[0] and tot[5] <= tot[0]
    assert np.all(base[:len(KINDS)] <= base[-1])


def test_bf16_input_smoothing_and_zero_inputs():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((16, 64)) + 4.0).astype(np.float32)
    x[3] = 0.0
    mu = x.mean(axis=0).astype(np.float32)
    got = underflow_map(x, mu=mu)
    assert np.array_equal(got, underflow_map((x - mu).astype(np.float32)))
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    xb = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(underflow_map(bits, "bf16"), underflow_map(xb))
    assert np.all(underflow_map(np.zeros((4, 32), np.float32)) == 0)
    with pytest.raises(ValueError):
        underflow_map(np.ones((2, 40), np.float32))
