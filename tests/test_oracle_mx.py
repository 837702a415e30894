"""Pins for the MX oracle (CPU only): the E2M1 table from its bit fields, brute-force nearest grid
value with ties to even, the ceil-vs-floor statistic the pages report, and the smoothing operand."""
import math

import numpy as np
import pytest

from oracle.mx import mx_dequantize, mx_quantize


def _e2m1_from_fields(code):
    """OCP E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent field 0 is subnormal."""
    s, e, m = code >> 3, (code >> 1) & 3, code & 1
    mag = (m * 0.5) if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
    return -mag if s else mag


def _nibbles(row):
    out = []
    for b in row:
        out += [int(b) & 15, int(b) >> 4]
    return out


def test_fp4_decode_matches_e2m1_fields():
    codes = np.array([[c | ((15 - c) << 4) for c in range(16)]], np.uint8)
    for sc in (0, 100, 127, 130, 254):
        v = mx_dequantize(codes, np.array([[sc]], np.uint8), "fp4")[0]
        for i, c in enumerate(_nibbles(codes[0])):
            assert v[i] == _e2m1_from_fields(c) * 2.0 ** (sc - 127)


def test_int4_decode_is_twos_complement():
    codes = np.array([[c | ((15 - c) << 4) for c in range(16)]], np.uint8)
    v = mx_dequantize(codes, np.array([[127 + 3]], np.uint8), "int4")[0]
    for i, c in enumerate(_nibbles(codes[0])):
        q = c - 16 if c >= 8 else c
        assert v[i] == q * 2.0 ** (3 - 2)


def _rand(rng, n, spread=10):
    return (rng.standard_normal((n, 32)) * np.exp2(rng.integers(-spread, spread, (n, 32)))).astype(np.float32)


def test_fp4_bruteforce_and_ceil_exponent():
    rng = np.random.default_rng(5)
    x = _rand(rng, 300)
    codes, scales = mx_quantize(x, "fp4")
    for b in range(x.shape[0]):
        amax = float(np.max(np.abs(x[b].astype(np.float64))))
        X = int(scales[b, 0]) - 127
        # ceil variant: the block max lands in (2, 4] after scaling -- never saturates
        assert 2 < amax / 2.0**X <= 4
        assert X == math.ceil(math.log2(amax)) - 2 or amax / 2.0**X == 4
        for i, c in enumerate(_nibbles(codes[b])):
            y = float(x[b, i]) / 2.0**X
            sgn = 1 if math.copysign(1.0, float(x[b, i])) < 0 else 0
            same = [k for k in range(16) if k >> 3 == sgn]
            dist = {k: abs(_e2m1_from_fields(k) - y) for k in same}
            near = [k for k in same if dist[k] == min(dist.values())]
            expect = near[0] if len(near) == 1 else [k for k in near if k % 2 == 0][0]
            assert c == expect, (y, c, near)


def test_int4_bruteforce():
    rng = np.random.default_rng(6)
    x = _rand(rng, 300)
    codes, scales = mx_quantize(x, "int4")
    for b in range(x.shape[0]):
        amax = float(np.max(np.abs(x[b].astype(np.float64))))
        X = int(scales[b, 0]) - 127
        assert 1 <= amax / 2.0**X < 2  # floor exponent
        for i, c in enumerate(_nibbles(codes[b])):
            y = float(x[b, i]) * 2.0 ** (2 - X)
            q = c - 16 if c >= 8 else c
            # nearest integer in [-7, 7], ties to even
            cands = sorted(range(-7, 8), key=lambda t: (abs(t - y), t & 1))
            assert q == cands[0], (y, q)


def test_floor_rule_leaves_two_fifths_of_maxima_unrepresentable():
    # P1 key results: under the OCP floor exponent about 40% of block maxima fall outside E2M1's
    # range (> 6 after scaling); the ceil rule the paper uses leaves none. Closed form for a
    # log-uniform mantissa: log2(8/6) = 0.415.
    rng = np.random.default_rng(1234)
    x = (0.02 * rng.standard_normal((20000, 32))).astype(np.float32)
    codes, scales = mx_quantize(x, "fp4")
    amax = np.abs(x.astype(np.float64)).max(axis=1)
    X_ceil = scales[:, 0].astype(np.int64) - 127
    assert np.all(amax / np.exp2(X_ceil) <= 4.0)
    X_floor = np.floor(np.log2(amax)).astype(np.int64) - 2
    frac = np.mean(amax / np.exp2(X_floor) > 6.0)
    assert abs(frac - math.log2(8 / 6)) < 0.03, frac


def test_zero_block_and_signed_zero():
    x = np.zeros((2, 32), np.float32)
    x[0, 3] = -0.0
    x[1, 0] = 3.0
    x[1, 1] = -0.0
    x[1, 2] = -1e-30  # rounds to zero, keeps its sign in FP4
    for fmt in ("fp4", "int4"):
        codes, scales = mx_quantize(x, fmt)
        assert scales[0, 0] == 0 and np.all(codes[0] == 0)
    codes, scales = mx_quantize(x, "fp4")
    n = _nibbles(codes[1])
    assert n[1] == 0x8 and n[2] == 0x8
    codes, scales = mx_quantize(x, "int4")
    n = _nibbles(codes[1])
    assert n[1] == 0 and n[2] == 0


def test_smoothing_operand_is_fp32_subtraction():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((8, 64)).astype(np.float32) + 3
    mu = rng.standard_normal(64).astype(np.float32)
    a = mx_quantize(x, "fp4", mu=mu)
    b = mx_quantize((x - mu).astype(np.float32), "fp4")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        mx_quantize(np.ones((1, 40), np.float32), "fp4")
    with pytest.raises(ValueError):
        mx_quantize(np.full((1, 32), np.nan, np.float32), "int4")


# ---- g16 variants (one shared exponent per 16 elements)

def test_g16_bruteforce_int4_and_fp4():
    rng = np.random.default_rng(16)
    x = _rand(rng, 200)
    for fmt in ("int4", "fp4"):
        codes, scales = mx_quantize(x, fmt, block=16)
        assert codes.shape == (200, 16) and scales.shape == (200, 2)
        for b in range(x.shape[0]):
            nib = _nibbles(codes[b])
            for h in range(2):
                part = x[b, 16 * h:16 * h + 16].astype(np.float64)
                amax = float(np.max(np.abs(part)))
                X = int(scales[b, h]) - 127
                if fmt == "int4":
                    assert 1 <= amax / 2.0**X < 2
                else:
                    assert 2 < amax / 2.0**X <= 4
                for i in range(16):
                    c = nib[16 * h + i]
                    if fmt == "int4":
                        y = float(part[i]) * 2.0 ** (2 - X)
                        q = c - 16 if c >= 8 else c
                        assert q == sorted(range(-7, 8), key=lambda t: (abs(t - y), t & 1))[0]
                    else:
                        y = float(part[i]) / 2.0**X
                        sgn = 1 if math.copysign(1.0, float(part[i])) < 0 else 0
                        same = [k for k in range(16) if k >> 3 == sgn]
                        dist = {k: abs(_e2m1_from_fields(k) - y) for k in same}
                        near = [k for k in same if dist[k] == min(dist.values())]
                        assert c == (near[0] if len(near) == 1 else [k for k in near if k % 2 == 0][0])


def test_g16_equals_32_block_coding_of_zero_padded_groups():
    # zeros never change a block maximum and code to 0, so each 16-element group coded alone
    # equals the first half of a 32-element block whose second half is zero
    rng = np.random.default_rng(17)
    x = _rand(rng, 64)
    for fmt in ("int4", "fp4"):
        c16, s16 = mx_quantize(x, fmt, block=16)
        pad = np.zeros((64, 64), np.float32)
        pad[:, 0:16], pad[:, 32:48] = x[:, 0:16], x[:, 16:32]
        c32, s32 = mx_quantize(pad, fmt)
        assert np.array_equal(s16, s32)
        assert np.array_equal(c16[:, 0:8], c32[:, 0:8]) and np.array_equal(c16[:, 8:16], c32[:, 16:24])
        assert not c32[:, 8:16].any() and not c32[:, 24:32].any()
        d16 = mx_dequantize(c16, s16, fmt, block=16)
        d32 = mx_dequantize(c32, s32, fmt)
        assert np.array_equal(d16, np.concatenate([d32[:, 0:16], d32[:, 32:48]], axis=1))


def test_g16_bit_accounting():
    # 4-bit elements plus one 8-bit shared exponent per 16 elements: 4.5 bits per element
    x = np.ones((4, 256), np.float32)
    codes, scales = mx_quantize(x, "int4", block=16)
    assert (codes.nbytes + scales.nbytes) * 8 / x.size == 4.5
    codes, scales = mx_quantize(x, "int4")
    assert (codes.nbytes + scales.nbytes) * 8 / x.size == 4.25


def test_fp4_floor_rule_bruteforce_and_saturation():
    # the OCP floor rule (a comparator only): X = floor(log2 amax) - 2, the block max lands in
    # [4, 8) after scaling and saturates to 6 above 6; elements are the nearest E2M1 value, ties
    # to the even code
    rng = np.random.default_rng(15)
    x = _rand(rng, 300)
    codes, scales = mx_quantize(x, "fp4", fp4_rule="floor")
    sat = 0
    for b in range(x.shape[0]):
        amax = float(np.max(np.abs(x[b].astype(np.float64))))
        X = int(scales[b, 0]) - 127
        assert 4 <= amax / 2.0**X < 8
        sat += amax / 2.0**X > 6
        for i, c in enumerate(_nibbles(codes[b])):
            y = float(x[b, i]) / 2.0**X
            sgn = 1 if math.copysign(1.0, float(x[b, i])) < 0 else 0
            same = [k for k in range(16) if k >> 3 == sgn]
            dist = {k: abs(_e2m1_from_fields(k) - y) for k in same}
            near = [k for k in same if dist[k] == min(dist.values())]
            expect = near[0] if len(near) == 1 else [k for k in near if k % 2 == 0][0]
            assert c == expect, (y, c, near)
    assert 0.3 < sat / x.shape[0] < 0.55   # about log2(8/6) of the maxima saturate
    with pytest.raises(ValueError):
        mx_quantize(x, "fp4", fp4_rule="round")
