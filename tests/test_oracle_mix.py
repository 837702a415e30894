"""Pins for the MiX oracle (CPU only).

Each test checks the oracle against something other than itself: the bit counts
the pages print, IEEE-754 bit patterns built by hand, a brute-force nearest-code
search over all 16 nibbles, and the reconstruction of the block maximum.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.mix import mix_dequantize, mix_quantize, storage_bits_per_block


# ---------------------------------------------------------------- independent decode

def _f32_from_fields(sign, exp_unbiased, mant3):
    """The float (-1)^sign * 1.mant3 * 2^exp built from IEEE-754 single-precision fields."""
    bits = (sign << 31) | ((exp_unbiased + 127) << 23) | (mant3 << 20)
    return struct.unpack("<f", struct.pack("<I", bits))[0]


def _code_value(nib, emax, m):
    """Value of one nibble for block fields (emax, m), built through IEEE fields, not the oracle."""
    s, de = nib >> 3, nib & 7
    if nib == 0x7:
        return 0.0
    if nib == 0xF:
        return _f32_from_fields(0, emax - 7, m)
    return _f32_from_fields(s, emax - de, m)


def _nearest_code(x, emax, m):
    """Brute force over all 16 nibbles: nearest value (exact rational distances), ties to the
    smaller magnitude."""
    best = None
    xf = Fraction(x)
    for nib in range(16):
        v = _code_value(nib, emax, m)
        key = (abs(xf - Fraction(v)), abs(v))
        if best is None or key < best[0]:
            best = (key, nib)
    return best[1]


def _fields(shared, fmt, b):
    s = int(shared[b])
    emax = (s & 15) - 7
    if fmt == "4.25b":
        return emax, [(s >> 4) & 7] * 4
    return emax, [(s >> (4 + 3 * k)) & 7 for k in range(4)]


def _nibbles(codes):
    out = []
    for byte in codes:
        out += [int(byte) & 15, int(byte) >> 4]
    return out


# ---------------------------------------------------------------- bit accounting

def test_bit_accounting_matches_pages():
    # P1 method overview: (8 + 128) / 32 = 4.25 and 4 + 4*3 + 32*4 = 144 bits = 4.5 bit/element.
    assert storage_bits_per_block("4.25b") == 136
    assert storage_bits_per_block("4.25b") / 32 == 4.25
    assert storage_bits_per_block("4.5b") == 144
    assert storage_bits_per_block("4.5b") / 32 == 4.5
    x = np.ones((3, 96), np.float32)
    for fmt, bits in (("4.25b", 136), ("4.5b", 144)):
        c, s = mix_quantize(x, fmt)
        assert (c.nbytes + s.nbytes) * 8 == bits * 3 * 3


# ---------------------------------------------------------------- decode closed form via IEEE fields

@pytest.mark.parametrize("fmt", ["4.25b", "4.5b"])
def test_decode_matches_ieee_fields_exhaustive(fmt):
    # every Emax code x every mantissa x every nibble
    for ecode in range(16):
        for m in range(8):
            shared = ecode | (m << 4) if fmt == "4.25b" else ecode | sum(m << (4 + 3 * k) for k in range(4))
            codes = np.array([[n | ((15 - n) << 4) for n in range(16)]], np.uint8)  # 32 nibbles
            sh = np.array([[shared]], np.uint8 if fmt == "4.25b" else np.uint16)
            val = mix_dequantize(codes, sh, fmt)[0]
            nibs = _nibbles(codes[0])
            for i, nib in enumerate(nibs):
                assert val[i] == _code_value(nib, ecode - 7, m), (ecode, m, nib)


def test_decode_value_set_properties():
    # 16 codes -> 16 distinct values; 0x7 is the only zero; positives reach one binade lower (0xF).
    for emax in (-7, 0, 8):
        for m in range(8):
            vals = [_code_value(n, emax, m) for n in range(16)]
            assert len(set(vals)) == 16
            assert vals[0x7] == 0.0
            pos = sorted(v for v in vals if v > 0)
            neg = sorted(-v for v in vals if v < 0)
            assert len(pos) == 8 and len(neg) == 7
            assert pos[0] == neg[0] / 2  # the reclaimed step
            ratios = {pos[i + 1] / pos[i] for i in range(7)}
            assert ratios == {2.0}


# ---------------------------------------------------------------- Emax / mshared (Algorithm 1, first steps)

def _rand_blocks(rng, nblk, spread=12):
    x = rng.standard_normal((nblk, 32)) * np.exp2(rng.integers(-spread, spread, size=(nblk, 32)))
    return x.astype(np.float32)


@pytest.mark.parametrize("fmt", ["4.25b", "4.5b"])
def test_emax_and_mantissa_from_block_max(fmt):
    rng = np.random.default_rng(7)
    x = _rand_blocks(rng, 400, spread=5)
    codes, shared = mix_quantize(x, fmt)
    for b in range(x.shape[0]):
        emax, ms = _fields(shared[:, 0], fmt, b)
        amax = float(np.max(np.abs(x[b].astype(np.float64))))
        f, e = math.frexp(amax)
        assert emax == min(max(e - 1, -7), 8)
        nibs = _nibbles(codes[b])
        subs = [range(32)] if fmt == "4.25b" else [range(8 * k, 8 * k + 8) for k in range(4)]
        for k, sub in enumerate(subs):
            i = max(sub, key=lambda j: abs(float(x[b, j])))
            xm = abs(float(x[b, i]))
            fm, em = math.frexp(xm)
            assert ms[k] == int((2 * fm - 1) * 8)  # top three fraction bits of the max (D3)
            # the (sub-)block max reconstructs from below within one mantissa step
            v = abs(_code_value(nibs[i], emax, ms[k]))
            if -7 <= em - 1 <= emax and emax - (em - 1) <= 6:
                assert v <= xm < v * (1 + 1 / (8 + ms[k])) + 1e-300


# ---------------------------------------------------------------- refinement = nearest code

@pytest.mark.parametrize("fmt", ["4.25b", "4.5b"])
def test_quantizer_equals_bruteforce_random(fmt):
    rng = np.random.default_rng(11)
    x = _rand_blocks(rng, 300)
    codes, shared = mix_quantize(x, fmt)
    for b in range(x.shape[0]):
        emax, ms = _fields(shared[:, 0], fmt, b)
        nibs = _nibbles(codes[b])
        for i in range(32):
            assert nibs[i] == _nearest_code(float(x[b, i]), emax, ms[i // 8]), (b, i)


@settings(max_examples=150, deadline=None)
@given(st.lists(st.floats(min_value=-1e4, max_value=1e4, allow_nan=False, width=32), min_size=32, max_size=32),
       st.sampled_from(["4.25b", "4.5b"]))
def test_quantizer_equals_bruteforce_hypothesis(vals, fmt):
    x = np.array([vals], np.float32)
    codes, shared = mix_quantize(x, fmt)
    emax, ms = _fields(shared[:, 0], fmt, 0)
    nibs = _nibbles(codes[0])
    for i in range(32):
        assert nibs[i] == _nearest_code(float(x[0, i]), emax, ms[i // 8])


@pytest.mark.parametrize("m", range(8))
@pytest.mark.parametrize("emax", [-7, -3, 0, 5, 8])
def test_exhaustive_bf16_sweep(emax, m):
    # Element 0 fixes the block's Emax and mantissa; the other 31 sweep every finite bf16 pattern
    # that does not exceed it. Every element must take the brute-force nearest code.
    top = _f32_from_fields(0, emax, m) * (1 + 1 / 32)  # 1.m + 1/32 ulp keeps the truncated mantissa m
    pats = np.arange(65536, dtype=np.uint32)
    vals = (pats << 16).view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= top)]
    n = -(-len(vals) // 31)
    body = np.zeros(n * 31, np.float32)
    body[: len(vals)] = vals
    x = np.concatenate([np.full((n, 1), top, np.float32), body.reshape(n, 31)], axis=1)
    codes, shared = mix_quantize(x, "4.25b")
    assert np.all(shared == ((emax + 7) | (m << 4)))
    # vectorised brute force over the 16 codes (values via IEEE fields)
    table = np.array([_code_value(c, emax, m) for c in range(16)], np.float64)
    xx = x.astype(np.float64)[:, :, None]
    err = np.abs(xx - table[None, None, :])  # exact here: |x| <= top keeps every difference in 30 bits
    best = np.argmin(err, axis=2)
    # resolve exact ties toward the smaller magnitude
    minerr = np.take_along_axis(err, best[:, :, None], axis=2)
    tied = err == minerr
    mag = np.where(tied, np.abs(table)[None, None, :], np.inf)
    best = np.argmin(mag, axis=2)
    nib = np.empty((n, 32), np.int64)
    nib[:, 0::2] = codes & 15
    nib[:, 1::2] = codes >> 4
    assert np.array_equal(nib, best)


# ---------------------------------------------------------------- special cases

@pytest.mark.parametrize("fmt", ["4.25b", "4.5b"])
def test_zero_block(fmt):
    x = np.zeros((2, 64), np.float32)
    x[1, :32] = -0.0
    codes, shared = mix_quantize(x, fmt)
    assert np.all(codes == 0x77) and np.all(shared == 0)
    assert np.all(mix_dequantize(codes, shared, fmt) == 0.0)


def test_asymmetric_zero_and_ties():
    M = 1.25  # m = 2
    base = [M * 2.0**3] + [0.0] * 31  # Emax = 3
    x = np.array([base], np.float32)
    # positive midpoint between 0 and M*2^(3-7): tie -> zero; just above -> 0xF
    x[0, 1] = M * 2.0 ** (3 - 8)
    x[0, 2] = np.nextafter(np.float32(M * 2.0 ** (3 - 8)), np.float32(1))
    # -M*2^(3-7) is the midpoint of 0 and -M*2^(3-6) (negatives stop at dE = 6)
    x[0, 3] = -np.float32(M * 2.0 ** (3 - 7))
    # midpoint between M*2^(3-7) and M*2^(3-6) for positives: tie -> the smaller (0xF)
    x[0, 4] = 1.5 * M * 2.0 ** (3 - 7)
    # midpoint between M*2^1 and M*2^2: tie -> smaller magnitude (dE = 2)
    x[0, 5] = 1.5 * M * 2.0**1
    x[0, 6] = -1.5 * M * 2.0**1
    codes, shared = mix_quantize(x, "4.25b")
    nib = _nibbles(codes[0])
    assert shared[0, 0] == (3 + 7) | (2 << 4)
    assert nib[0] == 0x0
    assert nib[1] == 0x7 and nib[2] == 0xF
    assert nib[3] == 0x7  # the midpoint of 0 and -M*2^(3-6): tie -> zero
    assert nib[4] == 0xF
    assert nib[5] == 0x2 and nib[6] == 0xA


def test_negative_tie_goes_to_zero():
    M = 1.25
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = M * 8.0
    x[0, 1] = -M * 2.0 ** (3 - 7)  # exactly half of the smallest negative magnitude M*2^(3-6)
    codes, _ = mix_quantize(x, "4.25b")
    assert _nibbles(codes[0])[1] == 0x7


def test_saturation_above_range():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1000.0  # 2^9 * 1.95: Emax clamps to 8, mantissa 7
    x[0, 1] = -700.0
    codes, shared = mix_quantize(x, "4.25b")
    assert shared[0, 0] == 15 | (7 << 4)
    d = mix_dequantize(codes, shared, "4.25b")[0]
    assert d[0] == 480.0 and d[1] == -480.0


def test_below_range_and_subnormal():
    x = np.zeros((2, 32), np.float32)
    x[0, 0] = 2.0**-10 * 1.5  # block max below 2^-7 -> Emax = -7
    x[0, 1] = 2.0**-15
    x[1, 0] = np.float32(1e-40)  # subnormal block max
    codes, shared = mix_quantize(x, "4.25b")
    assert (shared[0, 0] & 15) == 0 and (shared[1, 0] & 15) == 0
    d = mix_dequantize(codes, shared, "4.25b")
    assert d[0, 0] == _nearest_value(float(x[0, 0]), -7, (shared[0, 0] >> 4) & 7)
    assert np.all(d[1] == 0.0)
    f, e = math.frexp(float(np.float32(1e-40)))
    assert (shared[1, 0] >> 4) & 7 == int((2 * f - 1) * 8)


def _nearest_value(x, emax, m):
    return _code_value(_nearest_code(x, emax, int(m)), emax, int(m))


def test_bf16_input_equals_f32_input():
    rng = np.random.default_rng(3)
    x = _rand_blocks(rng, 64)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    xt = (bits.astype(np.uint32) << 16).view(np.float32)
    for fmt in ("4.25b", "4.5b"):
        a = mix_quantize(bits, fmt, "bf16")
        b = mix_quantize(xt, fmt, "f32")
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rejects_bad_shapes_and_nonfinite():
    with pytest.raises(ValueError):
        mix_quantize(np.ones((2, 33), np.float32), "4.5b")
    with pytest.raises(ValueError):
        mix_quantize(np.full((1, 32), np.inf, np.float32), "4.5b")
    with pytest.raises(ValueError):
        mix_quantize(np.ones((1, 32), np.float32), "5b")


@pytest.mark.parametrize("fmt", ["4.25b", "4.5b"])
def test_far_above_range_saturates_to_nearest(fmt):
    # A block whose maximum is far above 2^9 clamps Emax to 8; its elements take the nearest of the
    # representable values, which for huge magnitudes is the largest one, never zero.
    x = np.zeros((1, 32), np.float32)
    x[0, :8] = [1e30, -3e38, 5e20, 1e10, 700.0, -1e6, 3.0, -2.0**-20]
    x[0, 8:16] = [2.0e36, 1e-30, -1e-10, 0.5, 96.0, -65536.0, 1e3, 3e38]
    codes, shared = mix_quantize(x, fmt)
    emax, ms = _fields(shared[:, 0], fmt, 0)
    assert emax == 8
    nibs = _nibbles(codes[0])
    for i in range(32):
        assert nibs[i] == _nearest_code(float(x[0, i]), emax, ms[i // 8]), i
    assert nibs[0] == 0x0 and nibs[1] == 0x8
