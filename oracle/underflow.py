"""Underflow ("dead zone") map of the 4-bit block formats -- oracle (test infrastructure only).

What it follows:

* P1, 逐图理解论文 (figure walk), the underflow-map figure: keys of one layer coded with
  32-element blocks in MXINT4, MXFP4, NVFP4 (its block forced from 16 to 32) and MiX; the
  elements that are nonzero but decode to zero are mathematical underflow (the dark regions),
  reported as a fraction per format (44.8%, 38.4%, 38.3% against 23.9% for MiX).
* P1, 关键结果与论文证据 (key results), the MXFP4 bullet: the OCP floor exponent rule against
  the ceil rule, so MXFP4 appears with both.
* P1, 研究缺口 (research gap), the bit-layout figure description: NVFP4 blocks carry E2M1
  elements with an FP8 block scale and an FP32 tensor scale.

Readings (the pages fix none of the arithmetic of the comparators):

* U1 underflow: an element whose input (after the optional smoothing, fp32(x - mu)) is nonzero
  and whose decoded value is zero. Elements that are zero on input are not counted.
* U2 NVFP4 at B = 32: tensor scale g = amax_T / (6 * 448) with amax_T the largest magnitude of
  the whole operand, kept as an exact real; block scale s = the E4M3 value nearest to
  amax_b / (6 g) = 448 amax_b / amax_T (ties to the even code; the quotient never exceeds 448);
  elements = E2M1 value nearest to x / (s g), ties to the even code, saturating at 6; s = 0
  decodes the whole block to zero. Every decision is an exact comparison of products of
  float32 values with small integers, done in fp64 where all of them are exact.
* U3 MXFP4 under both rules (``oracle.mx.mx_quantize(..., fp4_rule=...)``); MXINT4, MiX-4.25b and
  MiX-4.5b as everywhere else.

Pins (tests/test_oracle_underflow.py): the E4M3 magnitudes from the format's bit fields;
NVFP4 against a brute-force nearest search over exact rationals on tiny blocks; thresholds of a
block worked out by hand for every format; invariance of every count under scaling by powers of
two.
"""
import numpy as np

from .mix import mix_dequantize, mix_quantize
from .mx import E2M1_GRID, mx_dequantize, mx_quantize, smooth
from .numerics import as_f32

KINDS = ("mxint4", "mxfp4_floor", "mxfp4_ceil", "nvfp4_b32", "mix_4.25b", "mix_4.5b")
NV_BLOCK = 32
E4M3_MAX = 448.0
E2M1_MAX = 6.0


def e4m3_magnitudes():
    """The 127 finite non-negative E4M3 values in code order (codes 0..126; 127 is NaN).

    Bit fields: 4 exponent bits (bias 7) and 3 mantissa bits; exponent field 0 holds the
    subnormals m * 2^-9, field e > 0 holds (1 + m/8) * 2^(e - 7).
    """
    v = []
    for c in range(127):
        e, m = c >> 3, c & 7
        v.append(np.ldexp(float(m), -9) if e == 0 else np.ldexp(1.0 + m / 8.0, e - 7))
    return np.array(v, dtype=np.float64)


def _rne_index(lhs, mids, rhs_scale):
    """Index of the nearest grid value to lhs / rhs_scale for a grid whose midpoints are ``mids``
    (ascending, the midpoint between entries k and k+1), ties to the even index.

    The comparisons lhs > mids[k] * rhs_scale are exact: both sides are exact fp64 products.
    lhs, rhs_scale: arrays broadcast against each other; returns int64 of their shape.
    """
    lhs = np.asarray(lhs, dtype=np.float64)[..., None]
    rhs = np.asarray(rhs_scale, dtype=np.float64)[..., None] * mids
    above = lhs > rhs
    tie_up = (lhs == rhs) & ((np.arange(1, len(mids) + 1) % 2) == 0)
    return (above | tie_up).sum(axis=-1).astype(np.int64)


def nvfp4_quantize(x, dtype="f32", mu=None, block=NV_BLOCK):
    """NVFP4 with ``block`` elements per E4M3 scale (U2).

    Returns (codes uint8 [rows, cols/2] E2M1 nibbles sign<<3 | index, scale codes uint8
    [rows, cols/block] E4M3, amax_T float32).
    """
    x = as_f32(x, dtype)
    if mu is not None:
        x = smooth(x, mu)
    rows, cols = x.shape
    if cols % block:
        raise ValueError("cols must be a multiple of the block")
    amax_t = np.float32(np.abs(x).max()) if x.size else np.float32(0.0)
    xb = x.astype(np.float64).reshape(rows, cols // block, block)
    amax_b = np.abs(xb).max(axis=2)
    mags = e4m3_magnitudes()
    e4_mids = (mags[:-1] + mags[1:]) / 2.0
    T = float(amax_t)
    # s = nearest E4M3 to 448 amax_b / amax_T: compare 448 amax_b with mid * amax_T
    sc = _rne_index(448.0 * amax_b, e4_mids, np.full_like(amax_b, T)) if T > 0 else np.zeros_like(amax_b, np.int64)
    s = mags[sc]
    # element: nearest E2M1 to x / (s g) = 2688 x / (s amax_T): compare 2688 |x| with mid * s * amax_T
    e2_mids = (E2M1_GRID[:-1] + E2M1_GRID[1:]) / 2.0
    idx = _rne_index(2688.0 * np.abs(xb), e2_mids, (s * T)[:, :, None])
    idx = np.where((s == 0.0)[:, :, None], 0, idx)
    nib = (np.signbit(xb).astype(np.int64) << 3) | idx
    flat = nib.reshape(rows, cols).astype(np.uint8)
    codes = (flat[:, 0::2] | (flat[:, 1::2] << 4)).astype(np.uint8)
    return codes, sc.astype(np.uint8), amax_t


def nvfp4_dequantize(codes, scale_codes, amax_t, block=NV_BLOCK):
    """Decode: (-1)^s * E2M1(idx) * s_b * amax_T / 2688, float64 [rows, cols]."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows = codes.shape[0]
    nib = np.empty((rows, codes.shape[1] * 2), dtype=np.int64)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    s = np.repeat(e4m3_magnitudes()[np.asarray(scale_codes, dtype=np.int64)], block, axis=1)
    v = np.where(nib & 8, -1.0, 1.0) * E2M1_GRID[nib & 7]
    return v * s * (float(amax_t) / (6.0 * E4M3_MAX))


def decoded(x, kind, dtype="f32", mu=None):
    """Decoded values (float64 [rows, cols]) of the operand in one of KINDS."""
    if kind == "mxint4":
        return mx_dequantize(*mx_quantize(x, "int4", dtype, mu), "int4")
    if kind in ("mxfp4_floor", "mxfp4_ceil"):
        rule = kind.split("_")[1]
        return mx_dequantize(*mx_quantize(x, "fp4", dtype, mu, fp4_rule=rule), "fp4")
    if kind == "nvfp4_b32":
        return nvfp4_dequantize(*nvfp4_quantize(x, dtype, mu))
    if kind in ("mix_4.25b", "mix_4.5b"):
        fmt = kind.split("_")[1]
        xs = as_f32(x, dtype)
        if mu is not None:
            xs = smooth(xs, mu)
        return mix_dequantize(*mix_quantize(xs, fmt, "f32"), fmt)
    raise ValueError(f"unknown kind {kind!r}")


def underflow_map(x, dtype="f32", mu=None):
    """Per-column underflow counts (U1): int64 [len(KINDS) + 1, cols]; row i counts, for format
    KINDS[i], the elements of each column that are nonzero on input and decode to zero; the last
    row counts the nonzero input elements of each column."""
    xs = as_f32(x, dtype)
    if mu is not None:
        xs = smooth(xs, mu)
    nz = xs != 0.0
    out = [((decoded(xs, k) == 0.0) & nz).sum(axis=0) for k in KINDS]
    out.append(nz.sum(axis=0))
    return np.stack(out).astype(np.int64)
