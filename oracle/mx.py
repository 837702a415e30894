"""MX (shared-exponent) weight quantizers MXINT4 and MXFP4 -- oracle (test infrastructure only).

What it follows:

* P1, 逐图理解论文 (figure walk), the Fig. 4 bit-layout description: MXINT4 and
  MXFP4 blocks of 32 share an 8-bit exponent; each element keeps a 4-bit integer
  or an E2M1 value.
* P1, 关键结果与论文证据 (key results), the MXFP4 bullet, and 阅读时需要注意
  (caveats): the OCP floor rule leaves roughly two fifths of block maxima outside
  the E2M1 range; the paper's MXFP4 always uses the ceil rule instead.
* P1, method overview, the accelerator/quantizer bullet: the MX path shifts each
  element by the difference between the block's largest exponent and its own.
* P1, method overview, last bullet: K-smoothing subtracts the per-channel mean of
  K before coding (the optional ``mu`` operand).

* P1, 实验如何设计 (experiment design), the format bullet: the 4.5-bit tier holds
  "g16" variants of the MX weights, one shared exponent per 16 elements (4 bits per
  element plus 8 per 16 = 4.5 bits); MiX-INT4g16 pairs MiX-4.5b activations with
  MXINT4g16 weights (``block=16`` here; the element rules do not change).

Readings: D8 (X = ceil(log2 amax) - 2 for FP4), D9 (INT4 as OCP-style 1.2
fixed point, symmetric clamp), D10 (RNE, saturating, FP4 keeps the sign of
zero), D11 (zero block, exponent clamps), D15 (smoothing in fp32); a g16 block is
coded exactly as a 32-element block whose other 16 elements are zero.

Pins (tests/test_oracle_mx.py): brute-force nearest grid value with
ties-to-even on tiny blocks; the closed-form decode by enumeration; the ~41.5%
floor statistic for MXFP4 and 0% under ceil; scale bytes against frexp; g16:
brute force on 16-element blocks, equality with the 32-element coding of each
16-element group padded with zeros, and the 4.5-bit accounting.
"""
import numpy as np

from .numerics import as_f32, ceil_log2, floor_log2

BLOCK = 32
BLOCKS = (16, 32)
FORMATS = ("int4", "fp4")
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _check(fmt, x, block):
    if fmt not in FORMATS:
        raise ValueError(f"unknown MX format {fmt!r}")
    if block not in BLOCKS:
        raise ValueError("MX blocks hold 16 or 32 elements")
    if x.ndim != 2 or x.shape[1] % 32 != 0:
        raise ValueError("MX blocks run along the last axis, whose length must be a multiple of 32")


def smooth(x, mu):
    """K-smoothing operand: fp32(x - mu) with mu broadcast along rows (one value per column)."""
    x = np.asarray(x, dtype=np.float32)
    mu = np.asarray(mu, dtype=np.float32)
    if mu.shape != (x.shape[1],):
        raise ValueError("mu must hold one value per column")
    return (x - mu[None, :]).astype(np.float32)


def _rne_grid_index(y):
    """Index into E2M1_GRID of the value nearest |y|, ties to the even index, saturating at 6."""
    a = np.abs(y)[..., None]
    d = np.abs(a - E2M1_GRID)
    first = np.argmin(d, axis=-1)  # lowest index among equal distances
    nxt = np.minimum(first + 1, 7)
    tie = (np.take_along_axis(d, nxt[..., None], axis=-1)[..., 0] == np.take_along_axis(d, first[..., None], axis=-1)[..., 0]) & (nxt != first)
    return np.where(tie & (first % 2 == 1), nxt, first)


def mx_quantize(x, fmt, dtype="f32", mu=None, block=BLOCK, fp4_rule="ceil"):
    """Quantize rows of ``x`` to MX blocks of ``block`` (32, or 16 for the g16 variants) along
    the last axis.

    x: [rows, cols] float32 values or bf16 bit patterns; mu: optional float32 [cols]
    subtracted first in fp32 (K-smoothing). fp4_rule: the MXFP4 shared exponent, "ceil"
    (X = ceil(log2 amax) - 2, the paper's MXFP4) or "floor" (the OCP rule X = floor(log2 amax) - 2,
    which leaves block maxima in (6, 8) * 2^X to saturate; used only as a comparator).
    Returns (codes uint8 [rows, cols/2], scales uint8 [rows, cols/block] as E8M0 = X + 127).
    """
    x = as_f32(x, dtype)
    _check(fmt, x, block)
    if fp4_rule not in ("ceil", "floor"):
        raise ValueError(f"unknown MXFP4 exponent rule {fp4_rule!r}")
    if mu is not None:
        x = smooth(x, mu)
    rows, cols = x.shape
    nb = cols // block
    xb = x.astype(np.float64).reshape(rows, nb, block)
    amax = np.abs(xb).max(axis=2)
    zero = amax == 0.0
    safe = np.where(zero, 1.0, amax)
    if fmt == "fp4":
        X = np.maximum((ceil_log2(safe) if fp4_rule == "ceil" else floor_log2(safe)) - 2, -127)
        y = np.ldexp(xb, -X[:, :, None])
        idx = _rne_grid_index(y)
        nib = (np.signbit(xb).astype(np.int64) << 3) | idx
    else:
        X = np.clip(floor_log2(safe), -125, 127)
        q = np.clip(np.rint(np.ldexp(xb, (2 - X)[:, :, None])), -7, 7).astype(np.int64)
        nib = q & 0xF
    nib = np.where(zero[:, :, None], 0, nib).astype(np.uint8)
    scales = np.where(zero, 0, X + 127).astype(np.uint8)
    flat = nib.reshape(rows, cols)
    codes = (flat[:, 0::2] | (flat[:, 1::2] << 4)).astype(np.uint8)
    return codes, scales


def mx_dequantize(codes, scales, fmt, block=BLOCK):
    """Closed-form decode to float64 [rows, cols] (``block`` elements per scale).

    FP4: (-1)^s * E2M1(idx) * 2^(scale-127). INT4: two's-complement q * 2^(scale-127-2).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    rows = codes.shape[0]
    nib = np.empty((rows, codes.shape[1] * 2), dtype=np.int64)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    cols = nib.shape[1]
    X = np.asarray(scales).astype(np.int64) - 127
    if block not in BLOCKS or X.shape[1] * block != cols:
        raise ValueError("scales do not match the codes for this block size")
    Xe = np.repeat(X, block, axis=1)
    if fmt == "fp4":
        v = np.where(nib & 8, -1.0, 1.0) * E2M1_GRID[nib & 7]
        return np.ldexp(v, Xe).reshape(rows, cols)
    if fmt == "int4":
        q = np.where(nib >= 8, nib - 16, nib).astype(np.float64)
        return np.ldexp(q, Xe - 2).reshape(rows, cols)
    raise ValueError(fmt)
