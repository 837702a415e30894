"""MiX (Micro-Inverted-Scaling) quantizer and decoder -- oracle (test infrastructure only).

What it follows (P1 = the pchao.org digest, see ``oracle/__init__.py``):

* Formats -- P1, section 方法概览 (method overview), the MiX-4.25b and MiX-4.5b
  bullets, and the Fig. 4 bit-layout description in 逐图理解论文 (figure walk):
  a 32-element block carries a 4-bit Emax and a 3-bit shared mantissa with an
  implicit leading one; each element carries a sign bit and a 3-bit relative
  exponent dE; the value is (-1)^s * (1.m)_2 * 2^(Emax - dE); dE = 7 is zero.
  MiX-4.5b keeps one Emax but splits the block into four 8-element sub-blocks,
  each with its own 3-bit mantissa.
* Quantizer -- P1, method overview, the Algorithm 1 bullet: Emax from the block's
  largest magnitude; the shared mantissa from that largest element (not a mean
  or an MSE fit); a naive dE = Emax - floor(log2|x|); then the best of
  {dE-1, dE, dE+1} by reconstruction error.
* Asymmetric zero -- P1, method overview, the accelerator/quantizer bullet: the
  negative-zero pattern is reused as one more positive step.

Readings of what the pages leave open: D1 (Emax bias 7, range [-7, 8]), D2, D3
(mantissa truncated to 3 bits), D4 (shared-field layout), D5 (0x7 = 0,
0xF = +M*2^(Emax-7)), D6 (nibble order), D7 (nearest value, ties to the
smaller magnitude), D11 (all-zero block).

Pins (tests/test_oracle_mix.py): bit accounting; the dequantisation closed form
by enumeration; brute-force nearest code over all 16 nibbles on random and
exhaustive inputs; the max element's own reconstruction; zero/asymmetric codes.
"""
import numpy as np

from .numerics import as_f32, floor_log2, significand

BLOCK = 32
SUB = 8
FORMATS = ("4.25b", "4.5b")
EMAX_MIN, EMAX_MAX = -7, 8  # D1: 4-bit field, bias 7


def storage_bits_per_block(fmt):
    """Bits one 32-element block occupies in memory (P1, MiX-4.25b / MiX-4.5b bullets).

    4.25b: a 4-bit Emax and one 3-bit mantissa, padded to an 8-bit field, plus
    32 four-bit element codes. 4.5b: the 4-bit Emax, four 3-bit mantissas and 32
    element codes, with no padding.
    """
    if fmt == "4.25b":
        return 8 + BLOCK * 4
    if fmt == "4.5b":
        return 4 + 4 * 3 + BLOCK * 4
    raise ValueError(fmt)


def _check(fmt, x):
    if fmt not in FORMATS:
        raise ValueError(f"unknown MiX format {fmt!r}")
    if x.ndim != 2 or x.shape[1] % BLOCK != 0:
        raise ValueError("MiX blocks run along the last axis, whose length must be a multiple of 32")


def _exact_abs_diff(x, v):
    """|x - v| as an unevaluated pair (hi, lo) with hi = fl(|x - v|), exactly (TwoSum).

    Pairs compare exactly in lexicographic order; v = +inf gives (inf, nan), which never wins.
    """
    with np.errstate(invalid="ignore"):
        s = x - v
        bb = s - x
        e = (x - (s - bb)) + (-v - bb)
        sign = np.where(s < 0, -1.0, 1.0)
        return np.abs(s), sign * e


def mix_quantize(x, fmt, dtype="f32"):
    """Quantize rows of ``x`` to MiX codes, following Algorithm 1 step by step.

    x: [rows, cols] float32 values (``dtype='f32'``) or bf16 bit patterns
    (``dtype='bf16'``); cols % 32 == 0.
    Returns (codes uint8 [rows, cols/2], shared uint8|uint16 [rows, cols/32]).
    """
    x = as_f32(x, dtype)
    _check(fmt, x)
    rows, cols = x.shape
    nb = cols // BLOCK
    xb = x.astype(np.float64).reshape(rows, nb, BLOCK)
    ax = np.abs(xb)

    # Step 1: Emax from the block's largest magnitude (D1 clamp; zero block -> Emax code 0).
    amax = ax.max(axis=2)
    blk_zero = amax == 0.0
    emax = np.where(blk_zero, EMAX_MIN, np.clip(floor_log2(np.where(blk_zero, 1.0, amax)), EMAX_MIN, EMAX_MAX))

    # Step 2: the shared mantissa from the largest element of the block (4.25b) or of each
    # 8-element sub-block (4.5b), truncated to 3 fraction bits (D2, D3). Zero (sub-)block -> 0.
    if fmt == "4.25b":
        smax = amax[:, :, None]  # [rows, nb, 1]
    else:
        smax = ax.reshape(rows, nb, BLOCK // SUB, SUB).max(axis=3)  # [rows, nb, 4]
    sub_zero = smax == 0.0
    mant = np.where(sub_zero, 0, np.floor(8.0 * (significand(np.where(sub_zero, 1.0, smax)) - 1.0))).astype(np.int64)
    if fmt == "4.25b":
        m_elem = np.broadcast_to(mant, (rows, nb, BLOCK))
    else:
        m_elem = np.repeat(mant, SUB, axis=2)  # element e belongs to sub-block e // 8
    M = 1.0 + m_elem / 8.0
    E = emax[:, :, None]

    # Step 3: naive relative exponent dE = Emax - floor(log2|x|) (zero elements: far below range).
    nz = ax > 0.0
    de_naive = np.where(nz, E - floor_log2(np.where(nz, ax, 1.0)), 1 << 20)

    # Step 4: refinement -- the best of {dE-1, dE, dE+1}, clamped to the codes a sign can use, with
    # zero and (for x > 0) the reclaimed dE = 7 step as further candidates (D5, D7).
    # Candidates are listed by increasing magnitude so that argmin picks the smaller one on a tie.
    pos = xb > 0.0
    sgn = np.where(xb < 0.0, -1.0, 1.0)
    cands_de = [np.clip(de_naive + 1, 0, 6), np.clip(de_naive, 0, 6), np.clip(de_naive - 1, 0, 6)]
    values = [np.zeros_like(xb), np.where(pos, M * np.ldexp(1.0, E - 7), np.inf)]
    values += [sgn * M * np.ldexp(1.0, E - d) for d in cands_de]
    # Reconstruction error |x - v| compared exactly: fp64 subtraction alone can round two
    # different distances to one value when |x| is far above the block's range (saturation).
    pick = np.zeros(xb.shape, np.int64)  # first minimum = smallest magnitude on a tie
    best_hi, best_lo = _exact_abs_diff(xb, values[0])
    for c in range(1, len(values)):
        hi, lo = _exact_abs_diff(xb, values[c])
        better = (hi < best_hi) | ((hi == best_hi) & (lo < best_lo))
        pick = np.where(better, c, pick)
        best_hi = np.where(better, hi, best_hi)
        best_lo = np.where(better, lo, best_lo)

    de_pick = np.choose(np.clip(pick - 2, 0, 2), cands_de)
    nib = np.where(xb < 0.0, 8, 0) | de_pick
    nib = np.where(pick == 0, 0x7, nib)
    nib = np.where(pick == 1, 0xF, nib).astype(np.uint8)

    flat = nib.reshape(rows, cols)
    codes = (flat[:, 0::2] | (flat[:, 1::2] << 4)).astype(np.uint8)

    ecode = (emax + 7).astype(np.uint32)
    if fmt == "4.25b":
        shared = (ecode | (mant[:, :, 0].astype(np.uint32) << 4)).astype(np.uint8)
    else:
        shared = ecode.copy()
        for k in range(4):
            shared |= mant[:, :, k].astype(np.uint32) << (4 + 3 * k)
        shared = shared.astype(np.uint16)
    return codes, shared


def unpack_nibbles(codes):
    """uint8 [rows, n] -> uint8 [rows, 2n]; element 2j is the low nibble of byte j (D6)."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = codes & 0xF
    out[..., 1::2] = codes >> 4
    return out


def split_shared(shared, fmt):
    """Shared field -> (Emax int64 [rows, nb], mantissas int64 [rows, nb, 4]) per D4."""
    s = np.asarray(shared).astype(np.int64)
    emax = (s & 0xF) - 7
    if fmt == "4.25b":
        m = np.repeat(((s >> 4) & 7)[:, :, None], 4, axis=2)
    elif fmt == "4.5b":
        m = np.stack([(s >> (4 + 3 * k)) & 7 for k in range(4)], axis=2)
    else:
        raise ValueError(fmt)
    return emax, m


def mix_dequantize(codes, shared, fmt):
    """Closed-form decode: (-1)^s * (1 + m/8) * 2^(Emax - dE); 0x7 -> 0; 0xF -> +(1+m/8)*2^(Emax-7).

    Returns float64 [rows, cols].
    """
    nib = unpack_nibbles(codes).astype(np.int64)
    rows, cols = nib.shape
    nb = cols // BLOCK
    emax, m = split_shared(shared, fmt)
    nibb = nib.reshape(rows, nb, 4, SUB)
    M = (1.0 + m / 8.0)[:, :, :, None]
    E = emax[:, :, None, None]
    s = nibb >> 3
    de = nibb & 7
    val = np.where(s == 1, -1.0, 1.0) * M * np.ldexp(1.0, E - de)
    val = np.where(nibb == 0x7, 0.0, val)
    val = np.where(nibb == 0xF, M * np.ldexp(1.0, E - 7), val)
    return val.reshape(rows, cols)
