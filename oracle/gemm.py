"""A-MiX x W-MX matrix product -- oracle (test infrastructure only).

What it follows:

* P1, 方法概览 (method overview), the dual-format bullet and Eq. (6): activations
  are MiX-coded, weights MX-coded; in a block dot product the shared MiX mantissa
  (1.m)_2 and the global exponent factor out of the sum, so each element
  contributes the MX mantissa shifted right by its dE; the block sum is then
  scaled once by the mantissa and once by the exponent. MiX-4.5b keeps one
  partial sum per 8-element sub-block, each multiplied by its own mantissa. The
  MXFP variant adds the FP4 element exponent to the shift.

Two functions:

* ``gemm_ref`` -- the plain definition C = deq(A) . deq(B)^T in fp64 (products of
  dequantised values are exact in fp64; the BLAS sum is within K*2^-53*sum|ab|).
* ``eq6_block_sums`` / ``gemm_exact`` -- Eq. (6) written out in integers: for every
  (row, column, block) T_k = sum_{i in k} s_i * Wint_i * 2^(7 - dE_i),
  blk = sum_k (8 + m_k) * T_k, value = blk * 2^(Emax + X - 10 - c_w), with
  c_w = 2 and Wint = q for MXINT4, c_w = 1 and Wint = 2*E2M1 in {0..12} for
  MXFP4. ``gemm_exact`` adds the block values with Python integers, so it is the
  exact dot product; it is for small shapes only.

Pins (tests/test_oracle_gemm.py): per block, the Eq. (6) value equals the fp64
dot product of the dequantised block exactly; ``gemm_ref`` is within the fp64
error bound of ``gemm_exact``; special cases (identity-like operands) reduce to
sums a reader can check.
"""
from fractions import Fraction

import numpy as np

from .mix import mix_dequantize, split_shared, unpack_nibbles
from .mx import E2M1_GRID, mx_dequantize

BLOCK = 32


def gemm_ref(a_deq, b_deq):
    """C = A . B^T in fp64. a_deq [M, K], b_deq [N, K] (dequantised operands)."""
    return np.asarray(a_deq, np.float64) @ np.asarray(b_deq, np.float64).T


def gemm_ref_entries(a_deq, b_deq, rows, cols):
    """Selected entries C[rows[t], cols[t]] = sum_k A[rows[t], k] * B[cols[t], k] in fp64."""
    a = np.asarray(a_deq, np.float64)[rows]
    b = np.asarray(b_deq, np.float64)[cols]
    return np.einsum("tk,tk->t", a, b)


def gemm_abs_bound(a_deq, b_deq):
    """sum_k |A[i,k]| * |B[j,k]| -- the scale of the fp32 accumulation error bound (D18)."""
    return np.abs(np.asarray(a_deq, np.float64)) @ np.abs(np.asarray(b_deq, np.float64)).T


def _mix_ints(a_codes, a_shared, a_fmt):
    """Per element: s * 2^(7 - dE) as int64 (0 for the zero code, +1 for 0xF), plus Emax and m."""
    nib = unpack_nibbles(a_codes).astype(np.int64)
    rows, cols = nib.shape
    de = nib & 7
    sig = np.where(nib >> 3 == 1, -1, 1)
    sig = np.where(nib == 0x7, 0, sig)
    sig = np.where(nib == 0xF, 1, sig)
    a_int = sig * (1 << (7 - de))
    emax, m = split_shared(a_shared, a_fmt)
    return a_int.reshape(rows, cols // BLOCK, 4, 8), emax, m


def _mx_ints(b_codes, b_scales, b_fmt):
    """Per element the integer MX mantissa Wint, the block exponent X and c_w."""
    codes = np.asarray(b_codes, np.uint8)
    n = codes.shape[0]
    nib = np.empty((n, codes.shape[1] * 2), np.int64)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    if b_fmt == "int4":
        w = np.where(nib >= 8, nib - 16, nib)
        cw = 2
    elif b_fmt == "fp4":
        w = (np.where(nib & 8, -1, 1) * (2 * E2M1_GRID[nib & 7]).astype(np.int64))
        cw = 1
    else:
        raise ValueError(b_fmt)
    X = np.asarray(b_scales).astype(np.int64) - 127
    return w.reshape(n, -1, 4, 8), X, cw


def eq6_block_sums(a_codes, a_shared, a_fmt, b_codes, b_scales, b_fmt):
    """Eq. (6) per (row i, column j, block b): integer blk[i,j,b] and exponent e[i,j,b].

    The block's dot product equals blk * 2**e exactly. |blk| < 2**21.
    """
    a_int, emax, m = _mix_ints(a_codes, a_shared, a_fmt)
    w_int, X, cw = _mx_ints(b_codes, b_scales, b_fmt)
    # T_k: integer shift-add over each 8-element sub-block
    T = np.einsum("ibke,jbke->ijbk", a_int, w_int)
    blk = np.einsum("ibk,ijbk->ijb", 8 + m, T)
    e = emax[:, None, :] + X[None, :, :] - 10 - cw
    return blk, e


def gemm_exact(a_codes, a_shared, a_fmt, b_codes, b_scales, b_fmt):
    """Exact A-MiX x W-MX product, summing the Eq. (6) block values as rationals.

    Returns (fp64 nearest value [M, N], list of Fractions row-major). Small shapes only.
    """
    blk, e = eq6_block_sums(a_codes, a_shared, a_fmt, b_codes, b_scales, b_fmt)
    M, N, nb = blk.shape
    out = np.empty((M, N), np.float64)
    exact = []
    for i in range(M):
        for j in range(N):
            ee = e[i, j]
            base = int(ee.min())
            tot = 0
            for b in range(nb):
                tot += int(blk[i, j, b]) << int(ee[b] - base)
            fr = Fraction(tot) * (Fraction(2) ** base)
            exact.append(fr)
            out[i, j] = float(fr)  # Fraction -> float rounds to nearest
    return out, exact


def dequant_a(a_codes, a_shared, a_fmt):
    return mix_dequantize(a_codes, a_shared, a_fmt)


def dequant_b(b_codes, b_scales, b_fmt):
    return mx_dequantize(b_codes, b_scales, b_fmt)
