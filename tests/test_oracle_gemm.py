"""Pins for the GEMM oracle (CPU only): the Eq. (6) identity per block, the fp64 reference against
the exact rational product, and operands that reduce the product to a selection a reader can check."""
from fractions import Fraction

import numpy as np
import pytest

from oracle.gemm import eq6_block_sums, gemm_exact, gemm_ref, gemm_ref_entries
from oracle.mix import mix_dequantize, mix_quantize
from oracle.mx import mx_dequantize, mx_quantize

PAIRS = [(a, b) for a in ("4.25b", "4.5b") for b in ("int4", "fp4")]


def _operands(rng, M, N, K, a_fmt, b_fmt, spread=6):
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-spread, spread, (M, K)))).astype(np.float32)
    w = (rng.standard_normal((N, K)) * np.exp2(rng.integers(-3, 3, (N, K)))).astype(np.float32)
    ac, as_ = mix_quantize(x, a_fmt)
    bc, bs = mx_quantize(w, b_fmt)
    return ac, as_, bc, bs


@pytest.mark.parametrize("a_fmt,b_fmt", PAIRS)
def test_eq6_identity_per_block(a_fmt, b_fmt):
    # P1 method overview, Eq. (6): the block dot product equals the factored shift-add form exactly.
    rng = np.random.default_rng(21)
    M, N, K = 6, 5, 128
    ac, as_, bc, bs = _operands(rng, M, N, K, a_fmt, b_fmt)
    blk, e = eq6_block_sums(ac, as_, a_fmt, bc, bs, b_fmt)
    ad = mix_dequantize(ac, as_, a_fmt)
    bd = mx_dequantize(bc, bs, b_fmt)
    assert np.abs(blk).max() < 2**21
    for i in range(M):
        for j in range(N):
            for b in range(K // 32):
                exact = sum(Fraction(float(ad[i, 32 * b + t])) * Fraction(float(bd[j, 32 * b + t])) for t in range(32))
                assert Fraction(int(blk[i, j, b])) * Fraction(2) ** int(e[i, j, b]) == exact


@pytest.mark.parametrize("a_fmt,b_fmt", PAIRS)
def test_fp64_reference_within_bound_of_exact(a_fmt, b_fmt):
    rng = np.random.default_rng(22)
    M, N, K = 8, 6, 512
    ac, as_, bc, bs = _operands(rng, M, N, K, a_fmt, b_fmt)
    ad = mix_dequantize(ac, as_, a_fmt)
    bd = mx_dequantize(bc, bs, b_fmt)
    ref = gemm_ref(ad, bd)
    ex, fr = gemm_exact(ac, as_, a_fmt, bc, bs, b_fmt)
    bound = K * 2.0**-53 * (np.abs(ad) @ np.abs(bd).T)
    assert np.all(np.abs(ref - ex) <= bound)
    # the exact value is the rational sum of the products, independently summed here
    for t, (i, j) in enumerate([(0, 0), (3, 2), (7, 5)]):
        want = sum(Fraction(float(ad[i, k])) * Fraction(float(bd[j, k])) for k in range(K))
        assert fr[i * N + j] == want
    sel = gemm_ref_entries(ad, bd, np.array([0, 3, 7]), np.array([0, 2, 5]))
    assert np.array_equal(sel, np.array([ref[0, 0], ref[3, 2], ref[7, 5]]))


def test_selection_operands():
    # W^T rows that are unit vectors pick columns of deq(A): C[:, j] = deq(A)[:, k_j].
    rng = np.random.default_rng(23)
    M, K = 16, 256
    x = rng.standard_normal((M, K)).astype(np.float32)
    ac, as_ = mix_quantize(x, "4.5b")
    picks = [0, 5, 31, 32, 100, 255]
    w = np.zeros((len(picks), K), np.float32)
    for j, k in enumerate(picks):
        w[j, k] = 1.0
    for b_fmt in ("int4", "fp4"):
        bc, bs = mx_quantize(w, b_fmt)
        bd = mx_dequantize(bc, bs, b_fmt)
        assert np.array_equal(bd, w.astype(np.float64))
        ad = mix_dequantize(ac, as_, "4.5b")
        c = gemm_ref(ad, bd)
        for j, k in enumerate(picks):
            assert np.array_equal(c[:, j], ad[:, k])
        ex, _ = gemm_exact(ac, as_, "4.5b", bc, bs, b_fmt)
        assert np.array_equal(ex, c)
