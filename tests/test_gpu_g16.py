"""g16 weights (MXINT4g16 / MXFP4g16: one shared exponent per 16 elements, the 4.5-bit tier of the
pages' experiment design (实验如何设计)): the GPU quantizer against the oracle bit for bit, and the products
(MFMA from the folded image, and Eq. (6)) against the oracle's exact dyadic dot products within
the fp32-accumulation tolerance, including MiX-INT4g16 at the prefill-linear size."""
import numpy as np
import pytest
import torch

from helpers import assert_bf16_matches, assert_codes_equal, assert_gemm_close, dev_bf16, dev_f32, dev_u8, dev_u16, host
from oracle.gemm import gemm_abs_bound, gemm_ref, gemm_ref_entries
from oracle.mix import mix_dequantize as o_mix_deq, mix_quantize as o_mix_q
from oracle.mx import mx_dequantize as o_mx_deq, mx_quantize as o_mx_q
from quantized_gemm_algorithm_amd import synth

pytestmark = pytest.mark.gpu

G16 = ("int4g16", "fp4g16")


def _base(fmt):
    return fmt[:-3]


def _q():
    import quantized_gemm_algorithm_amd as q
    return q


@pytest.mark.parametrize("fmt", G16)
@pytest.mark.parametrize("rows,cols,dtype", [(7, 32, "f32"), (300, 512, "f32"), (129, 3584, "bf16"), (64, 1280, "bf16")])
def test_g16_quantizer_bit_exact(fmt, rows, cols, dtype):
    q = _q()
    rng = np.random.default_rng(rows * 7 + cols)
    x = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-12, 12, (rows, cols)))).astype(np.float32)
    x[0, :16] = 0.0                      # an all-zero 16-element block
    x[-1, 16:32] = -x[-1, 16:32]
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(x)
        xd, xin = dev_bf16(bits), bits
    else:
        xd, xin = dev_f32(x), x
    codes, scales = q.mx_quantize(xd, fmt)
    torch.cuda.synchronize()
    wc, ws = o_mx_q(xin, _base(fmt), dtype, block=16)
    assert_codes_equal(host(codes), wc, f"{fmt} codes {rows}x{cols} {dtype}")
    assert_codes_equal(host(scales), ws, f"{fmt} scales {rows}x{cols} {dtype}")
    dq = q.mx_dequantize(codes, scales, fmt)
    torch.cuda.synchronize()
    assert np.array_equal(host(dq).astype(np.float64), o_mx_deq(wc, ws, _base(fmt), block=16))


@pytest.mark.parametrize("fmt", G16)
def test_g16_quantizer_smoothing_operand(fmt):
    q = _q()
    rng = np.random.default_rng(5)
    k = (rng.standard_normal((96, 256)) + 3.0).astype(np.float32)
    mu = k.mean(axis=0).astype(np.float32)
    codes, scales = q.mx_quantize(dev_f32(k), fmt, mu=dev_f32(mu))
    torch.cuda.synchronize()
    wc, ws = o_mx_q(k, _base(fmt), "f32", mu=mu, block=16)
    assert_codes_equal(host(codes), wc, f"{fmt} smoothed codes")
    assert_codes_equal(host(scales), ws, f"{fmt} smoothed scales")


def _operands(M, N, K, seed, spread=3):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-8, 8, (M, K)))).astype(np.float32)
    w = (0.05 * rng.standard_normal((N, K)) * np.exp2(rng.integers(-spread, spread, (N, K)))).astype(np.float32)
    return x, w


@pytest.mark.parametrize("fmt", G16)
@pytest.mark.parametrize("M,N,K", [(16, 300, 512), (5, 1000, 3584), (64, 256, 128), (300, 520, 1024), (257, 300, 384)])
def test_g16_image_product(fmt, M, N, K):
    # MiX-4.5b activations x g16 weights through the folded E4M3 image: M <= 16 takes the weight
    # stream, larger M the tiled product
    q = _q()
    x, w = _operands(M, N, K, 3 * M + N + K)
    ac, as_ = o_mix_q(x, "4.5b", "f32")
    bc, bs = o_mx_q(w, _base(fmt), "f32", block=16)
    ad, bd = o_mix_deq(ac, as_, "4.5b"), o_mx_deq(bc, bs, _base(fmt), block=16)
    ref, bound = gemm_ref(ad, bd), gemm_abs_bound(ad, bd)
    ai = q.mix_gemm_a_image(dev_u8(ac), dev_u16(as_), "4.5b")
    bi = q.mx_gemm_b_image(dev_u8(bc), dev_u8(bs), fmt)
    got = q.mix_mx_gemm_images(ai, bi, out_dtype=torch.float32)
    gotb = q.mix_mx_gemm_images(ai, bi, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert int(bi.unfoldable.item()) == 0
    assert_gemm_close(host(got), ref, bound, f"4.5b x {fmt} fp32 {M}x{N}x{K}")
    assert_bf16_matches(host(gotb), ref, bound, f"4.5b x {fmt} bf16 {M}x{N}x{K}")


@pytest.mark.parametrize("fmt", G16)
@pytest.mark.parametrize("a_fmt", ["4.25b", "4.5b"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (64, 256, 512), (200, 136, 352), (16, 18, 4096)])
def test_g16_eq6_product(fmt, a_fmt, M, N, K):
    q = _q()
    x, w = _operands(M, N, K, 5 * M + N + 3 * K, spread=12)
    ac, as_ = o_mix_q(x, a_fmt, "f32")
    bc, bs = o_mx_q(w, _base(fmt), "f32", block=16)
    ad, bd = o_mix_deq(ac, as_, a_fmt), o_mx_deq(bc, bs, _base(fmt), block=16)
    ref, bound = gemm_ref(ad, bd), gemm_abs_bound(ad, bd)
    S = dev_u16(as_) if a_fmt == "4.5b" else dev_u8(as_)
    got = q.mix_mx_gemm_eq6(dev_u8(ac), S, a_fmt, dev_u8(bc), dev_u8(bs), fmt, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_gemm_close(host(got), ref, bound, f"eq6 {a_fmt} x {fmt} {M}x{N}x{K}")


@pytest.mark.parametrize("fmt", G16)
def test_g16_wide_exponent_gaps_fold_exactly(fmt):
    # halves up to 14 binades apart share one scale exactly (the E4M3 element takes the difference),
    # so the image product is exact on every column
    q = _q()
    M, N, K = 32, 256, 256
    x, w = _operands(M, N, K, 9, spread=1)
    w[3, 32:48] *= 2.0 ** -12        # row 3, block 1: first half 2^-12 smaller
    w[200, 144:160] *= 2.0 ** 11     # row 200, block 4: second half 2^11 larger
    w[17, 64:80] *= 2.0 ** -5
    w[90, 0:16] *= 2.0 ** 12
    ac, as_ = o_mix_q(x, "4.5b", "f32")
    bc, bs = o_mx_q(w, _base(fmt), "f32", block=16)
    s16 = bs.astype(np.int64).reshape(N, K // 32, 2)
    nz = (s16[..., 0] > 0) & (s16[..., 1] > 0)
    assert (np.abs(s16[..., 0] - s16[..., 1]) * nz).max() >= 12
    bi = q.mx_gemm_b_image(dev_u8(bc), dev_u8(bs), fmt)
    torch.cuda.synchronize()
    assert int(bi.unfoldable.item()) == 0
    ad, bd = o_mix_deq(ac, as_, "4.5b"), o_mx_deq(bc, bs, _base(fmt), block=16)
    ref, bound = gemm_ref(ad, bd), gemm_abs_bound(ad, bd)
    img = q.mix_mx_gemm_images(q.mix_gemm_a_image(dev_u8(ac), dev_u16(as_), "4.5b"), bi, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_gemm_close(host(img), ref, bound, f"image {fmt} with wide exponent gaps")


@pytest.mark.parametrize("fmt", G16)
def test_g16_unfoldable_blocks_are_refused(fmt):
    # a 32-block whose halves' exponents differ by more than the fold holds (here 2^20) cannot share
    # one scale exactly: building its image raises unless inexact images are allowed, and then the
    # image counts it; Eq. (6) stays exact on the same weights
    q = _q()
    M, N, K = 32, 256, 256
    x, w = _operands(M, N, K, 9, spread=1)
    w[3, 32:48] *= 2.0 ** -20        # row 3, block 1: first half 2^-20 smaller
    w[200, 144:160] *= 2.0 ** 19     # row 200, block 4: second half 2^19 larger
    w[17, 64:80] *= 2.0 ** -5        # a difference of a few binades still folds exactly
    ac, as_ = o_mix_q(x, "4.5b", "f32")
    bc, bs = o_mx_q(w, _base(fmt), "f32", block=16)
    with pytest.raises(q.MixError, match="not be exact"):
        q.mx_gemm_b_image(dev_u8(bc), dev_u8(bs), fmt)
    bi = q.mx_gemm_b_image(dev_u8(bc), dev_u8(bs), fmt, allow_inexact=True)
    torch.cuda.synchronize()
    assert int(bi.unfoldable.item()) == 2
    ad, bd = o_mix_deq(ac, as_, "4.5b"), o_mx_deq(bc, bs, _base(fmt), block=16)
    ref, bound = gemm_ref(ad, bd), gemm_abs_bound(ad, bd)
    got = q.mix_mx_gemm_eq6(dev_u8(ac), dev_u16(as_), "4.5b", dev_u8(bc), dev_u8(bs), fmt, out_dtype=torch.float32)
    img = q.mix_mx_gemm_images(q.mix_gemm_a_image(dev_u8(ac), dev_u16(as_), "4.5b"), bi, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_gemm_close(host(got), ref, bound, f"eq6 {fmt} with unfoldable blocks")
    # the image product is exact in every column whose blocks all fold
    cols = [n for n in range(N) if n not in (3, 200)]
    assert_gemm_close(host(img)[:, cols], ref[:, cols], bound[:, cols], f"image {fmt} foldable columns")


def test_mix_int4g16_prefill_linear_full_size_sampled():
    # the pages' 4.5-bit headline pairing, MiX-INT4g16 (MiX-4.5b x MXINT4g16), on the Qwen2-VL-7B
    # prefill-linear shape 4096 x 18944 x 3584, bf16 out, sampled entries against the oracle
    q = _q()
    g = synth.prefill_linear()
    xd, wd = dev_bf16(g["x"]), dev_bf16(g["w_t"])
    ac, as_, ai = q.mix_quantize_gemm(xd, "4.5b")
    bc, bs = q.mx_quantize(wd, "int4g16")
    bi = q.mx_gemm_b_image(bc, bs, "int4g16")
    out = q.mix_mx_gemm_images(ai, bi, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert int(bi.unfoldable.item()) == 0
    wc, ws = o_mx_q(g["w_t"][:256], "int4", "bf16", block=16)
    assert_codes_equal(host(bc)[:256], wc, "weight codes slice")
    assert_codes_equal(host(bs)[:256], ws, "weight scales slice")
    acn, asn, bcn, bsn = host(ac), host(as_), host(bc), host(bs)
    rng = np.random.default_rng(16)
    rows, cols = rng.integers(0, 4096, 4096), rng.integers(0, 18944, 4096)
    ur, uc = np.unique(rows), np.unique(cols)
    ad = o_mix_deq(acn[ur], asn[ur], "4.5b")
    bd = o_mx_deq(bcn[uc], bsn[uc], "int4", block=16)
    ri, ci = np.searchsorted(ur, rows), np.searchsorted(uc, cols)
    ref = gemm_ref_entries(ad, bd, ri, ci)
    bound = np.einsum("tk,tk->t", np.abs(ad[ri]), np.abs(bd[ci]))
    assert_bf16_matches(host(out)[rows, cols], ref, bound, "MiX-INT4g16 workload 2")
