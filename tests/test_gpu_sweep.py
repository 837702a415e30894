"""Seeded random sweep over shapes, formats and paths: every product path (codes, images in fp32 and
bf16, Eq. (6)) for MiX-4.25b/4.5b x MXFP4/MXINT4/g16 with ragged extents and mixed magnitudes, and
prefill/decode attention with random sequence lengths, head counts and head sizes, each against the
oracle with the same checks as the dedicated tests."""
import numpy as np
import pytest
import torch

import test_gpu_attention as ta
from helpers import assert_bf16_matches, assert_codes_equal, assert_gemm_close, dev_bf16, dev_f32, host
from oracle.gemm import gemm_abs_bound, gemm_ref
from oracle.mix import mix_dequantize as o_mix_deq, mix_quantize as o_mix_q
from oracle.mx import mx_dequantize as o_mx_deq, mx_quantize as o_mx_q
from quantized_gemm_algorithm_amd import synth

pytestmark = pytest.mark.gpu


def _gemm_case(seed):
    rng = np.random.default_rng(1000 + seed)
    M = int(rng.choice([1, 3, 8, 16, 17, 64, 65, 200, 256, 300, 513]))
    N = int(rng.choice([1, 5, 32, 100, 256, 257, 300, 520, 777]))
    K = 128 * int(rng.integers(1, 13))
    a_fmt = str(rng.choice(["4.25b", "4.5b"]))
    b_fmt = str(rng.choice(["fp4", "int4", "fp4g16", "int4g16"]))
    spread = int(rng.integers(0, 10))
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-spread, spread + 1, (M, K)))).astype(np.float32)
    w = (0.05 * rng.standard_normal((N, K)) * np.exp2(rng.integers(-2, 3, (N, K)))).astype(np.float32)
    if rng.random() < 0.2:
        x[:, rng.integers(0, K)] *= 60.0
    return M, N, K, a_fmt, b_fmt, x, w


@pytest.mark.parametrize("seed", range(32))
def test_sweep_gemm(seed):
    import quantized_gemm_algorithm_amd as q
    M, N, K, a_fmt, b_fmt, x, w = _gemm_case(seed)
    base = b_fmt[:-3] if b_fmt.endswith("g16") else b_fmt
    blk = 16 if b_fmt.endswith("g16") else 32
    what = f"{M}x{N}x{K} {a_fmt} x {b_fmt}"
    if seed % 2:   # bf16 inputs (the quantizers' other instantiation)
        xb, wb = synth.f32_to_bf16_bits(x), synth.f32_to_bf16_bits(w)
        ac, as_ = q.mix_quantize(dev_bf16(xb), a_fmt)
        bc, bs = q.mx_quantize(dev_bf16(wb), b_fmt)
        wac, was = o_mix_q(xb, a_fmt, "bf16")
        wbc, wbs = o_mx_q(wb, base, "bf16", block=blk)
        what += " bf16 in"
    else:
        ac, as_ = q.mix_quantize(dev_f32(x), a_fmt)
        bc, bs = q.mx_quantize(dev_f32(w), b_fmt)
        wac, was = o_mix_q(x, a_fmt, "f32")
        wbc, wbs = o_mx_q(w, base, "f32", block=blk)
    torch.cuda.synchronize()
    assert_codes_equal(host(ac), wac, what + " A codes")
    assert_codes_equal(host(as_), was, what + " A shared")
    assert_codes_equal(host(bc), wbc, what + " B codes")
    assert_codes_equal(host(bs), wbs, what + " B scales")
    ad, bd = o_mix_deq(wac, was, a_fmt), o_mx_deq(wbc, wbs, base, block=blk)
    ref, bound = gemm_ref(ad, bd), gemm_abs_bound(ad, bd)
    outs = {"eq6": q.mix_mx_gemm_eq6(ac, as_, a_fmt, bc, bs, b_fmt, out_dtype=torch.float32)}
    if not b_fmt.endswith("g16"):
        outs["codes"] = q.mix_mx_gemm(ac, as_, a_fmt, bc, bs, b_fmt, out_dtype=torch.float32)
    ai = q.mix_gemm_a_image(ac, as_, a_fmt)
    bi = q.mx_gemm_b_image(bc, bs, b_fmt)
    outs["images"] = q.mix_mx_gemm_images(ai, bi, out_dtype=torch.float32)
    ob = q.mix_mx_gemm_images(ai, bi, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    if b_fmt.endswith("g16"):
        assert int(bi.unfoldable.item()) == 0
    for k, v in outs.items():
        assert_gemm_close(host(v), ref, bound, what + " " + k)
    assert_bf16_matches(host(ob), ref, bound, what + " images bf16")


@pytest.mark.parametrize("seed", range(12))
def test_sweep_attention(seed):
    rng = np.random.default_rng(2000 + seed)
    Hkv = int(rng.choice([1, 2, 4]))
    if seed % 2 == 0:
        Hq = Hkv * int(rng.choice([1, 2, 3, 7]))
        d = int(rng.choice([32, 64, 128, 128]))
        T = int(rng.integers(1, 700))
        causal = bool(rng.random() < 0.7)
        g = synth.attention_qkv(T=T, Hq=Hq, Hkv=Hkv, d=d, seed_cfg=int(rng.integers(0, 1000)))
        rows = sorted(set([0, T - 1] + [int(v) for v in rng.integers(0, T, 12)]))
        ta._prefill_stages(g, T, Hq, Hkv, d, causal, rows, list(range(Hq)))
    else:
        B = int(rng.integers(1, 6))
        Hq = Hkv * int(rng.choice([1, 2, 7]))
        L = [int(v) for v in rng.integers(1, 1500, B)]
        r = ta._decode_case(B=B, Hq=Hq, Hkv=Hkv, L_each=L, seed=int(rng.integers(0, 1000)))
        ta._check_decode(r, Hq, Hkv)


@pytest.mark.parametrize("seed", range(8))
def test_sweep_underflow_map(seed):
    import quantized_gemm_algorithm_amd as q
    from oracle.underflow import underflow_map as o_map
    rng = np.random.default_rng(3000 + seed)
    rows = int(rng.integers(1, 900))
    cols = 32 * int(rng.integers(1, 40))
    spread = int(rng.integers(0, 40))
    x = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-spread, spread + 1, (rows, cols)))).astype(np.float32)
    if rng.random() < 0.5:
        x[rng.random((rows, cols)) < 0.1] = 0.0
    mu = rng.standard_normal(cols).astype(np.float32) if seed % 2 else None
    counts, amax = q.mix_underflow_map(dev_f32(x), mu=dev_f32(mu) if mu is not None else None)
    torch.cuda.synchronize()
    want = o_map(x, "f32", mu)
    assert np.array_equal(host(counts), want), f"{rows}x{cols} spread {spread}"
    xs = (x - mu).astype(np.float32) if mu is not None else x
    assert float(host(amax)[0]) == float(np.abs(xs).max())
