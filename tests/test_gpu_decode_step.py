"""GPU parity of the whole decode step (mix_decode_step): the linear x -> MiX-4.5b x W-MX -> bf16 and
the attention step, run together in three launches.

The step must equal its parts bit for bit: y equals mix_mx_gemm_images of the quantizer's A image
(the same per-wave K ranges and sum order), and o equals mix_attn_decode on an identical cache (the
same kernels); the cache it leaves is the oracle's coding. The parts are checked against the oracle
elsewhere (tests/test_gpu_attention.py, tests/test_gpu_gemm.py); here y is also compared with the
oracle's product on every element, and the full-size attention stages on every batch row. The
single-launch form (mix_decode_step_single) must equal the three-launch step bit for bit, over two
steps in a row.
"""
import numpy as np
import pytest
import torch

from helpers import assert_bf16_matches, assert_codes_equal, dev_bf16, host
from oracle.gemm import gemm_abs_bound, gemm_ref
from oracle.mix import mix_dequantize as o_mix_deq, mix_quantize as o_mix_q
from oracle.mx import mx_dequantize as o_mx_deq, mx_quantize as o_mx_q
from quantized_gemm_algorithm_amd import synth

pytestmark = pytest.mark.gpu


def _q():
    import quantized_gemm_algorithm_amd as q
    return q


def _caches(q, B, Lmax, Hkv, d, kh, vh, pos, n=2):
    """n identical caches holding tokens [0, pos[b]) of each row, and the rows' K-means."""
    mus = []
    caches = [q.KVCache(B, Lmax, Hkv, d) for _ in range(n)]
    for b in range(B):
        T0 = int(pos[b])
        kd = dev_bf16(kh[b, :T0])
        mu = q.mix_kmean(kd.reshape(T0, Hkv * d)).reshape(Hkv, d)
        mus.append(mu)
        for c in caches:
            q.mix_kv_cache_prefill(c, b, kd, dev_bf16(vh[b, :T0]), mu)
    return caches, torch.stack(mus)


def _same_cache(a, b):
    for name in ("k_codes", "k_scales", "v_codes", "v_scales", "v_stage"):
        assert torch.equal(getattr(a, name).view(torch.uint8), getattr(b, name).view(torch.uint8)), name


@pytest.mark.parametrize("fmt", ["fp4", "int4"])
@pytest.mark.parametrize("B,Hq,Hkv,L_each,N,K", [
    (4, 8, 2, [40, 63, 255, 300], 300, 256),
    (3, 28, 4, [511, 17, 1000], 1000, 3584),
    (16, 14, 2, [5 + 37 * i for i in range(16)], 64, 128),
])
def test_decode_step_equals_its_parts(fmt, B, Hq, Hkv, L_each, N, K):
    q = _q()
    d = 128
    rng = np.random.default_rng(B * 1000 + N + K)
    Lmax = ((max(L_each) + 1 + 31) // 32) * 32 + 32
    kh = np.zeros((B, Lmax, Hkv, d), np.uint16)
    vh = np.zeros((B, Lmax, Hkv, d), np.uint16)
    for b in range(B):
        g = synth.attention_qkv(T=Lmax, Hq=1, Hkv=Hkv, d=d, rng=rng)
        kh[b], vh[b] = g["k"], g["v"]
    pos = np.array(L_each, np.int32)
    (c1, c2), mu = _caches(q, B, Lmax, Hkv, d, kh, vh, pos)
    qd = dev_bf16(synth.f32_to_bf16_bits(rng.standard_normal((B, Hq, d)).astype(np.float32) * 3))
    knew = dev_bf16(np.stack([kh[b, pos[b]] for b in range(B)]))
    vnew = dev_bf16(np.stack([vh[b, pos[b]] for b in range(B)]))
    xb = synth.f32_to_bf16_bits((rng.standard_normal((B, K)) * np.exp2(rng.integers(-6, 6, (B, K)))).astype(np.float32))
    wb = synth.f32_to_bf16_bits((0.02 * rng.standard_normal((N, K))).astype(np.float32))
    bc, bs = q.mx_quantize(dev_bf16(wb), fmt)
    bimg = q.mx_gemm_b_image(bc, bs, fmt)
    x = dev_bf16(xb)
    pos_d = torch.as_tensor(pos, device="cuda")
    max_pos = int(pos.max())

    y, o = q.mix_decode_step(x, bimg, qd, knew, vnew, c1, pos_d, max_pos, mu)
    _, _, aimg = q.mix_quantize_gemm(x, "4.5b")
    y_ref = q.mix_mx_gemm_images(aimg, bimg, out_dtype=torch.bfloat16)
    o_ref, _ = q.mix_attn_decode(qd, knew, vnew, c2, pos_d, max_pos, mu)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), "decode step y differs from the image product"
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), "decode step o differs from mix_attn_decode"
    _same_cache(c1, c2)
    # y against the oracle, every element
    ac, as_ = o_mix_q(xb, "4.5b", "bf16")
    obc, obs = o_mx_q(wb, fmt, "bf16")
    assert_codes_equal(host(bc), obc, "weight codes")
    ad, bd = o_mix_deq(ac, as_, "4.5b"), o_mx_deq(obc, obs, fmt)
    assert_bf16_matches(host(y), gemm_ref(ad, bd), gemm_abs_bound(ad, bd), f"decode step y {fmt}")


def test_decode_step_workload5_full_size():
    # batch 16: x [16, 3584] -> y [16, 18944] with MXFP4 weights, every element against the oracle;
    # attention over 8192 tokens (28 / 4 heads, d = 128) equal to mix_attn_decode on an identical cache,
    # whose stages are checked against the oracle on every batch row in tests/test_gpu_attention.py
    q = _q()
    g = synth.decode_step()
    B, L, Hkv, d = g["k_hist"].shape
    Hq = g["q"].shape[1]
    N, K = g["w_t"].shape
    pos = np.full(B, L - 1, np.int32)
    (c1, c2), mu = _caches(q, B, L, Hkv, d, g["k_hist"], g["v_hist"], pos)
    bc, bs = q.mx_quantize(dev_bf16(g["w_t"]), "fp4")
    bimg = q.mx_gemm_b_image(bc, bs, "fp4")
    x, qd = dev_bf16(g["x"]), dev_bf16(g["q"])
    knew, vnew = dev_bf16(g["k_hist"][:, L - 1]), dev_bf16(g["v_hist"][:, L - 1])
    pos_d = torch.as_tensor(pos, device="cuda")
    y, o = q.mix_decode_step(x, bimg, qd, knew, vnew, c1, pos_d, L - 1, mu)
    o_ref, _ = q.mix_attn_decode(qd, knew, vnew, c2, pos_d, L - 1, mu)
    # the linear alone through the codes path (quantizer, images, weight stream) gives the same y
    ac, as_ = q.mix_quantize(x, "4.5b")
    y_codes = q.mix_mx_gemm(ac, as_, "4.5b", bc, bs, "fp4", out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(y.view(torch.int16), y_codes.view(torch.int16))
    _same_cache(c1, c2)
    ac, as_ = o_mix_q(g["x"], "4.5b", "bf16")
    obc, obs = o_mx_q(g["w_t"], "fp4", "bf16")
    assert_codes_equal(host(bc), obc, "weight codes, all 18944 rows")
    ad, bd = o_mix_deq(ac, as_, "4.5b"), o_mx_deq(obc, obs, "fp4")
    assert_bf16_matches(host(y), gemm_ref(ad, bd), gemm_abs_bound(ad, bd), "decode step y, workload 5")


def test_decode_step_repeated_calls_and_bad_rows():
    # no state is carried between calls: two steps in a row (the second appends the next token) equal
    # two separate mix_attn_decode calls; a row outside [0, max_pos] gives zeros
    q = _q()
    B, Hq, Hkv, d, N, K = 3, 8, 2, 128, 256, 256
    rng = np.random.default_rng(77)
    Lmax = 640
    kh = np.zeros((B, Lmax, Hkv, d), np.uint16)
    vh = np.zeros((B, Lmax, Hkv, d), np.uint16)
    for b in range(B):
        g = synth.attention_qkv(T=Lmax, Hq=1, Hkv=Hkv, d=d, rng=rng)
        kh[b], vh[b] = g["k"], g["v"]
    pos = np.array([300, 33, 511], np.int32)
    (c1, c2), mu = _caches(q, B, Lmax, Hkv, d, kh, vh, pos)
    bc, bs = q.mx_quantize(dev_bf16(synth.f32_to_bf16_bits((0.02 * rng.standard_normal((N, K))).astype(np.float32))),
                           "fp4")
    bimg = q.mx_gemm_b_image(bc, bs, "fp4")
    x = dev_bf16(synth.f32_to_bf16_bits(rng.standard_normal((B, K)).astype(np.float32)))
    qd = dev_bf16(synth.f32_to_bf16_bits(rng.standard_normal((B, Hq, d)).astype(np.float32)))
    for step in range(2):
        p = pos + step
        p[2] = 900 if step == 1 else p[2]          # row 2 beyond max_pos in the second step
        knew = dev_bf16(np.stack([kh[b, min(p[b], Lmax - 1)] for b in range(B)]))
        vnew = dev_bf16(np.stack([vh[b, min(p[b], Lmax - 1)] for b in range(B)]))
        pd = torch.as_tensor(p, device="cuda")
        max_pos = 512
        y, o = q.mix_decode_step(x, bimg, qd, knew, vnew, c1, pd, max_pos, mu)
        o_ref, _ = q.mix_attn_decode(qd, knew, vnew, c2, pd, max_pos, mu)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), step
        _same_cache(c1, c2)
    assert torch.all(o[2].float() == 0)


def _single_vs_three(q, B, Hq, Hkv, L_each, N, K, fmt, rng, kh, vh, Lmax, steps=2):
    """mix_decode_step_single against mix_decode_step on identical caches, `steps` steps in a row
    (each appends the next token): y, o and the caches bit for bit."""
    d = 128
    pos = np.array(L_each, np.int32)
    (c1, c2), mu = _caches(q, B, Lmax, Hkv, d, kh, vh, pos)
    wb = synth.f32_to_bf16_bits((0.02 * rng.standard_normal((N, K))).astype(np.float32))
    bc, bs = q.mx_quantize(dev_bf16(wb), fmt)
    bimg = q.mx_gemm_b_image(bc, bs, fmt)
    for s in range(steps):
        p = pos + s
        qd = dev_bf16(synth.f32_to_bf16_bits(rng.standard_normal((B, Hq, d)).astype(np.float32) * 3))
        knew = dev_bf16(np.stack([kh[b, p[b]] for b in range(B)]))
        vnew = dev_bf16(np.stack([vh[b, p[b]] for b in range(B)]))
        x = dev_bf16(synth.f32_to_bf16_bits(rng.standard_normal((B, K)).astype(np.float32)))
        pos_d = torch.as_tensor(p, device="cuda")
        max_pos = int(p.max())
        y3, o3 = q.mix_decode_step(x, bimg, qd, knew, vnew, c1, pos_d, max_pos, mu)
        y1, o1 = q.mix_decode_step(x, bimg, qd, knew, vnew, c2, pos_d, max_pos, mu, single=True)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y3.view(torch.int16)), f"step {s}: y differs"
        assert torch.equal(o1.view(torch.int16), o3.view(torch.int16)), f"step {s}: o differs"
        _same_cache(c1, c2)


@pytest.mark.parametrize("fmt", ["fp4", "int4"])
@pytest.mark.parametrize("B,Hq,Hkv,L_each,N,K", [
    (4, 8, 2, [40, 63, 255, 300], 300, 256),
    (3, 28, 4, [511, 17, 1000], 1000, 3584),
    (16, 14, 2, [5 + 37 * i for i in range(16)], 64, 128),
])
def test_decode_step_single_launch_equals_three_launches(fmt, B, Hq, Hkv, L_each, N, K):
    q = _q()
    d = 128
    print(f"single-launch decode step: {fmt} B={B} Hq={Hq} Hkv={Hkv} N={N} K={K}", flush=True)
    rng = np.random.default_rng(7 * B + N + K)
    Lmax = ((max(L_each) + 2 + 31) // 32) * 32 + 32
    kh = np.zeros((B, Lmax, Hkv, d), np.uint16)
    vh = np.zeros((B, Lmax, Hkv, d), np.uint16)
    for b in range(B):
        g = synth.attention_qkv(T=Lmax, Hq=1, Hkv=Hkv, d=d, rng=rng)
        kh[b], vh[b] = g["k"], g["v"]
    _single_vs_three(q, B, Hq, Hkv, L_each, N, K, fmt, rng, kh, vh, Lmax)


def test_decode_step_single_launch_workload5():
    # batch 16, x [16, 3584] -> y [16, 18944] (MXFP4), attention over 8192 cached tokens, 28 / 4 heads
    q = _q()
    print("single-launch decode step: workload 5 full size", flush=True)
    g = synth.decode_step()
    B, L, Hkv, d = g["k_hist"].shape
    Hq = g["q"].shape[1]
    N, K = g["w_t"].shape
    rng = np.random.default_rng(5)
    _single_vs_three(q, B, Hq, Hkv, [L - 2] * B, N, K, "fp4", rng, g["k_hist"], g["v_hist"], L)
