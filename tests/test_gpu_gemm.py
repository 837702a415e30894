"""GPU parity of the A-MiX x W-MX product (MFMA path and the Eq. (6) vector-ALU path) against the
oracle's exact dyadic dot products, within the fp32-accumulation tolerance (1e-5 of sum|a b| per
element and normwise). Inputs are coded by the oracle, so the product is checked on its own."""
import numpy as np
import pytest
import torch

from helpers import assert_bf16_matches, assert_codes_equal, assert_gemm_close, dev_bf16, dev_f32, dev_u8, dev_u16, host
from oracle.gemm import gemm_abs_bound, gemm_exact, gemm_ref, gemm_ref_entries
from oracle.mix import mix_dequantize as o_mix_deq, mix_quantize as o_mix_q
from oracle.mx import mx_dequantize as o_mx_deq, mx_quantize as o_mx_q
from quantized_gemm_algorithm_amd import synth

pytestmark = pytest.mark.gpu

PAIRS = [(a, b) for a in ("4.25b", "4.5b") for b in ("int4", "fp4")]


def _lib():
    import quantized_gemm_algorithm_amd as q
    return q


def _code(x, w_t, a_fmt, b_fmt, dtype="f32"):
    ac, as_ = o_mix_q(x, a_fmt, dtype)
    bc, bs = o_mx_q(w_t, b_fmt, dtype)
    return ac, as_, bc, bs


def _to_dev(ac, as_, bc, bs, a_fmt):
    return dev_u8(ac), (dev_u16(as_) if a_fmt == "4.5b" else dev_u8(as_)), dev_u8(bc), dev_u8(bs)


def _run(fn_name, ac, as_, bc, bs, a_fmt, b_fmt, out_dtype, workspace="auto"):
    q = _lib()
    A, S, B, Bs = _to_dev(ac, as_, bc, bs, a_fmt)
    if fn_name == "mix_mx_gemm":
        out = q.mix_mx_gemm(A, S, a_fmt, B, Bs, b_fmt, out_dtype=out_dtype, workspace=workspace)
    else:
        out = getattr(q, fn_name)(A, S, a_fmt, B, Bs, b_fmt, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("a_fmt,b_fmt", PAIRS)
@pytest.mark.parametrize("workspace", ["auto", None])
@pytest.mark.parametrize("M,N,K", [(64, 256, 128), (300, 520, 1024), (257, 300, 384), (512, 768, 3584)])
def test_gemm_fast_path_shapes(a_fmt, b_fmt, workspace, M, N, K):
    # shapes the decode-once path takes (K % 128 == 0, M >= 64, N >= 256), with ragged M/N tails;
    # workspace=None runs the same shapes through the decode-in-GEMM kernels
    q = _lib()
    assert q.mix_mx_gemm_workspace_bytes(a_fmt, b_fmt, M, N, K) > 0
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-8, 8, (M, K)))).astype(np.float32)
    w = (0.05 * rng.standard_normal((N, K)) * np.exp2(rng.integers(-3, 3, (N, K)))).astype(np.float32)
    ac, as_, bc, bs = _code(x, w, a_fmt, b_fmt)
    ad, bd = o_mix_deq(ac, as_, a_fmt), o_mx_deq(bc, bs, b_fmt)
    ref = gemm_ref(ad, bd)
    bound = gemm_abs_bound(ad, bd)
    got = _run("mix_mx_gemm", ac, as_, bc, bs, a_fmt, b_fmt, torch.float32, workspace)
    assert_gemm_close(got, ref, bound, f"{a_fmt}x{b_fmt} fp32 {M}x{N}x{K} ws={workspace}")
    gotb = _run("mix_mx_gemm", ac, as_, bc, bs, a_fmt, b_fmt, torch.bfloat16, workspace)
    assert_bf16_matches(gotb, ref, bound, f"{a_fmt}x{b_fmt} bf16 {M}x{N}x{K} ws={workspace}")


@pytest.mark.parametrize("a_fmt,b_fmt", PAIRS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (300, 520, 1024), (257, 300, 384), (64, 256, 3584)])
def test_gemm_images(a_fmt, b_fmt, M, N, K):
    # the image path: operand images built from the codes (and straight from x by the fused
    # quantizer), then the GEMM from images, against the oracle
    q = _lib()
    rng = np.random.default_rng(11 * M + 5 * N + K)
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-8, 8, (M, K)))).astype(np.float32)
    w = (0.05 * rng.standard_normal((N, K)) * np.exp2(rng.integers(-3, 3, (N, K)))).astype(np.float32)
    ac, as_, bc, bs = _code(x, w, a_fmt, b_fmt)
    ad, bd = o_mix_deq(ac, as_, a_fmt), o_mx_deq(bc, bs, b_fmt)
    ref, bound = gemm_ref(ad, bd), gemm_abs_bound(ad, bd)
    A, S, B, Bs = _to_dev(ac, as_, bc, bs, a_fmt)
    na = q.mix_gemm_a_image_bytes(M, K)
    ai = q.mix_gemm_a_image(A, S, a_fmt, out=torch.zeros(na, dtype=torch.uint8, device="cuda"))
    bi = q.mx_gemm_b_image(B, Bs, b_fmt)
    got = q.mix_mx_gemm_images(ai, bi, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_gemm_close(host(got), ref, bound, f"images {a_fmt}x{b_fmt} fp32 {M}x{N}x{K}")
    gotb = q.mix_mx_gemm_images(ai, bi, out_dtype=torch.bfloat16)
    assert_bf16_matches(host(gotb), ref, bound, f"images {a_fmt}x{b_fmt} bf16 {M}x{N}x{K}")
    # the fused quantizer writes the oracle's codes and the same image bytes
    xd = dev_f32(x)
    c2, s2, ai2 = q.mix_quantize_gemm(xd, a_fmt, image=torch.zeros(na, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert_codes_equal(host(c2), ac, "fused codes")
    assert_codes_equal(host(s2), as_, "fused shared")
    assert torch.equal(ai2.buf, ai.buf), "fused image differs from mix_gemm_a_image"
    _, _, ai3 = q.mix_quantize_gemm(xd, a_fmt, write_codes=False,
                                    image=torch.zeros(na, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(ai3.buf, ai.buf), "image-only quantize differs"
    _, _, ai4 = q.mix_quantize_gemm(xd, a_fmt, codes=c2, shared=s2, image=ai3)  # an AImage is reused in place
    torch.cuda.synchronize()
    assert ai4.buf.data_ptr() == ai3.buf.data_ptr() and torch.equal(ai4.buf, ai.buf)
    # same kernel as mix_mx_gemm's fast path: identical bits where that path is taken
    if q.mix_mx_gemm_workspace_bytes(a_fmt, b_fmt, M, N, K):
        ws = q.mix_mx_gemm(A, S, a_fmt, B, Bs, b_fmt, out_dtype=torch.float32, workspace="auto")
        assert torch.equal(ws, got)


@pytest.mark.parametrize("b_fmt,M,N,K", [("fp4", 300, 512, 256), ("int4", 64, 256, 128), ("fp4", 1000, 384, 384),
                                         ("fp4", 257, 640, 512), ("fp4", 8, 512, 256), ("int4", 16, 384, 128),
                                         ("fp4", 200, 288, 256), ("int4", 96, 352, 128), ("fp4", 130, 1152, 256),
                                         ("fp4", 4096, 18944, 3584)])
def test_gemm_images_quantized_output(b_fmt, M, N, K):
    """The product with its output quantized in the epilogue equals the unfused flow bit for bit:
    C in bf16, then mix_quantize_gemm of that C (codes, shared fields and the next product's A
    image); and the codes are the oracle's MiX-4.5b coding of the GPU's bf16 C."""
    q = _lib()
    if M * N * K > 1e9:
        # full size: the workload's own inputs, coded by the GPU quantizers (bit-exact with the
        # oracle in the quantizer tests)
        g = synth.prefill_linear()
        A, S, _ = q.mix_quantize_gemm(dev_bf16(g["x"]), "4.5b")
        B, Bs = q.mx_quantize(dev_bf16(g["w_t"]), b_fmt)
    else:
        rng = np.random.default_rng(3 * M + 7 * N + K)
        x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-6, 6, (M, K)))).astype(np.float32)
        w = (0.05 * rng.standard_normal((N, K))).astype(np.float32)
        ac, as_, bc, bs = _code(x, w, "4.5b", b_fmt)
        A, S, B, Bs = _to_dev(ac, as_, bc, bs, "4.5b")
    ai = q.mix_gemm_a_image(A, S, "4.5b")
    bi = q.mx_gemm_b_image(B, Bs, b_fmt)
    c_ref = q.mix_mx_gemm_images(ai, bi, out_dtype=torch.bfloat16)
    img = N % 128 == 0   # the output's A image needs N (its K) a multiple of 128
    nq = q.mix_gemm_a_image_bytes(M, N) if img else 0
    zimg = (lambda: torch.zeros(nq, dtype=torch.uint8, device="cuda")) if img else (lambda: None)
    if img:
        rc, rs, rimg = q.mix_quantize_gemm(c_ref, "4.5b", image=zimg())
    else:
        rc, rs = q.mix_quantize(c_ref, "4.5b")
    c1, qc1, qs1, qi1 = q.mix_mx_gemm_images_quantize(ai, bi, keep_c=True, image=img, q_image=zimg())
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c_ref.view(torch.int16)), "C differs from the image product"
    assert torch.equal(qc1, rc) and torch.equal(qs1, rs), "fused output codes differ from the quantizer's"
    if img:
        assert torch.equal(qi1.buf, rimg.buf), "fused output image differs from the quantizer's"
    if M > 16:   # without C (only the codes, shared fields and image leave the epilogue)
        c2, qc2, qs2, qi2 = q.mix_mx_gemm_images_quantize(ai, bi, keep_c=False, image=img, q_image=zimg())
        torch.cuda.synchronize()
        assert c2 is None
        assert torch.equal(qc2, rc) and torch.equal(qs2, rs)
        if img:
            assert torch.equal(qi2.buf, rimg.buf)
    # against the oracle, on a sample of rows at full size
    rows = np.arange(M) if M <= 1024 else np.unique(np.linspace(0, M - 1, 64).astype(np.int64))
    cb = host(c_ref)[rows]
    oc, osh = o_mix_q(cb, "4.5b", "bf16")
    assert_codes_equal(host(qc1)[rows], oc, "fused output codes vs oracle")
    assert_codes_equal(host(qs1)[rows], osh, "fused output shared vs oracle")



@pytest.mark.parametrize("a_fmt,b_fmt", PAIRS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (5, 300, 3584), (16, 18, 4096), (16, 5000, 4224), (3, 700, 896),
                                   (16, 40000, 256), (16, 8192, 128), (7, 4099, 1152)])
def test_gemv_shapes(a_fmt, b_fmt, M, N, K):
    # M <= 16: the weight-streaming kernel (row groups per workgroup, K chunks, 4-way K split);
    # ragged N, K above one LDS chunk, and more row groups than fit one workgroup
    q = _lib()
    rng = np.random.default_rng(3 * M + 7 * N + K)
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-8, 8, (M, K)))).astype(np.float32)
    w = (0.05 * rng.standard_normal((N, K)) * np.exp2(rng.integers(-3, 3, (N, K)))).astype(np.float32)
    ac, as_, bc, bs = _code(x, w, a_fmt, b_fmt)
    ad, bd = o_mix_deq(ac, as_, a_fmt), o_mx_deq(bc, bs, b_fmt)
    ref, bound = gemm_ref(ad, bd), gemm_abs_bound(ad, bd)
    for dt in (torch.float32, torch.bfloat16):
        got = _run("mix_mx_gemm", ac, as_, bc, bs, a_fmt, b_fmt, dt)
        what = f"gemv {a_fmt}x{b_fmt} {dt} {M}x{N}x{K}"
        if dt == torch.float32:
            assert_gemm_close(got, ref, bound, what)
        else:
            assert_bf16_matches(got, ref, bound, what)


@pytest.mark.parametrize("a_fmt,b_fmt", PAIRS)
@pytest.mark.parametrize("fn", ["mix_mx_gemm", "mix_mx_gemm_eq6"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (64, 256, 512), (200, 136, 352), (130, 300, 96), (16, 18, 4096)])
def test_gemm_random_shapes(a_fmt, b_fmt, fn, M, N, K):
    rng = np.random.default_rng(M * 131 + N * 7 + K)
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-6, 6, (M, K)))).astype(np.float32)
    w = (0.05 * rng.standard_normal((N, K))).astype(np.float32)
    ac, as_, bc, bs = _code(x, w, a_fmt, b_fmt)
    ad, bd = o_mix_deq(ac, as_, a_fmt), o_mx_deq(bc, bs, b_fmt)
    ref = gemm_ref(ad, bd)
    bound = gemm_abs_bound(ad, bd)
    got = _run(fn, ac, as_, bc, bs, a_fmt, b_fmt, torch.float32)
    assert_gemm_close(got, ref, bound, f"{fn} {a_fmt}x{b_fmt} fp32 {M}x{N}x{K}")
    gotb = _run(fn, ac, as_, bc, bs, a_fmt, b_fmt, torch.bfloat16)
    assert_bf16_matches(gotb, ref, bound, f"{fn} {a_fmt}x{b_fmt} bf16 {M}x{N}x{K}")


def test_gemm_workload1_against_exact_integer_product():
    g = synth.tiny()
    ac, as_, bc, bs = _code(g["x"], g["w_t"], "4.5b", "int4")
    exact, _ = gemm_exact(ac, as_, "4.5b", bc, bs, "int4")
    ad, bd = o_mix_deq(ac, as_, "4.5b"), o_mx_deq(bc, bs, "int4")
    bound = gemm_abs_bound(ad, bd)
    for fn in ("mix_mx_gemm", "mix_mx_gemm_eq6"):
        got = _run(fn, ac, as_, bc, bs, "4.5b", "int4", torch.float32)
        assert_gemm_close(got, exact, bound, fn)


@pytest.mark.parametrize("pitch,dtype", [((1 << 21), torch.bfloat16), ((1 << 21) + 16, torch.bfloat16),
                                         ((1 << 21), torch.float32)])
def test_gemm_images_wide_row_pitch(pitch, dtype):
    # whole 256 x 256 tiles written into an output with a very wide row pitch: up to 2^21 elements the
    # tiles leave through the buffer-store path (32-bit offsets from each pass's first row), beyond it
    # through the bounds-checked path; both must give the contiguous result and leave the rest of
    # each row untouched
    q = _lib()
    M, N, K = 256, 512, 256
    rng = np.random.default_rng(pitch % 997)
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-6, 6, (M, K)))).astype(np.float32)
    w = (0.05 * rng.standard_normal((N, K))).astype(np.float32)
    ac, as_, bc, bs = _code(x, w, "4.5b", "fp4")
    A, S, B, Bs = _to_dev(ac, as_, bc, bs, "4.5b")
    ai = q.mix_gemm_a_image(A, S, "4.5b")
    bi = q.mx_gemm_b_image(B, Bs, "fp4")
    ref = q.mix_mx_gemm_images(ai, bi, out_dtype=dtype)
    big = torch.full((M, pitch), -3.0, dtype=dtype, device="cuda")
    out = big[:, :N]
    q.mix_mx_gemm_images(ai, bi, out_dtype=dtype, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), f"pitch {pitch}: tiles differ from the contiguous product"
    assert bool((big[:, N:N + 4096] == -3.0).all()) and bool((big[:, -4096:] == -3.0).all()), "row tail touched"
    del big


def test_gemm_zero_and_empty():
    q = _lib()
    # K = 0 gives zeros; M = 0 is an empty call
    A = torch.zeros((4, 0), dtype=torch.uint8, device="cuda")
    S = torch.zeros((4, 0), dtype=torch.int16, device="cuda")
    B = torch.zeros((3, 0), dtype=torch.uint8, device="cuda")
    Bs = torch.zeros((3, 0), dtype=torch.uint8, device="cuda")
    out = torch.full((4, 3), 7.0, device="cuda")
    q.mix_mx_gemm(A, S, "4.5b", B, Bs, "fp4", out=out)
    assert torch.all(out == 0)
    A = torch.zeros((0, 16), dtype=torch.uint8, device="cuda")
    S = torch.zeros((0, 1), dtype=torch.int16, device="cuda")
    B = torch.zeros((3, 16), dtype=torch.uint8, device="cuda")
    Bs = torch.zeros((3, 1), dtype=torch.uint8, device="cuda")
    out = q.mix_mx_gemm(A, S, "4.5b", B, Bs, "fp4")
    assert out.shape == (0, 3)


def _sampled_check(out_bits, ac, as_, a_fmt, bc, bs, b_fmt, nsamp, seed, what):
    rng = np.random.default_rng(seed)
    M, N = ac.shape[0], bc.shape[0]
    rows = rng.integers(0, M, nsamp)
    cols = rng.integers(0, N, nsamp)
    ur = np.unique(rows)
    uc = np.unique(cols)
    ad = o_mix_deq(ac[ur], as_[ur], a_fmt)
    bd = o_mx_deq(bc[uc], bs[uc], b_fmt)
    ri = np.searchsorted(ur, rows)
    ci = np.searchsorted(uc, cols)
    ref = gemm_ref_entries(ad, bd, ri, ci)
    bound = np.einsum("tk,tk->t", np.abs(ad[ri]), np.abs(bd[ci]))
    got = out_bits[rows, cols]
    assert_bf16_matches(got, ref, bound, what)


def _full_size_chain(g, a_fmt, b_fmt, what):
    """The bench's chain at full size -- the quantizer writing codes and the A image in one pass, the
    weights' MX codes and B image, the product from the images (bf16 C) -- against the oracle: every
    activation and weight code, and every element of C against the fp64 product of the oracle's codes."""
    q = _lib()
    xd, wd = dev_bf16(g["x"]), dev_bf16(g["w_t"])
    ac, as_, aimg = q.mix_quantize_gemm(xd, a_fmt)
    bc, bs = q.mx_quantize(wd, b_fmt)
    bimg = q.mx_gemm_b_image(bc, bs, b_fmt)
    out = q.mix_mx_gemm_images(aimg, bimg, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    del xd, wd
    oac, oas = o_mix_q(g["x"], a_fmt, "bf16")
    assert_codes_equal(host(ac), oac, f"{what} activation codes")
    assert_codes_equal(host(as_), oas, f"{what} activation shared fields")
    obc, obs = o_mx_q(g["w_t"], b_fmt, "bf16")
    assert_codes_equal(host(bc), obc, f"{what} weight codes")
    assert_codes_equal(host(bs), obs, f"{what} weight scales")
    ad, bd = o_mix_deq(oac, oas, a_fmt), o_mx_deq(obc, obs, b_fmt)
    del oac, oas, obc, obs
    ref, bound = gemm_ref(ad, bd), gemm_abs_bound(ad, bd)
    del ad, bd
    assert_bf16_matches(host(out), ref, bound, f"{what} C, every element")


def test_gemm_workload2_full_size():
    # Qwen2-VL-7B-shaped prefill linear: 4096 x 18944 x 3584, MiX-4.5b x MXFP4, bf16 out
    _full_size_chain(synth.prefill_linear(), "4.5b", "fp4", "workload 2")


def test_gemm_workload3_full_size():
    # vision-encoder linear: 16384 x 5120 x 1280, MiX-4.25b x MXINT4, bf16 out
    _full_size_chain(synth.vision_linear(), "4.25b", "int4", "workload 3")


def test_gemm_eq6_workload3_sampled():
    q = _lib()
    g = synth.vision_linear()
    ac, as_ = q.mix_quantize(dev_bf16(g["x"]), "4.25b")
    bc, bs = q.mx_quantize(dev_bf16(g["w_t"]), "int4")
    out = q.mix_mx_gemm_eq6(ac, as_, "4.25b", bc, bs, "int4", out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _sampled_check(host(out), host(ac), host(as_), "4.25b", host(bc), host(bs), "int4", 2048, 4, "workload 3 eq6")


@pytest.mark.parametrize("M,N,K,b_fmt", [(65536, 512, 4096, "fp4"), (512, 1024, 65536, "int4"), (8, 2048, 65536, "fp4")])
def test_gemm_images_large_extents_sampled(M, N, K, b_fmt):
    # extents far from the workloads' (a 268 MB activation image; 512 K steps per tile; the weight
    # stream over K = 65536), seeded on the device: the sampled rows' codes are checked against the
    # oracle's coding of the same values, then sampled outputs against the oracle's dot products
    q = _lib()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(M + N + K)
    x = (torch.randn((M, K), generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
    w = (torch.randn((N, K), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
    ac, as_, ai = q.mix_quantize_gemm(x, "4.5b")
    bc, bs = q.mx_quantize(w, b_fmt)
    bi = q.mx_gemm_b_image(bc, bs, b_fmt)
    out = q.mix_mx_gemm_images(ai, bi, out_dtype=torch.float32 if b_fmt == "int4" else torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(K)
    rows = np.unique(rng.integers(0, M, 6))
    xs = x[torch.as_tensor(rows, device="cuda")].view(torch.int16).cpu().numpy().view(np.uint16)
    wc, ws = o_mix_q(xs, "4.5b", "bf16")
    assert_codes_equal(host(ac)[rows], wc, "sampled activation codes")
    assert_codes_equal(host(as_)[rows], ws, "sampled shared fields")
    cols = np.unique(rng.integers(0, N, 6))
    ad = o_mix_deq(wc, ws, "4.5b")
    bd = o_mx_deq(host(bc)[cols], host(bs)[cols], b_fmt)
    ref, bound = gemm_ref(ad, bd), gemm_abs_bound(ad, bd)
    got = host(out)[np.ix_(rows, cols)]
    if b_fmt == "int4":
        assert_gemm_close(got, ref, bound, f"{M}x{N}x{K} {b_fmt}")
    else:
        assert_bf16_matches(got, ref, bound, f"{M}x{N}x{K} {b_fmt}")
