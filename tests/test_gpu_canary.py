"""Guard bands around device outputs: every output of a ragged-tail call is placed inside a larger
buffer filled with a sentinel, and the bytes outside the output must be untouched afterwards (a
kernel writing past C, an image, a code buffer or O would change them). The outputs themselves are
checked against the oracle in the other GPU tests; here only the margins are.
"""
import numpy as np
import pytest
import torch

from helpers import dev_bf16, dev_f32
from quantized_gemm_algorithm_amd import synth

pytestmark = pytest.mark.gpu

PAD = 4096   # guard bytes on each side of a 1-D output


def _q():
    import quantized_gemm_algorithm_amd as q
    return q


def _guarded(n, dtype, fill):
    """A dense 1-D view of n elements inside a sentinel-filled buffer; returns (view, check)."""
    esz = torch.empty((), dtype=dtype).element_size()
    pad = PAD // esz
    big = torch.empty((n + 2 * pad,), dtype=dtype, device="cuda")
    big.view(torch.uint8).fill_(fill)
    view = big[pad:pad + n]

    def check(what):
        torch.cuda.synchronize()
        b = big.view(torch.uint8).cpu().numpy()
        lo, hi = b[:PAD], b[PAD + n * esz:]
        assert np.all(lo == fill) and np.all(hi == fill), f"{what}: bytes outside the output were written"
    return view, check


def _guarded_matrix(M, N, dtype, fill, extra_cols=40, extra_rows=3):
    """An [M, N] view with row pitch N + extra_cols inside a sentinel-filled [M + extra_rows, pitch]."""
    ld = N + extra_cols
    big = torch.empty((M + extra_rows, ld), dtype=dtype, device="cuda")
    big.view(torch.uint8).fill_(fill)
    view = big[:M, :N]

    def check(what):
        torch.cuda.synchronize()
        b = big.view(torch.uint8).cpu().numpy().reshape(M + extra_rows, -1)
        esz = big.element_size()
        assert np.all(b[:M, N * esz:] == fill), f"{what}: a row was written past column N"
        assert np.all(b[M:] == fill), f"{what}: rows past M were written"
    return view, check


def _ops(M, N, K, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-4, 4, (M, K)))).astype(np.float32)
    w = (0.05 * rng.standard_normal((N, K))).astype(np.float32)
    return x, w


@pytest.mark.parametrize("M,N,K", [(200, 136, 352), (130, 300, 96), (5, 300, 3584), (257, 300, 384), (16, 18, 4096),
                                   (64, 256, 512), (16, 320, 256), (300, 288, 256)])
@pytest.mark.parametrize("b_fmt", ["fp4", "int4"])
def test_gemm_outputs_stay_inside(M, N, K, b_fmt):
    q = _q()
    x, w = _ops(M, N, K, M + N + K)
    xd, wd = dev_f32(x), dev_f32(w)
    # codes of both operands into guarded buffers
    ac, chk_ac = _guarded(M * K // 2, torch.uint8, 0xA5)
    as_, chk_as = _guarded(M * K // 32, torch.int16, 0x5A)
    q.mix_quantize(xd, "4.5b", codes=ac.view(M, K // 2), shared=as_.view(M, K // 32))
    bc, chk_bc = _guarded(N * K // 2, torch.uint8, 0xA5)
    bs, chk_bs = _guarded(N * K // 32, torch.uint8, 0x3C)
    q.mx_quantize(wd, b_fmt, codes=bc.view(N, K // 2), scales=bs.view(N, K // 32))
    for chk, what in ((chk_ac, "MiX codes"), (chk_as, "MiX shared"), (chk_bc, "MX codes"), (chk_bs, "MX scales")):
        chk(what)
    ac, as_, bc, bs = ac.view(M, K // 2), as_.view(M, K // 32), bc.view(N, K // 2), bs.view(N, K // 32)
    for dt, fill in ((torch.float32, 0x7F), (torch.bfloat16, 0x7F)):
        out, chk = _guarded_matrix(M, N, dt, fill)
        q.mix_mx_gemm(ac, as_, "4.5b", bc, bs, b_fmt, out=out)
        chk(f"mix_mx_gemm {dt}")
        out, chk = _guarded_matrix(M, N, dt, fill)
        q.mix_mx_gemm_eq6(ac, as_, "4.5b", bc, bs, b_fmt, out=out)
        chk(f"mix_mx_gemm_eq6 {dt}")
    if K % 128 == 0:
        na, nb = q.mix_gemm_a_image_bytes(M, K), q.mx_gemm_b_image_bytes(b_fmt, N, K)
        ia, chk_ia = _guarded(na, torch.uint8, 0xC3)
        ib, chk_ib = _guarded(nb, torch.uint8, 0xC3)
        _, _, ai = q.mix_quantize_gemm(xd, "4.5b", image=ia, write_codes=False)
        bi = q.mx_gemm_b_image(bc, bs, b_fmt, out=ib)
        chk_ia("A image")
        chk_ib("B image")
        out, chk = _guarded_matrix(M, N, torch.bfloat16, 0x7F)
        q.mix_mx_gemm_images(ai, bi, out=out)
        chk("mix_mx_gemm_images")
        if N % 32 == 0:
            qc, chk_qc = _guarded(M * N // 2, torch.uint8, 0xA5)
            qs, chk_qs = _guarded(M * N // 32, torch.int16, 0x5A)
            out, chk = _guarded_matrix(M, N, torch.bfloat16, 0x7F)
            q.mix_mx_gemm_images_quantize(ai, bi, keep_c=True, image=False, out=out, codes=qc.view(M, N // 2),
                                          shared=qs.view(M, N // 32))
            chk("quantized product C")
            chk_qc("quantized product codes")
            chk_qs("quantized product shared")
            # with the next product's A image (N % 128 == 0), and with the code buffer 4 bytes off a
            # 16-byte boundary (the epilogue's narrower stores)
            nq = q.mix_gemm_a_image_bytes(M, N) if N % 128 == 0 else 0
            for off in (0, 4):
                qc2, chk_qc2 = _guarded(M * N // 2 + off, torch.uint8, 0xA5)
                qs2, chk_qs2 = _guarded(M * N // 32, torch.int16, 0x5A)
                qi2, chk_qi2 = _guarded(nq, torch.uint8, 0x3C) if nq else (None, None)
                _, qc_o, qs_o, _ = q.mix_mx_gemm_images_quantize(
                    ai, bi, keep_c=False, image=nq > 0, codes=qc2[off:].view(M, N // 2),
                    shared=qs2.view(M, N // 32), q_image=qi2)
                chk_qc2(f"quantized product codes (offset {off})")
                chk_qs2(f"quantized product shared (offset {off})")
                if nq:
                    chk_qi2("quantized product image")
                assert torch.equal(qc_o, qc.view(M, N // 2)) and torch.equal(qs_o, qs.view(M, N // 32)), \
                    f"quantized outputs depend on the code buffer's alignment (offset {off})"


@pytest.mark.parametrize("T,Hq,Hkv", [(200, 4, 1), (77, 6, 3)])
def test_prefill_output_stays_inside(T, Hq, Hkv):
    q = _q()
    d = 128
    g = synth.attention_qkv(T=T, Hq=Hq, Hkv=Hkv, d=d, seed_cfg=4)
    o, chk = _guarded(T * Hq * d, torch.bfloat16, 0x7F)
    q.mix_attn_prefill(dev_bf16(g["q"]), dev_bf16(g["k"]), dev_bf16(g["v"]), causal=True, o=o.view(T, Hq, d))
    chk("prefill O")


def test_decode_step_outputs_stay_inside():
    q = _q()
    B, K, N, L, Hq, Hkv, d = 3, 384, 300, 320, 8, 2, 128
    g = synth.decode_step(B=B, K=K, N=N, L=L, Hq=Hq, Hkv=Hkv, d=d, seed_cfg=12)
    bc, bs = q.mx_quantize(dev_bf16(g["w_t"]), "fp4")
    bimg = q.mx_gemm_b_image(bc, bs, "fp4")
    cache = q.KVCache(B, L, Hkv, d)
    mus = []
    for b in range(B):
        T0 = 100 + 50 * b
        kd = dev_bf16(g["k_hist"][b, :T0])
        mus.append(q.mix_kmean(kd.reshape(T0, Hkv * d)).reshape(Hkv, d))
        q.mix_kv_cache_prefill(cache, b, kd, dev_bf16(g["v_hist"][b, :T0]), mus[-1])
    pos = torch.tensor([100, 150, 200], dtype=torch.int32, device="cuda")
    y, chk_y = _guarded(B * N, torch.bfloat16, 0x7F)
    o, chk_o = _guarded(B * Hq * d, torch.bfloat16, 0x7F)
    q.mix_decode_step(dev_bf16(g["x"]), bimg, dev_bf16(g["q"]), dev_bf16(g["k_hist"][:, 0]),
                      dev_bf16(g["v_hist"][:, 0]), cache, pos, 200, torch.stack(mus), y=y.view(B, N),
                      o=o.view(B, Hq, d))
    chk_y("decode y")
    chk_o("decode O")
