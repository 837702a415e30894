"""The allocation-free decode step (mix_decode_step_static, its workspace a file-scope device array)
against the decode step with a caller workspace (mix_decode_step), through the C-ABI: bit for bit on
two calls in a row, the second with a smaller input, so that contents the first call left in the
shared array cannot leak into the second's results."""
import ctypes

import numpy as np
import pytest
import torch

from helpers import dev_bf16
from quantized_gemm_algorithm_amd import synth

pytestmark = pytest.mark.gpu


def _case(q, B, K, N, L, Hq, Hkv, seed):
    d = 128
    g = synth.decode_step(B=B, K=K, N=N, L=L, Hq=Hq, Hkv=Hkv, d=d, seed_cfg=seed)
    bc, bs = q.mx_quantize(dev_bf16(g["w_t"]), "fp4")
    bimg = q.mx_gemm_b_image(bc, bs, "fp4")
    caches = [q.KVCache(B, L, Hkv, d) for _ in range(2)]
    mus = []
    for b in range(B):
        kd = dev_bf16(g["k_hist"][b, : L - 1])
        mus.append(q.mix_kmean(kd.reshape(L - 1, Hkv * d)).reshape(Hkv, d))
        for c in caches:
            q.mix_kv_cache_prefill(c, b, kd, dev_bf16(g["v_hist"][b, : L - 1]), mus[-1])
    return dict(x=dev_bf16(g["x"]), q=dev_bf16(g["q"]), k_new=dev_bf16(g["k_hist"][:, L - 1]),
                v_new=dev_bf16(g["v_hist"][:, L - 1]), mu=torch.stack(mus), bimg=bimg, caches=caches,
                pos=torch.full((B,), L - 1, dtype=torch.int32, device="cuda"), B=B, K=K, N=N, L=L, Hq=Hq, d=d)


def _static_call(q, c, cache, y, o):
    lib = q._lib_()
    P = ctypes.c_void_p
    st = lib.mix_decode_step_static(P(c["x"].data_ptr()), c["K"], c["N"], q.MX_FMT["fp4"], P(c["bimg"].buf.data_ptr()),
                                    P(y.data_ptr()), P(c["q"].data_ptr()), P(c["k_new"].data_ptr()),
                                    P(c["v_new"].data_ptr()), cache.ref, P(c["pos"].data_ptr()), c["L"] - 1, c["Hq"],
                                    P(c["mu"].data_ptr()), P(o.data_ptr()),
                                    P(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.mix_last_error()


def test_static_decode_step_equals_workspace_decode_step():
    import quantized_gemm_algorithm_amd as q
    assert q._lib_().mix_decode_step_static_max_bytes() == 32 << 20
    for (B, K, N, L, Hq, Hkv, seed) in ((8, 1024, 2048, 2048, 16, 4, 21), (3, 512, 600, 672, 8, 2, 22)):
        c = _case(q, B, K, N, L, Hq, Hkv, seed)
        need = q._lib_().mix_decode_step_workspace_bytes(B, K, Hq, Hkv, c["d"], L - 1)
        assert need <= 32 << 20
        y_s = torch.full((B, N), -7.0, dtype=torch.bfloat16, device="cuda")
        o_s = torch.full((B, Hq, c["d"]), -7.0, dtype=torch.bfloat16, device="cuda")
        _static_call(q, c, c["caches"][0], y_s, o_s)
        y_w, o_w = q.mix_decode_step(c["x"], c["bimg"], c["q"], c["k_new"], c["v_new"], c["caches"][1], c["pos"],
                                     L - 1, c["mu"])
        torch.cuda.synchronize()
        assert torch.equal(y_s.view(torch.int16), y_w.view(torch.int16)), (B, K, N, L)
        assert torch.equal(o_s.view(torch.int16), o_w.view(torch.int16)), (B, K, N, L)
        for name in ("k_codes", "k_scales", "v_codes", "v_scales", "v_stage"):
            assert torch.equal(getattr(c["caches"][0], name).view(torch.uint8),
                               getattr(c["caches"][1], name).view(torch.uint8)), name
        assert np.isfinite(o_s.float().cpu().numpy()).all()


def test_static_decode_step_rejects_shapes_beyond_its_array():
    import quantized_gemm_algorithm_amd as q
    lib = q._lib_()
    P = ctypes.c_void_p
    B, K, N, L, Hq, Hkv = 16, 3584, 18944, 65536, 28, 4
    assert lib.mix_decode_step_workspace_bytes(B, K, Hq, Hkv, 128, L - 1) > 32 << 20
    cache = q.KVCache(B, 64, Hkv, 128)   # small real buffers; the shape check fails before any launch
    cache._st.Lmax = L
    fake = P(1 << 20)
    st = lib.mix_decode_step_static(fake, K, N, 1, fake, fake, fake, fake, fake, cache.ref, fake, L - 1, Hq, fake,
                                    fake, None)
    assert st == 7 and b"scratch" in lib.mix_last_error()
