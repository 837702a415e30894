"""A decode step (MiX quantize of x with its A image, the weight-stream product, attention over an
MX-coded KV cache) captured in a HIP graph and replayed: every replay, with eager work and
synchronizations between replays, must reproduce the eager step bit for bit (the kernels are
deterministic and the step is idempotent: it appends the same token at the same position)."""
import numpy as np
import pytest
import torch

from helpers import dev_bf16
from quantized_gemm_algorithm_amd import synth

pytestmark = pytest.mark.gpu


def test_decode_step_graph_replays_match_eager():
    import quantized_gemm_algorithm_amd as q
    B, K, N, L, Hq, Hkv, d = 4, 512, 1024, 640, 8, 2, 128
    g = synth.decode_step(B=B, K=K, N=N, L=L, Hq=Hq, Hkv=Hkv, d=d, seed_cfg=11)
    x = dev_bf16(g["x"])
    qd = dev_bf16(g["q"])
    bc, bs = q.mx_quantize(dev_bf16(g["w_t"]), "fp4")
    bimg = q.mx_gemm_b_image(bc, bs, "fp4")
    cache = q.KVCache(B, L, Hkv, d)
    mus = []
    for b in range(B):
        kd = dev_bf16(g["k_hist"][b, : L - 1])
        mus.append(q.mix_kmean(kd.reshape(L - 1, Hkv * d)).reshape(Hkv, d))
        q.mix_kv_cache_prefill(cache, b, kd, dev_bf16(g["v_hist"][b, : L - 1]), mus[-1])
    mu = torch.stack(mus)
    pos = torch.full((B,), L - 1, dtype=torch.int32, device="cuda")
    k_new = dev_bf16(g["k_hist"][:, L - 1])
    v_new = dev_bf16(g["v_hist"][:, L - 1])
    y = torch.empty((B, N), dtype=torch.bfloat16, device="cuda")
    ac, as_, aimg = q.mix_quantize_gemm(x, "4.5b")
    ws = torch.empty((q._lib_().mix_attn_decode_workspace_bytes(B, Hq, Hkv, d, L - 1),), dtype=torch.uint8,
                     device="cuda")
    outs = {}

    def step():
        q.mix_quantize_gemm(x, "4.5b", codes=ac, shared=as_, image=aimg)
        q.mix_mx_gemm_images(aimg, bimg, out=y)
        o, _ = q.mix_attn_decode(qd, k_new, v_new, cache, pos, L - 1, mu, workspace=ws)
        outs["o"] = o

    step()
    torch.cuda.synchronize()
    y_ref, o_ref = y.clone(), outs["o"].clone()
    kc_ref, vc_ref = cache.k_codes.clone(), cache.v_codes.clone()

    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        step()
    o_graph = outs["o"]
    for rep in range(3):
        y.zero_()
        o_graph.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"replay {rep}: GEMV output differs from the eager step"
        assert torch.equal(o_graph, o_ref), f"replay {rep}: attention output differs from the eager step"
        assert torch.equal(cache.k_codes, kc_ref) and torch.equal(cache.v_codes, vc_ref), f"replay {rep}: cache"
        # eager work between replays
        step()
        torch.cuda.synchronize()
        assert torch.equal(outs["o"], o_ref)
    assert np.isfinite(o_ref.float().cpu().numpy()).all()


def test_fused_decode_step_graph_replays_match_eager():
    # the same step through mix_decode_step (three launches, no memset node): every replay equals the
    # eager call, and its y equals the separate image product
    import quantized_gemm_algorithm_amd as q
    B, K, N, L, Hq, Hkv, d = 4, 512, 1024, 640, 8, 2, 128
    g = synth.decode_step(B=B, K=K, N=N, L=L, Hq=Hq, Hkv=Hkv, d=d, seed_cfg=11)
    x = dev_bf16(g["x"])
    qd = dev_bf16(g["q"])
    bc, bs = q.mx_quantize(dev_bf16(g["w_t"]), "fp4")
    bimg = q.mx_gemm_b_image(bc, bs, "fp4")
    cache = q.KVCache(B, L, Hkv, d)
    mus = []
    for b in range(B):
        kd = dev_bf16(g["k_hist"][b, : L - 1])
        mus.append(q.mix_kmean(kd.reshape(L - 1, Hkv * d)).reshape(Hkv, d))
        q.mix_kv_cache_prefill(cache, b, kd, dev_bf16(g["v_hist"][b, : L - 1]), mus[-1])
    mu = torch.stack(mus)
    pos = torch.full((B,), L - 1, dtype=torch.int32, device="cuda")
    k_new = dev_bf16(g["k_hist"][:, L - 1])
    v_new = dev_bf16(g["v_hist"][:, L - 1])
    y = torch.empty((B, N), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((q._lib_().mix_decode_step_workspace_bytes(B, K, Hq, Hkv, d, L - 1),), dtype=torch.uint8,
                     device="cuda")

    def step():
        q.mix_decode_step(x, bimg, qd, k_new, v_new, cache, pos, L - 1, mu, y=y, o=o, workspace=ws)

    step()
    torch.cuda.synchronize()
    y_ref, o_ref = y.clone(), o.clone()
    _, _, aimg = q.mix_quantize_gemm(x, "4.5b")
    y_parts = q.mix_mx_gemm_images(aimg, bimg, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y_ref, y_parts)
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        step()
    for rep in range(3):
        y.zero_()
        o.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"replay {rep}: linear output differs from the eager step"
        assert torch.equal(o, o_ref), f"replay {rep}: attention output differs from the eager step"
        step()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(y, y_ref)
