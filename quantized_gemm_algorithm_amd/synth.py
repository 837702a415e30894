"""Seeded synthetic inputs shaped like the workloads the MiX pages measure on.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic, and both the CPU oracle's tests and the GPU path take their
inputs from it. Every generator uses ``numpy.random.default_rng(1000 + cfg)`` and
draws in the order written; bf16 outputs are the RNE rounding of the fp32 draws,
returned as uint16 bit patterns.

Workloads (the models and benchmarks the pages use are not available; these
generators take only their shapes and the activation statistics the pages
report):

1. tiny: X[64x512] fp32 ~ N(0,1) with 1% of channels x30; W[512x256] ~ N(0,0.02).
2. Qwen2-VL-7B-shaped prefill linear: X[4096x3584] bf16, rows 0..3583 "visual"
   0.2301*t(2.12) (mean|x| ~0.31, p99 ~2.07), rows 3584..4095 "text"
   0.006681*t(2.12) (mean ~0.009, p99 ~0.061), 8 channels x40; W[3584x18944] ~ N(0,0.02).
3. vision-encoder linear: X[16384x1280] bf16 ~ Laplace(0,0.3) with 0.5% of elements
   replaced by +-U(10,50); W[1280x5120] ~ N(0,0.02).
4. prefill attention: Q[4096,28,128], K,V[4096,4,128] bf16 ~ N(0,1); K gets a
   per-(head, channel) N(0,1) bias; 4 fixed channels of Q and K x20; V tokens 0..15 x15.
5. decode: x[16x3584] as workload 1 (36 channels x30); W[3584x18944] ~ N(0,0.02);
   q[16,28,128] ~ N(0,1); per batch row a k/v history [8192, 4, 128] drawn like workload 4
   (the row's 4 spike channels also scale its q x20).

Weights are returned transposed, W^T [N, K], which is the layout the GEMM takes.
"""
import numpy as np


def f32_to_bf16_bits(x):
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r


def bf16_bits_to_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def rng_for(cfg):
    return np.random.default_rng(1000 + cfg)


def _spike_channels(rng, x, n, factor):
    ch = rng.choice(x.shape[1], n, replace=False)
    x[:, ch] *= factor
    return ch


def tiny(M=64, K=512, N=256, seed_cfg=1):
    """Workload 1 (sizes overridable for small parity cases). Returns dict(x f32 [M,K], w_t f32 [N,K])."""
    rng = rng_for(seed_cfg)
    x = rng.standard_normal((M, K)).astype(np.float32)
    _spike_channels(rng, x, max(1, round(0.01 * K)), 30.0)
    w = (0.02 * rng.standard_normal((K, N))).astype(np.float32)
    return {"x": x, "w_t": np.ascontiguousarray(w.T)}


def prefill_linear(M=4096, K=3584, N=18944, n_text=512, seed_cfg=2, with_weights=True):
    """Workload 2. Returns dict(x bf16 bits [M,K], w_t bf16 bits [N,K] or None)."""
    rng = rng_for(seed_cfg)
    n_vis = M - n_text
    x = np.empty((M, K), np.float32)
    x[:n_vis] = 0.2301 * rng.standard_t(2.12, size=(n_vis, K))
    x[n_vis:] = 0.006681 * rng.standard_t(2.12, size=(n_text, K))
    _spike_channels(rng, x, 8, 40.0)
    out = {"x": f32_to_bf16_bits(x), "n_visual": n_vis}
    if with_weights:
        w = (0.02 * rng.standard_normal((K, N))).astype(np.float32)
        out["w_t"] = f32_to_bf16_bits(np.ascontiguousarray(w.T))
    return out


def vision_linear(M=16384, K=1280, N=5120, seed_cfg=3, with_weights=True):
    """Workload 3. Returns dict(x bf16 bits [M,K], w_t bf16 bits [N,K] or None)."""
    rng = rng_for(seed_cfg)
    x = rng.laplace(0.0, 0.3, size=(M, K)).astype(np.float32)
    mask = rng.random((M, K)) < 0.005
    n = int(mask.sum())
    mag = rng.uniform(10.0, 50.0, size=n)
    sgn = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    x[mask] = (sgn * mag).astype(np.float32)
    out = {"x": f32_to_bf16_bits(x)}
    if with_weights:
        w = (0.02 * rng.standard_normal((K, N))).astype(np.float32)
        out["w_t"] = f32_to_bf16_bits(np.ascontiguousarray(w.T))
    return out


def attention_qkv(T=4096, Hq=28, Hkv=4, d=128, seed_cfg=4, rng=None):
    """Workload 4. Returns dict(q [T,Hq,d], k, v [T,Hkv,d]) as bf16 bits."""
    rng = rng_for(seed_cfg) if rng is None else rng
    q = rng.standard_normal((T, Hq, d)).astype(np.float32)
    k = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    v = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    k += rng.standard_normal((1, Hkv, d)).astype(np.float32)
    ch = rng.choice(d, 4, replace=False)
    q[:, :, ch] *= 20.0
    k[:, :, ch] *= 20.0
    v[:16] *= 15.0
    return {"q": f32_to_bf16_bits(q), "k": f32_to_bf16_bits(k), "v": f32_to_bf16_bits(v), "spike_channels": ch}


def decode_step(B=16, K=3584, N=18944, L=8192, Hq=28, Hkv=4, d=128, seed_cfg=5, with_weights=True,
                with_history=True):
    """Workload 5. x bf16 [B,K]; w_t bf16 [N,K]; q bf16 [B,Hq,d]; k_hist/v_hist bf16 [B,L,Hkv,d].

    Token L-1 of each history row is the new token of the step; tokens [0, L-1) are the prefill.
    """
    rng = rng_for(seed_cfg)
    x = rng.standard_normal((B, K)).astype(np.float32)
    _spike_channels(rng, x, max(1, round(0.01 * K)), 30.0)
    out = {"x": f32_to_bf16_bits(x)}
    if with_weights:
        w = (0.02 * rng.standard_normal((K, N))).astype(np.float32)
        out["w_t"] = f32_to_bf16_bits(np.ascontiguousarray(w.T))
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    if with_history:
        kh = np.empty((B, L, Hkv, d), np.uint16)
        vh = np.empty((B, L, Hkv, d), np.uint16)
        for b in range(B):
            k = rng.standard_normal((L, Hkv, d)).astype(np.float32)
            v = rng.standard_normal((L, Hkv, d)).astype(np.float32)
            k += rng.standard_normal((1, Hkv, d)).astype(np.float32)
            ch = rng.choice(d, 4, replace=False)
            k[:, :, ch] *= 20.0
            q[b][:, ch] *= 20.0
            v[:16] *= 15.0
            kh[b] = f32_to_bf16_bits(k)
            vh[b] = f32_to_bf16_bits(v)
        out["k_hist"] = kh
        out["v_hist"] = vh
    out["q"] = f32_to_bf16_bits(q)
    return out
