"""K-smoothed attention over MiX/MX-coded operands -- oracle (test infrastructure only).

What it follows:

* P1, 方法概览 (method overview), last bullet: Keys are smoothed training-free by
  subtracting their mean over tokens per channel (gamma(K) = K - mean(K), the
  SageAttention technique); softmax is unchanged by a constant shift per query
  row; decode keeps the per-channel mean from prefill frozen so the Key cache is
  never re-read or re-quantised.
* P1, 关键结果与论文证据 (key results), first bullet, and 阅读时需要注意
  (caveats), first bullet: the same static-mean choice and its reason.
* P1, 核心创新 (innovations), third bullet, and 这篇论文解决什么问题 (problem),
  Table I paragraph: the attention BMMs and the KV cache are coded low-bit too.
* P1, method overview, dual-format bullet and the abstract (P2..P5): activations
  take the MiX format, cached/stationary operands the MX format.

Readings: D14 (Q, P -> MiX-4.5b; smoothed K, V -> MXFP4; K and Q blocked along
the head dimension, V and P along tokens), D15 (K-mean arithmetic), D16
(softmax in fp32 with an exact row max and an unnormalised p; l sums the
unquantised p), D17 (partial V block at decode).

Pins (tests/test_oracle_attention.py): the K-mean against a brute-force Fraction
mean; smoothing invariance of the softmax on unquantised inputs; the staged
pipeline against a hand-built single-head example; decode with all keys present
equals the prefill's last row with the same mean. The composition: query head h
reads KV head h // (Hq / Hkv) (S against hand-indexed products with two different
key sets); V is blocked along tokens (a one-token spike moves only its own
block's scale in every channel, and a closed-form output where the token
blocking zeroes small values); the softmax scale is 1/sqrt(d) (d = 64 gives
z = S / 8 exactly, checked against exp of the hand-scaled logits).
"""
import math

import numpy as np

from .mix import mix_dequantize, mix_quantize
from .mx import mx_dequantize, mx_quantize
from .numerics import as_f32, round_f64_to_bf16_bits

BLOCK = 32


def kmean_ref(k, dtype="bf16"):
    """mu[h, c] = fp32( exact_sum_t K[t, h, c] / T ) with the division in fp64 (D15). k: [T, Hkv, d]."""
    kf = as_f32(np.asarray(k).reshape(k.shape[0], -1), dtype).astype(np.float64)
    T = kf.shape[0]
    mu = np.array([math.fsum(kf[:, c]) / T for c in range(kf.shape[1])], dtype=np.float64)
    return mu.astype(np.float32).reshape(k.shape[1], k.shape[2])


def code_q(q, dtype="bf16"):
    """Q [T, H, d] -> MiX-4.5b along d: codes [T, H, d/2], shared u16 [T, H, d/32]."""
    T, H, d = q.shape
    c, s = mix_quantize(np.asarray(q).reshape(T * H, d), "4.5b", dtype)
    return c.reshape(T, H, d // 2), s.reshape(T, H, d // 32)


def code_k(k, mu, dtype="bf16"):
    """K [T, Hkv, d], mu [Hkv, d] -> MXFP4(fp32(K - mu)) along d: codes [T, Hkv, d/2], scales [T, Hkv, d/32]."""
    T, H, d = k.shape
    kf = as_f32(np.asarray(k).reshape(T * H, d), dtype).reshape(T, H, d)
    codes = np.empty((T, H, d // 2), np.uint8)
    scales = np.empty((T, H, d // 32), np.uint8)
    for h in range(H):
        codes[:, h], scales[:, h] = mx_quantize(kf[:, h, :], "fp4", "f32", mu=mu[h])
    return codes, scales


def code_v(v, dtype="bf16"):
    """V [T, Hkv, d] -> MXFP4 along tokens: codes [Hkv, d, Tp/2], scales [Hkv, d, Tp/32].

    T is zero-padded up to a multiple of 32 (D17); padded tokens carry zero.
    """
    T, H, d = v.shape
    vf = as_f32(np.asarray(v).reshape(T * H, d), dtype).reshape(T, H, d)
    Tp = -(-T // BLOCK) * BLOCK
    vp = np.zeros((Tp, H, d), np.float32)
    vp[:T] = vf
    codes = np.empty((H, d, Tp // 2), np.uint8)
    scales = np.empty((H, d, Tp // 32), np.uint8)
    for h in range(H):
        codes[h], scales[h] = mx_quantize(np.ascontiguousarray(vp[:, h, :].T), "fp4", "f32")
    return codes, scales


def softmax_scale(d):
    """fp32 RNE of 1/sqrt(d) (D16)."""
    return np.float32(1.0 / math.sqrt(d))


def softmax_rows(s_rows, n_valid, d):
    """Unnormalised fp32 softmax of rows of fp32 logits (D16).

    s_rows: float32 [R, L]; n_valid: int [R], keys [0, n_valid) are unmasked.
    Returns (p float32 [R, L] with masked entries 0, l float32 [R], m float32 [R]).
    p = exp(z - m) is the correctly rounded fp32 value of the exponential of the
    fp32 difference; l is the fp32 rounding of the exact sum of p.
    """
    s = np.asarray(s_rows, np.float32)
    R, L = s.shape
    z = (s * softmax_scale(d)).astype(np.float32)
    mask = np.arange(L)[None, :] < np.asarray(n_valid)[:, None]
    m = np.where(mask, z, -np.inf).max(axis=1).astype(np.float32)
    diff = np.where(mask, z - m[:, None], np.float32(-np.inf)).astype(np.float32)
    p = np.exp(diff.astype(np.float64)).astype(np.float32)
    p = np.where(mask, p, np.float32(0.0)).astype(np.float32)
    l = np.array([math.fsum(row) for row in p.astype(np.float64)]).astype(np.float32)
    return p, l, m


def code_p(p):
    """P [R, L] fp32 -> MiX-4.5b along keys (L % 32 == 0)."""
    return mix_quantize(np.asarray(p, np.float32), "4.5b", "f32")


def attn_prefill_ref(q, k, v, dtype="bf16", causal=True, rows=None, heads=None):
    """Oracle prefill for Q [T, Hq, d], K/V [T, Hkv, d]; a ragged T is zero-padded to a multiple of 32.

    ``rows``/``heads`` restrict which query rows and heads are computed (all by
    default); everything they depend on (all keys, the K-mean) is still exact.
    Returns a dict with mu, the coded operands, and per (head, row): S (fp64, exact
    dot products), p, l, the P-hat codes, O before rounding (fp64) and O as bf16 bits.
    """
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    rows = np.arange(T) if rows is None else np.asarray(rows)
    heads = np.arange(Hq) if heads is None else np.asarray(heads)
    mu = kmean_ref(k, dtype)
    qc, qs = code_q(np.asarray(q)[rows], dtype)
    kc, ks = code_k(k, mu, dtype)
    vc, vs = code_v(v, dtype)
    out = {"mu": mu, "q_codes": qc, "q_shared": qs, "k_codes": kc, "k_scales": ks,
           "v_codes": vc, "v_scales": vs, "rows": rows, "heads": heads}
    n_valid = (rows + 1) if causal else np.full(len(rows), T)
    S_all, p_all, l_all, pc_all, ps_all, o_all, ob_all = [], [], [], [], [], [], []
    for h in heads:
        hk = h // G
        qd = mix_dequantize(qc[:, h], qs[:, h], "4.5b")  # [R, d]
        kd = mx_dequantize(kc[:, hk], ks[:, hk], "fp4")  # [T, d]
        vd = mx_dequantize(vc[hk], vs[hk], "fp4")  # [d, T]
        Tp = vd.shape[1]  # T rounded up to 32: keys past T are masked and code as zero (D17)
        S = np.zeros((len(rows), Tp))
        S[:, :T] = qd @ kd.T  # exact products, fp64 sum
        S = np.where(np.arange(Tp)[None, :] < n_valid[:, None], S, 0.0)
        p, l, _ = softmax_rows(S.astype(np.float32), n_valid, d)
        pc, ps = code_p(p)
        pd = mix_dequantize(pc, ps, "4.5b")
        o = (pd @ vd.T) / l.astype(np.float64)[:, None]
        S_all.append(S); p_all.append(p); l_all.append(l); pc_all.append(pc); ps_all.append(ps)
        o_all.append(o); ob_all.append(round_f64_to_bf16_bits(o))
    out.update(S=np.stack(S_all), p=np.stack(p_all), l=np.stack(l_all), p_codes=np.stack(pc_all),
               p_shared=np.stack(ps_all), o=np.stack(o_all), o_bf16=np.stack(ob_all))
    return out


def attn_decode_ref(q, k_hist, v_hist, mu, lens, dtype="bf16"):
    """Oracle decode: q [B, Hq, d]; k_hist/v_hist [B, Lmax, Hkv, d] hold every token so far
    (the new one included) in rows [0, lens[b]); mu [B, Hkv, d] is the frozen prefill mean.

    No mask beyond the sequence length. Returns dict with S, p, l, P codes, O (fp64) and O bf16 bits,
    each [B, Hq, ...].
    """
    B, Hq, d = q.shape
    Hkv = k_hist.shape[2]
    G = Hq // Hkv
    res = {k_: [] for k_ in ("S", "p", "l", "p_codes", "p_shared", "o", "o_bf16")}
    for b in range(B):
        L = int(lens[b])
        Lp = -(-L // BLOCK) * BLOCK
        qc, qs = code_q(np.asarray(q)[b][None], dtype)
        kc, ks = code_k(np.asarray(k_hist)[b, :L], mu[b], dtype)
        vc, vs = code_v(np.asarray(v_hist)[b, :L], dtype)
        Sb, pb, lb, pcb, psb, ob, obb = [], [], [], [], [], [], []
        for h in range(Hq):
            hk = h // G
            qd = mix_dequantize(qc[:, h], qs[:, h], "4.5b")  # [1, d]
            kd = mx_dequantize(kc[:, hk], ks[:, hk], "fp4")  # [L, d]
            vd = mx_dequantize(vc[hk], vs[hk], "fp4")  # [d, Lp]
            S = np.zeros((1, Lp))
            S[:, :L] = qd @ kd.T
            p, l, _ = softmax_rows(S.astype(np.float32), np.array([L]), d)
            pc, ps = code_p(p)
            pd = mix_dequantize(pc, ps, "4.5b")
            o = (pd @ vd.T) / np.float64(l[0])
            Sb.append(S[0]); pb.append(p[0]); lb.append(l[0]); pcb.append(pc[0]); psb.append(ps[0])
            ob.append(o[0]); obb.append(round_f64_to_bf16_bits(o[0]))
        for key, val in zip(("S", "p", "l", "p_codes", "p_shared", "o", "o_bf16"), (Sb, pb, lb, pcb, psb, ob, obb)):
            res[key].append(np.stack(val) if np.ndim(val[0]) else np.array(val))
    return res


def linear_ref(x, w_t, dtype="bf16", a_fmt="4.5b", b_fmt="fp4", rows=None, cols=None):
    """y = deq(MiX(x)) . deq(MX(W^T))^T in fp64. x [M, K]; w_t [N, K] (W transposed).

    ``rows``/``cols`` select entries (paired) to compute instead of the full product.
    """
    from .gemm import gemm_ref, gemm_ref_entries
    ac, as_ = mix_quantize(x, a_fmt, dtype)
    bc, bs = mx_quantize(w_t, b_fmt, dtype)
    ad = mix_dequantize(ac, as_, a_fmt)
    bd = mx_dequantize(bc, bs, b_fmt)
    if rows is None:
        return gemm_ref(ad, bd)
    return gemm_ref_entries(ad, bd, rows, cols)
