"""Underflow map on the GPU against the oracle: per-column counts of nonzero elements each format
codes to zero (MXINT4, MXFP4 floor and ceil, NVFP4 with 32-element blocks, MiX-4.25b/4.5b), bit
for bit, and the operand's largest magnitude; fp32 and bf16 inputs, with and without smoothing,
ragged row counts, subnormal and zero elements, and the attention workload's keys at full size."""
import numpy as np
import pytest
import torch

from helpers import dev_bf16, dev_f32, host
from oracle.underflow import underflow_map as o_map
from quantized_gemm_algorithm_amd import synth

pytestmark = pytest.mark.gpu


def _q():
    import quantized_gemm_algorithm_amd as q
    return q


def _check(got, want, what):
    got = host(got)
    if not np.array_equal(got, want):
        k, c = np.argwhere(got != want)[0]
        raise AssertionError(f"{what}: {int((got != want).sum())} counts differ; first kind {k} column {c}: "
                             f"{got[k, c]} vs {want[k, c]}")


@pytest.mark.parametrize("rows,cols", [(1, 32), (7, 96), (301, 512), (64, 544), (130, 1056)])
@pytest.mark.parametrize("smooth", [False, True])
def test_underflow_map_fp32(rows, cols, smooth):
    q = _q()
    rng = np.random.default_rng(rows * 31 + cols + smooth)
    x = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-10, 4, (rows, cols)))).astype(np.float32)
    x[:, rng.integers(0, cols)] *= 40.0              # an outlier channel
    x[0, :16] = 0.0
    x[-1, -32:] = 0.0                                # an all-zero block
    x[rows // 2, 3] = -0.0
    mu = (rng.standard_normal(cols) * 0.5).astype(np.float32) if smooth else None
    counts, amax = q.mix_underflow_map(dev_f32(x), mu=dev_f32(mu) if smooth else None)
    torch.cuda.synchronize()
    _check(counts, o_map(x, "f32", mu), f"fp32 {rows}x{cols} smooth={smooth}")
    xs = (x - mu).astype(np.float32) if smooth else x
    assert float(host(amax)[0]) == float(np.abs(xs).max())


@pytest.mark.parametrize("rows,cols", [(5, 64), (257, 512)])
def test_underflow_map_bf16(rows, cols):
    q = _q()
    rng = np.random.default_rng(rows + cols)
    x = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-6, 6, (rows, cols)))).astype(np.float32)
    bits = synth.f32_to_bf16_bits(x)
    counts, _ = q.mix_underflow_map(dev_bf16(bits))
    mu = rng.standard_normal(cols).astype(np.float32)
    counts_mu, _ = q.mix_underflow_map(dev_bf16(bits), mu=dev_f32(mu))
    torch.cuda.synchronize()
    _check(counts, o_map(bits, "bf16"), f"bf16 {rows}x{cols}")
    _check(counts_mu, o_map(bits, "bf16", mu), f"bf16 smoothed {rows}x{cols}")


def test_underflow_map_tiny_magnitudes_and_edges():
    q = _q()
    rng = np.random.default_rng(3)
    # subnormal and near-subnormal blocks (MX exponent clamps, E4M3 block scales that underflow)
    x = (rng.standard_normal((9, 128)) * np.exp2(rng.integers(-149, -100, (9, 128)))).astype(np.float32)
    x[0] = (rng.standard_normal(128) * 1e3).astype(np.float32)   # the tensor maximum far above
    counts, amax = q.mix_underflow_map(dev_f32(x))
    torch.cuda.synchronize()
    _check(counts, o_map(x, "f32"), "tiny magnitudes")
    z = np.zeros((4, 64), np.float32)
    counts, amax = q.mix_underflow_map(dev_f32(z))
    empty, amax0 = q.mix_underflow_map(torch.empty((0, 64), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert not host(counts).any() and float(host(amax)[0]) == 0.0
    assert not host(empty).any() and float(host(amax0)[0]) == 0.0


@pytest.mark.parametrize("smooth", [False, True])
def test_underflow_map_attention_keys_full_size(smooth):
    # the keys of the prefill-attention workload (4096 tokens x 4 KV heads x 128), blocks along the
    # head dimension, unsmoothed and with the per-channel K-mean subtracted
    q = _q()
    g = synth.attention_qkv()
    k = np.ascontiguousarray(g["k"].reshape(4096, 512))
    kd = dev_bf16(k)
    mu = q.mix_kmean(kd) if smooth else None
    counts, _ = q.mix_underflow_map(kd, mu=mu)
    torch.cuda.synchronize()
    _check(counts, o_map(k, "bf16", host(mu) if smooth else None), f"attention keys smooth={smooth}")
