"""The synthetic workload generators reproduce the activation statistics the pages report
(P1, 这篇论文解决什么问题 (problem), Fig. 1: visual channels mean 0.312 and p99 2.07, text channels
mean 0.0091 and p99 0.061) on the non-spike channels, within 5%."""
import numpy as np

from quantized_gemm_algorithm_amd.synth import bf16_bits_to_f32, prefill_linear, rng_for


def test_prefill_linear_statistics():
    g = prefill_linear(with_weights=False)
    x = np.abs(bf16_bits_to_f32(g["x"]).astype(np.float64))
    # channels that carry the x40 spikes are excluded (the 8 with the largest column mean)
    col = x.mean(axis=0)
    keep = np.argsort(col)[:-8]
    vis, txt = x[: g["n_visual"]][:, keep], x[g["n_visual"]:][:, keep]
    for arr, mean, p99 in ((vis, 0.312, 2.07), (txt, 0.0091, 0.061)):
        assert abs(arr.mean() / mean - 1) < 0.05, arr.mean()
        assert abs(np.quantile(arr, 0.99) / p99 - 1) < 0.05, np.quantile(arr, 0.99)


def test_generators_are_seeded():
    a = rng_for(2).standard_normal(4)
    b = rng_for(2).standard_normal(4)
    assert np.array_equal(a, b)
