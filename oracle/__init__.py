"""CPU oracle for the MiX (Micro-Inverted-Scaling) hot path.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously-correct NumPy
implementation of what the GPU library computes. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The product path (``quantized_gemm_algorithm_amd``) never imports or
calls anything here, and this package imports nothing from the product path: the
two share no code, no tables and no constants.

Sources. Citations name the page and the section, figure, table or equation on
it:

* **P1** -- the pchao.org digest of the paper, titled
  "MiX：面向端到端低比特视觉语言模型加速的微反缩放" (sections: 快速导读 quick
  read, 这篇论文解决什么问题 problem, 核心创新 innovations, 方法概览 method
  overview, 逐图理解论文 figure walk, 实验如何设计 experiment design,
  关键结果与论文证据 key results, 阅读时需要注意 caveats).
* **P2..P5** -- the arxivdaily, arxiv-daily-jp, mlsanity and weekinpapers pages
  for "MiX: Micro-Inverted-Scaling for End-to-End Low-Bit Vision-Language Model
  Acceleration"; they only restate the abstract.

Where the pages leave a point open, the oracle follows a stated reading
(``READINGS`` below, keyed D1..D18). The GPU path implements the same readings
independently.

Parity status of each function is given in its module docstring. Functions with
no independent pin say "parity unpinned" there.
"""

READINGS = {
    "D1": "Emax is a 4-bit biased exponent, bias 7: Emax = clamp(floor(log2 amax), -7, 8).",
    "D2": "MiX-4.5b: Emax from the 32-block max; each 8-element sub-block's mshared from that sub-block's max.",
    "D3": "mshared = the top 3 fraction bits of the max element's significand (truncation, no carry).",
    "D4": "Shared field: 4.25b byte = Emax code in bits 3:0, m in 6:4. 4.5b u16 = Emax code 3:0, m0 6:4, "
          "m1 9:7, m2 12:10, m3 15:13.",
    "D5": "Asymmetric zero: nibble 0x7 is zero; nibble 0xF is +M*2^(Emax-7); negatives stop at dE=6.",
    "D6": "Nibble = (sign<<3)|dE; element 2j in the low nibble of byte j. MX codes use the same order.",
    "D7": "Each element takes the representable value nearest to it; an exact tie goes to the smaller magnitude.",
    "D8": "MXFP4 shared exponent X = ceil(log2 amax) - 2 (the ceil variant), clamped to >= -127.",
    "D9": "MXINT4: X = floor(log2 amax) clamped to [-125,127]; q = clamp(RNE(x*2^(2-X)), -7, 7); value q*2^(X-2).",
    "D10": "MX element rounding is round-to-nearest-even on the element grid, saturating; FP4 keeps the sign "
           "of zero inside a nonzero block.",
    "D11": "An all-zero block: MiX shared field 0 and all nibbles 0x7; MX scale byte 0 and all nibbles 0. "
           "Non-finite input is rejected.",
    "D12": "GEMM operands are blocked along the contraction axis; B is passed as W^T [N,K].",
    "D13": "fp32 output is the fp32 accumulator; bf16 output is the RNE rounding of it.",
    "D14": "Attention: Q and P are MiX-4.5b (activations); smoothed K and V are MXFP4 (cached). K and Q "
           "blocks run along the head dimension; V and P blocks run along tokens.",
    "D15": "K-mean per (kv-head, channel) over all prefill tokens: exact sum, divided by T in fp64, then "
           "rounded to fp32. Smoothing is fp32(K - mu).",
    "D16": "Softmax in fp32: z = fp32(S) * fp32(1/sqrt(d)); m = exact row max over unmasked keys; "
           "p = exp(z - m); l = sum of the unquantized p; P-hat = MiX-4.5b(p) along keys; O = (P-hat V-hat)/l.",
    "D17": "Decode: V blocks cover tokens [32j, 32j+32); a trailing partial block is coded from the tokens "
           "present, zero-padded.",
    "D18": "GEMM/BMM tolerance: per element |c - c_ref| <= 1e-5 * sum|a b| and normwise 1e-5, on fp32 output.",
}
