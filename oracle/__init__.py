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

Where the pages leave a point open, the oracle follows a stated reading. The
readings are labelled D1..D25 in every source of this repository; each oracle
module states in words, next to its label, each reading it takes, and the GPU
path implements the same readings independently.

Parity status of each function is given in its module docstring. Functions with
no independent pin say "parity unpinned" there.
"""
