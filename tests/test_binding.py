"""Host-side checks of the Python binding and the bench's bookkeeping (no GPU): device-only inputs,
format tables that match the C enums, loud failure without the built library, and the traffic record
being dropped once the kernel sources it was measured on change."""
import json
import os

import pytest
import torch

import quantized_gemm_algorithm_amd as q
from quantized_gemm_algorithm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_cpu_tensors_are_refused():
    x = torch.zeros((4, 32), dtype=torch.float32)
    for call in (lambda: q.mix_quantize(x), lambda: q.mx_quantize(x, "fp4"), lambda: q.mix_kmean(x),
                 lambda: q.mix_underflow_map(x)):
        with pytest.raises(q.MixError):
            call()


def test_format_tables_match_the_header():
    hdr = open(os.path.join(ROOT, "include", "mixlib.h")).read()
    assert "MX_INT4 = 0, MX_FP4 = 1, MX_INT4_G16 = 2, MX_FP4_G16 = 3" in hdr
    assert q.MX_FMT == {"int4": 0, "fp4": 1, "int4g16": 2, "fp4g16": 3}
    assert q.MX_BLOCK == {"int4": 32, "fp4": 32, "int4g16": 16, "fp4g16": 16}
    assert len(q.UF_KINDS) == 7 and "MIX_UF_KINDS = 7" in hdr


def test_missing_library_fails_loudly(tmp_path):
    saved = _lib._lib
    try:
        _lib._lib = None
        with pytest.raises(RuntimeError, match="libmix.so not found"):
            _lib.load(str(tmp_path / "libmix.so"))
    finally:
        _lib._lib = saved


def test_traffic_record_follows_the_sources(tmp_path, monkeypatch):
    import bench
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert set(rec) >= {"prefill_linear", "vision_linear", "decode", "attention_prefill"}
    for w, r in rec.items():
        assert r["traffic_bytes"] == r["fetch_bytes"] + r["write_bytes"] > 0
    # a copy of the tree whose kernel source differs by one byte: the record no longer applies
    fake = tmp_path / "repo"
    (fake / "profiles").mkdir(parents=True)
    (fake / "profiles" / "traffic.json").write_text(json.dumps(rec))
    for f in rec["prefill_linear"]["source_files"]:
        dst = fake / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, f), "rb").read())
    monkeypatch.setattr(bench.os.path, "abspath", lambda p: str(fake / "bench.py"))
    assert bench.measured_traffic("prefill_linear") == rec["prefill_linear"]["traffic_bytes"]
    src = fake / rec["prefill_linear"]["source_files"][0]
    src.write_bytes(src.read_bytes() + b" ")
    assert bench.measured_traffic("prefill_linear") is None
    assert bench.measured_traffic("no_such_workload") is None
