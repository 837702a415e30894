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
    import hashlib

    import bench
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert set(rec) >= {"prefill_linear", "vision_linear", "decode", "attention_prefill"}
    for w, r in rec.items():
        assert r["traffic_bytes"] == r["fetch_bytes"] + r["write_bytes"] > 0
    # a copy of the tree with a record taken on its sources applies; once a kernel source differs by
    # one byte it no longer does
    fake = tmp_path / "repo"
    (fake / "profiles").mkdir(parents=True)
    r = dict(rec["prefill_linear"])
    h = hashlib.sha256()
    for f in r["source_files"]:
        dst = fake / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, f), "rb").read())
        h.update(dst.read_bytes())
    r["source_sha256"] = h.hexdigest()
    (fake / "profiles" / "traffic.json").write_text(json.dumps({"prefill_linear": r}))
    monkeypatch.setattr(bench.os.path, "abspath", lambda p: str(fake / "bench.py"))
    assert bench.measured_traffic("prefill_linear") == r["traffic_bytes"]
    src = fake / r["source_files"][0]
    src.write_bytes(src.read_bytes() + b" ")
    assert bench.measured_traffic("prefill_linear") is None
    assert bench.measured_traffic("no_such_workload") is None


def test_caller_outputs_and_decode_shapes_are_checked(monkeypatch):
    # the C-ABI takes only a pointer and a row pitch for C, so the binding refuses an output that
    # does not hold [M, N] with unit column stride, before any library call (CPU tensors stand in
    # for device ones here: the device check is switched off)
    monkeypatch.setattr(q, "_need_cuda", lambda *a: None)
    monkeypatch.setattr(q, "_lib_", lambda: (_ for _ in ()).throw(AssertionError("library reached")))
    a = q.AImage(torch.zeros(16, dtype=torch.uint8), 64, 256)
    b = q.BImage(torch.zeros(16, dtype=torch.uint8), "fp4", 300, 256, None)
    for bad in (torch.zeros((64, 299)), torch.zeros((63, 300)), torch.zeros((300, 64)).t(),
                torch.zeros((64, 300), dtype=torch.float16), torch.zeros(64 * 300)):
        with pytest.raises(q.MixError):
            q.mix_mx_gemm_images(a, b, out=bad)
    ac, bc = torch.zeros((64, 128), dtype=torch.uint8), torch.zeros((300, 128), dtype=torch.uint8)
    with pytest.raises(q.MixError):
        q.mix_mx_gemm(ac, None, "4.5b", bc, None, "fp4", out=torch.zeros((64, 200)))
    with pytest.raises(q.MixError):
        q.mix_mx_gemm_eq6(ac, None, "4.5b", bc, None, "fp4", out=torch.zeros((64, 300))[:, ::2])
    with pytest.raises(q.MixError):
        q.mix_mx_gemm_images_quantize(a, q.BImage(None, "fp4", 256, 256, None), image=False,
                                      out=torch.zeros((64, 256)))

    class FakeCache:
        B, Lmax, Hkv, d = 2, 64, 1, 32

    bf = torch.bfloat16
    qv, kn = torch.zeros((2, 2, 32), dtype=bf), torch.zeros((2, 1, 32), dtype=bf)
    pos, mu = torch.zeros(2, dtype=torch.int32), torch.zeros((2, 1, 32))
    ok = dict(q=qv, k_new=kn, v_new=kn, cache=FakeCache(), pos=pos, max_pos=10, mu=mu)
    for key, val in (("q", torch.zeros((3, 2, 32), dtype=bf)), ("q", torch.zeros((2, 2, 64), dtype=bf)),
                     ("q", torch.zeros((2, 32, 2), dtype=bf).transpose(1, 2)), ("k_new", torch.zeros((2, 2, 32), dtype=bf)),
                     ("pos", torch.zeros(2, dtype=torch.int64)), ("mu", torch.zeros((2, 16)))):
        with pytest.raises(q.MixError):
            q.mix_attn_decode(**{**ok, key: val})
    with pytest.raises(q.MixError):
        q.mix_attn_prefill(torch.zeros((8, 2, 32), dtype=bf), torch.zeros((8, 1, 64), dtype=bf),
                           torch.zeros((8, 1, 64), dtype=bf))
