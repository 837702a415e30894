"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source is compiled with the sanitizers on its host pass only (device code is built as usual and
never runs here), linked with tests/sanitize/abi_checks.c, and the driver calls every entry point
with invalid arguments and extreme extents: each call must return its documented status with no
sanitizer report (an out-of-bounds access, a signed overflow in a size computation, an enum read
outside its range). No GPU is needed: every call fails validation before any HIP call.
"""
import hashlib
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_gemm_algorithm_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "abi_checks.c")
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers absent")

# sanitizers on the host pass only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _sources():
    from quantized_gemm_algorithm_amd.build import SOURCES
    return SOURCES


def _stamp():
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)) + ["../../include/mixlib.h", DRIVER]:
        path = os.path.join(CSRC, name)
        if os.path.isfile(path):
            h.update(name.encode())
            h.update(open(path, "rb").read())
    h.update(" ".join(HOST_SAN).encode())
    return h.hexdigest()


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(" ".join(cmd) + "\n" + (r.stdout + r.stderr)[-4000:])


def _build():
    exe = os.path.join(OUT, "abi_checks")
    stamp_file = os.path.join(OUT, "stamp")
    stamp = _stamp()
    if os.path.exists(exe) and os.path.exists(stamp_file) and open(stamp_file).read() == stamp:
        return exe
    shutil.rmtree(OUT, ignore_errors=True)
    os.makedirs(OUT)
    objs = []
    cmds = []
    for src in _sources():
        obj = os.path.join(OUT, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *HOST_SAN,
                     "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                     "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj])
    drv = os.path.join(OUT, "abi_checks.o")
    cmds.append([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                 "-I", os.path.join(ROOT, "include"), "-c", DRIVER, "-o", drv])
    with ThreadPoolExecutor(max_workers=4) as ex:
        list(ex.map(_run, cmds))
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-o", exe, drv, *objs])
    open(stamp_file, "w").write(stamp)
    return exe


def test_host_checks_clean_under_sanitizers():
    exe = _build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "all host checks passed" in out
