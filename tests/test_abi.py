"""The C-ABI library loads, exports every entry point declared in include/mixlib.h, and rejects bad
arguments on the host before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mixlib.h")
LIB = os.path.join(ROOT, "quantized_gemm_algorithm_amd", "libmix.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmix.so not built")

MIX_OK, MIX_E_NULL, MIX_E_SHAPE, MIX_E_ALIGN, MIX_E_ENUM, MIX_E_UNSUPPORTED, MIX_E_HIP, MIX_E_WORKSPACE = range(8)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^(?:const\s+)?\w+\s*\*?\s+(mix\w+|mx\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    from quantized_gemm_algorithm_amd import _lib
    return _lib.load(LIB)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 15, names
    for n in names:
        assert hasattr(lib, n), n
    from quantized_gemm_algorithm_amd._lib import SIGNATURES
    assert set(names) == set(SIGNATURES), set(names) ^ set(SIGNATURES)


def test_version_and_status_strings(lib):
    assert lib.mix_abi_version() == 4
    for s in range(8):
        assert lib.mix_status_str(s)
    assert lib.mix_status_str(99) == b"unknown status"


P = ctypes.c_void_p
FAKE = P(0x10000)        # never dereferenced: validation fails or the call is empty first
MISALIGNED = P(0x10001)


def test_quantize_validation(lib):
    # unknown format / dtype
    assert lib.mix_quantize(7, FAKE, 0, 1, 32, 32, FAKE, FAKE, None) == MIX_E_ENUM
    assert lib.mix_quantize(1, FAKE, 5, 1, 32, 32, FAKE, FAKE, None) == MIX_E_ENUM
    assert b"dtype" in lib.mix_last_error()
    # shapes
    assert lib.mix_quantize(1, FAKE, 0, 1, 33, 33, FAKE, FAKE, None) == MIX_E_SHAPE
    assert lib.mix_quantize(1, FAKE, 0, -1, 32, 32, FAKE, FAKE, None) == MIX_E_SHAPE
    assert lib.mix_quantize(1, FAKE, 0, 2, 64, 32, FAKE, FAKE, None) == MIX_E_SHAPE
    # null pointers
    assert lib.mix_quantize(1, None, 0, 1, 32, 32, FAKE, FAKE, None) == MIX_E_NULL
    assert lib.mix_quantize(1, FAKE, 0, 1, 32, 32, None, FAKE, None) == MIX_E_NULL
    # alignment: pointer and pitch
    assert lib.mix_quantize(1, MISALIGNED, 0, 1, 32, 32, FAKE, FAKE, None) == MIX_E_ALIGN
    assert lib.mix_quantize(1, FAKE, 1, 2, 32, 36, FAKE, FAKE, None) == MIX_E_ALIGN
    # empty calls succeed without touching memory
    assert lib.mix_quantize(1, None, 0, 0, 32, 32, None, None, None) == MIX_OK
    assert lib.mix_quantize(1, None, 0, 5, 0, 0, None, None, None) == MIX_OK
    assert lib.mx_quantize(4, FAKE, 0, 1, 32, 32, None, FAKE, FAKE, None) == MIX_E_ENUM
    assert lib.mx_quantize(1, FAKE, 0, 1, 32, 32, MISALIGNED, FAKE, FAKE, None) == MIX_E_ALIGN
    assert lib.mx_quantize(1, None, 0, 0, 64, 64, None, None, None, None) == MIX_OK
    assert lib.mx_quantize_cols(FAKE, 1, 10, 4, 2, FAKE, FAKE, None) == MIX_E_SHAPE


def test_gemm_validation(lib):
    def gemm(*a):
        return lib.mix_mx_gemm(*a[:-1], None, 0, a[-1])

    for fn in (gemm, lib.mix_mx_gemm_eq6):
        assert fn(3, FAKE, FAKE, 1, FAKE, FAKE, 4, 4, 32, FAKE, 0, 4, None) == MIX_E_ENUM
        assert fn(1, FAKE, FAKE, 9, FAKE, FAKE, 4, 4, 32, FAKE, 0, 4, None) == MIX_E_ENUM
        assert fn(1, FAKE, FAKE, 1, FAKE, FAKE, 4, 4, 40, FAKE, 0, 4, None) == MIX_E_SHAPE
        assert fn(1, FAKE, FAKE, 1, FAKE, FAKE, 4, 4, 32, FAKE, 0, 3, None) == MIX_E_SHAPE
        assert fn(1, FAKE, FAKE, 1, FAKE, FAKE, -4, 4, 32, FAKE, 0, 4, None) == MIX_E_SHAPE
        assert fn(1, None, FAKE, 1, FAKE, FAKE, 4, 4, 32, FAKE, 0, 4, None) == MIX_E_NULL
        assert fn(1, FAKE, FAKE, 1, FAKE, FAKE, 4, 4, 32, None, 0, 4, None) == MIX_E_NULL
        assert fn(1, MISALIGNED, FAKE, 1, FAKE, FAKE, 4, 4, 32, FAKE, 0, 4, None) == MIX_E_ALIGN
        assert fn(1, None, None, 1, None, None, 0, 4, 32, None, 0, 4, None) == MIX_OK
        assert fn(1, None, None, 1, None, None, 4, 0, 32, None, 0, 0, None) == MIX_OK
        assert fn(1, FAKE, FAKE, 1, FAKE, FAKE, 2**31, 4, 32, FAKE, 0, 4, None) == MIX_E_SHAPE
    # fast-path workspace size: zero when the shape does not take it
    # E4M3 A + per-(K step, 256-row tile) 1 KB scale blocks for A and B + the B operand (MXFP4 codes
    # step-major, E4M3 B for MXINT4) + the B scales per 16-row group
    assert lib.mix_mx_gemm_workspace_bytes(1, 1, 4096, 18944, 3584) == (4096 * 3584 + 28 * 16 * 1024 + 28 * 74 * 1024
                                                                       + 18944 * 1792 + 1184 * 28 * 64)
    assert lib.mix_mx_gemm_workspace_bytes(1, 0, 256, 256, 128) == 256 * 128 + 1024 + 1024 + 256 * 128 + 16 * 64
    assert lib.mix_mx_gemm_workspace_bytes(1, 1, 256, 256, 96) == 0
    # M <= 16 streams the weights through the same images
    assert lib.mix_mx_gemm_workspace_bytes(1, 1, 16, 18944, 3584) == (16 * 3584 + 28 * 1024 + 28 * 74 * 1024
                                                                     + 18944 * 1792 + 1184 * 28 * 64)
    assert lib.mix_mx_gemm_workspace_bytes(1, 1, 32, 18944, 3584) == 0
    # a misaligned workspace is rejected when the fast path is taken
    assert lib.mix_mx_gemm(1, FAKE, FAKE, 1, FAKE, FAKE, 256, 256, 128, FAKE, 0, 256, MISALIGNED, 1 << 20,
                           None) == MIX_E_ALIGN


def test_kmean_validation(lib):
    assert lib.mix_kmean(FAKE, 1, 0, 32, 32, FAKE, None) == MIX_E_SHAPE
    assert lib.mix_kmean(None, 1, 4, 32, 32, FAKE, None) == MIX_E_NULL
    assert lib.mix_kmean(FAKE, 1, 4, 32, 16, FAKE, None) == MIX_E_SHAPE
    assert lib.mix_kmean(None, 1, 4, 0, 0, None, None) == MIX_OK
    assert lib.mix_kmean(FAKE, 1, 4, 40, 40, FAKE, None) == MIX_E_SHAPE
    assert lib.mix_kmean(MISALIGNED, 1, 4, 32, 32, FAKE, None) == MIX_E_ALIGN
    assert lib.mix_kmean(FAKE, 1, 4, 32, 36, FAKE, None) == MIX_E_ALIGN


def test_image_sizes(lib):
    # A image: E4M3 [M, K] (256-byte rounded) + one 1 KB scale block per (128-wide K step, 256-row tile)
    assert lib.mix_gemm_a_image_bytes(4096, 3584) == 4096 * 3584 + 28 * 16 * 1024
    assert lib.mix_gemm_a_image_bytes(1, 128) == 256 + 1024
    assert lib.mix_gemm_a_image_bytes(4, 96) == 0
    assert lib.mix_gemm_a_image_bytes(0, 128) == 0
    # B image: permuted scales + the operand (MXFP4: the codes step-major, N K / 2 bytes; MXINT4: E4M3
    # bytes of q/4, N K) + the scales per 16-row group [ceil(N/16)][K/128][64] for the small-M product
    # (each part 256-byte rounded)
    assert lib.mx_gemm_b_image_bytes(1, 18944, 3584) == 28 * 74 * 1024 + 18944 * 1792 + 1184 * 28 * 64
    assert lib.mx_gemm_b_image_bytes(1, 300, 256) == 2 * 2 * 1024 + 300 * 128 + 2560
    assert lib.mx_gemm_b_image_bytes(0, 300, 256) == 2 * 2 * 1024 + 300 * 256 + 2560
    assert lib.mx_gemm_b_image_bytes(4, 300, 256) == 0
    assert lib.mx_gemm_b_image_bytes(1, 300, 0) == 0


def test_image_validation(lib):
    A16 = P(0x10010)  # 16-byte but not 256-byte aligned
    assert lib.mix_gemm_a_image(3, FAKE, FAKE, 4, 128, FAKE, 1 << 20, None) == MIX_E_ENUM
    assert lib.mix_gemm_a_image(1, FAKE, FAKE, 4, 96, FAKE, 1 << 20, None) == MIX_E_SHAPE
    assert lib.mix_gemm_a_image(1, None, FAKE, 4, 128, FAKE, 1 << 20, None) == MIX_E_NULL
    assert lib.mix_gemm_a_image(1, FAKE, FAKE, 4, 128, A16, 1 << 20, None) == MIX_E_ALIGN
    assert lib.mix_gemm_a_image(1, FAKE, FAKE, 4, 128, FAKE, 100, None) == MIX_E_WORKSPACE
    assert lib.mix_gemm_a_image(1, None, None, 0, 128, None, 0, None) == MIX_OK
    # codes and shared go together; cols must be a multiple of 128
    assert lib.mix_quantize_gemm(1, FAKE, 1, 4, 128, 128, FAKE, None, FAKE, 1 << 20, None) == MIX_E_NULL
    assert lib.mix_quantize_gemm(1, FAKE, 1, 4, 96, 96, None, None, FAKE, 1 << 20, None) == MIX_E_SHAPE
    assert lib.mix_quantize_gemm(1, FAKE, 1, 4, 128, 128, None, None, FAKE, 10, None) == MIX_E_WORKSPACE
    assert lib.mix_quantize_gemm(1, None, 1, 0, 128, 128, None, None, None, 0, None) == MIX_OK
    assert lib.mx_gemm_b_image(1, FAKE, None, 4, 128, FAKE, 1 << 20, None) == MIX_E_NULL
    assert lib.mx_gemm_b_image(1, None, FAKE, 4, 128, FAKE, 1 << 20, None) == MIX_E_NULL
    assert lib.mx_gemm_b_image(1, P(0x10008), FAKE, 4, 128, FAKE, 1 << 20, None) == MIX_E_ALIGN
    assert lib.mx_gemm_b_image(0, None, FAKE, 4, 128, FAKE, 1 << 20, None) == MIX_E_NULL
    assert lib.mx_gemm_b_image(0, FAKE, FAKE, 4, 128, A16, 1 << 20, None) == MIX_E_ALIGN
    # GEMM from images: K a multiple of 128; images 256-byte aligned (the codes are not needed)
    assert lib.mix_mx_gemm_images(1, None, FAKE, None, 4, 4, 128, FAKE, 0, 4, None) == MIX_E_NULL
    assert lib.mix_mx_gemm_images(0, FAKE, FAKE, None, 4, 4, 100, FAKE, 0, 4, None) == MIX_E_SHAPE
    assert lib.mix_mx_gemm_images(0, A16, FAKE, None, 4, 4, 128, FAKE, 0, 4, None) == MIX_E_ALIGN
    assert lib.mix_mx_gemm_images(0, FAKE, FAKE, None, 4, 4, 128, FAKE, 0, 3, None) == MIX_E_SHAPE
    assert lib.mix_mx_gemm_images(0, None, None, None, 0, 4, 128, None, 0, 4, None) == MIX_OK
    # 32-bit offsets inside the tiled kernel: a 2^31-byte A image is refused (M > 16)
    assert lib.mix_mx_gemm_images(1, FAKE, FAKE, FAKE, 1 << 20, 256, 2048, FAKE, 0, 256, None) == MIX_E_UNSUPPORTED
    assert lib.mix_mx_gemm_workspace_bytes(1, 1, 1 << 20, 256, 2048) == 0


def test_image_product_with_quantized_output_validation(lib):
    f = lib.mix_mx_gemm_images_quantize
    A16 = P(0x10010)
    BIG = 1 << 30
    # (b_fmt, a_img, b_img, b_codes, M, N, K, c, ldc, q_codes, q_shared, q_img, q_img_bytes, stream)
    assert f(4, FAKE, FAKE, FAKE, 64, 256, 128, None, 0, FAKE, FAKE, None, 0, None) == MIX_E_ENUM
    assert f(1, FAKE, FAKE, FAKE, 64, 250, 128, None, 0, FAKE, FAKE, None, 0, None) == MIX_E_SHAPE   # N % 32
    assert f(1, FAKE, FAKE, FAKE, 64, 256, 100, None, 0, FAKE, FAKE, None, 0, None) == MIX_E_SHAPE   # K % 128
    assert f(1, FAKE, FAKE, FAKE, 64, 160, 128, None, 0, FAKE, FAKE, FAKE, BIG, None) == MIX_E_SHAPE  # image: N % 128
    assert f(1, FAKE, FAKE, FAKE, 8, 256, 128, None, 0, FAKE, FAKE, None, 0, None) == MIX_E_NULL     # M <= 16 needs c
    assert f(1, FAKE, FAKE, FAKE, 64, 256, 128, None, 0, None, FAKE, None, 0, None) == MIX_E_NULL
    assert f(1, FAKE, None, None, 64, 256, 128, None, 0, FAKE, FAKE, None, 0, None) == MIX_E_NULL    # B image
    assert f(1, A16, FAKE, FAKE, 64, 256, 128, None, 0, FAKE, FAKE, None, 0, None) == MIX_E_ALIGN
    assert f(1, FAKE, FAKE, FAKE, 64, 256, 128, None, 0, FAKE, FAKE, A16, BIG, None) == MIX_E_ALIGN
    assert f(1, FAKE, FAKE, FAKE, 64, 256, 128, None, 0, P(0x10002), FAKE, None, 0, None) == MIX_E_ALIGN
    assert f(1, FAKE, FAKE, FAKE, 64, 256, 128, FAKE, 100, FAKE, FAKE, None, 0, None) == MIX_E_SHAPE  # ldc < N
    assert f(1, FAKE, FAKE, FAKE, 64, 256, 128, None, 0, FAKE, FAKE, FAKE, 1000, None) == MIX_E_WORKSPACE
    assert f(1, None, None, None, 0, 256, 128, None, 0, None, None, None, 0, None) == MIX_OK         # empty



def test_g16_validation(lib):
    # g16 weights: quantizer formats 2 and 3; the image entry point with its counter; the codes-path
    # product refers callers to the image or Eq. (6) paths
    assert lib.mx_gemm_b_image_bytes(2, 18944, 3584) == lib.mx_gemm_b_image_bytes(0, 18944, 3584)
    assert lib.mx_gemm_b_image_bytes(3, 300, 256) == lib.mx_gemm_b_image_bytes(0, 300, 256)
    assert lib.mx_gemm_b_image_bytes(4, 300, 256) == 0
    big = 1 << 30
    assert lib.mx_gemm_b_image(2, FAKE, FAKE, 256, 256, FAKE, big, None) == MIX_E_UNSUPPORTED
    assert lib.mx_gemm_b_image_g16(1, FAKE, FAKE, 256, 256, FAKE, big, FAKE, None) == MIX_E_ENUM
    assert lib.mx_gemm_b_image_g16(2, FAKE, FAKE, 256, 96, FAKE, big, FAKE, None) == MIX_E_SHAPE
    assert lib.mx_gemm_b_image_g16(2, FAKE, FAKE, 256, 256, FAKE, big, None, None) == MIX_E_NULL
    assert lib.mx_gemm_b_image_g16(3, FAKE, FAKE, 256, 256, FAKE, big, P(0x10002), None) == MIX_E_ALIGN
    assert lib.mx_gemm_b_image_g16(3, FAKE, FAKE, 256, 256, FAKE, 16, FAKE, None) == MIX_E_WORKSPACE
    assert lib.mx_gemm_b_image_g16(2, None, None, 0, 256, None, 0, None, None) == MIX_OK
    assert lib.mix_mx_gemm(1, FAKE, FAKE, 2, FAKE, FAKE, 4, 4, 32, FAKE, 0, 4, None, 0, None) == MIX_E_UNSUPPORTED
    assert lib.mix_mx_gemm_workspace_bytes(1, 2, 4096, 18944, 3584) == 0
    assert lib.mx_quantize(4, FAKE, 0, 4, 32, 32, None, FAKE, FAKE, None) == MIX_E_ENUM


def test_underflow_map_validation(lib):
    f = lib.mix_underflow_map
    W = 1 << 30
    # (x, dtype, rows, cols, ldx, mu, counts, amax, ws, ws_bytes, stream)
    assert f(FAKE, 5, 4, 32, 32, None, FAKE, FAKE, FAKE, W, None) == MIX_E_ENUM
    assert f(FAKE, 0, 4, 40, 40, None, FAKE, FAKE, FAKE, W, None) == MIX_E_SHAPE
    assert f(FAKE, 0, 4, 32, 16, None, FAKE, FAKE, FAKE, W, None) == MIX_E_SHAPE
    assert f(FAKE, 0, -1, 32, 32, None, FAKE, FAKE, FAKE, W, None) == MIX_E_SHAPE
    assert f(None, 0, 4, 32, 32, None, FAKE, FAKE, FAKE, W, None) == MIX_E_NULL
    assert f(FAKE, 0, 4, 32, 32, None, None, FAKE, FAKE, W, None) == MIX_E_NULL
    assert f(FAKE, 0, 4, 32, 32, None, FAKE, None, FAKE, W, None) == MIX_E_NULL
    assert f(FAKE, 0, 4, 32, 32, None, FAKE, FAKE, None, W, None) == MIX_E_NULL
    assert f(MISALIGNED, 0, 4, 32, 32, None, FAKE, FAKE, FAKE, W, None) == MIX_E_ALIGN
    assert f(FAKE, 1, 4, 32, 36, None, FAKE, FAKE, FAKE, W, None) == MIX_E_ALIGN
    assert f(FAKE, 0, 4, 32, 32, P(0x10004), FAKE, FAKE, FAKE, W, None) == MIX_E_ALIGN
    assert f(FAKE, 0, 4, 32, 32, None, P(0x10002), FAKE, FAKE, W, None) == MIX_E_ALIGN
    assert f(FAKE, 0, 4, 32, 32, None, FAKE, FAKE, P(0x10008), W, None) == MIX_E_ALIGN
    assert f(FAKE, 0, 1 << 31, 32, 32, None, FAKE, FAKE, FAKE, W, None) == MIX_E_SHAPE
    need = lib.mix_underflow_map_workspace_bytes(4096, 512)
    # 512 amax partials + per workgroup row 7 sums per column (32 workgroup rows of 128 rows here)
    assert need == 2048 + 32 * 7 * 512 * 4
    assert f(FAKE, 0, 4096, 512, 512, None, FAKE, FAKE, FAKE, need - 1, None) == MIX_E_WORKSPACE
    assert lib.mix_underflow_map_workspace_bytes(0, 512) == 0
    assert lib.mix_underflow_map_workspace_bytes(4, 40) == 0
    assert lib.mix_underflow_map_workspace_bytes(1, 32) == 2048 + 1024   # 7 x 32 x 4 rounded to 256
    assert f(None, 0, 4, 0, 0, None, None, None, None, 0, None) == MIX_OK


class _Cache(ctypes.Structure):
    _fields_ = [("k_codes", P), ("k_scales", P), ("v_codes", P), ("v_scales", P), ("v_stage", P),
                ("B", ctypes.c_int64), ("Lmax", ctypes.c_int64), ("Hkv", ctypes.c_int64), ("d", ctypes.c_int64)]


def _cache(B=16, Lmax=8192, Hkv=4, d=128):
    return _Cache(FAKE, FAKE, FAKE, FAKE, FAKE, B, Lmax, Hkv, d)


def test_decode_validation(lib):
    W = 1 << 30
    c = _cache()
    ref = ctypes.byref(c)
    f = lib.mix_attn_decode
    # (q, k_new, v_new, cache, pos, max_pos, Hq, mu, o, ws, ws_bytes, dbg, stream)
    assert f(FAKE, FAKE, FAKE, ref, FAKE, 8191, 30, FAKE, FAKE, FAKE, W, None, None) == MIX_E_SHAPE
    assert f(FAKE, FAKE, FAKE, ref, FAKE, 8192, 28, FAKE, FAKE, FAKE, W, None, None) == MIX_E_SHAPE
    assert f(FAKE, FAKE, FAKE, ref, FAKE, 8191, 68, FAKE, FAKE, FAKE, W, None, None) == MIX_E_UNSUPPORTED
    assert f(None, FAKE, FAKE, ref, FAKE, 8191, 28, FAKE, FAKE, FAKE, W, None, None) == MIX_E_NULL
    assert f(FAKE, FAKE, FAKE, ref, FAKE, 8191, 28, FAKE, FAKE, P(0x10010), W, None, None) == MIX_E_ALIGN
    need = lib.mix_attn_decode_workspace_bytes(16, 28, 4, 128, 8191)
    assert need >= 16 * 28 * 32 * 128 * 4   # at least the chunk partials
    assert f(FAKE, FAKE, FAKE, ref, FAKE, 8191, 28, FAKE, FAKE, FAKE, need - 1, None, None) == MIX_E_WORKSPACE
    assert lib.mix_attn_decode_workspace_bytes(16, 28, 0, 128, 8191) == 0
    c64 = _cache(d=64)
    assert f(FAKE, FAKE, FAKE, ctypes.byref(c64), FAKE, 8191, 28, FAKE, FAKE, FAKE, W, None, None) == MIX_E_UNSUPPORTED


def test_decode_step_validation(lib):
    W = 1 << 30
    c = _cache()
    ref = ctypes.byref(c)
    f = lib.mix_decode_step
    # (x, K, N, b_fmt, b_img, y, q, k_new, v_new, cache, pos, max_pos, Hq, mu, o, ws, ws_bytes, stream)
    args = [FAKE, 3584, 18944, 1, FAKE, FAKE, FAKE, FAKE, FAKE, ref, FAKE, 8191, 28, FAKE, FAKE, FAKE, W, None]

    def call(**kw):
        a = list(args)
        for i, name in enumerate(("x", "K", "N", "b_fmt", "b_img", "y", "q", "k_new", "v_new", "cache", "pos",
                                  "max_pos", "Hq", "mu", "o", "ws", "ws_bytes")):
            if name in kw:
                a[i] = kw[name]
        return f(*a)

    need = lib.mix_decode_step_workspace_bytes(16, 3584, 28, 4, 128, 8191)
    assert need == lib.mix_attn_decode_workspace_bytes(16, 28, 4, 128, 8191) + \
        lib.mix_gemm_a_image_bytes(16, 3584)   # plus the activations' A image
    assert lib.mix_decode_step_workspace_bytes(16, 0, 28, 4, 128, 8191) == 0
    assert call(b_fmt=7) == MIX_E_ENUM
    assert call(K=3600) == MIX_E_SHAPE
    assert call(N=0) == MIX_E_SHAPE
    assert call(Hq=30) == MIX_E_SHAPE
    assert call(max_pos=8192) == MIX_E_SHAPE
    assert call(x=None) == MIX_E_NULL
    assert call(b_img=None) == MIX_E_NULL
    assert call(y=None) == MIX_E_NULL
    assert call(b_img=P(0x10010)) == MIX_E_ALIGN
    assert call(x=MISALIGNED) == MIX_E_ALIGN
    assert call(ws=P(0x10010)) == MIX_E_ALIGN
    assert call(ws_bytes=need - 1) == MIX_E_WORKSPACE
    big = _cache(B=17)
    assert call(cache=ctypes.byref(big)) == MIX_E_UNSUPPORTED
    c64 = _cache(d=64)
    assert call(cache=ctypes.byref(c64)) == MIX_E_UNSUPPORTED


def test_decode_output_alignment(lib):
    c = _cache()
    ref = ctypes.byref(c)
    W = 1 << 30
    assert lib.mix_attn_decode(FAKE, FAKE, FAKE, ref, FAKE, 8191, 28, FAKE, P(0x10004), FAKE, W, None, None) == \
        MIX_E_ALIGN
    assert lib.mix_decode_step(FAKE, 3584, 18944, 1, FAKE, FAKE, FAKE, FAKE, FAKE, ref, FAKE, 8191, 28, FAKE,
                               P(0x10004), FAKE, W, None) == MIX_E_ALIGN
