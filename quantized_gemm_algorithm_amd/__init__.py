"""MiX (Micro-Inverted-Scaling) hot path on MI355X -- Python binding over the HIP C-ABI (libmix.so).

Every function here only marshals arguments: it allocates outputs with torch on the input's
device, passes raw device pointers and torch's current stream to the C entry point of the same
name, and raises ``MixError`` on a non-zero status. All arithmetic runs in the HIP kernels. There
is no CPU fallback: without a built ``libmix.so`` every call raises.

Format names: MiX ``"4.25b"`` / ``"4.5b"``; MX ``"int4"`` / ``"fp4"`` (one E8M0 scale per 32 elements)
and ``"int4g16"`` / ``"fp4g16"`` (one per 16: the 4.5-bit weights; their B image counts blocks whose
two halves cannot share one scale exactly in ``BImage.unfoldable``). bf16 inputs are
``torch.bfloat16`` tensors; MiX-4.5b shared fields come back as ``torch.int16`` holding the uint16
bit patterns.
"""
import ctypes

import torch

from . import _lib
from ._lib import MixError, check

MIX_FMT = {"4.25b": 0, "4.5b": 1}
MX_FMT = {"int4": 0, "fp4": 1, "int4g16": 2, "fp4g16": 3}
MX_BLOCK = {"int4": 32, "fp4": 32, "int4g16": 16, "fp4g16": 16}
DTYPE = {torch.float32: 0, torch.bfloat16: 1}

__all__ = [
    "MixError", "mix_quantize", "mx_quantize", "mx_quantize_cols", "mix_dequantize", "mx_dequantize",
    "mix_mx_gemm", "mix_mx_gemm_eq6", "AImage", "BImage", "mix_gemm_a_image", "mix_quantize_gemm",
    "mx_gemm_b_image", "mix_mx_gemm_images", "mix_mx_gemm_images_quantize", "mix_kmean", "mix_underflow_map", "mix_underflow_map_workspace_bytes", "UF_KINDS", "mix_attn_prefill", "KVCache", "mix_kv_cache_prefill",
    "mix_attn_decode", "mix_decode_step", "abi_version",
]


def _lib_():
    return _lib.load()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise MixError("libmix works on device tensors only (got a CPU tensor)")


def _matrix(x, name):
    if x.dim() != 2 or x.stride(1) != 1:
        raise MixError(f"{name} must be a 2-D tensor with unit column stride")
    if x.dtype not in DTYPE:
        raise MixError(f"{name} must be float32 or bfloat16")
    return x.shape[0], x.shape[1], x.stride(0)


def _out_matrix(out, M, N, what, dtypes=(torch.float32, torch.bfloat16)):
    """A caller-supplied output must hold [M, N] with unit column stride (the C-ABI takes only its
    pointer and row pitch, so a smaller buffer would be written past its end)."""
    _need_cuda(out)
    if out.dtype not in dtypes:
        raise MixError(f"{what}: out must be one of {dtypes}")
    if out.dim() != 2 or tuple(out.shape) != (M, N) or out.stride(1) != 1 or out.stride(0) < N:
        raise MixError(f"{what}: out must be a [{M}, {N}] tensor with unit column stride")
    return out


def _dense(t, shape, dtype, what):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise MixError(f"{what} must be a contiguous {dtype} tensor of shape {tuple(shape)}")


def abi_version():
    return _lib_().mix_abi_version()


def mix_quantize(x, fmt="4.5b", codes=None, shared=None):
    """MiX-quantize rows of x [rows, cols]. Returns (codes uint8 [rows, cols/2], shared [rows, cols/32]).

    ``codes``/``shared`` may be passed to write into existing dense tensors of those shapes.
    """
    _need_cuda(x, codes, shared)
    rows, cols, ld = _matrix(x, "x")
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    if shared is None:
        shared = torch.empty((rows, cols // 32), dtype=torch.uint8 if fmt == "4.25b" else torch.int16, device=x.device)
    if codes.numel() != rows * (cols // 2) or shared.numel() != rows * (cols // 32) or not codes.is_contiguous() \
            or not shared.is_contiguous() or shared.element_size() != (1 if fmt == "4.25b" else 2):
        raise MixError("codes/shared do not match the input's shape or the format")
    check(_lib_().mix_quantize(MIX_FMT[fmt], _p(x), DTYPE[x.dtype], rows, cols, ld, _p(codes), _p(shared), _stream()),
          "mix_quantize")
    return codes, shared


def mx_quantize(x, fmt="fp4", mu=None, codes=None, scales=None):
    """MX-quantize rows of x [rows, cols] (optionally fp32(x - mu)). Returns (codes, scales uint8);
    ``codes``/``scales`` may be passed to write into existing dense tensors of those shapes."""
    _need_cuda(x, mu, codes, scales)
    rows, cols, ld = _matrix(x, "x")
    if mu is not None and (mu.dtype != torch.float32 or mu.numel() != cols or not mu.is_contiguous()):
        raise MixError("mu must be a contiguous float32 tensor with one value per column")
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, cols // MX_BLOCK[fmt]), dtype=torch.uint8, device=x.device)
    _dense(codes, (rows, cols // 2), torch.uint8, "codes")
    _dense(scales, (rows, cols // MX_BLOCK[fmt]), torch.uint8, "scales")
    check(_lib_().mx_quantize(MX_FMT[fmt], _p(x), DTYPE[x.dtype], rows, cols, ld, _p(mu), _p(codes), _p(scales),
                              _stream()), "mx_quantize")
    return codes, scales


def mx_quantize_cols(x):
    """MXFP4 with 32-row blocks down each column of x [rows, cols]. Returns codes [cols, prows/2], scales."""
    _need_cuda(x)
    rows, cols, ld = _matrix(x, "x")
    prows = (rows + 31) // 32 * 32
    codes = torch.empty((cols, prows // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((cols, prows // 32), dtype=torch.uint8, device=x.device)
    check(_lib_().mx_quantize_cols(_p(x), DTYPE[x.dtype], rows, cols, ld, _p(codes), _p(scales), _stream()),
          "mx_quantize_cols")
    return codes, scales


def mix_dequantize(codes, shared, fmt="4.5b"):
    _need_cuda(codes, shared)
    rows, cols = codes.shape[0], codes.shape[1] * 2
    out = torch.empty((rows, cols), dtype=torch.float32, device=codes.device)
    check(_lib_().mix_dequantize(MIX_FMT[fmt], _p(codes), _p(shared), rows, cols, _p(out), _stream()), "mix_dequantize")
    return out


def mx_dequantize(codes, scales, fmt="fp4"):
    _need_cuda(codes, scales)
    rows, cols = codes.shape[0], codes.shape[1] * 2
    out = torch.empty((rows, cols), dtype=torch.float32, device=codes.device)
    check(_lib_().mx_dequantize(MX_FMT[fmt], _p(codes), _p(scales), rows, cols, _p(out), _stream()), "mx_dequantize")
    return out


def _gemm_shapes(a_codes, b_codes):
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = b_codes.shape[0]
    if b_codes.shape[1] * 2 != K:
        raise MixError("A and B disagree on K")
    return M, N, K


def mix_mx_gemm_workspace_bytes(a_fmt, b_fmt, M, N, K):
    return _lib_().mix_mx_gemm_workspace_bytes(MIX_FMT[a_fmt], MX_FMT[b_fmt], M, N, K)


def mix_mx_gemm(a_codes, a_shared, a_fmt, b_codes, b_scales, b_fmt, out_dtype=torch.float32, out=None,
                workspace="auto"):
    """C = deq(A) . deq(B)^T on the block-scaled MFMA. A: MiX [M, K]; B: MX [N, K] (W^T).

    ``workspace``: "auto" allocates the fast path's scratch with torch; a uint8 tensor is used as
    given; None selects the in-GEMM decode (same results).
    """
    _need_cuda(a_codes, a_shared, b_codes, b_scales, out)
    M, N, K = _gemm_shapes(a_codes, b_codes)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_codes.device)
    _out_matrix(out, M, N, "mix_mx_gemm")
    ws = None
    if isinstance(workspace, str):
        nb = mix_mx_gemm_workspace_bytes(a_fmt, b_fmt, M, N, K)
        if nb:
            ws = torch.empty((nb,), dtype=torch.uint8, device=a_codes.device)
    elif workspace is not None:
        _need_cuda(workspace)
        ws = workspace
    check(_lib_().mix_mx_gemm(MIX_FMT[a_fmt], _p(a_codes), _p(a_shared), MX_FMT[b_fmt], _p(b_codes), _p(b_scales),
                              M, N, K, _p(out), DTYPE[out.dtype], out.stride(0), _p(ws),
                              0 if ws is None else ws.numel(), _stream()), "mix_mx_gemm")
    return out


class AImage:
    """Decode-once GEMM operand of an [M, K] MiX matrix: opaque device bytes (``buf``)."""

    def __init__(self, buf, M, K):
        self.buf, self.M, self.K = buf, M, K


class BImage:
    """Decode-once GEMM operand of an [N, K] MX matrix (it holds every operand byte; ``codes`` is the
    tensor it was built from). g16 images carry ``unfoldable``: a device uint32 counting the 32-blocks
    that could not be folded into one scale exactly (0: products from the image are exact)."""

    def __init__(self, buf, fmt, N, K, codes, unfoldable=None):
        self.buf, self.fmt, self.N, self.K, self.codes = buf, fmt, N, K, codes
        self.unfoldable = unfoldable


def mix_gemm_a_image_bytes(M, K):
    return _lib_().mix_gemm_a_image_bytes(M, K)


def mx_gemm_b_image_bytes(b_fmt, N, K):
    return _lib_().mx_gemm_b_image_bytes(MX_FMT[b_fmt], N, K)


def _image_buf(nbytes, device, buf, what):
    if nbytes == 0:
        raise MixError(f"{what}: no image for this shape (K must be a positive multiple of 128)")
    if buf is None:
        return torch.empty((nbytes,), dtype=torch.uint8, device=device)
    _need_cuda(buf)
    if buf.dtype != torch.uint8 or not buf.is_contiguous() or buf.numel() < nbytes:
        raise MixError(f"{what}: image buffer must be a contiguous uint8 tensor of at least {nbytes} bytes")
    return buf


def mix_gemm_a_image(codes, shared, fmt="4.5b", out=None):
    """A image of MiX codes [M, K/2] + shared fields [M, K/32]."""
    _need_cuda(codes, shared)
    M, K = codes.shape[0], codes.shape[1] * 2
    buf = _image_buf(mix_gemm_a_image_bytes(M, K), codes.device, out, "mix_gemm_a_image")
    check(_lib_().mix_gemm_a_image(MIX_FMT[fmt], _p(codes), _p(shared), M, K, _p(buf), buf.numel(), _stream()),
          "mix_gemm_a_image")
    return AImage(buf, M, K)


def mix_quantize_gemm(x, fmt="4.5b", codes=None, shared=None, image=None, write_codes=True):
    """mix_quantize that also writes the A image in the same pass. Returns (codes, shared, AImage);
    with ``write_codes=False`` only the image is written and codes/shared are None."""
    if isinstance(image, AImage):
        image = image.buf
    _need_cuda(x, codes, shared, image)
    rows, cols, ld = _matrix(x, "x")
    if write_codes:
        if codes is None:
            codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
        if shared is None:
            shared = torch.empty((rows, cols // 32), dtype=torch.uint8 if fmt == "4.25b" else torch.int16,
                                 device=x.device)
        if codes.numel() != rows * (cols // 2) or shared.numel() != rows * (cols // 32) or not codes.is_contiguous() \
                or not shared.is_contiguous() or shared.element_size() != (1 if fmt == "4.25b" else 2):
            raise MixError("codes/shared do not match the input's shape or the format")
    else:
        codes = shared = None
    buf = _image_buf(mix_gemm_a_image_bytes(rows, cols), x.device, image, "mix_quantize_gemm")
    check(_lib_().mix_quantize_gemm(MIX_FMT[fmt], _p(x), DTYPE[x.dtype], rows, cols, ld, _p(codes), _p(shared),
                                    _p(buf), buf.numel(), _stream()), "mix_quantize_gemm")
    return codes, shared, AImage(buf, rows, cols)


def mx_gemm_b_image(codes, scales, fmt="fp4", out=None, allow_inexact=False):
    """B image of MX codes [N, K/2] + E8M0 scales [N, K/32] ([N, K/16] for the g16 formats; built
    once per weight).

    g16 formats: the call waits for the image and reads its count of 32-blocks whose halves could
    not share one scale exactly; if there are any it raises MixError (their products would not be
    exact; ``mix_mx_gemm_eq6`` is exact for every input) unless ``allow_inexact`` is set, in which
    case the image is returned with the count in ``BImage.unfoldable``."""
    _need_cuda(codes, scales)
    N, K = codes.shape[0], codes.shape[1] * 2
    buf = _image_buf(mx_gemm_b_image_bytes(fmt, N, K), codes.device, out, "mx_gemm_b_image")
    if MX_BLOCK[fmt] == 16:
        unf = torch.empty((1,), dtype=torch.int32, device=codes.device)
        check(_lib_().mx_gemm_b_image_g16(MX_FMT[fmt], _p(codes), _p(scales), N, K, _p(buf), buf.numel(), _p(unf),
                                          _stream()), "mx_gemm_b_image_g16")
        n_unf = int(unf.item())   # synchronises: an image is built once per weight, off the product path
        if n_unf and not allow_inexact:
            raise MixError(f"mx_gemm_b_image: {n_unf} {fmt} block(s) have halves whose exponents differ by more "
                           "than the E4M3 fold holds exactly; their image products would not be exact "
                           "(use mix_mx_gemm_eq6, or pass allow_inexact=True)")
        return BImage(buf, fmt, N, K, codes, unf)
    check(_lib_().mx_gemm_b_image(MX_FMT[fmt], _p(codes), _p(scales), N, K, _p(buf), buf.numel(), _stream()),
          "mx_gemm_b_image")
    return BImage(buf, fmt, N, K, codes)


def mix_mx_gemm_images(a_img, b_img, out_dtype=torch.float32, out=None):
    """C [M, N] = A . B^T from an AImage and a BImage (same results as mix_mx_gemm on the codes)."""
    if a_img.K != b_img.K:
        raise MixError("A and B images disagree on K")
    M, N, K = a_img.M, b_img.N, a_img.K
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_img.buf.device)
    _out_matrix(out, M, N, "mix_mx_gemm_images")
    check(_lib_().mix_mx_gemm_images(MX_FMT[b_img.fmt], _p(a_img.buf), _p(b_img.buf),
                                     None, M, N, K, _p(out),
                                     DTYPE[out.dtype], out.stride(0), _stream()), "mix_mx_gemm_images")
    return out


def mix_mx_gemm_images_quantize(a_img, b_img, keep_c=False, image=True, out=None, codes=None, shared=None,
                                q_image=None):
    """The image product with its output quantized in the same pass: MiX-4.5b codes [M, N/2] and
    shared fields [M, N/32] of the bf16 rounding of C (as mix_quantize of that bf16 matrix), and
    with ``image`` that output's AImage for a next product. Returns (C bf16 or None, codes, shared,
    AImage or None); C is kept with ``keep_c`` (always written when M <= 16)."""
    if a_img.K != b_img.K:
        raise MixError("A and B images disagree on K")
    M, N, K = a_img.M, b_img.N, a_img.K
    dev = a_img.buf.device
    if (keep_c or M <= 16) and out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if codes is None:
        codes = torch.empty((M, N // 2), dtype=torch.uint8, device=dev)
    if shared is None:
        shared = torch.empty((M, N // 32), dtype=torch.int16, device=dev)
    if isinstance(q_image, AImage):
        q_image = q_image.buf
    img = _image_buf(mix_gemm_a_image_bytes(M, N), dev, q_image, "mix_mx_gemm_images_quantize") if image else None
    _need_cuda(out, codes, shared)
    if out is not None:
        _out_matrix(out, M, N, "mix_mx_gemm_images_quantize", (torch.bfloat16,))
    _dense(codes, (M, N // 2), torch.uint8, "codes")
    _dense(shared, (M, N // 32), torch.int16, "shared")
    check(_lib_().mix_mx_gemm_images_quantize(MX_FMT[b_img.fmt], _p(a_img.buf), _p(b_img.buf),
                                              None, M, N, K, _p(out),
                                              out.stride(0) if out is not None else N, _p(codes), _p(shared),
                                              _p(img), img.numel() if img is not None else 0, _stream()),
          "mix_mx_gemm_images_quantize")
    return out, codes, shared, (AImage(img, M, N) if img is not None else None)


def mix_mx_gemm_eq6(a_codes, a_shared, a_fmt, b_codes, b_scales, b_fmt, out_dtype=torch.float32, out=None):
    """The same product by Eq. (6) integer shift-add on the vector ALUs."""
    _need_cuda(a_codes, a_shared, b_codes, b_scales, out)
    M, N, K = _gemm_shapes(a_codes, b_codes)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_codes.device)
    _out_matrix(out, M, N, "mix_mx_gemm_eq6")
    check(_lib_().mix_mx_gemm_eq6(MIX_FMT[a_fmt], _p(a_codes), _p(a_shared), MX_FMT[b_fmt], _p(b_codes),
                                  _p(b_scales), M, N, K, _p(out), DTYPE[out.dtype], out.stride(0), _stream()),
          "mix_mx_gemm_eq6")
    return out


def mix_kmean(k):
    """Per-column mean of k [T, C] (exact sum, fp64 division, fp32 result)."""
    _need_cuda(k)
    T, C, ld = _matrix(k, "k")
    mu = torch.empty((C,), dtype=torch.float32, device=k.device)
    check(_lib_().mix_kmean(_p(k), DTYPE[k.dtype], T, C, ld, _p(mu), _stream()), "mix_kmean")
    return mu


def mix_underflow_map_workspace_bytes(rows, cols):
    return _lib_().mix_underflow_map_workspace_bytes(rows, cols)


UF_KINDS = ("mxint4", "mxfp4_floor", "mxfp4_ceil", "nvfp4_b32", "mix_4.25b", "mix_4.5b", "nonzero")


def mix_underflow_map(x, mu=None, workspace=None):
    """Underflow map of x [rows, cols] (optionally smoothed, fp32(x - mu)): returns (counts, amax),
    counts an int64 tensor [7, cols] -- per column, the nonzero elements each format of UF_KINDS[:6]
    codes to zero, then the nonzero elements -- and amax the operand's largest magnitude."""
    _need_cuda(x, mu, workspace)
    rows, cols, ld = _matrix(x, "x")
    counts = torch.empty((len(UF_KINDS), cols), dtype=torch.int32, device=x.device)
    amax = torch.empty((1,), dtype=torch.float32, device=x.device)
    need = _lib_().mix_underflow_map_workspace_bytes(rows, cols)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    check(_lib_().mix_underflow_map(_p(x), DTYPE[x.dtype], rows, cols, ld, _p(mu), _p(counts), _p(amax),
                                    _p(workspace), workspace.numel() * workspace.element_size(), _stream()),
          "mix_underflow_map")
    return counts.to(torch.int64) & 0xFFFFFFFF, amax


# ---------------------------------------------------------------- attention


class _Debug(ctypes.Structure):
    _fields_ = [("s", ctypes.c_void_p), ("p", ctypes.c_void_p), ("p_codes", ctypes.c_void_p),
                ("p_shared", ctypes.c_void_p), ("l", ctypes.c_void_p)]


def _debug_struct(d):
    if d is None:
        return None, None
    st = _Debug(*(None if d.get(k) is None else d[k].data_ptr() for k in ("s", "p", "p_codes", "p_shared", "l")))
    return st, ctypes.byref(st)


def mix_attn_prefill(q, k, v, causal=True, debug=False, workspace=None, o=None):
    """K-smoothed MiX/MX attention prefill. q [T, Hq, d], k/v [T, Hkv, d] bf16.

    Returns (o bf16 [T, Hq, d], mu fp32 [Hkv, d], dbg dict or None). With ``debug`` the dict holds
    s / p (fp32 [Hq, T, Tp]), p_codes, p_shared and l from inside the call.
    """
    _need_cuda(q, k, v)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise MixError("q, k, v must be contiguous bfloat16")
    if k.dim() != 3 or tuple(k.shape) != (T, Hkv, d) or tuple(v.shape) != (T, Hkv, d):
        raise MixError("k and v must be [T, Hkv, d] with q's T and d")
    lib = _lib_()
    wsb = lib.mix_attn_prefill_workspace_bytes(T, Hq, Hkv, d)
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty((max(wsb, 1),), dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=q.device)
    _need_cuda(o)
    _dense(o, (T, Hq, d), torch.bfloat16, "o")
    mu = torch.empty((Hkv, d), dtype=torch.float32, device=q.device)
    dbg = None
    if debug:
        Tp = (T + 31) // 32 * 32
        dev = q.device
        dbg = {"s": torch.zeros((Hq, T, Tp), dtype=torch.float32, device=dev),
               "p": torch.zeros((Hq, T, Tp), dtype=torch.float32, device=dev),
               "p_codes": torch.empty((Hq, T, Tp // 2), dtype=torch.uint8, device=dev),
               "p_shared": torch.empty((Hq, T, Tp // 32), dtype=torch.int16, device=dev),
               "l": torch.empty((Hq, T), dtype=torch.float32, device=dev)}
    st, ref = _debug_struct(dbg)
    check(lib.mix_attn_prefill(_p(q), _p(k), _p(v), T, Hq, Hkv, d, int(bool(causal)), _p(mu), _p(o), _p(workspace),
                               workspace.numel(), ref, _stream()), "mix_attn_prefill")
    return o, mu, dbg


class _Cache(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("v_scales", ctypes.c_void_p), ("v_stage", ctypes.c_void_p), ("B", ctypes.c_int64),
                ("Lmax", ctypes.c_int64), ("Hkv", ctypes.c_int64), ("d", ctypes.c_int64)]


class KVCache:
    """Device buffers of an MX-coded KV cache (layouts as in mixlib.h), allocated with torch."""

    def __init__(self, B, Lmax, Hkv, d, device="cuda"):
        if Lmax % 32 or d % 32:
            raise MixError("Lmax and d must be multiples of 32")
        self.B, self.Lmax, self.Hkv, self.d = B, Lmax, Hkv, d
        self.k_codes = torch.zeros((B, Hkv, Lmax, d // 2), dtype=torch.uint8, device=device)
        self.k_scales = torch.zeros((B, Hkv, Lmax, d // 32), dtype=torch.uint8, device=device)
        self.v_codes = torch.zeros((B, Hkv, d, Lmax // 2), dtype=torch.uint8, device=device)
        self.v_scales = torch.zeros((B, Hkv, d, Lmax // 32), dtype=torch.uint8, device=device)
        self.v_stage = torch.zeros((B, 32, Hkv, d), dtype=torch.bfloat16, device=device)
        self._st = _Cache(self.k_codes.data_ptr(), self.k_scales.data_ptr(), self.v_codes.data_ptr(),
                          self.v_scales.data_ptr(), self.v_stage.data_ptr(), B, Lmax, Hkv, d)

    @property
    def ref(self):
        return ctypes.byref(self._st)


def mix_kv_cache_prefill(cache, b, k, v, mu):
    """Write a prefill of T tokens (k/v [T, Hkv, d] bf16) into row b of the cache with frozen mean mu."""
    _need_cuda(k, v, mu)
    T = k.shape[0]
    check(_lib_().mix_kv_cache_prefill(cache.ref, b, _p(k), _p(v), T, _p(mu), _stream()), "mix_kv_cache_prefill")


def mix_attn_decode(q, k_new, v_new, cache, pos, max_pos, mu, debug=False, workspace=None):
    """One decode step. q [B, Hq, d], k_new/v_new [B, Hkv, d] bf16; pos int32 [B] (device);
    mu fp32 [B, Hkv, d]. Returns (o bf16 [B, Hq, d], dbg dict or None)."""
    _need_cuda(q, k_new, v_new, pos, mu)
    if q.dim() != 3:
        raise MixError("q must be [B, Hq, d]")
    B, Hq, d = q.shape
    if B != cache.B or d != cache.d:
        raise MixError(f"q is [{B}, {Hq}, {d}] but the cache holds B = {cache.B}, d = {cache.d}")
    _dense(q, (B, Hq, d), torch.bfloat16, "q")
    _dense(k_new, (B, cache.Hkv, d), torch.bfloat16, "k_new")
    _dense(v_new, (B, cache.Hkv, d), torch.bfloat16, "v_new")
    _dense(pos, (B,), torch.int32, "pos")
    if mu.dtype != torch.float32 or mu.numel() != B * cache.Hkv * d or not mu.is_contiguous():
        raise MixError(f"mu must be a contiguous float32 tensor of {B} x {cache.Hkv} x {d} values")
    lib = _lib_()
    wsb = lib.mix_attn_decode_workspace_bytes(B, Hq, cache.Hkv, d, max_pos)
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty((max(wsb, 1),), dtype=torch.uint8, device=q.device)
    o = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=q.device)
    dbg = None
    if debug:
        Lp = (max_pos + 1 + 255) // 256 * 256
        dev = q.device
        dbg = {"s": torch.zeros((B, Hq, Lp), dtype=torch.float32, device=dev),
               "p": torch.zeros((B, Hq, Lp), dtype=torch.float32, device=dev),
               "p_codes": torch.empty((B, Hq, Lp // 2), dtype=torch.uint8, device=dev),
               "p_shared": torch.empty((B, Hq, Lp // 32), dtype=torch.int16, device=dev),
               "l": torch.empty((B, Hq), dtype=torch.float32, device=dev)}
    st, ref = _debug_struct(dbg)
    check(lib.mix_attn_decode(_p(q), _p(k_new), _p(v_new), cache.ref, _p(pos), max_pos, Hq, _p(mu), _p(o),
                              _p(workspace), workspace.numel(), ref, _stream()), "mix_attn_decode")
    return o, dbg


def mix_decode_step(x, b_img, q, k_new, v_new, cache, pos, max_pos, mu, y=None, o=None, workspace=None,
                    single=False):
    """One whole decode step: y = bf16(MiX-4.5b(x) . W^T) for x [B, K] bf16 and the weights' BImage
    (N x K), and the attention step of mix_attn_decode (q [B, Hq, d], k_new/v_new [B, Hkv, d] bf16,
    pos int32 [B], mu fp32 [B, Hkv, d]). Returns (y bf16 [B, N], o bf16 [B, Hq, d]). ``single``:
    the same step in one cooperative launch (mix_decode_step_single)."""
    _need_cuda(x, q, k_new, v_new, pos, mu, y, o, workspace)
    if q.dim() != 3:
        raise MixError("q must be [B, Hq, d]")
    B, Hq, d = q.shape
    if B != cache.B or d != cache.d:
        raise MixError(f"q is [{B}, {Hq}, {d}] but the cache holds B = {cache.B}, d = {cache.d}")
    if x.dim() != 2 or x.shape[0] != B or x.shape[1] != b_img.K:
        raise MixError(f"x must be [{B}, {b_img.K}] (the batch and the weights' K)")
    N, K = b_img.N, b_img.K
    _dense(x, (B, K), torch.bfloat16, "x")
    _dense(q, (B, Hq, d), torch.bfloat16, "q")
    _dense(k_new, (B, cache.Hkv, d), torch.bfloat16, "k_new")
    _dense(v_new, (B, cache.Hkv, d), torch.bfloat16, "v_new")
    _dense(pos, (B,), torch.int32, "pos")
    if mu.dtype != torch.float32 or mu.numel() != B * cache.Hkv * d or not mu.is_contiguous():
        raise MixError(f"mu must be a contiguous float32 tensor of {B} x {cache.Hkv} x {d} values")
    if y is None:
        y = torch.empty((B, N), dtype=torch.bfloat16, device=x.device)
    _dense(y, (B, N), torch.bfloat16, "y")
    if o is None:
        o = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=x.device)
    _dense(o, (B, Hq, d), torch.bfloat16, "o")
    lib = _lib_()
    wsb = lib.mix_decode_step_workspace_bytes(B, K, Hq, cache.Hkv, d, max_pos)
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty((max(wsb, 1),), dtype=torch.uint8, device=x.device)
    entry = lib.mix_decode_step_single if single else lib.mix_decode_step
    check(entry(_p(x), K, N, MX_FMT[b_img.fmt], _p(b_img.buf), _p(y), _p(q), _p(k_new), _p(v_new), cache.ref,
                _p(pos), max_pos, Hq, _p(mu), _p(o), _p(workspace), workspace.numel(), _stream()),
          "mix_decode_step_single" if single else "mix_decode_step")
    return y, o
