"""ctypes loader for libmix.so.

torch is imported first so that the HIP runtime torch ships is the one already loaded when the
library resolves ``libamdhip64.so``; device pointers and streams then belong to one runtime.
"""
import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime before libmix.so)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmix.so")

_lib = None

c_i64 = ctypes.c_int64
c_ptr = ctypes.c_void_p
c_int = ctypes.c_int

# name -> (restype, argtypes)
SIGNATURES = {
    "mix_abi_version": (c_int, []),
    "mix_status_str": (ctypes.c_char_p, [c_int]),
    "mix_last_error": (ctypes.c_char_p, []),
    "mix_quantize": (c_int, [c_int, c_ptr, c_int, c_i64, c_i64, c_i64, c_ptr, c_ptr, c_ptr]),
    "mx_quantize": (c_int, [c_int, c_ptr, c_int, c_i64, c_i64, c_i64, c_ptr, c_ptr, c_ptr, c_ptr]),
    "mx_quantize_cols": (c_int, [c_ptr, c_int, c_i64, c_i64, c_i64, c_ptr, c_ptr, c_ptr]),
    "mix_dequantize": (c_int, [c_int, c_ptr, c_ptr, c_i64, c_i64, c_ptr, c_ptr]),
    "mx_dequantize": (c_int, [c_int, c_ptr, c_ptr, c_i64, c_i64, c_ptr, c_ptr]),
    "mix_mx_gemm": (c_int, [c_int, c_ptr, c_ptr, c_int, c_ptr, c_ptr, c_i64, c_i64, c_i64, c_ptr, c_int, c_i64, c_ptr,
                            ctypes.c_size_t, c_ptr]),
    "mix_mx_gemm_workspace_bytes": (ctypes.c_size_t, [c_int, c_int, c_i64, c_i64, c_i64]),
    "mix_mx_gemm_eq6": (c_int, [c_int, c_ptr, c_ptr, c_int, c_ptr, c_ptr, c_i64, c_i64, c_i64, c_ptr, c_int, c_i64,
                                c_ptr]),
    "mix_gemm_a_image_bytes": (ctypes.c_size_t, [c_i64, c_i64]),
    "mx_gemm_b_image_bytes": (ctypes.c_size_t, [c_int, c_i64, c_i64]),
    "mix_gemm_a_image": (c_int, [c_int, c_ptr, c_ptr, c_i64, c_i64, c_ptr, ctypes.c_size_t, c_ptr]),
    "mix_quantize_gemm": (c_int, [c_int, c_ptr, c_int, c_i64, c_i64, c_i64, c_ptr, c_ptr, c_ptr, ctypes.c_size_t,
                                  c_ptr]),
    "mx_gemm_b_image": (c_int, [c_int, c_ptr, c_ptr, c_i64, c_i64, c_ptr, ctypes.c_size_t, c_ptr]),
    "mx_gemm_b_image_g16": (c_int, [c_int, c_ptr, c_ptr, c_i64, c_i64, c_ptr, ctypes.c_size_t, c_ptr, c_ptr]),
    "mix_mx_gemm_images": (c_int, [c_int, c_ptr, c_ptr, c_ptr, c_i64, c_i64, c_i64, c_ptr, c_int, c_i64, c_ptr]),
    "mix_mx_gemm_images_quantize": (c_int, [c_int, c_ptr, c_ptr, c_ptr, c_i64, c_i64, c_i64, c_ptr, c_i64, c_ptr,
                                            c_ptr, c_ptr, ctypes.c_size_t, c_ptr]),
    "mix_kmean": (c_int, [c_ptr, c_int, c_i64, c_i64, c_i64, c_ptr, c_ptr]),
    "mix_underflow_map_workspace_bytes": (ctypes.c_size_t, [c_i64, c_i64]),
    "mix_underflow_map": (c_int, [c_ptr, c_int, c_i64, c_i64, c_i64, c_ptr, c_ptr, c_ptr, c_ptr, ctypes.c_size_t, c_ptr]),
    "mix_attn_prefill_workspace_bytes": (ctypes.c_size_t, [c_i64, c_i64, c_i64, c_i64]),
    "mix_attn_prefill": (c_int, [c_ptr, c_ptr, c_ptr, c_i64, c_i64, c_i64, c_i64, c_int, c_ptr, c_ptr, c_ptr,
                                 ctypes.c_size_t, c_ptr, c_ptr]),
    "mix_kv_cache_prefill": (c_int, [c_ptr, c_i64, c_ptr, c_ptr, c_i64, c_ptr, c_ptr]),
    "mix_attn_decode_workspace_bytes": (ctypes.c_size_t, [c_i64, c_i64, c_i64, c_i64, c_i64]),
    "mix_attn_decode": (c_int, [c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_i64, c_i64, c_ptr, c_ptr, c_ptr, ctypes.c_size_t,
                                c_ptr, c_ptr]),
    "mix_decode_step_workspace_bytes": (ctypes.c_size_t, [c_i64, c_i64, c_i64, c_i64, c_i64, c_i64]),
    "mix_decode_step": (c_int, [c_ptr, c_i64, c_i64, c_int, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_i64,
                                c_i64, c_ptr, c_ptr, c_ptr, ctypes.c_size_t, c_ptr]),
    "mix_decode_step_single": (c_int, [c_ptr, c_i64, c_i64, c_int, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr,
                                       c_i64, c_i64, c_ptr, c_ptr, c_ptr, ctypes.c_size_t, c_ptr]),
    "mix_decode_step_static_max_bytes": (ctypes.c_size_t, []),
    "mix_decode_step_static": (c_int, [c_ptr, c_i64, c_i64, c_int, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr,
                                       c_i64, c_i64, c_ptr, c_ptr, c_ptr]),
}


def load(path=LIB_PATH):
    """Load (once) and return the library. Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libmix.so not found at {path}; build it with `python -m quantized_gemm_algorithm_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class MixError(RuntimeError):
    pass


def check(status, what):
    if status != 0:
        lib = load()
        raise MixError(f"{what}: {lib.mix_status_str(status).decode()} ({lib.mix_last_error().decode()})")
