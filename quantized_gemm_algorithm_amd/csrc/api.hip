// C-ABI of the MiX library: argument validation on the host, then kernel dispatch on the caller's
// stream. Nothing here allocates, frees or synchronises.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "../../include/mixlib.h"
#include "f8_image.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

mix_status_t fail(mix_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

mix_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MIX_OK;
  return fail(MIX_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Enum arguments come from C callers and foreign-function bindings, which can pass any int, and in
// C++ a value outside an unscoped enum's range may not be read as that enum type. Validation
// therefore reads such an argument's bits as an int, through its address, before anything uses it
// as the enum.
template <class E>
inline int enum_bits(const E* e) {
  static_assert(sizeof(E) == sizeof(int), "the C enums are int-sized");
  int v;
  memcpy(&v, e, sizeof v);
  return v;
}
inline bool mix_known(int f) { return f == MIX_4P25 || f == MIX_4P5; }
inline int dtype_size(int dt) { return dt == MIX_BF16 ? 2 : 4; }

mix_status_t check_dtype(int dt) {
  if (dt != MIX_F32 && dt != MIX_BF16) return fail(MIX_E_ENUM, "unknown dtype %d", dt);
  return MIX_OK;
}

// Largest input matrix (elements, pitch included): 2^46, with every extent below 2^31, so that no
// size or grid computation below can overflow.
constexpr int64_t kMaxElems = (int64_t)1 << 46;

// Common checks for a [rows, cols] input with blocks along cols. Sets *empty for zero extents.
mix_status_t check_matrix_in(const char* fn, const void* x, int dt, int64_t rows, int64_t cols, int64_t ldx,
                             bool* empty) {
  *empty = false;
  if (rows < 0 || cols < 0) return fail(MIX_E_SHAPE, "%s: negative extent (rows=%lld cols=%lld)", fn, (long long)rows, (long long)cols);
  if (cols % 32) return fail(MIX_E_SHAPE, "%s: cols=%lld is not a multiple of 32", fn, (long long)cols);
  if (rows == 0 || cols == 0) { *empty = true; return MIX_OK; }
  if (ldx < cols) return fail(MIX_E_SHAPE, "%s: ldx=%lld < cols=%lld", fn, (long long)ldx, (long long)cols);
  if (rows > INT32_MAX || ldx > INT32_MAX || rows * ldx > kMaxElems)
    return fail(MIX_E_SHAPE, "%s: %lld rows of pitch %lld exceed the library's extents", fn, (long long)rows, (long long)ldx);
  if (!x) return fail(MIX_E_NULL, "%s: x is NULL", fn);
  if (!aligned16(x) || (ldx * dtype_size(dt)) % 16) return fail(MIX_E_ALIGN, "%s: x or its row pitch is not 16-byte aligned", fn);
  return MIX_OK;
}

}  // namespace

extern "C" {

int mix_abi_version(void) { return MIX_ABI_VERSION; }

const char* mix_status_str(mix_status_t s) {
  switch (enum_bits(&s)) {
    case MIX_OK: return "ok";
    case MIX_E_NULL: return "null pointer";
    case MIX_E_SHAPE: return "bad shape";
    case MIX_E_ALIGN: return "misaligned pointer or pitch";
    case MIX_E_ENUM: return "unknown enum value";
    case MIX_E_UNSUPPORTED: return "unsupported combination";
    case MIX_E_HIP: return "HIP error";
    case MIX_E_WORKSPACE: return "workspace too small";
  }
  return "unknown status";
}

const char* mix_last_error(void) { return g_err.c_str(); }

mix_status_t mix_quantize(mix_fmt_t fmt, const void* x, mix_dtype_t dtype, int64_t rows, int64_t cols, int64_t ldx,
                          uint8_t* codes, void* shared, void* stream) {
  g_err.clear();
  if (!mix_known(enum_bits(&fmt))) return fail(MIX_E_ENUM, "mix_quantize: unknown MiX format %d", enum_bits(&fmt));
  if (mix_status_t st = check_dtype(enum_bits(&dtype))) return st;
  bool empty;
  if (mix_status_t st = check_matrix_in("mix_quantize", x, dtype, rows, cols, ldx, &empty)) return st;
  if (empty) return MIX_OK;
  if (!codes || !shared) return fail(MIX_E_NULL, "mix_quantize: codes or shared is NULL");
  if (!aligned16(codes) || ((uintptr_t)shared & 1u)) return fail(MIX_E_ALIGN, "mix_quantize: codes not 16-byte aligned or shared not 2-byte aligned");
  return hip_status(mix::launch_mix_quantize((int)fmt, x, (int)dtype, rows, cols, ldx, codes, shared, (hipStream_t)stream),
                    "mix_quantize launch");
}

static bool mx_known(int f) { return f == MX_INT4 || f == MX_FP4 || f == MX_INT4_G16 || f == MX_FP4_G16; }
static bool mx_fp4(mx_fmt_t f) { return f == MX_FP4 || f == MX_FP4_G16; }
static bool mx_g16(mx_fmt_t f) { return f == MX_INT4_G16 || f == MX_FP4_G16; }

mix_status_t mx_quantize(mx_fmt_t fmt, const void* x, mix_dtype_t dtype, int64_t rows, int64_t cols, int64_t ldx,
                         const float* mu, uint8_t* codes, uint8_t* scales, void* stream) {
  g_err.clear();
  if (!mx_known(enum_bits(&fmt))) return fail(MIX_E_ENUM, "mx_quantize: unknown MX format %d", enum_bits(&fmt));
  if (mix_status_t st = check_dtype(enum_bits(&dtype))) return st;
  bool empty;
  if (mix_status_t st = check_matrix_in("mx_quantize", x, dtype, rows, cols, ldx, &empty)) return st;
  if (empty) return MIX_OK;
  if (!codes || !scales) return fail(MIX_E_NULL, "mx_quantize: codes or scales is NULL");
  if (!aligned16(codes) || (mu && !aligned16(mu))) return fail(MIX_E_ALIGN, "mx_quantize: codes or mu not 16-byte aligned");
  return hip_status(mix::launch_mx_quantize(mx_fp4(fmt), x, (int)dtype, rows, cols, ldx, mu, codes, scales,
                                            (hipStream_t)stream, mx_g16(fmt)),
                    "mx_quantize launch");
}

mix_status_t mx_quantize_cols(const void* x, mix_dtype_t dtype, int64_t rows, int64_t cols, int64_t ldx,
                              uint8_t* codes, uint8_t* scales, void* stream) {
  g_err.clear();
  if (mix_status_t st = check_dtype(enum_bits(&dtype))) return st;
  if (rows < 0 || cols < 0) return fail(MIX_E_SHAPE, "mx_quantize_cols: negative extent");
  if (rows == 0 || cols == 0) return MIX_OK;
  if (ldx < cols) return fail(MIX_E_SHAPE, "mx_quantize_cols: ldx < cols");
  if (rows > INT32_MAX || ldx > INT32_MAX || rows * ldx > kMaxElems)
    return fail(MIX_E_SHAPE, "mx_quantize_cols: extents too large");
  if (!x || !codes || !scales) return fail(MIX_E_NULL, "mx_quantize_cols: NULL pointer");
  if (!aligned16(codes)) return fail(MIX_E_ALIGN, "mx_quantize_cols: codes not 16-byte aligned");
  if ((uintptr_t)x % dtype_size(dtype)) return fail(MIX_E_ALIGN, "mx_quantize_cols: x misaligned");
  int64_t prows = (rows + 31) / 32 * 32;
  if (prows / 32 > 65535) return fail(MIX_E_SHAPE, "mx_quantize_cols: rows too large");
  return hip_status(mix::launch_mx_quantize_cols(x, (int)dtype, rows, prows, cols, ldx, codes, scales, prows / 2,
                                                 prows / 32, (hipStream_t)stream),
                    "mx_quantize_cols launch");
}

mix_status_t mix_dequantize(mix_fmt_t fmt, const uint8_t* codes, const void* shared, int64_t rows, int64_t cols,
                            float* out, void* stream) {
  g_err.clear();
  if (!mix_known(enum_bits(&fmt))) return fail(MIX_E_ENUM, "mix_dequantize: unknown MiX format %d", enum_bits(&fmt));
  if (rows < 0 || cols < 0 || cols % 32) return fail(MIX_E_SHAPE, "mix_dequantize: bad shape");
  if (rows == 0 || cols == 0) return MIX_OK;
  if (!codes || !shared || !out) return fail(MIX_E_NULL, "mix_dequantize: NULL pointer");
  if (fmt == MIX_4P5 && ((uintptr_t)shared & 1u)) return fail(MIX_E_ALIGN, "mix_dequantize: shared misaligned");
  return hip_status(mix::launch_mix_dequantize((int)fmt, codes, shared, rows, cols, out, (hipStream_t)stream),
                    "mix_dequantize launch");
}

mix_status_t mx_dequantize(mx_fmt_t fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                           float* out, void* stream) {
  g_err.clear();
  if (!mx_known(enum_bits(&fmt))) return fail(MIX_E_ENUM, "mx_dequantize: unknown MX format %d", enum_bits(&fmt));
  if (rows < 0 || cols < 0 || cols % 32) return fail(MIX_E_SHAPE, "mx_dequantize: bad shape");
  if (rows == 0 || cols == 0) return MIX_OK;
  if (!codes || !scales || !out) return fail(MIX_E_NULL, "mx_dequantize: NULL pointer");
  return hip_status(mix::launch_mx_dequantize(mx_fp4(fmt), codes, scales, rows, cols, out, (hipStream_t)stream,
                                              mx_g16(fmt)),
                    "mx_dequantize launch");
}

// the enums arrive by address: a by-value copy would already read them as the enum type
static mix_status_t gemm_common(const char* fn, bool eq6, const mix_fmt_t* a_fmt_p, const uint8_t* a_codes,
                                const void* a_shared, const mx_fmt_t* b_fmt_p, const uint8_t* b_codes,
                                const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* c,
                                const mix_dtype_t* c_dtype_p, int64_t ldc, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (!mix_known(enum_bits(a_fmt_p))) return fail(MIX_E_ENUM, "%s: unknown MiX format %d", fn, enum_bits(a_fmt_p));
  if (!mx_known(enum_bits(b_fmt_p))) return fail(MIX_E_ENUM, "%s: unknown MX format %d", fn, enum_bits(b_fmt_p));
  if (mix_status_t st = check_dtype(enum_bits(c_dtype_p))) return st;
  const mix_fmt_t a_fmt = *a_fmt_p;
  const mx_fmt_t b_fmt = *b_fmt_p;
  const mix_dtype_t c_dtype = *c_dtype_p;
  if (mx_g16(b_fmt) && !eq6)
    return fail(MIX_E_UNSUPPORTED, "%s: g16 weights go through mx_gemm_b_image_g16 + mix_mx_gemm_images, or "
                "mix_mx_gemm_eq6", fn);
  if (M < 0 || N < 0 || K < 0) return fail(MIX_E_SHAPE, "%s: negative extent", fn);
  if (K % 32) return fail(MIX_E_SHAPE, "%s: K=%lld is not a multiple of 32", fn, (long long)K);
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return fail(MIX_E_SHAPE, "%s: extent above 2^31-1", fn);
  if (M == 0 || N == 0) return MIX_OK;
  if (ldc < N) return fail(MIX_E_SHAPE, "%s: ldc=%lld < N=%lld", fn, (long long)ldc, (long long)N);
  if (!c) return fail(MIX_E_NULL, "%s: c is NULL", fn);
  if (K > 0 && (!a_codes || !a_shared || !b_codes || !b_scales)) return fail(MIX_E_NULL, "%s: operand pointer is NULL", fn);
  if (K > 0 && (!aligned16(a_codes) || !aligned16(b_codes))) return fail(MIX_E_ALIGN, "%s: code buffers must be 16-byte aligned", fn);
  if (K > 0 && a_fmt == MIX_4P5 && ((uintptr_t)a_shared & 1u)) return fail(MIX_E_ALIGN, "%s: a_shared misaligned", fn);
  if ((uintptr_t)c % dtype_size(c_dtype)) return fail(MIX_E_ALIGN, "%s: c misaligned", fn);
  int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  if (tiles > INT32_MAX) return fail(MIX_E_SHAPE, "%s: too many tiles", fn);
  if (!eq6 && ws && mix::gemm_f8_eligible(M, N, K) && ws_bytes >= mix::gemm_f8_ws_bytes(b_fmt == MX_FP4, M, N, K)) {
    if ((uintptr_t)ws & 255u) return fail(MIX_E_ALIGN, "%s: workspace must be 256-byte aligned", fn);
    if (a_fmt == MIX_4P5 && ((uintptr_t)a_shared & 1u)) return fail(MIX_E_ALIGN, "%s: a_shared misaligned", fn);
    return hip_status(mix::launch_gemm_f8(a_fmt == MIX_4P5, b_fmt == MX_FP4, c_dtype == MIX_BF16, a_codes, a_shared,
                                          b_codes, b_scales, M, N, K, c, ldc, ws, (hipStream_t)stream),
                      "mix_mx_gemm launch");
  }
  mix::GemmArgs g{};
  g.a_codes = a_codes; g.a_shared = a_shared; g.a_pitch = K / 2; g.a_sh_pitch = K / 32;
  g.b_codes = b_codes; g.b_scales = b_scales; g.b_pitch = K / 2; g.b_sc_pitch = mx_g16(b_fmt) ? K / 16 : K / 32;
  g.b_group = 1; g.b_g16 = mx_g16(b_fmt);
  g.c = c; g.ldc = ldc; g.row_div = nullptr;
  g.M = (int)M; g.N = (int)N; g.K = (int)K; g.batch = 1; g.causal = 0;
  hipError_t e = eq6 ? mix::launch_gemm_eq6(a_fmt == MIX_4P5, mx_fp4(b_fmt), c_dtype == MIX_BF16, g, (hipStream_t)stream)
                     : mix::launch_gemm_mfma(a_fmt == MIX_4P5, b_fmt == MX_FP4, c_dtype == MIX_BF16, g, (hipStream_t)stream);
  return hip_status(e, eq6 ? "mix_mx_gemm_eq6 launch" : "mix_mx_gemm launch");
}

size_t mix_mx_gemm_workspace_bytes(mix_fmt_t a_fmt, mx_fmt_t b_fmt, int64_t M, int64_t N, int64_t K) {
  (void)a_fmt;
  const int bf = enum_bits(&b_fmt);
  if (M <= 0 || N <= 0 || K <= 0 || (bf != MX_INT4 && bf != MX_FP4)) return 0;   // g16: no workspace path
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return 0;
  if (!mix::gemm_f8_eligible(M, N, K)) return 0;
  return mix::gemm_f8_ws_bytes(b_fmt == MX_FP4, M, N, K);
}

mix_status_t mix_mx_gemm(mix_fmt_t a_fmt, const uint8_t* a_codes, const void* a_shared, mx_fmt_t b_fmt,
                         const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* c,
                         mix_dtype_t c_dtype, int64_t ldc, void* ws, size_t ws_bytes, void* stream) {
  return gemm_common("mix_mx_gemm", false, &a_fmt, a_codes, a_shared, &b_fmt, b_codes, b_scales, M, N, K, c, &c_dtype,
                     ldc, ws, ws_bytes, stream);
}

mix_status_t mix_mx_gemm_eq6(mix_fmt_t a_fmt, const uint8_t* a_codes, const void* a_shared, mx_fmt_t b_fmt,
                             const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N, int64_t K,
                             void* c, mix_dtype_t c_dtype, int64_t ldc, void* stream) {
  return gemm_common("mix_mx_gemm_eq6", true, &a_fmt, a_codes, a_shared, &b_fmt, b_codes, b_scales, M, N, K, c,
                     &c_dtype, ldc, nullptr, 0, stream);
}

// ---------------------------------------------------------------- GEMM operand images

static bool image_k_ok(int64_t K) { return K > 0 && K % mix::FK == 0 && K <= INT32_MAX; }

size_t mix_gemm_a_image_bytes(int64_t M, int64_t K) {
  if (M <= 0 || M > INT32_MAX || !image_k_ok(K)) return 0;
  return mix::f8_a_image_layout(M, K).total;
}

size_t mx_gemm_b_image_bytes(mx_fmt_t b_fmt, int64_t N, int64_t K) {
  if (!mx_known(enum_bits(&b_fmt)) || N <= 0 || N > INT32_MAX || !image_k_ok(K)) return 0;
  return mix::f8_b_image_layout(b_fmt == MX_FP4, N, K).total;   // g16 images are E4M3 (the MXINT4 layout)
}

static mix_status_t check_image(const char* fn, const void* img, size_t img_bytes, size_t need) {
  if (!img) return fail(MIX_E_NULL, "%s: image is NULL", fn);
  if ((uintptr_t)img & 255u) return fail(MIX_E_ALIGN, "%s: image must be 256-byte aligned", fn);
  if (img_bytes < need) return fail(MIX_E_WORKSPACE, "%s: image buffer %zu < %zu bytes", fn, img_bytes, need);
  return MIX_OK;
}

mix_status_t mix_gemm_a_image(mix_fmt_t a_fmt, const uint8_t* a_codes, const void* a_shared, int64_t M, int64_t K,
                              void* img, size_t img_bytes, void* stream) {
  g_err.clear();
  const char* fn = "mix_gemm_a_image";
  if (!mix_known(enum_bits(&a_fmt))) return fail(MIX_E_ENUM, "%s: unknown MiX format %d", fn, enum_bits(&a_fmt));
  if (M < 0 || K < 0) return fail(MIX_E_SHAPE, "%s: negative extent", fn);
  if (M == 0) return MIX_OK;
  if (M > INT32_MAX || !image_k_ok(K)) return fail(MIX_E_SHAPE, "%s: K=%lld is not a positive multiple of 128", fn, (long long)K);
  if (!a_codes || !a_shared) return fail(MIX_E_NULL, "%s: codes or shared is NULL", fn);
  if (!aligned16(a_codes) || (a_fmt == MIX_4P5 && ((uintptr_t)a_shared & 1u)))
    return fail(MIX_E_ALIGN, "%s: codes not 16-byte aligned or shared misaligned", fn);
  if (mix_status_t st = check_image(fn, img, img_bytes, mix::f8_a_image_layout(M, K).total)) return st;
  return hip_status(mix::launch_gemm_a_image(a_fmt == MIX_4P5, a_codes, a_shared, M, K, img, (hipStream_t)stream), fn);
}

mix_status_t mix_quantize_gemm(mix_fmt_t fmt, const void* x, mix_dtype_t dtype, int64_t rows, int64_t cols,
                               int64_t ldx, uint8_t* codes, void* shared, void* img, size_t img_bytes, void* stream) {
  g_err.clear();
  const char* fn = "mix_quantize_gemm";
  if (!mix_known(enum_bits(&fmt))) return fail(MIX_E_ENUM, "%s: unknown MiX format %d", fn, enum_bits(&fmt));
  if (mix_status_t st = check_dtype(enum_bits(&dtype))) return st;
  bool empty;
  if (mix_status_t st = check_matrix_in(fn, x, dtype, rows, cols, ldx, &empty)) return st;
  if (rows == 0) return MIX_OK;
  if (rows > INT32_MAX || !image_k_ok(cols))
    return fail(MIX_E_SHAPE, "%s: cols=%lld is not a positive multiple of 128", fn, (long long)cols);
  if (!codes != !shared) return fail(MIX_E_NULL, "%s: codes and shared must both be given or both be NULL", fn);
  if (codes && (!aligned16(codes) || ((uintptr_t)shared & 1u)))
    return fail(MIX_E_ALIGN, "%s: codes not 16-byte aligned or shared not 2-byte aligned", fn);
  if (mix_status_t st = check_image(fn, img, img_bytes, mix::f8_a_image_layout(rows, cols).total)) return st;
  return hip_status(mix::launch_mix_quantize_img((int)fmt, x, (int)dtype, rows, cols, ldx, codes, shared, img,
                                                 (hipStream_t)stream),
                    fn);
}

mix_status_t mx_gemm_b_image(mx_fmt_t b_fmt, const uint8_t* b_codes, const uint8_t* b_scales, int64_t N, int64_t K,
                             void* img, size_t img_bytes, void* stream) {
  g_err.clear();
  const char* fn = "mx_gemm_b_image";
  if (!mx_known(enum_bits(&b_fmt))) return fail(MIX_E_ENUM, "%s: unknown MX format %d", fn, enum_bits(&b_fmt));
  if (mx_g16(b_fmt)) return fail(MIX_E_UNSUPPORTED, "%s: g16 weights: use mx_gemm_b_image_g16", fn);
  if (N < 0 || K < 0) return fail(MIX_E_SHAPE, "%s: negative extent", fn);
  if (N == 0) return MIX_OK;
  if (N > INT32_MAX || !image_k_ok(K)) return fail(MIX_E_SHAPE, "%s: K=%lld is not a positive multiple of 128", fn, (long long)K);
  if (!b_scales || !b_codes) return fail(MIX_E_NULL, "%s: codes or scales is NULL", fn);
  if (!aligned16(b_codes)) return fail(MIX_E_ALIGN, "%s: codes not 16-byte aligned", fn);
  if (mix_status_t st = check_image(fn, img, img_bytes, mix::f8_b_image_layout(b_fmt == MX_FP4, N, K).total)) return st;
  return hip_status(mix::launch_gemm_b_image(b_fmt == MX_FP4, b_codes, b_scales, N, K, img, (hipStream_t)stream), fn);
}

mix_status_t mx_gemm_b_image_g16(mx_fmt_t b_fmt, const uint8_t* b_codes, const uint8_t* b_scales16, int64_t N,
                                 int64_t K, void* img, size_t img_bytes, uint32_t* unfoldable, void* stream) {
  g_err.clear();
  const char* fn = "mx_gemm_b_image_g16";
  if (enum_bits(&b_fmt) != MX_INT4_G16 && enum_bits(&b_fmt) != MX_FP4_G16)
    return fail(MIX_E_ENUM, "%s: format %d is not a g16 format", fn, enum_bits(&b_fmt));
  if (N < 0 || K < 0) return fail(MIX_E_SHAPE, "%s: negative extent", fn);
  if (N == 0) return MIX_OK;
  if (N > INT32_MAX || !image_k_ok(K)) return fail(MIX_E_SHAPE, "%s: K=%lld is not a positive multiple of 128", fn, (long long)K);
  if (!b_codes || !b_scales16 || !unfoldable) return fail(MIX_E_NULL, "%s: codes, scales or the counter is NULL", fn);
  if (!aligned16(b_codes) || ((uintptr_t)unfoldable & 3u))
    return fail(MIX_E_ALIGN, "%s: codes not 16-byte aligned or the counter not 4-byte aligned", fn);
  if (mix_status_t st = check_image(fn, img, img_bytes, mix::f8_b_image_layout(0, N, K).total)) return st;
  return hip_status(mix::launch_gemm_b_image_g16(b_fmt == MX_FP4_G16, b_codes, b_scales16, N, K, img, unfoldable,
                                                 (hipStream_t)stream),
                    fn);
}

mix_status_t mix_mx_gemm_images(mx_fmt_t b_fmt, const void* a_img, const void* b_img, const uint8_t* b_codes,
                                int64_t M, int64_t N, int64_t K, void* c, mix_dtype_t c_dtype, int64_t ldc,
                                void* stream) {
  g_err.clear();
  const char* fn = "mix_mx_gemm_images";
  if (!mx_known(enum_bits(&b_fmt))) return fail(MIX_E_ENUM, "%s: unknown MX format %d", fn, enum_bits(&b_fmt));
  if (mix_status_t st = check_dtype(enum_bits(&c_dtype))) return st;
  if (M < 0 || N < 0 || K < 0) return fail(MIX_E_SHAPE, "%s: negative extent", fn);
  if (M == 0 || N == 0) return MIX_OK;
  if (M > INT32_MAX || N > INT32_MAX || !image_k_ok(K))
    return fail(MIX_E_SHAPE, "%s: K=%lld is not a positive multiple of 128 (or an extent is above 2^31-1)", fn, (long long)K);
  if (ldc < N) return fail(MIX_E_SHAPE, "%s: ldc=%lld < N=%lld", fn, (long long)ldc, (long long)N);
  if (M > 16 && !mix::gemm_f8_offsets_ok(M, N, K))
    return fail(MIX_E_UNSUPPORTED, "%s: an operand image of %lld x %lld x %lld reaches 2^31 bytes", fn, (long long)M,
                (long long)N, (long long)K);
  if (!c || !a_img || !b_img) return fail(MIX_E_NULL, "%s: c or an image is NULL", fn);
  (void)b_codes;   // the B image holds every operand byte
  if (((uintptr_t)a_img & 255u) || ((uintptr_t)b_img & 255u)) return fail(MIX_E_ALIGN, "%s: images must be 256-byte aligned", fn);
  if ((uintptr_t)c % dtype_size(c_dtype)) return fail(MIX_E_ALIGN, "%s: c misaligned", fn);
  return hip_status(mix::launch_gemm_images(b_fmt == MX_FP4, c_dtype == MIX_BF16, a_img, b_img, M, N, K, c, ldc,
                                            (hipStream_t)stream),
                    fn);
}

mix_status_t mix_mx_gemm_images_quantize(mx_fmt_t b_fmt, const void* a_img, const void* b_img, const uint8_t* b_codes,
                                         int64_t M, int64_t N, int64_t K, void* c, int64_t ldc, uint8_t* q_codes,
                                         void* q_shared, void* q_img, size_t q_img_bytes, void* stream) {
  g_err.clear();
  const char* fn = "mix_mx_gemm_images_quantize";
  if (!mx_known(enum_bits(&b_fmt))) return fail(MIX_E_ENUM, "%s: unknown MX format %d", fn, enum_bits(&b_fmt));
  if (M < 0 || N < 0 || K < 0) return fail(MIX_E_SHAPE, "%s: negative extent", fn);
  if (M == 0 || N == 0) return MIX_OK;
  if (M > INT32_MAX || N > INT32_MAX || !image_k_ok(K))
    return fail(MIX_E_SHAPE, "%s: K=%lld is not a positive multiple of 128 (or an extent is above 2^31-1)", fn, (long long)K);
  if (N % 32) return fail(MIX_E_SHAPE, "%s: N=%lld is not a multiple of 32 (MiX blocks run along N)", fn, (long long)N);
  if (q_img && N % 128)
    return fail(MIX_E_SHAPE, "%s: the output's A image needs N (its K) a multiple of 128, got %lld", fn, (long long)N);
  if (c && ldc < N) return fail(MIX_E_SHAPE, "%s: ldc=%lld < N=%lld", fn, (long long)ldc, (long long)N);
  if (M <= 16 && !c) return fail(MIX_E_NULL, "%s: M <= 16 needs c (the weight stream writes C first)", fn);
  if (M > 16 && (!mix::gemm_f8_offsets_ok(M, N, K) || (q_img && !mix::gemm_f8_offsets_ok(M, 1, N))))
    return fail(MIX_E_UNSUPPORTED, "%s: an operand or output image of %lld x %lld x %lld reaches 2^31 bytes", fn,
                (long long)M, (long long)N, (long long)K);
  if (!a_img || !b_img || !q_codes || !q_shared) return fail(MIX_E_NULL, "%s: an image or an output is NULL", fn);
  (void)b_codes;   // the B image holds every operand byte
  if (((uintptr_t)a_img & 255u) || ((uintptr_t)b_img & 255u) || ((uintptr_t)q_img & 255u))
    return fail(MIX_E_ALIGN, "%s: images must be 256-byte aligned", fn);
  if (((uintptr_t)q_codes & 3u) || ((uintptr_t)q_shared & 1u) || ((uintptr_t)c & 1u))
    return fail(MIX_E_ALIGN, "%s: q_codes must be 4-byte aligned, q_shared and c 2-byte aligned", fn);
  if (M <= 16 && (!aligned16(c) || (ldc * 2) % 16))
    return fail(MIX_E_ALIGN, "%s: for M <= 16, c and its row pitch must be 16-byte aligned", fn);
  if (q_img && q_img_bytes < mix::f8_a_image_layout(M, N).total)
    return fail(MIX_E_WORKSPACE, "%s: output image buffer %zu < %zu bytes", fn, q_img_bytes,
                mix::f8_a_image_layout(M, N).total);
  return hip_status(mix::launch_gemm_images_q(b_fmt == MX_FP4, a_img, b_img, M, N, K, c, ldc, q_codes, q_shared,
                                              q_img, (hipStream_t)stream),
                    fn);
}

mix_status_t mix_kmean(const void* k, mix_dtype_t dtype, int64_t T, int64_t C, int64_t ldk, float* mu, void* stream) {
  g_err.clear();
  if (mix_status_t st = check_dtype(enum_bits(&dtype))) return st;
  if (T < 0 || C < 0) return fail(MIX_E_SHAPE, "mix_kmean: negative extent");
  if (C == 0) return MIX_OK;
  if (T == 0) return fail(MIX_E_SHAPE, "mix_kmean: the mean of zero tokens is undefined");
  if (C % 32) return fail(MIX_E_SHAPE, "mix_kmean: C=%lld is not a multiple of 32", (long long)C);
  if (ldk < C) return fail(MIX_E_SHAPE, "mix_kmean: ldk < C");
  if (!k || !mu) return fail(MIX_E_NULL, "mix_kmean: NULL pointer");
  if (!aligned16(k) || (ldk * dtype_size(dtype)) % 16)
    return fail(MIX_E_ALIGN, "mix_kmean: k or its row pitch is not 16-byte aligned");
  return hip_status(mix::launch_kmean(k, (int)dtype, T, C, ldk, mu, (hipStream_t)stream), "mix_kmean launch");
}

size_t mix_underflow_map_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0 || cols % 32 || rows > INT32_MAX || cols > INT32_MAX || rows * cols > kMaxElems) return 0;
  return mix::uf_plan(rows, cols).bytes;
}

mix_status_t mix_underflow_map(const void* x, mix_dtype_t dtype, int64_t rows, int64_t cols, int64_t ldx,
                               const float* mu, uint32_t* counts, float* amax, void* ws, size_t ws_bytes,
                               void* stream) {
  g_err.clear();
  if (mix_status_t st = check_dtype(enum_bits(&dtype))) return st;
  bool empty;
  if (mix_status_t st = check_matrix_in("mix_underflow_map", x, dtype, rows, cols, ldx, &empty)) return st;
  if (rows > INT32_MAX) return fail(MIX_E_SHAPE, "mix_underflow_map: rows above 2^31-1");
  if (cols == 0) return MIX_OK;
  if (!counts || !amax) return fail(MIX_E_NULL, "mix_underflow_map: counts or amax is NULL");
  if (((uintptr_t)counts & 3u) || ((uintptr_t)amax & 3u) || (mu && !aligned16(mu)))
    return fail(MIX_E_ALIGN, "mix_underflow_map: counts/amax not 4-byte aligned or mu not 16-byte aligned");
  if (empty) rows = 0;   // zero rows: the counts and amax are still cleared
  const size_t need = rows ? mix::uf_plan(rows, cols).bytes : 0;
  if (need) {
    if (!ws) return fail(MIX_E_NULL, "mix_underflow_map: workspace is NULL (%zu bytes needed)", need);
    if (ws_bytes < need) return fail(MIX_E_WORKSPACE, "mix_underflow_map: workspace of %zu bytes, %zu needed", ws_bytes, need);
    if (!aligned16(ws)) return fail(MIX_E_ALIGN, "mix_underflow_map: workspace not 16-byte aligned");
  }
  return hip_status(mix::launch_underflow_map(x, (int)dtype, rows, cols, ldx, mu, counts, amax, ws, (hipStream_t)stream),
                    "mix_underflow_map launch");
}

}  // extern "C"

// ---------------------------------------------------------------- attention
extern "C" {

// Extents the attention entry points accept (each checked before any product of them is formed).
static bool prefill_extents_ok(int64_t T, int64_t Hq, int64_t Hkv, int64_t d) {
  return T <= (1 << 24) && Hq <= (1 << 20) && Hkv <= Hq && d <= (1 << 20) && Hq * d <= (1 << 20);
}

static bool decode_extents_ok(int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t L) {
  if (B > (1 << 20) || Hq > (1 << 20) || Hkv > (1 << 20) || d > 1024 || L > INT32_MAX) return false;
  const int64_t bh = B * (Hq > Hkv ? Hq : Hkv);   // below 2^40
  return bh <= (1 << 24) && bh * L <= kMaxElems && bh * L * d <= kMaxElems;
}

size_t mix_attn_prefill_workspace_bytes(int64_t T, int64_t Hq, int64_t Hkv, int64_t d) {
  if (T <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || !prefill_extents_ok(T, Hq, Hkv, d)) return 0;
  return mix::attn_prefill_ws_bytes(T, Hq, Hkv, d);
}

mix_status_t mix_attn_prefill(const void* q, const void* k, const void* v, int64_t T, int64_t Hq, int64_t Hkv,
                              int64_t d, int causal, float* mu, void* o, void* ws, size_t ws_bytes,
                              const mix_attn_debug_t* dbg, void* stream) {
  g_err.clear();
  if (T < 0 || Hq < 0 || Hkv < 0 || d < 0) return fail(MIX_E_SHAPE, "mix_attn_prefill: negative extent");
  if (T == 0 || Hq == 0 || d == 0) return MIX_OK;
  if (Hkv == 0 || Hq % Hkv) return fail(MIX_E_SHAPE, "mix_attn_prefill: Hq=%lld is not a multiple of Hkv=%lld", (long long)Hq, (long long)Hkv);
  if (d % 32) return fail(MIX_E_SHAPE, "mix_attn_prefill: head dim %lld is not a multiple of 32", (long long)d);
  if (!prefill_extents_ok(T, Hq, Hkv, d)) return fail(MIX_E_SHAPE, "mix_attn_prefill: extent too large");
  if (!q || !k || !v || !mu || !o || !ws) return fail(MIX_E_NULL, "mix_attn_prefill: NULL pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(mu) || ((uintptr_t)ws & 255u) || ((uintptr_t)o & 1u))
    return fail(MIX_E_ALIGN, "mix_attn_prefill: q/k/v/mu must be 16-byte aligned and ws 256-byte aligned");
  if (dbg && (!aligned16(dbg->p) || ((uintptr_t)dbg->p_shared & 1u)))
    return fail(MIX_E_ALIGN, "mix_attn_prefill: debug p must be 16-byte aligned");
  size_t need = mix::attn_prefill_ws_bytes(T, Hq, Hkv, d);
  if (ws_bytes < need) return fail(MIX_E_WORKSPACE, "mix_attn_prefill: workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(mix::attn_prefill_run(q, k, v, T, Hq, Hkv, d, causal, mu, o, ws, dbg, (hipStream_t)stream),
                    "mix_attn_prefill");
}

static mix_status_t check_cache(const char* fn, const mix_kv_cache_t* c) {
  if (!c) return fail(MIX_E_NULL, "%s: cache is NULL", fn);
  if (!c->k_codes || !c->k_scales || !c->v_codes || !c->v_scales || !c->v_stage)
    return fail(MIX_E_NULL, "%s: a cache buffer is NULL", fn);
  if (c->B <= 0 || c->Hkv <= 0 || c->Lmax <= 0 || c->Lmax % 32 || c->d <= 0 || c->d % 32)
    return fail(MIX_E_SHAPE, "%s: bad cache extents (Lmax and d must be positive multiples of 32)", fn);
  if (!decode_extents_ok(c->B, c->Hkv, c->Hkv, c->d, c->Lmax))
    return fail(MIX_E_SHAPE, "%s: cache extents too large", fn);
  if (!aligned16(c->k_codes) || !aligned16(c->v_codes) || !aligned16(c->v_stage))
    return fail(MIX_E_ALIGN, "%s: cache code buffers must be 16-byte aligned", fn);
  return MIX_OK;
}

mix_status_t mix_kv_cache_prefill(const mix_kv_cache_t* cache, int64_t b, const void* k, const void* v, int64_t T,
                                  const float* mu, void* stream) {
  g_err.clear();
  if (mix_status_t st = check_cache("mix_kv_cache_prefill", cache)) return st;
  if (b < 0 || b >= cache->B) return fail(MIX_E_SHAPE, "mix_kv_cache_prefill: row %lld outside [0, %lld)", (long long)b, (long long)cache->B);
  if (T <= 0 || T > cache->Lmax) return fail(MIX_E_SHAPE, "mix_kv_cache_prefill: T=%lld outside (0, Lmax]", (long long)T);
  if (!k || !v || !mu) return fail(MIX_E_NULL, "mix_kv_cache_prefill: NULL pointer");
  if (!aligned16(k) || !aligned16(v) || !aligned16(mu)) return fail(MIX_E_ALIGN, "mix_kv_cache_prefill: k/v/mu must be 16-byte aligned");
  return hip_status(mix::kv_cache_prefill_run(cache, b, k, v, T, mu, (hipStream_t)stream), "mix_kv_cache_prefill");
}

size_t mix_attn_decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t max_pos) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || max_pos < 0 || max_pos >= INT32_MAX || !decode_extents_ok(B, Hq, Hkv, d, max_pos + 1)) return 0;
  return mix::attn_decode_ws_bytes(B, Hq, Hkv, d, max_pos);
}

mix_status_t mix_attn_decode(const void* q, const void* k_new, const void* v_new, const mix_kv_cache_t* cache,
                             const int32_t* pos, int64_t max_pos, int64_t Hq, const float* mu, void* o, void* ws,
                             size_t ws_bytes, const mix_attn_debug_t* dbg, void* stream) {
  g_err.clear();
  if (mix_status_t st = check_cache("mix_attn_decode", cache)) return st;
  if (Hq <= 0 || Hq % cache->Hkv) return fail(MIX_E_SHAPE, "mix_attn_decode: Hq must be a positive multiple of Hkv");
  if (cache->d != 128) return fail(MIX_E_UNSUPPORTED, "mix_attn_decode: head dim %lld (only 128 is implemented)", (long long)cache->d);
  if (Hq / cache->Hkv > 16) return fail(MIX_E_UNSUPPORTED, "mix_attn_decode: more than 16 query heads per KV head");
  if (!decode_extents_ok(cache->B, Hq, cache->Hkv, cache->d, cache->Lmax))
    return fail(MIX_E_SHAPE, "mix_attn_decode: extents too large");
  if (max_pos < 0 || max_pos >= cache->Lmax) return fail(MIX_E_SHAPE, "mix_attn_decode: max_pos=%lld outside [0, Lmax)", (long long)max_pos);
  if (!q || !k_new || !v_new || !pos || !mu || !o || !ws) return fail(MIX_E_NULL, "mix_attn_decode: NULL pointer");
  if (((uintptr_t)ws & 255u) || !aligned16(q) || ((uintptr_t)o & 7u) || ((uintptr_t)pos & 3u) || ((uintptr_t)mu & 3u))
    return fail(MIX_E_ALIGN, "mix_attn_decode: misaligned argument (ws must be 256-byte aligned, q 16-byte, o 8-byte)");
  if (dbg && !aligned16(dbg->p)) return fail(MIX_E_ALIGN, "mix_attn_decode: debug p must be 16-byte aligned");
  size_t need = mix::attn_decode_ws_bytes(cache->B, Hq, cache->Hkv, cache->d, max_pos);
  if (ws_bytes < need) return fail(MIX_E_WORKSPACE, "mix_attn_decode: workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(mix::attn_decode_run(q, k_new, v_new, cache, pos, max_pos, Hq, mu, o, ws, dbg, (hipStream_t)stream),
                    "mix_attn_decode");
}

size_t mix_decode_step_workspace_bytes(int64_t B, int64_t K, int64_t Hq, int64_t Hkv, int64_t d, int64_t max_pos) {
  if (B <= 0 || K <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || max_pos < 0 || max_pos >= INT32_MAX || K > INT32_MAX ||
      !decode_extents_ok(B, Hq, Hkv, d, max_pos + 1) || B * K > kMaxElems)
    return 0;
  return mix::decode_step_ws_bytes(B, K, Hq, Hkv, d, max_pos);
}

static mix_status_t check_decode_step(const char* fn, const void* x, int64_t K, int64_t N, const mx_fmt_t* b_fmt,
                                      const void* b_img, void* y, const void* q, const void* k_new,
                                      const void* v_new, const mix_kv_cache_t* cache, const int32_t* pos,
                                      int64_t max_pos, int64_t Hq, const float* mu, void* o) {
  if (mix_status_t st = check_cache(fn, cache)) return st;
  if (!mx_known(enum_bits(b_fmt))) return fail(MIX_E_ENUM, "%s: unknown MX format %d", fn, enum_bits(b_fmt));
  if (Hq <= 0 || Hq % cache->Hkv) return fail(MIX_E_SHAPE, "%s: Hq must be a positive multiple of Hkv", fn);
  if (cache->d != 128) return fail(MIX_E_UNSUPPORTED, "%s: head dim %lld (only 128 is implemented)", fn, (long long)cache->d);
  if (Hq / cache->Hkv > 16) return fail(MIX_E_UNSUPPORTED, "%s: more than 16 query heads per KV head", fn);
  if (!decode_extents_ok(cache->B, Hq, cache->Hkv, cache->d, cache->Lmax))
    return fail(MIX_E_SHAPE, "%s: extents too large", fn);
  if (cache->B > 16) return fail(MIX_E_UNSUPPORTED, "%s: batch %lld above 16 (the weight stream's rows)", fn, (long long)cache->B);
  if (max_pos < 0 || max_pos >= cache->Lmax) return fail(MIX_E_SHAPE, "%s: max_pos=%lld outside [0, Lmax)", fn, (long long)max_pos);
  if (N <= 0 || N > INT32_MAX || !image_k_ok(K) || K > INT32_MAX)
    return fail(MIX_E_SHAPE, "%s: K=%lld must be a positive multiple of 128 and N=%lld positive", fn, (long long)K, (long long)N);
  if (!mix::gemm_f8_offsets_ok(1, N, K) || cache->B * K >= ((int64_t)1 << 31))
    return fail(MIX_E_UNSUPPORTED, "%s: an operand image of %lld x %lld reaches 2^31 bytes", fn, (long long)N, (long long)K);
  if (!x || !b_img || !y || !q || !k_new || !v_new || !pos || !mu || !o) return fail(MIX_E_NULL, "%s: NULL pointer", fn);
  if (((uintptr_t)b_img & 255u) || !aligned16(x) || !aligned16(q) || ((uintptr_t)y & 1u) || ((uintptr_t)o & 7u) ||
      ((uintptr_t)pos & 3u) || ((uintptr_t)mu & 3u))
    return fail(MIX_E_ALIGN, "%s: misaligned argument (b_img 256-byte, x and q 16-byte, o 8-byte)", fn);
  return MIX_OK;
}

mix_status_t mix_decode_step(const void* x, int64_t K, int64_t N, mx_fmt_t b_fmt, const void* b_img, void* y,
                             const void* q, const void* k_new, const void* v_new, const mix_kv_cache_t* cache,
                             const int32_t* pos, int64_t max_pos, int64_t Hq, const float* mu, void* o, void* ws,
                             size_t ws_bytes, void* stream) {
  g_err.clear();
  const char* fn = "mix_decode_step";
  if (mix_status_t st = check_decode_step(fn, x, K, N, &b_fmt, b_img, y, q, k_new, v_new, cache, pos, max_pos, Hq, mu,
                                          o))
    return st;
  if (!ws) return fail(MIX_E_NULL, "%s: ws is NULL", fn);
  if ((uintptr_t)ws & 255u) return fail(MIX_E_ALIGN, "%s: ws must be 256-byte aligned", fn);
  const size_t need = mix::decode_step_ws_bytes(cache->B, K, Hq, cache->Hkv, cache->d, max_pos);
  if (ws_bytes < need) return fail(MIX_E_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  return hip_status(mix::decode_step_run(x, K, N, b_fmt == MX_FP4, b_img, y, q, k_new, v_new, cache, pos, max_pos, Hq,
                                         mu, o, ws, (hipStream_t)stream),
                    fn);
}

mix_status_t mix_decode_step_single(const void* x, int64_t K, int64_t N, mx_fmt_t b_fmt, const void* b_img, void* y,
                                    const void* q, const void* k_new, const void* v_new,
                                    const mix_kv_cache_t* cache, const int32_t* pos, int64_t max_pos, int64_t Hq,
                                    const float* mu, void* o, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  const char* fn = "mix_decode_step_single";
  if (mix_status_t st = check_decode_step(fn, x, K, N, &b_fmt, b_img, y, q, k_new, v_new, cache, pos, max_pos, Hq, mu,
                                          o))
    return st;
  if (!ws) return fail(MIX_E_NULL, "%s: ws is NULL", fn);
  if ((uintptr_t)ws & 255u) return fail(MIX_E_ALIGN, "%s: ws must be 256-byte aligned", fn);
  const size_t need = mix::decode_step_ws_bytes(cache->B, K, Hq, cache->Hkv, cache->d, max_pos);
  if (ws_bytes < need) return fail(MIX_E_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  return hip_status(mix::decode_step_single_run(x, K, N, b_fmt == MX_FP4, b_img, y, q, k_new, v_new, cache, pos,
                                                max_pos, Hq, mu, o, ws, (hipStream_t)stream),
                    fn);
}

size_t mix_decode_step_static_max_bytes(void) { return mix::DECODE_SCRATCH_BYTES; }

mix_status_t mix_decode_step_static(const void* x, int64_t K, int64_t N, mx_fmt_t b_fmt, const void* b_img, void* y,
                                    const void* q, const void* k_new, const void* v_new,
                                    const mix_kv_cache_t* cache, const int32_t* pos, int64_t max_pos, int64_t Hq,
                                    const float* mu, void* o, void* stream) {
  g_err.clear();
  const char* fn = "mix_decode_step_static";
  if (mix_status_t st = check_decode_step(fn, x, K, N, &b_fmt, b_img, y, q, k_new, v_new, cache, pos, max_pos, Hq, mu,
                                          o))
    return st;
  const size_t need = mix::decode_step_ws_bytes(cache->B, K, Hq, cache->Hkv, cache->d, max_pos);
  if (need > mix::DECODE_SCRATCH_BYTES)
    return fail(MIX_E_WORKSPACE, "%s: this shape needs %zu bytes of scratch, above the library's %zu", fn, need,
                mix::DECODE_SCRATCH_BYTES);
  return hip_status(mix::decode_step_static_run(x, K, N, b_fmt == MX_FP4, b_img, y, q, k_new, v_new, cache, pos,
                                                max_pos, Hq, mu, o, (hipStream_t)stream),
                    fn);
}

}  // extern "C"
