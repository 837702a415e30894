/*
 * Host-side argument checks of every mixlib entry point, run under AddressSanitizer and
 * UndefinedBehaviorSanitizer (a build of the library's host code only, no GPU needed): each call
 * must return its documented status before any HIP call, and the size functions must not overflow
 * for extreme extents. Exit status 0 when every check holds; a sanitizer report aborts the run.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mixlib.h"

static int failures = 0;

#define EXPECT(call, want)                                                                          \
  do {                                                                                              \
    int got_ = (int)(call);                                                                         \
    if (got_ != (int)(want)) {                                                                      \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d (%s)\n", __FILE__, __LINE__, #call, got_, \
              (int)(want), mix_last_error());                                                       \
      failures++;                                                                                   \
    }                                                                                               \
  } while (0)

#define EXPECT_TRUE(cond)                                                            \
  do {                                                                               \
    if (!(cond)) {                                                                   \
      fprintf(stderr, "%s:%d: %s does not hold\n", __FILE__, __LINE__, #cond);       \
      failures++;                                                                    \
    }                                                                                \
  } while (0)

/* never dereferenced: every call below fails validation or is empty first */
#define FAKE ((void*)(uintptr_t)0x10000)
#define MIS1 ((void*)(uintptr_t)0x10001)
#define MIS2 ((void*)(uintptr_t)0x10002)
#define MIS4 ((void*)(uintptr_t)0x10004)
#define MIS8 ((void*)(uintptr_t)0x10008)
#define A16 ((void*)(uintptr_t)0x10010)

static const int64_t HUGE_EXT[] = {INT64_MAX, INT64_MAX / 2, (int64_t)1 << 62, (int64_t)1 << 40, (int64_t)1 << 31,
                                   INT64_MIN, -1};
#define NHUGE (int)(sizeof(HUGE_EXT) / sizeof(HUGE_EXT[0]))

static void quantizers(void) {
  EXPECT(mix_quantize((mix_fmt_t)7, FAKE, MIX_F32, 1, 32, 32, FAKE, FAKE, NULL), MIX_E_ENUM);
  EXPECT(mix_quantize(MIX_4P5, FAKE, (mix_dtype_t)5, 1, 32, 32, FAKE, FAKE, NULL), MIX_E_ENUM);
  EXPECT(mix_quantize(MIX_4P5, FAKE, MIX_F32, 1, 33, 33, FAKE, FAKE, NULL), MIX_E_SHAPE);
  EXPECT(mix_quantize(MIX_4P5, FAKE, MIX_F32, 2, 64, 32, FAKE, FAKE, NULL), MIX_E_SHAPE);
  EXPECT(mix_quantize(MIX_4P5, NULL, MIX_F32, 1, 32, 32, FAKE, FAKE, NULL), MIX_E_NULL);
  EXPECT(mix_quantize(MIX_4P5, MIS1, MIX_F32, 1, 32, 32, FAKE, FAKE, NULL), MIX_E_ALIGN);
  EXPECT(mix_quantize(MIX_4P5, FAKE, MIX_BF16, 2, 32, 36, FAKE, FAKE, NULL), MIX_E_ALIGN);
  EXPECT(mix_quantize(MIX_4P5, NULL, MIX_F32, 0, 32, 32, NULL, NULL, NULL), MIX_OK);
  EXPECT(mx_quantize((mx_fmt_t)4, FAKE, MIX_F32, 1, 32, 32, NULL, FAKE, FAKE, NULL), MIX_E_ENUM);
  EXPECT(mx_quantize(MX_FP4, FAKE, MIX_F32, 1, 32, 32, MIS1, FAKE, FAKE, NULL), MIX_E_ALIGN);
  EXPECT(mx_quantize(MX_FP4_G16, FAKE, MIX_F32, 1, 48, 48, NULL, FAKE, FAKE, NULL), MIX_E_SHAPE);
  EXPECT(mx_quantize_cols(FAKE, MIX_BF16, 10, 4, 2, FAKE, FAKE, NULL), MIX_E_SHAPE);
  EXPECT(mx_quantize_cols(FAKE, MIX_BF16, 10, 4, 4, MIS8, FAKE, NULL), MIX_E_ALIGN);
  EXPECT(mx_quantize_cols(FAKE, MIX_BF16, (int64_t)1 << 40, 4, 4, FAKE, FAKE, NULL), MIX_E_SHAPE);
  for (int i = 0; i < NHUGE; i++) {
    const int64_t h = HUGE_EXT[i];
    /* a huge extent is refused (or is the documented empty call), never wrapped */
    int st = mix_quantize(MIX_4P5, FAKE, MIX_F32, h, 32, 32, FAKE, FAKE, NULL);
    EXPECT_TRUE(st != MIX_OK || h == 0);
    st = mix_quantize(MIX_4P5, FAKE, MIX_F32, 1, h, h, FAKE, FAKE, NULL);
    EXPECT_TRUE(st != MIX_OK);
    st = mx_quantize(MX_INT4, FAKE, MIX_BF16, 4, h, h, NULL, FAKE, FAKE, NULL);
    EXPECT_TRUE(st != MIX_OK);
    st = mx_quantize_cols(FAKE, MIX_F32, h, 32, 32, FAKE, FAKE, NULL);
    EXPECT_TRUE(st != MIX_OK);
  }
}

static void gemm(void) {
  EXPECT(mix_mx_gemm((mix_fmt_t)3, FAKE, FAKE, MX_FP4, FAKE, FAKE, 4, 4, 32, FAKE, MIX_F32, 4, NULL, 0, NULL), MIX_E_ENUM);
  EXPECT(mix_mx_gemm(MIX_4P5, FAKE, FAKE, MX_FP4, FAKE, FAKE, 4, 4, 40, FAKE, MIX_F32, 4, NULL, 0, NULL), MIX_E_SHAPE);
  EXPECT(mix_mx_gemm(MIX_4P5, FAKE, FAKE, MX_FP4, FAKE, FAKE, 4, 4, 32, FAKE, MIX_F32, 3, NULL, 0, NULL), MIX_E_SHAPE);
  EXPECT(mix_mx_gemm(MIX_4P5, NULL, FAKE, MX_FP4, FAKE, FAKE, 4, 4, 32, FAKE, MIX_F32, 4, NULL, 0, NULL), MIX_E_NULL);
  EXPECT(mix_mx_gemm(MIX_4P5, FAKE, FAKE, MX_FP4, FAKE, FAKE, 256, 256, 128, FAKE, MIX_F32, 256, MIS1, 1 << 20, NULL),
         MIX_E_ALIGN);
  EXPECT(mix_mx_gemm(MIX_4P5, FAKE, FAKE, MX_INT4_G16, FAKE, FAKE, 4, 4, 32, FAKE, MIX_F32, 4, NULL, 0, NULL),
         MIX_E_UNSUPPORTED);
  EXPECT(mix_mx_gemm_eq6(MIX_4P25, FAKE, FAKE, MX_INT4, FAKE, FAKE, -4, 4, 32, FAKE, MIX_F32, 4, NULL), MIX_E_SHAPE);
  EXPECT(mix_mx_gemm_eq6(MIX_4P25, NULL, NULL, MX_INT4, NULL, NULL, 0, 4, 32, NULL, MIX_F32, 4, NULL), MIX_OK);
  EXPECT(mix_gemm_a_image(MIX_4P5, FAKE, FAKE, 4, 128, A16, 1 << 20, NULL), MIX_E_ALIGN);
  EXPECT(mix_gemm_a_image(MIX_4P5, FAKE, FAKE, 4, 128, FAKE, 100, NULL), MIX_E_WORKSPACE);
  EXPECT(mix_quantize_gemm(MIX_4P5, FAKE, MIX_BF16, 4, 128, 128, FAKE, NULL, FAKE, 1 << 20, NULL), MIX_E_NULL);
  EXPECT(mx_gemm_b_image(MX_INT4, FAKE, FAKE, 4, 128, A16, 1 << 20, NULL), MIX_E_ALIGN);
  EXPECT(mx_gemm_b_image_g16(MX_FP4_G16, FAKE, FAKE, 256, 256, FAKE, 16, FAKE, NULL), MIX_E_WORKSPACE);
  EXPECT(mix_mx_gemm_images(MX_FP4, FAKE, FAKE, NULL, (int64_t)1 << 20, 256, 2048, FAKE, MIX_BF16, 256, NULL),
         MIX_E_UNSUPPORTED);
  EXPECT(mix_mx_gemm_images_quantize(MX_FP4, FAKE, FAKE, NULL, 8, 256, 128, NULL, 0, FAKE, FAKE, NULL, 0, NULL),
         MIX_E_NULL);
  for (int i = 0; i < NHUGE; i++) {
    const int64_t h = HUGE_EXT[i];
    /* the size functions return 0 or a size that does not wrap; the entry points refuse */
    const size_t a = mix_gemm_a_image_bytes(h, 128), b = mix_gemm_a_image_bytes(4, h);
    EXPECT_TRUE(a == 0 || a >= (size_t)h * 128u);
    EXPECT_TRUE(b == 0 || b >= (size_t)h * 4u);
    for (int f = 0; f < 4; f++) {
      const size_t s1 = mx_gemm_b_image_bytes((mx_fmt_t)f, h, 3584), s2 = mx_gemm_b_image_bytes((mx_fmt_t)f, 256, h);
      EXPECT_TRUE(s1 == 0 || s1 >= (size_t)h * 1792u);
      EXPECT_TRUE(s2 == 0 || s2 >= (size_t)h * 128u);
      const size_t w = mix_mx_gemm_workspace_bytes(MIX_4P5, (mx_fmt_t)f, h, 18944, 3584);
      EXPECT_TRUE(w == 0 || w >= (size_t)h * 3584u);
      const size_t w2 = mix_mx_gemm_workspace_bytes(MIX_4P5, (mx_fmt_t)f, 4096, h, 3584);
      EXPECT_TRUE(w2 == 0 || w2 >= (size_t)h * 1792u);
      (void)mix_mx_gemm_workspace_bytes(MIX_4P25, (mx_fmt_t)f, 4096, 4096, h);
    }
    int st = mix_mx_gemm(MIX_4P5, FAKE, FAKE, MX_FP4, FAKE, FAKE, h, 256, 128, FAKE, MIX_F32, 256, NULL, 0, NULL);
    EXPECT_TRUE(st != MIX_OK);
    st = mix_mx_gemm(MIX_4P5, FAKE, FAKE, MX_FP4, FAKE, FAKE, 256, h, 128, FAKE, MIX_F32, h, NULL, 0, NULL);
    EXPECT_TRUE(st != MIX_OK);
    st = mix_mx_gemm(MIX_4P5, FAKE, FAKE, MX_FP4, FAKE, FAKE, 256, 256, h, FAKE, MIX_F32, 256, NULL, 0, NULL);
    EXPECT_TRUE(st != MIX_OK);
    st = mix_mx_gemm_eq6(MIX_4P5, FAKE, FAKE, MX_INT4, FAKE, FAKE, 256, 256, h, FAKE, MIX_F32, 256, NULL);
    EXPECT_TRUE(st != MIX_OK);
    st = mix_mx_gemm_images(MX_FP4, FAKE, FAKE, NULL, h, 256, 128, FAKE, MIX_BF16, 256, NULL);
    EXPECT_TRUE(st != MIX_OK);
    st = mix_mx_gemm_images(MX_FP4, FAKE, FAKE, NULL, 256, 256, h, FAKE, MIX_BF16, 256, NULL);
    EXPECT_TRUE(st != MIX_OK);
    st = mix_mx_gemm_images_quantize(MX_FP4, FAKE, FAKE, NULL, 64, h, 128, NULL, 0, FAKE, FAKE, NULL, 0, NULL);
    EXPECT_TRUE(st != MIX_OK);
    st = mix_gemm_a_image(MIX_4P5, FAKE, FAKE, h, 128, FAKE, 1 << 20, NULL);
    EXPECT_TRUE(st != MIX_OK);
    st = mx_gemm_b_image(MX_FP4, FAKE, FAKE, h, 128, FAKE, 1 << 20, NULL);
    EXPECT_TRUE(st != MIX_OK);
    st = mx_gemm_b_image_g16(MX_INT4_G16, FAKE, FAKE, 256, h, FAKE, 1 << 20, FAKE, NULL);
    EXPECT_TRUE(st != MIX_OK);
  }
}

static void attention(void) {
  EXPECT(mix_kmean(FAKE, MIX_BF16, 0, 32, 32, FAKE, NULL), MIX_E_SHAPE);
  EXPECT(mix_kmean(MIS1, MIX_BF16, 4, 32, 32, FAKE, NULL), MIX_E_ALIGN);
  EXPECT(mix_underflow_map(FAKE, MIX_F32, (int64_t)1 << 31, 32, 32, NULL, FAKE, FAKE, FAKE, 1 << 30, NULL), MIX_E_SHAPE);
  EXPECT(mix_underflow_map(FAKE, MIX_F32, 4, 32, 32, NULL, MIS2, FAKE, FAKE, 1 << 30, NULL), MIX_E_ALIGN);
  EXPECT(mix_attn_prefill(FAKE, FAKE, FAKE, 100, 28, 3, 128, 1, FAKE, FAKE, FAKE, 1 << 30, NULL, NULL), MIX_E_SHAPE);
  EXPECT(mix_attn_prefill(NULL, FAKE, FAKE, 100, 28, 4, 128, 1, FAKE, FAKE, FAKE, 1 << 30, NULL, NULL), MIX_E_NULL);
  mix_kv_cache_t c = {FAKE, FAKE, FAKE, FAKE, FAKE, 16, 8192, 4, 128};
  const size_t W = (size_t)1 << 30;
  EXPECT(mix_kv_cache_prefill(&c, 16, FAKE, FAKE, 100, FAKE, NULL), MIX_E_SHAPE);
  EXPECT(mix_kv_cache_prefill(&c, 0, FAKE, FAKE, 8193, FAKE, NULL), MIX_E_SHAPE);
  EXPECT(mix_attn_decode(FAKE, FAKE, FAKE, &c, FAKE, 8191, 30, FAKE, FAKE, FAKE, W, NULL, NULL), MIX_E_SHAPE);
  EXPECT(mix_attn_decode(FAKE, FAKE, FAKE, &c, FAKE, 8192, 28, FAKE, FAKE, FAKE, W, NULL, NULL), MIX_E_SHAPE);
  EXPECT(mix_attn_decode(FAKE, FAKE, FAKE, &c, FAKE, 8191, 28, FAKE, MIS4, FAKE, W, NULL, NULL), MIX_E_ALIGN);
  EXPECT(mix_attn_decode(FAKE, FAKE, FAKE, NULL, FAKE, 8191, 28, FAKE, FAKE, FAKE, W, NULL, NULL), MIX_E_NULL);
  const size_t need = mix_decode_step_workspace_bytes(16, 3584, 28, 4, 128, 8191);
  EXPECT(mix_decode_step(FAKE, 3584, 18944, MX_FP4, FAKE, FAKE, FAKE, FAKE, FAKE, &c, FAKE, 8191, 28, FAKE, FAKE, FAKE,
                         need - 1, NULL),
         MIX_E_WORKSPACE);
  mix_kv_cache_t big = c;
  big.B = 17;
  EXPECT(mix_decode_step(FAKE, 3584, 18944, MX_FP4, FAKE, FAKE, FAKE, FAKE, FAKE, &big, FAKE, 8191, 28, FAKE, FAKE, FAKE,
                         W, NULL),
         MIX_E_UNSUPPORTED);
  /* the allocation-free step refuses shapes beyond its fixed array before touching the device */
  mix_kv_cache_t longc = c;
  longc.Lmax = 65536;
  EXPECT(mix_decode_step_static(FAKE, 3584, 18944, MX_FP4, FAKE, FAKE, FAKE, FAKE, FAKE, &longc, FAKE, 65535, 28, FAKE,
                                FAKE, NULL),
         MIX_E_WORKSPACE);
  EXPECT_TRUE(mix_decode_step_static_max_bytes() == (size_t)32 << 20);
  for (int i = 0; i < NHUGE; i++) {
    const int64_t h = HUGE_EXT[i];
    (void)mix_attn_prefill_workspace_bytes(h, 28, 4, 128);
    (void)mix_attn_prefill_workspace_bytes(4096, h, 4, 128);
    (void)mix_attn_prefill_workspace_bytes(4096, 28, h, 128);
    (void)mix_attn_prefill_workspace_bytes(4096, 28, 4, h);
    (void)mix_attn_decode_workspace_bytes(h, 28, 4, 128, 8191);
    (void)mix_attn_decode_workspace_bytes(16, h, 4, 128, 8191);
    (void)mix_attn_decode_workspace_bytes(16, 28, 4, 128, h);
    (void)mix_decode_step_workspace_bytes(16, h, 28, 4, 128, 8191);
    (void)mix_underflow_map_workspace_bytes(h, 512);
    (void)mix_underflow_map_workspace_bytes(4096, h);
    int st = mix_attn_prefill(FAKE, FAKE, FAKE, h, 28, 4, 128, 1, FAKE, FAKE, FAKE, W, NULL, NULL);
    EXPECT_TRUE(st != MIX_OK || h == 0);
    st = mix_kmean(FAKE, MIX_BF16, h, 512, 512, FAKE, NULL);
    EXPECT_TRUE(st != MIX_OK);
    st = mix_underflow_map(FAKE, MIX_F32, h, 32, 32, NULL, FAKE, FAKE, FAKE, W, NULL);
    EXPECT_TRUE(st != MIX_OK);
    mix_kv_cache_t hc = c;
    hc.Lmax = h;
    st = mix_attn_decode(FAKE, FAKE, FAKE, &hc, FAKE, 8191, 28, FAKE, FAKE, FAKE, W, NULL, NULL);
    EXPECT_TRUE(st != MIX_OK);
    hc = c;
    hc.B = h;
    st = mix_attn_decode(FAKE, FAKE, FAKE, &hc, FAKE, 8191, 28, FAKE, FAKE, FAKE, W, NULL, NULL);
    EXPECT_TRUE(st != MIX_OK);
    st = mix_decode_step(FAKE, h, 18944, MX_FP4, FAKE, FAKE, FAKE, FAKE, FAKE, &c, FAKE, 8191, 28, FAKE, FAKE, FAKE, W,
                         NULL);
    EXPECT_TRUE(st != MIX_OK);
    st = mix_decode_step_static(FAKE, 3584, h, MX_FP4, FAKE, FAKE, FAKE, FAKE, FAKE, &c, FAKE, 8191, 28, FAKE, FAKE,
                                NULL);
    EXPECT_TRUE(st != MIX_OK);
  }
}

int main(void) {
  EXPECT_TRUE(mix_abi_version() == MIX_ABI_VERSION);
  for (int s = 0; s < 9; s++) EXPECT_TRUE(mix_status_str((mix_status_t)s) != NULL);
  quantizers();
  gemm();
  attention();
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("all host checks passed\n");
  return 0;
}
