/*
 * mixlib -- MiX (Micro-Inverted-Scaling) quantizers, the A-MiX x W-MX matrix product and
 * K-smoothed attention on AMD Instinct MI355X (gfx950).
 *
 * Sources. "P1" is the pchao.org digest of the paper, titled
 * "MiX：面向端到端低比特视觉语言模型加速的微反缩放"; each declaration below names the section,
 * figure or equation of P1 that defines the operation.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Memory: every buffer argument is DEVICE memory owned by the caller, except where a comment
 *   says "host". The library never allocates, frees or synchronises; it enqueues kernels on
 *   `stream` (a hipStream_t; NULL is the null stream) and returns.
 * - Validation happens on the host before any HIP call; on failure nothing is enqueued, a status
 *   code is returned and mix_last_error() (per thread) describes the problem.
 * - Shapes: `rows`/`cols`/M/N/K are element counts. Every block axis (MiX and MX blocks hold 32
 *   elements) must be a multiple of 32. A zero extent is a valid empty call (MIX_OK, nothing is
 *   read or written, pointers may be NULL). Negative extents are MIX_E_SHAPE.
 * - Alignment: element pointers and row pitches of fp32/bf16 inputs must be 16-byte aligned
 *   (MIX_E_ALIGN); code/scale buffers must be 16-byte aligned.
 * - Inputs must be finite. A non-finite input gives unspecified codes (no error is raised).
 * - Device faults surface at the caller's next synchronisation as HIP errors.
 *
 * Data formats (P1, 方法概览 / method overview, format bullets; Fig. 4 in 逐图理解论文)
 * -----------------------------------------------------------------------------------
 * MiX codes: one nibble per element, element 2j in the low nibble of byte j; nibble =
 *   (sign << 3) | dE, value (-1)^s (1 + m/8) 2^(Emax - dE); nibble 0x7 is zero and nibble 0xF is
 *   +(1 + m/8) 2^(Emax - 7) (the reclaimed negative zero).
 * MiX shared field per 32-element block: MIX_4P25 -> uint8, bits 3:0 = Emax + 7, bits 6:4 = m.
 *   MIX_4P5 -> uint16, bits 3:0 = Emax + 7, then m0..m3 (one per 8-element sub-block) in bits
 *   6:4, 9:7, 12:10, 15:13.
 * MX codes: same nibble order; MX_FP4 nibbles are OCP E2M1, MX_INT4 nibbles are two's-complement
 *   q with value q 2^(X - 2). MX scale per block: uint8 E8M0 = X + 127 (0 for an all-zero block).
 */
#ifndef MIXLIB_H
#define MIXLIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MIX_ABI_VERSION 4

typedef enum {
  MIX_OK = 0,
  MIX_E_NULL = 1,        /* a required pointer is NULL */
  MIX_E_SHAPE = 2,       /* negative extent, block axis not a multiple of 32, pitch < row length, ... */
  MIX_E_ALIGN = 3,       /* pointer or pitch not 16-byte aligned */
  MIX_E_ENUM = 4,        /* unknown format / dtype value */
  MIX_E_UNSUPPORTED = 5, /* a valid but unimplemented combination */
  MIX_E_HIP = 6,         /* a HIP call failed (launch error); see mix_last_error() */
  MIX_E_WORKSPACE = 7    /* workspace smaller than the size the matching *_workspace_bytes returned */
} mix_status_t;

typedef enum { MIX_4P25 = 0, MIX_4P5 = 1 } mix_fmt_t; /* MiX-4.25b, MiX-4.5b */
/* MXINT4 (floor exponent), MXFP4 (ceil exponent), one E8M0 per 32 elements; the g16 variants share
 * one E8M0 per 16 elements (the 4.5-bit weight tier; scales are then [rows, cols/16]) */
typedef enum { MX_INT4 = 0, MX_FP4 = 1, MX_INT4_G16 = 2, MX_FP4_G16 = 3 } mx_fmt_t;
typedef enum { MIX_F32 = 0, MIX_BF16 = 1 } mix_dtype_t;

/* ABI version compiled into the library (MIX_ABI_VERSION). */
int mix_abi_version(void);
/* Static text for a status code. */
const char* mix_status_str(mix_status_t status);
/* Description of the last error on the calling thread ("" if none). The pointer stays valid until
 * the next library call on this thread. */
const char* mix_last_error(void);

/*
 * MiX activation quantizer -- P1, method overview, the Algorithm 1 bullet.
 * Per 32-element block along each row: Emax = clamp(floor(log2 max|x|), -7, 8); the shared
 * mantissa m = the top three fraction bits of the largest element's significand (of the block for
 * MIX_4P25, of each 8-element sub-block for MIX_4P5); each element takes the nearest
 * representable value (the naive dE = Emax - floor(log2|x|) refined by +-1), ties to the smaller
 * magnitude. An all-zero block has shared field 0 and nibbles 0x7.
 *   x       [rows, cols] fp32 or bf16 (dtype), row pitch ldx elements (ldx >= cols)
 *   codes   [rows, cols/2] uint8, dense
 *   shared  [rows, cols/32] uint8 (MIX_4P25) or uint16 (MIX_4P5), dense
 */
mix_status_t mix_quantize(mix_fmt_t fmt, const void* x, mix_dtype_t dtype, int64_t rows, int64_t cols, int64_t ldx,
                          uint8_t* codes, void* shared, void* stream);

/*
 * MX weight quantizer -- P1, figure walk (Fig. 4: shared 8-bit exponent, 4-bit element) and key
 * results (the MXFP4 bullet: the shared exponent uses ceil instead of OCP's floor).
 * MX_FP4: X = ceil(log2 max|x|) - 2 (>= -127); elements x 2^-X rounded to nearest-even on the
 *   E2M1 grid, sign of zero kept. MX_INT4: X = clamp(floor(log2 max|x|), -125, 127);
 *   q = clamp(RNE(x 2^(2-X)), -7, 7).
 * If mu != NULL the operand is fp32(x - mu[col]) (K-smoothing, P1 method overview last bullet).
 * MX_INT4_G16 / MX_FP4_G16 (P1 实验如何设计 (experiment design), the format bullet: the 4.5-bit g16 weights)
 * apply the same rules to blocks of 16 elements.
 *   x       [rows, cols] fp32 or bf16, row pitch ldx
 *   mu      NULL or [cols] fp32
 *   codes   [rows, cols/2] uint8; scales [rows, cols/32] uint8 (E8M0), [rows, cols/16] for g16
 */
mix_status_t mx_quantize(mx_fmt_t fmt, const void* x, mix_dtype_t dtype, int64_t rows, int64_t cols, int64_t ldx,
                         const float* mu, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * MXFP4 (the ceil rule of mx_quantize) with blocks running down the columns -- P1, 核心创新
 * (innovations), third bullet: the attention products, the KV cache included, are coded too. In
 * P^ V the contraction runs along tokens, so V is the MX operand of that product with its blocks
 * along tokens (one block per 32 tokens of a channel). Block j of column c covers rows
 * [32 j, 32 j + 32); rows at or beyond `rows` count as zero.
 *   x       [rows, cols] fp32 or bf16, row pitch ldx elements (ldx >= cols), element-aligned
 *   codes   [cols, prows/2] uint8, 16-byte aligned; scales [cols, prows/32] E8M0, where
 *           prows = rows rounded up to 32 (the output is written transposed: one row per column)
 * Errors: MIX_E_SHAPE for negative extents, ldx < cols or prows / 32 > 65535; MIX_E_NULL,
 * MIX_E_ALIGN as above. Empty input: MIX_OK, nothing written.
 */
mix_status_t mx_quantize_cols(const void* x, mix_dtype_t dtype, int64_t rows, int64_t cols, int64_t ldx,
                              uint8_t* codes, uint8_t* scales, void* stream);

/* Decoders (closed forms above) to fp32 [rows, cols]; for tests and inspection. */
mix_status_t mix_dequantize(mix_fmt_t fmt, const uint8_t* codes, const void* shared, int64_t rows, int64_t cols,
                            float* out, void* stream);
mix_status_t mx_dequantize(mx_fmt_t fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                           float* out, void* stream);

/*
 * A-MiX x W-MX product -- P1, method overview, the dual-format bullet and Eq. (6).
 * C = deq(A) . deq(B)^T with fp32 accumulation; fp32 output is the accumulator, bf16 output its
 * round-to-nearest-even. Runs on the gfx950 block-scaled MFMA (E4M3 A x E2M1/E4M3 B with per-32
 * power-of-two scales; every product is exact).
 *   A: a_codes [M, K/2], a_shared [M, K/32] (uint8 or uint16 by a_fmt)
 *   B: b_codes [N, K/2], b_scales [N, K/32]   (B holds W^T: one row per output column)
 *   c  [M, N] fp32 or bf16 (c_dtype), row pitch ldc elements (ldc >= N)
 *   ws, ws_bytes: optional workspace (see mix_mx_gemm_workspace_bytes); NULL is allowed
 * g16 weights: MIX_E_UNSUPPORTED (mx_gemm_b_image_g16 + mix_mx_gemm_images, or mix_mx_gemm_eq6).
 */
mix_status_t mix_mx_gemm(mix_fmt_t a_fmt, const uint8_t* a_codes, const void* a_shared, mx_fmt_t b_fmt,
                         const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* c,
                         mix_dtype_t c_dtype, int64_t ldc, void* ws, size_t ws_bytes, void* stream);

/*
 * Workspace for mix_mx_gemm's fast path: the MiX codes of A decoded once into E4M3 bytes plus E8M0
 * scales (and MXINT4 weights into E4M3 bytes), so the MFMA loop streams operands without decoding.
 * Returns 0 when the shape does not take the fast path (K % 128 != 0, M < 64 or N < 256). With
 * ws == NULL or ws_bytes below this size mix_mx_gemm decodes inside the GEMM instead (same results).
 * ws must be 256-byte aligned; its contents are scratch (overwritten by each call).
 */
size_t mix_mx_gemm_workspace_bytes(mix_fmt_t a_fmt, mx_fmt_t b_fmt, int64_t M, int64_t N, int64_t K);

/*
 * GEMM operand images: the decode-once form mix_mx_gemm's fast path streams, exposed so that a
 * weight's image is built once and an activation's image comes straight out of the quantizer.
 * The values are exactly those of the codes (same product as mix_mx_gemm, P1 method overview,
 * dual-format bullet and Eq. (6)): a MiX element (1.m)_2 2^(Emax - dE) is stored as the E4M3
 * byte of (1.m)_2 2^(1 - dE) under the E8M0 block scale 2^(Emax - 1); an MXINT4 element
 * q 2^(X - 2) as the E4M3 byte of q/4 under its unchanged scale 2^X; MXFP4 codes are the E2M1
 * operand, copied step-major (each 128-wide K step's 64-byte row slices contiguous over the rows).
 * Images are opaque byte buffers of the sizes below (0 = no image for that shape: K must be a
 * positive multiple of 128), 256-byte aligned, owned by the caller. An image depends only on the
 * operand's codes and shape (not on the other operand).
 */
size_t mix_gemm_a_image_bytes(int64_t M, int64_t K);
size_t mx_gemm_b_image_bytes(mx_fmt_t b_fmt, int64_t N, int64_t K);

/*
 * A image from MiX codes -- P1, 方法概览 (method overview), the dual-format bullet: the MiX
 * activation's shared mantissa factors out of the block dot product, which leaves a per-element
 * power of two (the E4M3 byte) under a per-block power of two (the E8M0 scale).
 *   a_codes [M, K/2] uint8 (16-byte aligned), a_shared [M, K/32] uint8 / uint16 by a_fmt
 *   img     mix_gemm_a_image_bytes(M, K) bytes at least (MIX_E_WORKSPACE below), 256-byte aligned
 * Errors: MIX_E_SHAPE unless K is a positive multiple of 128 (M <= 2^31 - 1); MIX_E_NULL,
 * MIX_E_ALIGN, MIX_E_ENUM. M == 0: MIX_OK, nothing written.
 */
mix_status_t mix_gemm_a_image(mix_fmt_t a_fmt, const uint8_t* a_codes, const void* a_shared, int64_t M, int64_t K,
                              void* img, size_t img_bytes, void* stream);

/*
 * mix_quantize that also writes the A image of the quantized rows in the same pass (rows = M,
 * cols = K) -- P1, 方法概览 (method overview): the Algorithm 1 bullet (the quantizer) and the
 * dual-format bullet (the operand the product consumes). codes and shared may both be NULL: then
 * only the image is written. The image equals mix_gemm_a_image of the codes mix_quantize produces.
 *   x, dtype, rows, cols, ldx, codes, shared  as for mix_quantize (cols a positive multiple of 128)
 *   img     mix_gemm_a_image_bytes(rows, cols) bytes at least, 256-byte aligned
 * Errors: as for mix_quantize and mix_gemm_a_image; MIX_E_NULL if exactly one of codes / shared
 * is NULL.
 */
mix_status_t mix_quantize_gemm(mix_fmt_t fmt, const void* x, mix_dtype_t dtype, int64_t rows, int64_t cols,
                               int64_t ldx, uint8_t* codes, void* shared, void* img, size_t img_bytes, void* stream);

/*
 * B image from MX codes -- P1, 方法概览 (method overview), the dual-format bullet (W-MX weights),
 * and 逐图理解论文 (figure walk), Fig. 4 (the MXINT4 / MXFP4 fields): MXINT4 elements become E4M3
 * bytes of q/4 under their unchanged scale, MXFP4 codes are copied step-major.
 *   b_codes [N, K/2] uint8, 16-byte aligned; b_scales [N, K/32] E8M0
 *   img     mx_gemm_b_image_bytes(b_fmt, N, K) bytes at least, 256-byte aligned
 * Errors: MIX_E_UNSUPPORTED for the g16 formats (use mx_gemm_b_image_g16); MIX_E_SHAPE unless K
 * is a positive multiple of 128; MIX_E_NULL, MIX_E_ALIGN, MIX_E_WORKSPACE (image too small).
 * N == 0: MIX_OK, nothing written.
 */
mix_status_t mx_gemm_b_image(mx_fmt_t b_fmt, const uint8_t* b_codes, const uint8_t* b_scales, int64_t N, int64_t K,
                             void* img, size_t img_bytes, void* stream);

/*
 * B image of g16 weights (MX_INT4_G16 / MX_FP4_G16; P1 实验如何设计 (experiment design), the 4.5-bit g16
 * variants; MiX-INT4g16 = MiX-4.5b activations x MXINT4g16 weights). The matrix core takes one
 * scale per 32 K elements, so each 32-block's two 16-element exponents are folded into E4M3
 * element bytes over one shared scale (MXINT4g16: the smaller exponent; MXFP4g16: the larger),
 * exact when the two exponents differ by at most 8. The number of 32-blocks that could not be
 * folded exactly is written to *unfoldable (device memory, set by this call on the stream); the
 * products from this image equal the exact ones when it is 0 (mix_mx_gemm_eq6 is exact for every
 * input). The image has mx_gemm_b_image_bytes(b_fmt, N, K) bytes (the MX_INT4 layout).
 *   b_codes [N, K/2] uint8 (16-byte aligned); b_scales16 [N, K/16] E8M0; K a multiple of 128
 *   unfoldable  uint32 in device memory, 4-byte aligned
 */
mix_status_t mx_gemm_b_image_g16(mx_fmt_t b_fmt, const uint8_t* b_codes, const uint8_t* b_scales16, int64_t N,
                                 int64_t K, void* img, size_t img_bytes, uint32_t* unfoldable, void* stream);

/*
 * C = A . B^T from the two images -- P1, 方法概览 (method overview), the dual-format bullet and
 * Eq. (6): the same exact products and fp32 sums as mix_mx_gemm on the codes (bit-identical
 * results). The images hold every operand byte: b_codes is not read and may be NULL (kept for the
 * signature). M <= 16 runs the weight stream (each weight byte read once), larger M the tiled
 * product.
 *   a_img, b_img  images of an [M, K] and an [N, K] operand, 256-byte aligned
 *   c      [M, N] fp32 or bf16 (c_dtype), row pitch ldc >= N elements, element-aligned
 * Errors: MIX_E_SHAPE unless K is a positive multiple of 128 (M, N <= 2^31 - 1) or if ldc < N;
 * MIX_E_UNSUPPORTED for M > 16 when an operand image reaches 2^31 bytes (mix_mx_gemm then decodes
 * inside the GEMM instead); MIX_E_NULL, MIX_E_ALIGN, MIX_E_ENUM. M or N == 0: MIX_OK.
 */
mix_status_t mix_mx_gemm_images(mx_fmt_t b_fmt, const void* a_img, const void* b_img, const uint8_t* b_codes,
                                int64_t M, int64_t N, int64_t K, void* c, mix_dtype_t c_dtype, int64_t ldc,
                                void* stream);

/*
 * The product of the two images with its output quantized in the same pass -- the pages' output
 * quantizer at the array output (P1 method overview; the fused quantizer): q_codes [M, N/2] and
 * q_shared [M, N/32] (u16) are the MiX-4.5b coding along N of the bf16 rounding of C, exactly what
 * mix_quantize would give for that bf16 matrix; q_img (optional, NULL to skip; needs N a multiple
 * of 128 and q_img_bytes >= mix_gemm_a_image_bytes(M, N)) receives the A image of those codes for
 * a next product with K = N. C itself (bf16, pitch ldc) is written only if c is not NULL; for
 * M <= 16 c is required (the weight stream writes C, then the quantizer reads it) and must be
 * 16-byte aligned with a 16-byte row pitch. N must be a multiple of 32; other arguments as for
 * mix_mx_gemm_images.
 */
mix_status_t mix_mx_gemm_images_quantize(mx_fmt_t b_fmt, const void* a_img, const void* b_img, const uint8_t* b_codes,
                                         int64_t M, int64_t N, int64_t K, void* c, int64_t ldc, uint8_t* q_codes,
                                         void* q_shared, void* q_img, size_t q_img_bytes, void* stream);

/*
 * The same product computed as P1's Eq. (6) on the vector ALUs: integer sub-block sums of the MX
 * mantissas scaled by 2^(7 - dE), times (8 + m_k), one power-of-two scale per block, fp32
 * accumulation across blocks. Same arguments and results (to fp32 rounding) as mix_mx_gemm. For the
 * g16 formats (b_scales [N, K/16]) each block's sum is split by weight half, one power-of-two
 * scale per half: exact for every input.
 */
mix_status_t mix_mx_gemm_eq6(mix_fmt_t a_fmt, const uint8_t* a_codes, const void* a_shared, mx_fmt_t b_fmt,
                             const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N, int64_t K,
                             void* c, mix_dtype_t c_dtype, int64_t ldc, void* stream);

/*
 * Per-channel mean of the keys -- P1, method overview, last bullet (K-smoothing with the prefill
 * mean frozen for decode). mu[c] = fp32(exact_sum_t k[t, c] / T), the division in fp64.
 *   k  [T, C] fp32 or bf16 (C = kv_heads * head_dim, a multiple of 32), row pitch ldk; k and the
 *      row pitch in bytes 16-byte aligned
 *   mu [C] fp32
 */
mix_status_t mix_kmean(const void* k, mix_dtype_t dtype, int64_t T, int64_t C, int64_t ldk, float* mu, void* stream);

/*
 * Underflow ("dead zone") map -- P1, figure walk, the underflow-map figure (keys coded with
 * 32-element blocks in MXINT4, MXFP4, NVFP4 with its block forced to 32, and MiX; nonzero elements
 * that decode to zero are mathematical underflow) and the key results' MXFP4 bullet (the OCP floor
 * exponent rule against the ceil rule). A diagnostic: nothing on the product path calls it.
 *   x      [rows, cols] fp32 or bf16, row pitch ldx (cols a multiple of 32; x and the row pitch in
 *          bytes 16-byte aligned); blocks of 32 run along cols
 *   mu     optional fp32 [cols] (16-byte aligned): the map is of fp32(x - mu), the smoothed operand
 *   counts device uint32 [MIX_UF_KINDS][cols], overwritten: counts[k][c] = the elements of column c
 *          that are nonzero on input and that format k codes to zero; counts[MIX_UF_NONZERO][c] =
 *          the nonzero elements of column c
 *   amax   device float [1], overwritten with the largest magnitude of the (smoothed) operand
 *   ws     device workspace of ws_bytes >= mix_underflow_map_workspace_bytes(rows, cols) bytes
 *          (16-byte aligned; caller-owned; its contents on entry do not matter); may be NULL when
 *          that size is 0
 * The formats: MXINT4 and MXFP4 (ceil) as mx_quantize codes them; MXFP4 under the OCP rule
 * X = floor(log2 amax_b) - 2; NVFP4 with a tensor scale g = amax / 2688, block scales the E4M3
 * value nearest to amax_b / (6 g) (ties to the even code) and E2M1 elements (an element is zero iff
 * |x| <= s g / 4); MiX-4.25b and MiX-4.5b as mix_quantize codes them. Every decision is exact.
 * Three launches on the stream (per-workgroup maxima, the map into per-workgroup sums, their
 * sum), no atomics, so the counts do not depend on scheduling; rows <= 2^31 - 1.
 */
typedef enum {
  MIX_UF_MXINT4 = 0,
  MIX_UF_MXFP4_FLOOR = 1,
  MIX_UF_MXFP4_CEIL = 2,
  MIX_UF_NVFP4_B32 = 3,
  MIX_UF_MIX_4_25B = 4,
  MIX_UF_MIX_4_5B = 5,
  MIX_UF_NONZERO = 6,
  MIX_UF_KINDS = 7
} mix_uf_kind_t;
size_t mix_underflow_map_workspace_bytes(int64_t rows, int64_t cols);
mix_status_t mix_underflow_map(const void* x, mix_dtype_t dtype, int64_t rows, int64_t cols, int64_t ldx,
                               const float* mu, uint32_t* counts, float* amax, void* ws, size_t ws_bytes,
                               void* stream);

/* Optional dumps of the attention stages (any pointer may be NULL). Prefill: s and p [Hq, T, Tp]
 * fp32, p_codes [Hq, T, Tp/2], p_shared [Hq, T, Tp/32], l [Hq, T], with Tp = T rounded up to 32.
 * Decode: s and p [B, Hq, Lp], p_codes [B, Hq, Lp/2], p_shared [B, Hq, Lp/32], l [B, Hq], with
 * Lp = max_pos + 1 rounded up to 256. Entries of s above the causal diagonal or past a sequence
 * are not written; p is written where P^ is. */
typedef struct {
  float* s;
  float* p;
  uint8_t* p_codes;
  uint16_t* p_shared;
  float* l;
} mix_attn_debug_t;

/*
 * K-smoothed prefill attention -- P1, method overview (last bullet), innovations (third bullet:
 * the attention products are coded too). Operand formats: Q and P as MiX-4.5b (blocks along the
 * head dimension and along keys), smoothed K and V as MXFP4 (blocks along the head dimension and
 * along tokens).
 *   1. mu = K-mean over the T tokens (written to `mu`, [Hkv, d], for decode)
 *   2. K^ = MXFP4(fp32(K - mu)), Q^ = MiX-4.5b(Q), V^ = MXFP4 along tokens
 *   3. S = Q^ K^T per query head (head h reads KV head h / (Hq / Hkv)), causal if `causal`
 *   4. z = fp32(S) * fp32(1/sqrt(d)); m = row max over unmasked keys; p = exp(z - m);
 *      l = sum of p; P^ = MiX-4.5b(p) along keys
 *   5. O = bf16((P^ V^) / l)
 *   q [T, Hq, d], k/v [T, Hkv, d] bf16, dense;  o [T, Hq, d] bf16;  mu [Hkv, d] fp32 (output)
 *   ws: workspace of at least mix_attn_prefill_workspace_bytes(T, Hq, Hkv, d) bytes, 256-B aligned
 * Requires d % 32 == 0 and Hq % Hkv == 0; T may be ragged.
 */
size_t mix_attn_prefill_workspace_bytes(int64_t T, int64_t Hq, int64_t Hkv, int64_t d);
mix_status_t mix_attn_prefill(const void* q, const void* k, const void* v, int64_t T, int64_t Hq, int64_t Hkv,
                              int64_t d, int causal, float* mu, void* o, void* ws, size_t ws_bytes,
                              const mix_attn_debug_t* dbg, void* stream);

/*
 * MX-coded KV cache for decode (caller-owned device buffers; all dense, head-major):
 *   k_codes  [B, Hkv, Lmax, d/2]   MXFP4 of fp32(k - mu_b) along d
 *   k_scales [B, Hkv, Lmax, d/32]
 *   v_codes  [B, Hkv, d, Lmax/2]   MXFP4 along tokens: block j covers tokens [32 j, 32 j + 32)
 *   v_scales [B, Hkv, d, Lmax/32]
 *   v_stage  [B, 32, Hkv, d] bf16  the tokens of each row's current (possibly partial) V block
 * Lmax % 32 == 0, d % 32 == 0. The block that holds the newest token is always coded from the
 * staged tokens present, the others zero (P1 leaves partial blocks open; see the design notes).
 */
typedef struct {
  uint8_t* k_codes;
  uint8_t* k_scales;
  uint8_t* v_codes;
  uint8_t* v_scales;
  void* v_stage;
  int64_t B, Lmax, Hkv, d;
} mix_kv_cache_t;

/*
 * Fill row b of the cache from a prefill of T tokens (k/v [T, Hkv, d] bf16 dense) with the frozen
 * mean mu [Hkv, d] fp32 (P1 method overview last bullet: the prefill mean is reused, so cached
 * keys are never re-coded). 0 < T <= Lmax.
 */
mix_status_t mix_kv_cache_prefill(const mix_kv_cache_t* cache, int64_t b, const void* k, const void* v, int64_t T,
                                  const float* mu, void* stream);

/*
 * One decode step of the attention -- P1, 方法概览 (method overview), last bullet, and 阅读时需要注意
 * (caveats), first bullet: keys are smoothed with the prefill K-mean frozen for decode, so the
 * cached MXFP4 keys are read once per step and never re-coded; the operand formats and softmax
 * are those of mix_attn_prefill. For B sequences: append k_new/v_new [B, Hkv, d] bf16 at
 * position pos[b] (device int32 [B]), then attend q [B, Hq, d] bf16 over keys [0, pos[b]] with no causal mask,
 * using the frozen mean mu [B, Hkv, d] fp32; o [B, Hq, d] bf16 (8-byte aligned). `max_pos`
 * (host) bounds every pos[b] (0 <= pos[b] <= max_pos < Lmax); rows whose pos is outside
 * [0, max_pos] write zeros to o and leave the cache untouched.
 *   q      [B, Hq, d] bf16 dense, 16-byte aligned; k_new, v_new [B, Hkv, d] bf16 dense
 *   pos    device int32 [B], 4-byte aligned; mu device fp32 [B, Hkv, d], 4-byte aligned
 *   ws: at least mix_attn_decode_workspace_bytes(B, Hq, Hkv, d, max_pos) bytes, 256-B aligned;
 *       scratch (its contents on entry do not matter)
 * Errors: MIX_E_NULL (a pointer or cache buffer), MIX_E_SHAPE (cache extents, Hq not a positive
 * multiple of Hkv, max_pos outside [0, Lmax)), MIX_E_UNSUPPORTED (d != 128 or more than 16 query
 * heads per KV head), MIX_E_ALIGN, MIX_E_WORKSPACE; nothing is enqueued on an error.
 */
size_t mix_attn_decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t max_pos);
mix_status_t mix_attn_decode(const void* q, const void* k_new, const void* v_new, const mix_kv_cache_t* cache,
                             const int32_t* pos, int64_t max_pos, int64_t Hq, const float* mu, void* o, void* ws,
                             size_t ws_bytes, const mix_attn_debug_t* dbg, void* stream);

/*
 * One whole decode step -- P1, 方法概览 (method overview), the dual-format bullet (the linear's
 * MiX-coded activations times its MX-coded weights) and the last bullet with 阅读时需要注意
 * (caveats), first bullet (K-smoothing with the prefill mean frozen, so decode streams the cached
 * keys once and never re-codes them):
 *   y = bf16( deq(MiX-4.5b(x)) . deq(W)^T )   for the linear x [B, K] -> y [B, N], and
 *   the attention step of mix_attn_decode (append k_new / v_new at pos[b], attend q over keys
 *   [0, pos[b]], o [B, Hq, d]).
 * The results equal mix_quantize_gemm(x) + mix_mx_gemm_images (bf16 out) followed by mix_attn_decode
 * with the same arguments; the two parts are independent and share three launches (the first
 * codes x beside the scores, the second streams the weights beside the values, the third adds the
 * per-chunk partial sums of O).
 *   x      [B, K] bf16, dense (B = cache->B <= 16; K a positive multiple of 128), 16-byte aligned
 *   b_fmt, b_img  the weights' B image (mx_gemm_b_image / mx_gemm_b_image_g16 for an [N, K] operand;
 *          g16 images must have no unfoldable block for the product to be exact), 256-byte aligned
 *   y      [B, N] bf16, dense
 *   q, k_new, v_new, cache, pos, max_pos, Hq, mu, o  as for mix_attn_decode (d = 128)
 *   ws     at least mix_decode_step_workspace_bytes(B, K, Hq, Hkv, d, max_pos) bytes, 256-byte
 *          aligned; scratch (its contents on entry do not matter)
 * Errors as for mix_attn_decode and mix_mx_gemm_images; MIX_E_UNSUPPORTED for B > 16.
 */
size_t mix_decode_step_workspace_bytes(int64_t B, int64_t K, int64_t Hq, int64_t Hkv, int64_t d, int64_t max_pos);
mix_status_t mix_decode_step(const void* x, int64_t K, int64_t N, mx_fmt_t b_fmt, const void* b_img, void* y,
                             const void* q, const void* k_new, const void* v_new, const mix_kv_cache_t* cache,
                             const int32_t* pos, int64_t max_pos, int64_t Hq, const float* mu, void* o, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * mix_decode_step in one launch -- the same passages: the exact row maximum that the P^ codes need
 * (the maximum over every cached key, P1 method overview, last bullet) is kept by a grid-wide barrier
 * between the scores and the values, and another before the partial sums of O are added, instead of
 * launch boundaries. Same arguments and workspace as mix_decode_step, and bit-identical results
 * (the same per-chunk work in the same order). The grid is launched cooperatively, sized to the
 * workgroups the device holds at once (the launch admits it only if all of them are resident);
 * MIX_E_HIP if the device cannot launch cooperatively. Not for HIP graph capture.
 */
mix_status_t mix_decode_step_single(const void* x, int64_t K, int64_t N, mx_fmt_t b_fmt, const void* b_img, void* y,
                                    const void* q, const void* k_new, const void* v_new,
                                    const mix_kv_cache_t* cache, const int32_t* pos, int64_t max_pos, int64_t Hq,
                                    const float* mu, void* o, void* ws, size_t ws_bytes, void* stream);

/*
 * mix_decode_step for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same arguments and results without ws and
 * ws_bytes. The workspace is a file-scope device array of mix_decode_step_static_max_bytes() bytes
 * (32 MiB) that the library holds on each device it runs on until the process ends; a shape whose
 * mix_decode_step_workspace_bytes exceeds it returns MIX_E_WORKSPACE. The call allocates nothing and
 * needs no cleared memory. Every call on a device shares that device's array, so calls that overlap
 * on one device (different streams, or host threads) race; serialise them.
 */
size_t mix_decode_step_static_max_bytes(void);
mix_status_t mix_decode_step_static(const void* x, int64_t K, int64_t N, mx_fmt_t b_fmt, const void* b_img, void* y,
                                    const void* q, const void* k_new, const void* v_new,
                                    const mix_kv_cache_t* cache, const int32_t* pos, int64_t max_pos, int64_t Hq,
                                    const float* mu, void* o, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MIXLIB_H */
