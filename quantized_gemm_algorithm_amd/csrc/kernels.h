// Host-side launchers of the MiX HIP kernels (internal to the library; the public C-ABI is
// include/mixlib.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mixlib.h"

namespace mix {

hipError_t launch_mix_quantize(int fmt, const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                               uint8_t* codes, void* shared, hipStream_t s);
hipError_t launch_mx_quantize(int fp4, const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                              const float* mu, uint8_t* codes, uint8_t* scales, hipStream_t s, int g16 = 0);
hipError_t launch_mx_quantize_cols(const void* x, int dtype, int64_t rows, int64_t prows, int64_t cols, int64_t ldx,
                                   uint8_t* codes, uint8_t* scales, int64_t cpitch, int64_t spitch, hipStream_t s);
hipError_t launch_mix_dequantize(int fmt, const uint8_t* codes, const void* shared, int64_t rows, int64_t cols,
                                 float* out, hipStream_t s);
hipError_t launch_mx_dequantize(int fp4, const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                                float* out, hipStream_t s, int g16 = 0);
hipError_t launch_kmean(const void* x, int dtype, int64_t T, int64_t C, int64_t ldx, float* mu, hipStream_t s);
// the K-mean in two launches through a workspace of kmean_ws_bytes(T, C) bytes (8-byte aligned)
size_t kmean_ws_bytes(int64_t T, int64_t C);
hipError_t launch_kmean_ws(const void* x, int dtype, int64_t T, int64_t C, int64_t ldx, float* mu, void* ws,
                           hipStream_t s);
// its second launch alone (the pairs of the first are in part)
hipError_t launch_kmean_fin(const void* part, int64_t T, int64_t C, float* mu, hipStream_t s);

// The prefill attention's independent operand passes in one launch (bf16 inputs, rows 16-byte
// aligned): V along tokens as MXFP4, the K-mean's row-slice pairs (finished by launch_kmean_fin)
// and Q as MiX-4.5b. The launcher fills the role counts (nvx .. nq).
struct PrefillOperandArgs {
  const uint16_t* q; int64_t cq, ldq; uint8_t* qc; uint16_t* qs;             // Q [T, cq]
  const uint16_t* v; int64_t cv, ldv; uint8_t* vc; uint8_t* vs; int64_t cpitch, spitch;   // V [T, cv]
  const uint16_t* k; int64_t ck, ldk; double2* part;                          // K [T, ck]
  int64_t T, Tp;
  int64_t nvx, nv, nkx, nk, nq;
};
hipError_t launch_prefill_operands(const PrefillOperandArgs& a, hipStream_t s);
// underflow.hip: counts [7][cols] (MXINT4, MXFP4 floor, MXFP4 ceil, NVFP4 B=32, MiX-4.25b, MiX-4.5b, nonzero)
struct UfPlan {
  int64_t cb, rpw, gy, ablocks;   // 32-column blocks, rows per workgroup, workgroup rows, amax workgroups
  size_t part_off, bytes;         // offset of the count partials in the workspace, workspace size
};
UfPlan uf_plan(int64_t rows, int64_t cols);
hipError_t launch_underflow_map(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, const float* mu,
                                uint32_t* counts, float* amax, void* ws, hipStream_t s);

// Operands of the block-scaled product C = deq(A) . deq(B)^T, optionally batched.
struct GemmArgs {
  const uint8_t* a_codes;   // MiX codes, rows of K/2 bytes
  const void* a_shared;     // MiX shared fields (u8 for 4.25b, u16 for 4.5b), rows of K/32
  int64_t a_pitch;          // bytes between consecutive rows of A codes
  int64_t a_sh_pitch;       // elements between consecutive rows of A shared fields
  int64_t a_bstride;        // bytes between batches of A codes
  int64_t a_sh_bstride;     // elements between batches of A shared fields
  const uint8_t* b_codes;   // MX codes, rows of K/2 bytes
  const uint8_t* b_scales;  // E8M0 scales, rows of K/32 bytes
  int64_t b_pitch, b_sc_pitch, b_bstride, b_sc_bstride;
  int b_group;              // batch b uses B batch b / b_group (grouped-query attention)
  void* c;                  // output, fp32 or bf16
  int64_t ldc;              // elements between rows of C
  int64_t c_bstride;        // elements between batches of C
  const float* row_div;     // optional: row m of C is divided by row_div[m] before rounding
  int64_t row_div_bstride;
  int M, N, K, batch;
  int causal;               // 0 none; 1 skip tiles strictly above the diagonal; 2 stop K at the tile's last row
  int b_g16;                // B scales per 16 elements (rows of K/16; Eq. (6) path only)
};

hipError_t launch_gemm_mfma(int a_fmt, int b_fp4, int c_bf16, const GemmArgs& g, hipStream_t s);
hipError_t launch_gemm_eq6(int a_fmt, int b_fp4, int c_bf16, const GemmArgs& g, hipStream_t s);

// fast path: decode pass into a workspace, then the MXFP8 x MX GEMM
bool gemm_f8_eligible(int64_t M, int64_t N, int64_t K);
bool gemm_f8_offsets_ok(int64_t M, int64_t N, int64_t K);
size_t gemm_f8_ws_bytes(int b_fp4, int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_f8(int a_fmt, int b_fp4, int c_bf16, const uint8_t* a_codes, const void* a_shared,
                          const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* c,
                          int64_t ldc, void* ws, hipStream_t s);
hipError_t launch_gemm_a_image(int a_fmt, const uint8_t* a_codes, const void* a_shared, int64_t M, int64_t K,
                               void* img, hipStream_t s);
hipError_t launch_gemm_b_image(int b_fp4, const uint8_t* b_codes, const uint8_t* b_scales, int64_t N, int64_t K,
                               void* img, hipStream_t s);
// the B image of g16 weights (one E8M0 per 16 elements): an E4M3 image (the MXINT4 layout) whose
// per-32 scale is folded from the two halves' exponents; 32-element blocks that cannot be folded
// exactly are counted into *unfoldable (device, zeroed first)
hipError_t launch_gemm_b_image_g16(int fp4, const uint8_t* b_codes, const uint8_t* b_scales16, int64_t N, int64_t K,
                                   void* img, uint32_t* unfoldable, hipStream_t s);
hipError_t launch_gemm_images(int b_fp4, int c_bf16, const void* a_img, const void* b_img, int64_t M, int64_t N,
                              int64_t K, void* c, int64_t ldc, hipStream_t s);
hipError_t launch_mix_quantize_img(int fmt, const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                                   uint8_t* codes, void* shared, void* img, hipStream_t s);
hipError_t launch_gemm_images_q(int b_fp4, const void* a_img, const void* b_img, int64_t M, int64_t N, int64_t K,
                                void* c, int64_t ldc, uint8_t* q_codes, void* q_shared, void* q_img, hipStream_t s);

// attention (arguments validated by the C-ABI layer)
size_t attn_prefill_ws_bytes(int64_t T, int64_t Hq, int64_t Hkv, int64_t d);
hipError_t attn_prefill_run(const void* q, const void* k, const void* v, int64_t T, int64_t Hq, int64_t Hkv,
                            int64_t d, int causal, float* mu, void* o, void* ws, const mix_attn_debug_t* dbg,
                            hipStream_t s);
hipError_t kv_cache_prefill_run(const mix_kv_cache_t* c, int64_t b, const void* k, const void* v, int64_t T,
                                const float* mu, hipStream_t s);
size_t attn_decode_ws_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t max_pos);
// the full decode step: the linear x [B, K] -> y [B, N] (bf16, weights as a B image) and the attention
// step, in the same two launches
size_t decode_step_ws_bytes(int64_t B, int64_t K, int64_t Hq, int64_t Hkv, int64_t d, int64_t max_pos);
hipError_t decode_step_run(const void* x, int64_t K, int64_t N, int b_fp4, const void* b_img, void* y, const void* q,
                           const void* k_new, const void* v_new, const mix_kv_cache_t* c, const int32_t* pos,
                           int64_t max_pos, int64_t Hq, const float* mu, void* o, void* ws, hipStream_t s);
// the same step in one cooperative launch (grid-wide barriers where the launch boundaries stood)
hipError_t decode_step_single_run(const void* x, int64_t K, int64_t N, int b_fp4, const void* b_img, void* y,
                                  const void* q, const void* k_new, const void* v_new, const mix_kv_cache_t* c,
                                  const int32_t* pos, int64_t max_pos, int64_t Hq, const float* mu, void* o, void* ws,
                                  hipStream_t s);
// the same with the workspace in a file-scope device array of DECODE_SCRATCH_BYTES (no allocation)
constexpr size_t DECODE_SCRATCH_BYTES = (size_t)32 << 20;
hipError_t decode_step_static_run(const void* x, int64_t K, int64_t N, int b_fp4, const void* b_img, void* y,
                                  const void* q, const void* k_new, const void* v_new, const mix_kv_cache_t* c,
                                  const int32_t* pos, int64_t max_pos, int64_t Hq, const float* mu, void* o,
                                  hipStream_t s);
hipError_t attn_decode_run(const void* q, const void* k_new, const void* v_new, const mix_kv_cache_t* c,
                           const int32_t* pos, int64_t max_pos, int64_t Hq, const float* mu, void* o, void* ws,
                           const mix_attn_debug_t* dbg, hipStream_t s);

}  // namespace mix
