// The weight stream of the A-MiX x W-MX product for at most 16 activation rows (decode), as a
// device function that a standalone kernel or the fused decode-step kernel runs per workgroup.
//
// P1 (the pchao.org digest "MiX：面向端到端低比特视觉语言模型加速的微反缩放", 方法概览 / method
// overview, dual-format bullet; 阅读时需要注意 / caveats): at decode the product is bound by reading
// the MX-coded weights once. Every weight byte is loaded straight into registers as an MFMA operand
// fragment (no LDS staging), so the function needs only a small LDS area for the final sum of the
// four waves' partial products and can share a CU with other work.
//
// Work of one workgroup: RG groups of 16 weight rows (16 RG output columns) over all of K. Its four
// waves split each K chunk of up to 32 steps (128 K elements each) into four contiguous ranges; a
// wave keeps the operands of D steps in flight (issued in order, consumed as each step's loads
// land), so a CU holds D * RG KB of weights in flight per wave.
//
// MFMA v_mfma_scale_f32_16x16x128_f8f6f4 with the weight rows as its A operand (lane l = r + 16 g:
// row r, FP4 K elements [32 g, 32 g + 32) in 16 bytes, or E4M3 [16 g, +16) and [64 + 16 g, +16)), the
// activation rows as its B operand (E4M3, the same split) and per-32 E8M0 scales (the weight's from
// the image's per-16-row-group copy, the activation's from the A image). Result register i of lane
// l is C^T[4 (l >> 4) + i][l & 15]: four consecutive output columns of activation row l & 15.
// Every product is exact; the sums are fp32.
#pragma once
#include "common.h"
#include "f8_image.h"

namespace mix {

typedef int gv_v4i __attribute__((ext_vector_type(4)));
typedef int gv_v8i __attribute__((ext_vector_type(8)));
typedef float gv_v4f __attribute__((ext_vector_type(4)));

struct GvOps {
  const uint8_t* a8;     // A image E4M3 [M, K]
  const uint8_t* as_p;   // A image scales [K/128][tiles_m][1024] (row r's four block scales at 4 r)
  const uint8_t* b8;     // B image operand: FP4 step-major [K/128][N][64], or E4M3 [N, K]
  const uint8_t* bs_v;   // B image scales per 16-row group [ceil(N/16)][K/128][16][4]
  void* c;               // C [M, ldc], fp32 or bf16
  int64_t ldc;
  int M, N, K;
  int tiles_m;           // ceil(M / 256) of the A image's scale layout (1 for M <= 16)
};

constexpr int GV_CHUNK = 32;   // K steps per chunk: at most 8 per wave

// LDS bytes gemv_block needs (the partial sums of the four waves)
template <int RG>
constexpr int gv_lds_bytes() { return 4 * RG * 64 * 16; }

template <int RG>
struct GvSlot {
  gv_v8i w[RG];   // weight fragments (FP4: the first four dwords)
  int ws[RG];     // their E8M0 scales
  gv_v8i a;       // activation fragment
  int as;         // its E8M0 scale
};

// raw buffer resource of n bytes at p (gfx9 data-format dword); loads through it take a wave-uniform
// offset in an SGPR and a 32-bit lane offset, and read zero past n bytes
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gv_rsrc(const void* p, int64_t n) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)(n < 0x7FFFFFFF ? n : 0x7FFFFFFF), 0x00020000);
}

// One workgroup of 256 threads: output columns [16 RG wg, 16 RG (wg + 1)) of all M rows.
// `red` is LDS of gv_lds_bytes<RG>() bytes (16-byte aligned).
template <int B_FP4, int C_BF16, int RG, int D>
__device__ __forceinline__ void gemv_block(const GvOps& g, int wg, float* red) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, gq = lane >> 4;
  const int ngrp = (g.N + 15) >> 4;
  const int nkt = g.K / FK;
  const int rowA = min(r, g.M - 1);
  // every load is a buffer load: a wave-uniform per-step offset plus a 32-bit lane offset fixed for
  // the whole loop
  const __amdgpu_buffer_rsrc_t rb = gv_rsrc(g.b8, B_FP4 ? (int64_t)g.N * g.K / 2 : (int64_t)g.N * g.K);
  const __amdgpu_buffer_rsrc_t rbs = gv_rsrc(g.bs_v, (int64_t)ngrp * nkt * 64);
  const __amdgpu_buffer_rsrc_t ra = gv_rsrc(g.a8, (int64_t)g.M * g.K);
  const __amdgpu_buffer_rsrc_t ras = gv_rsrc(g.as_p, (int64_t)nkt * g.tiles_m * 1024);
  int grp[RG];
  uint32_t boff[RG];
#pragma unroll
  for (int j = 0; j < RG; j++) {
    grp[j] = min(wg * RG + j, ngrp - 1);
    const int nrow = min(grp[j] * 16 + r, g.N - 1);   // rows past N repeat row N-1; outputs dropped
    boff[j] = B_FP4 ? (uint32_t)nrow * 64u + 16u * gq : (uint32_t)nrow * (uint32_t)g.K + 16u * gq;
  }
  const uint32_t soff = (uint32_t)(r * 4 + gq);                        // scale byte of (row, block)
  const uint32_t aoff = (uint32_t)rowA * (uint32_t)g.K + 16u * gq;     // activation bytes
  const uint32_t asoff = (uint32_t)(rowA * 4 + gq);
  gv_v4f acc[RG];
#pragma unroll
  for (int j = 0; j < RG; j++) acc[j] = gv_v4f{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](GvSlot<RG>& s, int ks) {
    const int bst = B_FP4 ? ks * g.N * 64 : ks * FK;
#pragma unroll
    for (int j = 0; j < RG; j++) {
      if (B_FP4) {
        const gv_v4i w = __builtin_amdgcn_raw_buffer_load_b128(rb, boff[j], bst, 0);
        s.w[j] = __builtin_shufflevector(w, w, 0, 1, 2, 3, -1, -1, -1, -1);   // FP4 reads dwords 0..3 only
      } else {
        const gv_v4i lo = __builtin_amdgcn_raw_buffer_load_b128(rb, boff[j], bst, 0);
        const gv_v4i hi = __builtin_amdgcn_raw_buffer_load_b128(rb, boff[j] + 64u, bst, 0);
        s.w[j] = gv_v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      s.ws[j] = __builtin_amdgcn_raw_buffer_load_b8(rbs, soff, (grp[j] * nkt + ks) * 64, 0);
    }
    const gv_v4i lo = __builtin_amdgcn_raw_buffer_load_b128(ra, aoff, ks * FK, 0);
    const gv_v4i hi = __builtin_amdgcn_raw_buffer_load_b128(ra, aoff + 64u, ks * FK, 0);
    s.a = gv_v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    s.as = __builtin_amdgcn_raw_buffer_load_b8(ras, asoff, ks * g.tiles_m * 1024, 0);
  };
  auto mma = [&](const GvSlot<RG>& s) {
#pragma unroll
    for (int j = 0; j < RG; j++)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(s.w[j], s.a, acc[j], B_FP4 ? 4 : 0, 0, 0, s.ws[j], 0,
                                                                s.as);
  };

  for (int c0 = 0; c0 < nkt; c0 += GV_CHUNK) {
    const int nks = min(GV_CHUNK, nkt - c0);
    const int spw = (nks + 3) >> 2;
    const int s0 = c0 + wave * spw;
    const int myn = max(0, min(spw, c0 + nks - s0));   // this wave's steps in the chunk
    if (myn == 0) continue;
    const int last = s0 + myn - 1;
    // D slots in flight: slot u holds steps u, u + D, ...; loads past the wave's last step repeat it
    // (cache hits, never used), so every slot is refilled unconditionally and the loads of a step
    // are always the oldest in flight when it is consumed
    GvSlot<RG> sl[D];
#pragma unroll
    for (int u = 0; u < D; u++) issue(sl[u], min(s0 + u, last));
    // straight-line over the chunk's at most GV_CHUNK / 4 steps (a loop would make the compiler's
    // wait placement drain every load at its head)
#pragma unroll
    for (int i = 0; i < GV_CHUNK / 4; i += D) {
      if (i < myn) {
#pragma unroll
        for (int u = 0; u < D; u++) {
          if (i + u < myn) mma(sl[u]);
          issue(sl[u], min(s0 + i + u + D, last));
        }
      }
    }
  }

  // the four waves' partial sums, added in wave order
#pragma unroll
  for (int j = 0; j < RG; j++) *(gv_v4f*)(red + ((wave * RG + j) * 64 + lane) * 4) = acc[j];
  __syncthreads();
  for (int t = threadIdx.x; t < RG * 64; t += 256) {   // RG > 4: some threads sum two groups
    const int j = t >> 6, l = t & 63;
    gv_v4f sum = *(const gv_v4f*)(red + (j * 64 + l) * 4);
#pragma unroll
    for (int w = 1; w < 4; w++) {
      const gv_v4f v = *(const gv_v4f*)(red + ((w * RG + j) * 64 + l) * 4);
      sum = gv_v4f{sum[0] + v[0], sum[1] + v[1], sum[2] + v[2], sum[3] + v[3]};
    }
    const int m = l & 15;
    const int64_t n = (int64_t)(wg * RG + j) * 16 + 4 * (l >> 4);
    if (m < g.M && n < g.N) {
      const bool vec = n + 4 <= g.N && (g.ldc % 4) == 0 && (((uintptr_t)g.c) & 15) == 0;
      if (C_BF16) {
        uint16_t* dst = (uint16_t*)g.c + (int64_t)m * g.ldc + n;
        if (vec) {
          *(uint2*)dst = make_uint2(pk_bf16_rne(sum[0], sum[1]), pk_bf16_rne(sum[2], sum[3]));
        } else {
          for (int e = 0; e < 4 && n + e < g.N; e++) dst[e] = f32_to_bf16_rne(sum[e]);
        }
      } else {
        float* dst = (float*)g.c + (int64_t)m * g.ldc + n;
        if (vec) *(float4*)dst = make_float4(sum[0], sum[1], sum[2], sum[3]);
        else for (int e = 0; e < 4 && n + e < g.N; e++) dst[e] = sum[e];
      }
    }
  }
}

}  // namespace mix
