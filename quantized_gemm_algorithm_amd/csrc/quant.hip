// MiX and MX quantizers, their decoders and the K-mean, for gfx950.
//
// MiX (P1 = the pchao.org digest "MiX：面向端到端低比特视觉语言模型加速的微反缩放", section
// 方法概览 / method overview, format bullets and the Algorithm 1 bullet; Fig. 4 in the figure
// walk): a 32-element block stores a 4-bit Emax and a 3-bit shared mantissa (one per block for
// MiX-4.25b, one per 8-element sub-block for MiX-4.5b); each element stores a sign and a 3-bit
// relative exponent dE; value = (-1)^s (1.m)_2 2^(Emax - dE); dE = 7 is zero and the negative
// zero pattern is one more positive step. Algorithm 1 takes Emax and the mantissa from the
// block's (sub-block's) largest element and picks dE among the naive exponent and its two
// neighbours by reconstruction error.
//
// Layout of one lane's work: a lane owns one 8-element sub-block (16 B of bf16 or 32 B of fp32),
// a quad of lanes owns one 32-element block. The block max is a quad reduction over DPP. Codes
// leave as one 32-bit word per lane (8 nibbles), so a wave stores 256 contiguous bytes.

#include "common.h"
#include "f8_image.h"
#include "kernels.h"
#include "quant_dev.h"

namespace mix {

// ------------------------------------------------------------------ MiX quantizer (K1)

// With IMG the lane also writes the GEMM A image of its sub-block (f8_image.h): 8 E4M3 bytes, and
// on quad lane 0 the block's E8M0 scale 2^(Emax-1). codes/shared may then be NULL (not written).
//
// Work layout: grid (column chunks, row groups); a workgroup codes R rows of one chunk of
// blockDim.x sub-blocks per pass (the launcher sizes blocks to the row when it has at most 1024
// sub-blocks), so every row-dependent offset is a wave-uniform scalar and a lane only adds its
// sub-block's offset. The R rows' loads are issued together, R 16-byte loads in flight per lane.
template <int DT, int FMT, int IMG, int R = 2>  // FMT 0 = MiX-4.25b, 1 = MiX-4.5b
__global__ void __launch_bounds__(1024) k_mix_quantize(const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
                                                        uint8_t* __restrict__ codes, void* __restrict__ shared,
                                                        uint8_t* __restrict__ a8, uint8_t* __restrict__ as_p,
                                                        int tiles_m) {
  __shared__ uint4 pk_tbl[128];   // block constants of the pair coder per (Emax, m)
  if (DT == 1) {
    mix_pk_table_fill(pk_tbl);
    __syncthreads();
  }
  const int spr = (int)(cols >> 3);                       // sub-blocks per row
  const int sc = blockIdx.x * blockDim.x + threadIdx.x;   // this lane's sub-block in the row
  // whole quads are in or out of range together (spr and the chunk size are multiples of 4)
  const bool col_ok = sc < spr;
  const int scc = col_ok ? sc : (sc & 3);
  const int q = scc & 3;
  const int blk = scc >> 2;
  // Row groups in XCD-contiguous bands (workgroup y runs on XCD y % 8 when the row fits one chunk):
  // the small per-row outputs (a row's shared fields and its scale dwords share cache lines with
  // the neighbouring rows) are then written whole by one XCD's L2 instead of in pieces by all eight.
  const int gy = gridDim.y, xb = blockIdx.y & 7;
  const int pr = xb * (gy >> 3) + min(xb, gy & 7) + (int)(blockIdx.y >> 3);
  for (int64_t r0 = (int64_t)pr * R; r0 < rows; r0 += (int64_t)gy * R) {
    uint32_t sdw[R];   // IMG: the four E8M0 scales of this lane's K step (valid on lane 16k)
    uint32_t xb[R][8];  // bf16: the 16 raw bytes in xb[u][0..3]; fp32: the 8 bit patterns
#pragma unroll
    for (int u = 0; u < R; u++) {
      const int64_t row = r0 + u < rows ? r0 + u : rows - 1;
      if (DT == 1) {
        const uint4 v = *(const uint4*)((const uint16_t*)x + row * ldx + (int64_t)scc * 8);
        xb[u][0] = v.x; xb[u][1] = v.y; xb[u][2] = v.z; xb[u][3] = v.w;
      } else {
        load8<DT>(x, row, ldx, (int64_t)scc * 8, xb[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < R; u++) {
      const int64_t row = r0 + u;
      int emax;
      uint32_t m, e0, e1;   // e0, e1: the sub-block's 8 E4M3 image bytes (IMG)
      uint32_t word;
      if (DT == 1) {
        const uint32_t w4[4] = {xb[u][0], xb[u][1], xb[u][2], xb[u][3]};
        word = mix_quant_lane_bf16_tbl<FMT, IMG != 0>(w4, pk_tbl, emax, m, e0, e1);
      } else {
        word = mix_quant_lane_img<FMT, IMG != 0>(xb[u], emax, m, e0, e1);
      }
      uint32_t f = 0;
      if (FMT == 1) f = quad_or_dpp((q == 0 ? (uint32_t)(emax + 7) : 0u) | (m << (4 + 3 * q)));
      if (IMG) {
        // a 16-lane DPP row is one K step (four blocks, Emax uniform over each quad): lane 16k gathers
        // the blocks' scales from lanes 16k + 4, + 8, + 12 (rotations right by 12, 8, 4)
        const int v = emax + 126;
        sdw[u] = (uint32_t)v | ((uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x12C, 0xF, 0xF, true) << 8) |
                 ((uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, true) << 16) |
                 ((uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, true) << 24);
      }
      if (!col_ok || row >= rows) continue;
      if (!IMG || codes) {
        *(uint32_t*)(codes + row * (cols >> 1) + scc * 4) = word;
        if (FMT == 1) {
          if (q == 0) ((uint16_t*)shared)[row * (cols >> 5) + blk] = (uint16_t)f;
        } else {
          if (q == 0) ((uint8_t*)shared)[row * (cols >> 5) + blk] = (uint8_t)((uint32_t)(emax + 7) | (m << 4));
        }
      }
      if (IMG) *(uint2*)(a8 + row * cols + scc * 8) = make_uint2(e0, e1);
    }
    if (IMG && col_ok && (scc & 15) == 0) {
      // the rows' scale dwords of this K step (f8_a_scale_pos: row-major, so the R rows of a
      // workgroup, R-aligned and in one 256-row tile, are adjacent)
      uint8_t* sp = as_p + ((int64_t)(scc >> 4) * tiles_m + (r0 >> 8)) * 1024 + (r0 & (FT - 1)) * 4;
      if (r0 + R <= rows) {
#pragma unroll
        for (int u = 0; u < R; u += 2) *(uint2*)(sp + 4 * u) = make_uint2(sdw[u], sdw[u + 1]);
      } else {
        for (int u = 0; u < R && r0 + u < rows; u++) *(uint32_t*)(sp + 4 * u) = sdw[u];
      }
    }
  }
}

// The bf16 quantizer with the work dealt to a fixed grid: a wave owns a segment of 64 sub-blocks
// (512 elements, four 128-wide K steps) of one row; the (row, segment) tasks in row-major order are
// dealt round-robin to the grid's waves, and each wave walks its tasks with the next task's 16-byte
// loads in flight while it codes the current one. Short-lived workgroups (one or two rows each)
// left the GPU waiting on workgroup launches: about one resident wave per SIMD on average.
// The coding, the outputs and their layout are those of k_mix_quantize.
// The body as a device function of workgroup wg of nwg (so that a kernel with other roles can run
// it on a part of its grid); pk_tbl is 128 uint4 of LDS.
template <int FMT, int IMG>
__device__ __forceinline__ void mq_seg_body(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
                                            uint8_t* __restrict__ codes, void* __restrict__ shared,
                                            uint8_t* __restrict__ a8, uint8_t* __restrict__ as_p, int tiles_m,
                                            int64_t nwg, int64_t wg, uint4* pk_tbl) {
  mix_pk_table_fill(pk_tbl);   // block constants of the pair coder per (Emax, m)
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int spr = (int)(cols >> 3);                 // sub-blocks per row (a multiple of 4)
  const int nseg = (spr + 63) >> 6;                 // segments per row
  const int64_t nw = nwg * 4;                       // waves dealt tasks
  const int dq = (int)(nw / nseg), dr = (int)(nw % nseg);
  const int64_t t0 = wg * 4 + wave;
  int64_t row = t0 / nseg;
  int seg = (int)(t0 % nseg);
  const int q = lane & 3;
  auto sub = [&](int sg) {                           // this lane's sub-block in segment sg, and whether it is real
    const int sc = sg * 64 + lane;
    return sc < spr ? sc : -1 - (sc & 3);           // past the row: a valid sub-block of the same quad position
  };
  auto load = [&](int64_t r, int sg) {
    const int sc = sub(sg);
    return *(const uint4*)(x + r * ldx + (int64_t)(sc >= 0 ? sc : -1 - sc) * 8);
  };
  uint4 cur = row < rows ? load(row, seg) : make_uint4(0, 0, 0, 0);
  while (row < rows) {
    int64_t nrow = row + dq;
    int nsg = seg + dr;
    if (nsg >= nseg) { nsg -= nseg; nrow++; }
    const uint4 nxt = nrow < rows ? load(nrow, nsg) : make_uint4(0, 0, 0, 0);   // next task's loads in flight
    const int sc0 = sub(seg);
    const bool ok = sc0 >= 0;
    const int scc = ok ? sc0 : -1 - sc0;
    const uint32_t w4[4] = {cur.x, cur.y, cur.z, cur.w};
    int emax;
    uint32_t m, e0, e1;
    const uint32_t word = mix_quant_lane_bf16_tbl<FMT, IMG != 0>(w4, pk_tbl, emax, m, e0, e1);
    uint32_t f = 0;
    if (FMT == 1) f = quad_or_dpp((q == 0 ? (uint32_t)(emax + 7) : 0u) | (m << (4 + 3 * q)));
    uint32_t sdw = 0;
    if (IMG) {
      const int v = emax + 126;
      sdw = (uint32_t)v | ((uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x12C, 0xF, 0xF, true) << 8) |
            ((uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, true) << 16) |
            ((uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, true) << 24);
    }
    if (ok) {
      const int blk = scc >> 2;
      if (!IMG || codes) {
        *(uint32_t*)(codes + row * (cols >> 1) + scc * 4) = word;
        if (FMT == 1) {
          if (q == 0) ((uint16_t*)shared)[row * (cols >> 5) + blk] = (uint16_t)f;
        } else {
          if (q == 0) ((uint8_t*)shared)[row * (cols >> 5) + blk] = (uint8_t)((uint32_t)(emax + 7) | (m << 4));
        }
      }
      if (IMG) {
        *(uint2*)(a8 + row * cols + scc * 8) = make_uint2(e0, e1);
        if ((scc & 15) == 0)
          *(uint32_t*)(as_p + ((int64_t)(scc >> 4) * tiles_m + (row >> 8)) * 1024 + (row & (FT - 1)) * 4) = sdw;
      }
    }
    row = nrow;
    seg = nsg;
    cur = nxt;
  }
}

template <int FMT, int IMG>
__global__ void __launch_bounds__(256) k_mix_quantize_seg(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                           int64_t ldx, uint8_t* __restrict__ codes,
                                                           void* __restrict__ shared, uint8_t* __restrict__ a8,
                                                           uint8_t* __restrict__ as_p, int tiles_m) {
  __shared__ uint4 pk_tbl[128];
  mq_seg_body<FMT, IMG>(x, rows, cols, ldx, codes, shared, a8, as_p, tiles_m, gridDim.x, blockIdx.x, pk_tbl);
}

// ------------------------------------------------------------------ MX quantizer (K2), blocks along rows

// G16: one shared exponent per 16 elements (a lane pair) instead of 32 (a quad); scales [rows, cols/16]
template <int DT, int FP4, int MU, int G16 = 0>
__global__ void __launch_bounds__(256) k_mx_quantize(const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
                                                      const float* __restrict__ mu, uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
  const int64_t sub_per_row = cols >> 3;
  const int64_t total = rows * sub_per_row;
  const int lane = threadIdx.x & 63;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g - lane < total;
       g += (int64_t)gridDim.x * blockDim.x) {
    if (g >= total) continue;
    int64_t row = g / sub_per_row;
    int64_t sc = g - row * sub_per_row;
    uint32_t xb[8];
    load8<DT>(x, row, ldx, sc * 8, xb);
    if (MU) {
      const float4* mp = (const float4*)(mu + sc * 8);
      float4 m0 = mp[0], m1 = mp[1];
      float mv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
      for (int i = 0; i < 8; i++) xb[i] = f32_bits(__fsub_rn(bits_f32(xb[i]), mv[i]));
    }
    uint32_t lmax = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      uint32_t a = xb[i] & 0x7FFFFFFFu;
      lmax = a > lmax ? a : lmax;
    }
    uint32_t bmax;
    if (G16) {
      const uint32_t t = (uint32_t)__builtin_amdgcn_mov_dpp((int)lmax, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
      bmax = lmax > t ? lmax : t;
    } else {
      bmax = quad_max_u32(lmax);
    }
    uint32_t word = 0;
    int X = mx_exponent(bmax, FP4);
    if (bmax != 0) {
      if (FP4) {
        Fp4Thr r = fp4_thresholds(X);
#pragma unroll
        for (int i = 0; i < 8; i++) word |= fp4_code(xb[i], r) << (4 * i);
      } else {
        Int4Thr r = int4_thresholds(X);
#pragma unroll
        for (int i = 0; i < 8; i++) word |= int4_code(xb[i], r) << (4 * i);
      }
    }
    *(uint32_t*)(codes + row * (cols >> 1) + sc * 4) = word;
    if (G16) {
      if ((sc & 1) == 0) scales[row * (cols >> 4) + (sc >> 1)] = bmax ? (uint8_t)(X + 127) : (uint8_t)0;
    } else if ((sc & 3) == 0) {
      scales[row * (cols >> 5) + (sc >> 2)] = bmax ? (uint8_t)(X + 127) : (uint8_t)0;
    }
  }
}

// ------------------------------------------------------------------ MX quantizer, blocks along columns
// x [rows, cols] (row pitch ldx); a block is 32 consecutive rows of one column. Output codes
// [cols, >= prows/2] and scales [cols, >= prows/32] with row pitches cpitch / spitch bytes (the
// transposed layout used for V along tokens). Rows beyond `rows` up to the padded count `prows`
// are zero.
template <int DT>
struct MqcTile {
  static constexpr int COLS = 64;                       // columns per workgroup
  static constexpr int ROWS = 128;                      // rows per workgroup: four 32-row blocks
  static constexpr int LPR = COLS * (DT == 1 ? 2 : 4) / 16;   // 16-byte loads per row
  static constexpr int RPP = 256 / LPR;                 // rows per load pass of the workgroup
};

// A workgroup of 256 threads owns 64 columns x 128 rows: its loads read whole row segments (VEC:
// 16 bytes a lane, consecutive lanes along the row; otherwise one element a lane, for inputs whose
// rows are not 16-byte aligned), the tile is transposed through LDS, and thread t then codes the
// 32-row block t >> 6 of column t & 63. Rows at or beyond `rows` read as zero. With PAD, the scale
// byte of block prows / 32 (the first block past the padded rows), when it lies inside the scale
// row's pitch, is set to 127 (scale 1): a product that reads a whole 64-row tile of V^ past the end
// then multiplies its zero weights by a finite scale.
template <int DT, int VEC, int PAD = 0>   // workgroup (bx, by); tile: TL::ROWS * TL::COLS elements of LDS, 16-byte aligned
__device__ __forceinline__ void mqc_body(const void* __restrict__ x, int64_t rows, int64_t prows, int64_t cols,
                                         int64_t ldx, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                         int64_t cpitch, int64_t spitch, int64_t bx, int64_t by, uint8_t* tile) {
  using TL = MqcTile<DT>;
  constexpr int ESZ = DT == 1 ? 2 : 4;
  const int64_t c0 = bx * TL::COLS;
  const int64_t r0 = by * TL::ROWS;
  if (VEC) {
    const int seg = threadIdx.x % TL::LPR, rr = threadIdx.x / TL::LPR;
    const int64_t cl = c0 + seg * (16 / ESZ);           // first column of this lane's 16 bytes
    uint4 v[TL::ROWS / TL::RPP];
#pragma unroll
    for (int p = 0; p < TL::ROWS / TL::RPP; p++) {
      const int64_t r = r0 + rr + p * TL::RPP;
      v[p] = make_uint4(0u, 0u, 0u, 0u);
      if (r < rows && cl < cols) v[p] = *(const uint4*)((const uint8_t*)x + (r * ldx + cl) * ESZ);
    }
#pragma unroll
    for (int p = 0; p < TL::ROWS / TL::RPP; p++)
      *(uint4*)(tile + ((rr + p * TL::RPP) * TL::COLS + seg * (16 / ESZ)) * ESZ) = v[p];
  } else {
    for (int e = threadIdx.x; e < TL::ROWS * TL::COLS; e += 256) {
      const int64_t r = r0 + e / TL::COLS, c = c0 + e % TL::COLS;
      if (DT == 1) {
        const uint16_t u = r < rows && c < cols ? ((const uint16_t*)x)[r * ldx + c] : (uint16_t)0;
        ((uint16_t*)tile)[e] = u;
      } else {
        const uint32_t u = r < rows && c < cols ? ((const uint32_t*)x)[r * ldx + c] : 0u;
        ((uint32_t*)tile)[e] = u;
      }
    }
  }
  __syncthreads();
  const int c = threadIdx.x & 63, blk = threadIdx.x >> 6;
  const int64_t cg = c0 + c, rb = r0 / 32 + blk;
  if (cg >= cols) return;
  if (rb * 32 >= prows) {
    if (PAD && rb * 32 == prows && rb < spitch) scales[cg * spitch + rb] = 127;
    return;
  }
  uint32_t xb[32];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 32; i++) {
    const int e = (blk * 32 + i) * TL::COLS + c;
    const uint32_t u = DT == 1 ? (uint32_t)((const uint16_t*)tile)[e] << 16 : ((const uint32_t*)tile)[e];
    xb[i] = u;
    const uint32_t a = u & 0x7FFFFFFFu;
    amax = a > amax ? a : amax;
  }
  uint32_t w[4] = {0, 0, 0, 0};
  const int X = mx_exponent(amax, 1);
  if (amax != 0) {
    const Fp4Thr r = fp4_thresholds(X);
#pragma unroll
    for (int i = 0; i < 32; i++) w[i >> 3] |= fp4_code(xb[i], r) << (4 * (i & 7));
  }
  *(uint4*)(codes + cg * cpitch + rb * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  scales[cg * spitch + rb] = amax ? (uint8_t)(X + 127) : (uint8_t)0;
}

template <int DT, int VEC>
__global__ void __launch_bounds__(256) k_mx_quantize_cols(const void* __restrict__ x, int64_t rows, int64_t prows,
                                                           int64_t cols, int64_t ldx, uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales, int64_t cpitch,
                                                           int64_t spitch) {
  using TL = MqcTile<DT>;
  __shared__ __align__(16) uint8_t tile[TL::ROWS * TL::COLS * (DT == 1 ? 2 : 4)];
  mqc_body<DT, VEC>(x, rows, prows, cols, ldx, codes, scales, cpitch, spitch, blockIdx.x, blockIdx.y, tile);
}

// ------------------------------------------------------------------ decoders (debug / tests)

__global__ void k_mix_dequantize(int fmt, const uint8_t* __restrict__ codes, const void* __restrict__ shared, int64_t rows,
                                 int64_t cols, float* __restrict__ out) {
  int64_t n = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = i / cols, c = i - r * cols;
    uint32_t nib = (codes[r * (cols >> 1) + (c >> 1)] >> ((c & 1) * 4)) & 0xF;
    uint32_t f = fmt ? ((const uint16_t*)shared)[r * (cols >> 5) + (c >> 5)]
                     : ((const uint8_t*)shared)[r * (cols >> 5) + (c >> 5)];
    int emax = (int)(f & 15) - 7;
    uint32_t m = fmt ? (f >> (4 + 3 * ((c & 31) >> 3))) & 7 : (f >> 4) & 7;
    float v;
    if (nib == 0x7) v = 0.f;
    else {
      int de = nib == 0xF ? 7 : (int)(nib & 7);
      v = ldexpf(1.0f + (float)m * 0.125f, emax - de);
      if (nib != 0xF && (nib & 8)) v = -v;
    }
    out[i] = v;
  }
}

__global__ void k_mx_dequantize(int fp4, int g16, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                int64_t rows, int64_t cols, float* __restrict__ out) {
  const float e2m1[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
  int64_t n = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = i / cols, c = i - r * cols;
    uint32_t nib = (codes[r * (cols >> 1) + (c >> 1)] >> ((c & 1) * 4)) & 0xF;
    int X = (int)(g16 ? scales[r * (cols >> 4) + (c >> 4)] : scales[r * (cols >> 5) + (c >> 5)]) - 127;
    float v;
    if (fp4) {
      v = ldexpf(e2m1[nib & 7], X);
      if (nib & 8) v = -v;
    } else {
      int q = nib >= 8 ? (int)nib - 16 : (int)nib;
      v = ldexpf((float)q, X - 2);
    }
    out[i] = v;
  }
}

// ------------------------------------------------------------------ K-mean (exact sum)
// mu[c] = fp32( sum_t x[t, c] / T ) with the sum carried exactly as an unevaluated pair of
// doubles (TwoSum): exact for the bf16 inputs here, whose binade spread is far below 100.
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}
struct DD { double hi, lo; };
__device__ __forceinline__ DD dd_add(DD x, double y) {
  double s, e;
  two_sum(x.hi, y, s, e);
  e += x.lo;
  double h, l;
  two_sum(s, e, h, l);
  return DD{h, l};
}
__device__ __forceinline__ DD dd_add(DD x, DD y) {
  double s, e;
  two_sum(x.hi, y.hi, s, e);
  e += x.lo + y.lo;
  double h, l;
  two_sum(s, e, h, l);
  return DD{h, l};
}

// One workgroup per group of KM_CW columns (16 bytes of a row): its 1024 threads take rows
// t, t + 1024, ... and keep one exact pair per column; the pairs are added across the wave by
// shuffles and across the 16 waves in LDS. The result does not depend on the order whenever the
// exact sum fits the pair (as above).
constexpr int KM_THREADS = 1024;

template <int DT>
__global__ void __launch_bounds__(KM_THREADS) k_kmean(const void* __restrict__ x, int64_t T, int64_t C, int64_t ldx,
                                                       float* __restrict__ mu) {
  constexpr int CW = DT == 1 ? 8 : 4;  // columns per thread (one 16-byte load)
  __shared__ double shi[KM_THREADS / 64][CW];
  __shared__ double slo[KM_THREADS / 64][CW];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * CW;
  DD acc[CW];
#pragma unroll
  for (int j = 0; j < CW; j++) acc[j] = DD{0.0, 0.0};
  for (int64_t t = threadIdx.x; t < T; t += KM_THREADS) {
    const uint4 v = DT == 1 ? *(const uint4*)((const uint16_t*)x + t * ldx + c0) : *(const uint4*)((const float*)x + t * ldx + c0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < CW; j++) {
      const float f = DT == 1 ? __uint_as_float(j & 1 ? (w[j >> 1] & 0xFFFF0000u) : (w[j >> 1] << 16)) : __uint_as_float(w[j]);
      acc[j] = dd_add(acc[j], (double)f);
    }
  }
#pragma unroll
  for (int j = 0; j < CW; j++) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const DD o{__shfl_xor(acc[j].hi, off, 64), __shfl_xor(acc[j].lo, off, 64)};
      acc[j] = dd_add(acc[j], o);
    }
    if (lane == 0) {
      shi[wave][j] = acc[j].hi;
      slo[wave][j] = acc[j].lo;
    }
  }
  __syncthreads();
  if (threadIdx.x < CW) {
    const int j = threadIdx.x;
    DD s2{shi[0][j], slo[0][j]};
    for (int w2 = 1; w2 < KM_THREADS / 64; w2++) s2 = dd_add(s2, DD{shi[w2][j], slo[w2][j]});
    const double sum = s2.hi + s2.lo;  // correctly rounded: the pair is normalised
    mu[c0 + j] = (float)(sum / (double)T);
  }
}

// The K-mean in two launches, for callers with a workspace: the first spreads the rows over the
// whole GPU (workgroup (x, y): rows [KMP_ROWS y, KMP_ROWS (y + 1)) of 64 CW columns, each wave
// reading whole row segments, 16 bytes a lane) and writes one exact pair per (row slice, column);
// the second adds each column's pairs. Same result as k_kmean whenever the exact sum fits the pair.
constexpr int KMP_ROWS = 16;

// workgroup (bx, by); red: 2 x 64 CW double2 of LDS (the four waves' pairs are added in two rounds)
template <int DT>
__device__ __forceinline__ void kmp_body(const void* __restrict__ x, int64_t T, int64_t C, int64_t ldx,
                                         double2* __restrict__ part, int64_t bx, int64_t by, double2* red) {
  constexpr int CW = DT == 1 ? 8 : 4;   // columns per lane (one 16-byte load)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t cbase = bx * 64 * CW;
  const int64_t c0 = cbase + (int64_t)lane * CW;
  const int64_t r0 = by * KMP_ROWS;
  DD acc[CW];
#pragma unroll
  for (int j = 0; j < CW; j++) acc[j] = DD{0.0, 0.0};
  if (c0 < C) {
    uint4 v[KMP_ROWS / 4];
    // every load is issued before the first use: rows past T repeat row T - 1 and add zero
#pragma unroll
    for (int i = 0; i < KMP_ROWS / 4; i++) {
      const int64_t t = min(r0 + wave + 4 * i, T - 1);
      v[i] = DT == 1 ? *(const uint4*)((const uint16_t*)x + t * ldx + c0) : *(const uint4*)((const float*)x + t * ldx + c0);
    }
#pragma unroll
    for (int i = 0; i < KMP_ROWS / 4; i++) {
      const bool ok = r0 + wave + 4 * i < T;
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int j = 0; j < CW; j++) {
        const float f = DT == 1 ? __uint_as_float(j & 1 ? (w[j >> 1] & 0xFFFF0000u) : (w[j >> 1] << 16)) : __uint_as_float(w[j]);
        acc[j] = dd_add(acc[j], ok ? (double)f : 0.0);
      }
    }
  }
  // waves 2, 3 hand their pairs to waves 0, 1; wave 1 then hands its sums to wave 0, which writes
  double2* mine = red + (wave & 1) * 64 * CW + lane * CW;
  if (wave >= 2) {
#pragma unroll
    for (int j = 0; j < CW; j++) mine[j] = make_double2(acc[j].hi, acc[j].lo);
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int j = 0; j < CW; j++) acc[j] = dd_add(acc[j], DD{mine[j].x, mine[j].y});
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int j = 0; j < CW; j++) red[lane * CW + j] = make_double2(acc[j].hi, acc[j].lo);
  }
  __syncthreads();
  if (wave == 0 && c0 < C) {
#pragma unroll
    for (int j = 0; j < CW; j++) {
      const DD sum = dd_add(acc[j], DD{red[lane * CW + j].x, red[lane * CW + j].y});
      part[by * C + c0 + j] = make_double2(sum.hi, sum.lo);
    }
  }
}

template <int DT>
__global__ void __launch_bounds__(256) k_kmean_part(const void* __restrict__ x, int64_t T, int64_t C, int64_t ldx,
                                                    double2* __restrict__ part) {
  __shared__ double2 red[2 * 64 * (DT == 1 ? 8 : 4)];
  kmp_body<DT>(x, T, C, ldx, part, blockIdx.x, blockIdx.y, red);
}

// The prefill attention's three independent operand passes in one launch: V^ coding along tokens
// (workgroups [0, nv)), the K-mean's row-slice pairs ([nv, nv + nk)) and Q^ coding (the rest, dealt
// the segment tasks of a grid of nq). The short roles come first so that they are dispatched
// before the Q coder's workgroups take every slot. Inputs bf16, rows 16-byte aligned.
__global__ void __launch_bounds__(256) k_prefill_operands(PrefillOperandArgs a) {
  __shared__ __align__(16) uint8_t lds[MqcTile<1>::ROWS * MqcTile<1>::COLS * 2];   // 16 KB, every role's LDS
  int64_t b = blockIdx.x;
  if (b < a.nv) {
    mqc_body<1, 1, 1>(a.v, a.T, a.Tp, a.cv, a.ldv, a.vc, a.vs, a.cpitch, a.spitch, b % a.nvx, b / a.nvx, lds);
    return;
  }
  b -= a.nv;
  if (b < a.nk) {
    kmp_body<1>(a.k, a.T, a.ck, a.ldk, a.part, b % a.nkx, b / a.nkx, (double2*)lds);
    return;
  }
  b -= a.nk;
  mq_seg_body<1, 0>(a.q, a.T, a.cq, a.ldq, a.qc, a.qs, nullptr, nullptr, 0, a.nq, b, (uint4*)lds);
}

// Workgroup of 256 threads per 8 columns: 32 threads per column each add every 32nd row slice's
// pair (their loads issued together), then a tree in LDS adds the 32 sums.
__global__ void __launch_bounds__(256) k_kmean_fin(const double2* __restrict__ part, int64_t nslices, int64_t T,
                                                   int64_t C, float* __restrict__ mu) {
  __shared__ double2 red[32][8];
  const int cc = threadIdx.x & 7, j = threadIdx.x >> 3;
  const int64_t c = (int64_t)blockIdx.x * 8 + cc;
  DD sum{0.0, 0.0};
  if (c < C) {
    int64_t p = j;
    for (; p + 7 * 32 < nslices; p += 8 * 32) {   // eight loads in flight
      double2 v[8];
#pragma unroll
      for (int u = 0; u < 8; u++) v[u] = part[(p + 32 * u) * C + c];
#pragma unroll
      for (int u = 0; u < 8; u++) sum = dd_add(sum, DD{v[u].x, v[u].y});
    }
    for (; p < nslices; p += 32) {
      const double2 a = part[p * C + c];
      sum = dd_add(sum, DD{a.x, a.y});
    }
  }
  red[j][cc] = make_double2(sum.hi, sum.lo);
#pragma unroll
  for (int h = 16; h >= 1; h >>= 1) {
    __syncthreads();
    if (j < h) {
      const DD o{red[j + h][cc].x, red[j + h][cc].y};
      const DD m{red[j][cc].x, red[j][cc].y};
      const DD r = dd_add(m, o);
      red[j][cc] = make_double2(r.hi, r.lo);
    }
  }
  if (j == 0 && c < C) mu[c] = (float)((red[0][cc].x + red[0][cc].y) / (double)T);
}

// ------------------------------------------------------------------ launchers

static inline int grid_for(int64_t threads_needed) {
  int64_t b = (threads_needed + 255) / 256;
  if (b > 65535 * 4) b = 65535 * 4;
  return (int)(b < 1 ? 1 : b);
}

// rows per workgroup pass of k_mix_quantize (fp32 input)
constexpr int MQ_ROWS = 2;

// compute units of the current device
static int mq_cu_count() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

static void mq_grid(int64_t rows, int64_t cols, int R, dim3& g, dim3& b) {
  const int64_t spr = cols >> 3;
  const int64_t bx = spr <= 1024 ? (spr + 63) / 64 * 64 : 1024;
  b = dim3((unsigned)bx);
  const int64_t gx = (spr + bx - 1) / bx;
  int64_t gy = (rows + R - 1) / R;
  if (gy > 65535) gy = 65535;
  g = dim3((unsigned)gx, (unsigned)(gy < 1 ? 1 : gy));
}

// bf16 input: the segment-dealt kernel on a grid of up to 8 workgroups (32 waves) per CU
static dim3 mq_seg_grid(int64_t rows, int64_t cols) {
  const int64_t tasks = rows * (((cols >> 3) + 63) >> 6);
  int64_t g = (tasks + 3) / 4;
  const int64_t cap = 8 * (int64_t)mq_cu_count();
  if (g > cap) g = cap;
  return dim3((unsigned)(g < 1 ? 1 : g));
}

hipError_t launch_mix_quantize(int fmt, const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                               uint8_t* codes, void* shared, hipStream_t s) {
  if (dtype == 1) {
    const dim3 g = mq_seg_grid(rows, cols);
    if (fmt == 1)
      hipLaunchKernelGGL((k_mix_quantize_seg<1, 0>), g, dim3(256), 0, s, (const uint16_t*)x, rows, cols, ldx, codes,
                         shared, nullptr, nullptr, 0);
    else
      hipLaunchKernelGGL((k_mix_quantize_seg<0, 0>), g, dim3(256), 0, s, (const uint16_t*)x, rows, cols, ldx, codes,
                         shared, nullptr, nullptr, 0);
    return hipGetLastError();
  }
  dim3 g, b;
  mq_grid(rows, cols, MQ_ROWS, g, b);
  if (fmt == 1)
    hipLaunchKernelGGL((k_mix_quantize<0, 1, 0, MQ_ROWS>), g, b, 0, s, x, rows, cols, ldx, codes, shared, nullptr,
                       nullptr, 0);
  else
    hipLaunchKernelGGL((k_mix_quantize<0, 0, 0, MQ_ROWS>), g, b, 0, s, x, rows, cols, ldx, codes, shared, nullptr,
                       nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_mix_quantize_img(int fmt, const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                                   uint8_t* codes, void* shared, void* img, hipStream_t s) {
  const F8AImage L = f8_a_image_layout(rows, cols);
  uint8_t* a8 = (uint8_t*)img + L.a8;
  uint8_t* as_p = (uint8_t*)img + L.as_p;
  const int tiles_m = (int)((rows + FT - 1) / FT);
  if (dtype == 1) {
    const dim3 g = mq_seg_grid(rows, cols);
    if (fmt == 1)
      hipLaunchKernelGGL((k_mix_quantize_seg<1, 1>), g, dim3(256), 0, s, (const uint16_t*)x, rows, cols, ldx, codes,
                         shared, a8, as_p, tiles_m);
    else
      hipLaunchKernelGGL((k_mix_quantize_seg<0, 1>), g, dim3(256), 0, s, (const uint16_t*)x, rows, cols, ldx, codes,
                         shared, a8, as_p, tiles_m);
    return hipGetLastError();
  }
  dim3 g, b;
  mq_grid(rows, cols, MQ_ROWS, g, b);
  if (fmt == 1)
    hipLaunchKernelGGL((k_mix_quantize<0, 1, 1, MQ_ROWS>), g, b, 0, s, x, rows, cols, ldx, codes, shared, a8, as_p,
                       tiles_m);
  else
    hipLaunchKernelGGL((k_mix_quantize<0, 0, 1, MQ_ROWS>), g, b, 0, s, x, rows, cols, ldx, codes, shared, a8, as_p,
                       tiles_m);
  return hipGetLastError();
}

hipError_t launch_mx_quantize(int fp4, const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                              const float* mu, uint8_t* codes, uint8_t* scales, hipStream_t s, int g16) {
  int64_t total = rows * (cols >> 3);
  dim3 g(grid_for(total)), b(256);
#define MXQ(DT, F, M) \
  if (g16) hipLaunchKernelGGL((k_mx_quantize<DT, F, M, 1>), g, b, 0, s, x, rows, cols, ldx, mu, codes, scales); \
  else hipLaunchKernelGGL((k_mx_quantize<DT, F, M, 0>), g, b, 0, s, x, rows, cols, ldx, mu, codes, scales)
  if (dtype == 1) {
    if (fp4) { if (mu) { MXQ(1, 1, 1); } else { MXQ(1, 1, 0); } }
    else { if (mu) { MXQ(1, 0, 1); } else { MXQ(1, 0, 0); } }
  } else {
    if (fp4) { if (mu) { MXQ(0, 1, 1); } else { MXQ(0, 1, 0); } }
    else { if (mu) { MXQ(0, 0, 1); } else { MXQ(0, 0, 0); } }
  }
#undef MXQ
  return hipGetLastError();
}

hipError_t launch_mx_quantize_cols(const void* x, int dtype, int64_t rows, int64_t prows, int64_t cols, int64_t ldx,
                                   uint8_t* codes, uint8_t* scales, int64_t cpitch, int64_t spitch, hipStream_t s) {
  dim3 g((unsigned)((cols + 63) / 64), (unsigned)((prows + 127) / 128)), b(256);
  const int esz = dtype == 1 ? 2 : 4;
  const bool vec = ((uintptr_t)x & 15) == 0 && (ldx * esz) % 16 == 0 && (cols * esz) % 16 == 0;
#define MQC(DT, V) \
  hipLaunchKernelGGL((k_mx_quantize_cols<DT, V>), g, b, 0, s, x, rows, prows, cols, ldx, codes, scales, cpitch, spitch)
  if (dtype == 1) {
    if (vec) MQC(1, 1); else MQC(1, 0);
  } else {
    if (vec) MQC(0, 1); else MQC(0, 0);
  }
#undef MQC
  return hipGetLastError();
}

hipError_t launch_mix_dequantize(int fmt, const uint8_t* codes, const void* shared, int64_t rows, int64_t cols,
                                 float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_mix_dequantize, dim3(grid_for(rows * cols)), dim3(256), 0, s, fmt, codes, shared, rows, cols, out);
  return hipGetLastError();
}

hipError_t launch_mx_dequantize(int fp4, const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                                float* out, hipStream_t s, int g16) {
  hipLaunchKernelGGL(k_mx_dequantize, dim3(grid_for(rows * cols)), dim3(256), 0, s, fp4, g16, codes, scales, rows, cols,
                     out);
  return hipGetLastError();
}

hipError_t launch_prefill_operands(const PrefillOperandArgs& a0, hipStream_t s) {
  PrefillOperandArgs a = a0;
  a.nvx = (a.cv + MqcTile<1>::COLS - 1) / MqcTile<1>::COLS;
  a.nv = a.nvx * ((a.Tp + MqcTile<1>::ROWS - 1) / MqcTile<1>::ROWS);
  a.nkx = (a.ck + 512 - 1) / 512;
  a.nk = a.nkx * ((a.T + KMP_ROWS - 1) / KMP_ROWS);
  a.nq = mq_seg_grid(a.T, a.cq).x;
  hipLaunchKernelGGL(k_prefill_operands, dim3((unsigned)(a.nv + a.nk + a.nq)), dim3(256), 0, s, a);
  return hipGetLastError();
}

size_t kmean_ws_bytes(int64_t T, int64_t C) { return (size_t)((T + KMP_ROWS - 1) / KMP_ROWS) * C * 16; }

hipError_t launch_kmean_ws(const void* x, int dtype, int64_t T, int64_t C, int64_t ldx, float* mu, void* ws,
                           hipStream_t s) {
  const int64_t nsl = (T + KMP_ROWS - 1) / KMP_ROWS;
  const int64_t cw = dtype == 1 ? 8 : 4;
  dim3 g((unsigned)((C + 64 * cw - 1) / (64 * cw)), (unsigned)nsl);
  if (dtype == 1) hipLaunchKernelGGL((k_kmean_part<1>), g, dim3(256), 0, s, x, T, C, ldx, (double2*)ws);
  else hipLaunchKernelGGL((k_kmean_part<0>), g, dim3(256), 0, s, x, T, C, ldx, (double2*)ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_kmean_fin(ws, T, C, mu, s);
}

hipError_t launch_kmean_fin(const void* part, int64_t T, int64_t C, float* mu, hipStream_t s) {
  const int64_t nsl = (T + KMP_ROWS - 1) / KMP_ROWS;
  hipLaunchKernelGGL(k_kmean_fin, dim3((unsigned)((C + 7) / 8)), dim3(256), 0, s, (const double2*)part, nsl, T, C,
                     mu);
  return hipGetLastError();
}

hipError_t launch_kmean(const void* x, int dtype, int64_t T, int64_t C, int64_t ldx, float* mu, hipStream_t s) {
  dim3 g((unsigned)(C / (dtype == 1 ? 8 : 4))), b(KM_THREADS);
  if (dtype == 1) hipLaunchKernelGGL((k_kmean<1>), g, b, 0, s, x, T, C, ldx, mu);
  else hipLaunchKernelGGL((k_kmean<0>), g, b, 0, s, x, T, C, ldx, mu);
  return hipGetLastError();
}

}  // namespace mix
