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
// Work layout: grid (column chunks, row pairs); a workgroup codes MQ_R rows of one chunk of
// blockDim.x sub-blocks (the launcher sizes blocks to the row when it has at most 1024
// sub-blocks), so every row-dependent offset is a wave-uniform scalar and a lane only adds its
// sub-block's offset. The MQ_R rows' loads are issued together.
constexpr int MQ_R = 2;

template <int DT, int FMT, int IMG>  // FMT 0 = MiX-4.25b, 1 = MiX-4.5b
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
  // Row pairs in XCD-contiguous bands (workgroup y runs on XCD y % 8 when the row fits one chunk):
  // the small per-row outputs (a row's shared fields and its scale dwords share cache lines with
  // the neighbouring rows) are then written whole by one XCD's L2 instead of in pieces by all eight.
  const int gy = gridDim.y, xb = blockIdx.y & 7;
  const int pr = xb * (gy >> 3) + min(xb, gy & 7) + (int)(blockIdx.y >> 3);
  for (int64_t r0 = (int64_t)pr * MQ_R; r0 < rows; r0 += (int64_t)gy * MQ_R) {
    uint32_t sdw[MQ_R];   // IMG: the four E8M0 scales of this lane's K step (valid on lane 16k)
    uint32_t xb[MQ_R][8];  // bf16: the 16 raw bytes in xb[u][0..3]; fp32: the 8 bit patterns
#pragma unroll
    for (int u = 0; u < MQ_R; u++) {
      const int64_t row = r0 + u < rows ? r0 + u : rows - 1;
      if (DT == 1) {
        const uint4 v = *(const uint4*)((const uint16_t*)x + row * ldx + (int64_t)scc * 8);
        xb[u][0] = v.x; xb[u][1] = v.y; xb[u][2] = v.z; xb[u][3] = v.w;
      } else {
        load8<DT>(x, row, ldx, (int64_t)scc * 8, xb[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < MQ_R; u++) {
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
      // the rows' scale dwords of this K step (f8_a_scale_pos: row-major, so the MQ_R = 2 rows of a
      // workgroup, even-aligned and in one 256-row tile, are adjacent)
      uint8_t* sp = as_p + ((int64_t)(scc >> 4) * tiles_m + (r0 >> 8)) * 1024 + (r0 & (FT - 1)) * 4;
      if (r0 + 1 < rows) *(uint2*)sp = make_uint2(sdw[0], sdw[1]);
      else *(uint32_t*)sp = sdw[0];
    }
  }
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
__global__ void __launch_bounds__(256) k_mx_quantize_cols(const void* __restrict__ x, int64_t rows, int64_t prows,
                                                           int64_t cols, int64_t ldx, uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales, int64_t cpitch,
                                                           int64_t spitch) {
  int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t rb = blockIdx.y;  // 32-row block
  if (c >= cols) return;
  uint32_t xb[32];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 32; i++) {
    int64_t r = rb * 32 + i;
    uint32_t v = 0;
    if (r < rows) {
      if (DT == 1) v = (uint32_t)((const uint16_t*)x)[r * ldx + c] << 16;
      else v = ((const uint32_t*)x)[r * ldx + c];
    }
    xb[i] = v;
    uint32_t a = v & 0x7FFFFFFFu;
    amax = a > amax ? a : amax;
  }
  uint32_t w[4] = {0, 0, 0, 0};
  int X = mx_exponent(amax, 1);
  if (amax != 0) {
    Fp4Thr r = fp4_thresholds(X);
#pragma unroll
    for (int i = 0; i < 32; i++) w[i >> 3] |= fp4_code(xb[i], r) << (4 * (i & 7));
  }
  uint4 o = {w[0], w[1], w[2], w[3]};
  *(uint4*)(codes + c * cpitch + rb * 16) = o;
  scales[c * spitch + rb] = amax ? (uint8_t)(X + 127) : (uint8_t)0;
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

// ------------------------------------------------------------------ launchers

static inline int grid_for(int64_t threads_needed) {
  int64_t b = (threads_needed + 255) / 256;
  if (b > 65535 * 4) b = 65535 * 4;
  return (int)(b < 1 ? 1 : b);
}

static void mq_grid(int64_t rows, int64_t cols, dim3& g, dim3& b) {
  const int64_t spr = cols >> 3;
  const int64_t bx = spr <= 1024 ? (spr + 63) / 64 * 64 : 1024;
  b = dim3((unsigned)bx);
  const int64_t gx = (spr + bx - 1) / bx;
  int64_t gy = (rows + MQ_R - 1) / MQ_R;
  if (gy > 65535) gy = 65535;
  g = dim3((unsigned)gx, (unsigned)(gy < 1 ? 1 : gy));
}

hipError_t launch_mix_quantize(int fmt, const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                               uint8_t* codes, void* shared, hipStream_t s) {
  dim3 g, b;
  mq_grid(rows, cols, g, b);
#define MQ(DT, F) hipLaunchKernelGGL((k_mix_quantize<DT, F, 0>), g, b, 0, s, x, rows, cols, ldx, codes, shared, \
                                     nullptr, nullptr, 0)
  if (dtype == 1) { if (fmt == 1) MQ(1, 1); else MQ(1, 0); }
  else { if (fmt == 1) MQ(0, 1); else MQ(0, 0); }
#undef MQ
  return hipGetLastError();
}

hipError_t launch_mix_quantize_img(int fmt, const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                                   uint8_t* codes, void* shared, void* img, hipStream_t s) {
  dim3 g, b;
  mq_grid(rows, cols, g, b);
  const F8AImage L = f8_a_image_layout(rows, cols);
  uint8_t* a8 = (uint8_t*)img + L.a8;
  uint8_t* as_p = (uint8_t*)img + L.as_p;
  const int tiles_m = (int)((rows + FT - 1) / FT);
#define MQ(DT, F) hipLaunchKernelGGL((k_mix_quantize<DT, F, 1>), g, b, 0, s, x, rows, cols, ldx, codes, shared, a8, \
                                     as_p, tiles_m)
  if (dtype == 1) { if (fmt == 1) MQ(1, 1); else MQ(1, 0); }
  else { if (fmt == 1) MQ(0, 1); else MQ(0, 0); }
#undef MQ
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
  dim3 g((unsigned)((cols + 255) / 256), (unsigned)(prows / 32)), b(256);
  if (dtype == 1)
    hipLaunchKernelGGL((k_mx_quantize_cols<1>), g, b, 0, s, x, rows, prows, cols, ldx, codes, scales, cpitch, spitch);
  else
    hipLaunchKernelGGL((k_mx_quantize_cols<0>), g, b, 0, s, x, rows, prows, cols, ldx, codes, scales, cpitch, spitch);
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

hipError_t launch_kmean(const void* x, int dtype, int64_t T, int64_t C, int64_t ldx, float* mu, hipStream_t s) {
  dim3 g((unsigned)(C / (dtype == 1 ? 8 : 4))), b(KM_THREADS);
  if (dtype == 1) hipLaunchKernelGGL((k_kmean<1>), g, b, 0, s, x, T, C, ldx, mu);
  else hipLaunchKernelGGL((k_kmean<0>), g, b, 0, s, x, T, C, ldx, mu);
  return hipGetLastError();
}

}  // namespace mix
