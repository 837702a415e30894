// Underflow ("dead zone") map of the 4-bit block formats on one operand.
//
// "P1" below is the pchao.org digest of the paper, titled
// "MiX：面向端到端低比特视觉语言模型加速的微反缩放"; citations name its sections and figures.
//
// P1 (逐图理解论文 / figure walk, the underflow-map figure) compares how many key elements each
// 4-bit format codes to zero with 32-element blocks: MXINT4, MXFP4, NVFP4 (its block forced to
// 32) and MiX; the MXFP4 bullet of the key results adds the floor-versus-ceil exponent rule. Per
// column of a [rows, cols] operand (optionally smoothed, fp32(x - mu)) the map counts, for each
// format, the elements that are nonzero on input and decode to zero, plus the nonzero elements.
//
// Every decision is exact. MX and MiX use the quantizers' own thresholds (quant_dev.h). NVFP4
// with 32-element blocks: tensor scale g = amax_T / 2688 (6 * 448), block scale s = the E4M3
// value nearest to 448 amax_b / amax_T (ties to the even code), element zero iff
// |x| / (s g) <= 1/4, i.e. 10752 |x| <= s amax_T; these products of a float32 with small
// integers and E4M3 values have at most 29 significant bits, so the fp64 comparisons are exact.
//
// Three launches, no atomics: per-workgroup maxima of the operand, the map (each workgroup reduces
// those maxima, counts its rows of one 32-column block and stores its sums), and the sum of the
// workgroups' sums per (format, column). The caller's workspace holds both sets of partials.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "quant_dev.h"

namespace mix {

constexpr int UF_KINDS = 7;     // MXINT4, MXFP4 floor, MXFP4 ceil, NVFP4 (32), MiX-4.25b, MiX-4.5b, nonzero
constexpr int UF_UNROLL = 2;    // 64-row steps of a workgroup whose loads are in flight together
constexpr int UF_AMAX_PARTS = 512;

UfPlan uf_plan(int64_t rows, int64_t cols) {
  UfPlan p{};
  if (rows <= 0 || cols <= 0) return p;
  p.cb = cols / 32;
  const int64_t groups = rows * (cols >> 3);
  p.ablocks = std::max<int64_t>(1, std::min<int64_t>((groups + 255) / 256, UF_AMAX_PARTS));
  // about 512 workgroups; a workgroup takes 64 rows of its 32 columns per step
  const int64_t steps = (rows + 63) / 64;
  int64_t gy = std::max<int64_t>(1, std::min<int64_t>((512 + p.cb - 1) / p.cb, steps));
  gy = std::max<int64_t>(gy, (steps + 14) / 15);   // at most 15 steps each (byte-packed sums)
  p.rpw = ((steps + gy - 1) / gy) * 64;
  p.gy = (rows + p.rpw - 1) / p.rpw;
  p.part_off = UF_AMAX_PARTS * 4;
  p.bytes = p.part_off + (((size_t)p.gy * UF_KINDS * cols * 4 + 255) & ~(size_t)255);
  return p;
}

__global__ void __launch_bounds__(256) k_uf_clear(uint32_t* __restrict__ counts, int64_t n, uint32_t* __restrict__ amax) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    counts[i] = 0u;
  if (blockIdx.x == 0 && threadIdx.x == 0) *amax = 0u;
}

template <int DT, int MU>
__device__ __forceinline__ void uf_load(const void* x, int64_t row, int64_t ldx, int64_t col, const float (&mv)[8],
                                        uint32_t (&xb)[8]) {
  load8<DT>(x, row, ldx, col, xb);
  if (MU) {
#pragma unroll
    for (int i = 0; i < 8; i++) xb[i] = f32_bits(__fsub_rn(bits_f32(xb[i]), mv[i]));
  }
}

// Largest magnitude of each workgroup's share of the (smoothed) operand, as the bit pattern of a
// non-negative float, into part[blockIdx.x].
template <int DT, int MU>
__global__ void __launch_bounds__(256) k_uf_amax(const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
                                                  const float* __restrict__ mu, uint32_t* __restrict__ part) {
  const int64_t groups = cols >> 3, total = rows * groups;
  uint32_t m = 0;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total; g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = g / groups, c = (g - row * groups) * 8;
    float mv[8] = {};
    if (MU) {
#pragma unroll
      for (int i = 0; i < 8; i++) mv[i] = mu[c + i];
    }
    uint32_t xb[8];
    uf_load<DT, MU>(x, row, ldx, c, mv, xb);
#pragma unroll
    for (int i = 0; i < 8; i++) m = max(m, xb[i] & 0x7FFFFFFFu);
  }
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  __shared__ uint32_t wm[4];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = max(max(wm[0], wm[1]), max(wm[2], wm[3]));
}

// E4M3 magnitude of code c in 0..126: c 2^-9 below 8, else (8 + (c & 7)) 2^((c >> 3) - 10)
__device__ __forceinline__ double e4m3_mag(int c) {
  return c < 8 ? ldexp((double)c, -9) : ldexp((double)(8 + (c & 7)), (c >> 3) - 10);
}

// E4M3 code nearest to L / T (ties to the even code), L, T > 0 exact fp64 values with L <= 448 T:
// the number of midpoints the quotient rounds past, found by bisection on exact comparisons.
__device__ __forceinline__ int e4m3_nearest(double L, double T) {
  int lo = 0, hi = 126;
  while (lo < hi) {
    const int k = (lo + hi) >> 1;
    const double R = 0.5 * (e4m3_mag(k) + e4m3_mag(k + 1)) * T;
    const bool up = L > R || (L == R && ((k + 1) & 1) == 0);
    if (up) lo = k + 1;
    else hi = k;
  }
  return lo;
}

// NVFP4 zero threshold of a block with scale code sc: an element a is zero iff 10752 a <= s T
// (|x| / (s g) <= 1/4 with g = T / 2688), i.e. a <= the largest float f with 10752 f <= s T. f is
// found from the fp64 quotient and settled by exact comparisons (10752 f and s T have at most 29
// significant bits). s = 0 decodes the whole block to zero.
__device__ __forceinline__ uint32_t nv_zero_threshold(int sc, double T) {
  if (sc == 0) return 0x7FFFFFFFu;
  const double S = e4m3_mag(sc) * T;
  uint32_t f = f32_bits((float)(S / 10752.0));
  if (10752.0 * (double)bits_f32(f) > S) f = f ? f - 1u : 0u;
  else if (10752.0 * (double)bits_f32(f + 1u) <= S) f = f + 1u;
  return f;
}

// Adds one row's decisions for this lane's 8 elements (a quad holds one 32-element block; the
// whole wave must call it, for the quad reductions). A row of zeros (also the padding of inactive
// lanes and of rows past the end) adds nothing.
__device__ __forceinline__ void uf_count_row(const uint32_t (&xb)[8], double T, uint32_t (&cnt)[UF_KINDS][8]) {
  uint32_t lmax = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) lmax = max(lmax, xb[i] & 0x7FFFFFFFu);
  const uint32_t bmax = quad_max_u32(lmax);
  int em;
  uint32_t mm;
  const uint32_t w425 = mix_quant_lane<0>(xb, em, mm);
  const uint32_t w45 = mix_quant_lane<1>(xb, em, mm);
  if (bmax == 0) return;   // an all-zero block has no nonzero element
  const uint32_t t_int4 = exact_f32_bits(1, mx_exponent(bmax, 0) - 3);
  const uint32_t t_ceil = exact_f32_bits(1, mx_exponent(bmax, 1) - 2);
  const int eb = (int)(bmax >> 23);
  const int xf = eb == 0 ? -127 : max(eb - 129, -127);   // floor(log2 amax) - 2, at least -127
  const uint32_t t_floor = exact_f32_bits(1, xf - 2);
  const int sc = e4m3_nearest(448.0 * (double)bits_f32(bmax), T);
  const uint32_t t_nv = nv_zero_threshold(sc, T);
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const uint32_t a = xb[i] & 0x7FFFFFFFu;
    const uint32_t nz = a != 0u;
    cnt[0][i] += nz & (a <= t_int4);
    cnt[1][i] += nz & (a <= t_floor);
    cnt[2][i] += nz & (a <= t_ceil);
    cnt[3][i] += nz & (a <= t_nv);
    cnt[4][i] += nz & (((w425 >> (4 * i)) & 15u) == 7u);
    cnt[5][i] += nz & (((w45 >> (4 * i)) & 15u) == 7u);
    cnt[6][i] += nz;
  }
}

// One workgroup: one 32-column block (a quad of lanes holds a row's block, a lane 8 columns) and
// rows r0 .. r0 + rows_per_wg - 1, 64 per step (wave w, quad q: row r0 + 64 j + 16 w + q). Each lane
// keeps its 8 columns' counts in registers; the 16 quads of a wave and then the 4 waves are summed,
// and the workgroup stores its 7 x 32 sums in part[gy][7][cols]. Workgroup 0 also writes amax.
template <int DT, int MU>
__global__ void __launch_bounds__(256) k_underflow_map(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                        int64_t ldx, const float* __restrict__ mu, int64_t cb,
                                                        int64_t rows_per_wg, const uint32_t* __restrict__ amax_part,
                                                        int nparts, uint32_t* __restrict__ amax,
                                                        uint32_t* __restrict__ part) {
  __shared__ uint32_t red[4][UF_KINDS][32];
  __shared__ uint32_t wm[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t by = blockIdx.x / cb, bx = blockIdx.x - by * cb;
  const int64_t c0 = bx * 32 + (lane & 3) * 8;
  const int64_t r0 = by * rows_per_wg;
  const int64_t r1 = min(rows, r0 + rows_per_wg);
  // the operand's largest magnitude from the per-workgroup maxima
  uint32_t m = 0;
  for (int i = threadIdx.x; i < nparts; i += 256) m = max(m, amax_part[i]);
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if (lane == 0) wm[wave] = m;
  __syncthreads();
  m = max(max(wm[0], wm[1]), max(wm[2], wm[3]));
  if (blockIdx.x == 0 && threadIdx.x == 0) *amax = m;
  const double T = (double)bits_f32(m);
  float mv[8] = {};
  if (MU) {
#pragma unroll
    for (int i = 0; i < 8; i++) mv[i] = mu[c0 + i];
  }
  uint32_t cnt[UF_KINDS][8];
#pragma unroll
  for (int k = 0; k < UF_KINDS; k++)
#pragma unroll
    for (int i = 0; i < 8; i++) cnt[k][i] = 0u;

  const int64_t rq = r0 + 16 * wave + (lane >> 2);
  for (int64_t row = rq; row - rq + r0 < r1; row += 64 * UF_UNROLL) {
    uint32_t xb[UF_UNROLL][8];
#pragma unroll
    for (int u = 0; u < UF_UNROLL; u++) {
      if (row + 64 * u < r1) uf_load<DT, MU>(x, row + 64 * u, ldx, c0, mv, xb[u]);
      else
#pragma unroll
        for (int i = 0; i < 8; i++) xb[u][i] = 0u;
    }
#pragma unroll
    for (int u = 0; u < UF_UNROLL; u++) uf_count_row(xb[u], T, cnt);
  }
  // sum over the 16 quads (lanes with equal lane & 3 hold the same columns), four counts a word:
  // a lane's count is at most rows_per_wg / 64 <= 15, so a byte holds the sum of 16 lanes
  uint32_t pk[UF_KINDS * 2];
#pragma unroll
  for (int k = 0; k < UF_KINDS; k++)
#pragma unroll
    for (int h = 0; h < 2; h++)
      pk[2 * k + h] = cnt[k][4 * h] | (cnt[k][4 * h + 1] << 8) | (cnt[k][4 * h + 2] << 16) | (cnt[k][4 * h + 3] << 24);
#pragma unroll
  for (int j = 0; j < UF_KINDS * 2; j++) {
#pragma unroll
    for (int off = 4; off < 64; off <<= 1) pk[j] += (uint32_t)__shfl_xor((int)pk[j], off, 64);
  }
  if (lane < 4) {
#pragma unroll
    for (int k = 0; k < UF_KINDS; k++)
#pragma unroll
      for (int i = 0; i < 8; i++) red[wave][k][lane * 8 + i] = (pk[2 * k + (i >> 2)] >> (8 * (i & 3))) & 0xFFu;
  }
  __syncthreads();
  if (threadIdx.x < UF_KINDS * 32) {
    const int k = threadIdx.x >> 5, c = threadIdx.x & 31;
    part[(by * UF_KINDS + k) * cols + bx * 32 + c] = red[0][k][c] + red[1][k][c] + red[2][k][c] + red[3][k][c];
  }
}

// counts[i] = sum over the gy workgroup rows of part[.][i], i < 7 cols: a workgroup takes 64
// outputs, its 4 waves every 4th workgroup row, 4 loads in flight per lane
__global__ void __launch_bounds__(256) k_uf_reduce(const uint32_t* __restrict__ part, int64_t gy, int64_t n,
                                                    uint32_t* __restrict__ counts) {
  __shared__ uint32_t red[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t i = (int64_t)blockIdx.x * 64 + lane;
  uint32_t s0 = 0, s1 = 0, s2 = 0, s3 = 0;
  if (i < n) {
    int64_t y = wave;
    for (; y + 12 < gy; y += 16) {
      s0 += part[y * n + i];
      s1 += part[(y + 4) * n + i];
      s2 += part[(y + 8) * n + i];
      s3 += part[(y + 12) * n + i];
    }
    for (; y < gy; y += 4) s0 += part[y * n + i];
  }
  red[wave][lane] = s0 + s1 + s2 + s3;
  __syncthreads();
  if (wave == 0 && i < n) counts[i] = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
}

hipError_t launch_underflow_map(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, const float* mu,
                                uint32_t* counts, float* amax, void* ws, hipStream_t s) {
  const int64_t n = (int64_t)UF_KINDS * cols;
  uint32_t* am = (uint32_t*)amax;
  if (rows == 0) {   // nothing to map: counts and amax are cleared
    hipLaunchKernelGGL(k_uf_clear, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 1024)), dim3(256), 0, s, counts,
                       n, am);
    return hipGetLastError();
  }
  const UfPlan p = uf_plan(rows, cols);
  uint32_t* apart = (uint32_t*)ws;
  uint32_t* part = (uint32_t*)((uint8_t*)ws + p.part_off);
  const unsigned nwg = (unsigned)(p.cb * p.gy);
#define UF_LAUNCH(DT, MU)                                                                                          \
  do {                                                                                                             \
    hipLaunchKernelGGL((k_uf_amax<DT, MU>), dim3((unsigned)p.ablocks), dim3(256), 0, s, x, rows, cols, ldx, mu,    \
                       apart);                                                                                     \
    hipLaunchKernelGGL((k_underflow_map<DT, MU>), dim3(nwg), dim3(256), 0, s, x, rows, cols, ldx, mu, p.cb, p.rpw, \
                       apart, (int)p.ablocks, am, part);                                                           \
  } while (0)
  if (dtype == 1) {
    if (mu) UF_LAUNCH(1, 1);
    else UF_LAUNCH(1, 0);
  } else {
    if (mu) UF_LAUNCH(0, 1);
    else UF_LAUNCH(0, 0);
  }
#undef UF_LAUNCH
  hipLaunchKernelGGL(k_uf_reduce, dim3((unsigned)((n + 63) / 64)), dim3(256), 0, s, part, p.gy, n, counts);
  return hipGetLastError();
}

}  // namespace mix
