// The GEMM B image of g16 weights: MXINT4g16 / MXFP4g16, one shared exponent per 16 elements.
//
// "P1" below is the pchao.org digest of the paper, titled
// "MiX：面向端到端低比特视觉语言模型加速的微反缩放"; citations name its sections and figures.
//
// P1 (实验如何设计 / experiment design, the format bullet) lists the 4.5-bit "g16" weight
// variants; MiX-INT4g16 pairs MiX-4.5b activations with MXINT4g16 weights. The block-scaled MFMA
// takes one E8M0 scale per 32 K elements, so the two 16-element halves of a 32-block share one
// scale 2^b here and each half's own exponent X_h moves into its elements: an element v 2^X_h is
// stored as the E4M3 byte of v 2^(X_h - b). An MXINT4 element q 2^(X_h - 2) (|q| <= 7, three
// significant bits) is the E4M3 value |q| 2^(d - 2) with d = X_h - b, representable for d - 2 in
// [-9, 6] (down to the subnormal step 2^-9, up to 7 * 2^6 = 448, the largest E4M3); an MXFP4
// element (E2M1 magnitude k/2, k in {0, 1, 2, 3, 4, 6, 8, 12}) is k 2^(d - 1), representable for
// d - 1 in [-9, 5] (12 * 2^5 = 384). So a block folds exactly when its halves' exponents differ by
// at most 15 (MXINT4g16) or 14 (MXFP4g16): b is the smaller exponent (MXINT4g16) or the larger
// (MXFP4g16) when they differ by at most 8, otherwise the value that keeps both halves in range.
// A block beyond that (one half more than 2^14 times smaller than the other, never seen in
// Gaussian weights) cannot be folded exactly: its unrepresentable elements are stored as zero and
// the block is counted, so the caller knows whether this image gives the exact product (the
// Eq. (6) path is exact for every input). The image layout is the MXINT4 one (f8_image.h): the
// permuted per-32 scales, E4M3 bytes, scales per 16-row group.
#include "common.h"
#include "f8_image.h"
#include "kernels.h"

namespace mix {

// E4M3 byte of (-1)^neg k 2^E (k <= 15), or ok = false if that value is not an E4M3 number.
// In units of the smallest subnormal 2^-9 the value is t = k 2^(E+9): subnormal when t < 8,
// otherwise normal with exponent field p - 2 (p = floor(log2 t)) and mantissa t / 2^(p-3) - 8.
__device__ __forceinline__ uint32_t e4m3_exact(uint32_t k, int E, uint32_t neg, bool& ok) {
  if (k == 0) return 0u;
  const int sh = E + 9;
  uint32_t t;
  if (sh >= 0) {
    if (sh > 20) { ok = false; return 0u; }
    t = k << sh;
  } else {
    if (sh < -4 || (k & ((1u << -sh) - 1u))) { ok = false; return 0u; }
    t = k >> -sh;
  }
  uint32_t byte;
  if (t < 8) {
    byte = t;
  } else {
    const int p = 31 - __builtin_clz(t);
    const int field = p - 2;
    const uint32_t m = (t >> (p - 3)) - 8u;
    if ((t & ((1u << (p - 3)) - 1u)) || field > 15 || (field == 15 && m == 7u)) { ok = false; return 0u; }
    byte = ((uint32_t)field << 3) | m;
  }
  return byte | (neg << 7);
}

// One thread per 32-element block of a weight row: the folded scale into both scale layouts and
// 32 E4M3 bytes.
template <int FP4>
__global__ void __launch_bounds__(256) k_expand_b_g16(const uint8_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ sc16, int64_t N, int64_t K,
                                                       int tiles_n, uint8_t* __restrict__ bs_p,
                                                       uint8_t* __restrict__ b8, uint8_t* __restrict__ bs_v,
                                                       uint32_t* __restrict__ unfoldable) {
  const int64_t nb = K >> 5;
  const int64_t total = N * nb;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total; g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = g / nb, blk = g - row * nb;
    const int s0 = sc16[row * (K >> 4) + 2 * blk], s1 = sc16[row * (K >> 4) + 2 * blk + 1];
    // base E8M0 byte; a zero half (scale byte 0, codes 0) places no constraint
    int base;
    if (s0 == 0 || s1 == 0) {
      base = s0 + s1;
    } else {
      const int lo = min(s0, s1), hi = max(s0, s1);
      base = FP4 ? min(hi, lo + 8) : max(lo, hi - 8);
    }
    const uint4 w = *(const uint4*)(codes + row * (K >> 1) + blk * 16);
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
    uint32_t out[8];
    bool ok = true;
#pragma unroll
    for (int e = 0; e < 32; e++) {
      const uint32_t nib = (wv[e >> 3] >> (4 * (e & 7))) & 15u;
      const int sh = e < 16 ? s0 : s1;
      uint32_t byte;
      if (FP4) {
        const uint32_t kk = (0xC8643210ull >> (4 * (nib & 7))) & 15u;   // 2 x E2M1 magnitude
        byte = e4m3_exact(kk, -1 - (base - sh), nib >> 3, ok);
      } else {
        const int q = nib >= 8 ? (int)nib - 16 : (int)nib;
        byte = e4m3_exact((uint32_t)(q < 0 ? -q : q), (sh - base) - 2, q < 0 ? 1u : 0u, ok);
      }
      if ((e & 3) == 0) out[e >> 2] = 0;
      out[e >> 2] |= byte << (8 * (e & 3));
    }
    uint8_t* dst = b8 + row * K + blk * 32;
    *(uint4*)dst = make_uint4(out[0], out[1], out[2], out[3]);
    *(uint4*)(dst + 16) = make_uint4(out[4], out[5], out[6], out[7]);
    const int64_t st = blk >> 2, tile = row / FT;
    bs_p[(st * tiles_n + tile) * 1024 + f8_scale_pos((int)(row % FT), (int)(blk & 3))] = (uint8_t)base;
    bs_v[((row >> 4) * (K >> 7) + st) * 64 + (row & 15) * 4 + (blk & 3)] = (uint8_t)base;
    if (!ok) atomicAdd(unfoldable, 1u);
  }
}

__global__ void k_clear_u32(uint32_t* p) {
  if (threadIdx.x == 0) *p = 0u;
}

hipError_t launch_gemm_b_image_g16(int fp4, const uint8_t* b_codes, const uint8_t* b_scales16, int64_t N, int64_t K,
                                   void* img, uint32_t* unfoldable, hipStream_t s) {
  const F8BImage L = f8_b_image_layout(0, N, K);
  uint8_t* base = (uint8_t*)img;
  const int tiles_n = (int)((N + FT - 1) / FT);
  // the counter is cleared by a kernel, not a memset node, so the call can also be captured in a graph
  hipLaunchKernelGGL(k_clear_u32, dim3(1), dim3(64), 0, s, unfoldable);
  int64_t blocks = (N * (K >> 5) + 255) / 256;
  if (blocks > 65535 * 4) blocks = 65535 * 4;
  if (fp4)
    hipLaunchKernelGGL(k_expand_b_g16<1>, dim3((unsigned)blocks), dim3(256), 0, s, b_codes, b_scales16, N, K, tiles_n,
                       base + L.bs_p, base + L.b8, base + L.bs_v, unfoldable);
  else
    hipLaunchKernelGGL(k_expand_b_g16<0>, dim3((unsigned)blocks), dim3(256), 0, s, b_codes, b_scales16, N, K, tiles_n,
                       base + L.bs_p, base + L.b8, base + L.bs_v, unfoldable);
  return hipGetLastError();
}

}  // namespace mix
