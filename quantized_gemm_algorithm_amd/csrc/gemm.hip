// A-MiX x W-MX matrix product for gfx950.
//
// "P1" below is the pchao.org digest of the paper, titled
// "MiX：面向端到端低比特视觉语言模型加速的微反缩放"; citations name its sections and figures.
//
// The method (P1, 方法概览 / method overview, the dual-format bullet and Eq. (6)): activations are
// MiX-coded and weights MX-coded; in each 32-element block dot product the shared MiX mantissa
// and the exponents factor out, leaving per-element shifts of the MX mantissa.
//
// Two kernels compute the same product:
//
// * k_gemm_mfma -- the MI355X path. Each MiX element (1.m)_2 2^(Emax-dE) is written, exactly, as
//   the E4M3 byte (1.m)_2 2^(1-dE) times a per-block power of two 2^(Emax-1); 4 significant bits
//   over 8 binades fit E4M3 without rounding. MXFP4 elements are already E2M1; MXINT4 elements q
//   become the E4M3 byte of q/4. The per-32 powers of two (2^(Emax-1) for A, the E8M0 exponent for
//   B) are exactly the block scales of the gfx950 block-scaled MFMA
//   (v_mfma_scale_f32_16x16x128_f8f6f4), so every product is exact and the MFMA accumulates in
//   fp32. Codes are decoded into LDS once per workgroup tile.
// * k_gemm_eq6 -- Eq. (6) on the vector ALUs: per 8-element sub-block an integer sum
//   T_k = sum s_i Wint_i 2^(7-dE_i), then blk = sum_k (8+m_k) T_k and one exact power-of-two
//   scale 2^(Emax+X-10-c_w) per block, accumulated in fp32. (The power-of-two factor is applied
//   with an integer multiply-add, the vector-ALU form of the shifter.)
//
// Operand layout of v_mfma_scale_f32_16x16x128_f8f6f4 (established on the device): lane
// l = r + 16 g (r < 16, g < 4) supplies row/column r; an FP4 operand holds K elements
// [32 g, 32 g + 32) of that row in 16 bytes, low nibble first; an FP8 operand holds elements
// [16 g, 16 g + 16) in bytes 0..15 and [64 + 16 g, 64 + 16 g + 16) in bytes 16..31; the scale
// operand of lane l is the E8M0 scale of row/column r for K block g. Result register i of lane l
// is C[4 (l >> 4) + i][l & 15].
#include "common.h"
#include "kernels.h"
#include "quant_dev.h"

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

namespace mix {

// ------------------------------------------------------------------ MFMA kernel

constexpr int BM = 128, BN = 128, BK = 128;

template <int A_FMT, int B_FP4>
struct TileRegs {
  uint4 a[2];      // 32 MiX code bytes (2 blocks) of this thread's A row
  uint32_t a_sh[2];
  uint4 b[2];      // 32 MX code bytes of this thread's B row
  uint32_t b_sc[2];
};

// Thread t loads row t >> 1, blocks 2 (t & 1) and 2 (t & 1) + 1 of the K step, for A and B.
template <int A_FMT, int B_FP4>
__device__ __forceinline__ void load_tile(const GemmArgs& g, const uint8_t* ab, const void* ash, const uint8_t* bb,
                                          const uint8_t* bsc, int m0, int n0, int k0, TileRegs<A_FMT, B_FP4>& R) {
  const int t = threadIdx.x;
  const int row = t >> 1, hb = t & 1;
  const int nkb = g.K >> 5;
  const int gm = m0 + row, gn = n0 + row;
#pragma unroll
  for (int q = 0; q < 2; q++) {
    int gb = (k0 >> 5) + 2 * hb + q;
    bool ka = gm < g.M && gb < nkb;
    bool kb = gn < g.N && gb < nkb;
    R.a[q] = ka ? *(const uint4*)(ab + (int64_t)gm * g.a_pitch + (int64_t)gb * 16) : make_uint4(0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u);
    if (A_FMT == 1) R.a_sh[q] = ka ? ((const uint16_t*)ash)[(int64_t)gm * g.a_sh_pitch + gb] : 0u;
    else R.a_sh[q] = ka ? ((const uint8_t*)ash)[(int64_t)gm * g.a_sh_pitch + gb] : 0u;
    R.b[q] = kb ? *(const uint4*)(bb + (int64_t)gn * g.b_pitch + (int64_t)gb * 16) : make_uint4(0, 0, 0, 0);
    R.b_sc[q] = kb ? bsc[(int64_t)gn * g.b_sc_pitch + gb] : 127u;
  }
}

// LDS tile: A as E4M3 [128 rows][128 B] with 16-byte chunk c of row r stored at chunk c ^ (r & 7);
// B as raw FP4 [128][64 B] (chunk c at c ^ (r & 3)) or E4M3 [128][128 B] for MXINT4; scales as
// [g][half][r][i] bytes so that one lane reads the scales of its four 16-row sub-tiles at once.
template <int B_FP4>
struct Smem {
  uint8_t a[BM * BK];
  uint8_t b[B_FP4 ? BN * BK / 2 : BN * BK];
  uint8_t as[4 * 2 * 16 * 4];
  uint8_t bs[4 * 2 * 16 * 4];
};

__device__ __forceinline__ int scale_slot(int row, int g) {
  // row = 64 half + 16 i + r
  int half = row >> 6, i = (row >> 4) & 3, r = row & 15;
  return ((g * 2 + half) * 16 + r) * 4 + i;
}

template <int A_FMT, int B_FP4>
__device__ __forceinline__ void store_tile(Smem<B_FP4>& S, const TileRegs<A_FMT, B_FP4>& R) {
  const int t = threadIdx.x;
  const int row = t >> 1, hb = t & 1;
#pragma unroll
  for (int q = 0; q < 2; q++) {
    const int kb = 2 * hb + q;  // block within the K step
    uint32_t sh = R.a_sh[q];
    uint32_t words[4] = {R.a[q].x, R.a[q].y, R.a[q].z, R.a[q].w};
    uint32_t e[8];
#pragma unroll
    for (int sb = 0; sb < 4; sb++) {
      uint32_t m = A_FMT == 1 ? (sh >> (4 + 3 * sb)) & 7u : (sh >> 4) & 7u;
      mix8_to_e4m3(words[sb], m, e[2 * sb], e[2 * sb + 1]);
    }
    // block kb covers bytes [32 kb, 32 kb + 32) = chunks 2 kb, 2 kb + 1
#pragma unroll
    for (int hc = 0; hc < 2; hc++) {
      int ch = (2 * kb + hc) ^ (row & 7);
      *(uint4*)(S.a + row * BK + ch * 16) = make_uint4(e[4 * hc], e[4 * hc + 1], e[4 * hc + 2], e[4 * hc + 3]);
    }
    S.as[scale_slot(row, kb)] = (uint8_t)((sh & 15u) + 119u);  // E8M0 of 2^(Emax - 1)
    if (B_FP4) {
      int ch = kb ^ (row & 3);
      *(uint4*)(S.b + row * (BK / 2) + ch * 16) = R.b[q];
    } else {
      uint32_t bw[4] = {R.b[q].x, R.b[q].y, R.b[q].z, R.b[q].w};
      uint32_t f[8];
#pragma unroll
      for (int sb = 0; sb < 4; sb++) int4x8_to_e4m3(bw[sb], f[2 * sb], f[2 * sb + 1]);
#pragma unroll
      for (int hc = 0; hc < 2; hc++) {
        int ch = (2 * kb + hc) ^ (row & 7);
        *(uint4*)(S.b + row * BK + ch * 16) = make_uint4(f[4 * hc], f[4 * hc + 1], f[4 * hc + 2], f[4 * hc + 3]);
      }
    }
    S.bs[scale_slot(row, kb)] = (uint8_t)R.b_sc[q];
  }
}

template <int A_FMT, int B_FP4, int C_BF16>
__global__ void __launch_bounds__(256, 2) k_gemm_mfma(GemmArgs g) {
  __shared__ Smem<B_FP4> S;
  const int tiles_n = (g.N + BN - 1) / BN;
  int tile = blockIdx.x, batch = blockIdx.z;
  if (g.causal == 2) {
    // K ranges grow with the row tile: the last row tiles of every batch entry run first
    const int lin = blockIdx.z * gridDim.x + blockIdx.x;
    batch = lin % g.batch;
    tile = gridDim.x - 1 - lin / g.batch;
  }
  const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  if (g.causal == 1 && n0 > m0 + BM - 1) return;
  int kend = g.K;
  if (g.causal == 2) kend = min(g.K, m0 + BM);

  const uint8_t* ab = g.a_codes + (int64_t)batch * g.a_bstride;
  const void* ash = A_FMT == 1 ? (const void*)((const uint16_t*)g.a_shared + (int64_t)batch * g.a_sh_bstride)
                               : (const void*)((const uint8_t*)g.a_shared + (int64_t)batch * g.a_sh_bstride);
  const int bbatch = batch / g.b_group;
  const uint8_t* bb = g.b_codes + (int64_t)bbatch * g.b_bstride;
  const uint8_t* bsc = g.b_scales + (int64_t)bbatch * g.b_sc_bstride;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 15, gq = lane >> 4;

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  TileRegs<A_FMT, B_FP4> R;
  load_tile<A_FMT, B_FP4>(g, ab, ash, bb, bsc, m0, n0, 0, R);
  for (int k0 = 0; k0 < kend; k0 += BK) {
    __syncthreads();
    store_tile<A_FMT, B_FP4>(S, R);
    __syncthreads();
    if (k0 + BK < kend) load_tile<A_FMT, B_FP4>(g, ab, ash, bb, bsc, m0, n0, k0 + BK, R);

    v8i af[4], bf[4];
    int sa[4], sb[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      int row = 64 * wm + 16 * i + r;
      uint4 lo = *(const uint4*)(S.a + row * BK + ((gq) ^ (row & 7)) * 16);
      uint4 hi = *(const uint4*)(S.a + row * BK + ((4 + gq) ^ (row & 7)) * 16);
      af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      sa[i] = S.as[scale_slot(row, gq)];
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
      int row = 64 * wn + 16 * j + r;
      if (B_FP4) {
        uint4 v = *(const uint4*)(S.b + row * (BK / 2) + ((gq) ^ (row & 3)) * 16);
        bf[j] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      } else {
        uint4 lo = *(const uint4*)(S.b + row * BK + ((gq) ^ (row & 7)) * 16);
        uint4 hi = *(const uint4*)(S.b + row * BK + ((4 + gq) ^ (row & 7)) * 16);
        bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      sb[j] = S.bs[scale_slot(row, gq)];
    }
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf[j], acc[i][j], 0, B_FP4 ? 4 : 0, 0,
                                                                      sa[i], 0, sb[j]);
  }

  // epilogue
  const float* rdiv = g.row_div ? g.row_div + (int64_t)batch * g.row_div_bstride : nullptr;
#pragma unroll
  for (int i = 0; i < 4; i++) {
#pragma unroll
    for (int e = 0; e < 4; e++) {
      int m = m0 + 64 * wm + 16 * i + 4 * gq + e;
      if (m >= g.M) continue;
      float dv = rdiv ? rdiv[m] : 1.0f;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        int n = n0 + 64 * wn + 16 * j + r;
        if (n >= g.N) continue;
        float v = acc[i][j][e];
        if (rdiv) v = __fdiv_rn(v, dv);
        int64_t idx = (int64_t)batch * g.c_bstride + (int64_t)m * g.ldc + n;
        if (C_BF16) ((uint16_t*)g.c)[idx] = f32_to_bf16_rne(v);
        else ((float*)g.c)[idx] = v;
      }
    }
  }
}

// ------------------------------------------------------------------ MFMA kernel, 256 x 256 tiles
//
// Each of the 4 waves owns a 128 x 128 sub-tile (8 x 8 MFMAs, 256 fp32 accumulators per lane).
// LDS holds two K steps (double buffer): while the MFMAs consume one, the codes of the next step
// are already in registers and are decoded into the other buffer; one barrier per K step.
// Thread t loads and decodes row t of A and row t of B for each K step.

constexpr int GM = 256, GN = 256;

template <int A_FMT, int B_FP4>
struct BigRegs {
  uint4 a[4];
  uint32_t a_sh[4];
  uint4 b[4];
  uint32_t b_sc[4];
};

template <int B_FP4>
struct BigSmem {
  uint8_t a[2][GM * BK];
  uint8_t b[2][B_FP4 ? GN * BK / 2 : GN * BK];
  uint8_t as[2][GM * 4];
  uint8_t bs[2][GN * 4];
};

// scale byte of (row, K block g) at [g][wave half][r][i] so a lane reads its 8 sub-tiles' scales at once
__device__ __forceinline__ int big_scale_slot(int row, int g) {
  int half = row >> 7, i = (row >> 4) & 7, r = row & 15;
  return ((g * 2 + half) * 16 + r) * 8 + i;
}

template <int A_FMT, int B_FP4>
__device__ __forceinline__ void big_load(const GemmArgs& g, const uint8_t* ab, const void* ash, const uint8_t* bb,
                                         const uint8_t* bsc, int m0, int n0, int k0, BigRegs<A_FMT, B_FP4>& R) {
  const int row = threadIdx.x;
  const int nkb = g.K >> 5;
  const int gm = m0 + row, gn = n0 + row;
  const int kb0 = k0 >> 5;
  const bool am = gm < g.M, bn = gn < g.N;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const int gb = kb0 + q;
    const bool ka = am && gb < nkb, kb = bn && gb < nkb;
    R.a[q] = ka ? *(const uint4*)(ab + (int64_t)gm * g.a_pitch + (int64_t)gb * 16)
                : make_uint4(0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u);
    if (A_FMT == 1) R.a_sh[q] = ka ? ((const uint16_t*)ash)[(int64_t)gm * g.a_sh_pitch + gb] : 0u;
    else R.a_sh[q] = ka ? ((const uint8_t*)ash)[(int64_t)gm * g.a_sh_pitch + gb] : 0u;
    R.b[q] = kb ? *(const uint4*)(bb + (int64_t)gn * g.b_pitch + (int64_t)gb * 16) : make_uint4(0, 0, 0, 0);
    R.b_sc[q] = kb ? bsc[(int64_t)gn * g.b_sc_pitch + gb] : 127u;
  }
}

template <int A_FMT, int B_FP4>
__device__ __forceinline__ void big_store(BigSmem<B_FP4>& S, int buf, const BigRegs<A_FMT, B_FP4>& R) {
  const int row = threadIdx.x;
  uint8_t* sa = S.a[buf] + row * BK;
  uint8_t* sbm = S.b[buf];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    uint32_t sh = R.a_sh[q];
    uint32_t w[4] = {R.a[q].x, R.a[q].y, R.a[q].z, R.a[q].w};
    uint32_t e[8];
#pragma unroll
    for (int sb = 0; sb < 4; sb++) {
      uint32_t m = A_FMT == 1 ? (sh >> (4 + 3 * sb)) & 7u : (sh >> 4) & 7u;
      mix8_to_e4m3(w[sb], m, e[2 * sb], e[2 * sb + 1]);
    }
#pragma unroll
    for (int hc = 0; hc < 2; hc++) {
      int ch = (2 * q + hc) ^ (row & 7);
      *(uint4*)(sa + ch * 16) = make_uint4(e[4 * hc], e[4 * hc + 1], e[4 * hc + 2], e[4 * hc + 3]);
    }
    S.as[buf][big_scale_slot(row, q)] = (uint8_t)((sh & 15u) + 119u);
    if (B_FP4) {
      int ch = q ^ ((row >> 1) & 3);
      *(uint4*)(sbm + row * (BK / 2) + ch * 16) = R.b[q];
    } else {
      uint32_t bw[4] = {R.b[q].x, R.b[q].y, R.b[q].z, R.b[q].w};
      uint32_t f[8];
#pragma unroll
      for (int sb = 0; sb < 4; sb++) int4x8_to_e4m3(bw[sb], f[2 * sb], f[2 * sb + 1]);
#pragma unroll
      for (int hc = 0; hc < 2; hc++) {
        int ch = (2 * q + hc) ^ (row & 7);
        *(uint4*)(sbm + row * BK + ch * 16) = make_uint4(f[4 * hc], f[4 * hc + 1], f[4 * hc + 2], f[4 * hc + 3]);
      }
    }
    S.bs[buf][big_scale_slot(row, q)] = (uint8_t)R.b_sc[q];
  }
}

// Tile order: workgroups are dispatched round-robin over the 8 XCDs (workgroup b on XCD b % 8);
// give each XCD a contiguous range of tiles and walk M fastest, so the workgroups resident on one
// XCD share B columns in its L2.
__device__ __forceinline__ int xcd_tile(int bid, int nt) {
  const int x = bid & 7, idx = bid >> 3;
  const int base = nt >> 3, rem = nt & 7;
  return x * base + min(x, rem) + idx;
}

template <int A_FMT, int B_FP4, int C_BF16>
__global__ void __launch_bounds__(256, 1) k_gemm_mfma_big(GemmArgs g) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  BigSmem<B_FP4>& S = *reinterpret_cast<BigSmem<B_FP4>*>(smem_raw);
  const int tiles_m = (g.M + GM - 1) / GM, tiles_n = (g.N + GN - 1) / GN;
  const int t = xcd_tile(blockIdx.x, tiles_m * tiles_n);
  const int tn = t / tiles_m, tm = t - tn * tiles_m;
  const int m0 = tm * GM, n0 = tn * GN;
  const int batch = blockIdx.z;
  if (g.causal == 1 && n0 > m0 + GM - 1) return;
  int kend = g.K;
  if (g.causal == 2) kend = min(g.K, m0 + GM);

  const uint8_t* ab = g.a_codes + (int64_t)batch * g.a_bstride;
  const void* ash = A_FMT == 1 ? (const void*)((const uint16_t*)g.a_shared + (int64_t)batch * g.a_sh_bstride)
                               : (const void*)((const uint8_t*)g.a_shared + (int64_t)batch * g.a_sh_bstride);
  const int bbatch = batch / g.b_group;
  const uint8_t* bb = g.b_codes + (int64_t)bbatch * g.b_bstride;
  const uint8_t* bsc = g.b_scales + (int64_t)bbatch * g.b_sc_bstride;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 15, gq = lane >> 4;

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < 8; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int nk = (kend + BK - 1) / BK;
  BigRegs<A_FMT, B_FP4> R;
  big_load<A_FMT, B_FP4>(g, ab, ash, bb, bsc, m0, n0, 0, R);
  big_store<A_FMT, B_FP4>(S, 0, R);
  __syncthreads();
  for (int kt = 0; kt < nk; kt++) {
    const int cur = kt & 1;
    if (kt + 1 < nk) big_load<A_FMT, B_FP4>(g, ab, ash, bb, bsc, m0, n0, (kt + 1) * BK, R);
    const uint8_t* sa = S.a[cur];
    const uint8_t* sbm = S.b[cur];
    // B fragments and scales of this wave's 8 column sub-tiles
    v8i bf[8];
    const uint2 bsw = *(const uint2*)(S.bs[cur] + ((gq * 2 + wn) * 16 + r) * 8);
    const uint2 asw = *(const uint2*)(S.as[cur] + ((gq * 2 + wm) * 16 + r) * 8);
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int row = 128 * wn + 16 * j + r;
      if (B_FP4) {
        uint4 v = *(const uint4*)(sbm + row * (BK / 2) + (gq ^ ((row >> 1) & 3)) * 16);
        bf[j] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      } else {
        uint4 lo = *(const uint4*)(sbm + row * BK + (gq ^ (row & 7)) * 16);
        uint4 hi = *(const uint4*)(sbm + row * BK + ((4 + gq) ^ (row & 7)) * 16);
        bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    }
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int row = 128 * wm + 16 * i + r;
      uint4 lo = *(const uint4*)(sa + row * BK + (gq ^ (row & 7)) * 16);
      uint4 hi = *(const uint4*)(sa + row * BK + ((4 + gq) ^ (row & 7)) * 16);
      v8i af = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const int sa_i = (int)(((i < 4 ? asw.x : asw.y) >> (8 * (i & 3))) & 0xFFu);
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int sb_j = (int)(((j < 4 ? bsw.x : bsw.y) >> (8 * (j & 3))) & 0xFFu);
        // the B fragment is the MFMA's A operand, so result register e of lane l holds
        // C[m = l & 15][n = 4 (l >> 4) + e]: four consecutive outputs of one row
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, acc[i][j], B_FP4 ? 4 : 0, 0, 0, sb_j,
                                                                      0, sa_i);
      }
    }
    if (kt + 1 < nk) big_store<A_FMT, B_FP4>(S, cur ^ 1, R);
    __syncthreads();
  }

  const float* rdiv = g.row_div ? g.row_div + (int64_t)batch * g.row_div_bstride : nullptr;
  const bool vec_ok = (g.ldc % 4) == 0 && (g.c_bstride % 4) == 0 && (((uintptr_t)g.c) & 15) == 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int m = m0 + 128 * wm + 16 * i + r;
    if (m >= g.M) continue;
    const float dv = rdiv ? rdiv[m] : 1.0f;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int n = n0 + 128 * wn + 16 * j + 4 * gq;
      if (n >= g.N) continue;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; e++) v[e] = rdiv ? __fdiv_rn(acc[i][j][e], dv) : acc[i][j][e];
      const int64_t idx = (int64_t)batch * g.c_bstride + (int64_t)m * g.ldc + n;
      if (vec_ok && n + 4 <= g.N) {
        if (C_BF16)
          *(uint2*)((uint16_t*)g.c + idx) =
              make_uint2((uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16),
                         (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16));
        else
          *(float4*)((float*)g.c + idx) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; e++) {
          if (n + e >= g.N) break;
          if (C_BF16) ((uint16_t*)g.c)[idx + e] = f32_to_bf16_rne(v[e]);
          else ((float*)g.c)[idx + e] = v[e];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ Eq. (6) vector-ALU kernel

constexpr int EM = 64, EN = 64;

template <int A_FMT, int B_FP4, int C_BF16>
__global__ void __launch_bounds__(256) k_gemm_eq6(GemmArgs g) {
  // per K block: A as s*2^(7-dE) (int16) [32][64], B as Wint (int16) [32][64], k-major
  __shared__ int16_t sa[32][EM];
  __shared__ int16_t sb[32][EN];
  __shared__ int sam[EM][4];  // 8 + m_k
  __shared__ int sae[EM];     // Emax
  __shared__ int sbe[EN];     // X (g16: of the block's first half)
  __shared__ int sbe1[EN];    // g16: X of the second half
  const int tiles_n = (g.N + EN - 1) / EN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int m0 = tm * EM, n0 = tn * EN;
  const int batch = blockIdx.z;
  if (g.causal == 1 && n0 > m0 + EM - 1) return;
  int kend = g.K;
  if (g.causal == 2) kend = min(g.K, m0 + EM);
  const uint8_t* ab = g.a_codes + (int64_t)batch * g.a_bstride;
  const int bbatch = batch / g.b_group;
  const uint8_t* bb = g.b_codes + (int64_t)bbatch * g.b_bstride;
  const uint8_t* bsc = g.b_scales + (int64_t)bbatch * g.b_sc_bstride;
  const int cw = B_FP4 ? 1 : 2;

  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;  // thread owns rows 4 ty .. +3, cols 4 tx .. +3
  float acc[4][4] = {};
  const int nkb = g.K >> 5;
  for (int k0 = 0; k0 < kend; k0 += 32) {
    const int gb = k0 >> 5;
    __syncthreads();
    {  // 64 rows x 16 bytes of A and of B: thread -> (row = tid >> 2, 4-byte word tid & 3)
      int row = tid >> 2, wd = tid & 3;
      int gm = m0 + row, gn = n0 + row;
      uint32_t aw = 0x77777777u, bw = 0;
      uint32_t sh = 0;
      if (gm < g.M && gb < nkb) {
        aw = *(const uint32_t*)(ab + (int64_t)gm * g.a_pitch + gb * 16 + wd * 4);
        sh = A_FMT == 1 ? ((const uint16_t*)g.a_shared)[(int64_t)batch * g.a_sh_bstride + (int64_t)gm * g.a_sh_pitch + gb]
                        : ((const uint8_t*)g.a_shared)[(int64_t)batch * g.a_sh_bstride + (int64_t)gm * g.a_sh_pitch + gb];
      }
      int X = 0, X1 = 0;
      if (gn < g.N && gb < nkb) {
        bw = *(const uint32_t*)(bb + (int64_t)gn * g.b_pitch + gb * 16 + wd * 4);
        if (g.b_g16) {
          X = (int)bsc[(int64_t)gn * g.b_sc_pitch + 2 * gb] - 127;
          X1 = (int)bsc[(int64_t)gn * g.b_sc_pitch + 2 * gb + 1] - 127;
        } else {
          X = X1 = (int)bsc[(int64_t)gn * g.b_sc_pitch + gb] - 127;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; e++) {
        uint32_t na = (aw >> (4 * e)) & 15u, nb = (bw >> (4 * e)) & 15u;
        int av;
        if (na == 0x7) av = 0;
        else if (na == 0xF) av = 1;
        else av = (na & 8) ? -(1 << (7 - (int)(na & 7))) : (1 << (7 - (int)(na & 7)));
        int wv;
        if (B_FP4) {
          const int tab[8] = {0, 1, 2, 3, 4, 6, 8, 12};
          wv = (nb & 8) ? -tab[nb & 7] : tab[nb & 7];
        } else {
          wv = nb >= 8 ? (int)nb - 16 : (int)nb;
        }
        sa[wd * 8 + e][row] = (int16_t)av;
        sb[wd * 8 + e][row] = (int16_t)wv;
      }
      if (wd == 0) {
        sae[row] = (int)(sh & 15u) - 7;
        sbe[row] = X;
        sbe1[row] = X1;
#pragma unroll
        for (int k = 0; k < 4; k++) sam[row][k] = 8 + (int)(A_FMT == 1 ? (sh >> (4 + 3 * k)) & 7u : (sh >> 4) & 7u);
      }
    }
    __syncthreads();
    // the block sum of Eq. (6), split by weight half: sub-blocks 0-1 and 2-3 (one weight exponent
    // each for g16 weights; the same one otherwise)
    int blk[4][4] = {}, blk1[4][4] = {};
#pragma unroll
    for (int k = 0; k < 4; k++) {
      int T[4][4] = {};
#pragma unroll
      for (int e = 0; e < 8; e++) {
        int a[4], w[4];
#pragma unroll
        for (int i = 0; i < 4; i++) a[i] = sa[k * 8 + e][4 * ty + i];
#pragma unroll
        for (int j = 0; j < 4; j++) w[j] = sb[k * 8 + e][4 * tx + j];
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
          for (int j = 0; j < 4; j++) T[i][j] += a[i] * w[j];
      }
#pragma unroll
      for (int i = 0; i < 4; i++) {
        int mk = sam[4 * ty + i][k];
#pragma unroll
        for (int j = 0; j < 4; j++) {
          if (k < 2) blk[i][j] += mk * T[i][j];
          else blk1[i][j] += mk * T[i][j];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if (g.b_g16) {
          acc[i][j] += ldexpf((float)blk[i][j], sae[4 * ty + i] + sbe[4 * tx + j] - 10 - cw);
          acc[i][j] += ldexpf((float)blk1[i][j], sae[4 * ty + i] + sbe1[4 * tx + j] - 10 - cw);
        } else {
          acc[i][j] += ldexpf((float)(blk[i][j] + blk1[i][j]), sae[4 * ty + i] + sbe[4 * tx + j] - 10 - cw);
        }
      }
  }
  const float* rdiv = g.row_div ? g.row_div + (int64_t)batch * g.row_div_bstride : nullptr;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    int m = m0 + 4 * ty + i;
    if (m >= g.M) continue;
    float dv = rdiv ? rdiv[m] : 1.0f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      int n = n0 + 4 * tx + j;
      if (n >= g.N) continue;
      float v = acc[i][j];
      if (rdiv) v = __fdiv_rn(v, dv);
      int64_t idx = (int64_t)batch * g.c_bstride + (int64_t)m * g.ldc + n;
      if (C_BF16) ((uint16_t*)g.c)[idx] = f32_to_bf16_rne(v);
      else ((float*)g.c)[idx] = v;
    }
  }
}

// ------------------------------------------------------------------ launchers

#define DISPATCH3(KERN, GRID, BLOCK, ...)                                                        \
  do {                                                                                           \
    if (a_fmt) {                                                                                 \
      if (b_fp4) { if (c_bf16) hipLaunchKernelGGL((KERN<1, 1, 1>), GRID, BLOCK, 0, s, __VA_ARGS__); \
                   else hipLaunchKernelGGL((KERN<1, 1, 0>), GRID, BLOCK, 0, s, __VA_ARGS__); }       \
      else { if (c_bf16) hipLaunchKernelGGL((KERN<1, 0, 1>), GRID, BLOCK, 0, s, __VA_ARGS__);        \
             else hipLaunchKernelGGL((KERN<1, 0, 0>), GRID, BLOCK, 0, s, __VA_ARGS__); }             \
    } else {                                                                                     \
      if (b_fp4) { if (c_bf16) hipLaunchKernelGGL((KERN<0, 1, 1>), GRID, BLOCK, 0, s, __VA_ARGS__); \
                   else hipLaunchKernelGGL((KERN<0, 1, 0>), GRID, BLOCK, 0, s, __VA_ARGS__); }       \
      else { if (c_bf16) hipLaunchKernelGGL((KERN<0, 0, 1>), GRID, BLOCK, 0, s, __VA_ARGS__);        \
             else hipLaunchKernelGGL((KERN<0, 0, 0>), GRID, BLOCK, 0, s, __VA_ARGS__); }             \
    }                                                                                            \
  } while (0)

template <int A_FMT, int B_FP4, int C_BF16>
static hipError_t launch_big(const GemmArgs& g, hipStream_t s) {
  const size_t lds = sizeof(BigSmem<B_FP4>);
  static bool attr_set = false;  // raise the dynamic LDS limit once per instantiation
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k_gemm_mfma_big<A_FMT, B_FP4, C_BF16>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  int tiles = ((g.M + GM - 1) / GM) * ((g.N + GN - 1) / GN);
  hipLaunchKernelGGL((k_gemm_mfma_big<A_FMT, B_FP4, C_BF16>), dim3(tiles, 1, g.batch), dim3(256), lds, s, g);
  return hipGetLastError();
}

hipError_t launch_gemm_mfma(int a_fmt, int b_fp4, int c_bf16, const GemmArgs& g, hipStream_t s) {
  if (g.M >= GM && g.N >= GN) {
    if (a_fmt) {
      if (b_fp4) return c_bf16 ? launch_big<1, 1, 1>(g, s) : launch_big<1, 1, 0>(g, s);
      return c_bf16 ? launch_big<1, 0, 1>(g, s) : launch_big<1, 0, 0>(g, s);
    }
    if (b_fp4) return c_bf16 ? launch_big<0, 1, 1>(g, s) : launch_big<0, 1, 0>(g, s);
    return c_bf16 ? launch_big<0, 0, 1>(g, s) : launch_big<0, 0, 0>(g, s);
  }
  int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  dim3 grid(tiles, 1, g.batch), block(256);
  DISPATCH3(k_gemm_mfma, grid, block, g);
  return hipGetLastError();
}

hipError_t launch_gemm_eq6(int a_fmt, int b_fp4, int c_bf16, const GemmArgs& g, hipStream_t s) {
  int tiles = ((g.M + EM - 1) / EM) * ((g.N + EN - 1) / EN);
  dim3 grid(tiles, 1, g.batch), block(256);
  DISPATCH3(k_gemm_eq6, grid, block, g);
  return hipGetLastError();
}

}  // namespace mix
