// Fast A-MiX x W-MX product: a decode pass, then an MXFP8 x MX{FP4,FP8} block-scaled MFMA GEMM.
//
// P1 (method overview, the dual-format bullet and Eq. (6)) factors the shared MiX mantissa out of
// each block sum. On MI355X the exact multiplier is the matrix core. Each MiX element
// (1.m)_2 2^(Emax-dE) is exactly the E4M3 byte (1.m)_2 2^(1-dE) times the block power of two
// 2^(Emax-1). That power of two is an E8M0 block scale of v_mfma_scale_f32_32x32x64_f8f6f4, so
// the product is exact and the MFMA accumulates in fp32.
//
// Decoding codes into MFMA operands inside the GEMM would repeat the work once per tile column
// (74 times for a 4096 x 18944 x 3584 product). So the codes are decoded once by k_expand_a into
// a workspace: E4M3 bytes [M, K] plus E8M0 scales laid out per 128-wide K step, [K/128][M][4].
// MXINT4 weights become E4M3 bytes of q/4 (k_expand_b_int4), which keeps their E8M0 scales
// unchanged. MXFP4 weights are used as stored: the E2M1 nibbles are the FP4 MFMA operand.
//
// The GEMM streams both operands global->LDS with global_load_lds_dwordx4 (no registers, no VALU).
// It uses 256 x 256 tiles, 4 waves of 128 x 128 (4 x 4 MFMAs of 32 x 32 per 64-wide K half, 256
// fp32 accumulators per lane), and an NS-stage LDS ring with one barrier per 128-wide K step.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 operand layout (established on the device): lane
// l = r + 32 g (r < 32, g < 2) supplies row/column r. An FP8 operand holds K elements
// [16 g, 16 g + 16) in bytes 0..15 and [32 + 16 g, 32 + 16 g + 16) in bytes 16..31. An FP4
// operand holds [32 g, 32 g + 32) in 16 bytes, low nibble first. The scale of lane l is the E8M0
// scale of row/column r for K block g. Result register k of lane l is
// C[8 (k >> 2) + 4 (l >> 5) + (k & 3)][l & 31].
#include "common.h"
#include "kernels.h"
#include "quant_dev.h"

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

namespace mix {

// ------------------------------------------------------------------ decode passes

// One lane per 8-element sub-block: 4 code bytes -> 8 E4M3 bytes. Quad lane 0 writes the block's
// E8M0 scale 2^(Emax-1) into the per-K-step layout [K/128][M][4].
template <int A_FMT>
__global__ void __launch_bounds__(256) k_expand_a(const uint8_t* __restrict__ codes, const void* __restrict__ shared,
                                                   int64_t M, int64_t K, uint8_t* __restrict__ a8,
                                                   uint8_t* __restrict__ as_t) {
  const int64_t sub_per_row = K >> 3;
  const int64_t total = M * sub_per_row;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total; g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = g / sub_per_row;
    const int64_t sb = g - row * sub_per_row;
    const int64_t blk = sb >> 2;
    const uint32_t w = *(const uint32_t*)(codes + row * (K >> 1) + sb * 4);
    const uint32_t sh = A_FMT == 1 ? ((const uint16_t*)shared)[row * (K >> 5) + blk]
                                   : ((const uint8_t*)shared)[row * (K >> 5) + blk];
    const uint32_t m = A_FMT == 1 ? (sh >> (4 + 3 * (sb & 3))) & 7u : (sh >> 4) & 7u;
    uint32_t e0, e1;
    mix8_to_e4m3(w, m, e0, e1);
    *(uint2*)(a8 + row * K + sb * 8) = make_uint2(e0, e1);
    if ((sb & 3) == 0) as_t[((blk >> 2) * M + row) * 4 + (blk & 3)] = (uint8_t)((sh & 15u) + 119u);
  }
}

// MXINT4 codes [N, K/2] -> E4M3 bytes of q/4 [N, K] (scales unchanged).
__global__ void __launch_bounds__(256) k_expand_b_int4(const uint8_t* __restrict__ codes, int64_t N, int64_t K,
                                                        uint8_t* __restrict__ b8) {
  const int64_t total = N * (K >> 3);
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total; g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = g / (K >> 3), sb = g - row * (K >> 3);
    const uint32_t w = *(const uint32_t*)(codes + row * (K >> 1) + sb * 4);
    uint32_t e0, e1;
    int4x8_to_e4m3(w, e0, e1);
    *(uint2*)(b8 + row * K + sb * 8) = make_uint2(e0, e1);
  }
}

// ------------------------------------------------------------------ GEMM

constexpr int FT = 256;   // tile M = tile N
constexpr int FK = 128;   // K per stage

template <int B_FP4>
struct F8Stage {
  static constexpr int A_BYTES = FT * FK;                          // E4M3 A, 128 B per row
  static constexpr int B_BYTES = B_FP4 ? FT * FK / 2 : FT * FK;    // FP4 (64 B/row) or E4M3 B
  static constexpr int AS_OFF = A_BYTES + B_BYTES;
  static constexpr int BS_OFF = AS_OFF + FT * 4;
  static constexpr int BYTES = BS_OFF + FT * 4;
};

struct F8Args {
  const uint8_t* a8;      // [M, K] E4M3
  const uint8_t* as_t;    // [K/128][M][4] E8M0
  const uint8_t* b;       // [N, K/2] FP4 codes or [N, K] E4M3
  const uint8_t* bs;      // [N, K/32] E8M0
  void* c;
  int64_t ldc;
  const float* row_div;
  int M, N, K;
};

__device__ __forceinline__ int f8_xcd_tile(int bid, int nt) {
  const int x = bid & 7, idx = bid >> 3;
  const int base = nt >> 3, rem = nt & 7;
  return x * base + min(x, rem) + idx;
}

// global -> LDS copies (global_load_lds_dword[x4]): lane i's bytes land at LDS byte
// m0 + size * i. The copy has no destination register; it is written as a statement so that the
// compiler does not drain every outstanding copy before each LDS read of another stage -- the
// kernel waits for its copies explicitly (vmcnt) before the barrier that publishes a stage.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(gptr) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_base), "v"(gptr) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t)p;
}

// Issue the global->LDS copies of one K step into stage buffer `st`. Every wave issues the same
// number of copy instructions (f8_loads_per_stage), so per-wave vmcnt arithmetic is a constant.
template <int B_FP4>
__device__ __forceinline__ void f8_issue(const F8Args& g, uint8_t* st, int m0, int n0, int k0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // A: 2048 16-byte chunks; chunk q lands at LDS byte 16 q; q -> (row q/8, slot q%8) holding
  // logical chunk slot ^ (row & 7) of that row.
#pragma unroll
  for (int p = 0; p < 8; p++) {
    const int q = p * 256 + wave * 64 + lane;
    const int row = q >> 3, slot = q & 7;
    const int c = slot ^ (row & 7);
    const int grow = min(m0 + row, g.M - 1);
    const uint8_t* src = g.a8 + (int64_t)grow * g.K + k0 + 16 * c;
    dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(st + (p * 256 + wave * 64) * 16)));
  }
  if (B_FP4) {
    // B: 1024 chunks of 16 B; (row q/4, slot q%4) holds logical chunk slot ^ ((row >> 1) & 3)
#pragma unroll
    for (int p = 0; p < 4; p++) {
      const int q = p * 256 + wave * 64 + lane;
      const int row = q >> 2, slot = q & 3;
      const int c = slot ^ ((row >> 1) & 3);
      const int grow = min(n0 + row, g.N - 1);
      const uint8_t* src = g.b + (int64_t)grow * (g.K >> 1) + (k0 >> 1) + 16 * c;
      dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(st + F8Stage<B_FP4>::A_BYTES + (p * 256 + wave * 64) * 16)));
    }
  } else {
#pragma unroll
    for (int p = 0; p < 8; p++) {
      const int q = p * 256 + wave * 64 + lane;
      const int row = q >> 3, slot = q & 7;
      const int c = slot ^ (row & 7);
      const int grow = min(n0 + row, g.N - 1);
      const uint8_t* src = g.b + (int64_t)grow * g.K + k0 + 16 * c;
      dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(st + F8Stage<B_FP4>::A_BYTES + (p * 256 + wave * 64) * 16)));
    }
  }
  // scales: 4 bytes per row; wave w copies rows 64 w .. 64 w + 63
  {
    const int row = wave * 64 + lane;
    const int ga = min(m0 + row, g.M - 1);
    const uint8_t* sa = g.as_t + ((int64_t)(k0 >> 7) * g.M + ga) * 4;
    dma4(sa, __builtin_amdgcn_readfirstlane(lds_addr(st + F8Stage<B_FP4>::AS_OFF + wave * 256)));
    const int gb = min(n0 + row, g.N - 1);
    const uint8_t* sb = g.bs + (int64_t)gb * (g.K >> 5) + (k0 >> 5);
    dma4(sb, __builtin_amdgcn_readfirstlane(lds_addr(st + F8Stage<B_FP4>::BS_OFF + wave * 256)));
  }
}

template <int B_FP4>
constexpr int f8_loads_per_stage() { return 8 + (B_FP4 ? 4 : 8) + 2; }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// One 128-wide K step from stage buffer `st`. The MFMA computes C^T tiles: its A operand is the
// weight tile (rows n), its B operand the activation tile (rows m), so result register k of lane
// l holds C[m = l & 31][n = 8 (k >> 2) + 4 (l >> 5) + (k & 3)] -- four consecutive n per lane,
// which the epilogue writes as 8-byte runs.
template <int B_FP4>
__device__ __forceinline__ void f8_compute(const uint8_t* st, v16f (&acc)[4][4], int wm, int wn, int r, int gq) {
  const uint8_t* sa = st;
  const uint8_t* sbm = st + F8Stage<B_FP4>::A_BYTES;
  const uint8_t* sas = st + F8Stage<B_FP4>::AS_OFF;
  const uint8_t* sbs = st + F8Stage<B_FP4>::BS_OFF;
#pragma unroll
  for (int h = 0; h < 2; h++) {  // 64-wide K halves
    v8i xf[4];  // activation fragments (m sub-tiles)
    int xs[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int row = 128 * wm + 32 * i + r;
      const int c0 = 4 * h + gq, c1 = 4 * h + 2 + gq;
      uint4 lo = *(const uint4*)(sa + row * 128 + ((c0 ^ (row & 7)) * 16));
      uint4 hi = *(const uint4*)(sa + row * 128 + ((c1 ^ (row & 7)) * 16));
      xf[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      xs[i] = sas[row * 4 + 2 * h + gq];
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int row = 128 * wn + 32 * j + r;
      v8i wf;
      if (B_FP4) {
        const int c = 2 * h + gq;
        uint4 v = *(const uint4*)(sbm + row * 64 + ((c ^ ((row >> 1) & 3)) * 16));
        wf = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      } else {
        const int c0 = 4 * h + gq, c1 = 4 * h + 2 + gq;
        uint4 lo = *(const uint4*)(sbm + row * 128 + ((c0 ^ (row & 7)) * 16));
        uint4 hi = *(const uint4*)(sbm + row * 128 + ((c1 ^ (row & 7)) * 16));
        wf = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      const int ws = sbs[row * 4 + 2 * h + gq];
#pragma unroll
      for (int i = 0; i < 4; i++)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf, xf[i], acc[i][j], B_FP4 ? 4 : 0, 0, 0, ws, 0,
                                                                     xs[i]);
    }
  }
}

template <int B_FP4, int C_BF16, int NS>
__global__ void __launch_bounds__(256, 1) k_gemm_f8(F8Args g) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int SB = F8Stage<B_FP4>::BYTES;
  constexpr int LPS = f8_loads_per_stage<B_FP4>();
  const int tiles_m = (g.M + FT - 1) / FT, tiles_n = (g.N + FT - 1) / FT;
  const int t = f8_xcd_tile(blockIdx.x, tiles_m * tiles_n);
  const int tn = t / tiles_m, tm = t - tn * tiles_m;
  const int m0 = tm * FT, n0 = tn * FT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, gq = lane >> 5;
  const int nk = g.K / FK;

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = v16f{};

  // prologue: steps 0 .. NS-2 in flight
#pragma unroll
  for (int s = 0; s < NS - 1; s++)
    if (s < nk) f8_issue<B_FP4>(g, smem + s * SB, m0, n0, s * FK);

  for (int kt = 0; kt < nk; kt++) {
    // this wave's copies for step kt are complete once only the later steps' copies are pending
    if (NS == 3 && kt + 1 < nk) wait_vmcnt<LPS>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();  // every wave's copies of step kt are in LDS; step kt-1 is consumed
    if (kt + NS - 1 < nk) f8_issue<B_FP4>(g, smem + ((kt + NS - 1) % NS) * SB, m0, n0, (kt + NS - 1) * FK);
    f8_compute<B_FP4>(smem + (kt % NS) * SB, acc, wm, wn, r, gq);
  }

  // Epilogue. Each wave stages its 128 x 128 tile in LDS row-major (row pitch padded by 16 bytes)
  // and writes whole rows with 16-byte stores: 64 lanes cover 4 rows (bf16) or 2 rows (fp32) per
  // instruction. fp32 output goes in two 64-row passes to fit.
  __builtin_amdgcn_s_barrier();  // the last step's operands are consumed before LDS is reused
  constexpr int ES = C_BF16 ? 2 : 4;           // bytes per output element
  constexpr int PASS_ROWS = C_BF16 ? 128 : 64;
  constexpr int PITCH = 128 * ES + 16;
  uint8_t* ep = smem + wave * (PASS_ROWS * PITCH);
  const int mw = m0 + 128 * wm, nw = n0 + 128 * wn;
  const bool vec_ok = (g.ldc % (16 / ES)) == 0 && (((uintptr_t)g.c) & 15) == 0;
#pragma unroll
  for (int pass = 0; pass < 128 / PASS_ROWS; pass++) {
    // registers -> LDS: lane holds C[m = 32 i + r][n = 32 j + 8 (k>>2) + 4 gq + (0..3)]
#pragma unroll
    for (int i = 0; i < 4; i++) {
      if ((32 * i) / PASS_ROWS != pass) continue;
      const int lr = 32 * i + r - pass * PASS_ROWS;
      const int gm = mw + 32 * i + r;
      const float dv = (g.row_div && gm < g.M) ? g.row_div[gm] : 1.0f;
#pragma unroll
      for (int j = 0; j < 4; j++) {
#pragma unroll
        for (int q = 0; q < 4; q++) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; e++) {
            v[e] = acc[i][j][4 * q + e];
            if (g.row_div) v[e] = __fdiv_rn(v[e], dv);
          }
          const int col = 32 * j + 8 * q + 4 * gq;
          if (C_BF16) {
            uint32_t lo = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
            uint32_t hi = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
            *(uint2*)(ep + lr * PITCH + col * 2) = make_uint2(lo, hi);
          } else {
            *(float4*)(ep + lr * PITCH + col * 4) = make_float4(v[0], v[1], v[2], v[3]);
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    // LDS -> global: 16-byte chunks, whole rows
    constexpr int CHUNKS = 128 * ES / 16;           // per row
    constexpr int ROWS_PER_INSTR = 64 / CHUNKS;
#pragma unroll 4
    for (int it = 0; it < PASS_ROWS / ROWS_PER_INSTR; it++) {
      const int lr = it * ROWS_PER_INSTR + lane / CHUNKS;
      const int ch = lane % CHUNKS;
      const int gm = mw + pass * PASS_ROWS + lr;
      const int gn = nw + ch * (16 / ES);
      if (gm >= g.M) continue;
      const uint4 v = *(const uint4*)(ep + lr * PITCH + ch * 16);
      uint8_t* dst = (uint8_t*)g.c + ((int64_t)gm * g.ldc + gn) * ES;
      if (vec_ok && gn + 16 / ES <= g.N) {
        *(uint4*)dst = v;
      } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 16 / ES; e++) {
          if (gn + e >= g.N) break;
          if (C_BF16) ((uint16_t*)dst)[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
          else ((uint32_t*)dst)[e] = w[e];
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ------------------------------------------------------------------ host side

static inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

bool gemm_f8_eligible(int64_t M, int64_t N, int64_t K) { return K > 0 && K % FK == 0 && M >= 64 && N >= FT; }

size_t gemm_f8_ws_bytes(int b_fp4, int64_t M, int64_t N, int64_t K) {
  size_t s = al256((size_t)M * K) + al256((size_t)M * (K / 32));
  if (!b_fp4) s += al256((size_t)N * K);
  return s;
}

// LDS the kernel needs: the stage ring, or the epilogue's per-wave staging if that is larger
template <int B_FP4, int C_BF16, int NS>
constexpr size_t f8_lds_bytes() {
  constexpr size_t ring = (size_t)NS * F8Stage<B_FP4>::BYTES;
  constexpr size_t epi = 4 * (C_BF16 ? 128 * (128 * 2 + 16) : 64 * (128 * 4 + 16));
  return ring > epi ? ring : epi;
}

template <int B_FP4, int C_BF16, int NS>
static hipError_t launch_f8(const F8Args& a, hipStream_t s) {
  const size_t lds = f8_lds_bytes<B_FP4, C_BF16, NS>();
  static_assert(f8_lds_bytes<B_FP4, C_BF16, NS>() <= 160 * 1024, "LDS budget");
  static bool attr = false;  // raise the dynamic LDS limit once per instantiation
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)k_gemm_f8<B_FP4, C_BF16, NS>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int tiles = ((a.M + FT - 1) / FT) * ((a.N + FT - 1) / FT);
  hipLaunchKernelGGL((k_gemm_f8<B_FP4, C_BF16, NS>), dim3(tiles), dim3(256), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_f8(int a_fmt, int b_fp4, int c_bf16, const uint8_t* a_codes, const void* a_shared,
                          const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* c,
                          int64_t ldc, const float* row_div, void* ws, hipStream_t s) {
  uint8_t* base = (uint8_t*)ws;
  uint8_t* a8 = base;
  uint8_t* as_t = base + al256((size_t)M * K);
  uint8_t* b8 = as_t + al256((size_t)M * (K / 32));
  {
    const int64_t total = M * (K >> 3);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65535 * 4) blocks = 65535 * 4;
    if (a_fmt) hipLaunchKernelGGL(k_expand_a<1>, dim3((unsigned)blocks), dim3(256), 0, s, a_codes, a_shared, M, K, a8, as_t);
    else hipLaunchKernelGGL(k_expand_a<0>, dim3((unsigned)blocks), dim3(256), 0, s, a_codes, a_shared, M, K, a8, as_t);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!b_fp4) {
    const int64_t total = N * (K >> 3);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65535 * 4) blocks = 65535 * 4;
    hipLaunchKernelGGL(k_expand_b_int4, dim3((unsigned)blocks), dim3(256), 0, s, b_codes, N, K, b8);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  F8Args a{};
  a.a8 = a8; a.as_t = as_t; a.b = b_fp4 ? b_codes : b8; a.bs = b_scales;
  a.c = c; a.ldc = ldc; a.row_div = row_div; a.M = (int)M; a.N = (int)N; a.K = (int)K;
  if (b_fp4) return c_bf16 ? launch_f8<1, 1, 3>(a, s) : launch_f8<1, 0, 3>(a, s);
  return c_bf16 ? launch_f8<0, 1, 2>(a, s) : launch_f8<0, 0, 2>(a, s);
}

}  // namespace mix
