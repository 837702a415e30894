// Fast A-MiX x W-MX product: a decode pass, then an MXFP8 x MX{FP4,FP8} block-scaled MFMA GEMM.
//
// "P1" below is the pchao.org digest of the paper, titled
// "MiX：面向端到端低比特视觉语言模型加速的微反缩放"; citations name its sections and figures.
//
// P1 (method overview, the dual-format bullet and Eq. (6)) factors the shared MiX mantissa out of
// each block sum. On MI355X the exact multiplier is the matrix core. Each MiX element
// (1.m)_2 2^(Emax-dE) is exactly the E4M3 byte (1.m)_2 2^(1-dE) times the block power of two
// 2^(Emax-1). That power of two is an E8M0 block scale of v_mfma_scale_f32_32x32x64_f8f6f4, so
// the product is exact and the MFMA accumulates in fp32.
//
// Decoding codes into MFMA operands inside the GEMM would repeat the work once per tile column
// (74 times for a 4096 x 18944 x 3584 product). So each operand is decoded once into an image
// (layout in f8_image.h): k_expand_a (or the quantizer itself) turns MiX codes into E4M3 bytes
// plus permuted E8M0 scales; a weight's image (k_permute_b_scales, and k_expand_b_int4 for MXINT4
// weights, whose q/4 is exact in E4M3 under the unchanged E8M0 scale) depends on the weight only
// and can be built once. MXFP4 weights are used as stored: the E2M1 nibbles are the FP4 MFMA
// operand.
//
// The GEMM streams both operands global->LDS with global_load_lds_dwordx4 (no registers, no
// VALU). Each workgroup computes one 256 x 256 tile with 8 waves, each wave 64 x 128 outputs
// (2 x 4 MFMAs of 32 x 32 per 64-wide K half, 128 fp32 accumulators per lane). The waves form two
// groups with one wave of each on every SIMD, and the groups alternate between reading a K step's
// operands from LDS into registers and running the 16 MFMAs of a step from registers, so a SIMD's
// matrix pipe always has one wave feeding it (a barrier between phases). An LDS ring of three
// stages (two for E4M3 weights) lets a step's copies land while two phases run. Tiles are
// ordered in bands of 8 tile rows and split into
// XCD-contiguous chunks, so the tiles an XCD runs at once share A and B panels in its L2. Block
// scales are laid out per (K step, tile) in the order the lanes read them: one 8-byte LDS read
// gives a lane all its scales for a K step, and the MFMA's scale op_sel picks the byte. The
// epilogue goes through LDS so that every global store writes whole output rows.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 operand layout (established on the device): lane
// l = r + 32 g (r < 32, g < 2) supplies row/column r. An FP8 operand holds K elements
// [16 g, 16 g + 16) in bytes 0..15 and [32 + 16 g, 32 + 16 g + 16) in bytes 16..31. An FP4
// operand holds [32 g, 32 g + 32) in 16 bytes, low nibble first. The scale of lane l is the E8M0
// scale of row/column r for K block g. Result register k of lane l is
// C[8 (k >> 2) + 4 (l >> 5) + (k & 3)][l & 31].
#include "common.h"
#include "f8_image.h"
#include "gemv_dev.h"
#include "kernels.h"
#include "quant_dev.h"

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

namespace mix {

// ------------------------------------------------------------------ decode passes

// One lane per 8-element sub-block: 4 code bytes -> 8 E4M3 bytes. Quad lane 0 writes the block's
// E8M0 scale 2^(Emax-1) into the scale layout [K/128][tiles_m][256][4].
template <int A_FMT>
__global__ void __launch_bounds__(256) k_expand_a(const uint8_t* __restrict__ codes, const void* __restrict__ shared,
                                                   int64_t M, int64_t K, int tiles_m, uint8_t* __restrict__ a8,
                                                   uint8_t* __restrict__ as_p) {
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
    if ((sb & 3) == 0) {
      const int64_t st = blk >> 2, tile = row / FT;
      as_p[(st * tiles_m + tile) * 1024 + f8_a_scale_pos((int)(row % FT), (int)(blk & 3))] = (uint8_t)((sh & 15u) + 119u);
    }
  }
}

// MX scales [N, K/32] -> the permuted layout [K/128][tiles_n][1024].
__global__ void __launch_bounds__(256) k_permute_b_scales(const uint8_t* __restrict__ bs, int64_t N, int64_t K,
                                                           int tiles_n, uint8_t* __restrict__ bs_p,
                                                           uint8_t* __restrict__ bs_v) {
  const int64_t nb = K >> 5;
  const int64_t total = N * nb;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total; g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = g / nb, blk = g - row * nb;
    const int64_t st = blk >> 2, tile = row / FT;
    bs_p[(st * tiles_n + tile) * 1024 + f8_scale_pos((int)(row % FT), (int)(blk & 3))] = bs[g];
    bs_v[((row >> 4) * (K >> 7) + st) * 64 + (row & 15) * 4 + (blk & 3)] = bs[g];
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

template <int B_FP4>
struct F8Stage {
  static constexpr int A_BYTES = FT * FK;                          // E4M3 A, 128 B per row
  static constexpr int B_BYTES = B_FP4 ? FT * FK / 2 : FT * FK;    // FP4 (64 B/row) or E4M3 B
  static constexpr int AS_OFF = A_BYTES + B_BYTES;
  static constexpr int BS_OFF = AS_OFF + 1024;
  static constexpr int BYTES = BS_OFF + 1024;
  static constexpr int NS = B_FP4 ? 3 : 2;   // ring stages within 160 KB of LDS
  // copy instructions per issuing wave and K step: A (8), B (4 FP4 or 8 E4M3), two scale dwords
  static constexpr int PER = 8 + (B_FP4 ? 4 : 8) + 2;
};

struct F8Args {
  const uint8_t* a8;      // [M, K] E4M3
  const uint8_t* as_p;    // [K/128][tiles_m][256][4] E8M0 (f8_a_scale_pos)
  const uint8_t* b;       // [N, K/2] FP4 codes or [N, K] E4M3
  const uint8_t* bs_p;    // [K/128][bs_tn][1024] E8M0, permuted
  const uint8_t* bs_v;    // [ceil(N/16)][K/128][16][4] E8M0 (small-M product)
  void* c;                // C [M, ldc] (may be NULL when the output is quantized)
  int64_t ldc;
  int M, N, K;
  int bs_tn;              // 256-row tiles of the B image (its scale layout)
  // output quantization (k_gemm_f8<..., OQ = 1>): the bf16 rounding of C as MiX-4.5b along N
  uint8_t* qc;            // codes [M, N/2]
  uint16_t* qsh;          // shared fields [M, N/32]
  uint8_t* qa8;           // the A image of C for a next product (K = N): E4M3 [M, N], or NULL
  uint8_t* qas_p;         //   and its scales [N/128][ceil(M/256)][256][4]
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int F8_C_CPOL = 17;            // buffer store cache policy: sc0 | sc1 (system scope)
constexpr int F8_RSRC_W3 = 0x00020000;   // buffer resource word 3 for raw 32-bit-offset access
constexpr int F8_THREADS = 512;   // 8 waves: 4 along M x 2 along N, 64 x 128 outputs each

// LDS slot of 16-byte chunk c of a stage row: 128-byte rows (E4M3) take c ^ aswz(row), 64-byte rows
// (FP4) c ^ bswz(row). With either 8 or 16 lanes served per LDS cycle, the lanes of one read
// (consecutive rows, the same logical chunk) then fall in distinct banks.
__device__ __forceinline__ int aswz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int bswz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// Copies of one K step of tile (tm, tn) into the stage at LDS byte address `st`, issued by the
// four waves of the copying group (w = 0..3, wave-uniform); each copies whole 1 KB runs (64 lanes x
// 16 bytes) of the stage image. A and E4M3 B: chunk q = 256 p + 64 w + lane lands at LDS byte 16 q
// and holds (row q / 8, logical chunk (q % 8) ^ aswz(row)) of the operand tile; FP4 B: (row q / 4,
// chunk (q % 4) ^ bswz(row)). The swizzle depends on row bits the copy index p does not touch, so a
// lane keeps one chunk column across p. Rows past M (N) repeat the last row; they are never
// stored. The per-copy offsets are recomputed at each call (the empty asm hides the lane index
// from loop-invariant hoisting), which costs a few VALU instructions instead of 8 to 16 registers
// held across the K loop. PART 0 issues the whole step; PART 1 the first half of the A and B copies
// and the A scales, PART 2 the rest (two groups of waves can then share a step's copies).
template <int B_FP4, int PART>
__device__ __forceinline__ void f8_issue(const F8Args& g, uint32_t st, int tm, int tn, int tiles_m, int ks, int w,
                                         int lane) {
  constexpr int NA = 8, NB = B_FP4 ? 4 : 8;
  constexpr int A0 = PART == 2 ? NA / 2 : 0, A1 = PART == 1 ? NA / 2 : NA;
  constexpr int B0 = PART == 2 ? NB / 2 : 0, B1 = PART == 1 ? NB / 2 : NB;
  const int m0 = tm * FT, n0 = tn * FT, k0 = ks * FK;
  int ln = lane;
  asm volatile("" : "+v"(ln));
  {
    const int ta = w * 8 + (ln >> 3);            // tile row of copy p = 0; copy p reads row 32 p + ta
    const int ca = (ln & 7) ^ aswz(ta);
    const int lim = g.M - 1 - m0;
    const uint8_t* base = g.a8 + (size_t)m0 * g.K + k0;
#pragma unroll
    for (int p = A0; p < A1; p++)
      dma16s(base, (uint32_t)(min(32 * p + ta, lim) * g.K + 16 * ca), st + (p * 256 + w * 64) * 16);
  }
  if (B_FP4) {
    const int tb = w * 16 + (ln >> 2);           // copy p reads row 64 p + tb (64-byte rows)
    const int cb = (ln & 3) ^ bswz(tb);
    const int lim = g.N - 1 - n0;
    const uint8_t* base = g.b + ((size_t)ks * g.N + n0) * 64;   // step-major image: rows 64 bytes apart
#pragma unroll
    for (int p = B0; p < B1; p++)
      dma16s(base, (uint32_t)(min(64 * p + tb, lim) * 64 + 16 * cb),
             st + F8Stage<B_FP4>::A_BYTES + (p * 256 + w * 64) * 16);
  } else {
    const int tb = w * 8 + (ln >> 3);
    const int cb = (ln & 7) ^ aswz(tb);
    const int lim = g.N - 1 - n0;
    const uint8_t* base = g.b + (size_t)n0 * g.K + k0;
#pragma unroll
    for (int p = B0; p < B1; p++)
      dma16s(base, (uint32_t)(min(32 * p + tb, lim) * g.K + 16 * cb),
             st + F8Stage<B_FP4>::A_BYTES + (p * 256 + w * 64) * 16);
  }
  // scales: the (K step, tile) 1 KB blocks are contiguous; a wave copies 256 bytes of each
  if (PART != 2)
    dma4(g.as_p + (uint32_t)((ks * tiles_m + tm) * 1024 + w * 256 + ln * 4), st + F8Stage<B_FP4>::AS_OFF + w * 256);
  if (PART != 1)
    dma4(g.bs_p + (uint32_t)((ks * g.bs_tn + tn) * 1024 + w * 256 + ln * 4), st + F8Stage<B_FP4>::BS_OFF + w * 256);
}

// Workgroup barrier that the compiler neither moves memory accesses across (the empty asm with a
// memory clobber) nor schedules instructions across; it waits for nothing by itself.
__device__ __forceinline__ void f8_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// s_waitcnt lgkmcnt(0) alone: this wave's LDS reads have returned
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

typedef int v4i __attribute__((ext_vector_type(4)));

// Tile order: a banded order (bands of GM tile rows, column by column inside a band) cut into 8
// contiguous chunks, one per XCD (workgroup b runs on XCD b % 8). The workgroups of an XCD take
// their chunk's tiles in turn, so the ~32 tiles an XCD runs at once share a few A and B panels in
// its L2.
__device__ __forceinline__ void f8_tile(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GM = 8;
  const int band_sz = GM * tiles_n;
  const int band = t / band_sz;
  const int rem = t - band * band_sz;
  const int gm = min(GM, tiles_m - band * GM);
  tn = rem / gm;
  tm = band * GM + (rem - tn * gm);
}

// Persistent: one workgroup per CU takes 256 x 256 output tiles of its XCD's chunk in turn. The
// MFMA computes C^T tiles: its A operand is the weight fragment (rows n), its B operand the
// activation fragment (rows m), so result register k of lane l holds
// C[m = l & 31][n = 8 (k >> 2) + 4 (l >> 5) + (k & 3)].
//
// Main loop: ping-pong between two groups of four waves, one wave of each group per SIMD. Every
// phase ends with a workgroup barrier; in a phase one group reads the operands of a K step from
// LDS into registers while the other runs the 16 MFMAs of its previous step from registers, so
// each SIMD's matrix pipe is fed by one wave while the other waits on LDS. Group 0 reads step j in
// phase 2j and multiplies in 2j + 1; group 1 runs one phase later. The global->LDS copies of step
// j + NS - 1 go into the ring slot that step j - 1 left (both groups read it by phase 2j - 1): with
// three slots group 0 issues half of them in phase 2j and group 1 the other half in phase 2j + 1
// (a CU's texture path moves about 64 bytes a cycle, so one group issuing all 50 KB of a step
// would outlast the other group's MFMA phase); each group waits for its own copies of step j + 1
// before the barrier that ends phase 2j + 1. With two slots (E4M3 weights) group 0 issues them
// all. Steps 0 .. NS - 2 of the next tile are issued before the epilogue, which stages C through
// the last ring slot, so their latency hides behind it.
template <int B_FP4, int C_BF16, int OQ = 0>
__global__ void __launch_bounds__(F8_THREADS, 1) k_gemm_f8(F8Args g) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int SB = F8Stage<B_FP4>::BYTES;
  constexpr int NS = F8Stage<B_FP4>::NS;
  // with three ring slots both groups issue half of each step's copies (group 1 in its read phase);
  // with two, group 0 issues them all (a copy issued in group 1's read phase would have one phase)
  constexpr bool SPLIT = NS == 3;
  constexpr int PH = SPLIT ? F8Stage<B_FP4>::PER / 2 : F8Stage<B_FP4>::PER;   // copies per wave and step
  const int tiles_m = (g.M + FT - 1) / FT, tiles_n = (g.N + FT - 1) / FT;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w4 = wave & 3;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, gq = lane >> 5;
  const int nk = g.K / FK;
  const uint32_t lds0 = lds_addr(smem);
  // A scales: the dwords of this lane's two rows 64 wm + 32 i + r (byte b = block b of the K step;
  // shifted right by 8 gq, byte 2h is the lane's block 2h + gq); B: this lane's 8 bytes [h][sub-tile]
  // in the permuted 1 KB block (see f8_scale_pos)
  const int sc_a = (64 * wm + r) * 4;
  const int sc_b = ((wn * 2 + gq) * 32 + r) * 8;

  // this workgroup's tiles: c0 + ix, c0 + ix + gx, ... below c0 + csz
  const int nt = tiles_m * tiles_n;
  const int xcd = blockIdx.x & 7, ix = blockIdx.x >> 3;
  const int gx = ((int)gridDim.x - xcd + 7) >> 3;
  const int c0 = xcd * (nt >> 3) + min(xcd, nt & 7), csz = (nt >> 3) + (xcd < (nt & 7) ? 1 : 0);
  int ti = ix;
  if (ti >= csz) return;
  // Every workgroup runs tiles of the same length, so without a stagger all CUs would reach their
  // epilogues together and store every round's C in one burst, while they also issue the next
  // tiles' first copies together. Part of the workgroups start about 6000 cycles (s_sleep 96 x 64)
  // later, so the store bursts and first copies of the two sets fall apart in time: those that run
  // one tile fewer than the rest (they finish early anyway), or the odd ones of an XCD when all run
  // the same count; only where each workgroup has at least two tiles. Measured with the outputs
  // unchanged: 16384 x 5120 x 1280 100-104 -> 97-99 us, 4096 x 18944 x 3584 187-200 -> 186-196 us.
  {
    const int rem = csz % gx;   // workgroups ix < rem run one tile more than the rest
    const bool late = rem ? ix >= rem : (ix & 1);
    if (late && csz >= 2 * gx) __builtin_amdgcn_s_sleep(96);
  }
  int tm, tn;
  f8_tile(c0 + ti, tiles_m, tiles_n, tm, tn);
  // steps 0 .. NS - 2 of a tile
  auto issue_first = [&]() {
    if (wave < 4) {
#pragma unroll
      for (int s = 0; s < NS - 1; s++)
        if (s < nk) f8_issue<B_FP4, SPLIT ? 1 : 0>(g, lds0 + s * SB, tm, tn, tiles_m, s, w4, lane);
    } else if (SPLIT) {
#pragma unroll
      for (int s = 0; s < NS - 1; s++)
        if (s < nk) f8_issue<B_FP4, 2>(g, lds0 + s * SB, tm, tn, tiles_m, s, w4, lane);
    }
  };
  issue_first();

  v16f acc[2][4];
  // operands of one K step, held in registers between a wave's read phase and its MFMA phase
  v8i xf[2][2];
  v8i wf[2][4];
  int xsw[2], wsw[2];   // A scale word per sub-tile i, B scale word per K half h

  auto read_step = [&](int slot) {
    const uint8_t* st = smem + slot * SB;
    const uint8_t* sa = st;
    const uint8_t* sbm = st + F8Stage<B_FP4>::A_BYTES;
    const uint32_t xs0 = *(const uint32_t*)(st + F8Stage<B_FP4>::AS_OFF + sc_a);
    const uint32_t xs1 = *(const uint32_t*)(st + F8Stage<B_FP4>::AS_OFF + sc_a + 32 * 4);
    const uint2 ws8 = *(const uint2*)(st + F8Stage<B_FP4>::BS_OFF + sc_b);
    xsw[0] = (int)(xs0 >> (8 * gq));
    xsw[1] = (int)(xs1 >> (8 * gq));
#pragma unroll
    for (int h = 0; h < 2; h++) {
      wsw[h] = (int)(h ? ws8.y : ws8.x);
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const int row = 64 * wm + 32 * i + r;
        const int c0 = 4 * h + gq, c1 = 4 * h + 2 + gq;
        const uint4 lo = *(const uint4*)(sa + row * 128 + ((c0 ^ aswz(row)) * 16));
        const uint4 hi = *(const uint4*)(sa + row * 128 + ((c1 ^ aswz(row)) * 16));
        xf[h][i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int row = 128 * wn + 32 * j + r;
        if (B_FP4) {
          // FP4 operands read only the low 4 registers of the 8-register tuple
          const int c = 2 * h + gq;
          const v4i w = *(const v4i*)(sbm + row * 64 + ((c ^ bswz(row)) * 16));
          wf[h][j] = __builtin_shufflevector(w, w, 0, 1, 2, 3, -1, -1, -1, -1);
        } else {
          const int c0 = 4 * h + gq, c1 = 4 * h + 2 + gq;
          const v4i lo = *(const v4i*)(sbm + row * 128 + ((c0 ^ aswz(row)) * 16));
          const v4i hi = *(const v4i*)(sbm + row * 128 + ((c1 ^ aswz(row)) * 16));
          wf[h][j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      }
    }
  };
  // the scale operands' op_sel picks byte J of the weight word and byte 2H of the activation word
  auto mfma_step = [&]() {
#define F8_MFMA(H, I, J)                                                                                   \
  acc[I][J] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[H][J], xf[H][I], acc[I][J], B_FP4 ? 4 : 0, 0, J, \
                                                              wsw[H], 2 * H, xsw[I])
    F8_MFMA(0, 0, 0); F8_MFMA(0, 1, 0); F8_MFMA(0, 0, 1); F8_MFMA(0, 1, 1);
    F8_MFMA(0, 0, 2); F8_MFMA(0, 1, 2); F8_MFMA(0, 0, 3); F8_MFMA(0, 1, 3);
    F8_MFMA(1, 0, 0); F8_MFMA(1, 1, 0); F8_MFMA(1, 0, 1); F8_MFMA(1, 1, 1);
    F8_MFMA(1, 0, 2); F8_MFMA(1, 1, 2); F8_MFMA(1, 0, 3); F8_MFMA(1, 1, 3);
#undef F8_MFMA
    // all 16 are issued before anything that follows (a copy wait placed between them would hold
    // the rest of the phase's MFMAs back)
    __builtin_amdgcn_sched_barrier(0);
  };

  // epilogue geometry: a pass stages a wave's 32 x CW outputs (128 bytes of each row) in its own
  // region of the last ring slot, then stores whole 128-byte row segments. Rows are 128 bytes with
  // the 16-byte chunk c of row r at slot c ^ (r & 7): every access stays 16-byte aligned (a padded
  // 136-byte pitch makes the row read-backs unaligned, which costs this part about three times the
  // LDS cycles of the whole staging) and the MFMA-layout writes of one chunk column spread over
  // eight slots.
  constexpr int ES = C_BF16 ? 2 : 4;                 // output element size
  constexpr int CW = 128 / ES;                       // columns per pass (64 or 32)
  constexpr int JP = CW / 32;                        // MFMA column blocks per pass (2 or 1)
  constexpr int PITCH = 128;                         // row pitch of the region
  constexpr int EPL = 16 / ES;                       // outputs per 16-byte chunk
  uint8_t* reg = smem + (NS - 1) * SB + wave * (32 * PITCH);
  const bool vec_ok = (g.ldc % EPL) == 0 && (((uintptr_t)g.c) & 15) == 0;
  // Whole-tile stores of C go out as buffer stores (a wave-uniform base and a 32-bit offset a lane)
  // with system scope (sc0 sc1): they write through the XCD's L2 instead of leaving dirty lines
  // there for a later write-back. Measured on the 16384 x 5120 x 1280 product (168 MB of C; outputs
  // unchanged): 101.6 -> 97.3 us; within noise on 4096 x 18944 x 3584.

  while (true) {
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) acc[i][j] = v16f{};

    if (wave < 4) {
      // group 0: reads step j in phase 2j, multiplies in phase 2j + 1
      if (NS == 3 && nk > 1) wait_vmcnt<PH>(); else wait_vmcnt<0>();   // its copies of step 0 have landed
      f8_sync();
      int rs = 0;                 // ring slot of step j
      int is = NS - 1;            // ring slot of step j + NS - 1
      int j = 0;
      // Steps that still issue a copy, then the last NS - 1 steps: each loop body is straight-line
      // code, so the compiler cannot sink the MFMAs below the copy wait and the barrier that end
      // the MFMA phase (they would then wait for the next step's copies).
      for (; j + NS - 1 < nk; j++) {
        f8_issue<B_FP4, SPLIT ? 1 : 0>(g, lds0 + is * SB, tm, tn, tiles_m, j + NS - 1, w4, lane);
        read_step(rs);
        wait_lgkm0();
        f8_sync();
        mfma_step();
        wait_vmcnt<(NS - 2) * PH>();   // its copies of step j + 1 have landed (step j + NS - 1's may not)
        f8_sync();
        rs = rs + 1 == NS ? 0 : rs + 1;
        is = is + 1 == NS ? 0 : is + 1;
      }
      for (; j < nk; j++) {
        read_step(rs);
        wait_lgkm0();
        f8_sync();
        mfma_step();
        wait_vmcnt<0>();
        f8_sync();
        rs = rs + 1 == NS ? 0 : rs + 1;
      }
      f8_sync();   // group 1's last MFMA phase
    } else {
      // group 1: one phase behind; with SPLIT it issues the other half of step j + 2's copies in
      // its read phase of step j and waits for its half of step j + 1 before that phase ends
      if (SPLIT) {
        if (nk > 1) wait_vmcnt<PH>(); else wait_vmcnt<0>();
      }
      f8_sync();
      f8_sync();
      int rs = 0, is = NS - 1, j = 0;
      if (SPLIT) {
        for (; j + NS - 1 < nk; j++) {
          f8_issue<B_FP4, 2>(g, lds0 + is * SB, tm, tn, tiles_m, j + NS - 1, w4, lane);
          read_step(rs);
          wait_vmcnt<PH>();
          wait_lgkm0();
          f8_sync();
          mfma_step();
          f8_sync();
          rs = rs + 1 == NS ? 0 : rs + 1;
          is = is + 1 == NS ? 0 : is + 1;
        }
      }
      for (; j < nk; j++) {
        read_step(rs);
        if (SPLIT) wait_vmcnt<0>();
        wait_lgkm0();
        f8_sync();
        mfma_step();
        f8_sync();
        rs = rs + 1 == NS ? 0 : rs + 1;
      }
    }

    // every wave is past its last LDS read of this tile: the ring is free
    const int cur_tm = tm, cur_tn = tn;
    ti += gx;
    const bool more = ti < csz;
    if (more) {
      f8_tile(c0 + ti, tiles_m, tiles_n, tm, tn);
      issue_first();
    }

    // Epilogue, staged through LDS so that global stores write whole 128-byte row segments.
    const int mw = cur_tm * FT + 64 * wm, nw = cur_tn * FT + 128 * wn;
    // a tile inside C with aligned rows: each pass reads its four rows back and stores them with no
    // per-store bounds checks, so the four LDS reads are in flight together
    const bool fast = !OQ && vec_ok && g.ldc <= (1 << 21) && (cur_tm + 1) * FT <= g.M && (cur_tn + 1) * FT <= g.N;
#pragma unroll
    for (int i = 0; i < 2; i++) {
#pragma unroll
      for (int jp = 0; jp < 4 / JP; jp++) {
#pragma unroll
        for (int jj = 0; jj < JP; jj++)
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int j = jp * JP + jj;
            const int cb = (32 * jj + 8 * q + 4 * gq) * ES;   // byte of the row segment
            uint8_t* dst = reg + r * PITCH + ((((cb >> 4) ^ r) & 7) << 4) + (cb & 15);
            const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1], v2 = acc[i][j][4 * q + 2],
                        v3 = acc[i][j][4 * q + 3];
            if (C_BF16)
              *(uint2*)dst = make_uint2(pk_bf16_rne(v0, v1), pk_bf16_rne(v2, v3));
            else
              *(float4*)dst = make_float4(v0, v1, v2, v3);
          }
        if (fast) {
          const int ch = lane & 7;
          uint4 v[4];
#pragma unroll
          for (int it = 0; it < 4; it++) {
            const int row = it * 8 + (lane >> 3);
            v[it] = *(const uint4*)(reg + row * PITCH + ((ch ^ row) & 7) * 16);
          }
          // the pass's 32 rows from a wave-uniform base: the lane offsets stay below 2^31 (fast
          // requires ldc <= 2^21)
          const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
              (uint8_t*)g.c + (int64_t)(mw + 32 * i) * g.ldc * ES, 0, 0x7FFFFFFF, F8_RSRC_W3);
          const int off = ((lane >> 3) * (int)g.ldc + nw + jp * CW + ch * EPL) * ES;
          const int step8 = 8 * (int)g.ldc * ES;   // 8 rows
#pragma unroll
          for (int it = 0; it < 4; it++) {
            const u32x4_t d = {v[it].x, v[it].y, v[it].z, v[it].w};
            __builtin_amdgcn_raw_buffer_store_b128(d, rs, off + it * step8, 0, F8_C_CPOL);
          }
          continue;
        }
#pragma unroll
        for (int it = 0; it < 4; it++) {
          const int row = it * 8 + (lane >> 3), ch = lane & 7;
          const uint4 v = *(const uint4*)(reg + row * PITCH + ((ch ^ row) & 7) * 16);
          const int gm = mw + 32 * i + row, gn = nw + jp * CW + ch * EPL;
          if (OQ) {
            // this lane's 8 bf16 outputs are a MiX sub-block, the 4 lanes of a quad one 32-column
            // block (N is a multiple of 32, so quads are in or past N together)
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
            int emax;
            uint32_t m, e0, e1;
            const uint32_t word = mix_quant_lane_bf16_img<1, true>(w4, emax, m, e0, e1);
            const int qd = ch & 3;
            const uint32_t f = quad_or_dpp((qd == 0 ? (uint32_t)(emax + 7) : 0u) | (m << (4 + 3 * qd)));
            if (gm < g.M && gn < g.N) {
              *(uint32_t*)(g.qc + (int64_t)gm * (g.N >> 1) + (gn >> 1)) = word;
              if (qd == 0) g.qsh[(int64_t)gm * (g.N >> 5) + (gn >> 5)] = (uint16_t)f;
              if (g.qa8) {
                *(uint2*)(g.qa8 + (int64_t)gm * g.N + gn) = make_uint2(e0, e1);
                if (qd == 0)
                  g.qas_p[((int64_t)(gn >> 7) * tiles_m + (gm >> 8)) * 1024 +
                          f8_a_scale_pos(gm & (FT - 1), (gn >> 5) & 3)] = (uint8_t)(emax + 126);
              }
            }
            if (!g.c) continue;
          }
          if (gm >= g.M) continue;
          uint8_t* out = (uint8_t*)g.c + ((int64_t)gm * g.ldc + gn) * ES;
          if (vec_ok && gn + EPL <= g.N) {
            store16_nt(out, v);
          } else {
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < EPL; e++) {
              if (gn + e >= g.N) break;
              if (C_BF16) ((uint16_t*)out)[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
              else ((uint32_t*)out)[e] = w4[e];
            }
          }
        }
      }
    }
    // the next tile's step NS - 1 goes into the staging slot only after its first barrier, which
    // every wave reaches with its read-backs returned (their data went to the stores above)
    if (!more) break;
  }
}

// ------------------------------------------------------------------ small-M product (decode)

typedef float v4f __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ host side

bool gemm_f8_offsets_ok(int64_t M, int64_t N, int64_t K);

// Shapes mix_mx_gemm sends through the images: the tiled GEMM for M >= 64 and N >= 256, the
// weight stream (k_gemv_rs, gemv_dev.h) for M <= 16; others decode inside k_gemm_mfma.
bool gemm_f8_eligible(int64_t M, int64_t N, int64_t K) {
  return K > 0 && K % FK == 0 && ((M >= 64 && N >= FT) || (M >= 1 && M <= 16)) && gemm_f8_offsets_ok(M, N, K);
}

// The tiled kernel addresses its operands with 32-bit byte offsets.
bool gemm_f8_offsets_ok(int64_t M, int64_t N, int64_t K) {
  const int64_t lim = (int64_t)1 << 31;
  return M * K < lim && N * K < lim && (K / FK) * ((M + FT - 1) / FT) * 1024 < lim &&
         (K / FK) * ((N + FT - 1) / FT) * 1024 < lim;
}

size_t gemm_f8_ws_bytes(int b_fp4, int64_t M, int64_t N, int64_t K) {
  return f8_a_image_layout(M, K).total + f8_b_image_layout(b_fp4, N, K).total;
}

template <int B_FP4, int C_BF16>
constexpr size_t f8_lds_bytes() {
  // the ring, whose last slot (and what lies past it) also holds the epilogue's 8 x 32 x 128 bytes
  const size_t ring = (size_t)F8Stage<B_FP4>::NS * F8Stage<B_FP4>::BYTES;
  const size_t epi = (size_t)(F8Stage<B_FP4>::NS - 1) * F8Stage<B_FP4>::BYTES + (F8_THREADS / 64) * 32 * 128;
  return ring > epi ? ring : epi;
}

// compute units of the current device (one persistent GEMM workgroup each)
static int f8_cu_count() {
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

template <int B_FP4, int C_BF16, int OQ = 0>
static hipError_t launch_f8(const F8Args& a, hipStream_t s) {
  constexpr size_t lds = f8_lds_bytes<B_FP4, C_BF16>();
  static_assert(lds <= 160 * 1024, "LDS budget");
  static bool attr = false;  // raise the dynamic LDS limit once per instantiation
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)k_gemm_f8<B_FP4, C_BF16, OQ>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int tiles = ((a.M + FT - 1) / FT) * ((a.N + FT - 1) / FT);
  const int cus = f8_cu_count();
  hipLaunchKernelGGL((k_gemm_f8<B_FP4, C_BF16, OQ>), dim3(tiles < cus ? tiles : cus), dim3(F8_THREADS), lds, s, a);
  return hipGetLastError();
}

static inline unsigned grid1d(int64_t n) {
  int64_t b = (n + 255) / 256;
  if (b > 65535 * 4) b = 65535 * 4;
  return (unsigned)(b < 1 ? 1 : b);
}

hipError_t launch_gemm_a_image(int a_fmt, const uint8_t* a_codes, const void* a_shared, int64_t M, int64_t K,
                               void* img, hipStream_t s) {
  const F8AImage L = f8_a_image_layout(M, K);
  uint8_t* base = (uint8_t*)img;
  const int tiles_m = (int)((M + FT - 1) / FT);
  if (a_fmt)
    hipLaunchKernelGGL(k_expand_a<1>, dim3(grid1d(M * (K >> 3))), dim3(256), 0, s, a_codes, a_shared, M, K, tiles_m,
                       base + L.a8, base + L.as_p);
  else
    hipLaunchKernelGGL(k_expand_a<0>, dim3(grid1d(M * (K >> 3))), dim3(256), 0, s, a_codes, a_shared, M, K, tiles_m,
                       base + L.a8, base + L.as_p);
  return hipGetLastError();
}

// MXFP4 codes [N, K/2] -> the image's step-major copy [K/128][N][64]; one thread per 16 bytes
__global__ void __launch_bounds__(256) k_b4_step_major(const uint8_t* __restrict__ codes, int64_t N, int64_t K,
                                                        uint8_t* __restrict__ dst) {
  const int64_t cpr = K >> 5;   // 16-byte chunks per row
  const int64_t total = N * cpr;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = t / cpr, c = t - row * cpr;
    const uint4 v = *(const uint4*)(codes + row * (K >> 1) + c * 16);
    *(uint4*)(dst + ((c >> 2) * N + row) * 64 + (c & 3) * 16) = v;
  }
}

hipError_t launch_gemm_b_image(int b_fp4, const uint8_t* b_codes, const uint8_t* b_scales, int64_t N, int64_t K,
                               void* img, hipStream_t s) {
  const F8BImage L = f8_b_image_layout(b_fp4, N, K);
  uint8_t* base = (uint8_t*)img;
  const int tiles_n = (int)((N + FT - 1) / FT);
  hipLaunchKernelGGL(k_permute_b_scales, dim3(grid1d(N * (K >> 5))), dim3(256), 0, s, b_scales, N, K, tiles_n,
                     base + L.bs_p, base + L.bs_v);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (b_fp4)
    hipLaunchKernelGGL(k_b4_step_major, dim3(grid1d(N * (K >> 5))), dim3(256), 0, s, b_codes, N, K, base + L.b8);
  else
    hipLaunchKernelGGL(k_expand_b_int4, dim3(grid1d(N * (K >> 3))), dim3(256), 0, s, b_codes, N, K, base + L.b8);
  return hipGetLastError();
}

// M <= 16 as a plain launch of the weight stream (gemv_dev.h): each workgroup owns RG groups of 16
// output columns, with RG chosen so that about one workgroup lands on each CU (fewer, longer
// workgroups streamed faster than many short ones: 10.8 against 13.1 us for 18944 x 3584 MXFP4);
// its four waves split K and keep two steps of operands in flight in registers.
constexpr int GV_D = 2;

template <int B_FP4, int C_BF16, int RG>
__global__ void __launch_bounds__(256) k_gemv_rs(GvOps g) {
  __shared__ __align__(16) float red[gv_lds_bytes<RG>() / 4];
  gemv_block<B_FP4, C_BF16, RG, GV_D>(g, (int)blockIdx.x, red);
}

template <int B_FP4, int C_BF16>
static hipError_t launch_gv_rs(const GvOps& g, hipStream_t s) {
  const int ngrp = (g.N + 15) / 16;
  const int need = (ngrp + f8_cu_count() - 1) / f8_cu_count();
#define GVL(RG) hipLaunchKernelGGL((k_gemv_rs<B_FP4, C_BF16, RG>), dim3((unsigned)((ngrp + RG - 1) / RG)), dim3(256), 0, s, g)
  if (need <= 1) GVL(1);
  else if (need <= 2) GVL(2);
  else if (need <= 4) GVL(4);
  else if (need <= 5) GVL(5);
  else GVL(8);
#undef GVL
  return hipGetLastError();
}

static hipError_t launch_gemv_f8(int b_fp4, int c_bf16, const F8Args& f, hipStream_t s) {
  GvOps g{};
  g.a8 = f.a8; g.as_p = f.as_p; g.b8 = f.b; g.bs_v = f.bs_v;
  g.c = f.c; g.ldc = f.ldc; g.M = f.M; g.N = f.N; g.K = f.K; g.tiles_m = (f.M + FT - 1) / FT;
  if (b_fp4) return c_bf16 ? launch_gv_rs<1, 1>(g, s) : launch_gv_rs<1, 0>(g, s);
  return c_bf16 ? launch_gv_rs<0, 1>(g, s) : launch_gv_rs<0, 0>(g, s);
}

hipError_t launch_gemm_images(int b_fp4, int c_bf16, const void* a_img, const void* b_img, int64_t M, int64_t N,
                              int64_t K, void* c, int64_t ldc, hipStream_t s) {
  const F8AImage LA = f8_a_image_layout(M, K);
  const F8BImage LB = f8_b_image_layout(b_fp4, N, K);
  F8Args a{};
  a.a8 = (const uint8_t*)a_img + LA.a8;
  a.as_p = (const uint8_t*)a_img + LA.as_p;
  a.b = (const uint8_t*)b_img + LB.b8;
  a.bs_p = (const uint8_t*)b_img + LB.bs_p;
  a.bs_v = (const uint8_t*)b_img + LB.bs_v;
  a.c = c; a.ldc = ldc; a.M = (int)M; a.N = (int)N; a.K = (int)K;
  a.bs_tn = (int)((N + FT - 1) / FT);
  if (M <= 16) return launch_gemv_f8(b_fp4, c_bf16, a, s);
  if (b_fp4) return c_bf16 ? launch_f8<1, 1>(a, s) : launch_f8<1, 0>(a, s);
  return c_bf16 ? launch_f8<0, 1>(a, s) : launch_f8<0, 0>(a, s);
}

// The product from the two images with its output quantized: MiX-4.5b codes and shared fields of
// the bf16 rounding of C along N, and optionally that output's A image for a next product; C
// itself (bf16) only if c is given. M > 16: in the tiled product's epilogue; M <= 16: the weight
// stream writes C (required then) and the quantizer codes it.
hipError_t launch_gemm_images_q(int b_fp4, const void* a_img, const void* b_img, int64_t M, int64_t N, int64_t K,
                                void* c, int64_t ldc, uint8_t* q_codes, void* q_shared, void* q_img, hipStream_t s) {
  if (M <= 16) {
    hipError_t e = launch_gemm_images(b_fp4, 1, a_img, b_img, M, N, K, c, ldc, s);
    if (e != hipSuccess) return e;
    if (q_img) return launch_mix_quantize_img(1, c, 1, M, N, ldc, q_codes, q_shared, q_img, s);
    return launch_mix_quantize(1, c, 1, M, N, ldc, q_codes, q_shared, s);
  }
  const F8AImage LA = f8_a_image_layout(M, K);
  const F8BImage LB = f8_b_image_layout(b_fp4, N, K);
  F8Args a{};
  a.a8 = (const uint8_t*)a_img + LA.a8;
  a.as_p = (const uint8_t*)a_img + LA.as_p;
  a.b = (const uint8_t*)b_img + LB.b8;
  a.bs_p = (const uint8_t*)b_img + LB.bs_p;
  a.bs_v = (const uint8_t*)b_img + LB.bs_v;
  a.c = c; a.ldc = ldc; a.M = (int)M; a.N = (int)N; a.K = (int)K;
  a.bs_tn = (int)((N + FT - 1) / FT);
  a.qc = q_codes;
  a.qsh = (uint16_t*)q_shared;
  if (q_img) {
    const F8AImage LQ = f8_a_image_layout(M, N);
    a.qa8 = (uint8_t*)q_img + LQ.a8;
    a.qas_p = (uint8_t*)q_img + LQ.as_p;
  }
  return b_fp4 ? launch_f8<1, 1, 1>(a, s) : launch_f8<0, 1, 1>(a, s);
}

hipError_t launch_gemm_f8(int a_fmt, int b_fp4, int c_bf16, const uint8_t* a_codes, const void* a_shared,
                          const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* c,
                          int64_t ldc, void* ws, hipStream_t s) {
  uint8_t* a_img = (uint8_t*)ws;
  uint8_t* b_img = a_img + f8_a_image_layout(M, K).total;
  hipError_t e = launch_gemm_a_image(a_fmt, a_codes, a_shared, M, K, a_img, s);
  if (e != hipSuccess) return e;
  if ((e = launch_gemm_b_image(b_fp4, b_codes, b_scales, N, K, b_img, s)) != hipSuccess) return e;
  return launch_gemm_images(b_fp4, c_bf16, a_img, b_img, M, N, K, c, ldc, s);
}

}  // namespace mix
