// K-smoothed attention over MiX/MX-coded operands, prefill and decode, for gfx950.
//
// "P1" below is the pchao.org digest of the paper, titled
// "MiX：面向端到端低比特视觉语言模型加速的微反缩放"; citations name its sections and figures.
//
// What it computes (P1, 方法概览 / method overview, last bullet; 核心创新 / innovations, third
// bullet; 关键结果 / key results, first bullet): keys are smoothed by subtracting their per-channel
// mean over the prefill tokens (softmax is unchanged by a constant shift per query row), the mean is
// kept frozen for decode so cached keys are never re-coded, and both attention products run on
// low-bit operands. Operand formats: Q and P as MiX-4.5b (activations, blocks along the head
// dimension and along keys); smoothed K and V as MXFP4 (cached operands, blocks along the head
// dimension and along tokens).
//
// Prefill (d = 128) codes the operands, then makes two passes over S without storing it: pass 1
// finds each query row's exact maximum (the P^ codes depend on it), pass 2 recomputes S tile by
// tile, forms z = fp32(S) * fp32(1/sqrt(d)), p = exp(z - m), l = sum p and P^ = MiX-4.5b(p) along
// keys, and accumulates P^ V^ on the MFMA; O = (P^ V^)/l. Other head sizes take the unfused path:
// S on the block-scaled MFMA GEMM, one wave per query row for p and P^, O on the same GEMM.
//
// Decode keeps the exact global row max with two passes over the keys: pass 1 (scores) computes S
// for 256-key chunks on the MFMA and per-chunk maxima; pass 2 (pv) takes the global max, forms p
// and P^ for its chunk and multiplies by V^ on the MFMA; a third launch sums the chunk partials.
#include <hip/hip_cooperative_groups.h>
#include <mutex>
#include <type_traits>

#include "../../include/mixlib.h"
#include "common.h"
#include "f8_image.h"
#include "gemv_dev.h"
#include "kernels.h"
#include "quant_dev.h"

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

namespace mix {

// ------------------------------------------------------------------ one MiX-4.5b sub-block of p

// Codes the 8 values of this lane (one 8-element sub-block; a quad of lanes is one 32-element
// block) as MiX-4.5b. Returns the code word; *shared receives the block's field on the quad's
// first lane; *m_out this sub-block's mantissa.
__device__ __forceinline__ uint32_t mix45_code8(const float (&p)[8], int quad_pos, uint32_t* shared,
                                                uint32_t* m_out) {
  uint32_t xb[8];
#pragma unroll
  for (int e = 0; e < 8; e++) xb[e] = f32_bits(p[e]);
  int emax;
  uint32_t m;
  const uint32_t word = mix_quant_lane<1>(xb, emax, m);
  uint32_t f = (quad_pos == 0 ? (uint32_t)(emax + 7) : 0u) | (m << (4 + 3 * quad_pos));
  *shared = quad_or_u32(f);
  *m_out = m;
  return word;
}

// ------------------------------------------------------------------ prefill softmax + P coding

constexpr int SM_NREG = 8;  // row chunks of 512 logits kept in registers (rows up to 4096 keys)

__device__ __forceinline__ void load8f(const float* p, float (&v)[8]) {
  float4 a = *(const float4*)p;
  float4 b = *(const float4*)(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void softmax_chunk(const float (&s)[8], int j0, int n_valid, float scale, float m,
                                              int64_t row, int Tp, float& lsum, uint8_t* pc, uint16_t* ps,
                                              float* dbg_p, int lane) {
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; e++) {
    float v = 0.f;
    if (j0 + e < n_valid) v = expf(__fsub_rn(__fmul_rn(s[e], scale), m));
    p[e] = v;
    lsum += v;
  }
  uint32_t sh, msub;
  uint32_t word = mix45_code8(p, lane & 3, &sh, &msub);
  *(uint32_t*)(pc + row * (int64_t)(Tp >> 1) + (j0 >> 1)) = word;
  if ((lane & 3) == 0) ps[row * (int64_t)(Tp >> 5) + (j0 >> 5)] = (uint16_t)sh;
  if (dbg_p) {
    float* d = dbg_p + row * (int64_t)Tp + j0;
    *(float4*)d = make_float4(p[0], p[1], p[2], p[3]);
    *(float4*)(d + 4) = make_float4(p[4], p[5], p[6], p[7]);
  }
}

// One wave per query row (h, i) of S [Hq, T, Tp]. Writes P^ codes [Hq, T, Tp/2] and shared
// [Hq, T, Tp/32] for keys [0, n_write), l [Hq, T]; masked keys are zero.
__global__ void __launch_bounds__(256) k_softmax_pquant(const float* __restrict__ S, int T, int Tp, int64_t nrows,
                                                         int causal, float scale, uint8_t* __restrict__ pc,
                                                         uint16_t* __restrict__ ps, float* __restrict__ l,
                                                         float* __restrict__ dbg_p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= nrows) return;
  const int i = (int)(row % T);
  const int n_valid = causal ? i + 1 : T;
  const int n_write = causal ? min(Tp, ((i + 1 + 255) / 256) * 256) : Tp;
  const float* srow = S + row * (int64_t)Tp;
  const int nit_valid = (n_valid + 511) / 512;
  const int nit_write = (n_write + 511) / 512;

  // all of the row's register chunks are requested before any is used
  float cache[SM_NREG][8];
#pragma unroll
  for (int it = 0; it < SM_NREG; it++) {
    const int j0 = it * 512 + lane * 8;
    if (it < nit_valid && j0 < n_valid) load8f(srow + j0, cache[it]);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int it = 0; it < SM_NREG; it++) {
    const int j0 = it * 512 + lane * 8;
    if (it < nit_valid && j0 < n_valid) {
#pragma unroll
      for (int e = 0; e < 8; e++)
        if (j0 + e < n_valid) mx = fmaxf(mx, cache[it][e]);
    }
  }
  for (int it = SM_NREG; it < nit_valid; it++) {
    int j0 = it * 512 + lane * 8;
    if (j0 < n_valid) {
      float v[8];
      load8f(srow + j0, v);
#pragma unroll
      for (int e = 0; e < 8; e++)
        if (j0 + e < n_valid) mx = fmaxf(mx, v[e]);
    }
  }
  mx = wave_max_f32(mx);
  const float m = __fmul_rn(mx, scale);  // rounding is monotone: max of z = fp32(max S * scale)

  float lsum = 0.f;
#pragma unroll
  for (int it = 0; it < SM_NREG; it++) {
    if (it < nit_write) {
      int j0 = it * 512 + lane * 8;
      if (j0 < n_write) {  // n_write is a multiple of 32: quads stay whole
        float v[8];
        if (it < nit_valid && j0 < n_valid) {
#pragma unroll
          for (int e = 0; e < 8; e++) v[e] = cache[it][e];
        } else {
#pragma unroll
          for (int e = 0; e < 8; e++) v[e] = 0.f;
        }
        softmax_chunk(v, j0, n_valid, scale, m, row, Tp, lsum, pc, ps, dbg_p, lane);
      }
    }
  }
  for (int it = SM_NREG; it < nit_write; it++) {
    int j0 = it * 512 + lane * 8;
    if (j0 < n_write) {
      float v[8];
      if (j0 < n_valid) load8f(srow + j0, v);
      else {
#pragma unroll
        for (int e = 0; e < 8; e++) v[e] = 0.f;
      }
      softmax_chunk(v, j0, n_valid, scale, m, row, Tp, lsum, pc, ps, dbg_p, lane);
    }
  }
  lsum = wave_sum_f32(lsum);
  if (lane == 0) l[row] = lsum;
}

// ------------------------------------------------------------------ prefill: fused S passes

// S = Q^ K^T is never stored. Pass 1 computes each query row's exact maximum over its unmasked
// keys; pass 2 recomputes S, turns it into p = exp(z - m), sums l and codes P^ (MiX-4.5b along
// keys). Workgroup: 4 waves, 64 query rows of one head (wave w: rows 16 w .. 16 w + 15), key tiles
// of 64. MFMA v_mfma_scale_f32_16x16x128_f8f6f4 over the whole head dimension (d = 128): its A
// operand is 16 keys of K^ (FP4, lane l = r + 16 g holds key r, elements [32 g, 32 g + 32)), its
// B operand 16 query rows of Q^ decoded to E4M3 (row r, elements [16 g, +16) and [64 + 16 g, +16)),
// so result register e of lane l is S[query r][key 4 g + e]: each lane holds, per 16-key group j,
// four consecutive keys of one query.
constexpr int PQ = 64;   // query rows per workgroup
constexpr int PK = 64;   // keys per tile

struct PrefillOps {
  const uint8_t* qc;     // Q^ codes [T, Hq, d/2]
  const uint16_t* qs;    // Q^ shared fields [T, Hq, d/32]
  const uint8_t* kc;     // K^ codes [T, Hkv, d/2]
  const uint8_t* ks;     // K^ scales [T, Hkv, d/32]
  const uint8_t* vc;     // V^ codes [Hkv, d, Tp/2] (blocks along tokens)
  const uint8_t* vs;     // V^ scales [Hkv, d, vsp] (vsp = Tp/32 rounded up to a multiple of 4; block Tp/32,
                         // when it is padding, holds 127)
  int T, Tp, Hq, Hkv, causal, vsp;
};

// Q^ operand of query row q (head h) for this lane's K group g, decoded from MiX codes to E4M3
__device__ __forceinline__ void q_operand(const PrefillOps& P, int q, int h, int g, v8i& qf, int& qsc) {
  const int64_t qrow = (int64_t)q * P.Hq + h;
  const uint8_t* qrc = P.qc + qrow * 64;
  const uint16_t* qrs = P.qs + qrow * 4;
  uint32_t o[8];
#pragma unroll
  for (int half = 0; half < 2; half++) {
    const int blk = (g >> 1) + 2 * half;   // elements [16 g + 64 half, +16): sub-blocks 2 (g & 1), 2 (g & 1) + 1
    const uint32_t sh = qrs[blk];
    const uint2 wv = *(const uint2*)(qrc + blk * 16 + (g & 1) * 8);
    mix8_to_e4m3(wv.x, (sh >> (4 + 3 * (2 * (g & 1)))) & 7u, o[4 * half + 0], o[4 * half + 1]);
    mix8_to_e4m3(wv.y, (sh >> (4 + 3 * (2 * (g & 1) + 1))) & 7u, o[4 * half + 2], o[4 * half + 3]);
  }
  qf = v8i{(int)o[0], (int)o[1], (int)o[2], (int)o[3], (int)o[4], (int)o[5], (int)o[6], (int)o[7]};
  qsc = (int)(qrs[g] & 15u) + 119;
}

// K^ tiles are staged in LDS once per workgroup (its 4 waves use the same 64 keys): a 2-stage ring
// filled by global_load_lds, the copy of tile t + 1 overlapping the use of tile t. A stage holds
// 64 keys x 64 code bytes, the 16-byte chunk g of key kl at slot g ^ kswz(kl), then the 64 x 4 scale
// bytes. On this part a ds_read_b128 takes its nominal four cycles when, within each half-wave, the
// 16-byte slots' indices mod 16 are a one-to-one function of lane bits 0-3 with lane bit 4 free (or
// of bits 0-2 and 4 with bit 3 free): a model fitted to SQ_LDS_BANK_CONFLICT counts of probe
// patterns. The MFMA operand read (lane r + 16 g: key 16 j + r, chunk g) has slot index mod 16 =
// 4 (r & 3) + (g ^ kswz(r)), one-to-one in lane bits 0, 1, 2, 4 for kswz(kl) = 2 bit2(kl); rows
// without the swizzle take twice the cycles. The copies keep four consecutive lanes on one key's
// 64 bytes, which the global loads need.
constexpr int KST = PK * 64 + PK * 4;
__device__ __forceinline__ int kswz(int kl) { return (kl >> 1) & 2; }

// a wave-uniform address as the scalar operand of a copy (the compiler may otherwise keep a value it
// computed inside a loop in vector registers)
__device__ __forceinline__ const uint8_t* sgpr_ptr(const uint8_t* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Lane offsets of the tile copies (relative to the tile's scalar base) for a tile with all 64 keys
// below T: computed once per workgroup, so an inner tile's copies cost no vector addressing.
struct KvOff {
  uint32_t k, ks;   // K^ codes (wave w: keys 16 w .. 16 w + 15) and scales (wave 0: key = lane)
  uint32_t v, vs;   // V^ codes (wave w: channels 32 w .. 32 w + 31) and scales (waves 0, 1)
};
__device__ __forceinline__ KvOff kv_offsets(const PrefillOps& P) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kl = 16 * wave + (lane >> 2), ch = 32 * wave + (lane >> 1);
  KvOff o;
  o.k = (uint32_t)(kl * P.Hkv * 64 + 16 * ((lane & 3) ^ kswz(kl)));
  o.ks = (uint32_t)(lane * P.Hkv * 4);
  o.v = (uint32_t)(ch * (P.Tp >> 1) + 16 * (lane & 1));
  o.vs = (uint32_t)((64 * wave + lane) * P.vsp);
  return o;
}

// wave w copies keys 16 w .. 16 w + 15 of the tile at k0 (keys past T repeat key T-1 and are
// masked later); wave 0 also copies the scales. Each copy reads from a wave-uniform base (the
// tile's first key of KV head hk) plus a 32-bit lane offset; only the last tile recomputes the
// offsets with its keys clamped.
__device__ __forceinline__ void k_stage(const PrefillOps& P, int hk, int k0, uint8_t* st, const KvOff& o) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t koff = o.k, ksoff = o.ks;
  if (k0 + PK > P.T) {
    const int kl = 16 * wave + (lane >> 2);
    const int lim = P.T - 1 - k0;   // the last key, relative to the tile
    koff = (uint32_t)(min(kl, lim) * P.Hkv * 64 + 16 * ((lane & 3) ^ kswz(kl)));
    ksoff = (uint32_t)(min(lane, lim) * P.Hkv * 4);
  }
  const uint8_t* kb = sgpr_ptr(P.kc + ((int64_t)k0 * P.Hkv + hk) * 64);
  dma16s(kb, koff, __builtin_amdgcn_readfirstlane(lds_addr(st + wave * 1024)));
  if (wave == 0) {
    const uint8_t* sb = sgpr_ptr(P.ks + ((int64_t)k0 * P.Hkv + hk) * 4);
    dma4s(sb, ksoff, __builtin_amdgcn_readfirstlane(lds_addr(st + PK * 64)));
  }
}

// S for the wave's 16 queries and the 64 keys of stage st
__device__ __forceinline__ void s_tile(const uint8_t* st, int r, int g, const v8i& qf, int qsc, v4f (&acc)[4]) {
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int kl = 16 * j + r;
    const uint4 kv = *(const uint4*)(st + kl * 64 + 16 * (g ^ kswz(kl)));
    const int ksc = st[PK * 64 + kl * 4 + g];
    const v8i kf = v8i{(int)kv.x, (int)kv.y, (int)kv.z, (int)kv.w, 0, 0, 0, 0};
    acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, qf, v4f{0.f, 0.f, 0.f, 0.f}, 4, 0, 0, ksc, 0, qsc);
  }
}

// Workgroup -> (query tile, head): heads vary fastest and, with the causal mask, the query tiles
// run from the last (most keys) to the first, so the longest workgroups start first.
__device__ __forceinline__ int q_tile(const PrefillOps& P) {
  return P.causal ? (int)(gridDim.y - 1 - blockIdx.y) : (int)blockIdx.y;
}

// Kernels whose MFMA results feed vector code are limited to 256 registers a wave (two waves per
// SIMD): the compiler then selects the MFMA forms that read and write ordinary VGPRs. With the
// whole 512-register file allowed it selects the accumulation-register forms and copies every
// product and every running sum between the two files on each key tile.
#define MIX_MFMA_VGPR __attribute__((amdgpu_waves_per_eu(2)))

// grid (Hq, ceil(T / 64)), block 256. smax [Hq, T]: max of S over the unmasked keys of each row.
// When every workgroup fits on the GPU at once (4096 tokens x 28 heads: 1792 workgroups, eight per CU),
// the pass lasts as long as its longest workgroups (the last query tiles, which see every key), whose
// time is a chain of per-iteration latencies: each iteration therefore takes two key tiles (a 4-slot
// ring, one barrier per pair of tiles).
__global__ void __launch_bounds__(256) MIX_MFMA_VGPR k_attn_rowmax(PrefillOps P, float* __restrict__ smax) {
  __shared__ __align__(16) uint8_t kst[4][KST];
  const int h = blockIdx.x, hk = h / (P.Hq / P.Hkv), qt = q_tile(P);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int q0w = qt * PQ + 16 * wave;
  const int q = q0w + r;
  v8i qf;
  int qsc;
  q_operand(P, min(q, P.T - 1), h, g, qf, qsc);
  const int nvalid = P.causal ? min(q + 1, P.T) : P.T;
  const int nfull = P.causal ? min(q0w + 1, P.T) : P.T;        // keys unmasked for all the wave's rows
  const int kend = P.causal ? min(qt * PQ + PQ, P.T) : P.T;    // keys any row of the tile sees
  const int nt = (kend + PK - 1) / PK;
  float mx = -INFINITY;
  const KvOff ko = kv_offsets(P);
  if (nt > 0) k_stage(P, hk, 0, kst[0], ko);
  if (nt > 1) k_stage(P, hk, PK, kst[1], ko);
  // the row maxima over key tile it, staged at st
  auto tile = [&](int it, const uint8_t* st) {
    const int k0 = it * PK;
    v4f acc[4];
    s_tile(st, r, g, qf, qsc, acc);
    if (k0 + PK <= nfull) {
#pragma unroll
      for (int j = 0; j < 4; j++) mx = fmaxf(fmaxf(mx, fmaxf(acc[j][0], acc[j][1])), fmaxf(acc[j][2], acc[j][3]));
    } else {
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int e = 0; e < 4; e++)
          if (k0 + 16 * j + 4 * g + e < nvalid) mx = fmaxf(mx, acc[j][e]);
    }
  };
  // key tiles it and it + 1 from ring slots 2 H and 2 H + 1 (H a constant, so the LDS addresses are
  // immediates)
  auto pair = [&](int it, auto half) {
    constexpr int H = decltype(half)::value;
    wait_vmcnt<0>();
    __syncthreads();   // both tiles are complete; every wave is done with the other two slots
    if (it + 2 < nt) k_stage(P, hk, (it + 2) * PK, kst[2 * (H ^ 1)], ko);
    if (it + 3 < nt) k_stage(P, hk, (it + 3) * PK, kst[2 * (H ^ 1) + 1], ko);
    tile(it, kst[2 * H]);
    if (it + 1 < nt) tile(it + 1, kst[2 * H + 1]);
  };
  for (int it = 0; it < nt; it += 4) {
    pair(it, std::integral_constant<int, 0>{});
    if (it + 2 < nt) pair(it + 2, std::integral_constant<int, 1>{});
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  if (g == 0 && q < P.T) smax[(int64_t)h * P.T + q] = mx;
}

// exp(x) for finite x <= 0 as 2^t (1 + c): t = fp32(x L2E) with L2E the fp32 rounding of log2 e,
// and c = x - t ln 2 (exact reals: e^x = 2^t e^(x - t ln 2)), formed by two fmas with ln 2 split
// into LN2_HI + LN2_LO (Cody-Waite): x - t LN2_HI is rounded once and is tiny, so c carries an
// absolute error near 2^-40. |c| < 2^-18 wherever 2^t is not zero, so e^c = 1 + c up to c^2 / 2
// (far below an ulp), and the hardware exp2 of t is within about an ulp: p is within about 2 ulp of
// the correctly rounded exponential for p >= 2^-126. Below that (x < -87.3) the hardware exp2 may
// return 0; such a p is under every P^ code threshold (at most 2^-15 below the block maximum, which
// is >= 2^-7) and under half an ulp of l >= 1, so no output depends on it. x = 0 gives 1 exactly.
__device__ __forceinline__ float exp_nonpos(float x) {
  constexpr float L2E = 1.44269502162933349609375f;         // fp32 rounding of log2 e
  constexpr float LN2_HI = 0.693147182464599609375f;        // fp32 rounding of ln 2
  constexpr float LN2_LO = -1.9046542121259335544891655e-9f;  // fp32 rounding of ln 2 - LN2_HI
  const float t = __fmul_rn(x, L2E);
  const float c = __fmaf_rn(-t, LN2_LO, __fmaf_rn(-t, LN2_HI, x));
  const float y = __builtin_amdgcn_exp2f(t);
  return __fmaf_rn(y, c, y);
}

// MiX-4.5b codes of 8 consecutive softmax weights p = a ++ b (non-negative, this lane's sub-block
// of a 32-key block whose 4 sub-blocks sit in the 4 lanes of a quad). Emax comes from the block's
// fp32 maximum and the lane's 3-bit mantissa from its sub-block maximum. Only the rule for
// non-negative elements applies: on the 16-bit patterns a' of the values rounded up (all
// thresholds are 16-bit patterns, so the decisions are those on the fp32 values),
// d* = clamp(((mu0 - a') >> 7) + 1, 0, 7), and d* = 7 codes 0xF above M 2^(Emax-8), else 0x7 (zero).
// Elements i and i + 4 are coded together as the two halves of a word, whose codes land in
// nibbles i and i + 4. Returns the code word and sets the block's 16-bit shared field.
__device__ __forceinline__ uint32_t p_code8(const float4& a, const float4& b, int quad_pos, uint32_t& shared) {
  const uint32_t x[8] = {f32_bits(a.x), f32_bits(a.y), f32_bits(a.z), f32_bits(a.w),
                         f32_bits(b.x), f32_bits(b.y), f32_bits(b.z), f32_bits(b.w)};
  const uint32_t lmax = max(max(max(x[0], x[1]), max(x[2], x[3])), max(max(x[4], x[5]), max(x[6], x[7])));
  const uint32_t bmax = quad_max_u32(lmax);
  const int emax = min(max((int)(bmax >> 23) - 127, -7), 8);
  const uint32_t m = mant3_of(lmax);
  const uint32_t t3 = 24u + 3u * m;   // mid_0 = 1.5 M 2^(Emax-1) = t3 2^(Emax-5)
  const uint32_t mu = t3 < 32u ? (((uint32_t)(emax + 126) << 7) | ((t3 << 3) & 0x7Fu))
                               : (((uint32_t)(emax + 127) << 7) | ((t3 << 2) & 0x7Fu));
  const uint32_t pb = ((uint32_t)(emax + 119) << 7) | (m << 4);   // M 2^(Emax-8)
  const i16x2 MU1 = __builtin_bit_cast(i16x2, (mu + 128u) * 0x00010001u);
  const u16x2 PB2 = __builtin_bit_cast(u16x2, pb * 0x00010001u);
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t w = __builtin_amdgcn_perm(x[i + 4] + 0xFFFFu, x[i] + 0xFFFFu, 0x07060302u);
    i16x2 c = (MU1 - __builtin_bit_cast(i16x2, w)) >> (i16x2)7;
    c = __builtin_elementwise_min(__builtin_elementwise_max(c, (i16x2)0), (i16x2)7);
    const u16x2 cu = __builtin_bit_cast(u16x2, c);
    const u16x2 gt = (PB2 - __builtin_bit_cast(u16x2, w)) >> (u16x2)15;   // a' > pb
    const u16x2 e7 = (cu + (u16x2)1) >> (u16x2)3;                          // d* == 7
    const uint32_t c2 = __builtin_bit_cast(uint32_t, cu | ((gt & e7) << (u16x2)3));
    word |= c2 << (4 * i);
  }
  shared = quad_or_u32((quad_pos == 0 ? (uint32_t)(emax + 7) : 0u) | (m << (4 + 3 * quad_pos)));
  return word;
}

// p_code8 that also returns the 8 E4M3 bytes of the coded values in element order (the MFMA
// operand of P^ V^): 64 + m - 8 d for a nonzero code d, 0 for zero; the debug path's coder.
// The thresholds are those of p_code8 with the biased exponent eb = Emax + 127 folded in:
// mu0 + 128 = 128 eb + 64 + D(m), where D(m) is the low part of the 16-bit pattern of the first
// midpoint 1.5 M 2^(Emax-1) (D = 24 m below m = 3, where the midpoint stays in binade Emax - 1, and
// 12 m + 32 from m = 3 on, where it reaches binade Emax), looked up from an 8-byte table by v_perm.
__device__ __forceinline__ uint32_t pd_of(uint32_t m) {
  return __builtin_amdgcn_perm(0x74685C50u, 0x44301800u, m | 0x0C0C0C00u);
}
__device__ __forceinline__ uint32_t p_code8_img(const float4& a, const float4& b, int quad_pos, uint32_t& shared,
                                                uint32_t& out0, uint32_t& out1) {
  const uint32_t x[8] = {f32_bits(a.x), f32_bits(a.y), f32_bits(a.z), f32_bits(a.w),
                         f32_bits(b.x), f32_bits(b.y), f32_bits(b.z), f32_bits(b.w)};
  const uint32_t lmax = max(max(max(x[0], x[1]), max(x[2], x[3])), max(max(x[4], x[5]), max(x[6], x[7])));
  const uint32_t bmax = quad_max_dpp(lmax);
  const uint32_t eb = min(max(bmax >> 23, 120u), 135u);   // Emax + 127, Emax in [-7, 8]
  const uint32_t m = mant3_of(lmax);
  const i16x2 MU1 = __builtin_bit_cast(i16x2, ((eb << 7) + pd_of(m) + 64u) * 0x00010001u);
  const u16x2 M64 = __builtin_bit_cast(u16x2, (64u + m) * 0x00010001u);
  // a' > pb = M 2^(Emax-8) = 128 (eb - 8) + 16 m exactly when a' + (0x7FFF - pb) has bit 15 set
  // (a' and pb are below 2^15: p is non-negative and at most 1)
  const u16x2 NPB = __builtin_bit_cast(u16x2, (33791u - (((eb << 3) + m) << 4)) * 0x00010001u);
  uint32_t word = 0, im[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t w = __builtin_amdgcn_perm(x[i + 4] + 0xFFFFu, x[i] + 0xFFFFu, 0x07060302u);
    i16x2 c = (MU1 - __builtin_bit_cast(i16x2, w)) >> (i16x2)7;
    c = __builtin_elementwise_min(__builtin_elementwise_max(c, (i16x2)0), (i16x2)7);
    const u16x2 cu = __builtin_bit_cast(u16x2, c);
    // nz = 1 where the element codes nonzero (a' > pb; pb lies below the midpoint between the
    // dE = 6 and dE = 7 values, so every element at or below it has d* = 7 and codes to zero)
    const u16x2 nz = (__builtin_bit_cast(u16x2, w) + NPB) >> (u16x2)15;
    const u16x2 e7 = (cu + (u16x2)1) >> (u16x2)3;                          // d* == 7
    word |= __builtin_bit_cast(uint32_t, cu | ((nz & e7) << (u16x2)3)) << (4 * i);
    // the byte 64 + m - 8 d* (16-bit arithmetic: + d* 0xFFF8), times nz; elements i in the low half,
    // i + 4 in the high half
    im[i] = __builtin_bit_cast(uint32_t, (M64 + cu * (u16x2)0xFFF8u) * nz);
  }
  out0 = __builtin_amdgcn_perm(im[1], im[0], 0x0C0C0400u) | __builtin_amdgcn_perm(im[3], im[2], 0x04000C0Cu);
  out1 = __builtin_amdgcn_perm(im[1], im[0], 0x0C0C0602u) | __builtin_amdgcn_perm(im[3], im[2], 0x06020C0Cu);
  shared = quad_or_dpp((quad_pos == 0 ? eb - 120u : 0u) | (m << (4 + 3 * quad_pos)));
  return word;
}

// The E4M3 bytes of p_code8_img without the code words (the production path): the same decisions,
// rearranged into fewer instructions. With a' the rounded-up 16-bit pattern of p and MU1 = mu0 + 128
// (the pattern of 1.5 M 2^Emax), p_code8_img takes d* = clamp((MU1 - a') >> 7, 0, 7). Here
// MU1 - a' >= 0 always: p <= lmax < (M + 1/8) 2^E(lmax) <= 1.5 M 2^Emax, since M is lmax's mantissa
// cut to 3 bits and Emax >= E(lmax) (p <= 1 never meets the upper clamp of Emax), so d* needs no
// lower clamp. The byte 64 + m - 8 d* is 8 (8 - d*) + m, and 8 - d* = max(e, 1) with
// e = (a' + 1151 - MU1) >> 7 (8 - floor(n / 128) = floor((1151 - n) / 128) for an integer n). a' + K for
// a block constant K is the high half of the one 32-bit sum x + (K << 16) + 0xFFFF. The element codes
// nonzero where a' > pb, i.e. where (pb + 1151 - MU1) - (a' + 1151 - MU1) < 0; pb + 1151 - MU1 =
// 63 + 16 m - D(m) does not depend on Emax. A subnormal sub-block maximum (below 2^-126) has no
// element above pb >= 2^-15, so its m may be the raw field bits. Elements pair up as (2i, 2i + 1).
// Returns eb = Emax + 127.
__device__ __forceinline__ uint32_t p_img8(const float4& a, const float4& b, uint32_t& out0, uint32_t& out1) {
  const uint32_t x[8] = {f32_bits(a.x), f32_bits(a.y), f32_bits(a.z), f32_bits(a.w),
                         f32_bits(b.x), f32_bits(b.y), f32_bits(b.z), f32_bits(b.w)};
  const uint32_t lmax = max(max(max(max(max(x[0], x[1]), x[2]), max(max(x[3], x[4]), x[5])), x[6]), x[7]);
  const uint32_t bmax = quad_max_dpp(lmax);
  const uint32_t eb = min(max(bmax >> 23, 120u), 135u);
  const uint32_t m = (lmax >> 20) & 7u;
  const uint32_t dm = pd_of(m);
  const uint32_t m2 = m * 0x00010001u;
  const uint32_t c2 = 0x043FFFFFu - ((dm << 16) + (eb << 23));   // ((1151 - MU1) << 16) + 0xFFFF
  // 63 + 16 m - D(m) for m = 0..7 in both halves, from a byte table
  const i16x2 PK = __builtin_bit_cast(i16x2, __builtin_amdgcn_perm(0x3B37332Fu, 0x2B2F373Fu, m2 | 0x0C000C00u));
  uint32_t im[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const i16x2 v = __builtin_bit_cast(i16x2, __builtin_amdgcn_perm(x[2 * i + 1] + c2, x[2 * i] + c2, 0x07060302u));
    const i16x2 e = __builtin_elementwise_max(v >> (i16x2)7, (i16x2)1);
    const uint32_t nzm = __builtin_bit_cast(uint32_t, (PK - v) >> (i16x2)15);
    im[i] = ((__builtin_bit_cast(uint32_t, e) << 3) | m2) & nzm;   // e <= 8: no carry across halves
  }
  out0 = __builtin_amdgcn_perm(im[1], im[0], 0x06040200u);
  out1 = __builtin_amdgcn_perm(im[3], im[2], 0x06040200u);
  return eb;
}

// p = exp(fp32(S scale) - fp32(m scale)) of the lane's 16 scores into the wave's LDS p row, masked
// keys (key >= nvalid) as 0 unless the whole tile is unmasked (FULL); returns their sum.
template <bool FULL>
__device__ __forceinline__ float p_tile(const v4f (&acc)[4], float scale, float mz, int k0, int g, int nvalid,
                                        float* prow) {
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    float pv[4];
#pragma unroll
    for (int e = 0; e < 4; e++) {
      pv[e] = exp_nonpos(__fsub_rn(__fmul_rn(acc[j][e], scale), mz));
      if (!FULL && k0 + 16 * j + 4 * g + e >= nvalid) pv[e] = 0.f;
      sum += pv[e];
    }
    *(float4*)(prow + 16 * j + 4 * g) = make_float4(pv[0], pv[1], pv[2], pv[3]);
  }
  return sum;
}

// The V^ tile of 64 keys in LDS: 128 channel rows of 32 bytes in plain order (the operand read, lane
// r + 16 g: channel 16 t + r, chunk g & 1, meets the conflict-free form described at the K^ tile);
// then one scale dword per channel (the four 32-token blocks from floor(k0 / 128)).
constexpr int VST = 128 * 32 + 128 * 4;
constexpr int FST = KST + VST;   // one ring stage: the K^ tile, then the V^ tile

// wave w copies the V^ codes of channels 32 w .. 32 w + 31; waves 0 and 1 the scale dwords.
// When the tile's upper half lies past Tp (Tp is a multiple of 32, so only in the last tile) every
// chunk repeats chunk 0; those keys have p = 0.
__device__ __forceinline__ void v_stage(const PrefillOps& P, int hk, int k0, uint8_t* st, const KvOff& o) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t voff = o.v;
  if (k0 + PK > P.Tp) voff = (uint32_t)((32 * wave + (lane >> 1)) * (P.Tp >> 1));
  const uint8_t* vb = sgpr_ptr(P.vc + (int64_t)hk * 128 * (P.Tp >> 1) + (k0 >> 1));
  dma16s(vb, voff, __builtin_amdgcn_readfirstlane(lds_addr(st + wave * 1024)));
  if (wave < 2) {
    const uint8_t* sb = sgpr_ptr(P.vs + (int64_t)hk * 128 * P.vsp + ((k0 >> 5) & ~3));
    dma4s(sb, o.vs, __builtin_amdgcn_readfirstlane(lds_addr(st + 128 * 32 + wave * 256)));
  }
}

// The wave's P^ tile (16 query rows x 64 keys, E4M3) in LDS: row r's 16-byte chunk c (keys
// 16 c .. 16 c + 15) at byte 256 c + 16 r, so that the MFMA operand read (lane r + 16 g: row r,
// chunk g) is in lane order; the block scales (E8M0 2^(Emax-1)) of the rows' two 32-key blocks
// after the 1 KB of codes.

// grid (Hq, ceil(T / 64)), block 256. For d = 128: recomputes S tile by tile, forms p with the row
// maxima of k_attn_rowmax, codes P^ (MiX-4.5b along keys) and accumulates O^T += V^ P^ on the MFMA,
// then writes O = (P^ V^) / l rounded to bf16 [T, Hq, d] and l [Hq, T]. P^ codes [Hq, T, Tp/2] and
// shared fields [Hq, T, Tp/32] are written only when pc is given (for keys
// [0, min(Tp, round_up(i + 1, 256))) of row i, all Tp without the mask; masked keys code as zero);
// optional S and p dumps [Hq, T, Tp].
// PV: v_mfma_scale_f32_16x16x128_f8f6f4 with V^ (FP4, 16 channels) as A and P^ (E4M3, 16 queries)
// as B, the tile's 64 keys as K elements [0, 64) and zeros above; result register e of lane
// r + 16 g is O^T[channel 4 g + e][query r].
// Four workgroups per CU (39.5 KB of LDS each): at most 128 registers a wave, which also selects the
// VGPR forms of the MFMAs (the debug instantiation spills at that limit).
template <bool DBG>   // DBG: the debug dumps (S, p, P^ codes and shared fields) are written
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) k_attn_pcode(PrefillOps P, const float* __restrict__ smax, float scale,
                                                     uint16_t* __restrict__ o, uint8_t* __restrict__ pc,
                                                     uint16_t* __restrict__ ps, float* __restrict__ l,
                                                     float* __restrict__ dbg_s, float* __restrict__ dbg_p) {
  constexpr int PP = PK + 4;                     // padded LDS row (floats)
  __shared__ __align__(16) float sp[4][16][PP];  // each wave's p tile: 16 rows x 64 keys
  __shared__ __align__(16) uint8_t fst[2][FST];  // K^ and V^ tiles, two stages
  __shared__ __align__(16) uint8_t spb[4][16 * 64 + 16 * 2];   // each wave's P^ tile and block scales
  const int h = blockIdx.x, hk = h / (P.Hq / P.Hkv), qt = q_tile(P);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int q0w = qt * PQ + 16 * wave;   // the wave's first query row
  const int q = q0w + r;
  v8i qf;
  int qsc;
  q_operand(P, min(q, P.T - 1), h, g, qf, qsc);
  const int nvalid = P.causal ? min(q + 1, P.T) : P.T;
  const int nfull = P.causal ? min(q0w + 1, P.T) : P.T;
  const float mz = q < P.T ? __fmul_rn(smax[(int64_t)h * P.T + min(q, P.T - 1)], scale) : 0.f;
  const int qlast = min(qt * PQ + PQ, P.T) - 1;
  const int kend = P.causal ? qlast + 1 : P.T;                                    // keys with some unmasked entry
  const int kwrite = P.causal ? min(P.Tp, (qlast + 1 + 255) / 256 * 256) : P.Tp;  // keys whose codes are written
  float lsum = 0.f;
  v4f acc_o[8];
#pragma unroll
  for (int t = 0; t < 8; t++) acc_o[t] = v4f{0.f, 0.f, 0.f, 0.f};
  uint8_t* pbw = spb[wave];
  // read-back role: row rr = lane / 8 (+ 8 per pass), 8 keys kk = 8 (lane % 8); quads are 32-key blocks
  const int rr0 = lane >> 3, kk = 8 * (lane & 7);
  const int64_t crow0 = (int64_t)h * P.T + q0w + rr0;   // P^ row of pass 0 (pass 1: + 8)
  const bool st0 = q0w + rr0 < P.T, st1 = q0w + rr0 + 8 < P.T;
  // a tile's codes (debug) are stored at the start of the next tile (after its barrier) so that
  // the copy wait before the barrier does not wait for them
  uint32_t cw[2] = {0, 0}, cs[2] = {0, 0};
  int kprev = -1;
  auto store_codes = [&](int key) {   // Tp is a multiple of 32: quads stay whole
    if (key < P.Tp) {
#pragma unroll
      for (int pass = 0; pass < 2; pass++) {
        if (pass == 0 ? st0 : st1) {
          const int64_t row = crow0 + 8 * pass;
          *(uint32_t*)(pc + row * (P.Tp >> 1) + (key >> 1)) = cw[pass];
          if ((lane & 3) == 0) ps[row * (P.Tp >> 5) + (key >> 5)] = (uint16_t)cs[pass];
        }
      }
    }
  };
  const int ntc = (kend + PK - 1) / PK, nt = (kwrite + PK - 1) / PK;
  const KvOff ko = kv_offsets(P);
  if (ntc > 0) {
    k_stage(P, hk, 0, fst[0], ko);
    v_stage(P, hk, 0, fst[0] + KST, ko);
  }
  // one key tile from ring stage SG (a constant, so its LDS addresses are immediates)
  auto tile = [&](int it, auto stage) {
    constexpr int SG = decltype(stage)::value;
    const int k0 = it * PK;
    wait_vmcnt<0>();
    __syncthreads();
    if (DBG && pc && kprev >= 0) store_codes(kprev);
    if (it + 1 < ntc) {
      k_stage(P, hk, k0 + PK, fst[SG ^ 1], ko);
      v_stage(P, hk, k0 + PK, fst[SG ^ 1] + KST, ko);
    }
    const uint8_t* st = fst[SG];
    v4f acc[4];
    s_tile(st, r, g, qf, qsc, acc);
    if (k0 + PK <= nfull)
      lsum += p_tile<true>(acc, scale, mz, k0, g, nvalid, sp[wave][r]);
    else
      lsum += p_tile<false>(acc, scale, mz, k0, g, nvalid, sp[wave][r]);
    if (DBG && (dbg_s || dbg_p)) {
      const float* prow = sp[wave][r];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int key0 = k0 + 16 * j + 4 * g;
        if (q < P.T && key0 < P.Tp) {
          const int64_t oi = ((int64_t)h * P.T + q) * P.Tp + key0;
          if (dbg_s) *(float4*)(dbg_s + oi) = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
          if (dbg_p) *(float4*)(dbg_p + oi) = *(const float4*)(prow + 16 * j + 4 * g);
        }
      }
    }
    // code P^ from the wave's own tile (LDS is in order within a wave; no workgroup barrier) into
    // the wave's E4M3 tile; the code words and shared fields only for the debug dump
    auto code_pass = [&](auto codes, int pass) {
      const int rr = rr0 + 8 * pass;
      const float4 a = *(const float4*)&sp[wave][rr][kk];
      const float4 b = *(const float4*)&sp[wave][rr][kk + 4];
      uint32_t e0, e1, eb;
      if (decltype(codes)::value) {
        uint32_t sh;
        cw[pass] = p_code8_img(a, b, lane & 3, sh, e0, e1);
        cs[pass] = sh;
        eb = (sh & 15u) + 120u;
      } else {
        eb = p_img8(a, b, e0, e1);
      }
      *(uint2*)(pbw + 256 * (kk >> 4) + 16 * rr + (kk & 8)) = make_uint2(e0, e1);
      if ((lane & 3) == 0) pbw[16 * 64 + rr * 2 + (kk >> 5)] = (uint8_t)(eb - 1u);   // E8M0 2^(Emax-1)
    };
    if (DBG && pc) {
      code_pass(std::true_type{}, 0);
      code_pass(std::true_type{}, 1);
    } else {
      code_pass(std::false_type{}, 0);
      code_pass(std::false_type{}, 1);
    }
    kprev = k0 + kk;
    // O^T += V^ P^ over the tile's keys
    const uint4 pb = *(const uint4*)(pbw + 256 * g + 16 * r);
    const v8i pf = v8i{(int)pb.x, (int)pb.y, (int)pb.z, (int)pb.w, 0, 0, 0, 0};
    // Lane g gives the scale of K block g. Blocks 2 and 3 (K elements [64, 128)) are zero in P^, so
    // lanes g = 2, 3 may take any finite scale: they read the same bytes as lanes g - 2.
    const int psc = pbw[16 * 64 + r * 2 + (g & 1)];
    // V^ lanes g = 2, 3 carry K elements [64, 128) with the data of lanes g - 2 (finite FP4, times the
    // zeros of P^). When the tile's upper 32 keys lie past Tp (the last tile only), K block 1 reads the
    // scale byte after the last block, which the V coder sets to 127 (scale 1): its P^ is 0.
    const uint8_t* sv = st + KST;
    const int vblk = ((k0 >> 5) & 3) + (g & 1);              // byte of this lane's block in the dword
#pragma unroll
    for (int t = 0; t < 8; t++) {
      const int ch = 16 * t + r;
      const uint4 vf = *(const uint4*)(sv + ch * 32 + 16 * (g & 1));
      const int vsc = sv[128 * 32 + ch * 4 + vblk];
      const v8i vfa = v8i{(int)vf.x, (int)vf.y, (int)vf.z, (int)vf.w, 0, 0, 0, 0};
      acc_o[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vfa, pf, acc_o[t], 4, 0, 0, vsc, 0, psc);
      __builtin_amdgcn_sched_barrier(0);   // one V^ fragment live at a time
    }
  };
  for (int it = 0; it < ntc; it += 2) {
    tile(it, std::integral_constant<int, 0>{});
    if (it + 1 < ntc) tile(it + 1, std::integral_constant<int, 1>{});
  }
  if (DBG && pc) {
    if (kprev >= 0) store_codes(kprev);
    // tiles past every unmasked key of the tile rows: all-zero blocks (codes 0x7, shared field 0)
    cw[0] = cw[1] = 0x77777777u;
    cs[0] = cs[1] = 0u;
    for (int it = ntc; it < nt; it++) store_codes(it * PK + kk);
  }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (q < P.T) {
    if (g == 0) l[(int64_t)h * P.T + q] = lsum;
    uint16_t* orow = o + ((int64_t)q * P.Hq + h) * 128 + 4 * g;
#pragma unroll
    for (int t = 0; t < 8; t++) {
      const uint32_t lo = (uint32_t)f32_to_bf16_rne(__fdiv_rn(acc_o[t][0], lsum)) |
                          ((uint32_t)f32_to_bf16_rne(__fdiv_rn(acc_o[t][1], lsum)) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_rne(__fdiv_rn(acc_o[t][2], lsum)) |
                          ((uint32_t)f32_to_bf16_rne(__fdiv_rn(acc_o[t][3], lsum)) << 16);
      *(uint2*)(orow + 16 * t) = make_uint2(lo, hi);
    }
  }
}

// ------------------------------------------------------------------ decode: scores (pass 1)
//
// Decode attends the G = Hq/Hkv query rows of each (sequence b, KV head h) over keys [0, pos[b]]
// in chunks of DCH keys, in three launches. The first (scores) has one workgroup per chunk, which
// codes the query rows and writes S and the chunk maxima, and one more per (b, h), which appends
// the new key and value. The second (pv) turns S into p and P^ with the row maximum over all
// chunks, multiplies P^ by V^ on the MFMA and writes the chunk's partial sums; the third adds the
// partials of all chunks in chunk order into O. The exact global maximum is what P^ needs, and it
// is known only once every chunk's scores exist, hence the launch boundaries and the S round trip.
// (A last-arriving workgroup could combine inside the pv launch, but making the partials visible
// across CUs takes an agent-scope release and acquire per workgroup, which write back and
// invalidate the L2: far dearer on this part than a third launch.)
//
// The full decode step (mix_decode_step) puts its independent work into the same launches as
// further workgroups: the first also codes the linear's activation rows into their A image, a later
// one also streams the weights (gemv_block), so the weight stream and the KV-cache stream run side
// by side instead of one after the other.

constexpr int DCH = 256;  // keys per chunk

// Decode workgroup -> (chunk, KV head h, sequence b) from a role-local index vb over 8 per
// ceil(B Hkv / 8) groups of `per` workgroups. Workgroups are spread over the 8 XCDs round-robin
// (each role starts at a multiple of 8, so vb and the hardware index agree modulo 8), so the chunks
// of one (b, h) get ids equal modulo 8: they run on one XCD and share its L2 for the per-channel
// value scales (one 128-byte line serves 16 chunks), the chunk maxima, S and the chunk partials.
struct DecWg {
  int chunk, h, b;
  bool valid;
};
__device__ __forceinline__ DecWg dec_wg(int vb, int per, int Hkv, int B) {
  const int x = vb & 7, i = vb >> 3;
  const int bh = x + 8 * (i / per);
  DecWg w;
  w.chunk = i % per;
  w.b = bh / Hkv;
  w.h = bh - w.b * Hkv;
  w.valid = bh < B * Hkv;
  return w;
}

// The new key of a (sequence, KV head): MXFP4 of fp32(k - mu) along the head dimension, thread c
// of the first two waves holding channel c (a 32-channel block is half a wave). Even threads get
// the code byte of channels (c, c + 1); threads 0, 32, 64, 96 also the block's E8M0 scale.
__device__ __forceinline__ void new_key_code(uint32_t kraw, float muc, uint32_t& byte, uint32_t& scale) {
  const uint32_t kb = f32_bits(__fsub_rn(__uint_as_float(kraw << 16), muc));
  uint32_t amax = kb & 0x7FFFFFFFu;
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off, 32));
  const int X = mx_exponent(amax, 1);
  const uint32_t nib = amax ? fp4_code(kb, fp4_thresholds(X)) : 0u;
  byte = nib | ((uint32_t)__shfl_down((int)nib, 1, 32) << 4);
  scale = amax ? (uint32_t)(X + 127) : 0u;
}

// Arguments of both decode passes (d = 128, G <= 16).
struct DecOps {
  const uint16_t* q;        // [B, Hq, d] bf16
  const uint16_t* k_new;    // [B, Hkv, d]
  const uint16_t* v_new;    // [B, Hkv, d]
  const float* mu;          // [B, Hkv, d]
  const int32_t* pos;       // [B]
  int64_t max_pos, Lmax, Lp;
  int Hq, Hkv, B, nchunk;
  uint8_t* kc;              // cache K codes [B, Hkv, Lmax, d/2]
  uint8_t* ks;              //   scales [B, Hkv, Lmax, d/32]
  uint8_t* vc;              // cache V codes [B, Hkv, d, Lmax/2]
  uint8_t* vs;              //   scales [B, Hkv, d, Lmax/32]
  uint16_t* stage;          // [B, 32, Hkv, d] bf16
  float* S;                 // [B, Hq, Lp]
  float* pmax;              // [B, Hq, nchunk]
  float* lpart;             // [B, Hq, nchunk]
  float* opart;             // [B, Hq, nchunk, d]
  float scale;              // fp32(1 / sqrt(d))
  uint16_t* o;              // [B, Hq, d] bf16
  // debug dumps (NULL when not wanted)
  uint8_t* pc;              // [B, Hq, Lp/2]
  uint16_t* ps;             // [B, Hq, Lp/32]
  float* dbg_p;             // [B, Hq, Lp]
  float* dbg_l;             // [B, Hq]
};

// Scores pass, workgroup vb of 8 (nchunk + 1) ceil(B Hkv / 8) (dec_wg over nchunk + 1 per (b, h)),
// 256 threads. Workgroup `nchunk` of (b, h) appends the new token to the cache: the new key's codes into slot pos; the new value into the staging rows
// and the value block that holds pos re-coded along tokens from the staged tokens present (zero
// for the rest). The others, one per chunk of 256 keys (4 waves x 64 keys):
// 1. code the G query rows of this KV head: MiX-4.5b along the head dimension, decoded to the
//    MFMA's E4M3 operand (per-block E8M0 scale 2^(Emax-1)) in LDS;
// 2. the chunk that holds pos codes the new key too and uses it in place of the slot's contents;
// 3. write S [B, Hq, Lp] fp32 for keys <= pos and the chunk maxima pmax [B, Hq, nchunk]. Cache rows
//    past pos are never used: their loads are clamped to row pos and their products discarded.
__device__ __forceinline__ void dec_scores(const DecOps& a, int vb) {
  constexpr int d = 128;
  const DecWg wg = dec_wg(vb, a.nchunk + 1, a.Hkv, a.B);
  if (!wg.valid) return;
  const int h = wg.h, b = wg.b, Hkv = a.Hkv, Hq = a.Hq;
  const int64_t Lmax = a.Lmax;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t bh = (int64_t)b * Hkv + h;
  const int p = a.pos[b];
  if (p < 0 || p > a.max_pos) return;

  if (wg.chunk == a.nchunk) {
    // append: loads first (key channel, mean, value channel, the 16 staged rows of this thread)
    const int c = tid >> 1, half = tid & 1, slot = p & 31;
    const uint32_t kraw = a.k_new[bh * d + (tid & (d - 1))];
    const float muc = a.mu[bh * d + (tid & (d - 1))];
    const uint16_t vnew = a.v_new[bh * d + c];
    uint32_t u[16];
#pragma unroll
    for (int i = 0; i < 16; i++) u[i] = a.stage[(((int64_t)b * 32 + 16 * half + i) * Hkv + h) * d + c];
    if (tid < d) {
      uint32_t byte, sc;
      new_key_code(kraw, muc, byte, sc);
      const int64_t krow = bh * Lmax + p;
      if ((tid & 1) == 0) a.kc[krow * (d >> 1) + (tid >> 1)] = (uint8_t)byte;
      if ((tid & 31) == 0) a.ks[krow * (d >> 5) + (tid >> 5)] = (uint8_t)sc;
    }
    // value: thread -> (channel c, tokens [16 half, +16) of the block)
    uint32_t vmax = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int s2 = 16 * half + i;
      u[i] = s2 < slot ? u[i] << 16 : (s2 == slot ? (uint32_t)vnew << 16 : 0u);
      vmax = max(vmax, u[i] & 0x7FFFFFFFu);
    }
    vmax = max(vmax, (uint32_t)__shfl_xor((int)vmax, 1, 64));
    if (half == (slot >> 4)) a.stage[(((int64_t)b * 32 + slot) * Hkv + h) * d + c] = vnew;
    const int XV = mx_exponent(vmax, 1);
    uint32_t w0 = 0, w1 = 0;
    if (vmax) {
      const Fp4Thr thr = fp4_thresholds(XV);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        w0 |= fp4_code(u[i], thr) << (4 * i);
        w1 |= fp4_code(u[8 + i], thr) << (4 * i);
      }
    }
    const int64_t vrow = bh * d + c;
    *(uint2*)(a.vc + vrow * (Lmax >> 1) + (p >> 5) * 16 + 8 * half) = make_uint2(w0, w1);
    if (half == 0) a.vs[vrow * (Lmax >> 5) + (p >> 5)] = vmax ? (uint8_t)(XV + 127) : (uint8_t)0;
    return;
  }

  const int chunk = wg.chunk;
  if (chunk * DCH > p) return;
  const int G = Hq / Hkv;
  const int r = lane & 15, g = lane >> 4;
  const bool owner = chunk == p / DCH;
  __shared__ float smax[4][16];
  __shared__ __align__(16) uint8_t sq[16][d];   // query rows as E4M3
  __shared__ uint8_t sqs[16][4];                // their E8M0 block scales
  __shared__ __align__(16) uint8_t snk[d / 2];  // the new key's codes
  __shared__ uint8_t snks[d / 32];

  // loads first: K fragments of the wave's 4 groups of 16 keys, the query sub-block, the new key
  uint4 kv[4];
  int ksc[4];
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const int j = min(chunk * DCH + wave * 64 + t * 16 + r, p);
    kv[t] = *(const uint4*)(a.kc + (bh * Lmax + j) * 64 + g * 16);
    ksc[t] = a.ks[(bh * Lmax + j) * 4 + g];
  }
  const int qr = tid >> 4, qsb = tid & 15;   // query row, 8-element sub-block (quads are blocks)
  const uint4 qv = *(const uint4*)(a.q + ((int64_t)b * Hq + (int64_t)h * G + min(qr, G - 1)) * d + qsb * 8);
  const uint32_t kraw = a.k_new[bh * d + (tid & (d - 1))];
  const float muc = a.mu[bh * d + (tid & (d - 1))];
  // 1. query operand
  if (qr < G) {
    const uint32_t w4[4] = {qv.x, qv.y, qv.z, qv.w};
    int emax;
    uint32_t m, e0, e1;
    mix_quant_lane_bf16_img<1, true>(w4, emax, m, e0, e1);
    *(uint2*)&sq[qr][qsb * 8] = make_uint2(e0, e1);
    if ((qsb & 3) == 0) sqs[qr][qsb >> 2] = (uint8_t)(emax + 126);
  }
  // 2. new key
  if (owner && tid < d) {
    uint32_t byte, sc;
    new_key_code(kraw, muc, byte, sc);
    if ((tid & 1) == 0) snk[tid >> 1] = (uint8_t)byte;
    if ((tid & 31) == 0) snks[tid >> 5] = (uint8_t)sc;
  }
  __syncthreads();

  // A operand: query row r (rows past G repeat row G-1; their results are discarded), bytes
  // [16 g, +16) and [64 + 16 g, +16)
  const int rq = min(r, G - 1);
  const uint4 qlo = *(const uint4*)&sq[rq][16 * g];
  const uint4 qhi = *(const uint4*)&sq[rq][64 + 16 * g];
  const v8i af = v8i{(int)qlo.x, (int)qlo.y, (int)qlo.z, (int)qlo.w, (int)qhi.x, (int)qhi.y, (int)qhi.z, (int)qhi.w};
  const int sa = sqs[rq][g];

  float rmax[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const int j0 = chunk * DCH + wave * 64 + t * 16;
    const int j = j0 + r;
    const bool live = j <= p;
    if (owner && j == p) {
      kv[t] = *(const uint4*)&snk[16 * g];
      ksc[t] = snks[g];
    }
    const v8i bf = live ? v8i{(int)kv[t].x, (int)kv[t].y, (int)kv[t].z, (int)kv[t].w, 0, 0, 0, 0}
                        : v8i{0, 0, 0, 0, 0, 0, 0, 0};
    const int sb = live ? ksc[t] : 127;
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf, acc, 0, 4, 0, sa, 0, sb);
    // result register i: query row 4 g + i, key j0 + r
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int row = 4 * g + i;
      if (row < G && live) {
        a.S[((int64_t)b * Hq + (int64_t)h * G + row) * a.Lp + j] = acc[i];
        rmax[i] = fmaxf(rmax[i], acc[i]);
      }
    }
  }
  // max over the 16 lanes that share a query row (lane bits 0..3)
#pragma unroll
  for (int i = 0; i < 4; i++) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) rmax[i] = fmaxf(rmax[i], __shfl_xor(rmax[i], off, 64));
  }
  if (r == 0) {
#pragma unroll
    for (int i = 0; i < 4; i++) smax[wave][4 * g + i] = rmax[i];
  }
  __syncthreads();
  if (tid < G) {
    const float v = fmaxf(fmaxf(smax[0][tid], smax[1][tid]), fmaxf(smax[2][tid], smax[3][tid]));
    a.pmax[((int64_t)b * Hq + (int64_t)h * G + tid) * a.nchunk + chunk] = v;
  }
}

// The linear's activation rows coded into their A image inside the scores launch (the full decode
// step): M <= 16 rows of K bf16 values, row pitch ldx; a lane codes one 8-element sub-block (a quad
// is a 32-element block, a 16-lane DPP row one 128-wide K step) exactly as mix_quantize_gemm does,
// writing the 8 E4M3 bytes and, on the first lane of each DPP row, the row's four block scales of
// that K step.
struct XqOps {
  const uint16_t* x;
  int64_t ldx;
  int M, K;
  uint8_t* a8;    // [M, K] E4M3
  uint8_t* as_p;  // [K/128][1][256][4] (tiles_m = 1 for M <= 256)
};

__device__ __forceinline__ void dec_xquant(const XqOps& o, int vb) {
  const int spr = o.K >> 3;
  const int idx = vb * 256 + threadIdx.x;
  const bool ok = idx < o.M * spr;            // M spr is a multiple of 16: whole DPP rows in or out
  const int id = ok ? idx : (idx & 15);
  const int row = id / spr, sc = id - row * spr;
  const uint4 v = *(const uint4*)(o.x + (int64_t)row * o.ldx + (int64_t)sc * 8);
  const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
  int emax;
  uint32_t m, e0, e1;
  mix_quant_lane_bf16_img<1, true>(w4, emax, m, e0, e1);
  const int ev = emax + 126;
  const uint32_t sdw = (uint32_t)ev | ((uint32_t)__builtin_amdgcn_update_dpp(0, ev, 0x12C, 0xF, 0xF, true) << 8) |
                       ((uint32_t)__builtin_amdgcn_update_dpp(0, ev, 0x128, 0xF, 0xF, true) << 16) |
                       ((uint32_t)__builtin_amdgcn_update_dpp(0, ev, 0x124, 0xF, 0xF, true) << 24);
  if (!ok) return;
  *(uint2*)(o.a8 + (int64_t)row * o.K + sc * 8) = make_uint2(e0, e1);
  if ((sc & 15) == 0) *(uint32_t*)(o.as_p + (int64_t)(sc >> 4) * 1024 + row * 4) = sdw;
}

// grid nxq + 8 (nchunk + 1) ceil(B Hkv / 8), block 256: workgroups [0, nxq) code the linear's
// activations (nxq a multiple of 8, 0 for attention alone), the rest run dec_scores.
__global__ void __launch_bounds__(256) MIX_MFMA_VGPR k_decode_scores(DecOps a, XqOps xq, int nxq) {
  const int vb = (int)blockIdx.x;
  if (vb < nxq) {
    dec_xquant(xq, vb);
    return;
  }
  dec_scores(a, vb - nxq);
}

// ------------------------------------------------------------------ decode: p, P^, P^ V^, O (pass 2)

// The chunk's value codes in LDS: 128 channel rows of 128 bytes (the chunk's 8 blocks of 32
// tokens), the 16-byte block j of channel ch at slot j ^ vswz(ch) so that the 8 or 16 lanes an LDS
// read serves at once hit distinct banks.
__device__ __forceinline__ int vswz(int ch) { return (ch ^ (ch >> 3)) & 7; }

// LDS bytes of the pv pass: the value tile, then P^ as E4M3 [G][DCH] and its scales [G][DCH/32],
// then the row maxima
inline size_t decode_pv_lds_bytes(int G) { return 128 * 128 + (size_t)G * DCH + (size_t)G * (DCH / 32) + 4 + 16 * 4; }

// The pv pass for workgroup vb of 8 nchunk ceil(B Hkv / 8) (dec_wg), 256 threads, LDS dsm of
// decode_pv_lds_bytes(G) bytes. Writes the chunk partials lpart [B, Hq, nchunk] and opart [B, Hq,
// nchunk, 128]. P^ codes [B, Hq, Lp/2] and shared fields [B, Hq, Lp/32] are written only when pc /
// ps are given (debug dumps).
__device__ __forceinline__ void dec_pv(const DecOps& a, int vb, uint8_t* dsm) {
  constexpr int d = 128;
  const DecWg wg = dec_wg(vb, a.nchunk, a.Hkv, a.B);
  if (!wg.valid) return;
  const int chunk = wg.chunk, h = wg.h, b = wg.b, Hq = a.Hq, Hkv = a.Hkv;
  const int64_t Lmax = a.Lmax, Lp = a.Lp;
  const int nchunk = a.nchunk;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p = a.pos[b];
  const int64_t bh = (int64_t)b * Hkv + h;
  const int64_t qrow0 = (int64_t)b * Hq + (int64_t)h * G;
  if (p < 0 || p > a.max_pos) {
    // rows outside [0, max_pos]: O is zero (written once, by chunk 0)
    if (chunk == 0)
      for (int t = tid; t < G * d; t += 256) a.o[qrow0 * d + t] = 0;
    return;
  }
  if (chunk * DCH > p) return;
  const int r = lane & 15, g = lane >> 4;
  uint8_t* sV = dsm;                                   // [128][128] value codes
  uint8_t* sP = dsm + 128 * 128;                       // [G][DCH] P^ as E4M3
  uint8_t* sPs = sP + G * DCH;                         // [G][DCH/32] its scales
  float* sm = (float*)(((uintptr_t)(sPs + G * (DCH / 32)) + 3) & ~(uintptr_t)3);   // [16] scaled row maxima

  // loads first. Value codes -> LDS: wave w copies channel rows 32 w .. 32 w + 31, 8 per copy
  // (lane -> row + lane / 8, slot lane % 8); blocks past the newest token are clamped to its block
  // and their products discarded
  const int pb = p >> 5;
#pragma unroll
  for (int it = 0; it < 4; it++) {
    const int row0 = 32 * wave + 8 * it, ch = row0 + (lane >> 3), slot = lane & 7;
    const int kb = min(chunk * (DCH / 32) + (slot ^ vswz(ch)), pb);
    dma16(a.vc + (bh * d + ch) * (Lmax >> 1) + kb * 16, __builtin_amdgcn_readfirstlane(lds_addr(sV + row0 * 128)));
  }
  // value scales of the wave's channel tiles 2w, 2w+1 (16 channels each), K steps k2, blocks g
  int vsc[DCH / 128][2];
#pragma unroll
  for (int k2 = 0; k2 < DCH / 128; k2++) {
    const int kb = min(chunk * DCH + k2 * 128 + 32 * g, p) >> 5;
#pragma unroll
    for (int t = 0; t < 2; t++) vsc[k2][t] = a.vs[(bh * d + (2 * wave + t) * 16 + r) * (Lmax >> 5) + kb];
  }
  // S of the thread's (row, 8 keys): thread -> (row = tid / 32 + 8 pass, sub-block = tid % 32);
  // the first pass's values are loaded here, a second pass (G > 8) loads its own
  const int sbk = tid & 31, jb = chunk * DCH + sbk * 8;
  auto load_s = [&](int row, float (&v)[8]) {
    const float* sp = a.S + (qrow0 + row) * Lp + jb;
    const float4 s0 = *(const float4*)sp;
    const float4 s1 = *(const float4*)(sp + 4);
    v[0] = s0.x; v[1] = s0.y; v[2] = s0.z; v[3] = s0.w;
    v[4] = s1.x; v[5] = s1.y; v[6] = s1.z; v[7] = s1.w;
  };
  float sv[8];
  load_s(min(tid >> 5, G - 1), sv);   // rows past G load row G-1 (not used)
  // chunk maxima: 16 threads per row, the first two loads clamped to the last live chunk (repeats
  // do not change a maximum)
  const int last = p / DCH;
  const int mrow = min(tid >> 4, G - 1), part = tid & 15;
  const float* pm = a.pmax + (qrow0 + mrow) * nchunk;
  float pmv = fmaxf(pm[min(part, last)], pm[min(part + 16, last)]);
  for (int c = part + 32; c <= last; c += 16) pmv = fmaxf(pmv, pm[c]);
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) pmv = fmaxf(pmv, __shfl_xor(pmv, off, 64));
  if ((tid & 15) == 0 && (tid >> 4) < G) sm[tid >> 4] = __fmul_rn(pmv, a.scale);
  __syncthreads();

  // p and P^
#pragma unroll
  for (int pass = 0; pass < 2; pass++) {
    const int row = 8 * pass + (tid >> 5);
    if (row < G) {  // 32 threads per row: whole quads
      if (pass == 1) load_s(row, sv);
      const int64_t qrow = qrow0 + row;
      const float m = sm[row];
      float pv[8];
      float lsum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float v = exp_nonpos(__fsub_rn(__fmul_rn(sv[e], a.scale), m));
        pv[e] = jb + e <= p ? v : 0.f;
        lsum += pv[e];
      }
      uint32_t shf;
      const uint32_t word = p_code8(make_float4(pv[0], pv[1], pv[2], pv[3]), make_float4(pv[4], pv[5], pv[6], pv[7]),
                                    sbk & 3, shf);
      if (a.pc) *(uint32_t*)(a.pc + qrow * (Lp >> 1) + (jb >> 1)) = word;
      if ((sbk & 3) == 0) {
        if (a.ps) a.ps[qrow * (Lp >> 5) + (jb >> 5)] = (uint16_t)shf;
        sPs[row * (DCH / 32) + (sbk >> 2)] = (uint8_t)((shf & 15u) + 119u);
      }
      uint32_t e0, e1;
      mix8_to_e4m3(word, (shf >> (4 + 3 * (sbk & 3))) & 7u, e0, e1);
      *(uint2*)(sP + row * DCH + sbk * 8) = make_uint2(e0, e1);
      if (a.dbg_p) {
        float* dp = a.dbg_p + qrow * Lp + jb;
        *(float4*)dp = make_float4(pv[0], pv[1], pv[2], pv[3]);
        *(float4*)(dp + 4) = make_float4(pv[4], pv[5], pv[6], pv[7]);
      }
      // l partial: sum over the 32 threads of this row (half a wave)
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off, 32);
      if (sbk == 0) a.lpart[qrow * nchunk + chunk] = lsum;
    }
  }
  wait_vmcnt<0>();   // this wave's value copies have landed
  __syncthreads();

  // O partial = P^ V^ over this chunk (A operand: P^ row r; rows past G repeat row G-1, their
  // results are discarded)
  v4f acc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int k2 = 0; k2 < DCH / 128; k2++) {
    const int kbase = chunk * DCH + k2 * 128;  // first key of this K step
    if (kbase > p) break;
    const int pr = min(r, G - 1);
    const uint4 lo = *(const uint4*)(sP + pr * DCH + k2 * 128 + 16 * g);
    const uint4 hi = *(const uint4*)(sP + pr * DCH + k2 * 128 + 64 + 16 * g);
    const v8i af = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    const int sa = sPs[pr * (DCH / 32) + k2 * 4 + g];
    const bool blk_live = kbase + 32 * g <= p;
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const int ch = (2 * wave + t) * 16 + r, j = k2 * 4 + g;
      const uint4 vf = *(const uint4*)(sV + ch * 128 + 16 * (j ^ vswz(ch)));
      const int vscale = vsc[k2][t];
      const v8i bf = blk_live ? v8i{(int)vf.x, (int)vf.y, (int)vf.z, (int)vf.w, 0, 0, 0, 0}
                              : v8i{0, 0, 0, 0, 0, 0, 0, 0};
      const int sb = blk_live ? vscale : 127;
      acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf, acc[t], 0, 4, 0, sa, 0, sb);
    }
  }
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const int ch = (2 * wave + t) * 16 + r;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int row = 4 * g + i;
      if (row < G) a.opart[((qrow0 + row) * nchunk + chunk) * d + ch] = acc[t][i];
    }
  }

}

// The combine pass, workgroup vb of ceil(B Hq / 2), 256 threads: thread t owns channel t % 128 of
// query row 2 vb + t / 128 and adds the chunk partials in chunk order (eight loads in flight):
// O = sum_chunks O_part / sum_chunks l_part, rounded to bf16 (rows whose pos is outside
// [0, max_pos]: zeros, written by the pv pass).
__device__ __forceinline__ void dec_combine(const DecOps& a, int vb) {
  constexpr int d = 128;
  const int64_t qrow = (int64_t)vb * 2 + (threadIdx.x >> 7);
  if (qrow >= (int64_t)a.B * a.Hq) return;
  const int b = (int)(qrow / a.Hq), c = threadIdx.x & (d - 1);
  const int p = a.pos[b];
  if (p < 0 || p > a.max_pos) return;
  const int n = p / DCH + 1;
  const float* lp = a.lpart + qrow * a.nchunk;
  const float* op = a.opart + qrow * a.nchunk * d + c;
  float l = 0.f, acc = 0.f;
  int k = 0;
  // all loads of a group in flight together (a full 8192-token history is one group of 32 chunks:
  // one memory round trip), then the sums in chunk order
  auto group = [&](auto width) {
    constexpr int W = decltype(width)::value;
    float lv[W], ov[W];
#pragma unroll
    for (int u = 0; u < W; u++) {
      lv[u] = lp[k + u];
      ov[u] = op[(int64_t)(k + u) * d];
    }
#pragma unroll
    for (int u = 0; u < W; u++) {
      l += lv[u];
      acc += ov[u];
    }
  };
  for (; k + 32 <= n; k += 32) group(std::integral_constant<int, 32>{});
  for (; k + 8 <= n; k += 8) group(std::integral_constant<int, 8>{});
  for (; k < n; k++) {
    l += lp[k];
    acc += op[(int64_t)k * d];
  }
  a.o[qrow * d + c] = f32_to_bf16_rne(__fdiv_rn(acc, l));
  if (a.dbg_l && c == 0) a.dbg_l[qrow] = l;
}

// Weight-stream workgroups inside a decode launch: 16 DEC_GV_RG output columns each, DEC_GV_D K steps
// of operands in flight per wave (registers are shared with the pass they run beside).
constexpr int DEC_GV_RG = 2, DEC_GV_D = 2;

// grid 8 nchunk ceil(B Hkv / 8) + ngv, block 256, dynamic LDS max(decode_pv_lds_bytes(G),
// gv_lds_bytes): workgroups [0, npv) run the pv pass, the rest (ngv of them; GV = 0: none) stream the
// linear's weights (GV = 1: MXFP4 image, 2: E4M3 image) into bf16 C.
template <int GV>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) k_decode_pv(DecOps a, int npv, GvOps gv) {
  extern __shared__ __align__(16) uint8_t dsm[];
  const int vb = (int)blockIdx.x;
  if (GV && vb >= npv) {
    gemv_block<GV == 1, 1, DEC_GV_RG, DEC_GV_D>(gv, vb - npv, (float*)dsm);
    return;
  }
  dec_pv(a, vb, dsm);
}

// grid ncb + ngv, block 256, dynamic LDS gv_lds_bytes when GV: workgroups [0, ncb) add the chunk
// partials into O (ncb = ceil(B Hq / 2)), the rest stream the linear's weights as in k_decode_pv.
template <int GV>
__global__ void __launch_bounds__(256) k_decode_combine(DecOps a, int ncb, GvOps gv) {
  extern __shared__ __align__(16) uint8_t dsm[];
  const int vb = (int)blockIdx.x;
  if (GV && vb >= ncb) {
    gemv_block<GV == 1, 1, DEC_GV_RG, DEC_GV_D>(gv, vb - ncb, (float*)dsm);
    return;
  }
  dec_combine(a, vb);
}

// The whole decode step in one cooperative launch: the same roles as the three launches above, taken
// in turn by the grid's workgroups (role-local indices keep their residue modulo 8, so every role keeps
// its XCD placement), with a grid-wide barrier where a launch boundary stood: the scores need the exact
// maximum over every chunk before any P^ is coded, and the combine needs every chunk's partials. The
// cooperative launch admits the grid only if every workgroup is resident, so each barrier is reached
// by all of them. grid: a multiple of 8 workgroups of 256 threads, dynamic LDS as for k_decode_pv.
template <int GV>
__global__ void __launch_bounds__(256) MIX_MFMA_VGPR k_decode_single(DecOps a, XqOps xq, GvOps gv, int nxq, int nsc,
                                                                     int npv, int ngv, int ncb) {
  extern __shared__ __align__(16) uint8_t dsm[];
  const int nwg = (int)gridDim.x;
  for (int v = (int)blockIdx.x; v < nxq + nsc; v += nwg) {
    if (v < nxq) dec_xquant(xq, v);
    else dec_scores(a, v - nxq);
    __syncthreads();   // the next role's LDS writes wait for this one's reads
  }
  cooperative_groups::this_grid().sync();
  for (int v = (int)blockIdx.x; v < npv + ngv; v += nwg) {
    if (v < npv) dec_pv(a, v, dsm);
    else if (GV) gemv_block<GV == 1, 1, DEC_GV_RG, DEC_GV_D>(gv, v - npv, (float*)dsm);
    __syncthreads();
  }
  cooperative_groups::this_grid().sync();
  for (int v = (int)blockIdx.x; v < ncb; v += nwg) dec_combine(a, v);
}

// ------------------------------------------------------------------ host orchestration

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// V^ scale rows are padded to a multiple of 4 blocks (the fused pass copies them as dwords)
static inline int64_t prefill_vsp(int64_t Tp) { return (Tp / 32 + 3) / 4 * 4; }

struct PrefillWs {
  size_t qc, qs, kc, ks, vc, vs, s, pc, ps, l, km, total;
};

static PrefillWs prefill_layout(int64_t T, int64_t Hq, int64_t Hkv, int64_t d) {
  const int64_t Tp = (T + 31) / 32 * 32;
  PrefillWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  w.qc = take((size_t)T * Hq * d / 2);
  w.qs = take((size_t)T * Hq * (d / 32) * 2);
  w.kc = take((size_t)T * Hkv * d / 2);
  w.ks = take((size_t)T * Hkv * (d / 32));
  w.vc = take((size_t)Hkv * d * Tp / 2);
  w.vs = take((size_t)Hkv * d * prefill_vsp(Tp));
  // d = 128 takes the fused S passes (row maxima only); other head sizes store S
  w.s = take(d == 128 ? (size_t)Hq * T * 4 : (size_t)Hq * T * Tp * 4);
  w.pc = take((size_t)Hq * T * Tp / 2);
  w.ps = take((size_t)Hq * T * (Tp / 32) * 2);
  w.l = take((size_t)Hq * T * 4);
  w.km = take(kmean_ws_bytes(T, Hkv * d));
  w.total = off;
  return w;
}

size_t attn_prefill_ws_bytes(int64_t T, int64_t Hq, int64_t Hkv, int64_t d) {
  return prefill_layout(T, Hq, Hkv, d).total;
}

#define HIPCHK(x)                      \
  do {                                 \
    hipError_t e_ = (x);               \
    if (e_ != hipSuccess) return e_;   \
  } while (0)

hipError_t attn_prefill_run(const void* q, const void* k, const void* v, int64_t T, int64_t Hq, int64_t Hkv,
                            int64_t d, int causal, float* mu, void* o, void* ws, const mix_attn_debug_t* dbg,
                            hipStream_t s) {
  const int64_t Tp = (T + 31) / 32 * 32;
  const int64_t G = Hq / Hkv;
  PrefillWs w = prefill_layout(T, Hq, Hkv, d);
  uint8_t* base = (uint8_t*)ws;
  uint8_t* qc = base + w.qc;
  uint16_t* qs = (uint16_t*)(base + w.qs);
  uint8_t* kc = base + w.kc;
  uint8_t* ks = base + w.ks;
  uint8_t* vc = base + w.vc;
  uint8_t* vs = base + w.vs;
  float* S = (float*)(base + w.s);
  uint8_t* pc = base + w.pc;
  uint16_t* ps = (uint16_t*)(base + w.ps);
  float* l = (float*)(base + w.l);

  // 1. Q^, V^ and the K-mean's row-slice pairs in one launch; the K-mean; K^ (smoothed by it)
  const int64_t vsp = prefill_vsp(Tp);
  PrefillOperandArgs oa{};
  oa.q = (const uint16_t*)q; oa.cq = Hq * d; oa.ldq = Hq * d; oa.qc = qc; oa.qs = qs;
  oa.v = (const uint16_t*)v; oa.cv = Hkv * d; oa.ldv = Hkv * d; oa.vc = vc; oa.vs = vs; oa.cpitch = Tp / 2;
  oa.spitch = vsp;
  oa.k = (const uint16_t*)k; oa.ck = Hkv * d; oa.ldk = Hkv * d; oa.part = (double2*)(base + w.km);
  oa.T = T; oa.Tp = Tp;
  HIPCHK(launch_prefill_operands(oa, s));
  HIPCHK(launch_kmean_fin(base + w.km, T, Hkv * d, mu, s));
  HIPCHK(launch_mx_quantize(1, k, 1, T, Hkv * d, Hkv * d, mu, kc, ks, s));

  const float scale = (float)(1.0 / sqrt((double)d));
  if (d == 128) {
    // 3-5. fused: row maxima of S, then S again -> p, l, P^ and O += P^ V^ (S and P^ stay on chip;
    // P^ codes are written only for the debug dump)
    PrefillOps P{qc, qs, kc, ks, vc, vs, (int)T, (int)Tp, (int)Hq, (int)Hkv, causal ? 1 : 0, (int)vsp};
    dim3 grid((unsigned)Hq, (unsigned)((T + PQ - 1) / PQ));
    hipLaunchKernelGGL(k_attn_rowmax, grid, dim3(256), 0, s, P, S);
    HIPCHK(hipGetLastError());
    const bool want_codes = dbg && (dbg->p_codes || dbg->p_shared);
    if (dbg)
      hipLaunchKernelGGL(k_attn_pcode<true>, grid, dim3(256), 0, s, P, (const float*)S, scale, (uint16_t*)o,
                         want_codes ? pc : nullptr, want_codes ? ps : nullptr, l, dbg->s, dbg->p);
    else
      hipLaunchKernelGGL(k_attn_pcode<false>, grid, dim3(256), 0, s, P, (const float*)S, scale, (uint16_t*)o,
                         nullptr, nullptr, l, nullptr, nullptr);
    HIPCHK(hipGetLastError());
  } else {
    // 3. S = Q^ K^T per query head
    GemmArgs g1{};
    g1.a_codes = qc; g1.a_shared = qs; g1.a_pitch = Hq * d / 2; g1.a_sh_pitch = Hq * d / 32;
    g1.a_bstride = d / 2; g1.a_sh_bstride = d / 32;
    g1.b_codes = kc; g1.b_scales = ks; g1.b_pitch = Hkv * d / 2; g1.b_sc_pitch = Hkv * d / 32;
    g1.b_bstride = d / 2; g1.b_sc_bstride = d / 32; g1.b_group = (int)G;
    g1.c = S; g1.ldc = Tp; g1.c_bstride = T * Tp; g1.row_div = nullptr;
    g1.M = (int)T; g1.N = (int)T; g1.K = (int)d; g1.batch = (int)Hq; g1.causal = causal ? 1 : 0;
    HIPCHK(launch_gemm_mfma(1, 1, 0, g1, s));

    // 4. softmax and P^
    const int64_t nrows = Hq * T;
    hipLaunchKernelGGL(k_softmax_pquant, dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, s, S, (int)T, (int)Tp,
                       nrows, causal, scale, pc, ps, l, dbg ? dbg->p : nullptr);
    HIPCHK(hipGetLastError());
    if (dbg && dbg->s) HIPCHK(hipMemcpyAsync(dbg->s, S, (size_t)Hq * T * Tp * 4, hipMemcpyDeviceToDevice, s));

    // 5. O = (P^ V^) / l
    GemmArgs g2{};
    g2.a_codes = pc; g2.a_shared = ps; g2.a_pitch = Tp / 2; g2.a_sh_pitch = Tp / 32;
    g2.a_bstride = T * Tp / 2; g2.a_sh_bstride = T * (Tp / 32);
    g2.b_codes = vc; g2.b_scales = vs; g2.b_pitch = Tp / 2; g2.b_sc_pitch = vsp;
    g2.b_bstride = d * Tp / 2; g2.b_sc_bstride = d * vsp; g2.b_group = (int)G;
    g2.c = o; g2.ldc = Hq * d; g2.c_bstride = d; g2.row_div = l; g2.row_div_bstride = T;
    g2.M = (int)T; g2.N = (int)d; g2.K = (int)Tp; g2.batch = (int)Hq; g2.causal = causal ? 2 : 0;
    HIPCHK(launch_gemm_mfma(1, 1, 1, g2, s));
  }

  if (dbg) {
    if (dbg->p_codes) HIPCHK(hipMemcpyAsync(dbg->p_codes, pc, (size_t)Hq * T * Tp / 2, hipMemcpyDeviceToDevice, s));
    if (dbg->p_shared)
      HIPCHK(hipMemcpyAsync(dbg->p_shared, ps, (size_t)Hq * T * (Tp / 32) * 2, hipMemcpyDeviceToDevice, s));
    if (dbg->l) HIPCHK(hipMemcpyAsync(dbg->l, l, (size_t)Hq * T * 4, hipMemcpyDeviceToDevice, s));
  }
  return hipSuccess;
}

hipError_t kv_cache_prefill_run(const mix_kv_cache_t* c, int64_t b, const void* k, const void* v, int64_t T,
                                const float* mu, hipStream_t s) {
  const int64_t Hkv = c->Hkv, d = c->d, Lmax = c->Lmax;
  const int64_t Tp = (T + 31) / 32 * 32;
  for (int64_t h = 0; h < Hkv; h++) {
    const int64_t bh = b * Hkv + h;
    HIPCHK(launch_mx_quantize(1, (const uint16_t*)k + h * d, 1, T, d, Hkv * d, mu + h * d,
                              c->k_codes + bh * Lmax * (d / 2), c->k_scales + bh * Lmax * (d / 32), s));
    HIPCHK(launch_mx_quantize_cols((const uint16_t*)v + h * d, 1, T, Tp, d, Hkv * d, c->v_codes + bh * d * (Lmax / 2),
                                   c->v_scales + bh * d * (Lmax / 32), Lmax / 2, Lmax / 32, s));
  }
  const int64_t rem = T % 32;
  if (rem) {
    HIPCHK(hipMemcpyAsync((uint16_t*)c->v_stage + b * 32 * Hkv * d, (const uint16_t*)v + (T - rem) * Hkv * d,
                          (size_t)rem * Hkv * d * 2, hipMemcpyDeviceToDevice, s));
  }
  return hipSuccess;
}

struct DecodeWs {
  size_t s, pmax, pc, ps, lpart, opart, a_img, total;
};

// Workspace of a decode step: S, chunk maxima, debug copies of P^, the chunk partials and, for the
// full step (K > 0), the A image of the linear's B x K activations.
static DecodeWs decode_layout(int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t max_pos, int64_t K,
                              int64_t* Lp_out, int* nchunk_out) {
  const int nchunk = (int)((max_pos + 1 + DCH - 1) / DCH);
  const int64_t Lp = (int64_t)nchunk * DCH;
  DecodeWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  w.s = take((size_t)B * Hq * Lp * 4);
  w.pmax = take((size_t)B * Hq * nchunk * 4);
  w.pc = take((size_t)B * Hq * Lp / 2);
  w.ps = take((size_t)B * Hq * (Lp / 32) * 2);
  w.lpart = take((size_t)B * Hq * nchunk * 4);
  w.opart = take((size_t)B * Hq * nchunk * d * 4);
  w.a_img = take(K > 0 ? f8_a_image_layout(B, K).total : 0);
  w.total = off;
  if (Lp_out) *Lp_out = Lp;
  if (nchunk_out) *nchunk_out = nchunk;
  return w;
}

size_t attn_decode_ws_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t max_pos) {
  return decode_layout(B, Hq, Hkv, d, max_pos, 0, nullptr, nullptr).total;
}

size_t decode_step_ws_bytes(int64_t B, int64_t K, int64_t Hq, int64_t Hkv, int64_t d, int64_t max_pos) {
  return decode_layout(B, Hq, Hkv, d, max_pos, K, nullptr, nullptr).total;
}

// The two decode launches. lin == NULL: attention alone. Otherwise the full step: the scores launch
// also codes x [B, K] (bf16, row pitch K) into the A image in the workspace, and the pv launch also
// streams the weights' B image into y [B, N] (bf16, row pitch N).
struct DecodeLinear {
  const void* x;
  int64_t K, N;
  int b_fp4;
  const void* b_img;
  void* y;
};

// The resident grid of k_decode_single<GV> with `lds` bytes of dynamic LDS (a multiple of 8 workgroups),
// or 0 when the device cannot launch cooperatively.
template <int GV>
static hipError_t decode_single_grid(size_t lds, int* out) {
  int dev = 0, coop = 0, ncu = 0, per = 0;
  HIPCHK(hipGetDevice(&dev));
  HIPCHK(hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev));
  HIPCHK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
  HIPCHK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, (const void*)k_decode_single<GV>, 256, lds));
  *out = coop ? per * ncu / 8 * 8 : 0;
  return hipSuccess;
}

static hipError_t decode_run(const void* q, const void* k_new, const void* v_new, const mix_kv_cache_t* c,
                             const int32_t* pos, int64_t max_pos, int64_t Hq, const float* mu, void* o, void* ws,
                             const mix_attn_debug_t* dbg, const DecodeLinear* lin, hipStream_t s,
                             bool single = false) {
  const int64_t B = c->B, Hkv = c->Hkv, d = c->d, Lmax = c->Lmax;
  int64_t Lp;
  int nchunk;
  const DecodeWs w = decode_layout(B, Hq, Hkv, d, max_pos, lin ? lin->K : 0, &Lp, &nchunk);
  uint8_t* base = (uint8_t*)ws;
  DecOps a{};
  a.q = (const uint16_t*)q; a.k_new = (const uint16_t*)k_new; a.v_new = (const uint16_t*)v_new; a.mu = mu;
  a.pos = pos; a.max_pos = max_pos; a.Lmax = Lmax; a.Lp = Lp;
  a.Hq = (int)Hq; a.Hkv = (int)Hkv; a.B = (int)B; a.nchunk = nchunk;
  a.kc = c->k_codes; a.ks = c->k_scales; a.vc = c->v_codes; a.vs = c->v_scales; a.stage = (uint16_t*)c->v_stage;
  a.S = (float*)(base + w.s);
  a.pmax = (float*)(base + w.pmax);
  a.lpart = (float*)(base + w.lpart);
  a.opart = (float*)(base + w.opart);
  a.scale = (float)(1.0 / sqrt((double)d));
  a.o = (uint16_t*)o;
  a.pc = dbg && dbg->p_codes ? base + w.pc : nullptr;
  a.ps = dbg && dbg->p_shared ? (uint16_t*)(base + w.ps) : nullptr;
  a.dbg_p = dbg ? dbg->p : nullptr;
  a.dbg_l = dbg ? dbg->l : nullptr;

  XqOps xq{};
  GvOps gv{};
  int nxq = 0, ngv = 0;
  if (lin) {
    const F8AImage LA = f8_a_image_layout(B, lin->K);
    const F8BImage LB = f8_b_image_layout(lin->b_fp4, lin->N, lin->K);
    uint8_t* aimg = base + w.a_img;
    xq.x = (const uint16_t*)lin->x; xq.ldx = lin->K; xq.M = (int)B; xq.K = (int)lin->K;
    xq.a8 = aimg + LA.a8; xq.as_p = aimg + LA.as_p;
    nxq = (int)((B * (lin->K / 8) + 255) / 256 + 7) / 8 * 8;
    gv.a8 = aimg + LA.a8; gv.as_p = aimg + LA.as_p;
    gv.b8 = (const uint8_t*)lin->b_img + LB.b8; gv.bs_v = (const uint8_t*)lin->b_img + LB.bs_v;
    gv.c = lin->y; gv.ldc = lin->N; gv.M = (int)B; gv.N = (int)lin->N; gv.K = (int)lin->K; gv.tiles_m = 1;
    ngv = (int)(((lin->N + 15) / 16 + DEC_GV_RG - 1) / DEC_GV_RG);
  }

  const int bh8 = (int)((B * Hkv + 7) / 8);
  const int nsc = 8 * (nchunk + 1) * bh8, npv = 8 * nchunk * bh8, ncb = (int)((B * Hq + 1) / 2);
  const size_t lds_pv = decode_pv_lds_bytes((int)(Hq / Hkv));
  const size_t lds_gv = gv_lds_bytes<DEC_GV_RG>();
  if (single) {
    const int gvk = !lin ? 0 : (lin->b_fp4 ? 1 : 2);
    const size_t lds = gvk && lds_gv > lds_pv ? lds_gv : lds_pv;
    int grid = 0;
    if (gvk == 1) HIPCHK(decode_single_grid<1>(lds, &grid));
    else if (gvk == 2) HIPCHK(decode_single_grid<2>(lds, &grid));
    else HIPCHK(decode_single_grid<0>(lds, &grid));
    if (grid < 8) return hipErrorNotSupported;
    const int most = std::max(nxq + nsc, std::max(npv + (gvk ? ngv : 0), ncb));
    grid = std::min(grid, (most + 7) / 8 * 8);
    int n_xq = nxq, n_sc = nsc, n_pv = npv, n_gv = gvk ? ngv : 0, n_cb = ncb;
    void* args[] = {&a, &xq, &gv, &n_xq, &n_sc, &n_pv, &n_gv, &n_cb};
    const void* fn = gvk == 1 ? (const void*)k_decode_single<1>
                              : gvk == 2 ? (const void*)k_decode_single<2> : (const void*)k_decode_single<0>;
    HIPCHK(hipLaunchCooperativeKernel(fn, dim3((unsigned)grid), dim3(256), args, (unsigned)lds, s));
    return hipSuccess;
  }
  hipLaunchKernelGGL(k_decode_scores, dim3((unsigned)(nxq + nsc)), dim3(256), 0, s, a, xq, nxq);
  HIPCHK(hipGetLastError());
  // the weight stream runs beside the pv pass (measured: 50 us per workload-5 step, against 55 us
  // beside the combine, which it then no longer overlaps with the value stream)
  const int gvk = !lin ? 0 : (lin->b_fp4 ? 1 : 2);
  const int g2 = gvk, g3 = 0;
  const size_t l2 = g2 && lds_gv > lds_pv ? lds_gv : lds_pv;
  const unsigned n2 = (unsigned)(npv + (g2 ? ngv : 0)), n3 = (unsigned)(ncb + (g3 ? ngv : 0));
  if (g2 == 1) hipLaunchKernelGGL(k_decode_pv<1>, dim3(n2), dim3(256), l2, s, a, npv, gv);
  else if (g2 == 2) hipLaunchKernelGGL(k_decode_pv<2>, dim3(n2), dim3(256), l2, s, a, npv, gv);
  else hipLaunchKernelGGL(k_decode_pv<0>, dim3(n2), dim3(256), l2, s, a, npv, gv);
  HIPCHK(hipGetLastError());
  if (g3 == 1) hipLaunchKernelGGL(k_decode_combine<1>, dim3(n3), dim3(256), lds_gv, s, a, ncb, gv);
  else if (g3 == 2) hipLaunchKernelGGL(k_decode_combine<2>, dim3(n3), dim3(256), lds_gv, s, a, ncb, gv);
  else hipLaunchKernelGGL(k_decode_combine<0>, dim3(n3), dim3(256), 0, s, a, ncb, gv);
  HIPCHK(hipGetLastError());
  if (dbg) {
    if (dbg->s) HIPCHK(hipMemcpyAsync(dbg->s, a.S, (size_t)B * Hq * Lp * 4, hipMemcpyDeviceToDevice, s));
    if (dbg->p_codes)
      HIPCHK(hipMemcpyAsync(dbg->p_codes, a.pc, (size_t)B * Hq * Lp / 2, hipMemcpyDeviceToDevice, s));
    if (dbg->p_shared)
      HIPCHK(hipMemcpyAsync(dbg->p_shared, a.ps, (size_t)B * Hq * (Lp / 32) * 2, hipMemcpyDeviceToDevice, s));
  }
  return hipSuccess;
}

hipError_t attn_decode_run(const void* q, const void* k_new, const void* v_new, const mix_kv_cache_t* c,
                           const int32_t* pos, int64_t max_pos, int64_t Hq, const float* mu, void* o, void* ws,
                           const mix_attn_debug_t* dbg, hipStream_t s) {
  return decode_run(q, k_new, v_new, c, pos, max_pos, Hq, mu, o, ws, dbg, nullptr, s);
}

hipError_t decode_step_run(const void* x, int64_t K, int64_t N, int b_fp4, const void* b_img, void* y, const void* q,
                           const void* k_new, const void* v_new, const mix_kv_cache_t* c, const int32_t* pos,
                           int64_t max_pos, int64_t Hq, const float* mu, void* o, void* ws, hipStream_t s) {
  const DecodeLinear lin{x, K, N, b_fp4, b_img, y};
  return decode_run(q, k_new, v_new, c, pos, max_pos, Hq, mu, o, ws, nullptr, &lin, s);
}

hipError_t decode_step_single_run(const void* x, int64_t K, int64_t N, int b_fp4, const void* b_img, void* y,
                                  const void* q, const void* k_new, const void* v_new, const mix_kv_cache_t* c,
                                  const int32_t* pos, int64_t max_pos, int64_t Hq, const float* mu, void* o, void* ws,
                                  hipStream_t s) {
  const DecodeLinear lin{x, K, N, b_fp4, b_img, y};
  return decode_run(q, k_new, v_new, c, pos, max_pos, Hq, mu, o, ws, nullptr, &lin, s, true);
}

// ------------------------------------------------------------------ decode step without allocation

// The decode step's workspace as a file-scope device array, for callers that cannot allocate (code
// under graph capture, serving loops that forbid allocation). Each device that runs the library
// holds its own copy until the process ends; calls on one device share it and race if they overlap.
// Nothing in it needs to start at zero: every byte a launch reads was written earlier in the step.
static __device__ __align__(256) uint8_t scratch[DECODE_SCRATCH_BYTES];

// The device address of `scratch` on the current device, looked up once per device (the host-side
// name is only a stand-in, never a device address).
static hipError_t decode_scratch_ptr(void** out) {
  static std::mutex mu;
  static void* ptrs[64] = {nullptr};
  int dev = 0;
  HIPCHK(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    HIPCHK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

hipError_t decode_step_static_run(const void* x, int64_t K, int64_t N, int b_fp4, const void* b_img, void* y,
                                  const void* q, const void* k_new, const void* v_new, const mix_kv_cache_t* c,
                                  const int32_t* pos, int64_t max_pos, int64_t Hq, const float* mu, void* o,
                                  hipStream_t s) {
  void* ws = nullptr;
  HIPCHK(decode_scratch_ptr(&ws));
  return decode_step_run(x, K, N, b_fp4, b_img, y, q, k_new, v_new, c, pos, max_pos, Hq, mu, o, ws, s);
}

}  // namespace mix
