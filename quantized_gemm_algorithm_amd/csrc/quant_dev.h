// Device-side element coders shared by the quantizer kernels and the attention kernels.
//
// MiX element decision. With M = 1 + m/8 the nonzero magnitudes of a block are c_d = M 2^(Emax-d).
// The nearest one (ties to the smaller magnitude) is c_d* with d* = #{d : a <= mid_d}, mid_d the
// midpoint of c_d and c_(d+1). For d <= 5 the midpoints are 1.5 M 2^(Emax-1-d), a geometric
// sequence, so the count is an exponent difference plus one mantissa comparison (the naive dE
// with its +-1 refinement). Only the last step depends on the sign: positives have c_7 (the
// reclaimed pattern) and then zero; negatives go from c_6 to zero. All thresholds are exact fp32
// values and all comparisons are unsigned comparisons of fp32 bit patterns.
#pragma once
#include "common.h"

namespace mix {

// 8 consecutive elements of row `row` starting at column `col` as fp32 bit patterns (DT 1: bf16
// input, widened exactly; DT 0: fp32). The address must be 16-byte aligned.
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t row, int64_t ld, int64_t col, uint32_t (&x)[8]) {
  if (DT == 1) {  // bf16
    const uint16_t* p = (const uint16_t*)base + row * ld + col;
    uint4 v = *(const uint4*)p;
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      x[2 * i] = (w[i] & 0xFFFFu) << 16;
      x[2 * i + 1] = w[i] & 0xFFFF0000u;
    }
  } else {  // fp32
    const float* p = (const float*)base + row * ld + col;
    uint4 v0 = *(const uint4*)p;
    uint4 v1 = *(const uint4*)(p + 4);
    x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
    x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
  }
}

// Returns the 4-bit code of one element given the block's thresholds.
struct MixThresholds {
  uint32_t e_mu0;   // biased exponent of mid_0 = 1.5 M 2^(Emax-1)
  uint32_t m_mu0;   // its mantissa bits
  uint32_t pos_bottom;  // midpoint of c_7 and 0 for positives: M 2^(Emax-8)
  uint32_t neg_bottom;  // midpoint of c_6 and 0 for negatives: M 2^(Emax-7)
};

__device__ __forceinline__ MixThresholds mix_thresholds(int emax, uint32_t m) {
  MixThresholds t;
  uint32_t t3 = 3u * (8u + m);  // 1.5 M = t3 / 16
  uint32_t mu0 = exact_f32_bits(t3, emax - 5);
  t.e_mu0 = mu0 >> 23;
  t.m_mu0 = mu0 & 0x7FFFFFu;
  t.pos_bottom = exact_f32_bits(8u + m, emax - 11);
  t.neg_bottom = exact_f32_bits(8u + m, emax - 10);
  return t;
}

__device__ __forceinline__ uint32_t mix_code(uint32_t xbits, const MixThresholds& t) {
  uint32_t a = xbits & 0x7FFFFFFFu;
  int ea = (int)(a >> 23);
  uint32_t ma = a & 0x7FFFFFu;
  int cnt = (int)t.e_mu0 - ea - (t.m_mu0 < ma ? 1 : 0) + 1;  // #{d in 0..6 : mid_d >= a}
  cnt = cnt < 0 ? 0 : (cnt > 7 ? 7 : cnt);
  bool neg = (xbits >> 31) && a != 0;
  uint32_t code;
  if (!neg) {
    code = (cnt < 7) ? (uint32_t)cnt : (a <= t.pos_bottom ? 0x7u : 0xFu);
  } else {
    code = (cnt < 6) ? (0x8u | (uint32_t)cnt) : (a <= t.neg_bottom ? 0x7u : 0xEu);
  }
  return code;
}

// The same decision for bf16 inputs, two elements per 32-bit operation. Every threshold has at
// most 6 significant bits and stays in the normal range, so it is exact in bf16 (its fp32 pattern
// has 16 low zero bits) and the comparisons run on 16-bit patterns a (sign cleared) of the two
// halves. With mid_0 the pattern of 1.5 M 2^(Emax-1), cnt = #{d : mid_d >= a} =
// clamp(((mid_0 + 128 - a) >> 7), 0, 7) as a signed 16-bit shift (7 mantissa bits). A negative
// element has no value below c_6, so its index is v = min(cnt, 7 - s) for the sign s; it is zero
// (code 0x7) when a <= the midpoint of its last value and 0, M 2^(Emax-8) + s 2^(Emax-8) (one
// exponent step higher for negatives); otherwise its code is (s << 3) | v, the positive v = 7
// (the reclaimed step) giving 0xF. The E4M3 byte of a nonzero element is
// (s << 7) | ((8 - v) << 3) | m = 64 + m + 128 s - 8 v, and 0 for zero.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

// per-block constants of the pair coder, both halves equal
struct MixPk {
  uint32_t mu1;   // mid_0 pattern + 128
  uint32_t pb;    // pattern of M 2^(Emax-8)
  uint32_t m64;   // 64 + m (E4M3 byte of a positive element with v = 0)
};
__device__ __forceinline__ MixPk mix_pk(int emax, uint32_t m) {
  const uint32_t t3 = 24u + 3u * m;   // mid_0 = 1.5 M 2^(Emax-1) = t3 2^(Emax-5)
  const uint32_t mu = t3 < 32u ? (((uint32_t)(emax + 126) << 7) | ((t3 << 3) & 0x7Fu))
                               : (((uint32_t)(emax + 127) << 7) | ((t3 << 2) & 0x7Fu));
  MixPk k;
  k.mu1 = (mu + 128u) * 0x00010001u;
  k.pb = (((uint32_t)(emax + 119) << 7) | (m << 4)) * 0x00010001u;
  k.m64 = (64u + m) * 0x00010001u;
  return k;
}

// Two elements (bf16 patterns, element 2i in the low half of x) -> their codes in bits 0..3 and
// 16..19; with IMG also their E4M3 bytes in bits 0..7 and 16..23 of img. nzm is all ones in a half
// whose element lies above its zero threshold; a zero element takes w = 7, and bit 3 is added where
// w + 1 reaches 8 (the positive reclaimed step; negatives have it already).
template <bool IMG>
__device__ __forceinline__ uint32_t mix_pair(uint32_t x, const MixPk& k, uint32_t& img) {
  const u16x2 a = __builtin_bit_cast(u16x2, x & 0x7FFF7FFFu);
  const u16x2 s = __builtin_bit_cast(u16x2, x) >> (u16x2)15;
  // max((mu1 - a) >> 7, 0) as an unsigned saturating subtract and a logical shift (mu1 - a never
  // leaves the signed 16-bit range: mu1 < 2^15 and a < 2^15)
  const u16x2 c = __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2, k.mu1), a) >> (u16x2)7;
  const u16x2 v = __builtin_elementwise_min(c, s ^ (u16x2)7);   // 7 - s
  // shifts and adds that cannot carry between the halves as 32-bit operations (s is 0 or 1 a half,
  // v at most 7, pb and 64 + m below 2^15 - 128), so that they fuse into shift-and-add instructions
  const uint32_t s32 = __builtin_bit_cast(uint32_t, s), v32 = __builtin_bit_cast(uint32_t, v);
  const uint32_t s7pb = (s32 << 7) + k.pb;
  const uint32_t nzm = __builtin_bit_cast(
      uint32_t, (__builtin_bit_cast(i16x2, s7pb) - __builtin_bit_cast(i16x2, a)) >> (i16x2)15);
  const uint32_t w = (s32 << 3) | v32;
  const uint32_t wz = (w & nzm) | (0x00070007u & ~nzm);
  if (IMG) img = (((s32 << 7) + k.m64) - (v32 << 3)) & nzm;   // at least 64 + m - 56 > 0 a half: no borrow
  return wz | (__builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, wz) - __builtin_bit_cast(u16x2, nzm)) &
               0x00080008u);
}

// The 8 nibbles of a sub-block from its 16-bit patterns (two per word, element 2i in the low half
// of w[i]) and the block's constants; with IMG also the 8 E4M3 bytes in element order.
template <bool IMG>
__device__ __forceinline__ uint32_t mix_code8_pk(const uint32_t (&w)[4], const MixPk& k, uint32_t& out0,
                                                 uint32_t& out1) {
  uint32_t c2[4], im[4];
#pragma unroll
  for (int i = 0; i < 4; i++) c2[i] = mix_pair<IMG>(w[i], k, im[i]);   // nibbles at bits 0 and 16
  if (IMG) {
    out0 = __builtin_amdgcn_perm(im[1], im[0], 0x06040200u);
    out1 = __builtin_amdgcn_perm(im[3], im[2], 0x06040200u);
  }
  // two pairs in one word (elements 4j, 4j + 2 at bits 0 and 8, 4j + 1, 4j + 3 at bits 16 and 24),
  // then the odd elements' nibbles shifted down beside the even ones: the low half holds elements
  // 4j .. 4j + 3 in order
  const uint32_t p01 = c2[0] | (c2[1] << 8), p23 = c2[2] | (c2[3] << 8);
  return __builtin_amdgcn_perm(p23 | (p23 >> 12), p01 | (p01 >> 12), 0x05040100u);
}

__device__ __forceinline__ uint32_t mix_code8_packed(const uint32_t (&w)[4], int emax, uint32_t m) {
  uint32_t o0, o1;
  return mix_code8_pk<false>(w, mix_pk(emax, m), o0, o1);
}

// Block max of a quad of lanes (one 32-element block) through DPP quad permutes
__device__ __forceinline__ uint32_t quad_max_dpp(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
  return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true)); // quad_perm [2,3,0,1]
}

// mix_quant_lane for 8 bf16 elements held two per word (element 2i in the low half of w[i]); with
// IMG also the 8 E4M3 image bytes.
template <int FMT, bool IMG>
__device__ __forceinline__ uint32_t mix_quant_lane_bf16_img(const uint32_t (&w)[4], int& emax, uint32_t& m,
                                                            uint32_t& out0, uint32_t& out1) {
  const u16x2 a01 = __builtin_elementwise_max(__builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu),
                                              __builtin_bit_cast(u16x2, w[1] & 0x7FFF7FFFu));
  const u16x2 a23 = __builtin_elementwise_max(__builtin_bit_cast(u16x2, w[2] & 0x7FFF7FFFu),
                                              __builtin_bit_cast(u16x2, w[3] & 0x7FFF7FFFu));
  const u16x2 am = __builtin_elementwise_max(a01, a23);
  const uint32_t lmax = (uint32_t)(am[0] > am[1] ? am[0] : am[1]) << 16;
  const uint32_t bmax = quad_max_dpp(lmax);
  const int e = (int)(bmax >> 23) - 127;   // an all-zero block gives -127, clamped to -7
  emax = e < -7 ? -7 : (e > 8 ? 8 : e);
  m = mant3_of(FMT == 1 ? lmax : bmax);
  return mix_code8_pk<IMG>(w, mix_pk(emax, m), out0, out1);
}

// The block constants for every (Emax, m): entry (Emax + 7) * 8 + m = {mu1, pb, m64, 0}; a
// workgroup fills its copy in LDS once.
__device__ __forceinline__ void mix_pk_table_fill(uint4* tbl) {
  for (int t = threadIdx.x; t < 128; t += blockDim.x) {
    const MixPk k = mix_pk((t >> 3) - 7, (uint32_t)t & 7u);
    tbl[t] = make_uint4(k.mu1, k.pb, k.m64, 0u);
  }
}
__device__ __forceinline__ MixPk mix_pk_lookup(const uint4* tbl, int emax, uint32_t m) {
  const uint4 e = tbl[(emax + 7) * 8 + (int)m];
  MixPk k;
  k.mu1 = e.x;
  k.pb = e.y;
  k.m64 = e.z;
  return k;
}

// As mix_quant_lane_bf16_img with the block constants looked up in a filled table.
template <int FMT, bool IMG>
__device__ __forceinline__ uint32_t mix_quant_lane_bf16_tbl(const uint32_t (&w)[4], const uint4* tbl, int& emax,
                                                            uint32_t& m, uint32_t& out0, uint32_t& out1) {
  const u16x2 a01 = __builtin_elementwise_max(__builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu),
                                              __builtin_bit_cast(u16x2, w[1] & 0x7FFF7FFFu));
  const u16x2 a23 = __builtin_elementwise_max(__builtin_bit_cast(u16x2, w[2] & 0x7FFF7FFFu),
                                              __builtin_bit_cast(u16x2, w[3] & 0x7FFF7FFFu));
  const u16x2 am = __builtin_elementwise_max(a01, a23);
  const uint32_t lmax = (uint32_t)(am[0] > am[1] ? am[0] : am[1]) << 16;
  const uint32_t bmax = quad_max_dpp(lmax);
  const int e = (int)(bmax >> 23) - 127;
  emax = e < -7 ? -7 : (e > 8 ? 8 : e);
  m = mant3_of(FMT == 1 ? lmax : bmax);
  return mix_code8_pk<IMG>(w, mix_pk_lookup(tbl, emax, m), out0, out1);
}

// OR over a quad of lanes through DPP quad permutes
__device__ __forceinline__ uint32_t quad_or_dpp(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true);
  return v | (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true);
}

template <int FMT>
__device__ __forceinline__ uint32_t mix_quant_lane_bf16(const uint32_t (&w)[4], int& emax, uint32_t& m) {
  uint32_t o0, o1;
  return mix_quant_lane_bf16_img<FMT, false>(w, emax, m, o0, o1);
}

// One lane's share of a MiX block: the lane holds 8 consecutive elements (fp32 bit patterns) and
// the 4 sub-blocks of a 32-element block sit in the 4 lanes of a quad (sub-block = lane & 3).
// Returns the 8 nibbles (element e at bits 4e) and sets the block's Emax (clamped to [-7, 8]) and
// this lane's 3-bit shared mantissa m (its sub-block's for MiX-4.5b, the block's for MiX-4.25b).
// Emax and m come from the exact fp32 maxima. The element decisions compare against thresholds
// that are 16-bit patterns (see mix_pair), and for such a threshold t and |x| = a,
// a > t exactly when ceil(a / 2^16) > t / 2^16; so the elements are coded by the packed coder on
// their patterns rounded up to 16 bits, with the same result as mix_code on the fp32 patterns.
template <int FMT, bool IMG>  // FMT 0 = MiX-4.25b, 1 = MiX-4.5b
__device__ __forceinline__ uint32_t mix_quant_lane_img(const uint32_t (&xb)[8], int& emax, uint32_t& m,
                                                       uint32_t& out0, uint32_t& out1) {
  uint32_t lmax = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) lmax = max(lmax, xb[i] & 0x7FFFFFFFu);
  const uint32_t bmax = quad_max_dpp(lmax);
  const int e = (int)(bmax >> 23) - 127;   // an all-zero block gives -127, clamped to -7
  emax = e < -7 ? -7 : (e > 8 ? 8 : e);
  m = mant3_of(FMT == 1 ? lmax : bmax);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t x0 = xb[2 * i], x1 = xb[2 * i + 1];
    const uint32_t h0 = ((x0 >> 16) & 0x8000u) | (((x0 & 0x7FFFFFFFu) + 0xFFFFu) >> 16);
    const uint32_t h1 = ((x1 >> 16) & 0x8000u) | (((x1 & 0x7FFFFFFFu) + 0xFFFFu) >> 16);
    w[i] = h0 | (h1 << 16);
  }
  return mix_code8_pk<IMG>(w, mix_pk(emax, m), out0, out1);
}

template <int FMT>
__device__ __forceinline__ uint32_t mix_quant_lane(const uint32_t (&xb)[8], int& emax, uint32_t& m) {
  uint32_t o0, o1;
  return mix_quant_lane_img<FMT, false>(xb, emax, m, o0, o1);
}

// MXFP4 code of one element, thresholds at the E2M1 midpoints times 2^X, ties to the even code.
struct Fp4Thr { uint32_t t[7]; };
__device__ __forceinline__ Fp4Thr fp4_thresholds(int X) {
  Fp4Thr r;
  // midpoints 0.25 0.75 1.25 1.75 2.5 3.5 5 = k 2^s
  r.t[0] = exact_f32_bits(1, X - 2);
  r.t[1] = exact_f32_bits(3, X - 2);
  r.t[2] = exact_f32_bits(5, X - 2);
  r.t[3] = exact_f32_bits(7, X - 2);
  r.t[4] = exact_f32_bits(5, X - 1);
  r.t[5] = exact_f32_bits(7, X - 1);
  r.t[6] = exact_f32_bits(5, X);
  return r;
}
__device__ __forceinline__ uint32_t fp4_code(uint32_t xbits, const Fp4Thr& r) {
  uint32_t a = xbits & 0x7FFFFFFFu;
  uint32_t idx = (a > r.t[0]) + (a >= r.t[1]) + (a > r.t[2]) + (a >= r.t[3]) + (a > r.t[4]) + (a >= r.t[5]) +
                 (a > r.t[6]);
  return ((xbits >> 31) << 3) | idx;
}
// MXINT4: |q| = RNE(a 2^(2-X)) clamped to 7; thresholds (2k+1) 2^(X-3), ties to even.
struct Int4Thr { uint32_t t[7]; };
__device__ __forceinline__ Int4Thr int4_thresholds(int X) {
  Int4Thr r;
#pragma unroll
  for (int k = 0; k < 7; k++) r.t[k] = exact_f32_bits(2 * k + 1, X - 3);
  return r;
}
__device__ __forceinline__ uint32_t int4_code(uint32_t xbits, const Int4Thr& r) {
  uint32_t a = xbits & 0x7FFFFFFFu;
  uint32_t q = 0;
#pragma unroll
  for (int k = 0; k < 7; k++) q += (k & 1) ? (a >= r.t[k]) : (a > r.t[k]);
  return (xbits >> 31) ? ((0u - q) & 0xFu) : q;
}

__device__ __forceinline__ int mx_exponent(uint32_t bmax, int fp4) {
  int E = (int)(bmax >> 23);
  if (fp4) {  // ceil(log2 a) - 2, at least -127
    if (E == 0) return -127;
    int X = E - 127 + ((bmax & 0x7FFFFFu) != 0) - 2;
    return X < -127 ? -127 : X;
  }
  if (E == 0) return -125;  // floor(log2 a) - for a subnormal maximum - is below the clamp
  int X = E - 127;
  return X < -125 ? -125 : X;
}


// ------------------------------------------------------------------ code -> E4M3 decoders

// 8 MiX nibbles (element e at bits 4e) with shared mantissa m -> 8 E4M3 bytes in element order.
// byte = s<<7 | (8-dE)<<3 | m; nibble 0x7 (zero) -> 0x00; nibble 0xF -> (1<<3) | m.
__device__ __forceinline__ void mix8_to_e4m3(uint32_t w, uint32_t m, uint32_t& out0, uint32_t& out1) {
  const uint32_t m4 = m * 0x01010101u;
  uint32_t r[2];
#pragma unroll
  for (int h = 0; h < 2; h++) {
    uint32_t x = (w >> (4 * h)) & 0x0F0F0F0Fu;  // h=0: elements 0,2,4,6; h=1: 1,3,5,7
    uint32_t d = x & 0x07070707u;
    uint32_t s = x & 0x08080808u;
    uint32_t v = (0x40404040u - (d << 3)) | (s << 4) | m4;
    uint32_t d7 = (d + 0x01010101u) & 0x08080808u;  // 0x08 in bytes with dE == 7
    v &= ~(d7 << 4);                                // reclaimed pattern: positive
    uint32_t z = d7 & ~s;                           // dE == 7 with sign 0: zero
    v &= ~((z >> 3) * 0xFFu);
    r[h] = v;
  }
  out0 = __builtin_amdgcn_perm(r[1], r[0], 0x05010400u);
  out1 = __builtin_amdgcn_perm(r[1], r[0], 0x07030602u);
}

// 8 MXINT4 nibbles -> 8 E4M3 bytes of q/4 (q two's complement in [-8, 7]).
__device__ __forceinline__ void int4x8_to_e4m3(uint32_t w, uint32_t& out0, uint32_t& out1) {
  const uint32_t lo0 = 0x34302800u, lo1 = 0x3E3C3A38u;  // q = 0..7
  const uint32_t hi0 = 0xBABCBEC0u, hi1 = 0xA8B0B4B8u;  // q = -8..-1
  uint32_t r[2];
#pragma unroll
  for (int h = 0; h < 2; h++) {
    uint32_t x = (w >> (4 * h)) & 0x0F0F0F0Fu;
    uint32_t sel = x & 0x07070707u;
    uint32_t a = __builtin_amdgcn_perm(lo1, lo0, sel);
    uint32_t b = __builtin_amdgcn_perm(hi1, hi0, sel);
    uint32_t msk = ((x & 0x08080808u) >> 3) * 0xFFu;
    r[h] = (a & ~msk) | (b & msk);
  }
  out0 = __builtin_amdgcn_perm(r[1], r[0], 0x05010400u);
  out1 = __builtin_amdgcn_perm(r[1], r[0], 0x07030602u);
}

}  // namespace mix
