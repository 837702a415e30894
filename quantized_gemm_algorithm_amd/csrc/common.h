// Device helpers shared by the MiX HIP kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mix {

// ------------------------------------------------------------------ bit helpers

__device__ __forceinline__ uint32_t f32_bits(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float bits_f32(uint32_t u) { return __uint_as_float(u); }

// bf16 pattern -> exact fp32 bits
__device__ __forceinline__ uint32_t bf16_to_f32_bits(uint32_t b16) { return b16 << 16; }

// fp32 -> bf16 round-to-nearest-even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 -> packed bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32; the kernels keep fp32
// denormals, so subnormal inputs round like any other), a in the low half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16_rne(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// 16-byte global store marked non-temporal: an output written once and not read back by this
// kernel, so it should not displace the operand lines the L2 keeps for other tiles.
__device__ __forceinline__ void store16_nt(void* p, uint4 v) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, (u32x4_t*)p);
}

// Exact fp32 bit pattern of k * 2^e for 1 <= k < 2^24 (normal or subnormal result; e >= -149 - bits).
__device__ __forceinline__ uint32_t exact_f32_bits(uint32_t k, int e) {
  int nb = 31 - __builtin_clz(k);  // index of the leading one
  int ex = e + nb;                  // unbiased exponent of the value
  if (ex >= -126) {
    uint32_t mant = (nb <= 23) ? ((k << (23 - nb)) & 0x7FFFFFu) : ((k >> (nb - 23)) & 0x7FFFFFu);
    return ((uint32_t)(ex + 127) << 23) | mant;
  }
  int sh = e + 149;  // subnormal: value = k * 2^e = (k << sh) * 2^-149
  return sh >= 0 ? (k << sh) : (k >> (-sh));
}

// Top three fraction bits of the significand of a non-negative float given by its bits
// (subnormals are normalised first; zero gives 0).
__device__ __forceinline__ uint32_t mant3_of(uint32_t a) {
  if (a == 0) return 0;
  uint32_t e = a >> 23;
  uint32_t m = a & 0x7FFFFFu;
  if (e == 0) {
    int sh = __builtin_clz(m) - 8;  // move the leading one to bit 23
    m = (m << sh) & 0x7FFFFFu;
  }
  return m >> 20;
}

// ------------------------------------------------------------------ cross-lane reductions (DPP)

// max over the 4 lanes of a quad (lanes 4q..4q+3), unsigned
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  uint32_t t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  return v > t ? v : t;
}

// global -> LDS copies (global_load_lds_dword[x4]): lane i's bytes land at LDS byte
// m0 + size * i. The copy has no destination register; it is written as a statement so that the
// compiler does not drain every outstanding copy before each LDS read of another stage -- a kernel
// waits for its copies explicitly (vmcnt) before the barrier that publishes a stage.
typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(gptr) : "memory", "m0");
}
// the same copy from a wave-uniform base plus a 32-bit per-lane byte offset (one address register)
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds_base), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_base), "v"(gptr) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_ptr_t)p; }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Division of a flat index n < 2^31 by a fixed d < 2^31 as a multiply and a shift:
// q = (n * m) >> sh with sh = 31 + ceil(log2 d), m = ceil(2^sh / d) < 2^33. The error term is below
// n / 2^sh < 2^-ceil(log2 d) <= 1/d, less than the distance from n/d to the next integer, so q is
// floor(n / d) exactly. For larger indices (ok == 0) the plain 64-bit division is used.
struct FastDiv {
  uint64_t m;
  int sh;
  int ok;
};
inline FastDiv make_fastdiv(int64_t d, int64_t n_max) {
  FastDiv f{0, 0, 0};
  if (d <= 0 || d >= (int64_t(1) << 31) || n_max >= (int64_t(1) << 31)) return f;
  int l = 0;
  while ((int64_t(1) << l) < d) l++;
  f.sh = 31 + l;
  f.m = (((uint64_t)1 << f.sh) + (uint64_t)d - 1) / (uint64_t)d;
  f.ok = 1;
  return f;
}
__device__ __forceinline__ int64_t fast_div(int64_t n, int64_t d, const FastDiv& f) {
  return f.ok ? (int64_t)(((uint64_t)(uint32_t)n * f.m) >> f.sh) : n / d;
}

// bitwise OR over the 4 lanes of a quad
__device__ __forceinline__ uint32_t quad_or_u32(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
  return v;
}

// full-wave reductions through ds_swizzle / bpermute (64 lanes)
__device__ __forceinline__ float wave_max_f32(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace mix
