// Layout of the GEMM operand images: the decode-once form of A-MiX and W-MX operands that the
// block-scaled MFMA GEMM (gemm_f8.hip) streams.
//
// A image of an [M, K] MiX operand:
//   a8    [M, K]                      E4M3 bytes: element (1.m)_2 2^(Emax-dE) as (1.m)_2 2^(1-dE)
//   as_p  [K/128][tiles_m][256][4]    E8M0 block scales 2^(Emax-1): per (K step, tile), a row's
//                                     four block scales in one dword (f8_a_scale_pos)
// B image of an [N, K] MX operand:
//   bs_p  [K/128][tiles_n][1024]      E8M0 block scales, permuted (f8_scale_pos), for the tiled product
//   b8    MXFP4: [K/128][N][64]       the codes step-major: a K step's 64-byte slices of all rows are
//                                     contiguous, so a tile's slice of a step is whole cache lines
//         MXINT4 (and g16): [N, K]    E4M3 bytes of the element values (q/4, or the folded g16 values)
//   bs_v  [ceil(N/16)][K/128][16][4]  the same scales per 16-row group, for the small-M product
// tiles_m = ceil(M / 256), tiles_n = ceil(N / 256); every part starts on a 256-byte boundary.
#pragma once
#include <cstddef>
#include <cstdint>

namespace mix {

constexpr int FT = 256;   // GEMM tile rows (M) and columns (N)
constexpr int FK = 128;   // K per pipeline step

// Byte position of the A scale of (tile row rin, 32-wide block b4 of the K step) inside the 1 KB
// a (K step, tile) pair owns: row-major, so a row-wise producer writes one dword per K step.
__host__ __device__ inline int f8_a_scale_pos(int rin, int b4) { return rin * 4 + b4; }

// Byte position of the B scale of (tile row rin, block b4) inside its 1 KB: [half-tile w][lane
// group gq][r][K half h][sub-tile i], so that the 8 bytes a GEMM lane needs for one K step (four
// 32-row sub-tiles, two K halves) are contiguous.
__host__ __device__ inline int f8_scale_pos(int rin, int b4) {
  const int w = rin >> 7, i = (rin >> 5) & 3, r = rin & 31;
  const int h = b4 >> 1, gq = b4 & 1;
  return ((w * 2 + gq) * 32 + r) * 8 + h * 4 + i;
}

inline size_t f8_al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct F8AImage {
  size_t a8, as_p, total;
};
inline F8AImage f8_a_image_layout(int64_t M, int64_t K) {
  const int64_t tm = (M + FT - 1) / FT;
  F8AImage L{};
  L.a8 = 0;
  L.as_p = f8_al256((size_t)M * K);
  L.total = L.as_p + f8_al256((size_t)(K / FK) * tm * 1024);
  return L;
}

struct F8BImage {
  size_t bs_p, b8, bs_v, total;
};
inline F8BImage f8_b_image_layout(int b_fp4, int64_t N, int64_t K) {
  const int64_t tn = (N + FT - 1) / FT;
  F8BImage L{};
  L.bs_p = 0;
  L.b8 = f8_al256((size_t)(K / FK) * tn * 1024);
  L.bs_v = L.b8 + f8_al256(b_fp4 ? (size_t)N * K / 2 : (size_t)N * K);
  L.total = L.bs_v + f8_al256((size_t)((N + 15) / 16) * (K / FK) * 64);
  return L;
}

}  // namespace mix
