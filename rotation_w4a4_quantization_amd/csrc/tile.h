// Helpers shared by the GEMM kernels (gfx950, wave64): INT4 -> int8
// widening, the int8 MFMA, tile order and the output tile epilogue.
#pragma once

#include "common.h"

namespace w4a4 {

typedef int v4i __attribute__((ext_vector_type(4)));

// Packed two's-complement nibbles -> int8 lanes scaled by 16, without
// per-element shifts: the bytes of (p << 4) & 0xF0F0F0F0 are 16 x the even
// nibbles and those of p & 0xF0F0F0F0 16 x the odd ones, sign included.
__device__ __forceinline__ void widen_signed(uint32_t p, uint32_t& even16, uint32_t& odd16) {
  even16 = (p << 4) & 0xF0F0F0F0u;
  odd16 = p & 0xF0F0F0F0u;
}

__device__ __forceinline__ v4i mfma16(const v4i& a, const v4i& b, const v4i& c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// XCD-aware tile coordinates.  Workgroup i of a launch runs on XCD i % 8 of
// the 8 that share the chip, and each XCD has its own L2.  The first
// 8 * floor(T / 8) workgroups are renumbered so that XCD x receives the
// contiguous range [x T8/8, (x + 1) T8/8) of a grouped order with groups of
// 4 tile rows, i.e. compact blocks of tiles whose A and B rows its L2 shares
// (measured on the q_proj and 8192 x 4096 x 4096 shapes: 2-4% faster than
// a grouped order of 16 tile rows with no renumbering).  The remaining T % 8
// workgroups keep their own index.  The mapping is a bijection of [0, T).
__device__ __forceinline__ void tile_coords_xcd(int64_t tiles_m, int64_t tiles_n, int64_t& tm, int64_t& tn) {
  constexpr int64_t GM = 4;
  const int64_t T = tiles_m * tiles_n;
  const int64_t T8 = T - T % 8;
  int64_t pid = blockIdx.x;
  if (pid < T8) pid = (pid % 8) * (T8 / 8) + pid / 8;
  const int64_t in_group = GM * tiles_n;
  const int64_t gid = pid / in_group;
  const int64_t first_m = gid * GM;
  const int64_t gsz = tiles_m - first_m < GM ? tiles_m - first_m : GM;
  const int64_t r = pid - gid * in_group;
  tm = first_m + r % gsz;
  tn = r / gsz;
}

typedef float v4f __attribute__((ext_vector_type(4)));

// Stores two horizontally adjacent 16x16 fp32 output blocks held in the
// layout of an MFMA whose first operand is the weight fragment and second
// the activation fragment: lane (fr, g) = (lane & 15, lane >> 4) holds row
// r0 + fr, columns c0 + 4g .. c0 + 4g + 3 of the left block in ya and of
// the right block (columns + 16) in yb.  In the fast path (`full`: the
// 16 x 32 region lies inside M x N and ldy is a multiple of 4 floats) lanes
// fr and fr ^ 8 trade one block (one DPP row rotate by 8 per value), so that
// each of the two 16-byte non-temporal stores per lane writes 8 rows x 128
// contiguous bytes: full cache lines (the 32 MiB q_proj output phase drops
// from about 7 to 5.5 us against 64-byte row segments).  Otherwise every
// element is stored under its own row and column check.  The output is not
// re-read, so the stores bypass the caches' retention (measured 3-15%
// faster).
__device__ __forceinline__ void store_pair_rows(float* y, int64_t ldy, int64_t M, int64_t N, int64_t r0,
                                                int64_t c0, int fr, int g, bool full, v4f ya, v4f yb) {
  if (full) {
    const bool lo = fr < 8;
    v4f out1, out2;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float send = lo ? yb[v] : ya[v];
      const float recv = bitsf((uint32_t)__builtin_amdgcn_mov_dpp((int)fbits(send), 0x128, 0xF, 0xF, true));
      out1[v] = lo ? ya[v] : recv;    // rows r0 .. r0 + 7
      out2[v] = lo ? recv : yb[v];    // rows r0 + 8 .. r0 + 15
    }
    const int64_t r1 = r0 + (lo ? fr : fr - 8);
    const int64_t c = c0 + (lo ? 0 : 16) + 4 * g;
    __builtin_nontemporal_store(out1, reinterpret_cast<v4f*>(y + r1 * ldy + c));
    __builtin_nontemporal_store(out2, reinterpret_cast<v4f*>(y + (r1 + 8) * ldy + c));
  } else {
    const int64_t row = r0 + fr;
    if (row < M) {
      const int64_t c = c0 + 4 * g;
      float* dst = y + row * ldy + c;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (c + v < N) dst[v] = ya[v];
        if (c + 16 + v < N) dst[16 + v] = yb[v];
      }
    }
  }
}

}  // namespace w4a4
