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

// Tile coordinates of this workgroup.  Tiles are walked in groups of 16 tile
// rows, column by column inside a group, so the workgroups resident at one
// time cover a 16-row block of tiles and share both its A rows and its B
// rows in L2 (row-major order would stream every B tile once per pair of
// tile rows); measured 2-5% faster on the q_proj, down_proj and gate/up
// shapes.  The mapping is a bijection of [0, tiles_m * tiles_n).
__device__ __forceinline__ void tile_coords(int64_t tiles_m, int64_t tiles_n, int64_t& tm, int64_t& tn) {
  constexpr int64_t GM = 16;
  const int64_t pid = blockIdx.x;
  const int64_t in_group = GM * tiles_n;
  const int64_t gid = pid / in_group;
  const int64_t first_m = gid * GM;
  const int64_t gsz = tiles_m - first_m < GM ? tiles_m - first_m : GM;
  const int64_t r = pid - gid * in_group;
  tm = first_m + r % gsz;
  tn = r / gsz;
}

// 16-byte output store marked non-temporal: the fp32 result is written once
// and not re-read by this kernel, so it should not displace the operand rows
// that other tiles still read from L2 / MALL (measured 3-15% faster).
__device__ __forceinline__ void store_stream4(float* dst, const float* y) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(v4f{y[0], y[1], y[2], y[3]}, reinterpret_cast<v4f*>(dst));
}

// 4x4 transpose inside a quad of lanes: on entry lane k of the quad holds
// column k of a 4x4 block in y[0..3] (y[v] = row v); on exit it holds row k
// (y[c] = column c).  Two butterflies swap a lane-index bit with a
// register-index bit (DPP quad permutes).
__device__ __forceinline__ void quad_transpose4(float* y, int k) {
  {
    const bool hi = k & 1;
#pragma unroll
    for (int m = 0; m < 4; m += 2) {
      const float send = hi ? y[m] : y[m + 1];
      const float recv = dpp_f<0xB1>(send);
      y[m] = hi ? recv : y[m];
      y[m + 1] = hi ? y[m + 1] : recv;
    }
  }
  {
    const bool hi = k & 2;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float send = hi ? y[m] : y[m + 2];
      const float recv = dpp_f<0x4E>(send);
      y[m] = hi ? recv : y[m];
      y[m + 2] = hi ? y[m + 2] : recv;
    }
  }
}

// Stores two horizontally adjacent 16x16 fp32 output blocks as full 128-byte
// row segments.  On entry lane (fr, g) = (lane & 15, lane >> 4) holds rows
// 4g..4g+3 of column fr of the left block in y0[0..3] and of the right block
// in y1[0..3] (the MFMA output layout); `rb` is the output row of y*[0] and
// `cb` the first column of the left block.  After a quad transpose of each
// block, lane k of a quad holds 4 consecutive columns of row rb + k; lanes k
// and k ^ 2 then trade halves, so that each of the two 16-byte stores per
// lane writes 8 rows x 32 consecutive columns: 8 lanes cover each 128-byte
// row segment, instead of 16 rows x 64 bytes (measured on the q_proj GEMM:
// the 32 MiB output phase drops from about 7 to 5.5 us).  Rows at or past M
// and columns at or past N are not written.
__device__ __forceinline__ void store_block_pair(float* y, int64_t ldy, int64_t M, int64_t N,
                                                 int64_t rb, int64_t cb, int fr, float* y0, float* y1) {
  const int k = fr & 3;
  quad_transpose4(y0, k);
  quad_transpose4(y1, k);
  const bool hi = k & 2;
  float first[4], second[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float recv = dpp_f<0x4E>(hi ? y0[c] : y1[c]);   // from lane k ^ 2
    first[c] = hi ? recv : y0[c];
    second[c] = hi ? y1[c] : recv;
  }
  // first: row rb + (k & 1) of the left block (k < 2) or of the right block
  // (k >= 2); second: row rb + 2 + (k & 1), same blocks
  const int64_t r = rb + (k & 1);
  const int64_t c0 = cb + (fr & ~3) + (hi ? 16 : 0);
  const bool vec_ok = (ldy & 3) == 0 && c0 + 3 < N;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t row = r + 2 * h;
    const float* v = h ? second : first;
    if (row < M) {
      float* dst = y + row * ldy + c0;
      if (vec_ok) {
        store_stream4(dst, v);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (c0 + c < N) dst[c] = v[c];
      }
    }
  }
}

}  // namespace w4a4
