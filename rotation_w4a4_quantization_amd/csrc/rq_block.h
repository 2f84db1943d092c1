// Register-level pieces of the 128-point rotate + quantize step, shared by
// the rotate kernels and the fused decode kernel so that both compute the
// same values bit for bit (gfx950, wave64).
//
// Layout: a 128-element Hadamard block of a row is held by a quad of 4 lanes;
// lane q holds elements 32r + 8q + e in register 8r + e (r, e = 0..3, 0..7).
#pragma once

#include "common.h"

namespace w4a4 {

// Pack 8 codes whose value sits in the low 4 bits of each word (bits 4..7
// zero, higher bits ignored) into one dword, element 0 in bits 3:0.
__device__ __forceinline__ uint32_t pack8(const uint32_t* b) {
  const uint32_t p01 = (b[1] << 4) | b[0];
  const uint32_t p23 = (b[3] << 4) | b[2];
  const uint32_t p45 = (b[5] << 4) | b[4];
  const uint32_t p67 = (b[7] << 4) | b[6];
  const uint32_t lo = __builtin_amdgcn_perm(p23, p01, 0x0C0C0400u);   // [p01.b0, p23.b0, 0, 0]
  const uint32_t hi = __builtin_amdgcn_perm(p67, p45, 0x0C0C0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);                   // [lo.b0, lo.b1, hi.b0, hi.b1]
}

// In-quad 128-point FWHT of the 32 fp16 values a lane loaded (chunks q, q+4,
// q+8, q+12 of the block, as four uint4).  The first butterfly (element bit
// 0, the two halves of a dword) is fused with the conversion to fp32; the
// register bits (element bits 1-2 and 5-6) follow in registers and the two
// quad-lane bits (3-4) with DPP.  s0, s1 = -1 on the lanes whose quad bit 0,
// 1 is set; afterwards the lane holds sgn * z with
// sgn = -1 iff exactly one of those bits is set.
__device__ __forceinline__ void fwht128_quad(const uint4 (&w)[4], float (&v)[32], float s0, float s1) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const uint32_t d[4] = {w[r4].x, w[r4].y, w[r4].z, w[r4].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) cvt_bfly(d[j], v[8 * r4 + 2 * j], v[8 * r4 + 2 * j + 1]);
  }
#pragma unroll
  for (int b = 2; b < 32; b <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (!(i & b)) {
        const float a = v[i], c = v[i | b];
        v[i] = a + c;
        v[i | b] = a - c;
      }
    }
  }
  dpp_bfly_q0(v, s0);
  dpp_bfly_q0(v + 16, s0);
  dpp_bfly_q1(v, s1);
  dpp_bfly_q1(v + 16, s1);
}

// Symmetric INT4 codes of 8 consecutive values: fma gives 2^23*1.5 + 8 +
// rne(z*inv) (sinv = sgn * inv, so the lane's sign cancels exactly); the low
// nibble is the code in offset-8 binary, turned into two's complement by the
// final xor.  bitsum accumulates the 8 bit patterns (magic + 8 + code).
__device__ __forceinline__ uint32_t sym_word(const float* v8, float sinv, uint32_t& bitsum) {
  uint32_t b[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    b[e] = fbits(fmaf(v8[e], sinv, kRneMagic + 8.0f));
    bitsum += b[e];
  }
  return pack8(b) ^ 0x88888888u;
}

}  // namespace w4a4
