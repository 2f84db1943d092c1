// Device helpers shared by the rotate/quantize and GEMM kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a4 {

constexpr int kWave = 64;

// float -> integer trick: fmaf(t, inv, kRneMagic) rounds the exact product
// t*inv to the nearest integer (ties to even) when |t*inv| < 2^22, and the
// integer sits in the low mantissa bits (the float's ulp there is 1).
constexpr float kRneMagic = 12582912.0f;          // 1.5 * 2^23, bit pattern 0x4B400000
constexpr uint32_t kRneMagicBits = 0x4B400000u;

__device__ __forceinline__ uint32_t fbits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __builtin_bit_cast(float, u); }

// DPP lane shuffles inside a quad (4 consecutive lanes).
// quad_perm selectors: [1,0,3,2] = 0xB1 (partner = lane ^ 1), [2,3,0,1] = 0x4E (lane ^ 2).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return bitsf((uint32_t)__builtin_amdgcn_mov_dpp((int)fbits(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  return fmaxf(v, dpp_f<0x4E>(v));
}
__device__ __forceinline__ float quad_min(float v) {
  v = fminf(v, dpp_f<0xB1>(v));
  return fminf(v, dpp_f<0x4E>(v));
}
__device__ __forceinline__ int quad_sum(int v) {
  v += dpp_i<0xB1>(v);
  return v + dpp_i<0x4E>(v);
}

// xor shuffle across the wave (ds_bpermute); `mask` < 64.
__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  const int lane = __lane_id();
  return bitsf((uint32_t)__builtin_amdgcn_ds_bpermute(((lane ^ mask) << 2), (int)fbits(v)));
}

// fp16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float h2f(uint32_t h16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}

// Correctly rounded fp32 quotient a / b for finite positive operands: the
// float64 quotient is correctly rounded to 53 bits, and rounding that to 24
// bits again gives the correctly rounded fp32 quotient (53 >= 2*24 + 2).
__device__ __forceinline__ float div_rn(float a, float b) {
  return (float)((double)a / (double)b);
}

}  // namespace w4a4
