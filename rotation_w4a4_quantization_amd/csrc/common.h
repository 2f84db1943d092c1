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

// First butterfly fused with the fp16 -> fp32 conversion: for a dword holding
// two fp16 values (lo, hi), a = lo + hi and b = lo - hi, each one fma with a
// single rounding (v_fma_mix_f32 reads the fp16 halves directly).
__device__ __forceinline__ void cvt_bfly(uint32_t h2, float& a, float& b) {
  asm("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(a) : "v"(h2));
  asm("v_fma_mix_f32 %0, %1, -1.0, %1 op_sel:[1,0,0] op_sel_hi:[1,0,1]" : "=v"(b) : "v"(h2));
}

// Butterfly across a quad-lane bit with one VALU op per value:
//   v <- v + s * v[partner]   (v_fmac_f32 with a DPP quad permute on src0).
// With s = +1 in the lane whose bit is 0 and s = -1 in the lane whose bit is
// 1, the low lane gets x_lo + x_hi and the high lane x_hi - x_lo, i.e. the
// butterfly output negated; the caller tracks that sign per lane.  The
// leading s_nop covers the two wait states a DPP read needs after a VALU
// write of the same register.
#define W4A4_DPP_FMAC(SEL)                                                              \
  "v_fmac_f32_dpp %0, %0, %16 " SEL " row_mask:0xf bank_mask:0xf\n"                    \
  "v_fmac_f32_dpp %1, %1, %16 " SEL " row_mask:0xf bank_mask:0xf\n"                    \
  "v_fmac_f32_dpp %2, %2, %16 " SEL " row_mask:0xf bank_mask:0xf\n"                    \
  "v_fmac_f32_dpp %3, %3, %16 " SEL " row_mask:0xf bank_mask:0xf\n"                    \
  "v_fmac_f32_dpp %4, %4, %16 " SEL " row_mask:0xf bank_mask:0xf\n"                    \
  "v_fmac_f32_dpp %5, %5, %16 " SEL " row_mask:0xf bank_mask:0xf\n"                    \
  "v_fmac_f32_dpp %6, %6, %16 " SEL " row_mask:0xf bank_mask:0xf\n"                    \
  "v_fmac_f32_dpp %7, %7, %16 " SEL " row_mask:0xf bank_mask:0xf\n"                    \
  "v_fmac_f32_dpp %8, %8, %16 " SEL " row_mask:0xf bank_mask:0xf\n"                    \
  "v_fmac_f32_dpp %9, %9, %16 " SEL " row_mask:0xf bank_mask:0xf\n"                    \
  "v_fmac_f32_dpp %10, %10, %16 " SEL " row_mask:0xf bank_mask:0xf\n"                  \
  "v_fmac_f32_dpp %11, %11, %16 " SEL " row_mask:0xf bank_mask:0xf\n"                  \
  "v_fmac_f32_dpp %12, %12, %16 " SEL " row_mask:0xf bank_mask:0xf\n"                  \
  "v_fmac_f32_dpp %13, %13, %16 " SEL " row_mask:0xf bank_mask:0xf\n"                  \
  "v_fmac_f32_dpp %14, %14, %16 " SEL " row_mask:0xf bank_mask:0xf\n"                  \
  "v_fmac_f32_dpp %15, %15, %16 " SEL " row_mask:0xf bank_mask:0xf"

#define W4A4_DPP_OPS16(v, s)                                                            \
  : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), \
    "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]),           \
    "+v"(v[13]), "+v"(v[14]), "+v"(v[15])                                                \
  : "v"(s)

// quad lane bit 0 (partner = lane ^ 1) on 16 registers
__device__ __forceinline__ void dpp_bfly_q0(float* v, float s) {
  asm volatile("s_nop 1\n" W4A4_DPP_FMAC("quad_perm:[1,0,3,2]") W4A4_DPP_OPS16(v, s));
}
// quad lane bit 1 (partner = lane ^ 2) on 16 registers
__device__ __forceinline__ void dpp_bfly_q1(float* v, float s) {
  asm volatile("s_nop 1\n" W4A4_DPP_FMAC("quad_perm:[2,3,0,1]") W4A4_DPP_OPS16(v, s));
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
