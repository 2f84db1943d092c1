// W4A4 GEMM on gfx950 int8 MFMA.
//
// The product of the rotated, quantized operands is an integer dot product
// of 4-bit codes ("Rotations for 4-Bit Activations: QuaRot, SpinQuant, and
// Friends", sections "A rotation changes nothing, and that is the point" and
// "What it buys in 4 bits").  CDNA4 has no INT4 matrix instruction, so the
// packed nibbles are widened to int8 and multiplied with
// v_mfma_i32_16x16x64_i8 into an exact int32 accumulator.
//
// Widening (no per-element shifts): for a dword of 8 two's-complement
// nibbles p, the bytes of (p & 0xF0F0F0F0) are 16 * (odd nibbles) and the
// bytes of ((p << 4) & 0xF0F0F0F0) are 16 * (even nibbles), already sign
// extended.  Both operands are widened the same way, so the K order inside
// every 32-element chunk is permuted identically on both sides and the dot
// product is unchanged; the accumulator holds 256 * acc exactly
// (|256 acc| <= 256 * 49 * K < 2^31 for K <= 131072) and acc = that >> 8.
// Asymmetric activations (unsigned codes, one zero-point per row and group of
// 128) are widened to the exact levels u - zp in [-15, 15], so the weights'
// 16x factor leaves 16 * A_g in the accumulator.
#include "common.h"
#include "kernels.h"

namespace w4a4 {

typedef int v4i __attribute__((ext_vector_type(4)));

namespace {

constexpr int BM = 128, BN = 128, BK = 128;   // BK in 4-bit elements
constexpr int LROW = 144;                      // LDS bytes per int8 row: 128 + 16 pad
constexpr int TILE = 128 * LROW;               // one operand tile in LDS
constexpr int kStageBytes = 2 * TILE;          // A + B
constexpr int kGemmLds = 2 * kStageBytes + 2 * 128 * 4;   // 2 stages + asym row scales

__device__ __forceinline__ void widen_signed(uint32_t p, uint32_t& even16, uint32_t& odd16) {
  even16 = (p << 4) & 0xF0F0F0F0u;
  odd16 = p & 0xF0F0F0F0u;
}

// Unsigned nibbles u, zero-point z (replicated in every byte as zx4):
// bytes of the result are the int8 levels u - z.
__device__ __forceinline__ uint32_t levels(uint32_t u4, uint32_t zx4) {
  return ((u4 | 0x80808080u) - zx4) ^ 0x80808080u;
}

__device__ __forceinline__ v4i mfma16(const v4i& a, const v4i& b, const v4i& c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

}  // namespace

// ---------------------------------------------------------------- tiled kernel
// 128x128 output tile per workgroup, 4 waves of 64x64 (4x4 MFMA blocks of
// 16x16).  Each 128-wide K step: every thread loads 4 x 16 packed bytes,
// widens them once to int8 and writes them to the next LDS stage while the
// waves run 32 MFMAs each on the current stage.
template <bool ASYM>
__global__ void __launch_bounds__(256) gemm_tile_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* sxs = reinterpret_cast<float*>(smem + 2 * kStageBytes);   // [2][128] asym row scales

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tiles_n = (p.N + BN - 1) / BN;
  const int64_t tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int nkt = p.K / BK;
  const int64_t ldc = p.K / 2;   // packed bytes per row
  const int G = nkt;

  // loader coordinates: 4 chunks of 16 packed bytes per thread
  const int lrow = tid >> 2, lc = tid & 3;
  const uint8_t* gptr[4];
  bool gval[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = lrow + 64 * (j & 1);
    if (j < 2) {
      gval[j] = m0 + row < p.M;
      gptr[j] = p.xq + (gval[j] ? (m0 + row) : 0) * ldc + 16 * lc;
    } else {
      gval[j] = n0 + row < p.N;
      gptr[j] = p.wq + (gval[j] ? (n0 + row) : 0) * ldc + 16 * lc;
    }
  }

  uint4 g[4];
  uint32_t zx4[2] = {0u, 0u};
  float sxn = 0.0f;
  auto gload = [&](int kt) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      g[j] = gval[j] ? *reinterpret_cast<const uint4*>(gptr[j] + kt * 64) : make_uint4(0u, 0u, 0u, 0u);
    if constexpr (ASYM) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t row = m0 + lrow + 64 * j;
        zx4[j] = gval[j] ? (uint32_t)p.xz[row * G + kt] * 0x01010101u : 0u;
      }
      if (tid < 128) sxn = (m0 + tid < p.M) ? p.xs[(m0 + tid) * G + kt] * 0.0625f : 0.0f;
    }
  };
  auto lstore = [&](int stage) {
    uint8_t* base = smem + stage * kStageBytes;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = lrow + 64 * (j & 1);
      uint8_t* dst = base + (j >> 1) * TILE + row * LROW + 32 * lc;
      const uint32_t w[4] = {g[j].x, g[j].y, g[j].z, g[j].w};
      uint32_t o[8];
      if (ASYM && j < 2) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          o[2 * d] = levels(w[d] & 0x0F0F0F0Fu, zx4[j]);
          o[2 * d + 1] = levels((w[d] >> 4) & 0x0F0F0F0Fu, zx4[j]);
        }
      } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) widen_signed(w[d], o[2 * d], o[2 * d + 1]);
      }
      reinterpret_cast<uint4*>(dst)[0] = make_uint4(o[0], o[1], o[2], o[3]);
      reinterpret_cast<uint4*>(dst)[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
    if constexpr (ASYM) {
      if (tid < 128) sxs[stage * 128 + tid] = sxn;
    }
  };

  v4i acc[4][4];
  float yf[ASYM ? 4 : 1][ASYM ? 4 : 1][ASYM ? 4 : 1];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};
  if constexpr (ASYM) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) yf[i][j][v] = 0.0f;
  }

  const int fr = lane & 15, fk = 16 * (lane >> 4);
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int s = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);
    const uint8_t* As = smem + s * kStageBytes + (wm * 64 + fr) * LROW + fk;
    const uint8_t* Bs = smem + s * kStageBytes + TILE + (wn * 64 + fr) * LROW + fk;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v4i a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const v4i*>(As + i * 16 * LROW + 64 * h);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const v4i*>(Bs + j * 16 * LROW + 64 * h);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(a[i], b[j], acc[i][j]);
    }
    if constexpr (ASYM) {
      // one group of 128 per K step: fold 16*A_g into the float sums
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 sx = *reinterpret_cast<const float4*>(sxs + s * 128 + wm * 64 + 16 * i + 4 * (lane >> 4));
        const float sv[4] = {sx.x, sx.y, sx.z, sx.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int v = 0; v < 4; ++v) yf[i][j][v] = fmaf(sv[v], (float)acc[i][j][v], yf[i][j][v]);
          acc[i][j] = v4i{0, 0, 0, 0};
        }
      }
    }
    if (kt + 1 < nkt) lstore(s ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds rows 4*(lane/16)+v, column lane%16 of every 16x16 block
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t rb = m0 + wm * 64 + 16 * i + 4 * (lane >> 4);
    float sx[4];
    if constexpr (!ASYM) {
#pragma unroll
      for (int v = 0; v < 4; ++v) sx[v] = (rb + v < p.M) ? p.xs[rb + v] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 64 + 16 * j + fr;
      if (col >= p.N) continue;
      const float sw = p.ws[col];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (rb + v >= p.M) continue;
        float y;
        if constexpr (ASYM) y = yf[i][j][v] * sw;
        else y = (sx[v] * sw) * (float)(acc[i][j][v] >> 8);
        p.y[(rb + v) * p.ldy + col] = y;
      }
    }
  }
}

// ---------------------------------------------------------------- decode kernel
// M <= 16 rows (symmetric): one workgroup per 16 output columns; the 4 waves
// split the K steps and stream W's packed rows straight into registers, one
// 16x16x64 MFMA pair per 128-wide K step (rows of X beyond M are zero).
__global__ void __launch_bounds__(256) gemm_decode_kernel(GemmParams p) {
  __shared__ v4i red[3][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, kg = 16 * (lane >> 4);
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int nkt = p.K / BK;
  const int64_t ldc = p.K / 2;
  const bool xv = i < p.M, wv = n0 + i < p.N;
  const uint8_t* xp = p.xq + (xv ? i : 0) * ldc + kg;
  const uint8_t* wp = p.wq + (wv ? (n0 + i) : 0) * ldc + kg;

  v4i acc = v4i{0, 0, 0, 0};
#pragma unroll 4
  for (int kt = wave; kt < nkt; kt += 4) {
    const uint4 xa = xv ? *reinterpret_cast<const uint4*>(xp + kt * 64) : make_uint4(0u, 0u, 0u, 0u);
    const uint4 wb = wv ? *reinterpret_cast<const uint4*>(wp + kt * 64) : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t xw[4] = {xa.x, xa.y, xa.z, xa.w};
    const uint32_t ww[4] = {wb.x, wb.y, wb.z, wb.w};
    uint32_t ao[8], bo[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      widen_signed(xw[d], ao[2 * d], ao[2 * d + 1]);
      widen_signed(ww[d], bo[2 * d], bo[2 * d + 1]);
    }
    acc = mfma16(v4i{(int)ao[0], (int)ao[1], (int)ao[2], (int)ao[3]},
                 v4i{(int)bo[0], (int)bo[1], (int)bo[2], (int)bo[3]}, acc);
    acc = mfma16(v4i{(int)ao[4], (int)ao[5], (int)ao[6], (int)ao[7]},
                 v4i{(int)bo[4], (int)bo[5], (int)bo[6], (int)bo[7]}, acc);
  }
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    acc += red[0][lane];
    acc += red[1][lane];
    acc += red[2][lane];
    const int64_t col = n0 + i;
    if (col < p.N) {
      const float sw = p.ws[col];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 4 * (lane >> 4) + v;
        if (row < p.M) p.y[row * p.ldy + col] = (p.xs[row] * sw) * (float)(acc[v] >> 8);
      }
    }
  }
}

hipError_t gemm_prepare_device() {
  // The tiled kernel uses more than 64 KiB of LDS per workgroup (gfx950 has 160 KiB).
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_tile_kernel<false>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_tile_kernel<true>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
}

hipError_t launch_gemm(const GemmParams& p, int mode, hipStream_t st) {
  if (p.M == 0) return hipSuccess;
  if (mode == kModeSym && p.M <= 16) {
    const int64_t grid = (p.N + 15) / 16;
    hipLaunchKernelGGL(gemm_decode_kernel, dim3((uint32_t)grid), dim3(256), 0, st, p);
    return hipGetLastError();
  }
  const int64_t grid = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  if (mode == kModeSym)
    hipLaunchKernelGGL(gemm_tile_kernel<false>, dim3((uint32_t)grid), dim3(256), kGemmLds, st, p);
  else
    hipLaunchKernelGGL(gemm_tile_kernel<true>, dim3((uint32_t)grid), dim3(256), kGemmLds, st, p);
  return hipGetLastError();
}

}  // namespace w4a4
