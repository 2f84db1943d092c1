// Decode W4A4 linear in one launch: rotate + quantize the M <= 16 activation
// rows inside the weight-streaming GEMM.
//
// At decode sizes the activation step is a few kilobytes of work behind a
// whole launch and a round trip through HBM; the pages fuse the online
// rotation with the quantization ("Rotations for 4-Bit Activations: QuaRot,
// SpinQuant, and Friends", section "Where the rotations go"), and this kernel
// carries the same fusion one step further, into the product ("A rotation
// changes nothing, and that is the point": Y = (X Q)(W Q)^T).
//
// Every workgroup owns 16 output columns and needs every activation code, so
// each one transforms and quantizes all M rows itself (M * K values, a few
// microseconds of VALU at most) while the loads of its own 16 weight rows,
// issued first, are in flight.  The transform and the codes use the rotate
// kernel's own register code (rq_block.h) and its scale formulas, so codes,
// scales and outputs equal those of rotate_quant_act followed by w4a4_gemm
// bit for bit.
#include "common.h"
#include "kernels.h"
#include "rq_block.h"
#include "tile.h"

namespace w4a4 {
namespace {

constexpr int kFThreads = 1024;
constexpr int kFWaves = kFThreads / 64;
constexpr int kFMaxQuads = 512;                    // M * K / 128: two 128-blocks per thread
constexpr int kFCodeBytes = 32768 + 16 * 16;       // M * (K/2 + 16) for M * K <= 65536

}  // namespace

// S = 16-step rounds of the product per wave (K <= 2048 S=1, 4096 S=2, 8192 S=4);
// C = 128-blocks per thread in the activation step (1 or 2).
template <int S, int C>
__global__ void __launch_bounds__(kFThreads) gemm_decode_fused_kernel(FusedDecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t xq[kFCodeBytes];   // codes, row stride K/2 + 16
  __shared__ float blockmax[kFMaxQuads];
  __shared__ float rowinv[16], rowscale[16];
  __shared__ v4i red[kFWaves - 1][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int M = p.M, K = p.K;
  const int nb = K / 128, nkt = K / 128;
  const int ldc = K / 2;
  const int xld = ldc + 16;                         // padded LDS row: the 16 rows of a fragment read hit distinct banks
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t nw = p.N - n0 < 16 ? p.N - n0 : 16;

  // ---- 1. loads.  The activation chunks (and the sign words) are issued
  // first and the weight rows after them: vector-memory operations complete
  // in order, so the transform can wait for its inputs while the weight rows
  // are still in flight.  Thread t holds quad lanes t and t + 1024 (quad =
  // one 128-block of one row, 4 lanes of one wave).
  const int q = tid & 3;
  const float s0 = (q & 1) ? -1.0f : 1.0f;
  const float s1 = (q & 2) ? -1.0f : 1.0f;
  const float sgn = ((q ^ (q >> 1)) & 1) ? -1.0f : 1.0f;
  const int nquad = M * nb;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.x, (short)0, (int)(M * p.ldx * 2), 0x00020000);
  // without signs the range is empty: the loads return zeros and touch nothing
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.signs, (short)0, p.signs ? K * 2 : 0, 0x00020000);
  uint4 xw[C][4], sd[C][4];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int quad = (tid + kFThreads * c) >> 2;
    const bool ok = quad < nquad;
    const int row = ok ? quad / nb : 0, blk = ok ? quad - row * nb : 0;
    const int off = ok ? (row * p.ldx + blk * 128 + q * 8) * 2 : 0x7FFFFFF0;
    const int soff = (blk * 128 + q * 8) * 2;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      xw[c][r4] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 64 * r4, 0));
      sd[c][r4] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rd, soff, 64 * r4, 0));
    }
  }
  // this workgroup's 16 weight rows: wave w takes steps w, w + 16, ...; lane
  // (r, kg) 16 packed bytes of row n0 + r.  Consumed last.
  const int r = lane & 15, kg = 16 * (lane >> 4);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.wq + n0 * ldc), (short)0, (int)(nw * ldc), 0x00020000);
  uint4 wb[S];
#pragma unroll
  for (int u = 0; u < S; ++u) {
    const int kt = wave + kFWaves * u;
    const int off = kt < nkt ? r * ldc + kg + kt * 64 : 0x7FFFFFF0;
    wb[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0));
  }
  // all loads issued before the transform (left alone, the scheduler sinks
  // the second chunk's and the weights' loads below the first chunk's work)
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. rotate the M activation rows
  float v[C][32];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int quad = (tid + kFThreads * c) >> 2;
    const bool ok = quad < nquad;
    uint4 w[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      // randomized Hadamard: flip the sign bits of the columns whose d is negative
      w[r4] = xw[c][r4];
      w[r4].x ^= sd[c][r4].x & 0x80008000u;
      w[r4].y ^= sd[c][r4].y & 0x80008000u;
      w[r4].z ^= sd[c][r4].z & 0x80008000u;
      w[r4].w ^= sd[c][r4].w & 0x80008000u;
    }
    fwht128_quad(w, v[c], s0, s1);
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(v[c][i]));
    am = quad_max(am);
    if (ok && q == 0) blockmax[quad] = am;
  }
  __syncthreads();
  // per-row absmax: wave m reduces row m's block maxima
  if (wave < M) {
    float am = 0.0f;
    for (int b = lane; b < nb; b += 64) am = fmaxf(am, blockmax[wave * nb + b]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) am = fmaxf(am, shfl_xor_f(am, m));
    if (lane == 0) {
      rowinv[wave] = am > 0.0f ? div_rn(7.0f, am) : 0.0f;
      rowscale[wave] = am > 0.0f ? div_rn(am, p.cdiv) : 0.0f;
    }
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int quad = (tid + kFThreads * c) >> 2;
    if (quad < nquad) {
      const int row = quad / nb, blk = quad - row * nb;
      const float sinv = sgn * rowinv[row];
      uint32_t unused = 0;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<uint32_t*>(xq + row * xld + blk * 64 + 16 * r4 + 4 * q) =
            sym_word(v[c] + 8 * r4, sinv, unused);
    }
  }
  __syncthreads();

  // ---- 3. the product, as the decode GEMM: A fragments from LDS (rows >= M
  // read as zero), B from the weight registers; partial sums over K steps
  // meet through LDS
  v4i acc = v4i{0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < S; ++u) {
    const int kt = wave + kFWaves * u;
    if (kt < nkt) {
      const uint4 xa = r < M ? *reinterpret_cast<const uint4*>(xq + r * xld + kt * 64 + kg) : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t xw[4] = {xa.x, xa.y, xa.z, xa.w};
      const uint32_t ww[4] = {wb[u].x, wb[u].y, wb[u].z, wb[u].w};
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
  }
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w2 = 0; w2 < kFWaves - 1; ++w2) acc += red[w2][lane];
    const int64_t col = n0 + r;
    if (col < p.N) {
      const float sw = p.ws[col];
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) {
        const int row = 4 * (lane >> 4) + vv;
        if (row < M) p.y[row * p.ldy + col] = (rowscale[row] * sw) * (float)(acc[vv] >> 8);
      }
    }
  }
}

hipError_t launch_decode_fused(const FusedDecodeParams& p, hipStream_t st) {
  const int nkt = p.K / 128;
  const int S = (nkt + kFWaves - 1) / kFWaves;
  const int C = 4 * p.M * (p.K / 128) > kFThreads ? 2 : 1;
  const int64_t grid = (p.N + 15) / 16;
  if (p.M < 1 || p.M > 16 || p.K < 128 || p.K > 8192 || p.M * (p.K / 128) > kFMaxQuads)
    return hipErrorInvalidValue;
#define W4A4_FUSED(SS, CC) \
  if (S <= SS && C == CC) { W4A4_LAUNCH((gemm_decode_fused_kernel<SS, CC>), dim3((uint32_t)grid), dim3(kFThreads), 0, st, p); return hipGetLastError(); }
  W4A4_FUSED(1, 1)
  W4A4_FUSED(1, 2)
  W4A4_FUSED(2, 1)
  W4A4_FUSED(2, 2)
  W4A4_FUSED(4, 1)
  W4A4_FUSED(4, 2)
#undef W4A4_FUSED
  return hipErrorInvalidValue;
}

}  // namespace w4a4
