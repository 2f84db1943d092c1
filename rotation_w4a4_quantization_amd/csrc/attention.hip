// Single-query (decode) attention over a KV cache stored as rotated
// asymmetric INT4, one head vector of 128 per group.
//
// The KV step stored k Q and v Q with Q = diag(d) H_128 / sqrt(128) (d = 1
// without signs).  Q is orthogonal, so q . k = (q Q) . (k Q): the scores are
// taken between the rotated query and the dequantized rotated keys, the
// softmax-weighted sum of the dequantized rotated values is formed in the
// rotated domain, and the output is rotated back once, o = o_rot Q^T
// ("QuaRot (rotation-based outlier removal, W4A4KV4)", field "Activation
// scheme": the KV cache and parts of the attention computation are rotated;
// "Rotations for 4-Bit Activations: QuaRot, SpinQuant, and Friends",
// section "A rotation changes nothing, and that is the point").
//
// One workgroup of 8 waves per (batch, head).  Wave w takes a contiguous
// slice of the S tokens; inside a wave, lane group g = lane / 4 takes one
// token per step and lane j = lane % 4 of the group holds dimensions
// 32 j .. 32 j + 31 (16 bytes of codes).  The kernel is VALU-bound, so the
// per-token bookkeeping is shared by as few lanes as registers allow (4),
// and a lane group's running output is rescaled only when a score exceeds
// its reference maximum by more than 2^8.
// Dequantized values are s (u - z); the zero-point parts are factored out:
//   score  = scale * s_k * (sum_d q_d u_d - z_k * sum_d q_d)
//   o_rot  = sum_t p_t s_v,t u_t  -  (sum_t p_t s_v,t z_v,t) * 1
// The key dot products run on integer dot instructions: the rotated query
// is held in fixed point, q_d ~ sq * qi_d with |qi_d| <= 2^19 - 1 (sq =
// max|q| / (2^19 - 1), 20 significant bits, a relative error of at most
// 2^-20 of max|q| per element), and qi_d + 2^19 is split into five 4-bit
// digit planes, so sum_d qi_d u_d = sum_b 16^b udot8(plane_b, codes) -
// 2^19 sum_d u_d exactly in int32: 24 v_dot8_u32_u4 per token and lane
// instead of 32 nibble conversions and 32 fmas.
// Every lane group keeps its own online-softmax state (running max, sum,
// 32 output dims per lane); the groups of a wave are merged with xor
// shuffles, the waves through LDS.
//
// Split path (few heads, long caches): one workgroup per (batch, head, token
// range); each writes its merged state (the unnormalized rotated output
// sum, the running maximum and sum) to a partial-state buffer, and a second
// kernel merges a head's ranges (the same online-softmax merge), normalizes
// and rotates back.  This is the textbook split of the softmax sum; only the
// fp32 summation order differs from the single pass.
#include "common.h"
#include "kernels.h"

namespace w4a4 {
namespace {

constexpr int kAttnWaves = 8;
constexpr int kAttnThreads = kAttnWaves * 64;
constexpr float kNegBig = -3.0e38f;              // below every finite score, exp2 of the gap is 0
constexpr float kQiMax = 524287.0f;              // 2^19 - 1: largest fixed-point query magnitude
constexpr int kQiOff = 524288;                   // 2^19: makes the fixed-point query non-negative
constexpr float kSlack = 8.0f;                   // log2 units a score may exceed the reference maximum

// sum over the 4 lanes of a lane group (DPP quad swaps)
__device__ __forceinline__ float group4_sum(float v) {
  v += dpp_f<0xB1>(v);      // quad_perm [1,0,3,2]
  return v + dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
}

// x & m, opaque to the optimizer: it then cannot narrow the byte fields
// below to 4-bit extracts and converts each byte in place
// (v_cvt_f32_ubyte0..3, one instruction per value instead of two).
__device__ __forceinline__ uint32_t and_opaque(uint32_t x, uint32_t m) {
  uint32_t r;
  asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(m));
  return r;
}

// 32 unsigned nibbles (four dwords, dimension order) -> floats
__device__ __forceinline__ void nibbles32(const uint4& w, float* u) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const uint32_t lo = and_opaque(ws[h], 0x0F0F0F0Fu), hi = and_opaque(ws[h] >> 4, 0x0F0F0F0Fu);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      u[8 * h + 2 * b] = (float)((lo >> (8 * b)) & 0xFFu);
      u[8 * h + 2 * b + 1] = (float)((hi >> (8 * b)) & 0xFFu);
    }
  }
}

// Normalized 128-point Hadamard of the 128 values held two per lane by one
// wave (lane l: element l in a, element l + 64 in b); butterflies over lane
// bits with xor shuffles, the top bit inside the lane.
__device__ __forceinline__ void fwht128_wave(float& a, float& b) {
  const int lane = __lane_id();
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const float pa = shfl_xor_f(a, s), pb = shfl_xor_f(b, s);
    const bool hi = lane & s;
    a = hi ? pa - a : a + pa;
    b = hi ? pb - b : b + pb;
  }
  const float t = a;
  a = t + b;
  b = t - b;
  const float r = 0.08838834764831845f;          // 1 / sqrt(128), rounded to fp32
  a *= r;
  b *= r;
}

template <bool SPLIT>
__global__ void __launch_bounds__(kAttnThreads) kv4_attention_kernel(AttnParams p) {
  __shared__ int q_off[128];                     // fixed-point query + 2^19
  __shared__ uint32_t q_planes[5][16];           // digit b of dims 8 c .. 8 c + 7
  __shared__ float part_m[kAttnWaves], part_l[kAttnWaves];
  __shared__ float part_o[kAttnWaves][128];
  __shared__ float q_sq_sh, q_isum_sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 2, j = lane & 3;
  const int64_t bh = SPLIT ? blockIdx.x / p.nsplit : blockIdx.x;
  const int split = SPLIT ? (int)(blockIdx.x - bh * p.nsplit) : 0;

  // ---- rotate the query: q_rot = (q * d) H / sqrt(128)
  if (wave == 0) {
    const uint16_t* qp = p.q + bh * 128;
    uint32_t qa = qp[lane], qb = qp[lane + 64];
    if (p.signs) {
      qa ^= p.signs[lane] & 0x8000u;
      qb ^= p.signs[lane + 64] & 0x8000u;
    }
    float a = h2f(qa), b = h2f(qb);
    fwht128_wave(a, b);
    // fixed point: qi = rne(q / sq), sq = max|q| / (2^19 - 1)
    float amax = fmaxf(fabsf(a), fabsf(b));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, shfl_xor_f(amax, m));
    const float inv = amax > 0.0f ? kQiMax / amax : 0.0f;
    const int ia = (int)rintf(a * inv), ib = (int)rintf(b * inv);
    q_off[lane] = ia + kQiOff;
    q_off[lane + 64] = ib + kQiOff;
    int isum = ia + ib;                           // |sum over the head| < 2^26: int32 exact
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) isum += __builtin_amdgcn_ds_bpermute((lane ^ m) << 2, isum);
    if (lane == 0) {
      q_sq_sh = amax > 0.0f ? amax / kQiMax : 0.0f;
      q_isum_sh = (float)isum;
    }
  }
  __syncthreads();
  if (tid < 80) {                                // 5 digit planes x 16 dwords of 8 dims
    const int b = tid >> 4, c = tid & 15;
    uint32_t w = 0;
#pragma unroll
    for (int n = 0; n < 8; ++n) w |= (((uint32_t)q_off[8 * c + n] >> (4 * b)) & 15u) << (4 * n);
    q_planes[b][c] = w;
  }
  __syncthreads();
  uint32_t dq[5][4];                             // this lane's digit planes (dims 32 j ..)
#pragma unroll
  for (int b = 0; b < 5; ++b)
#pragma unroll
    for (int k = 0; k < 4; ++k) dq[b][k] = q_planes[b][4 * j + k];
  const float sq = q_sq_sh;
  const float q_isum = q_isum_sh;               // sum_d qi_d (float; |.| < 2^26)

  // ---- this wave's token slice of the workgroup's range (the whole cache
  // in the single pass)
  const int64_t S = p.S;
  const int64_t per_split = SPLIT ? (S + p.nsplit - 1) / p.nsplit : S;
  const int64_t r_begin = split * per_split;
  const int64_t r_end = r_begin + per_split < S ? r_begin + per_split : S;
  const int64_t per_wave = (r_end - r_begin + kAttnWaves - 1) / kAttnWaves;
  const int64_t t_begin = r_begin + wave * per_wave;
  const int64_t t_end = t_begin + per_wave < r_end ? t_begin + per_wave : r_end;

  const int64_t head = bh * S;                   // first token row of this head
  const int64_t code_bytes = S * 64;
  const __amdgpu_buffer_rsrc_t rkc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.k_codes + head * 64), (short)0, (int)code_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rvc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.v_codes + head * 64), (short)0, (int)code_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rks = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.k_scales + head), (short)0, (int)(S * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rvs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.v_scales + head), (short)0, (int)(S * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rkz = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.k_zeros + head), (short)0, (int)S, 0x00020000);
  const __amdgpu_buffer_rsrc_t rvz = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.v_zeros + head), (short)0, (int)S, 0x00020000);

  float m = kNegBig, l = 0.0f, zc = 0.0f;        // running max (log2 units), sum, zero-point term
  float o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = 0.0f;

  // Token batches of U steps (16 tokens per step, one per lane group) are
  // software-pipelined: the loads of the next batch are issued before the
  // current batch is computed, so a batch's memory latency is hidden behind
  // the previous batch's arithmetic.  Loads past the slice read out of range
  // (zeros) and those tokens are masked.
  constexpr int U = 2;
  struct Batch {
    uint4 kc[U], vc[U];
    float ks[U], vs[U];
    uint32_t kz[U], vz[U];
  };
  auto load = [&](Batch& b, int64_t t0) {
#pragma unroll
    for (int s = 0; s < U; ++s) {
      const int64_t t = t0 + 16 * s + g;
      const bool in = t < t_end;
      const int tt = in ? (int)t : 0x7FFFFFF;      // past the slice: out of range -> 0
      const int cb = in ? (int)(t * 64 + 16 * j) : 0x7FFFFFF0;
      b.kc[s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rkc, cb, 0, 0));
      b.vc[s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rvc, cb, 0, 0));
      b.ks[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rks, 4 * tt, 0, 0));
      b.vs[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rvs, 4 * tt, 0, 0));
      b.kz[s] = __builtin_amdgcn_raw_buffer_load_b8(rkz, tt, 0, 0);
      b.vz[s] = __builtin_amdgcn_raw_buffer_load_b8(rvz, tt, 0, 0);
    }
  };
  auto compute = [&](const Batch& b, int64_t t0) {
#pragma unroll
    for (int s = 0; s < U; ++s) {
      const bool ok = t0 + 16 * s + g < t_end;
      // sum_d qi_d u_d over this lane's 32 dims, exactly: digit-plane dot
      // products (each <= 32 * 15 * 15) recombined in int32 (< 2^29)
      const uint32_t kw[4] = {b.kc[s].x, b.kc[s].y, b.kc[s].z, b.kc[s].w};
      uint32_t acc[5] = {0u, 0u, 0u, 0u, 0u}, usum = 0u;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int d = 0; d < 5; ++d) acc[d] = __builtin_amdgcn_udot8(dq[d][k], kw[k], acc[d], false);
        usum = __builtin_amdgcn_udot8(0x11111111u, kw[k], usum, false);
      }
      const uint32_t comb = acc[0] + (acc[1] << 4) + (acc[2] << 8) + (acc[3] << 12) + (acc[4] << 16);
      const int part = (int)(comb - (usum << 19));
      const float dot = group4_sum((float)part);
      // score in log2 units: scale2 = softmax_scale * log2(e)
      const float sc = p.scale2 * sq * b.ks[s] * (dot - (float)b.kz[s] * q_isum);
      // the reference maximum m moves only when a score exceeds it by more
      // than kSlack (weights 2^(sc - m) stay <= 2^kSlack, far from fp32
      // overflow, and the result is scale-invariant): a lane group's 32
      // sums are then rescaled a few times per head rather than at almost
      // every step, and the branch is skipped when no lane of the wave
      // needs it
      const bool grow = ok && sc > m + kSlack;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float corr = grow ? exp2f(m - sc) : 1.0f;
        m = grow ? sc : m;
        l *= corr;
        zc *= corr;
#pragma unroll
        for (int i = 0; i < 32; ++i) o[i] *= corr;
      }
      const float pt = ok ? exp2f(sc - m) : 0.0f;
      l += pt;
      const float w = pt * b.vs[s];
      zc = fmaf(w, (float)b.vz[s], zc);
      float u[32];
      nibbles32(b.vc[s], u);
#pragma unroll
      for (int i = 0; i < 32; ++i) o[i] = fmaf(w, u[i], o[i]);
    }
  };
  constexpr int64_t kBatch = 16 * U;
  Batch ba, bb;
  load(ba, t_begin);
  for (int64_t t0 = t_begin; t0 < t_end; t0 += 2 * kBatch) {
    load(bb, t0 + kBatch);
    compute(ba, t0);
    if (t0 + kBatch >= t_end) break;             // uniform over the wave
    load(ba, t0 + 2 * kBatch);
    compute(bb, t0 + kBatch);
  }

  // ---- merge the 16 lane groups of the wave (xor partners 4, 8, 16, 32)
#pragma unroll
  for (int x = 4; x < 64; x <<= 1) {
    const float mp = shfl_xor_f(m, x), lp = shfl_xor_f(l, x), zp = shfl_xor_f(zc, x);
    const float mm = fmaxf(m, mp);
    const float f = exp2f(m - mm), fp = exp2f(mp - mm);
    m = mm;
    l = l * f + lp * fp;
    zc = zc * f + zp * fp;
#pragma unroll
    for (int i = 0; i < 32; ++i) o[i] = o[i] * f + shfl_xor_f(o[i], x) * fp;
  }
  // every group now holds the wave's merged state; group 0 publishes it
  if (g == 0) {
#pragma unroll
    for (int i = 0; i < 32; ++i) part_o[wave][32 * j + i] = o[i] - zc;
    if (j == 0) {
      part_m[wave] = m;
      part_l[wave] = l;
    }
  }
  __syncthreads();
  // ---- merge the waves: o_rot = sum_w 2^(m_w - M) o_w / sum_w 2^(m_w - M) l_w
  if (wave == 0) {
    float M = kNegBig;
#pragma unroll
    for (int k = 0; k < kAttnWaves; ++k) M = fmaxf(M, part_m[k]);
    float L = 0.0f, a = 0.0f, b = 0.0f;
#pragma unroll
    for (int k = 0; k < kAttnWaves; ++k) {
      const float f = exp2f(part_m[k] - M);
      L = fmaf(part_l[k], f, L);
      a = fmaf(part_o[k][lane], f, a);
      b = fmaf(part_o[k][lane + 64], f, b);
    }
    if constexpr (SPLIT) {
      // this range's state, unnormalized; an empty range leaves M = kNegBig
      // and L = 0, which the merge weighs by 0
      float* st = p.part + (bh * p.nsplit + split) * kAttnPartFloats;
      st[lane] = a;
      st[lane + 64] = b;
      if (lane == 0) {
        st[128] = M;
        st[129] = L;
      }
      return;
    }
    const float inv = 1.0f / L;
    a *= inv;
    b *= inv;
    // back to the original basis: o = o_rot H diag(d) / sqrt(128)
    fwht128_wave(a, b);
    if (p.signs) {
      if (p.signs[lane] & 0x8000u) a = -a;
      if (p.signs[lane + 64] & 0x8000u) b = -b;
    }
    float* op = p.out + bh * 128;
    op[lane] = a;
    op[lane + 64] = b;
  }
}

// Split path, second kernel: one workgroup per (batch, head) merges the
// nsplit (<= 64) partial states o_k, m_k, l_k (m in log2 units):
//   o_rot = sum_k 2^(m_k - M) o_k / sum_k 2^(m_k - M) l_k,  M = max_k m_k,
// then rotates back and applies the signs, as the single pass does.  The
// states are first copied to LDS with independent loads (one memory round
// trip), then one wave combines them.
constexpr int kMaxSplits = 64;
__global__ void __launch_bounds__(256) kv4_attention_merge_kernel(AttnParams p) {
  __shared__ float4 sts[kMaxSplits * kAttnPartFloats / 4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t bh = blockIdx.x;
  const int ns = p.nsplit;
  const float4* src = reinterpret_cast<const float4*>(p.part + bh * ns * kAttnPartFloats);
  const int n4 = ns * (kAttnPartFloats / 4);
  for (int i = tid; i < n4; i += 256) sts[i] = src[i];
  __syncthreads();
  if (tid >= 64) return;
  const float* st = reinterpret_cast<const float*>(sts);
  const float mk = lane < ns ? st[lane * kAttnPartFloats + 128] : kNegBig;
  float M = mk;
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) M = fmaxf(M, shfl_xor_f(M, x));
  const float f = lane < ns ? exp2f(mk - M) : 0.0f;
  float L = lane < ns ? st[lane * kAttnPartFloats + 129] * f : 0.0f;
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) L += shfl_xor_f(L, x);
  float a = 0.0f, b = 0.0f;
  for (int k = 0; k < ns; ++k) {
    const float fk = bitsf((uint32_t)__builtin_amdgcn_readlane((int)fbits(f), k));
    a = fmaf(st[k * kAttnPartFloats + lane], fk, a);
    b = fmaf(st[k * kAttnPartFloats + lane + 64], fk, b);
  }
  const float inv = 1.0f / L;
  a *= inv;
  b *= inv;
  fwht128_wave(a, b);
  if (p.signs) {
    if (p.signs[lane] & 0x8000u) a = -a;
    if (p.signs[lane + 64] & 0x8000u) b = -b;
  }
  float* op = p.out + bh * 128;
  op[lane] = a;
  op[lane + 64] = b;
}

}  // namespace

hipError_t launch_kv4_attention(const AttnParams& p, hipStream_t st) {
  if (p.BH == 0) return hipSuccess;
  W4A4_LAUNCH(kv4_attention_kernel<false>, dim3((uint32_t)p.BH), dim3(kAttnThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_kv4_attention_split(const AttnParams& p, hipStream_t st) {
  if (p.BH == 0) return hipSuccess;
  if (p.nsplit <= 1) return launch_kv4_attention(p, st);
  if (p.nsplit > kMaxSplits) return hipErrorInvalidValue;
  const LaunchTiming t = take_launch_timing();
  W4A4_LAUNCH_FIRST(t, kv4_attention_kernel<true>, dim3((uint32_t)(p.BH * p.nsplit)), dim3(kAttnThreads), 0, st, p);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  W4A4_LAUNCH_LAST(t, kv4_attention_merge_kernel, dim3((uint32_t)p.BH), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace w4a4
