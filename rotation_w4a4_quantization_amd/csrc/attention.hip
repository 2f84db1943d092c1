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
// and the running output is rescaled only when the running maximum grows.
// Dequantized values are s (u - z); the zero-point parts are factored out:
//   score  = scale * s_k * (sum_d q_d u_d - z_k * sum_d q_d)
//   o_rot  = sum_t p_t s_v,t u_t  -  (sum_t p_t s_v,t z_v,t) * 1
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

// sum over the 4 lanes of a lane group (DPP quad swaps)
__device__ __forceinline__ float group4_sum(float v) {
  v += dpp_f<0xB1>(v);      // quad_perm [1,0,3,2]
  return v + dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
}

// 32 unsigned nibbles (four dwords, dimension order) -> floats
__device__ __forceinline__ void nibbles32(const uint4& w, float* u) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const uint32_t lo = ws[h] & 0x0F0F0F0Fu, hi = (ws[h] >> 4) & 0x0F0F0F0Fu;
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
  __shared__ float q_rot[128];
  __shared__ float part_m[kAttnWaves], part_l[kAttnWaves];
  __shared__ float part_o[kAttnWaves][128];
  __shared__ float q_sum_sh;

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
    q_rot[lane] = a;
    q_rot[lane + 64] = b;
    float s = a + b;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s += shfl_xor_f(s, m);
    if (lane == 0) q_sum_sh = s;
  }
  __syncthreads();
  float q[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) q[i] = q_rot[32 * j + i];
  const float q_sum = q_sum_sh;

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

  constexpr int U = 2;                           // token steps whose loads are in flight together
  for (int64_t t0 = t_begin; t0 < t_end; t0 += 16 * U) {
    uint4 kc[U], vc[U];
    float ks[U], vs[U];
    uint32_t kz[U], vz[U];
    bool ok[U];
#pragma unroll
    for (int s = 0; s < U; ++s) {
      const int64_t t = t0 + 16 * s + g;
      ok[s] = t < t_end;
      const int tt = ok[s] ? (int)t : 0x7FFFFFF;      // past the slice: out of range -> 0
      const int cb = ok[s] ? (int)(t * 64 + 16 * j) : 0x7FFFFFF0;
      kc[s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rkc, cb, 0, 0));
      vc[s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rvc, cb, 0, 0));
      ks[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rks, 4 * tt, 0, 0));
      vs[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rvs, 4 * tt, 0, 0));
      kz[s] = __builtin_amdgcn_raw_buffer_load_b8(rkz, tt, 0, 0);
      vz[s] = __builtin_amdgcn_raw_buffer_load_b8(rvz, tt, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < U; ++s) {
      float u[32];
      nibbles32(kc[s], u);
      float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; i += 2) {
        d0 = fmaf(q[i], u[i], d0);
        d1 = fmaf(q[i + 1], u[i + 1], d1);
      }
      const float dot = group4_sum(d0 + d1);
      // score in log2 units: scale2 = softmax_scale * log2(e)
      const float sc = p.scale2 * ks[s] * (dot - (float)kz[s] * q_sum);
      if (ok[s] && sc > m) {                     // the running maximum grows: rescale once
        const float corr = exp2f(m - sc);
        m = sc;
        l *= corr;
        zc *= corr;
#pragma unroll
        for (int i = 0; i < 32; ++i) o[i] *= corr;
      }
      const float pt = ok[s] ? exp2f(sc - m) : 0.0f;
      l += pt;
      const float w = pt * vs[s];
      zc = fmaf(w, (float)vz[s], zc);
      nibbles32(vc[s], u);
#pragma unroll
      for (int i = 0; i < 32; ++i) o[i] = fmaf(w, u[i], o[i]);
    }
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

// Split path, second kernel: one wave per (batch, head) merges the
// nsplit partial states o_k, m_k, l_k (m in log2 units):
//   o_rot = sum_k 2^(m_k - M) o_k / sum_k 2^(m_k - M) l_k,  M = max_k m_k,
// then rotates back and applies the signs, as the single pass does.
__global__ void __launch_bounds__(256) kv4_attention_merge_kernel(AttnParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= p.BH) return;                         // uniform over the wave
  const float* st = p.part + bh * p.nsplit * kAttnPartFloats;
  float M = kNegBig;
  for (int k = 0; k < p.nsplit; ++k) M = fmaxf(M, st[k * kAttnPartFloats + 128]);
  float L = 0.0f, a = 0.0f, b = 0.0f;
  for (int k = 0; k < p.nsplit; ++k) {
    const float* sk = st + k * kAttnPartFloats;
    const float f = exp2f(sk[128] - M);
    L = fmaf(sk[129], f, L);
    a = fmaf(sk[lane], f, a);
    b = fmaf(sk[lane + 64], f, b);
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
  const LaunchTiming t = take_launch_timing();
  W4A4_LAUNCH_FIRST(t, kv4_attention_kernel<true>, dim3((uint32_t)(p.BH * p.nsplit)), dim3(kAttnThreads), 0, st, p);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  W4A4_LAUNCH_LAST(t, kv4_attention_merge_kernel, dim3((uint32_t)((p.BH + 3) / 4)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace w4a4
