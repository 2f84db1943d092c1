// Fused fast Walsh-Hadamard transform + INT4 quantization + nibble packing.
//
// One kernel serves the online activation step, the offline weight step and
// the KV-cache step:
//   Page "Rotations for 4-Bit Activations: QuaRot, SpinQuant, and Friends",
//   section "Where the rotations go": a rotation that cannot be folded into
//   the weights costs one fast Hadamard transform per token, so it is fused
//   with the quantization of the activations; section "What it buys in 4
//   bits": one INT4 scale per token (per output channel for weights).
//   Page "SpinQuant (learned rotations + W4A4KV4)", field "Activation
//   scheme": per-group asymmetric INT4 for activations and the KV cache.
//
// Data layout in registers.  A 128-element Hadamard block of a row is held by
// a quad of 4 lanes; lane q of the quad loads the four 16-byte chunks
// q, q+4, q+8, q+12 of the block, so element k = 32r + 8q + e (r, e: register
// coordinates) sits in register 8r + e of lane q.  The transform is the
// tensor product of 2x2 butterflies over the 7 index bits, and butterflies on
// different bits commute, so the 5 bits held in registers (e: bits 0-2,
// r: bits 5-6) are done in registers and the 2 lane bits (q: bits 3-4) with
// DPP quad permutes.  A full-width transform (block = K) continues over the
// block index through LDS.  The row's absmax (symmetric) or each block's
// min/max (asymmetric) is reduced across lanes, then every value is turned
// into a code with one fma against a magic constant (round to nearest even
// of the exact product z * inv) and 8 codes are packed per dword.
#include "common.h"
#include "kernels.h"
#include "rq_block.h"

namespace w4a4 {

namespace {

template <int LOG_N>
__device__ __forceinline__ void fwht_regs(float* v) {
  // In-register butterflies over bits 0..LOG_N-1 of the array index.
#pragma unroll
  for (int b = 1; b < (1 << LOG_N); b <<= 1) {
#pragma unroll
    for (int i = 0; i < (1 << LOG_N); ++i) {
      if (!(i & b)) {
        const float a = v[i], c = v[i | b];
        v[i] = a + c;
        v[i | b] = a - c;
      }
    }
  }
}

// Remaining butterflies of a full-width transform: FWHT over the block index
// (nb = 2^LOG_NB blocks of 128) of one row held in LDS as [nb][128] floats.
// T = 4 nb threads of the row slot take part; every pass reads, transforms
// and writes back 32 values per thread.
template <int LOG_NB>
__device__ __forceinline__ void fwht_block_axis(float* buf, int lt) {
  constexpr int NB = 1 << LOG_NB;
  constexpr int T = 4 * NB;
  constexpr int LA = LOG_NB < 5 ? LOG_NB : 5;         // pass A: block bits 0..LA-1
  constexpr int NA = 1 << LA;
  float v[32];
#pragma unroll
  for (int j = 0; j < 32 / NA; ++j) {
    const int it = lt + T * j;
    const int c = it & 127, grp = it >> 7;
#pragma unroll
    for (int t = 0; t < NA; ++t) v[j * NA + t] = buf[(grp * NA + t) * 128 + c];
  }
#pragma unroll
  for (int j = 0; j < 32 / NA; ++j) fwht_regs<LA>(v + j * NA);
#pragma unroll
  for (int j = 0; j < 32 / NA; ++j) {
    const int it = lt + T * j;
    const int c = it & 127, grp = it >> 7;
#pragma unroll
    for (int t = 0; t < NA; ++t) buf[(grp * NA + t) * 128 + c] = v[j * NA + t];
  }
  if constexpr (LOG_NB > 5) {
    constexpr int LB = LOG_NB - 5;                    // pass B: block bits 5..LOG_NB-1
    constexpr int NBB = 1 << LB;
    constexpr int ITEMS = 4096 / T;                   // (128 columns x 32 low block indices) / T
    __syncthreads();
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const int it = lt + T * j;
      const int c = it & 127, lo = it >> 7;
#pragma unroll
      for (int t = 0; t < NBB; ++t) v[j * NBB + t] = buf[(lo + 32 * t) * 128 + c];
    }
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) fwht_regs<LB>(v + j * NBB);
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const int it = lt + T * j;
      const int c = it & 127, lo = it >> 7;
#pragma unroll
      for (int t = 0; t < NBB; ++t) buf[(lo + 32 * t) * 128 + c] = v[j * NBB + t];
    }
  }
}

// 4x4 transpose of dwords inside a quad: on entry lane q holds w[r] = W[q][r],
// on exit w[r] = W[r][q].  A lane's four code words of a 128-block sit at
// byte offsets 16 r + 4 q of the block's 64 code bytes; after the transpose
// lane q holds bytes 16 q .. 16 q + 15, so one 16-byte store per lane writes
// the wave's 16 blocks as 1 KiB of contiguous codes (instead of four 4-byte
// stores per lane, each covering 16-byte pieces 64 bytes apart).
__device__ __forceinline__ void quad_transpose_u32(uint32_t (&w)[4], int q) {
  {
    const bool hi = q & 1;
    const uint32_t s0 = hi ? w[0] : w[1], s1 = hi ? w[2] : w[3];
    const uint32_t r0 = (uint32_t)dpp_i<0xB1>((int)s0), r1 = (uint32_t)dpp_i<0xB1>((int)s1);
    const uint32_t a0 = hi ? r0 : w[0], a1 = hi ? w[1] : r0;
    const uint32_t a2 = hi ? r1 : w[2], a3 = hi ? w[3] : r1;
    w[0] = a0; w[1] = a1; w[2] = a2; w[3] = a3;
  }
  {
    const bool hi = q & 2;
    const uint32_t s0 = hi ? w[0] : w[2], s1 = hi ? w[1] : w[3];
    const uint32_t r0 = (uint32_t)dpp_i<0x4E>((int)s0), r1 = (uint32_t)dpp_i<0x4E>((int)s1);
    const uint32_t a0 = hi ? r0 : w[0], a2 = hi ? w[2] : r0;
    const uint32_t a1 = hi ? r1 : w[1], a3 = hi ? w[3] : r1;
    w[0] = a0; w[1] = a1; w[2] = a2; w[3] = a3;
  }
}

}  // namespace

template <int MODE, int LOG_NB_FULL, bool GSUM, bool STRIDED, bool SIGNS>
__global__ void __launch_bounds__(512) rotate_quant_kernel(RQParams p) {
  extern __shared__ float lds[];
  const int tid = threadIdx.x;
  const int slot = p.rows_per_wg == 1 ? 0 : tid >> p.log2seg;
  const int lt = tid - slot * p.seg;
  const int blk = lt >> 2;
  const int q = lt & 3;
  const bool lane_ok = blk < p.nb;
  // cross-lane butterfly coefficients and the sign they leave on this lane
  const float s0 = (q & 1) ? -1.0f : 1.0f;
  const float s1 = (q & 2) ? -1.0f : 1.0f;
  const float sgn = ((q ^ (q >> 1)) & 1) ? -1.0f : 1.0f;
  // byte offset of this lane's first chunk inside its row group (dense rows);
  // padding lanes read past the buffer's end and get zeros
  const uint32_t lane_off = lane_ok ? (uint32_t)(((int64_t)slot * p.ss + blk * 128 + q * 8) * 2) : 0x7FFFFFF0u;
  const int64_t ngroups = (p.rows + p.rows_per_wg - 1) / p.rows_per_wg;

  // randomized Hadamard: the diagonal D depends on the column only, so each
  // lane loads the sign bits of its 32 columns once and flips its inputs'
  // signs (one XOR per pair of fp16 values) before the transform.  A
  // separate instantiation, so the plain rotation keeps its registers.
  uint4 sg[4] = {};
  if constexpr (SIGNS) {
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
        (void*)p.signs, (short)0, p.K * 2, 0x00020000);
    const uint32_t soff = lane_ok ? (uint32_t)((blk * 128 + q * 8) * 2) : 0x7FFFFFF0u;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const uint4 d = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rd, (int)soff, 64 * r4, 0));
      sg[r4] = make_uint4(d.x & 0x80008000u, d.y & 0x80008000u, d.z & 0x80008000u, d.w & 0x80008000u);
    }
  }

  for (int64_t rgi = blockIdx.x; rgi < ngroups; rgi += gridDim.x) {
    const int64_t row0 = rgi * p.rows_per_wg;
    const int64_t row = row0 + slot;
    const bool valid = lane_ok && row < p.rows;

    // ---- load 32 fp16 values (chunks q, q+4, q+8, q+12 of block `blk`)
    uint4 w[4];
    if constexpr (STRIDED) {
      const uint32_t r = (uint32_t)row;
      const uint32_t s = r % p.S, t = r / p.S;
      const uint32_t h = t % p.H, b = t / p.H;
      const uint16_t* src = p.x + (int64_t)b * p.sb + (int64_t)h * p.sh + (int64_t)s * p.ss + blk * 128 + q * 8;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        w[r4] = valid ? *reinterpret_cast<const uint4*>(src + 32 * r4) : make_uint4(0u, 0u, 0u, 0u);
    } else {
      const int64_t nrows = p.rows - row0 < p.rows_per_wg ? p.rows - row0 : p.rows_per_wg;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.x + row0 * p.ss), (short)0, (int)(nrows * p.ss * 2), 0x00020000);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        w[r4] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)lane_off, 64 * r4, 0));
    }

    if constexpr (SIGNS) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        w[r4].x ^= sg[r4].x;
        w[r4].y ^= sg[r4].y;
        w[r4].z ^= sg[r4].z;
        w[r4].w ^= sg[r4].w;
      }
    }

    // 128-point transform of the block: afterwards this lane holds sgn * z
    float v[32];
    fwht128_quad(w, v, s0, s1);

    // ---- full width: butterflies over the block index through LDS.  Values
    // at one in-block position share their sign, so the signed values
    // transform linearly and keep it.
    if constexpr (LOG_NB_FULL > 0) {
      float* buf = lds + (size_t)slot * p.K;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float4* dst = reinterpret_cast<float4*>(buf + blk * 128 + 32 * r4 + 8 * q);
        dst[0] = make_float4(v[8 * r4 + 0], v[8 * r4 + 1], v[8 * r4 + 2], v[8 * r4 + 3]);
        dst[1] = make_float4(v[8 * r4 + 4], v[8 * r4 + 5], v[8 * r4 + 6], v[8 * r4 + 7]);
      }
      __syncthreads();
      fwht_block_axis<LOG_NB_FULL>(buf, lt);
      __syncthreads();
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4* s4 = reinterpret_cast<const float4*>(buf + blk * 128 + 32 * r4 + 8 * q);
        const float4 a = s4[0], b = s4[1];
        v[8 * r4 + 0] = a.x; v[8 * r4 + 1] = a.y; v[8 * r4 + 2] = a.z; v[8 * r4 + 3] = a.w;
        v[8 * r4 + 4] = b.x; v[8 * r4 + 5] = b.y; v[8 * r4 + 6] = b.z; v[8 * r4 + 7] = b.w;
      }
      __syncthreads();   // the row buffer is reused for the reduction below
    }

    const int64_t crow = row * (int64_t)(p.K / 2);
    uint32_t words[4];

    if constexpr (MODE == kModeSym) {
      // ---- per-row absmax
      float am = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(v[i]));
      am = quad_max(am);
      if (p.seg <= kWave) {
        for (int m = 4; m < p.seg; m <<= 1) am = fmaxf(am, shfl_xor_f(am, m));
      } else {
        for (int m = 4; m < kWave; m <<= 1) am = fmaxf(am, shfl_xor_f(am, m));
        float* red = lds;
        const int nw = p.seg / kWave;
        if ((lt & (kWave - 1)) == 0) red[slot * 16 + (lt / kWave)] = am;
        __syncthreads();
        am = 0.0f;
        for (int w2 = 0; w2 < nw; ++w2) am = fmaxf(am, red[slot * 16 + w2]);
        __syncthreads();   // red is rewritten by the next row group
      }
      const float inv = am > 0.0f ? div_rn(7.0f, am) : 0.0f;
      const float sinv = sgn * inv;      // (sgn z) * (sgn inv) = z * inv exactly
      // codes: fma gives 2^23*1.5 + 8 + rne(z*inv); the low nibble is the code
      // in offset-8 binary, turned into two's complement by the final xor.
      uint32_t gsb = 0;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) words[r4] = sym_word(v + 8 * r4, sinv, gsb);
      quad_transpose_u32(words, q);
      if (valid) {
        *reinterpret_cast<uint4*>(p.codes + crow + blk * 64 + 16 * q) = make_uint4(words[0], words[1], words[2], words[3]);
        if (lt == 0) p.scales[row] = am > 0.0f ? div_rn(am, p.cdiv) : 0.0f;
      }
      if constexpr (GSUM) {
        // sum of the 32 codes: the bit patterns are magic + 8 + code
        const int gs = quad_sum((int)(gsb - 32u * (kRneMagicBits + 8u)));
        if (valid && q == 0) p.gsum[row * p.nb + blk] = gs;
      }
    } else if constexpr (MODE == kModeMx) {
      // ---- MXFP4: blocks of 32 (elements 32 r4 .. 32 r4 + 31 of this 128-block,
      // 8 in each lane of the quad), y = fl32(z / sqrt(b)), a power-of-two
      // scale 2^e with e = floor(log2 max|y|) - 2 (stored biased, e + 127,
      // at least 0), E2M1 codes rounded to nearest with ties to the even code
      // and saturation at 6.  v_cvt_scalef32_pk_fp4_f32 converts y / 2^e with
      // exactly that rounding (checked against the oracle's rounding on every
      // multiple of 1/64 in [-9, 9] and on scaled random values); it returns
      // -0 (code 8) for a negative value that rounds to zero, which this
      // format does not use, so those sign bits are cleared afterwards.
      const float sr = sgn * p.cdiv;     // (sgn z) * (sgn r) = z * r, one rounding
      uint32_t sbytes = 0;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float y[8];
        float am = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          y[e] = v[8 * r4 + e] * sr;
          am = fmaxf(am, fabsf(y[e]));
        }
        am = quad_max(am);
        const uint32_t ex = (fbits(am) >> 23) & 0xFFu;
        const uint32_t byte = ex > 2u ? ex - 2u : 0u;        // e + 127, clamped at e = -127
        // 2^e as an fp32; byte 0 only occurs for an all-zero block (fp16 inputs
        // give |y| >= 2^-32 when y != 0), where 2^-126 gives the same zero codes
        const float scale = bitsf((byte > 0u ? byte : 1u) << 23);
        uint32_t w = 0;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], scale, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], scale, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], scale, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], scale, 3);
        // per nibble: magnitude + 7 sets bit 3 iff the magnitude is non-zero
        // (at most 14, so no carry crosses a nibble); keep the sign only there
        const uint32_t nonzero = ((w & 0x77777777u) + 0x77777777u) & 0x88888888u;
        words[r4] = w & (nonzero | 0x77777777u);
        sbytes |= byte << (8 * r4);
      }
      quad_transpose_u32(words, q);
      if (valid) {
        *reinterpret_cast<uint4*>(p.codes + crow + blk * 64 + 16 * q) = make_uint4(words[0], words[1], words[2], words[3]);
        if (q == 0)
          *reinterpret_cast<uint32_t*>(p.mx_scales + row * (int64_t)(p.K / 32) + blk * 4) = sbytes;
      }
    } else {
      // ---- asymmetric, one group per 128-block
      float mn = 0.0f, mx = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        mn = fminf(mn, v[i]);
        mx = fmaxf(mx, v[i]);
      }
      // this lane holds sgn * z: the range of z is [mn, mx] or [-mx, -mn]
      float lo = sgn > 0.0f ? mn : -mx;
      float hi = sgn > 0.0f ? mx : -mn;
      lo = quad_min(lo);
      hi = quad_max(hi);
      const float rg = hi - lo;
      const float inv = rg > 0.0f ? div_rn(15.0f, rg) : 0.0f;
      const float sinv = sgn * inv;
      int zp = (int)(fbits(fmaf(-lo, inv, kRneMagic)) - kRneMagicBits);
      zp = zp < 0 ? 0 : (zp > 15 ? 15 : zp);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        uint32_t b[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t u = fbits(fmaf(v[8 * r4 + e], sinv, kRneMagic)) + (uint32_t)zp;
          b[e] = u < kRneMagicBits + 15u ? u : kRneMagicBits + 15u;
        }
        words[r4] = pack8(b);
      }
      quad_transpose_u32(words, q);
      if (valid) {
        *reinterpret_cast<uint4*>(p.codes + crow + blk * 64 + 16 * q) = make_uint4(words[0], words[1], words[2], words[3]);
        if (q == 0) {
          p.scales[row * p.nb + blk] = rg > 0.0f ? div_rn(rg, p.cdiv) : 0.0f;
          p.zeros[row * p.nb + blk] = (uint8_t)zp;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ launch
namespace {

template <int MODE, int LOGF, bool GSUM, bool STRIDED>
hipError_t launch_t(const RQParams& p, int threads, size_t lds, int64_t grid, hipStream_t st) {
  if (p.signs)
    W4A4_LAUNCH((rotate_quant_kernel<MODE, LOGF, GSUM, STRIDED, true>), dim3((uint32_t)grid),
                dim3(threads), lds, st, p);
  else
    W4A4_LAUNCH((rotate_quant_kernel<MODE, LOGF, GSUM, STRIDED, false>), dim3((uint32_t)grid),
                dim3(threads), lds, st, p);
  return hipGetLastError();
}

template <int MODE, bool GSUM>
hipError_t launch_full(const RQParams& p, int logf, int threads, size_t lds, int64_t grid,
                       hipStream_t st) {
  switch (logf) {
    case 1: return launch_t<MODE, 1, GSUM, false>(p, threads, lds, grid, st);
    case 2: return launch_t<MODE, 2, GSUM, false>(p, threads, lds, grid, st);
    case 3: return launch_t<MODE, 3, GSUM, false>(p, threads, lds, grid, st);
    case 4: return launch_t<MODE, 4, GSUM, false>(p, threads, lds, grid, st);
    case 5: return launch_t<MODE, 5, GSUM, false>(p, threads, lds, grid, st);
    case 6: return launch_t<MODE, 6, GSUM, false>(p, threads, lds, grid, st);
    case 7: return launch_t<MODE, 7, GSUM, false>(p, threads, lds, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

RQGeometry rq_geometry(int64_t rows, int K) {
  RQGeometry g{};
  const int nb = K / 128;
  const int T = 4 * nb;
  if (T <= kWave) {
    int seg = 4;
    while (seg < T) seg <<= 1;
    g.seg = seg;
    g.rows_per_wg = 256 / seg;
  } else {
    g.seg = (T + kWave - 1) / kWave * kWave;
    g.rows_per_wg = g.seg >= 256 ? 1 : 256 / g.seg;
  }
  g.threads = g.seg * g.rows_per_wg;
  // one row group per workgroup: measured faster than a grid capped at a few
  // rounds of workgroups per CU that loop over row groups (KV 8x32x4096x128
  // cold: 59.0 vs 63.1 us; down_proj 4096x14336: 28.3 vs 30.0 us).  The
  // kernel keeps its grid-stride loop, so a grid at the 2^31 - 1 limit still
  // covers every row.
  const int64_t groups = (rows + g.rows_per_wg - 1) / g.rows_per_wg;
  const int64_t cap = 0x7FFFFFFF;
  g.grid = groups < cap ? groups : cap;
  return g;
}

hipError_t launch_rotate_quant(RQParams p, int mode, bool full, bool gsum, bool strided,
                               hipStream_t st) {
  const RQGeometry g = rq_geometry(p.rows, p.K);
  p.seg = g.seg;
  p.rows_per_wg = g.rows_per_wg;
  p.log2seg = 0;
  while ((1 << p.log2seg) < g.seg) ++p.log2seg;   // seg is a power of two whenever rows_per_wg > 1
  p.nb = p.K / 128;
  int logf = 0;
  if (full && p.nb > 1) {
    while ((1 << logf) < p.nb) ++logf;
  }
  size_t lds = 0;
  if (logf > 0) lds = (size_t)g.rows_per_wg * p.K * sizeof(float);
  else if (mode == kModeSym && g.seg > kWave) lds = (size_t)g.rows_per_wg * 16 * sizeof(float);
  if (g.grid == 0) return hipSuccess;
  if (mode == kModeMx) {
    if (strided || gsum) return hipErrorInvalidValue;
    if (logf > 0) return launch_full<kModeMx, false>(p, logf, g.threads, lds, g.grid, st);
    return launch_t<kModeMx, 0, false, false>(p, g.threads, lds, g.grid, st);
  }
  if (mode == kModeSym) {
    if (strided) return hipErrorInvalidValue;
    if (logf > 0) return gsum ? launch_full<kModeSym, true>(p, logf, g.threads, lds, g.grid, st)
                              : launch_full<kModeSym, false>(p, logf, g.threads, lds, g.grid, st);
    return gsum ? launch_t<kModeSym, 0, true, false>(p, g.threads, lds, g.grid, st)
                : launch_t<kModeSym, 0, false, false>(p, g.threads, lds, g.grid, st);
  }
  if (gsum || logf > 0) return hipErrorInvalidValue;
  return strided ? launch_t<kModeAsym, 0, false, true>(p, g.threads, lds, g.grid, st)
                 : launch_t<kModeAsym, 0, false, false>(p, g.threads, lds, g.grid, st);
}

}  // namespace w4a4
