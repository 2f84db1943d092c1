// W4A4 GEMM on gfx950 int8 MFMA.
//
// The product of the rotated, quantized operands is an integer dot product
// of 4-bit codes ("Rotations for 4-Bit Activations: QuaRot, SpinQuant, and
// Friends", sections "A rotation changes nothing, and that is the point" and
// "What it buys in 4 bits").  CDNA4 has no INT4 matrix instruction, so the
// packed nibbles are widened to int8 and multiplied with
// v_mfma_i32_16x16x64_i8 (v_mfma_i32_32x32x32_i8 in the asymmetric kernel)
// into an exact int32 accumulator.
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
//
// Operand order: the prefill kernels pass the weight fragment as the MFMA's
// first operand and the activation fragment as its second, so each lane of
// a 16x16 output block ends up with one output row and four consecutive
// columns (16 contiguous bytes of Y): the epilogue stores them with one
// DPP exchange per value instead of a 4x4 transpose.
#include "common.h"
#include "kernels.h"
#include "tile.h"

namespace w4a4 {

namespace {

constexpr int BN = 128, BK = 128;   // BK in 4-bit elements
typedef __attribute__((address_space(3))) void lds_void;

// Workgroup barrier for LDS traffic: this wave's LDS operations complete, then
// s_barrier.  No memory fence, so loads still in flight (the next groups' A
// codes on their way into LDS, B codes into registers) are not waited for;
// each is waited for by the compiler where it is consumed.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
constexpr int LROW = 128;                      // LDS bytes per int8 row (one K step)

// LDS layout of an int8 operand row: its eight 16-byte chunks are stored at
// chunk position c ^ s(row), s(row) = (row & 7) ^ ((row >> 3) & 1).  The
// MFMA fragment reads (16 consecutive rows, one chunk per lane) then hit
// distinct bank groups both within every 8 lanes and within every 16 lanes;
// measured on gfx950 this pattern reads at ~165 B/clk/CU against ~110 for
// 16-byte padding or a (row >> 1) swizzle.
__device__ __forceinline__ int lds_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int lds_chunk(int row, int c) { return row * LROW + ((c ^ lds_swz(row)) << 4); }

typedef int v16i __attribute__((ext_vector_type(16)));
__device__ __forceinline__ v16i mfma32(const v4i& a, const v4i& b, const v16i& c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

template <int V>
struct IntTag {
  static constexpr int value = V;
};

}  // namespace

// ---------------------------------------------------------------- A-direct kernel (symmetric)
// BM x 128 output tile per workgroup, NW waves stacked along M, each wave
// 16*TM rows x 128 columns (TM x 8 MFMA blocks of 16x16).  gfx950's LDS
// writes are about three times slower per byte than its 16-byte reads, so
// only B (the 128 weight rows shared by every wave) is staged in LDS as
// int8; each wave streams its own A rows straight from global memory into
// registers (16 packed bytes per lane and row block per K step, two steps
// ahead) and widens them there.  K-order convention shared by both operands:
// the packed 16-byte chunk g of a 128-wide K step widens to int8 fragments
// (g, h = 0) = [lo0 hi0 lo1 hi1] and (g, h = 1) = [lo2 hi2 lo3 hi3].
template <int NW, int TM, int WPE>
__global__ void __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(WPE, WPE))) gemm_adirect_kernel(GemmParams p) {
  constexpr int BMD = NW * 16 * TM;
  constexpr int NT = NW * 64;
  constexpr int NCB = NT >= 512 ? 1 : 512 / NT;  // B chunks (16 packed bytes) per thread per K step
  const bool b_stager = NT <= 512 || threadIdx.x < 512;   // with 1024 threads, half of them stage B
  constexpr int BSTAGE = 128 * LROW;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BSTAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tiles_n = (p.N + BN - 1) / BN;
  const int64_t tiles_m = (p.M + BMD - 1) / BMD;
  int64_t tm, tn;
  tile_coords_xcd(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * BMD, n0 = tn * BN;
  const int nkt = p.K / BK;
  const int64_t ldc = p.K / 2;

  const int64_t a_bytes = (p.M - m0) * ldc, b_bytes = (p.N - n0) * ldc;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.xq + m0 * ldc), (short)0, (int)(a_bytes < 0x7fffffff ? a_bytes : 0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.wq + n0 * ldc), (short)0, (int)(b_bytes < 0x7fffffff ? b_bytes : 0x7fffffff), 0x00020000);

  const int fr = lane & 15, g = lane >> 4;
  // A: lane (fr, g) of row block i reads packed chunk g of row wave*16*TM + 16 i + fr
  const int a_off = (wave * 16 * TM + fr) * (int)ldc + 16 * g;
  // B staging: chunk cb = tid + NT * j -> row cb >> 2, packed chunk cb & 3
  int b_off[NCB], b_lds[NCB];
#pragma unroll
  for (int j = 0; j < NCB; ++j) {
    const int cb = tid + NT * j;
    b_off[j] = (cb >> 2) * (int)ldc + 16 * (cb & 3);
    b_lds[j] = lds_chunk(cb >> 2, 2 * (cb & 3));
  }
  // B fragment (g, h) of column block j: int8 chunk 2 g + h of row 16 j + fr
  const int bf0 = lds_chunk(fr, 2 * g), bf1 = lds_chunk(fr, 2 * g + 1);

  uint4 pa0[TM], pa1[TM], pb0[NCB], pb1[NCB];
  auto load_a = [&](uint4* pa, int kt) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      pa[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, a_off + i * 16 * (int)ldc + kt * 64, 0, 0));
  };
  auto load_b = [&](uint4* pb, int kt) {
    if (!b_stager) return;
#pragma unroll
    for (int j = 0; j < NCB; ++j)
      pb[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rb, b_off[j] + kt * 64, 0, 0));
  };
  auto store_b = [&](const uint4* pb, int stage) {
    if (!b_stager) return;
    uint8_t* base = smem + stage * BSTAGE;
#pragma unroll
    for (int j = 0; j < NCB; ++j) {
      const uint32_t w[4] = {pb[j].x, pb[j].y, pb[j].z, pb[j].w};
      uint32_t o[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) widen_signed(w[d], o[2 * d], o[2 * d + 1]);
      *reinterpret_cast<uint4*>(base + b_lds[j]) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4*>(base + (b_lds[j] ^ 16)) = make_uint4(o[4], o[5], o[6], o[7]);
    }
  };

  v4i acc[TM][8];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  auto compute = [&](const uint4* pa, int stage) {
    v4i a[TM][2];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const uint32_t w[4] = {pa[i].x, pa[i].y, pa[i].z, pa[i].w};
      uint32_t o[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) widen_signed(w[d], o[2 * d], o[2 * d + 1]);
      a[i][0] = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
      a[i][1] = v4i{(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
    }
    const uint8_t* Bs = smem + stage * BSTAGE;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const v4i b = *reinterpret_cast<const v4i*>(Bs + j * 16 * LROW + (h ? bf1 : bf0));
#pragma unroll
        for (int i = 0; i < TM; ++i) acc[i][j] = mfma16(b, a[i][h], acc[i][j]);
      }
    }
  };

  // prologue: A steps 0,1 and B steps 0,1 in flight; B step 0 in LDS
  load_a(pa0, 0);
  load_b(pb0, 0);
  load_a(pa1, 1);
  load_b(pb1, 1);
  store_b(pb0, 0);
  __syncthreads();
  for (int kt = 0; kt + 1 < nkt; kt += 2) {
    load_b(pb0, kt + 2);              // B step kt+2 (past the end: zeros / unused)
    compute(pa0, 0);                  // step kt (A from registers, B from stage 0)
    load_a(pa0, kt + 2);
    store_b(pb1, 1);                  // B step kt+1
    __syncthreads();
    load_b(pb1, kt + 3);
    compute(pa1, 1);                  // step kt+1
    load_a(pa1, kt + 3);
    store_b(pb0, 0);                  // B step kt+2
    __syncthreads();
  }
  if (nkt & 1) compute(pa0, 0);

  // epilogue: lane (fr, g) holds Y[m0 + wave*16*TM + 16 i + fr][n0 + 16 j +
  // 4 g + v] of block (i, j); scales come through range-checked buffer
  // loads (rows past M and columns past N read as 0 and are not stored)
  const int64_t mw = m0 + wave * 16 * TM;
  const __amdgpu_buffer_rsrc_t rws = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.ws + n0), (short)0, (int)((p.N - n0) * 4 < 0x7fffffff ? (p.N - n0) * 4 : 0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t rxs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.xs + m0), (short)0, (int)((p.M - m0) * 4 < 0x7fffffff ? (p.M - m0) * 4 : 0x7fffffff), 0x00020000);
  const bool ld_ok = (p.ldy & 3) == 0;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const float sx = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rxs, 4 * (wave * 16 * TM + 16 * i + fr), 0, 0));
    const int64_t r0 = mw + 16 * i;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const v4f swa = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rws, 4 * (16 * j + 4 * g), 0, 0));
      const v4f swb = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rws, 4 * (16 * j + 16 + 4 * g), 0, 0));
      v4f ya, yb;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        ya[v] = (sx * swa[v]) * (float)(acc[i][j][v] >> 8);
        yb[v] = (sx * swb[v]) * (float)(acc[i][j + 1][v] >> 8);
      }
      const bool full = ld_ok && r0 + 16 <= p.M && n0 + 16 * j + 32 <= p.N;
      store_pair_rows(p.y, p.ldy, p.M, p.N, r0, n0 + 16 * j, fr, g, full, ya, yb);
    }
  }
}

// ---------------------------------------------------------------- asymmetric kernel, 32x32x32 blocks
// Activation codes are unsigned with one zero-point per (row, group of 128);
// each wave widens its A rows straight to the int8 levels u - zp (|u - zp|
// <= 15), so the MFMA accumulates 16 * A_g exactly; every group's sum is
// folded into fp32 with that row's scale, y += s[m, g] * acc_g in group
// order, and the epilogue removes the factor 16 (exact) together with the
// weight scale.
// NW * 32 x 128 output tile (NW = 8: 256 rows, one workgroup per CU; NW = 4:
// 128 rows, two per CU), NW waves of 32 rows x 128 columns, each wave's tile
// as four 32x32 blocks of v_mfma_i32_32x32x32_i8.  With the weight fragment
// first, lane (h, r) = (lane >> 5, lane & 31) accumulates activation row r
// and weight columns 8 s + 4 h + v (s, v = 0..3) of each block, so one
// zero-point and one scale per lane and group serve all its 64 outputs.
// The kernel is bound by VALU issue: each output and group costs a convert
// and an fma of the fold, and widening the A codes to u - zp costs 14
// instructions per 32 K values of a row; one 32x32x32 MFMA hides about
// twice as many VALU instructions as the two 16x16x64 MFMAs doing the same
// work (32 against 16 issue cycles).
//
// Per group g (128 K values: a 64-byte packed segment of every row):
// - A: each wave's 32 rows go from global memory into its own LDS stage
//   (g & 1) with buffer_load_dwordx4 ... lds, row R's chunk c at
//   64 R + 16 (c ^ ((R >> 2) & 3)).  Lane (h, r) reads chunks 2h and 2h + 1
//   of row r; quarter q (K values 32 q .. 32 q + 31 of the fragment order)
//   widens dwords 2 (q & 1) and 2 (q & 1) + 1 of chunk 2h + (q >> 1).  Group
//   g + 2's codes are requested into the stage as soon as group g's are in
//   registers, a whole step ahead of their use.
// - B: int8 weight rows in LDS as in the other kernels; quarter q's fragment
//   of lane (h, r) is chunk 4h + q of row r, which is the same K order as
//   A's widening.  Four stages, filled two groups at a time, so one
//   workgroup barrier serves two groups.  The NW * 64 threads stage 512 / (NW
//   * 64) chunks of 16 packed bytes each per group.
// - Order inside a group: block c's four MFMAs run back to back with the
//   fold of block c + 1's previous group (during block 3: block 0's group g)
//   spread over them, 8 VALU instructions after each MFMA; block c + 1's
//   weight fragments are read during block c.  After the last group, blocks
//   1..3 are folded once more.
template <int NW>
__global__ void __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(2, 2))) gemm_asym_x32_kernel(GemmParams p) {
  constexpr int NT = NW * 64;
  constexpr int NCB = 512 / NT;                     // B chunks (16 packed bytes) per thread and group
  constexpr int BMD = NW * 32;
  constexpr int BSTAGE = 128 * LROW;                // one B stage: 128 rows x 128 int8
  constexpr int ASTAGE = NW * 2048;                 // one A stage: NW waves x 32 rows x 64 packed bytes
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * BSTAGE + 2 * ASTAGE];
  uint8_t* const sa0 = lds + 4 * BSTAGE;
  uint8_t* const sa1 = sa0 + ASTAGE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tiles_n = (p.N + BN - 1) / BN;
  const int64_t tiles_m = (p.M + BMD - 1) / BMD;
  int64_t tm, tn;
  tile_coords_xcd(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * BMD, n0 = tn * BN;
  const int nkt = p.K / BK;
  const int G = nkt;
  const int64_t ldc = p.K / 2;

  const int64_t a_bytes = (p.M - m0) * ldc, b_bytes = (p.N - n0) * ldc;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.xq + m0 * ldc), (short)0, (int)(a_bytes < 0x7fffffff ? a_bytes : 0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.wq + n0 * ldc), (short)0, (int)(b_bytes < 0x7fffffff ? b_bytes : 0x7fffffff), 0x00020000);
  // per-(row, group) zero-points and scales of this tile's rows; rows past M read as 0
  const int64_t zs_n = (p.M - m0) * G;
  const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.xz + m0 * G), (short)0, (int)(zs_n < 0x7fffffff ? zs_n : 0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.xs + m0 * G), (short)0, (int)(4 * zs_n < 0x7fffffff ? 4 * zs_n : 0x7fffffff), 0x00020000);

  const int h = lane >> 5, r = lane & 31;
  const int alr = lane >> 2;                        // DMA: lane 4 R + c' carries chunk c' ^ ((R >> 2) & 3) of row R
  const int a_goff = (wave * 32 + alr) * (int)ldc + 16 * ((lane & 3) ^ ((alr >> 2) & 3));
  const int a_roff0 = wave * 2048 + 64 * r + 16 * ((2 * h) ^ ((r >> 2) & 3));
  const int a_roff1 = wave * 2048 + 64 * r + 16 * ((2 * h + 1) ^ ((r >> 2) & 3));
  int b_off[NCB], b_lds[NCB];                       // B staging: chunk cb = tid + NT j -> row cb >> 2, packed chunk cb & 3
#pragma unroll
  for (int j = 0; j < NCB; ++j) {
    const int cb = tid + NT * j;
    b_off[j] = (cb >> 2) * (int)ldc + 16 * (cb & 3);
    b_lds[j] = lds_chunk(cb >> 2, 2 * (cb & 3));
  }
  int bfq[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) bfq[q] = lds_chunk(r, 4 * h + q);
  const int arow = (wave * 32 + r) * G;

  auto load_dma = [&](uint8_t* sa, int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(sa + wave * 2048 + i * 1024), 16,
                                               a_goff + i * 16 * (int)ldc + kt * 64, 0, 0, 0);
  };
  auto load_zs = [&](uint32_t& z, float& sx, int kt) {
    const int kc = kt < nkt ? kt : nkt - 1;
    z = __builtin_amdgcn_raw_buffer_load_b8(rz, arow + kc, 0, 0);
    sx = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (arow + kc), 0, 0));
  };
  auto load_b = [&](uint4* pb, int kt) {
#pragma unroll
    for (int j = 0; j < NCB; ++j)
      pb[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rb, b_off[j] + kt * 64, 0, 0));
  };
  auto store_b = [&](const uint4* pb, int stage) {
    uint8_t* base = lds + stage * BSTAGE;
#pragma unroll
    for (int j = 0; j < NCB; ++j) {
      const uint32_t w[4] = {pb[j].x, pb[j].y, pb[j].z, pb[j].w};
      uint32_t o[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) widen_signed(w[d], o[2 * d], o[2 * d + 1]);
      *reinterpret_cast<uint4*>(base + b_lds[j]) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4*>(base + (b_lds[j] ^ 16)) = make_uint4(o[4], o[5], o[6], o[7]);
    }
  };

  v16i acc[4];
  float yf[4][16];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      acc[c][e] = 0;
      yf[c][e] = 0.0f;
    }
  // byte-wise u - zp without cross-byte carries: (u + 128 - zp) ^ 0x80
  auto widen_q = [&](uint32_t d0, uint32_t d1, uint32_t z) -> v4i {
    const uint32_t bias = (128u - z) * 0x01010101u;
    const uint32_t o0 = ((d0 & 0x0F0F0F0Fu) + bias) ^ 0x80808080u;
    const uint32_t o1 = (((d0 >> 4) & 0x0F0F0F0Fu) + bias) ^ 0x80808080u;
    const uint32_t o2 = ((d1 & 0x0F0F0F0Fu) + bias) ^ 0x80808080u;
    const uint32_t o3 = (((d1 >> 4) & 0x0F0F0F0Fu) + bias) ^ 0x80808080u;
    return v4i{(int)o0, (int)o1, (int)o2, (int)o3};
  };
  const v16i zero16 = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

  // One group: A codes from stage sa, B rows from stage bst, zero-point z,
  // scales of this group (s_cur) and the previous one (s_prev).
  auto step = [&](uint8_t* sa, uint32_t z, float s_cur, float s_prev, int bst, int next_kt) {
    // The wait for this group's A codes (written into LDS, which the
    // compiler does not reliably track) is explicit.  Vector-memory
    // operations complete in order, and the ones issued after this group's
    // codes, zero-point and scale are B rows of two groups (2 NCB), the next
    // group's codes (2) and its zero-point and scale (2), in one order or
    // another, so vmcnt(2 NCB + 4) leaves the codes landed.  (A CPU test
    // walks the compiled code's paths for this.)
    if constexpr (NCB == 1) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    const uint4 pa0 = *reinterpret_cast<const uint4*>(sa + a_roff0);
    const uint4 pa1 = *reinterpret_cast<const uint4*>(sa + a_roff1);
    const uint8_t* Bs = lds + bst * BSTAGE;
    v4i a[4];
    a[0] = widen_q(pa0.x, pa0.y, z);
    a[1] = widen_q(pa0.z, pa0.w, z);
    a[2] = widen_q(pa1.x, pa1.y, z);
    a[3] = widen_q(pa1.z, pa1.w, z);
    // the stage has been read (the widened values exist) before group
    // next_kt's codes are requested into it
    asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
    load_dma(sa, next_kt);
    __builtin_amdgcn_sched_barrier(0);
    v4i bb[2][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) bb[0][q] = *reinterpret_cast<const v4i*>(Bs + bfq[q]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c + 1 < 4) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          bb[(c + 1) & 1][q] = *reinterpret_cast<const v4i*>(Bs + (c + 1) * 32 * LROW + bfq[q]);
      }
      const int fc = (c + 1) & 3;
      const float sf = c < 3 ? s_prev : s_cur;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[c] = mfma32(bb[c & 1][q], a[q], q == 0 ? zero16 : acc[c]);
#pragma unroll
        for (int e = 4 * q; e < 4 * q + 4; ++e) yf[fc][e] = fmaf(sf, (float)acc[fc][e], yf[fc][e]);
        // pinned: left to itself the compiler gathers the folds away from
        // the MFMAs
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Group g: A codes in stage g & 1, B rows in stage g & 3, zero-point in
  // z[g & 1], scale in s[g & 3].  A scale is used by its own step and the
  // next one and is loaded two groups ahead, so four slots rotate with no
  // register copies (a copy would wait for the load at once).
  uint32_t z[2];
  float s[4];
  s[3] = 0.0f;                                      // group "-1": the first step's folds add 0 * 0
  load_dma(sa0, 0);
  load_zs(z[0], s[0], 0);
  load_dma(sa1, 1);
  load_zs(z[1], s[1], 1);
  uint4 pb0[NCB], pb1[NCB];
  load_b(pb0, 0);
  load_b(pb1, 1);
  store_b(pb0, 0);
  store_b(pb1, 1);
  lds_barrier();
  // groups kt and kt + 1 (kt = 0 or 2 mod 4); B rows of kt + 2 and kt + 3
  // are loaded meanwhile and staged after both steps
  auto pair = [&](int kt, auto J, bool two) {
    constexpr int j = decltype(J)::value;
    load_b(pb0, kt + 2);
    load_b(pb1, kt + 3);
    step(sa0, z[0], s[j], s[(j + 3) & 3], j, kt + 2);
    load_zs(z[0], s[(j + 2) & 3], kt + 2);
    if (two) {
      step(sa1, z[1], s[j + 1], s[j], j + 1, kt + 3);
      load_zs(z[1], s[(j + 3) & 3], kt + 3);
    }
    store_b(pb0, (j + 2) & 3);
    store_b(pb1, (j + 3) & 3);
    lds_barrier();
  };
  int kt = 0;
  for (; kt + 3 < nkt; kt += 4) {
    pair(kt, IntTag<0>{}, true);
    pair(kt + 2, IntTag<2>{}, true);
  }
  if (kt < nkt) pair(kt, IntTag<0>{}, kt + 1 < nkt);
  if (kt + 2 < nkt) pair(kt + 2, IntTag<2>{}, kt + 3 < nkt);
  // blocks 1..3 still hold the last group
  const int jl = (nkt - 1) & 3;
  const float sl = jl == 0 ? s[0] : jl == 1 ? s[1] : jl == 2 ? s[2] : s[3];
#pragma unroll
  for (int c = 1; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) yf[c][e] = fmaf(sl, (float)acc[c][e], yf[c][e]);
  // the A codes requested past the last group are still writing the stages
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();                                  // the B stages become the epilogue areas

  // Epilogue: each 32 x 32 block goes through a 4 KiB LDS area of the wave
  // (rows of 128 bytes, chunk c of row R at c ^ s(R)) to full-line stores;
  // the accumulators hold 16 x the levels' products, removed here, once,
  // with the weight scale.
  uint8_t* ew = lds + wave * 32 * LROW;
  const int64_t mw = m0 + wave * 32;
  const __amdgpu_buffer_rsrc_t rws = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.ws + n0), (short)0, (int)((p.N - n0) * 4 < 0x7fffffff ? (p.N - n0) * 4 : 0x7fffffff), 0x00020000);
  const int eu = lane & 7, er = lane >> 3;
  const bool ld_ok = (p.ldy & 3) == 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const v4f swc = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rws, 4 * (32 * c + 4 * eu), 0, 0));
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<v4f*>(ew + r * LROW + 16 * ((2 * q + h) ^ lds_swz(r))) =
          v4f{yf[c][4 * q], yf[c][4 * q + 1], yf[c][4 * q + 2], yf[c][4 * q + 3]};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = er + 8 * q;
      const v4f av = *reinterpret_cast<const v4f*>(ew + rr * LROW + 16 * (eu ^ lds_swz(rr)));
      v4f yv;
#pragma unroll
      for (int v = 0; v < 4; ++v) yv[v] = av[v] * (swc[v] * 0.0625f);
      const int64_t row = mw + rr;
      const int64_t col = n0 + 32 * c + 4 * eu;
      if (ld_ok && row < p.M && col + 4 <= p.N) {
        __builtin_nontemporal_store(yv, reinterpret_cast<v4f*>(p.y + row * p.ldy + col));
      } else if (row < p.M) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (col + v < p.N) p.y[row * p.ldy + col + v] = yv[v];
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

// ---------------------------------------------------------------- symmetric kernel, 32x32x32 blocks (small shapes)
// gemm_asym_x32_kernel's structure for symmetric activations: both operands
// widened with widen_signed, every block's accumulator carried across all K
// (no per-group fold), and the symmetric epilogue y = (s_x[m] s_w[n]) *
// (acc >> 8) through the same LDS transpose.  Without zero-point and scale
// loads, the operations issued after a group's codes are B rows of two
// groups (2 NCB) and the next group's codes (2), hence vmcnt(2 NCB + 2).  Used
// as 128-row tiles of 4 waves where 256-row tiles would leave CUs idle but
// 128-row ones still give at least 160 workgroups.
template <int NW>
__global__ void __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(2, 2))) gemm_sym_x32_kernel(GemmParams p) {
  constexpr int NT = NW * 64;
  constexpr int NCB = 512 / NT;                     // B chunks (16 packed bytes) per thread and group
  constexpr int BMD = NW * 32;
  constexpr int BSTAGE = 128 * LROW;                // one B stage: 128 rows x 128 int8
  constexpr int ASTAGE = NW * 2048;                 // one A stage: NW waves x 32 rows x 64 packed bytes
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * BSTAGE + 2 * ASTAGE];
  uint8_t* const sa0 = lds + 4 * BSTAGE;
  uint8_t* const sa1 = sa0 + ASTAGE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tiles_n = (p.N + BN - 1) / BN;
  const int64_t tiles_m = (p.M + BMD - 1) / BMD;
  int64_t tm, tn;
  tile_coords_xcd(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * BMD, n0 = tn * BN;
  const int nkt = p.K / BK;
  const int G = nkt;
  const int64_t ldc = p.K / 2;

  const int64_t a_bytes = (p.M - m0) * ldc, b_bytes = (p.N - n0) * ldc;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.xq + m0 * ldc), (short)0, (int)(a_bytes < 0x7fffffff ? a_bytes : 0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.wq + n0 * ldc), (short)0, (int)(b_bytes < 0x7fffffff ? b_bytes : 0x7fffffff), 0x00020000);
  // per-(row, group) zero-points and scales of this tile's rows; rows past M read as 0
  const int64_t zs_n = (p.M - m0) * G;
  const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.xz + m0 * G), (short)0, (int)(zs_n < 0x7fffffff ? zs_n : 0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.xs + m0 * G), (short)0, (int)(4 * zs_n < 0x7fffffff ? 4 * zs_n : 0x7fffffff), 0x00020000);

  const int h = lane >> 5, r = lane & 31;
  const int alr = lane >> 2;                        // DMA: lane 4 R + c' carries chunk c' ^ ((R >> 2) & 3) of row R
  const int a_goff = (wave * 32 + alr) * (int)ldc + 16 * ((lane & 3) ^ ((alr >> 2) & 3));
  const int a_roff0 = wave * 2048 + 64 * r + 16 * ((2 * h) ^ ((r >> 2) & 3));
  const int a_roff1 = wave * 2048 + 64 * r + 16 * ((2 * h + 1) ^ ((r >> 2) & 3));
  int b_off[NCB], b_lds[NCB];                       // B staging: chunk cb = tid + NT j -> row cb >> 2, packed chunk cb & 3
#pragma unroll
  for (int j = 0; j < NCB; ++j) {
    const int cb = tid + NT * j;
    b_off[j] = (cb >> 2) * (int)ldc + 16 * (cb & 3);
    b_lds[j] = lds_chunk(cb >> 2, 2 * (cb & 3));
  }
  int bfq[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) bfq[q] = lds_chunk(r, 4 * h + q);
  const int arow = (wave * 32 + r) * G;

  auto load_dma = [&](uint8_t* sa, int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(sa + wave * 2048 + i * 1024), 16,
                                               a_goff + i * 16 * (int)ldc + kt * 64, 0, 0, 0);
  };

  auto load_b = [&](uint4* pb, int kt) {
#pragma unroll
    for (int j = 0; j < NCB; ++j)
      pb[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rb, b_off[j] + kt * 64, 0, 0));
  };
  auto store_b = [&](const uint4* pb, int stage) {
    uint8_t* base = lds + stage * BSTAGE;
#pragma unroll
    for (int j = 0; j < NCB; ++j) {
      const uint32_t w[4] = {pb[j].x, pb[j].y, pb[j].z, pb[j].w};
      uint32_t o[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) widen_signed(w[d], o[2 * d], o[2 * d + 1]);
      *reinterpret_cast<uint4*>(base + b_lds[j]) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4*>(base + (b_lds[j] ^ 16)) = make_uint4(o[4], o[5], o[6], o[7]);
    }
  };

  v16i acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0;
  auto widen_q = [&](uint32_t d0, uint32_t d1) -> v4i {
    uint32_t o[4];
    widen_signed(d0, o[0], o[1]);
    widen_signed(d1, o[2], o[3]);
    return v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
  };

  // One group: A codes from stage sa, B rows from stage bst, zero-point z,
  // scales of this group (s_cur) and the previous one (s_prev).
  auto step = [&](uint8_t* sa, int bst, int next_kt) {
    // The wait for this group's A codes (written into LDS, which the
    // compiler does not reliably track) is explicit.  Vector-memory
    // operations complete in order, and the ones issued after this group's
    // codes, zero-point and scale are B rows of two groups (2 NCB), the next
    // group's codes (2) and its zero-point and scale (2), in one order or
    // another, so vmcnt(2 NCB + 4) leaves the codes landed.  (A CPU test
    // walks the compiled code's paths for this.)
    if constexpr (NCB == 1) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    const uint4 pa0 = *reinterpret_cast<const uint4*>(sa + a_roff0);
    const uint4 pa1 = *reinterpret_cast<const uint4*>(sa + a_roff1);
    const uint8_t* Bs = lds + bst * BSTAGE;
    v4i a[4];
    a[0] = widen_q(pa0.x, pa0.y);
    a[1] = widen_q(pa0.z, pa0.w);
    a[2] = widen_q(pa1.x, pa1.y);
    a[3] = widen_q(pa1.z, pa1.w);
    // the stage has been read (the widened values exist) before group
    // next_kt's codes are requested into it
    asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
    load_dma(sa, next_kt);
    __builtin_amdgcn_sched_barrier(0);
    v4i bb[2][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) bb[0][q] = *reinterpret_cast<const v4i*>(Bs + bfq[q]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c + 1 < 4) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          bb[(c + 1) & 1][q] = *reinterpret_cast<const v4i*>(Bs + (c + 1) * 32 * LROW + bfq[q]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[c] = mfma32(bb[c & 1][q], a[q], acc[c]);
        // pinned: left to itself the compiler gathers the folds away from
        // the MFMAs
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  load_dma(sa0, 0);
  load_dma(sa1, 1);
  uint4 pb0[NCB], pb1[NCB];
  load_b(pb0, 0);
  load_b(pb1, 1);
  store_b(pb0, 0);
  store_b(pb1, 1);
  lds_barrier();
  auto pair = [&](int kt, auto J, bool two) {
    constexpr int j = decltype(J)::value;
    load_b(pb0, kt + 2);
    load_b(pb1, kt + 3);
    step(sa0, j, kt + 2);
    if (two) step(sa1, j + 1, kt + 3);
    store_b(pb0, (j + 2) & 3);
    store_b(pb1, (j + 3) & 3);
    lds_barrier();
  };
  int kt = 0;
  for (; kt + 3 < nkt; kt += 4) {
    pair(kt, IntTag<0>{}, true);
    pair(kt + 2, IntTag<2>{}, true);
  }
  if (kt < nkt) pair(kt, IntTag<0>{}, kt + 1 < nkt);
  if (kt + 2 < nkt) pair(kt + 2, IntTag<2>{}, kt + 3 < nkt);
  // the A codes requested past the last group are still writing the stages
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();                                  // the B stages become the epilogue areas

  // Epilogue: each 32 x 32 block goes through a 4 KiB LDS area of the wave
  // (rows of 128 bytes, chunk c of row R at c ^ s(R)) to full-line stores;
  // the accumulators hold 16 x the levels' products, removed here, once,
  // with the weight scale.
  uint8_t* ew = lds + wave * 32 * LROW;
  const int64_t mw = m0 + wave * 32;
  const __amdgpu_buffer_rsrc_t rws = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.ws + n0), (short)0, (int)((p.N - n0) * 4 < 0x7fffffff ? (p.N - n0) * 4 : 0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t rxs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.xs + m0), (short)0, (int)((p.M - m0) * 4 < 0x7fffffff ? (p.M - m0) * 4 : 0x7fffffff), 0x00020000);
  const int eu = lane & 7, er = lane >> 3;
  const bool ld_ok = (p.ldy & 3) == 0;
  float sxr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    sxr[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rxs, 4 * (wave * 32 + er + 8 * q), 0, 0));
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const v4f swc = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rws, 4 * (32 * c + 4 * eu), 0, 0));
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<v4i*>(ew + r * LROW + 16 * ((2 * q + h) ^ lds_swz(r))) =
          v4i{acc[c][4 * q], acc[c][4 * q + 1], acc[c][4 * q + 2], acc[c][4 * q + 3]};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = er + 8 * q;
      const v4i av = *reinterpret_cast<const v4i*>(ew + rr * LROW + 16 * (eu ^ lds_swz(rr)));
      v4f yv;
#pragma unroll
      for (int v = 0; v < 4; ++v) yv[v] = (sxr[q] * swc[v]) * (float)(av[v] >> 8);
      const int64_t row = mw + rr;
      const int64_t col = n0 + 32 * c + 4 * eu;
      if (ld_ok && row < p.M && col + 4 <= p.N) {
        __builtin_nontemporal_store(yv, reinterpret_cast<v4f*>(p.y + row * p.ldy + col));
      } else if (row < p.M) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (col + v < p.N) p.y[row * p.ldy + col + v] = yv[v];
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

// ---------------------------------------------------------------- decode kernel
// M <= 16 rows (symmetric): one workgroup per 16 output columns; the 4 waves
// split the 128-wide K steps (wave w takes steps w, w+4, ...).  The kernel is
// bound by streaming W's packed rows.  Every wave moves the 16 rows x 64
// bytes of 8 of its K steps at once straight into its own LDS area with
// buffer_load_dwordx4 ... lds (8 KiB per wave in flight), in the coalesced
// order: lane 4 r + c' reads chunk c' ^ ((r >> 2) & 3) of row r, so four
// adjacent lanes read one 64-byte row segment and the fragment reads in the
// MFMA layout (lane 16 g + r reads chunk g of row r) hit 16 distinct bank
// groups.  Loading the registers straight in the MFMA layout instead (lane
// 16 g + r reading row r) costs 4% at 16 x 4096 x 4096 and up to 25% warm on
// larger shapes.  X (M x K/2 bytes, read by every workgroup from L2) goes
// into registers.  Rows of X beyond M and steps beyond K read as zero through
// the buffer range check.
__global__ void __launch_bounds__(256) gemm_decode_kernel(GemmParams p) {
  __shared__ v4i red[3][64];
  __shared__ __attribute__((aligned(16))) uint8_t sw[4][8 * 1024];   // [wave][step of the batch][16 rows x 64 B]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, kg = 16 * (lane >> 4);
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int nkt = p.K / BK;
  const int ldc = p.K / 2;
  const int64_t nw = p.N - n0 < 16 ? p.N - n0 : 16;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.xq, (short)0, (int)(p.M * ldc), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.wq + n0 * ldc), (short)0, (int)(nw * ldc), 0x00020000);
  const int x_off = i * ldc + kg;
  const int lr = lane >> 2;
  const int w_goff = lr * ldc + 16 * ((lane & 3) ^ ((lr >> 2) & 3));
  const int w_roff = 64 * i + 16 * ((lane >> 4) ^ ((i >> 2) & 3));
  uint8_t* const mine = sw[wave];

  v4i acc = v4i{0, 0, 0, 0};
  for (int t0 = 0; 4 * t0 < nkt; t0 += 8) {
    uint4 xa[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int kt = wave + 4 * (t0 + u);
      const bool in = kt < nkt;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(mine + u * 1024), 16,
                                               in ? w_goff + kt * 64 : 0x7FFFFFF0, 0, 0, 0);
      xa[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, in ? x_off + kt * 64 : 0x7FFFFFF0, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint4 wb = *reinterpret_cast<const uint4*>(mine + u * 1024 + w_roff);
      const uint32_t xw[4] = {xa[u].x, xa[u].y, xa[u].z, xa[u].w};
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
    // this wave's reads of its LDS area are done before the next batch refills it
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    acc += red[0][lane];
    acc += red[1][lane];
    acc += red[2][lane];
    const int64_t col = n0 + i;
    if (col < p.N) {
      const float sw_n = p.ws[col];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 4 * (lane >> 4) + v;
        if (row < p.M) p.y[row * p.ldy + col] = (p.xs[row] * sw_n) * (float)(acc[v] >> 8);
      }
    }
  }
}

hipError_t gemm_prepare_device() { return hipSuccess; }   // no per-device setup needed

hipError_t launch_gemm(const GemmParams& p, int mode, hipStream_t st) {
  if (p.M == 0) return hipSuccess;
  if (mode == kModeSym && p.M <= 16) {
    const int64_t grid = (p.N + 15) / 16;
    W4A4_LAUNCH(gemm_decode_kernel, dim3((uint32_t)grid), dim3(256), 0, st, p);
    return hipGetLastError();
  }
  if (mode == kModeSym) {
    // A-direct kernel.  256-row tiles of 8 waves (32 x 128 each) from one
    // tile per CU up (measured faster than 16 waves of 16 x 128 at every
    // shape from 256 to 511 tiles: q_proj 32.8 vs 34.8 us, 3072 x 4096 x 4096
    // 49 vs 63 us).
    const int64_t grid = ((p.M + 255) / 256) * ((p.N + BN - 1) / BN);
    if (grid >= 256) {
      W4A4_LAUNCH((gemm_adirect_kernel<8, 2, 4>), dim3((uint32_t)grid), dim3(512), 0, st, p);
    } else {
      // fewer than one 256-row tile per CU: 128-row tiles of 4 waves on
      // 32x32 blocks from 160 of them up (1536 x 4096 x 4096: 31.2 against
      // 40.6 us for 64-row tiles; 600 x 4096 x 14336: 65.6 against 73.8),
      // else 64-row tiles of 4 waves (512 x 4096 x 4096, 128 tiles of 128
      // rows: 16.9 against 19.8 us)
      const int64_t tiles_n = (p.N + BN - 1) / BN;
      const int64_t grid128 = ((p.M + 127) / 128) * tiles_n;
      if (grid128 >= 160) {
        W4A4_LAUNCH(gemm_sym_x32_kernel<4>, dim3((uint32_t)grid128), dim3(256), 0, st, p);
      } else {
        const int64_t grid = ((p.M + 63) / 64) * tiles_n;
        W4A4_LAUNCH((gemm_adirect_kernel<4, 1, 2>), dim3((uint32_t)grid), dim3(256), 0, st, p);
      }
    }
    return hipGetLastError();
  }
  // asymmetric per-group activations: 256-row tiles of 8 waves from one tile
  // per CU up (gate/up 8192 x 28672 x 8192: 2.44-2.50 ms against 2.60-2.62
  // ms for the 16x16x64 kernel this one replaced, on the same boxes), else
  // 128-row tiles of 4 waves, two workgroups per CU, so that small shapes
  // still spread over the CUs (256 x 28672 x 8192: 87 against 109 us)
  const int64_t tiles_n = (p.N + BN - 1) / BN;
  const int64_t grid = ((p.M + 255) / 256) * tiles_n;
  if (grid >= 256) {
    W4A4_LAUNCH(gemm_asym_x32_kernel<8>, dim3((uint32_t)grid), dim3(512), 0, st, p);
  } else {
    const int64_t grid = ((p.M + 127) / 128) * tiles_n;
    W4A4_LAUNCH(gemm_asym_x32_kernel<4>, dim3((uint32_t)grid), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace w4a4
