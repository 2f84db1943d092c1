// MXFP4 GEMM on gfx950's block-scaled FP4 MFMA.
//
// MXFP4 is the other 4-bit activation format that rotations help: E2M1
// elements with one power-of-two scale per 32 consecutive values ("Rotations
// for 4-Bit Activations: QuaRot, SpinQuant, and Friends", sections "The full
// model in NVFP4, on vLLM" and "When to rotate").  With both operands
// rotated and quantized this way,
//   Y[m, n] = sum_j 2^(ea[m, j] + eb[n, j]) * sum_{k in block j} a[m, k] b[n, k],
// and CDNA4 computes exactly that in hardware: v_mfma_scale_f32_16x16x128_f8f6f4
// with both formats set to FP4 takes, per lane, 16 packed bytes (32 E2M1
// codes, even k in the low nibble, as the quantizer packs them) and one
// biased exponent byte for the 32 values it holds, and accumulates in fp32.
// No widening, no zero-points and no dequantization epilogue are needed.
//
// Lane layout of one 16x16x128 product (lane l = 16 g + r): A row r and
// B row r, K elements 32 g .. 32 g + 31 (packed bytes 16 g .. 16 g + 15 of
// the 64-byte step), exponent of (row r, block g); C rows 4 g .. 4 g + 3 of
// column r.  The prefill kernel passes the weight fragment first and the
// activation fragment second, so C's rows are output columns: lane (r, g)
// holds output row r, columns 4 g .. 4 g + 3 (16 contiguous bytes).  The
// packed operands need no widening, so both go from global memory straight
// into LDS (see the prefill kernel) and are read back in this lane layout.
//
// Exponent bytes: a row holds 4 per 128-wide K step, [4 kt + g].  A lane
// loads the 16 bytes of four steps of its row at once and gathers the 4
// bytes of its block g (one per step) into one dword; the MFMA's op_sel
// then picks byte s of that dword at step s of the group, so no per-step
// instruction touches the exponents.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "tile.h"

namespace w4a4 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBN = 128;       // output columns per workgroup
constexpr int kKS = 128;       // K elements per step (64 packed bytes of a row)
constexpr int kRow = 64;       // LDS bytes of one B row per step

// LDS position of 16-byte chunk c (0..3) of B row `row` in a step buffer:
// chunk c ^ ((row >> 1) & 3).  Chosen by measurement on gfx950 (ds_read_b128
// of the fragment pattern: 16 consecutive rows, one chunk per group of 16
// lanes): this layout reads at ~214 B/clk/CU, while the plain layout, XORs
// with row & 3, (row >> 2) & 3 or ((row >> 1) ^ (row >> 3)) & 3, and 80-byte
// padding all read at 108-116 B/clk/CU.
__device__ __forceinline__ int mx_chunk(int row, int c) { return row * kRow + ((c ^ ((row >> 1) & 3)) << 4); }

// Workgroup barrier for the prefill kernel's LDS stages: this wave's LDS
// operations complete and at most N of its vector-memory operations remain in
// flight, then s_barrier.  No memory fence: a __syncthreads would also wait
// for the loads of later steps that are still on their way.
template <int N>
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// One 16x16x128 FP4 x FP4 product with per-lane E8M0 scales; SEL picks the
// scale byte inside the scale dwords.
template <int SEL>
__device__ __forceinline__ v4f mfma_mx(const uint4& a, uint32_t sa, const uint4& b, uint32_t sb, const v4f& c) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, SEL, (int)sa, SEL, (int)sb);
}

// 4x4 byte transpose: byte g of d[s] -> byte s of e[g].
__device__ __forceinline__ uint4 transpose_bytes4(const uint4& d) {
  const uint32_t t0 = __builtin_amdgcn_perm(d.y, d.x, 0x05010400u);   // d0.0 d1.0 d0.1 d1.1
  const uint32_t t1 = __builtin_amdgcn_perm(d.y, d.x, 0x07030602u);   // d0.2 d1.2 d0.3 d1.3
  const uint32_t t2 = __builtin_amdgcn_perm(d.w, d.z, 0x05010400u);
  const uint32_t t3 = __builtin_amdgcn_perm(d.w, d.z, 0x07030602u);
  return make_uint4(__builtin_amdgcn_perm(t2, t0, 0x05040100u), __builtin_amdgcn_perm(t2, t0, 0x07060302u),
                    __builtin_amdgcn_perm(t3, t1, 0x05040100u), __builtin_amdgcn_perm(t3, t1, 0x07060302u));
}

// Byte g of each of d.x .. d.w gathered into one dword (sel = g | (g + 4) << 8
// | 0x0C0C0000: bytes g of the low and high source, then two zero bytes).
__device__ __forceinline__ uint32_t gather_bytes(const uint4& d, uint32_t sel) {
  const uint32_t lo = __builtin_amdgcn_perm(d.y, d.x, sel);
  const uint32_t hi = __builtin_amdgcn_perm(d.w, d.z, sel);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff), 0x00020000);
}

}  // namespace

// ---------------------------------------------------------------- prefill kernel
// BM x 128 output tile per workgroup, NW waves stacked along M, each wave
// 16*TM rows x 128 columns (TM x 8 products of 16x16 per step).
//
// Both operands go from global memory straight into LDS with gfx950's
// buffer_load_dwordx4 ... lds: one such load writes the 16 bytes of lane l at
// LDS offset 16 l of its destination, so no register staging and no LDS
// store instruction are needed.  Each lane is given the global address whose
// bytes belong at its LDS position:
//   - A (private to each wave, 16 rows per load): lane 4 r + c' reads chunk
//     c' ^ ((r >> 2) & 3) of row r, so that the fragment reads below (lane
//     16 g + r reads chunk g of row r) hit 16 distinct bank groups;
//   - B (shared, each wave moves 128 / NW rows, 16 per load): lane 4 r + c'
//     reads chunk c' ^ ((row >> 1) & 3), the layout of mx_chunk.
// Four adjacent lanes thus read one 64-byte row segment.  Registers loaded
// straight in the MFMA layout (lane 16 g + r reading row r, adjacent lanes in
// 16 different rows) cost the load path about 2.7 times this order's time.
//
// Steps are walked in groups of four (the four bytes of an exponent dword).
// Each operand has four LDS stages, step t in stage t & 3, each its own array
// so that the compiler's waits for a stage's loads are exact; the loads of
// step t + 2 are issued at the start of step t, into the stage step t - 2
// used.  At the end of step t the wave waits for its own share of B step t + 1
// (the last operation it issued before step t) by allowing only step t's own
// KS operand loads to remain in flight, then the workgroup barrier makes the
// whole stage visible.  At a group start the step also loads the next group's
// exponents, ahead of its operand loads; they are older, so the same count
// waits for them too, and it stays right where the compiler drops them (the
// last group's are never used) or a wave skips the B exponents.  The
// exponents of B (shared by every wave) go through a double-buffered LDS
// table once per group.  A step past the end of K is loaded (harmlessly,
// inside or past the operand's range) but not multiplied.
template <int NW, int TM, int WPE>
__global__ void __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(WPE, WPE))) mx_gemm_kernel(MxGemmParams p) {
  constexpr int BMD = NW * 16 * TM;
  static_assert(NW == 4 || NW == 8, "B: 16 or 32 rows per wave and step");
  constexpr int BPW = 128 / (16 * NW);      // B loads per wave and step
  constexpr int KS = TM + BPW;              // operand loads per step
  constexpr int BSTAGE = 128 * kRow;
  constexpr int ASTAGE = NW * TM * 1024;
  __shared__ __attribute__((aligned(16))) uint8_t sa0[ASTAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sa1[ASTAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sa2[ASTAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sa3[ASTAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sb0[BSTAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sb1[BSTAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sb2[BSTAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sb3[BSTAGE];
  __shared__ __attribute__((aligned(16))) uint32_t bexp[2][128 * 4];   // [group parity][B row][block g]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tiles_n = (p.N + kBN - 1) / kBN;
  const int64_t tiles_m = (p.M + BMD - 1) / BMD;
  int64_t tm, tn;
  tile_coords_xcd(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * BMD, n0 = tn * kBN;
  const int nkt = p.K / kKS;
  const int ngr = (nkt + 3) / 4;
  const int64_t ldc = p.K / 2, lde = p.K / 32;

  const __amdgpu_buffer_rsrc_t ra = rsrc(p.xq + m0 * ldc, (p.M - m0) * ldc);
  const __amdgpu_buffer_rsrc_t rb = rsrc(p.wq + n0 * ldc, (p.N - n0) * ldc);
  const __amdgpu_buffer_rsrc_t rae = rsrc(p.xe + m0 * lde, (p.M - m0) * lde);
  const __amdgpu_buffer_rsrc_t rbe = rsrc(p.we + n0 * lde, (p.N - n0) * lde);

  const int fr = lane & 15, g = lane >> 4;
  const int lr = lane >> 2;                                      // row of this lane's loads
  const int a_goff = (wave * 16 * TM + lr) * (int)ldc + 16 * ((lane & 3) ^ ((lr >> 2) & 3));
  const int a_roff = wave * TM * 1024 + 64 * fr + 16 * (g ^ ((fr >> 2) & 3));
  const int b_row = wave * 16 * BPW + lr;
  const int b_goff = b_row * (int)ldc + 16 * ((lane & 3) ^ ((b_row >> 1) & 3));
  const int ae_off = (wave * 16 * TM + fr) * (int)lde;           // + 16 i lde + 16 u
  const uint32_t gsel = (uint32_t)g | ((uint32_t)(g + 4) << 8) | 0x0C0C0000u;
  const int bf = mx_chunk(fr, g);        // fragment of column block j at bf + j * 16 * kRow
  const bool be_stager = tid < 128;      // thread t stages the exponents of B row t

  uint4 ae_raw[TM], be_raw;
  uint32_t ae[TM], be[8];

  auto issue = [&](uint8_t* sa, uint8_t* sb, int kt) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(sa + wave * TM * 1024 + i * 1024), 16,
                                               a_goff + i * 16 * (int)ldc + kt * 64, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < BPW; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(sb + (wave * BPW + q) * 1024), 16,
                                               b_goff + q * 16 * (int)ldc + kt * 64, 0, 0, 0);
  };
  auto load_exps = [&](int u) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      ae_raw[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rae, ae_off + i * 16 * (int)lde + 16 * u, 0, 0));
    if (be_stager)
      be_raw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rbe, tid * (int)lde + 16 * u, 0, 0));
  };
  auto store_bexp = [&](int par) {
    if (be_stager) *reinterpret_cast<uint4*>(&bexp[par][4 * tid]) = transpose_bytes4(be_raw);
  };
  auto take_exps = [&](int par) {
#pragma unroll
    for (int i = 0; i < TM; ++i) ae[i] = gather_bytes(ae_raw[i], gsel);
#pragma unroll
    for (int j = 0; j < 8; ++j) be[j] = bexp[par][4 * (16 * j + fr) + g];
  };

  v4f acc[TM][8];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](auto sel, const uint8_t* sa, const uint8_t* sb) {
    constexpr int S = decltype(sel)::value;
    uint4 a[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = *reinterpret_cast<const uint4*>(sa + a_roff + i * 1024);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint4 b = *reinterpret_cast<const uint4*>(sb + j * 16 * kRow + bf);
#pragma unroll
      for (int i = 0; i < TM; ++i) acc[i][j] = mfma_mx<S>(b, be[j], a[i], ae[i], acc[i][j]);
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;

  // prologue: exponents of group 0, steps 0 and 1 on their way, B exponents
  // of group 0 in LDS, this wave's share of B step 0 landed
  load_exps(0);
  issue(sa0, sb0, 0);
  issue(sa1, sb1, 1);
  store_bexp(0);
  stage_barrier<KS>();
  // one group of four steps; FULL: all four lie inside K.  The scheduling
  // fences keep each step's loads ahead of its multiplications, where the
  // barrier counts expect them.
  auto group = [&](int u, auto FULL) {
    constexpr bool full = decltype(FULL)::value;
    const int kt = 4 * u;
    const int par = u & 1;
    take_exps(par);                   // this group's exponents into registers ...
    load_exps(u + 1);                 // ... and the next group's on their way
    issue(sa2, sb2, kt + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(S0{}, sa0, sb0);          // step kt (always < nkt)
    __builtin_amdgcn_sched_barrier(0);
    stage_barrier<KS>();
    issue(sa3, sb3, kt + 3);
    __builtin_amdgcn_sched_barrier(0);
    if (full || kt + 1 < nkt) compute(S1{}, sa1, sb1);
    __builtin_amdgcn_sched_barrier(0);
    store_bexp(par ^ 1);              // B exponents of group u+1 (the other table was last read in group u-1)
    stage_barrier<KS>();
    issue(sa0, sb0, kt + 4);
    __builtin_amdgcn_sched_barrier(0);
    if (full || kt + 2 < nkt) compute(S2{}, sa2, sb2);
    __builtin_amdgcn_sched_barrier(0);
    stage_barrier<KS>();
    issue(sa1, sb1, kt + 5);
    __builtin_amdgcn_sched_barrier(0);
    if (full || kt + 3 < nkt) compute(S3{}, sa3, sb3);
    __builtin_amdgcn_sched_barrier(0);
    stage_barrier<KS>();
  };
  const int nfull = nkt / 4;
  for (int u = 0; u < nfull; ++u) group(u, std::true_type{});
  if (nfull < ngr) group(nfull, std::false_type{});
  // the loads of the two steps past the last one are still writing this
  // workgroup's LDS stages: let them land before the workgroup can end
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // epilogue: lane (fr, g) holds Y[m0 + wave*16*TM + 16 i + fr][n0 + 16 j +
  // 4 g + v] of block (i, j); pairs of blocks go out as full 128-byte rows
  const bool ld_ok = (p.ldy & 3) == 0;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t r0 = m0 + wave * 16 * TM + 16 * i;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const bool full = ld_ok && r0 + 16 <= p.M && n0 + 16 * j + 32 <= p.N;
      store_pair_rows(p.y, p.ldy, p.M, p.N, r0, n0 + 16 * j, fr, g, full, acc[i][j], acc[i][j + 1]);
    }
  }
}

// ---------------------------------------------------------------- decode kernel (M <= 16)
// The product is weight-bandwidth bound: one workgroup per 16 output
// columns, its 4 waves splitting the K steps into contiguous ranges with 8
// steps of loads in flight, partial sums added through LDS.  The weight codes
// go straight into each wave's LDS area with buffer_load_dwordx4 ... lds in the
// coalesced order of the int8 decode kernel (lane 4 r + c' reads chunk
// c' ^ ((r >> 2) & 3) of row r) and are read back in the MFMA lane layout.  A
// lane takes the exponents of 4 consecutive steps of its row in one 16-byte
// load and shifts out the byte of its block g per step.  Rows of X beyond M
// read as zero codes and exponents through the buffer range check; steps
// beyond K are not multiplied (their exponent bytes belong to the next row).
__global__ void __launch_bounds__(256) mx_gemm_decode_kernel(MxGemmParams p) {
  __shared__ v4f red[3][64];
  __shared__ __attribute__((aligned(16))) uint8_t sw[4][8 * 1024];   // [wave][step of the batch][16 rows x 64 B]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int nkt = p.K / kKS;
  const int spw = (((nkt + 3) / 4) + 3) & ~3;       // steps per wave, a multiple of 4
  const int k_first = wave * spw;
  const int ldc = p.K / 2, lde = p.K / 32;
  const int64_t nw = p.N - n0 < 16 ? p.N - n0 : 16;
  const __amdgpu_buffer_rsrc_t rx = rsrc(p.xq, p.M * ldc);
  const __amdgpu_buffer_rsrc_t rw = rsrc(p.wq + n0 * ldc, nw * ldc);
  const __amdgpu_buffer_rsrc_t rxe = rsrc(p.xe, p.M * lde);
  const __amdgpu_buffer_rsrc_t rwe = rsrc(p.we + n0 * lde, nw * lde);
  const int c_off = r * ldc + 16 * g;
  const int lr = lane >> 2;
  const int w_goff = lr * ldc + 16 * ((lane & 3) ^ ((lr >> 2) & 3));
  const int w_roff = 64 * r + 16 * (g ^ ((r >> 2) & 3));
  const int e_off = r * lde;
  const int gshift = 8 * g;
  uint8_t* const mine = sw[wave];

  v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  for (int t0 = 0; t0 < spw; t0 += 8) {
    uint4 xa[8], xe4[2], we4[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kt = k_first + t0 + 4 * h;          // exponents of steps kt .. kt + 3
      const int eo = kt < nkt ? e_off + 4 * kt : 0x7FFFFFF0;
      xe4[h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rxe, eo, 0, 0));
      we4[h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rwe, eo, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int kt = k_first + t0 + u;
      const bool in = t0 + u < spw && kt < nkt;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(mine + u * 1024), 16,
                                               in ? w_goff + kt * 64 : 0x7FFFFFF0, 0, 0, 0);
      xa[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, in ? c_off + kt * 64 : 0x7FFFFFF0, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int kt = k_first + t0 + u;
      if (t0 + u < spw && kt < nkt) {               // uniform over the wave
        const uint4 wb = *reinterpret_cast<const uint4*>(mine + u * 1024 + w_roff);
        const uint4 xe = xe4[u >> 2], we = we4[u >> 2];
        const uint32_t xd = (u & 3) == 0 ? xe.x : (u & 3) == 1 ? xe.y : (u & 3) == 2 ? xe.z : xe.w;
        const uint32_t wd = (u & 3) == 0 ? we.x : (u & 3) == 1 ? we.y : (u & 3) == 2 ? we.z : we.w;
        acc = mfma_mx<0>(xa[u], xd >> gshift, wb, wd >> gshift, acc);
      }
    }
    // every load of this batch has landed (its area is refilled next batch, and
    // none may still be writing LDS when the workgroup ends)
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  }
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    acc += red[0][lane];
    acc += red[1][lane];
    acc += red[2][lane];
    const int64_t col = n0 + r;
    if (col < p.N) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 4 * g + v;
        if (row < p.M) p.y[row * p.ldy + col] = acc[v];
      }
    }
  }
}

hipError_t launch_mx_gemm(const MxGemmParams& p, hipStream_t st) {
  if (p.M == 0) return hipSuccess;
  if (p.M <= 16) {
    const int64_t grid = (p.N + 15) / 16;
    W4A4_LAUNCH(mx_gemm_decode_kernel, dim3((uint32_t)grid), dim3(256), 0, st, p);
  } else if (((p.M + 255) / 256) * ((p.N + kBN - 1) / kBN) >= 256) {
    // 256-row tiles of 8 waves (32 rows each) from one tile per CU up; fewer:
    // 64-row tiles of 4 waves, so that small shapes still spread over the CUs
    const int64_t grid = ((p.M + 255) / 256) * ((p.N + kBN - 1) / kBN);
    W4A4_LAUNCH((mx_gemm_kernel<8, 2, 2>), dim3((uint32_t)grid), dim3(512), 0, st, p);
  } else {
    const int64_t grid = ((p.M + 63) / 64) * ((p.N + kBN - 1) / kBN);
    W4A4_LAUNCH((mx_gemm_kernel<4, 1, 2>), dim3((uint32_t)grid), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace w4a4
