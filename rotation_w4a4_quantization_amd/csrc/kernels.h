// Kernel parameter blocks and launchers (internal to the library).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a4 {

enum { kModeSym = 0, kModeAsym = 1, kModeMx = 2 };

// Rotate + quantize: one row of K fp16 values -> K/2 code bytes.
struct RQParams {
  const uint16_t* x;
  const uint16_t* signs;   // optional [K] fp16 +-1: the diagonal D of Q = D H / sqrt(b)
  uint8_t* codes;    // [rows][K/2]
  float* scales;     // sym: [rows]; asym: [rows][K/128]
  uint8_t* zeros;    // asym: [rows][K/128]
  uint8_t* mx_scales;  // MXFP4: [rows][K/32] biased power-of-two exponents
  int32_t* gsum;     // optional: [rows][K/128]
  int64_t rows;
  int64_t ss;        // row stride in elements (strided mode: the s stride)
  int64_t sh, sb;    // strided mode: h and b strides (elements)
  uint32_t S, H;     // strided mode: row r -> (b, h, s) = (r/(H S), (r/S)%H, r%S)
  int32_t K;
  int32_t nb;        // K / 128 (set by the launcher)
  int32_t seg;       // threads per row slot (set by the launcher)
  int32_t rows_per_wg;
  int32_t log2seg;   // log2(seg) when rows_per_wg > 1
  float cdiv;        // fl32(7 sqrt(b)) (sym), fl32(15 sqrt(b)) (asym), fl32(1 / sqrt(b)) (MXFP4)
};

struct RQGeometry {
  int seg, rows_per_wg, threads;
  int64_t grid;
};

RQGeometry rq_geometry(int64_t rows, int K);
hipError_t launch_rotate_quant(RQParams p, int mode, bool full, bool gsum, bool strided,
                               hipStream_t st);

// W4A4 GEMM: y[M][ldy] = dequant(xq) . dequant(wq)^T.
struct GemmParams {
  const uint8_t* xq;    // [M][K/2]
  const float* xs;      // sym: [M]; asym: [M][K/128]
  const uint8_t* xz;    // asym: [M][K/128]
  const uint8_t* wq;    // [N][K/2]
  const float* ws;      // [N]
  float* y;
  int64_t M, N, ldy;
  int32_t K;
};

hipError_t launch_gemm(const GemmParams& p, int mode, hipStream_t st);
hipError_t gemm_prepare_device();   // once per device, before the first GEMM launch

// Decode W4A4 linear in one launch: symmetric per-token INT4 of the rotated
// activation rows (128-blocks) fused into the weight-streaming GEMM.
struct FusedDecodeParams {
  const uint16_t* x;      // [M][ldx] fp16
  const uint16_t* signs;  // optional [K] fp16 +-1
  const uint8_t* wq;      // [N][K/2]
  const float* ws;        // [N]
  float* y;               // [M][ldy]
  int64_t N, ldy;
  int32_t M, K, ldx;
  float cdiv;             // fl32(7 sqrt(128))
};

hipError_t launch_decode_fused(const FusedDecodeParams& p, hipStream_t st);

// MXFP4 GEMM: Y = sum over 32-blocks of 2^(ea + eb) * (E2M1 codes . E2M1 codes).
struct MxGemmParams {
  const uint8_t* xq;    // [M][K/2] packed E2M1 codes
  const uint8_t* xe;    // [M][K/32] biased exponents
  const uint8_t* wq;    // [N][K/2]
  const uint8_t* we;    // [N][K/32]
  float* y;
  int64_t M, N, ldy;
  int32_t K;
};

hipError_t launch_mx_gemm(const MxGemmParams& p, hipStream_t st);

// Decode attention over the rotated INT4 KV cache (one query per head).
struct AttnParams {
  const uint16_t* q;          // [BH][128] fp16
  const uint8_t* k_codes;     // [BH][S][64]
  const float* k_scales;      // [BH][S]
  const uint8_t* k_zeros;     // [BH][S]
  const uint8_t* v_codes;
  const float* v_scales;
  const uint8_t* v_zeros;
  const uint16_t* signs;      // optional [128] fp16 +-1
  float* out;                 // [BH][128] fp32
  int64_t BH, S;
  float scale2;               // softmax scale * log2(e)
  float* part;                // split path: [BH][nsplit][kAttnPartFloats] partial states
  int32_t nsplit;             // split path: token ranges per (batch, head)
};

// Split path: floats per partial state (128 rotated output sums, running
// maximum, running sum, two pad floats so that every state is 16-byte aligned).
constexpr int kAttnPartFloats = 132;

hipError_t launch_kv4_attention(const AttnParams& p, hipStream_t st);
// Split path: p.part (p.BH * p.nsplit partial states) and p.nsplit set; with
// p.nsplit <= 1 the single pass.
hipError_t launch_kv4_attention_split(const AttnParams& p, hipStream_t st);

// Optional per-launch timing: events armed on this host thread are attached to
// the next kernel launch (the runtime writes the kernel's own start and end
// timestamps into them) and then disarmed.
struct LaunchTiming {
  hipEvent_t start = nullptr, stop = nullptr;
};
void arm_launch_timing(hipEvent_t start, hipEvent_t stop);
LaunchTiming take_launch_timing();

// Every kernel of the library is launched through this, so an armed pair of
// timing events always lands on the kernel an entry point enqueues.
#define W4A4_LAUNCH(KERNEL, GRID, BLOCK, LDS, STREAM, ...)                                 \
  do {                                                                                     \
    const ::w4a4::LaunchTiming t_ = ::w4a4::take_launch_timing();                          \
    hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, (uint32_t)(LDS), STREAM, t_.start, t_.stop, \
                          0u, __VA_ARGS__);                                                \
  } while (0)

// For an entry point that enqueues two kernels: the armed start event goes
// to the first launch and the stop event to the second (T is the pair taken
// with take_launch_timing() before the first launch).
#define W4A4_LAUNCH_FIRST(T, KERNEL, GRID, BLOCK, LDS, STREAM, ...)                                          \
  hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, (uint32_t)(LDS), STREAM, (T).start, nullptr, 0u, __VA_ARGS__)
#define W4A4_LAUNCH_LAST(T, KERNEL, GRID, BLOCK, LDS, STREAM, ...)                                           \
  hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, (uint32_t)(LDS), STREAM, nullptr, (T).stop, 0u, __VA_ARGS__)

}  // namespace w4a4
