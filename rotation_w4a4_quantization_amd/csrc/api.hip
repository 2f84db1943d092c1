// C ABI entry points: host-side validation, architecture check and launch.
// Nothing here allocates device memory; every call only enqueues kernels on
// the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/w4a4.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;
thread_local w4a4::LaunchTiming g_timing;

// Disarms the timing events when an entry point returns, launched or not.
struct TimingScope {
  ~TimingScope() { g_timing = w4a4::LaunchTiming{}; }
};

w4a4_status fail(w4a4_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

w4a4_status ok() {
  g_err.clear();
  return W4A4_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
int g_dev_state[kMaxDevices];   // 0 unknown, 1 gfx950, -1 other

// The code objects are built for gfx950 only: refuse any other device up
// front instead of failing inside a launch.
w4a4_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(W4A4_ERR_DEVICE, "no HIP device is available");
  if (dev >= kMaxDevices) return fail(W4A4_ERR_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_state[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(W4A4_ERR_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
    g_dev_state[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    if (g_dev_state[dev] == 1 && w4a4::gemm_prepare_device() != hipSuccess) {
      g_dev_state[dev] = 0;
      return fail(W4A4_ERR_DEVICE, "could not raise the LDS limit of the GEMM kernels");
    }
    if (g_dev_state[dev] == -1) {
      return fail(W4A4_ERR_DEVICE, "device %d is %s; this library is built for gfx950 only", dev,
                  prop.gcnArchName);
    }
  }
  if (g_dev_state[dev] != 1)
    return fail(W4A4_ERR_DEVICE, "device %d is not gfx950; this library is built for gfx950 only", dev);
  return W4A4_OK;
}

w4a4_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(W4A4_ERR_DEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

float sym_cdiv(int64_t b) { return (float)(7.0 * std::sqrt((double)b)); }
float asym_cdiv(int64_t b) { return (float)(15.0 * std::sqrt((double)b)); }

w4a4_status check_rows_k(int64_t rows, int64_t K, int64_t ld, const char* rn, const char* ldn) {
  if (rows < 0 || rows >= (int64_t(1) << 31)) return fail(W4A4_ERR_SHAPE, "%s=%lld out of range [0, 2^31)", rn, (long long)rows);
  if (K < 128 || K % 128 != 0 || K > 16384)
    return fail(W4A4_ERR_SHAPE, "K=%lld must be a multiple of 128 in [128, 16384]", (long long)K);
  if (ld < K) return fail(W4A4_ERR_SHAPE, "%s=%lld must be >= K=%lld", ldn, (long long)ld, (long long)K);
  if (ld >= (int64_t(1) << 24)) return fail(W4A4_ERR_SHAPE, "%s=%lld must be < 2^24 elements", ldn, (long long)ld);
  if (ld % 8 != 0) return fail(W4A4_ERR_ALIGN, "%s=%lld must be a multiple of 8 elements", ldn, (long long)ld);
  return W4A4_OK;
}

}  // namespace

namespace w4a4 {
void arm_launch_timing(hipEvent_t start, hipEvent_t stop) { g_timing = LaunchTiming{start, stop}; }
LaunchTiming take_launch_timing() {
  const LaunchTiming t = g_timing;
  g_timing = LaunchTiming{};
  return t;
}
}  // namespace w4a4

extern "C" {

const char* w4a4_last_error(void) { return g_err.c_str(); }

int32_t w4a4_abi_version(void) { return W4A4_ABI_VERSION; }

w4a4_status w4a4_time_next_launch(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(W4A4_ERR_NULL, "start_event and stop_event must both be NULL or both non-NULL");
  w4a4::arm_launch_timing(static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event));
  return ok();
}

w4a4_status rotate_quant_act(const uint16_t* x_f16, int64_t M, int64_t K, int64_t ldx,
                             int32_t had_block, const uint16_t* had_signs, int32_t act_mode,
                             uint8_t* codes, float* scales, uint8_t* zeros, void* stream) {
  TimingScope timing_scope;
  if (act_mode != W4A4_ACT_SYM_TOKEN && act_mode != W4A4_ACT_ASYM_G128)
    return fail(W4A4_ERR_MODE, "act_mode=%d is not W4A4_ACT_SYM_TOKEN or W4A4_ACT_ASYM_G128", act_mode);
  if (had_block != W4A4_HAD_FULL && had_block != W4A4_HAD_128)
    return fail(W4A4_ERR_MODE, "had_block=%d is not W4A4_HAD_FULL or W4A4_HAD_128", had_block);
  if (act_mode == W4A4_ACT_ASYM_G128 && had_block != W4A4_HAD_128)
    return fail(W4A4_ERR_MODE, "asymmetric per-group mode needs had_block=128");
  if (w4a4_status s = check_rows_k(M, K, ldx, "M", "ldx")) return s;
  if (had_block == W4A4_HAD_FULL && !pow2(K))
    return fail(W4A4_ERR_SHAPE, "full-width Hadamard needs K a power of two, got K=%lld", (long long)K);
  if (M == 0) return ok();   // nothing is read or written: pointers may be NULL
  if (!x_f16 || !codes || !scales) return fail(W4A4_ERR_NULL, "x_f16, codes and scales must be non-NULL");
  if (act_mode == W4A4_ACT_SYM_TOKEN && zeros)
    return fail(W4A4_ERR_MODE, "zeros must be NULL in symmetric mode");
  if (act_mode == W4A4_ACT_ASYM_G128 && !zeros)
    return fail(W4A4_ERR_MODE, "zeros must be non-NULL in asymmetric mode");
  if (!aligned16(x_f16) || !aligned16(codes) || !aligned16(scales) || (zeros && !aligned16(zeros)) ||
      (had_signs && !aligned16(had_signs)))
    return fail(W4A4_ERR_ALIGN, "every pointer must be 16-byte aligned");
  if (w4a4_status s = check_device()) return s;

  w4a4::RQParams p{};
  p.x = x_f16;
  p.signs = had_signs;
  p.codes = codes;
  p.scales = scales;
  p.zeros = zeros;
  p.rows = M;
  p.ss = ldx;
  p.K = (int32_t)K;
  const int64_t b = had_block == W4A4_HAD_FULL ? K : 128;
  const bool asym = act_mode == W4A4_ACT_ASYM_G128;
  p.cdiv = asym ? asym_cdiv(b) : sym_cdiv(b);
  return launched(w4a4::launch_rotate_quant(p, asym ? w4a4::kModeAsym : w4a4::kModeSym,
                                            had_block == W4A4_HAD_FULL, false, false,
                                            (hipStream_t)stream),
                  "rotate_quant_act");
}

w4a4_status quant_weight_offline(const uint16_t* w_f16, int64_t N, int64_t K, int64_t ldw,
                                 int32_t had_block, const uint16_t* had_signs, uint8_t* codes,
                                 float* scales, int32_t* gsum, void* stream) {
  TimingScope timing_scope;
  if (had_block != W4A4_HAD_FULL && had_block != W4A4_HAD_128)
    return fail(W4A4_ERR_MODE, "had_block=%d is not W4A4_HAD_FULL or W4A4_HAD_128", had_block);
  if (w4a4_status s = check_rows_k(N, K, ldw, "N", "ldw")) return s;
  if (had_block == W4A4_HAD_FULL && !pow2(K))
    return fail(W4A4_ERR_SHAPE, "full-width Hadamard needs K a power of two, got K=%lld", (long long)K);
  if (N == 0) return ok();   // nothing is read or written: pointers may be NULL
  if (!w_f16 || !codes || !scales) return fail(W4A4_ERR_NULL, "w_f16, codes and scales must be non-NULL");
  if (!aligned16(w_f16) || !aligned16(codes) || !aligned16(scales) || (gsum && !aligned16(gsum)) ||
      (had_signs && !aligned16(had_signs)))
    return fail(W4A4_ERR_ALIGN, "every pointer must be 16-byte aligned");
  if (w4a4_status s = check_device()) return s;

  w4a4::RQParams p{};
  p.x = w_f16;
  p.signs = had_signs;
  p.codes = codes;
  p.scales = scales;
  p.gsum = gsum;
  p.rows = N;
  p.ss = ldw;
  p.K = (int32_t)K;
  p.cdiv = sym_cdiv(had_block == W4A4_HAD_FULL ? K : 128);
  return launched(w4a4::launch_rotate_quant(p, w4a4::kModeSym, had_block == W4A4_HAD_FULL,
                                            gsum != nullptr, false, (hipStream_t)stream),
                  "quant_weight_offline");
}

w4a4_status w4a4_decode_fused(const uint16_t* x_f16, int64_t M, int64_t K, int64_t ldx,
                              const uint16_t* had_signs, const uint8_t* w_codes, const float* w_scales,
                              int64_t N, float* y, int64_t ldy, void* stream) {
  TimingScope timing_scope;
  if (M < 1 || M > 16) return fail(W4A4_ERR_SHAPE, "M=%lld must be in [1, 16]", (long long)M);
  if (K < 128 || K % 128 != 0 || K > 8192)
    return fail(W4A4_ERR_SHAPE, "K=%lld must be a multiple of 128 in [128, 8192]", (long long)K);
  if (M * K > 65536)
    return fail(W4A4_ERR_SHAPE, "M*K=%lld exceeds 65536 (the codes of all rows live in LDS)", (long long)(M * K));
  if (ldx < K) return fail(W4A4_ERR_SHAPE, "ldx=%lld must be >= K=%lld", (long long)ldx, (long long)K);
  if (ldx >= (int64_t(1) << 24)) return fail(W4A4_ERR_SHAPE, "ldx=%lld must be < 2^24 elements", (long long)ldx);
  if (ldx % 8 != 0) return fail(W4A4_ERR_ALIGN, "ldx=%lld must be a multiple of 8 elements", (long long)ldx);
  if (N < 1 || N >= (int64_t(1) << 31)) return fail(W4A4_ERR_SHAPE, "N=%lld out of range [1, 2^31)", (long long)N);
  if (ldy < N) return fail(W4A4_ERR_SHAPE, "ldy=%lld must be >= N=%lld", (long long)ldy, (long long)N);
  if (!x_f16 || !w_codes || !w_scales || !y)
    return fail(W4A4_ERR_NULL, "x_f16, w_codes, w_scales and y must be non-NULL");
  if (!aligned16(x_f16) || !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(y) ||
      (had_signs && !aligned16(had_signs)))
    return fail(W4A4_ERR_ALIGN, "every pointer must be 16-byte aligned");
  if (w4a4_status s = check_device()) return s;

  w4a4::FusedDecodeParams p{};
  p.x = x_f16;
  p.signs = had_signs;
  p.wq = w_codes;
  p.ws = w_scales;
  p.y = y;
  p.N = N;
  p.ldy = ldy;
  p.M = (int32_t)M;
  p.K = (int32_t)K;
  p.ldx = (int32_t)ldx;
  p.cdiv = sym_cdiv(128);
  return launched(w4a4::launch_decode_fused(p, (hipStream_t)stream), "w4a4_decode_fused");
}

w4a4_status rotate_quant_mxfp4(const uint16_t* x_f16, int64_t M, int64_t K, int64_t ldx,
                               int32_t had_block, const uint16_t* had_signs, uint8_t* codes,
                               uint8_t* scales_e8m0, void* stream) {
  TimingScope timing_scope;
  if (had_block != W4A4_HAD_FULL && had_block != W4A4_HAD_128)
    return fail(W4A4_ERR_MODE, "had_block=%d is not W4A4_HAD_FULL or W4A4_HAD_128", had_block);
  if (w4a4_status s = check_rows_k(M, K, ldx, "M", "ldx")) return s;
  if (had_block == W4A4_HAD_FULL && !pow2(K))
    return fail(W4A4_ERR_SHAPE, "full-width Hadamard needs K a power of two, got K=%lld", (long long)K);
  if (M == 0) return ok();   // nothing is read or written: pointers may be NULL
  if (!x_f16 || !codes || !scales_e8m0) return fail(W4A4_ERR_NULL, "x_f16, codes and scales_e8m0 must be non-NULL");
  if (!aligned16(x_f16) || !aligned16(codes) || !aligned16(scales_e8m0) || (had_signs && !aligned16(had_signs)))
    return fail(W4A4_ERR_ALIGN, "every pointer must be 16-byte aligned");
  if (w4a4_status s = check_device()) return s;

  w4a4::RQParams p{};
  p.x = x_f16;
  p.signs = had_signs;
  p.codes = codes;
  p.mx_scales = scales_e8m0;
  p.rows = M;
  p.ss = ldx;
  p.K = (int32_t)K;
  p.cdiv = (float)(1.0 / std::sqrt((double)(had_block == W4A4_HAD_FULL ? K : 128)));
  return launched(w4a4::launch_rotate_quant(p, w4a4::kModeMx, had_block == W4A4_HAD_FULL, false, false,
                                            (hipStream_t)stream),
                  "rotate_quant_mxfp4");
}

w4a4_status mxfp4_gemm(const uint8_t* x_codes, const uint8_t* x_scales_e8m0, const uint8_t* w_codes,
                       const uint8_t* w_scales_e8m0, int64_t M, int64_t N, int64_t K, float* y,
                       int64_t ldy, void* stream) {
  TimingScope timing_scope;
  if (M < 0 || M >= (int64_t(1) << 31)) return fail(W4A4_ERR_SHAPE, "M=%lld out of range [0, 2^31)", (long long)M);
  if (N < 1 || N >= (int64_t(1) << 31)) return fail(W4A4_ERR_SHAPE, "N=%lld out of range [1, 2^31)", (long long)N);
  if (K < 128 || K % 128 != 0 || K > 131072)
    return fail(W4A4_ERR_SHAPE, "K=%lld must be a multiple of 128 in [128, 131072]", (long long)K);
  if (ldy < N) return fail(W4A4_ERR_SHAPE, "ldy=%lld must be >= N=%lld", (long long)ldy, (long long)N);
  if (((M + 63) / 64) * ((N + 127) / 128) >= (int64_t(1) << 31))
    return fail(W4A4_ERR_SHAPE, "M x N is too large for one launch");
  if (M == 0) return ok();   // nothing is read or written: pointers may be NULL
  if (!x_codes || !x_scales_e8m0 || !w_codes || !w_scales_e8m0 || !y)
    return fail(W4A4_ERR_NULL, "x_codes, x_scales_e8m0, w_codes, w_scales_e8m0 and y must be non-NULL");
  if (!aligned16(x_codes) || !aligned16(x_scales_e8m0) || !aligned16(w_codes) || !aligned16(w_scales_e8m0) ||
      !aligned16(y))
    return fail(W4A4_ERR_ALIGN, "every pointer must be 16-byte aligned");
  if (w4a4_status s = check_device()) return s;

  w4a4::MxGemmParams p{};
  p.xq = x_codes;
  p.xe = x_scales_e8m0;
  p.wq = w_codes;
  p.we = w_scales_e8m0;
  p.y = y;
  p.M = M;
  p.N = N;
  p.ldy = ldy;
  p.K = (int32_t)K;
  return launched(w4a4::launch_mx_gemm(p, (hipStream_t)stream), "mxfp4_gemm");
}

w4a4_status w4a4_gemm(const uint8_t* x_codes, const float* x_scales, const uint8_t* x_zeros,
                      int32_t act_mode, const uint8_t* w_codes, const float* w_scales,
                      const int32_t* w_gsum, int64_t M, int64_t N, int64_t K, float* y, int64_t ldy,
                      void* stream) {
  TimingScope timing_scope;
  (void)w_gsum;   // zero-points are removed before the product; group sums are not needed
  if (act_mode != W4A4_ACT_SYM_TOKEN && act_mode != W4A4_ACT_ASYM_G128)
    return fail(W4A4_ERR_MODE, "act_mode=%d is not W4A4_ACT_SYM_TOKEN or W4A4_ACT_ASYM_G128", act_mode);
  if (M < 0 || M >= (int64_t(1) << 31)) return fail(W4A4_ERR_SHAPE, "M=%lld out of range [0, 2^31)", (long long)M);
  if (N < 1 || N >= (int64_t(1) << 31)) return fail(W4A4_ERR_SHAPE, "N=%lld out of range [1, 2^31)", (long long)N);
  if (K < 128 || K % 128 != 0 || K > 131072)
    return fail(W4A4_ERR_SHAPE, "K=%lld must be a multiple of 128 in [128, 131072]", (long long)K);
  if (ldy < N) return fail(W4A4_ERR_SHAPE, "ldy=%lld must be >= N=%lld", (long long)ldy, (long long)N);
  if (((M + 127) / 128) * ((N + 127) / 128) >= (int64_t(1) << 31))
    return fail(W4A4_ERR_SHAPE, "M x N is too large for one launch");
  if (M == 0) return ok();   // nothing is read or written: pointers may be NULL
  if (!x_codes || !x_scales || !w_codes || !w_scales || !y)
    return fail(W4A4_ERR_NULL, "x_codes, x_scales, w_codes, w_scales and y must be non-NULL");
  if (act_mode == W4A4_ACT_ASYM_G128 && !x_zeros)
    return fail(W4A4_ERR_MODE, "x_zeros must be non-NULL in asymmetric mode");
  if (!aligned16(x_codes) || !aligned16(x_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(y) || (x_zeros && !aligned16(x_zeros)))
    return fail(W4A4_ERR_ALIGN, "every pointer must be 16-byte aligned");
  if (w4a4_status s = check_device()) return s;

  w4a4::GemmParams p{};
  p.xq = x_codes;
  p.xs = x_scales;
  p.xz = x_zeros;
  p.wq = w_codes;
  p.ws = w_scales;
  p.y = y;
  p.M = M;
  p.N = N;
  p.ldy = ldy;
  p.K = (int32_t)K;
  return launched(w4a4::launch_gemm(p, act_mode == W4A4_ACT_ASYM_G128 ? w4a4::kModeAsym : w4a4::kModeSym,
                                    (hipStream_t)stream),
                  "w4a4_gemm");
}

w4a4_status kv_rotate_quant4(const uint16_t* kv_f16, int64_t B, int64_t H, int64_t S, int64_t D,
                             int64_t stride_b, int64_t stride_h, int64_t stride_s,
                             const uint16_t* had_signs, uint8_t* codes, float* scales,
                             uint8_t* zeros, void* stream) {
  TimingScope timing_scope;
  if (D != 128) return fail(W4A4_ERR_SHAPE, "D=%lld must be 128", (long long)D);
  if (B < 0 || H < 0 || S < 0) return fail(W4A4_ERR_SHAPE, "B, H and S must be >= 0");
  if (H >= (int64_t(1) << 31) || S >= (int64_t(1) << 31) ||
      (B > 0 && H > 0 && S > 0 && B * H * S >= (int64_t(1) << 31)))
    return fail(W4A4_ERR_SHAPE, "B*H*S must be < 2^31");
  if (stride_b < 0 || stride_h < 0 || stride_s < 0) return fail(W4A4_ERR_SHAPE, "strides must be >= 0");
  if (stride_b % 8 || stride_h % 8 || stride_s % 8)
    return fail(W4A4_ERR_ALIGN, "strides must be multiples of 8 elements");
  const int64_t rows = B * H * S;
  if (rows == 0) return ok();   // nothing is read or written: pointers may be NULL
  if (!kv_f16 || !codes || !scales || !zeros)
    return fail(W4A4_ERR_NULL, "kv_f16, codes, scales and zeros must be non-NULL");
  if (!aligned16(kv_f16) || !aligned16(codes) || !aligned16(scales) || !aligned16(zeros) ||
      (had_signs && !aligned16(had_signs)))
    return fail(W4A4_ERR_ALIGN, "every pointer must be 16-byte aligned");
  if (w4a4_status s = check_device()) return s;

  w4a4::RQParams p{};
  p.x = kv_f16;
  p.signs = had_signs;
  p.codes = codes;
  p.scales = scales;
  p.zeros = zeros;
  p.rows = rows;
  p.K = 128;
  p.cdiv = asym_cdiv(128);
  const bool dense = stride_s == 128 && stride_h == S * 128 && stride_b == H * S * 128;
  if (dense) {
    p.ss = 128;
  } else {
    p.ss = stride_s;
    p.sh = stride_h;
    p.sb = stride_b;
    p.S = (uint32_t)S;
    p.H = (uint32_t)H;
  }
  return launched(w4a4::launch_rotate_quant(p, w4a4::kModeAsym, false, false, !dense, (hipStream_t)stream),
                  "kv_rotate_quant4");
}

w4a4_status kv4_attention_decode(const uint16_t* q_f16, const uint8_t* k_codes, const float* k_scales,
                                 const uint8_t* k_zeros, const uint8_t* v_codes, const float* v_scales,
                                 const uint8_t* v_zeros, int64_t B, int64_t H, int64_t S, int64_t D,
                                 float softmax_scale, const uint16_t* had_signs, float* out,
                                 void* stream) {
  TimingScope timing_scope;
  if (D != 128) return fail(W4A4_ERR_SHAPE, "D=%lld must be 128", (long long)D);
  if (B < 0 || H < 0) return fail(W4A4_ERR_SHAPE, "B and H must be >= 0");
  if (S < 1 || S >= (int64_t(1) << 25)) return fail(W4A4_ERR_SHAPE, "S=%lld must be in [1, 2^25)", (long long)S);
  if (H >= (int64_t(1) << 31) || (B > 0 && B * H >= (int64_t(1) << 31)))
    return fail(W4A4_ERR_SHAPE, "B*H must be < 2^31");
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
    return fail(W4A4_ERR_SHAPE, "softmax_scale must be finite and > 0");
  const int64_t bh = B * H;
  if (bh == 0) return ok();   // nothing is read or written: pointers may be NULL
  if (!q_f16 || !k_codes || !k_scales || !k_zeros || !v_codes || !v_scales || !v_zeros || !out)
    return fail(W4A4_ERR_NULL, "q, the K and V codes, scales and zeros, and out must be non-NULL");
  if (!aligned16(q_f16) || !aligned16(k_codes) || !aligned16(k_scales) || !aligned16(k_zeros) ||
      !aligned16(v_codes) || !aligned16(v_scales) || !aligned16(v_zeros) || !aligned16(out) ||
      (had_signs && !aligned16(had_signs)))
    return fail(W4A4_ERR_ALIGN, "every pointer must be 16-byte aligned");
  if (w4a4_status s = check_device()) return s;

  w4a4::AttnParams p{};
  p.q = q_f16;
  p.k_codes = k_codes;
  p.k_scales = k_scales;
  p.k_zeros = k_zeros;
  p.v_codes = v_codes;
  p.v_scales = v_scales;
  p.v_zeros = v_zeros;
  p.signs = had_signs;
  p.out = out;
  p.BH = bh;
  p.S = S;
  p.scale2 = (float)((double)softmax_scale * 1.4426950408889634);
  return launched(w4a4::launch_kv4_attention(p, (hipStream_t)stream), "kv4_attention_decode");
}

}  // extern "C"
