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
#include "validate.h"

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

// A validation verdict: an error status keeps its message, W4A4_OK passes.
w4a4_status verdict(w4a4_status s, const w4a4v::Msg& m) {
  if (s != W4A4_OK) g_err = m.text;
  return s;
}

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
int g_dev_state[kMaxDevices];   // 0 unknown, 1 gfx950, -1 other

// Partial states of kv4_attention_decode_noalloc: a file-scope device array,
// one copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device
// address); it uses the address hipGetSymbolAddress gives for each device.
// The split path needs at most 510 states of 528 bytes (269,280 bytes).
constexpr int64_t kScratchBytes = int64_t(512) << 10;
static __device__ __align__(256) float scratch[kScratchBytes / 4];
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device (under g_dev_mu)

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
    w4a4v::Msg m;
    if (w4a4v::arch(prop.gcnArchName, dev, m) != W4A4_OK) {
      g_dev_state[dev] = -1;
      return verdict(W4A4_ERR_DEVICE, m);
    }
    if (w4a4::gemm_prepare_device() != hipSuccess)
      return fail(W4A4_ERR_DEVICE, "GEMM set-up failed on device %d", dev);
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(W4A4_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch[dev] = ptr;
    g_dev_state[dev] = 1;
  }
  if (g_dev_state[dev] != 1)
    return fail(W4A4_ERR_DEVICE, "device %d is not gfx950; this library is built for gfx950 only", dev);
  return W4A4_OK;
}

// The current device's address of `scratch` (check_device() has set it).
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  return g_scratch[dev];
}

w4a4_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(W4A4_ERR_DEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

float sym_cdiv(int64_t b) { return (float)(7.0 * std::sqrt((double)b)); }
float asym_cdiv(int64_t b) { return (float)(15.0 * std::sqrt((double)b)); }

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
  w4a4v::Msg m;
  bool noop = false;
  if (w4a4_status s = w4a4v::rotate_quant_act(x_f16, M, K, ldx, had_block, had_signs, act_mode, codes, scales,
                                              zeros, noop, m))
    return verdict(s, m);
  if (noop) return ok();
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
  w4a4v::Msg m;
  bool noop = false;
  if (w4a4_status s = w4a4v::quant_weight_offline(w_f16, N, K, ldw, had_block, had_signs, codes, scales, gsum,
                                                  noop, m))
    return verdict(s, m);
  if (noop) return ok();
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
  w4a4v::Msg m;
  if (w4a4_status s = w4a4v::w4a4_decode_fused(x_f16, M, K, ldx, had_signs, w_codes, w_scales, N, y, ldy, m))
    return verdict(s, m);
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
  w4a4v::Msg m;
  bool noop = false;
  if (w4a4_status s = w4a4v::rotate_quant_mxfp4(x_f16, M, K, ldx, had_block, had_signs, codes, scales_e8m0, noop,
                                                m))
    return verdict(s, m);
  if (noop) return ok();
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
  w4a4v::Msg m;
  bool noop = false;
  if (w4a4_status s = w4a4v::mxfp4_gemm(x_codes, x_scales_e8m0, w_codes, w_scales_e8m0, M, N, K, y, ldy, noop, m))
    return verdict(s, m);
  if (noop) return ok();
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
  w4a4v::Msg m;
  bool noop = false;
  if (w4a4_status s = w4a4v::w4a4_gemm(x_codes, x_scales, x_zeros, act_mode, w_codes, w_scales, M, N, K, y, ldy,
                                       noop, m))
    return verdict(s, m);
  if (noop) return ok();
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
  w4a4v::Msg m;
  bool noop = false;
  if (w4a4_status s = w4a4v::kv_rotate_quant4(kv_f16, B, H, S, D, stride_b, stride_h, stride_s, had_signs, codes,
                                              scales, zeros, noop, m))
    return verdict(s, m);
  if (noop) return ok();
  const int64_t rows = B * H * S;
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
  w4a4v::Msg m;
  bool noop = false;
  if (w4a4_status s = w4a4v::kv4_attention_decode(q_f16, k_codes, k_scales, k_zeros, v_codes, v_scales, v_zeros, B,
                                                  H, S, D, softmax_scale, had_signs, out, noop, m))
    return verdict(s, m);
  if (noop) return ok();
  const int64_t bh = B * H;
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

int64_t kv4_attention_workspace_bytes(int64_t B, int64_t H, int64_t S) {
  if (B < 0 || H < 0 || S < 1 || S >= (int64_t(1) << 25) || H >= (int64_t(1) << 31) ||
      (B > 0 && (B >= (int64_t(1) << 31) || B * H >= (int64_t(1) << 31)))) {
    fail(W4A4_ERR_SHAPE, "B=%lld, H=%lld, S=%lld out of range", (long long)B, (long long)H, (long long)S);
    return -1;
  }
  ok();
  return w4a4v::attention_workspace_bytes(B * H, S);
}

w4a4_status kv4_attention_decode_ws(const uint16_t* q_f16, const uint8_t* k_codes, const float* k_scales,
                                    const uint8_t* k_zeros, const uint8_t* v_codes, const float* v_scales,
                                    const uint8_t* v_zeros, int64_t B, int64_t H, int64_t S, int64_t D,
                                    float softmax_scale, const uint16_t* had_signs, float* out, void* workspace,
                                    int64_t workspace_bytes, void* stream) {
  static_assert(w4a4::kAttnPartFloats * 4 == w4a4v::kAttnPartBytes, "partial-state size");
  TimingScope timing_scope;
  w4a4v::Msg m;
  bool noop = false;
  if (w4a4_status s = w4a4v::kv4_attention_decode_ws(q_f16, k_codes, k_scales, k_zeros, v_codes, v_scales, v_zeros,
                                                     B, H, S, D, softmax_scale, had_signs, out, workspace,
                                                     workspace_bytes, noop, m))
    return verdict(s, m);
  if (noop) return ok();
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
  p.BH = B * H;
  p.S = S;
  p.scale2 = (float)((double)softmax_scale * 1.4426950408889634);
  p.nsplit = w4a4v::attention_splits(p.BH, S);
  p.part = static_cast<float*>(workspace);
  return launched(w4a4::launch_kv4_attention_split(p, (hipStream_t)stream), "kv4_attention_decode_ws");
}

w4a4_status kv4_attention_decode_noalloc(const uint16_t* q_f16, const uint8_t* k_codes, const float* k_scales,
                                         const uint8_t* k_zeros, const uint8_t* v_codes, const float* v_scales,
                                         const uint8_t* v_zeros, int64_t B, int64_t H, int64_t S, int64_t D,
                                         float softmax_scale, const uint16_t* had_signs, float* out, void* stream) {
  TimingScope timing_scope;
  w4a4v::Msg m;
  bool noop = false;
  if (w4a4_status s = w4a4v::kv4_attention_decode_noalloc(q_f16, k_codes, k_scales, k_zeros, v_codes, v_scales,
                                                          v_zeros, B, H, S, D, softmax_scale, had_signs, out,
                                                          kScratchBytes, noop, m))
    return verdict(s, m);
  if (noop) return ok();
  if (w4a4_status s = check_device()) return s;
  void* part = device_scratch();
  if (!part) return fail(W4A4_ERR_DEVICE, "no scratch address for the current device");

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
  p.BH = B * H;
  p.S = S;
  p.scale2 = (float)((double)softmax_scale * 1.4426950408889634);
  p.nsplit = w4a4v::attention_splits(p.BH, S);
  p.part = static_cast<float*>(part);
  return launched(w4a4::launch_kv4_attention_split(p, (hipStream_t)stream), "kv4_attention_decode_noalloc");
}

}  // extern "C"
