// Host-side argument validation of every C-ABI entry point, and the
// device-architecture rule.  Plain C++ (no HIP): the library includes it in
// front of its launches, and the CPU test suite compiles it on its own under
// AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Each check takes the entry point's own arguments (the stream aside) and
// returns W4A4_OK or the status the call must return, with a message in
// `m`.  `noop` is set when the arguments are valid and there is nothing to
// enqueue (zero rows); pointers are not checked then.  The rules are the
// ones declared in include/w4a4.h.
//
// The architecture rule follows page "Rotations for 4-Bit Activations:
// QuaRot, SpinQuant, and Friends", section "Gotchas": online rotation
// kernels are hardware specific, so the library refuses to run on any GPU
// other than the one its code objects are built for (gfx950).
#pragma once

#include <stdint.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "../../include/w4a4.h"

namespace w4a4v {

struct Msg {
  char text[512] = {0};
};

inline w4a4_status say(Msg& m, w4a4_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(m.text, sizeof(m.text), fmt, ap);
  va_end(ap);
  return s;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// The code objects are built for gfx950 only.  `gcn_arch_name` is the
// runtime's architecture string, "gfx950" optionally followed by target
// features (":sramecc+:xnack-"); anything else, including NULL, an empty
// name or a longer processor name that merely starts with "gfx950", is
// refused with W4A4_ERR_DEVICE.
inline w4a4_status arch(const char* gcn_arch_name, int device, Msg& m) {
  static const char kWant[] = "gfx950";
  if (gcn_arch_name == nullptr)
    return say(m, W4A4_ERR_DEVICE, "device %d reports no architecture name", device);
  int i = 0;
  for (; kWant[i] != '\0'; ++i) {
    if (gcn_arch_name[i] != kWant[i]) break;
  }
  const bool ok = kWant[i] == '\0' && (gcn_arch_name[i] == '\0' || gcn_arch_name[i] == ':');
  if (!ok) {
    char shown[64];
    std::snprintf(shown, sizeof(shown), "%s", gcn_arch_name);
    return say(m, W4A4_ERR_DEVICE, "device %d is %s; this library is built for gfx950 only", device,
               shown[0] ? shown : "(unnamed)");
  }
  return W4A4_OK;
}

inline w4a4_status rows_k(int64_t rows, int64_t K, int64_t ld, const char* rn, const char* ldn, Msg& m) {
  if (rows < 0 || rows >= (int64_t(1) << 31))
    return say(m, W4A4_ERR_SHAPE, "%s=%lld out of range [0, 2^31)", rn, (long long)rows);
  if (K < 128 || K % 128 != 0 || K > 16384)
    return say(m, W4A4_ERR_SHAPE, "K=%lld must be a multiple of 128 in [128, 16384]", (long long)K);
  if (ld < K) return say(m, W4A4_ERR_SHAPE, "%s=%lld must be >= K=%lld", ldn, (long long)ld, (long long)K);
  if (ld >= (int64_t(1) << 24)) return say(m, W4A4_ERR_SHAPE, "%s=%lld must be < 2^24 elements", ldn, (long long)ld);
  if (ld % 8 != 0) return say(m, W4A4_ERR_ALIGN, "%s=%lld must be a multiple of 8 elements", ldn, (long long)ld);
  return W4A4_OK;
}

inline w4a4_status had_block_mode(int32_t had_block, Msg& m) {
  if (had_block != W4A4_HAD_FULL && had_block != W4A4_HAD_128)
    return say(m, W4A4_ERR_MODE, "had_block=%d is not W4A4_HAD_FULL or W4A4_HAD_128", had_block);
  return W4A4_OK;
}

inline w4a4_status full_width(int32_t had_block, int64_t K, Msg& m) {
  if (had_block == W4A4_HAD_FULL && !pow2(K))
    return say(m, W4A4_ERR_SHAPE, "full-width Hadamard needs K a power of two, got K=%lld", (long long)K);
  return W4A4_OK;
}

inline w4a4_status rotate_quant_act(const void* x_f16, int64_t M, int64_t K, int64_t ldx, int32_t had_block,
                                    const void* had_signs, int32_t act_mode, const void* codes,
                                    const void* scales, const void* zeros, bool& noop, Msg& m) {
  noop = false;
  if (act_mode != W4A4_ACT_SYM_TOKEN && act_mode != W4A4_ACT_ASYM_G128)
    return say(m, W4A4_ERR_MODE, "act_mode=%d is not W4A4_ACT_SYM_TOKEN or W4A4_ACT_ASYM_G128", act_mode);
  if (w4a4_status s = had_block_mode(had_block, m)) return s;
  if (act_mode == W4A4_ACT_ASYM_G128 && had_block != W4A4_HAD_128)
    return say(m, W4A4_ERR_MODE, "asymmetric per-group mode needs had_block=128");
  if (w4a4_status s = rows_k(M, K, ldx, "M", "ldx", m)) return s;
  if (w4a4_status s = full_width(had_block, K, m)) return s;
  if (M == 0) {
    noop = true;
    return W4A4_OK;
  }
  if (!x_f16 || !codes || !scales) return say(m, W4A4_ERR_NULL, "x_f16, codes and scales must be non-NULL");
  if (act_mode == W4A4_ACT_SYM_TOKEN && zeros) return say(m, W4A4_ERR_MODE, "zeros must be NULL in symmetric mode");
  if (act_mode == W4A4_ACT_ASYM_G128 && !zeros)
    return say(m, W4A4_ERR_MODE, "zeros must be non-NULL in asymmetric mode");
  if (!aligned16(x_f16) || !aligned16(codes) || !aligned16(scales) || (zeros && !aligned16(zeros)) ||
      (had_signs && !aligned16(had_signs)))
    return say(m, W4A4_ERR_ALIGN, "every pointer must be 16-byte aligned");
  return W4A4_OK;
}

inline w4a4_status quant_weight_offline(const void* w_f16, int64_t N, int64_t K, int64_t ldw, int32_t had_block,
                                        const void* had_signs, const void* codes, const void* scales,
                                        const void* gsum, bool& noop, Msg& m) {
  noop = false;
  if (w4a4_status s = had_block_mode(had_block, m)) return s;
  if (w4a4_status s = rows_k(N, K, ldw, "N", "ldw", m)) return s;
  if (w4a4_status s = full_width(had_block, K, m)) return s;
  if (N == 0) {
    noop = true;
    return W4A4_OK;
  }
  if (!w_f16 || !codes || !scales) return say(m, W4A4_ERR_NULL, "w_f16, codes and scales must be non-NULL");
  if (!aligned16(w_f16) || !aligned16(codes) || !aligned16(scales) || (gsum && !aligned16(gsum)) ||
      (had_signs && !aligned16(had_signs)))
    return say(m, W4A4_ERR_ALIGN, "every pointer must be 16-byte aligned");
  return W4A4_OK;
}

inline w4a4_status w4a4_gemm(const void* x_codes, const void* x_scales, const void* x_zeros, int32_t act_mode,
                             const void* w_codes, const void* w_scales, int64_t M, int64_t N, int64_t K,
                             const void* y, int64_t ldy, bool& noop, Msg& m) {
  noop = false;
  if (act_mode != W4A4_ACT_SYM_TOKEN && act_mode != W4A4_ACT_ASYM_G128)
    return say(m, W4A4_ERR_MODE, "act_mode=%d is not W4A4_ACT_SYM_TOKEN or W4A4_ACT_ASYM_G128", act_mode);
  if (M < 0 || M >= (int64_t(1) << 31)) return say(m, W4A4_ERR_SHAPE, "M=%lld out of range [0, 2^31)", (long long)M);
  if (N < 1 || N >= (int64_t(1) << 31)) return say(m, W4A4_ERR_SHAPE, "N=%lld out of range [1, 2^31)", (long long)N);
  if (K < 128 || K % 128 != 0 || K > 131072)
    return say(m, W4A4_ERR_SHAPE, "K=%lld must be a multiple of 128 in [128, 131072]", (long long)K);
  if (ldy < N) return say(m, W4A4_ERR_SHAPE, "ldy=%lld must be >= N=%lld", (long long)ldy, (long long)N);
  if (((M + 127) / 128) * ((N + 127) / 128) >= (int64_t(1) << 31))
    return say(m, W4A4_ERR_SHAPE, "M x N is too large for one launch");
  if (M == 0) {
    noop = true;
    return W4A4_OK;
  }
  if (!x_codes || !x_scales || !w_codes || !w_scales || !y)
    return say(m, W4A4_ERR_NULL, "x_codes, x_scales, w_codes, w_scales and y must be non-NULL");
  if (act_mode == W4A4_ACT_ASYM_G128 && !x_zeros)
    return say(m, W4A4_ERR_MODE, "x_zeros must be non-NULL in asymmetric mode");
  if (!aligned16(x_codes) || !aligned16(x_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(y) || (x_zeros && !aligned16(x_zeros)))
    return say(m, W4A4_ERR_ALIGN, "every pointer must be 16-byte aligned");
  return W4A4_OK;
}

inline w4a4_status kv_rotate_quant4(const void* kv_f16, int64_t B, int64_t H, int64_t S, int64_t D,
                                    int64_t stride_b, int64_t stride_h, int64_t stride_s, const void* had_signs,
                                    const void* codes, const void* scales, const void* zeros, bool& noop,
                                    Msg& m) {
  noop = false;
  if (D != 128) return say(m, W4A4_ERR_SHAPE, "D=%lld must be 128", (long long)D);
  if (B < 0 || H < 0 || S < 0) return say(m, W4A4_ERR_SHAPE, "B, H and S must be >= 0");
  if (H >= (int64_t(1) << 31) || S >= (int64_t(1) << 31) ||
      (B > 0 && H > 0 && S > 0 && (B >= (int64_t(1) << 31) || B * H >= (int64_t(1) << 31) ||
                                   B * H * S >= (int64_t(1) << 31))))
    return say(m, W4A4_ERR_SHAPE, "B*H*S must be < 2^31");
  if (stride_b < 0 || stride_h < 0 || stride_s < 0) return say(m, W4A4_ERR_SHAPE, "strides must be >= 0");
  if (stride_b % 8 || stride_h % 8 || stride_s % 8)
    return say(m, W4A4_ERR_ALIGN, "strides must be multiples of 8 elements");
  if (B == 0 || H == 0 || S == 0) {
    noop = true;
    return W4A4_OK;
  }
  if (!kv_f16 || !codes || !scales || !zeros)
    return say(m, W4A4_ERR_NULL, "kv_f16, codes, scales and zeros must be non-NULL");
  if (!aligned16(kv_f16) || !aligned16(codes) || !aligned16(scales) || !aligned16(zeros) ||
      (had_signs && !aligned16(had_signs)))
    return say(m, W4A4_ERR_ALIGN, "every pointer must be 16-byte aligned");
  return W4A4_OK;
}

inline w4a4_status kv4_attention_decode(const void* q_f16, const void* k_codes, const void* k_scales,
                                        const void* k_zeros, const void* v_codes, const void* v_scales,
                                        const void* v_zeros, int64_t B, int64_t H, int64_t S, int64_t D,
                                        float softmax_scale, const void* had_signs, const void* out, bool& noop,
                                        Msg& m) {
  noop = false;
  if (D != 128) return say(m, W4A4_ERR_SHAPE, "D=%lld must be 128", (long long)D);
  if (B < 0 || H < 0) return say(m, W4A4_ERR_SHAPE, "B and H must be >= 0");
  if (S < 1 || S >= (int64_t(1) << 25)) return say(m, W4A4_ERR_SHAPE, "S=%lld must be in [1, 2^25)", (long long)S);
  if (H >= (int64_t(1) << 31) || (B > 0 && (B >= (int64_t(1) << 31) || B * H >= (int64_t(1) << 31))))
    return say(m, W4A4_ERR_SHAPE, "B*H must be < 2^31");
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
    return say(m, W4A4_ERR_SHAPE, "softmax_scale must be finite and > 0");
  if (B == 0 || H == 0) {
    noop = true;
    return W4A4_OK;
  }
  if (!q_f16 || !k_codes || !k_scales || !k_zeros || !v_codes || !v_scales || !v_zeros || !out)
    return say(m, W4A4_ERR_NULL, "q, the K and V codes, scales and zeros, and out must be non-NULL");
  if (!aligned16(q_f16) || !aligned16(k_codes) || !aligned16(k_scales) || !aligned16(k_zeros) ||
      !aligned16(v_codes) || !aligned16(v_scales) || !aligned16(v_zeros) || !aligned16(out) ||
      (had_signs && !aligned16(had_signs)))
    return say(m, W4A4_ERR_ALIGN, "every pointer must be 16-byte aligned");
  return W4A4_OK;
}

// Token ranges per (batch, head) of the split attention path: enough for
// about 256 workgroups (one per CU), each range at least 512 tokens (64 per
// wave of 8), at most 64; 1 means the single pass.  Measured cold on
// MI355X with the KV workload's value distribution: 1 x 8 heads x 32768
// tokens 230 -> 49 us, 1 x 32 x 4096 43 -> 28 us; with 8 x 32 heads (256
// workgroups already) one range per head is the fastest.
inline int32_t attention_splits(int64_t BH, int64_t S) {
  if (BH <= 0 || S <= 0) return 1;
  int64_t ns = (256 + BH - 1) / BH;
  const int64_t by_len = S / 512;
  if (ns > by_len) ns = by_len;
  if (ns > 64) ns = 64;
  return ns < 2 ? 1 : (int32_t)ns;
}

// Bytes of partial states the split path needs (0: single pass): one state
// of 132 floats per (batch, head, range).
constexpr int64_t kAttnPartBytes = 132 * 4;
inline int64_t attention_workspace_bytes(int64_t BH, int64_t S) {
  const int32_t ns = attention_splits(BH, S);
  return ns > 1 ? BH * ns * kAttnPartBytes : 0;
}

inline w4a4_status kv4_attention_decode_ws(const void* q_f16, const void* k_codes, const void* k_scales,
                                           const void* k_zeros, const void* v_codes, const void* v_scales,
                                           const void* v_zeros, int64_t B, int64_t H, int64_t S, int64_t D,
                                           float softmax_scale, const void* had_signs, const void* out,
                                           const void* workspace, int64_t workspace_bytes, bool& noop, Msg& m) {
  if (w4a4_status s = kv4_attention_decode(q_f16, k_codes, k_scales, k_zeros, v_codes, v_scales, v_zeros, B, H,
                                           S, D, softmax_scale, had_signs, out, noop, m))
    return s;
  if (noop) return W4A4_OK;
  const int64_t need = attention_workspace_bytes(B * H, S);
  if (workspace_bytes < need)
    return say(m, W4A4_ERR_SHAPE, "workspace_bytes=%lld is below the %lld this shape needs (kv4_attention_workspace_bytes)",
               (long long)workspace_bytes, (long long)need);
  if (need > 0 && !workspace) return say(m, W4A4_ERR_NULL, "workspace must be non-NULL for this shape");
  if (need > 0 && !aligned16(workspace)) return say(m, W4A4_ERR_ALIGN, "workspace must be 16-byte aligned");
  return W4A4_OK;
}

// The allocation-free variant keeps the partial states in a static device
// array of scratch_bytes; a shape that needs more is refused.
inline w4a4_status kv4_attention_decode_noalloc(const void* q_f16, const void* k_codes, const void* k_scales,
                                                const void* k_zeros, const void* v_codes, const void* v_scales,
                                                const void* v_zeros, int64_t B, int64_t H, int64_t S, int64_t D,
                                                float softmax_scale, const void* had_signs, const void* out,
                                                int64_t scratch_bytes, bool& noop, Msg& m) {
  if (w4a4_status s = kv4_attention_decode(q_f16, k_codes, k_scales, k_zeros, v_codes, v_scales, v_zeros, B, H,
                                           S, D, softmax_scale, had_signs, out, noop, m))
    return s;
  if (noop) return W4A4_OK;
  const int64_t need = attention_workspace_bytes(B * H, S);
  if (need > scratch_bytes)
    return say(m, W4A4_ERR_SHAPE,
               "this shape needs %lld bytes of partial states, more than the %lld-byte static scratch of "
               "kv4_attention_decode_noalloc (use kv4_attention_decode_ws)",
               (long long)need, (long long)scratch_bytes);
  return W4A4_OK;
}

inline w4a4_status rotate_quant_mxfp4(const void* x_f16, int64_t M, int64_t K, int64_t ldx, int32_t had_block,
                                      const void* had_signs, const void* codes, const void* scales_e8m0,
                                      bool& noop, Msg& m) {
  noop = false;
  if (w4a4_status s = had_block_mode(had_block, m)) return s;
  if (w4a4_status s = rows_k(M, K, ldx, "M", "ldx", m)) return s;
  if (w4a4_status s = full_width(had_block, K, m)) return s;
  if (M == 0) {
    noop = true;
    return W4A4_OK;
  }
  if (!x_f16 || !codes || !scales_e8m0)
    return say(m, W4A4_ERR_NULL, "x_f16, codes and scales_e8m0 must be non-NULL");
  if (!aligned16(x_f16) || !aligned16(codes) || !aligned16(scales_e8m0) || (had_signs && !aligned16(had_signs)))
    return say(m, W4A4_ERR_ALIGN, "every pointer must be 16-byte aligned");
  return W4A4_OK;
}

inline w4a4_status mxfp4_gemm(const void* x_codes, const void* x_scales_e8m0, const void* w_codes,
                              const void* w_scales_e8m0, int64_t M, int64_t N, int64_t K, const void* y,
                              int64_t ldy, bool& noop, Msg& m) {
  noop = false;
  if (M < 0 || M >= (int64_t(1) << 31)) return say(m, W4A4_ERR_SHAPE, "M=%lld out of range [0, 2^31)", (long long)M);
  if (N < 1 || N >= (int64_t(1) << 31)) return say(m, W4A4_ERR_SHAPE, "N=%lld out of range [1, 2^31)", (long long)N);
  if (K < 128 || K % 128 != 0 || K > 131072)
    return say(m, W4A4_ERR_SHAPE, "K=%lld must be a multiple of 128 in [128, 131072]", (long long)K);
  if (ldy < N) return say(m, W4A4_ERR_SHAPE, "ldy=%lld must be >= N=%lld", (long long)ldy, (long long)N);
  if (((M + 63) / 64) * ((N + 127) / 128) >= (int64_t(1) << 31))
    return say(m, W4A4_ERR_SHAPE, "M x N is too large for one launch");
  if (M == 0) {
    noop = true;
    return W4A4_OK;
  }
  if (!x_codes || !x_scales_e8m0 || !w_codes || !w_scales_e8m0 || !y)
    return say(m, W4A4_ERR_NULL, "x_codes, x_scales_e8m0, w_codes, w_scales_e8m0 and y must be non-NULL");
  if (!aligned16(x_codes) || !aligned16(x_scales_e8m0) || !aligned16(w_codes) || !aligned16(w_scales_e8m0) ||
      !aligned16(y))
    return say(m, W4A4_ERR_ALIGN, "every pointer must be 16-byte aligned");
  return W4A4_OK;
}

inline w4a4_status w4a4_decode_fused(const void* x_f16, int64_t M, int64_t K, int64_t ldx, const void* had_signs,
                                     const void* w_codes, const void* w_scales, int64_t N, const void* y,
                                     int64_t ldy, Msg& m) {
  if (M < 1 || M > 16) return say(m, W4A4_ERR_SHAPE, "M=%lld must be in [1, 16]", (long long)M);
  if (K < 128 || K % 128 != 0 || K > 8192)
    return say(m, W4A4_ERR_SHAPE, "K=%lld must be a multiple of 128 in [128, 8192]", (long long)K);
  if (M * K > 65536)
    return say(m, W4A4_ERR_SHAPE, "M*K=%lld exceeds 65536 (the codes of all rows live in LDS)", (long long)(M * K));
  if (ldx < K) return say(m, W4A4_ERR_SHAPE, "ldx=%lld must be >= K=%lld", (long long)ldx, (long long)K);
  if (ldx >= (int64_t(1) << 24)) return say(m, W4A4_ERR_SHAPE, "ldx=%lld must be < 2^24 elements", (long long)ldx);
  if (ldx % 8 != 0) return say(m, W4A4_ERR_ALIGN, "ldx=%lld must be a multiple of 8 elements", (long long)ldx);
  if (N < 1 || N >= (int64_t(1) << 31)) return say(m, W4A4_ERR_SHAPE, "N=%lld out of range [1, 2^31)", (long long)N);
  if (ldy < N) return say(m, W4A4_ERR_SHAPE, "ldy=%lld must be >= N=%lld", (long long)ldy, (long long)N);
  if (!x_f16 || !w_codes || !w_scales || !y)
    return say(m, W4A4_ERR_NULL, "x_f16, w_codes, w_scales and y must be non-NULL");
  if (!aligned16(x_f16) || !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(y) ||
      (had_signs && !aligned16(had_signs)))
    return say(m, W4A4_ERR_ALIGN, "every pointer must be 16-byte aligned");
  return W4A4_OK;
}

}  // namespace w4a4v
