// CPU self-test of the host validation unit (validate.h): every rule of
// every entry point, the architecture rule (including the wrong-architecture
// branch, which no CPU run of the library can reach), and size arguments
// large enough to overflow a naive product.  Built and run by
// tests/test_validate_native.py under AddressSanitizer and
// UndefinedBehaviorSanitizer; prints "validate selftest ok" and exits 0 when
// every case gives the expected status.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>
#include <string>

#include "validate.h"

namespace {

int g_fail = 0, g_cases = 0;

void expect(const char* what, w4a4_status got, w4a4_status want, const w4a4v::Msg& m) {
  ++g_cases;
  if (got != want) {
    ++g_fail;
    std::printf("FAIL %s: status %d, want %d (%s)\n", what, (int)got, (int)want, m.text);
  } else if (got != W4A4_OK && m.text[0] == '\0') {
    ++g_fail;
    std::printf("FAIL %s: error status without a message\n", what);
  }
}

void expect_noop(const char* what, bool noop, bool want) {
  ++g_cases;
  if (noop != want) {
    ++g_fail;
    std::printf("FAIL %s: noop %d, want %d\n", what, (int)noop, (int)want);
  }
}

alignas(16) unsigned char g_buf[256];
const void* A = g_buf;            // aligned, non-NULL
const void* U = g_buf + 2;        // misaligned
const void* Z = nullptr;
constexpr int64_t BIG = int64_t(1) << 31;

void arch_cases() {
  struct Case { const char* name; w4a4_status want; } cases[] = {
      {"gfx950", W4A4_OK},
      {"gfx950:sramecc+:xnack-", W4A4_OK},
      {"gfx950:xnack+", W4A4_OK},
      {"gfx942", W4A4_ERR_DEVICE},
      {"gfx942:sramecc+:xnack-", W4A4_ERR_DEVICE},
      {"gfx90a", W4A4_ERR_DEVICE},
      {"gfx9500", W4A4_ERR_DEVICE},
      {"gfx95", W4A4_ERR_DEVICE},
      {"GFX950", W4A4_ERR_DEVICE},
      {"", W4A4_ERR_DEVICE},
  };
  for (const Case& c : cases) {
    w4a4v::Msg m;
    std::string what = std::string("arch '") + c.name + "'";
    expect(what.c_str(), w4a4v::arch(c.name, 3, m), c.want, m);
    if (c.want != W4A4_OK && std::strstr(m.text, "gfx950 only") == nullptr) {
      ++g_fail;
      std::printf("FAIL %s: message does not name the supported architecture: %s\n", what.c_str(), m.text);
    }
  }
  w4a4v::Msg m;
  expect("arch NULL", w4a4v::arch(nullptr, 0, m), W4A4_ERR_DEVICE, m);
  // a name longer than the message buffer is truncated, not overrun
  std::string long_name(2000, 'x');
  expect("arch long name", w4a4v::arch(long_name.c_str(), 1, m), W4A4_ERR_DEVICE, m);
  if (std::strlen(m.text) >= sizeof(m.text)) {
    ++g_fail;
    std::printf("FAIL arch long name: message not terminated\n");
  }
}

void rotate_cases() {
  struct C { const char* what; const void* x; int64_t M, K, ldx; int32_t hb; const void* sg; int32_t mode;
             const void *c, *s, *z; w4a4_status want; bool noop; };
  const C cases[] = {
      {"ok sym 128", A, 4, 128, 128, 128, Z, 0, A, A, Z, W4A4_OK, false},
      {"ok sym full", A, 4, 4096, 4096, 0, A, 0, A, A, Z, W4A4_OK, false},
      {"ok asym", A, 4, 256, 264, 128, Z, 1, A, A, A, W4A4_OK, false},
      {"null x", Z, 4, 128, 128, 128, Z, 0, A, A, Z, W4A4_ERR_NULL, false},
      {"null codes", A, 4, 128, 128, 128, Z, 0, Z, A, Z, W4A4_ERR_NULL, false},
      {"null scales", A, 4, 128, 128, 128, Z, 0, A, Z, Z, W4A4_ERR_NULL, false},
      {"K % 128", A, 4, 100, 128, 128, Z, 0, A, A, Z, W4A4_ERR_SHAPE, false},
      {"K zero", A, 4, 0, 128, 128, Z, 0, A, A, Z, W4A4_ERR_SHAPE, false},
      {"K > 16384", A, 4, 32768, 32768, 128, Z, 0, A, A, Z, W4A4_ERR_SHAPE, false},
      {"M < 0", A, -1, 128, 128, 128, Z, 0, A, A, Z, W4A4_ERR_SHAPE, false},
      {"M >= 2^31", A, BIG, 128, 128, 128, Z, 0, A, A, Z, W4A4_ERR_SHAPE, false},
      {"ldx < K", A, 4, 256, 128, 128, Z, 0, A, A, Z, W4A4_ERR_SHAPE, false},
      {"ldx >= 2^24", A, 4, 128, int64_t(1) << 24, 128, Z, 0, A, A, Z, W4A4_ERR_SHAPE, false},
      {"full needs 2^p", A, 4, 384, 384, 0, Z, 0, A, A, Z, W4A4_ERR_SHAPE, false},
      {"ldx % 8", A, 4, 128, 132, 128, Z, 0, A, A, Z, W4A4_ERR_ALIGN, false},
      {"x misaligned", U, 4, 128, 128, 128, Z, 0, A, A, Z, W4A4_ERR_ALIGN, false},
      {"signs misaligned", A, 4, 128, 128, 128, U, 0, A, A, Z, W4A4_ERR_ALIGN, false},
      {"zeros misaligned", A, 4, 128, 128, 128, Z, 1, A, A, U, W4A4_ERR_ALIGN, false},
      {"had_block 64", A, 4, 128, 128, 64, Z, 0, A, A, Z, W4A4_ERR_MODE, false},
      {"act_mode 2", A, 4, 128, 128, 128, Z, 2, A, A, Z, W4A4_ERR_MODE, false},
      {"zeros in sym", A, 4, 128, 128, 128, Z, 0, A, A, A, W4A4_ERR_MODE, false},
      {"no zeros in asym", A, 4, 128, 128, 128, Z, 1, A, A, Z, W4A4_ERR_MODE, false},
      {"asym + full", A, 4, 256, 256, 0, Z, 1, A, A, A, W4A4_ERR_MODE, false},
      {"M == 0", A, 0, 128, 128, 128, Z, 0, A, A, Z, W4A4_OK, true},
      {"M == 0 NULL buffers", Z, 0, 128, 128, 128, Z, 0, Z, Z, Z, W4A4_OK, true},
      {"M == 0 sizes checked", Z, 0, 100, 128, 128, Z, 0, Z, Z, Z, W4A4_ERR_SHAPE, false},
  };
  for (const C& c : cases) {
    w4a4v::Msg m;
    bool noop = true;
    std::string what = std::string("rotate_quant_act ") + c.what;
    expect(what.c_str(), w4a4v::rotate_quant_act(c.x, c.M, c.K, c.ldx, c.hb, c.sg, c.mode, c.c, c.s, c.z, noop, m),
           c.want, m);
    expect_noop(what.c_str(), noop, c.noop);
    // the MXFP4 rotate call shares the rotate rules that do not involve modes or zeros
    if (c.mode == 0 && c.z == Z) {
      w4a4v::Msg m2;
      bool noop2 = true;
      std::string w2 = std::string("rotate_quant_mxfp4 ") + c.what;
      expect(w2.c_str(), w4a4v::rotate_quant_mxfp4(c.x, c.M, c.K, c.ldx, c.hb, c.sg, c.c, c.s, noop2, m2), c.want,
             m2);
      expect_noop(w2.c_str(), noop2, c.noop);
    }
  }
}

void weight_cases() {
  struct C { const char* what; const void* w; int64_t N, K, ldw; int32_t hb; const void *sg, *c, *s, *g;
             w4a4_status want; bool noop; };
  const C cases[] = {
      {"ok", A, 8, 256, 256, 128, Z, A, A, A, W4A4_OK, false},
      {"ok no gsum", A, 8, 256, 256, 0, Z, A, A, Z, W4A4_OK, false},
      {"gsum misaligned", A, 8, 256, 256, 128, Z, A, A, U, W4A4_ERR_ALIGN, false},
      {"null w", Z, 8, 256, 256, 128, Z, A, A, A, W4A4_ERR_NULL, false},
      {"full non pow2", A, 8, 384, 384, 0, Z, A, A, A, W4A4_ERR_SHAPE, false},
      {"had 256", A, 8, 256, 256, 256, Z, A, A, A, W4A4_ERR_MODE, false},
      {"N == 0", Z, 0, 256, 256, 128, Z, Z, Z, Z, W4A4_OK, true},
  };
  for (const C& c : cases) {
    w4a4v::Msg m;
    bool noop = true;
    std::string what = std::string("quant_weight_offline ") + c.what;
    expect(what.c_str(), w4a4v::quant_weight_offline(c.w, c.N, c.K, c.ldw, c.hb, c.sg, c.c, c.s, c.g, noop, m),
           c.want, m);
    expect_noop(what.c_str(), noop, c.noop);
  }
}

void gemm_cases() {
  struct C { const char* what; const void *xc, *xs, *xz; int32_t mode; const void *wc, *ws;
             int64_t M, N, K; const void* y; int64_t ldy; w4a4_status want; bool noop; };
  const C cases[] = {
      {"ok sym", A, A, Z, 0, A, A, 16, 64, 256, A, 64, W4A4_OK, false},
      {"ok asym", A, A, A, 1, A, A, 16, 64, 256, A, 80, W4A4_OK, false},
      {"asym no zeros", A, A, Z, 1, A, A, 16, 64, 256, A, 64, W4A4_ERR_MODE, false},
      {"mode 3", A, A, Z, 3, A, A, 16, 64, 256, A, 64, W4A4_ERR_MODE, false},
      {"N == 0", A, A, Z, 0, A, A, 16, 0, 256, A, 64, W4A4_ERR_SHAPE, false},
      {"K % 128", A, A, Z, 0, A, A, 16, 64, 200, A, 64, W4A4_ERR_SHAPE, false},
      {"K > 131072", A, A, Z, 0, A, A, 16, 64, 131200, A, 64, W4A4_ERR_SHAPE, false},
      {"ldy < N", A, A, Z, 0, A, A, 16, 64, 256, A, 63, W4A4_ERR_SHAPE, false},
      {"M >= 2^31", A, A, Z, 0, A, A, BIG, 64, 256, A, 64, W4A4_ERR_SHAPE, false},
      {"N >= 2^31", A, A, Z, 0, A, A, 16, BIG, 256, A, BIG, W4A4_ERR_SHAPE, false},
      {"null y", A, A, Z, 0, A, A, 16, 64, 256, Z, 64, W4A4_ERR_NULL, false},
      {"y misaligned", A, A, Z, 0, A, A, 16, 64, 256, U, 64, W4A4_ERR_ALIGN, false},
      {"M == 0", Z, Z, Z, 0, Z, Z, 0, 64, 256, Z, 64, W4A4_OK, true},
  };
  for (const C& c : cases) {
    w4a4v::Msg m;
    bool noop = true;
    std::string what = std::string("w4a4_gemm ") + c.what;
    expect(what.c_str(), w4a4v::w4a4_gemm(c.xc, c.xs, c.xz, c.mode, c.wc, c.ws, c.M, c.N, c.K, c.y, c.ldy, noop, m),
           c.want, m);
    expect_noop(what.c_str(), noop, c.noop);
    if (c.mode == 0 && c.xz == Z) {
      w4a4v::Msg m2;
      bool noop2 = true;
      std::string w2 = std::string("mxfp4_gemm ") + c.what;
      expect(w2.c_str(), w4a4v::mxfp4_gemm(c.xc, c.xs, c.wc, c.ws, c.M, c.N, c.K, c.y, c.ldy, noop2, m2), c.want, m2);
      expect_noop(w2.c_str(), noop2, c.noop);
    }
  }
}

void kv_cases() {
  const int64_t huge = int64_t(1) << 40, h30 = int64_t(1) << 30;
  struct C { const char* what; int64_t B, H, S, D, sb, sh, ss; const void* kv; w4a4_status want; bool noop; };
  const C cases[] = {
      {"ok dense", 2, 4, 100, 128, 4 * 100 * 128, 100 * 128, 128, A, W4A4_OK, false},
      {"ok strided", 2, 4, 100, 128, 4 * 100 * 128, 128, 4 * 128, A, W4A4_OK, false},
      {"D 64", 2, 4, 100, 64, 0, 0, 64, A, W4A4_ERR_SHAPE, false},
      {"negative S", 2, 4, -1, 128, 0, 0, 128, A, W4A4_ERR_SHAPE, false},
      {"B*H*S >= 2^31", 4, 1 << 20, 1 << 10, 128, 0, 0, 128, A, W4A4_ERR_SHAPE, false},
      {"huge B, no overflow", huge, h30, h30, 128, 0, 0, 128, A, W4A4_ERR_SHAPE, false},
      {"max B", std::numeric_limits<int64_t>::max(), 2, 2, 128, 0, 0, 128, A, W4A4_ERR_SHAPE, false},
      {"stride % 8", 2, 4, 100, 128, 0, 0, 132, A, W4A4_ERR_ALIGN, false},
      {"negative stride", 2, 4, 100, 128, -8, 0, 128, A, W4A4_ERR_SHAPE, false},
      {"null kv", 2, 4, 100, 128, 0, 0, 128, Z, W4A4_ERR_NULL, false},
      {"misaligned kv", 2, 4, 100, 128, 0, 0, 128, U, W4A4_ERR_ALIGN, false},
      {"S == 0", 2, 4, 0, 128, 0, 0, 128, Z, W4A4_OK, true},
      {"B == 0, H huge", 0, h30, 7, 128, 0, 0, 128, Z, W4A4_OK, true},
  };
  for (const C& c : cases) {
    w4a4v::Msg m;
    bool noop = true;
    std::string what = std::string("kv_rotate_quant4 ") + c.what;
    expect(what.c_str(), w4a4v::kv_rotate_quant4(c.kv, c.B, c.H, c.S, c.D, c.sb, c.sh, c.ss, Z, A, A, A, noop, m),
           c.want, m);
    expect_noop(what.c_str(), noop, c.noop);
  }
}

void attention_cases() {
  const float nan = std::numeric_limits<float>::quiet_NaN(), inf = std::numeric_limits<float>::infinity();
  struct C { const char* what; int64_t B, H, S, D; float sc; const void* q; w4a4_status want; bool noop; };
  const C cases[] = {
      {"ok", 2, 4, 4097, 128, 0.088f, A, W4A4_OK, false},
      {"S == 0", 2, 4, 0, 128, 0.088f, A, W4A4_ERR_SHAPE, false},
      {"S >= 2^25", 2, 4, int64_t(1) << 25, 128, 0.088f, A, W4A4_ERR_SHAPE, false},
      {"D 256", 2, 4, 10, 256, 0.088f, A, W4A4_ERR_SHAPE, false},
      {"scale 0", 2, 4, 10, 128, 0.0f, A, W4A4_ERR_SHAPE, false},
      {"scale NaN", 2, 4, 10, 128, nan, A, W4A4_ERR_SHAPE, false},
      {"scale inf", 2, 4, 10, 128, inf, A, W4A4_ERR_SHAPE, false},
      {"huge B, no overflow", std::numeric_limits<int64_t>::max(), 4, 10, 128, 0.1f, A, W4A4_ERR_SHAPE, false},
      {"null q", 2, 4, 10, 128, 0.1f, Z, W4A4_ERR_NULL, false},
      {"misaligned q", 2, 4, 10, 128, 0.1f, U, W4A4_ERR_ALIGN, false},
      {"B == 0", 0, 4, 10, 128, 0.1f, Z, W4A4_OK, true},
  };
  for (const C& c : cases) {
    w4a4v::Msg m;
    bool noop = true;
    std::string what = std::string("kv4_attention_decode ") + c.what;
    expect(what.c_str(),
           w4a4v::kv4_attention_decode(c.q, A, A, A, A, A, A, c.B, c.H, c.S, c.D, c.sc, Z, A, noop, m), c.want, m);
    expect_noop(what.c_str(), noop, c.noop);
  }
}

void split_attention_cases() {
  // the number of token ranges: fill 256 workgroups, at least 512 tokens
  // per range, at most 64 ranges, 1 = the single pass
  struct N { int64_t BH, S; int32_t want; };
  const N ns[] = {{256, 4096, 1}, {255, 1 << 20, 2}, {32, 4096, 8}, {8, 32768, 32}, {1, 1 << 20, 64},
                  {2, 700, 1},    {2, 1024, 2},      {1, 511, 1},   {0, 10, 1},     {5, 0, 1},
                  {int64_t(1) << 40, 10, 1}};
  for (const N& c : ns) {
    ++g_cases;
    const int32_t got = w4a4v::attention_splits(c.BH, c.S);
    if (got != c.want) {
      ++g_fail;
      std::printf("FAIL attention_splits(%lld, %lld) = %d, want %d\n", (long long)c.BH, (long long)c.S, got,
                  c.want);
    }
    ++g_cases;
    const int64_t bytes = w4a4v::attention_workspace_bytes(c.BH, c.S);
    const int64_t want_bytes = c.want > 1 ? c.BH * c.want * w4a4v::kAttnPartBytes : 0;
    if (bytes != want_bytes) {
      ++g_fail;
      std::printf("FAIL attention_workspace_bytes(%lld, %lld) = %lld\n", (long long)c.BH, (long long)c.S,
                  (long long)bytes);
    }
  }
  // every valid shape needs at most (BH + 255) states, BH < 256
  int64_t most = 0;
  for (int64_t bh = 1; bh <= 300; ++bh) {
    const int64_t b = w4a4v::attention_workspace_bytes(bh, int64_t(1) << 24);
    most = b > most ? b : most;
  }
  ++g_cases;
  if (most != 510 * w4a4v::kAttnPartBytes) {
    ++g_fail;
    std::printf("FAIL largest split workspace %lld bytes\n", (long long)most);
  }

  const int64_t need = 8 * 32 * w4a4v::kAttnPartBytes;   // 1 x 8 heads x 32768 tokens
  struct C { const char* what; int64_t B, S; const void* ws; int64_t bytes; w4a4_status want; bool noop; };
  const C cases[] = {
      {"ok", 1, 32768, A, need, W4A4_OK, false},
      {"workspace one byte short", 1, 32768, A, need - 1, W4A4_ERR_SHAPE, false},
      {"negative workspace size", 1, 32768, A, -1, W4A4_ERR_SHAPE, false},
      {"null workspace", 1, 32768, Z, need, W4A4_ERR_NULL, false},
      {"misaligned workspace", 1, 32768, U, need, W4A4_ERR_ALIGN, false},
      {"single pass needs none", 32, 4096, Z, 0, W4A4_OK, false},
      {"S == 0", 1, 0, A, need, W4A4_ERR_SHAPE, false},
      {"B == 0", 0, 32768, Z, 0, W4A4_OK, true},
  };
  for (const C& c : cases) {
    w4a4v::Msg m;
    bool noop = true;
    std::string what = std::string("kv4_attention_decode_ws ") + c.what;
    expect(what.c_str(),
           w4a4v::kv4_attention_decode_ws(A, A, A, A, A, A, A, c.B, 8, c.S, 128, 0.088f, Z, A, c.ws, c.bytes, noop,
                                          m),
           c.want, m);
    expect_noop(what.c_str(), noop, c.noop);
  }

  // the allocation-free variant: the same rules, and the partial states must
  // fit its static scratch (a small limit here forces the refusal)
  struct N2 { const char* what; int64_t B, S, limit; w4a4_status want; bool noop; };
  const N2 na[] = {
      {"fits", 1, 32768, need, W4A4_OK, false},
      {"one byte over the scratch", 1, 32768, need - 1, W4A4_ERR_SHAPE, false},
      {"single pass needs no scratch", 32, 4096, 0, W4A4_OK, false},
      {"S == 0", 1, 0, need, W4A4_ERR_SHAPE, false},
      {"B == 0", 0, 32768, 0, W4A4_OK, true},
      {"largest need fits 512 KiB", 1, int64_t(1) << 24, 512 * 1024, W4A4_OK, false},
  };
  for (const N2& c : na) {
    w4a4v::Msg m;
    bool noop = true;
    std::string what = std::string("kv4_attention_decode_noalloc ") + c.what;
    expect(what.c_str(),
           w4a4v::kv4_attention_decode_noalloc(A, A, A, A, A, A, A, c.B, 8, c.S, 128, 0.088f, Z, A, c.limit, noop, m),
           c.want, m);
    expect_noop(what.c_str(), noop, c.noop);
  }
}

void fused_cases() {
  struct C { const char* what; int64_t M, K, ldx, N, ldy; const void* x; w4a4_status want; };
  const C cases[] = {
      {"ok", 16, 4096, 4096, 4096, 4096, A, W4A4_OK},
      {"M 0", 0, 4096, 4096, 4096, 4096, A, W4A4_ERR_SHAPE},
      {"M 17", 17, 128, 128, 64, 64, A, W4A4_ERR_SHAPE},
      {"K 16384", 1, 16384, 16384, 64, 64, A, W4A4_ERR_SHAPE},
      {"M*K > 65536", 16, 8192, 8192, 64, 64, A, W4A4_ERR_SHAPE},
      {"ldx % 8", 2, 128, 132, 64, 64, A, W4A4_ERR_ALIGN},
      {"ldy < N", 2, 128, 128, 64, 60, A, W4A4_ERR_SHAPE},
      {"null x", 2, 128, 128, 64, 64, Z, W4A4_ERR_NULL},
      {"misaligned x", 2, 128, 128, 64, 64, U, W4A4_ERR_ALIGN},
  };
  for (const C& c : cases) {
    w4a4v::Msg m;
    std::string what = std::string("w4a4_decode_fused ") + c.what;
    expect(what.c_str(), w4a4v::w4a4_decode_fused(c.x, c.M, c.K, c.ldx, Z, A, A, c.N, A, c.ldy, m), c.want, m);
  }
}

}  // namespace

int main() {
  arch_cases();
  rotate_cases();
  weight_cases();
  gemm_cases();
  kv_cases();
  attention_cases();
  split_attention_cases();
  fused_cases();
  if (g_fail) {
    std::printf("validate selftest: %d of %d cases failed\n", g_fail, g_cases);
    return 1;
  }
  std::printf("validate selftest ok (%d cases)\n", g_cases);
  return 0;
}
