// Calls every entry point of the C ABI with bad and with valid arguments on a
// host without a usable GPU, under AddressSanitizer and
// UndefinedBehaviorSanitizer. Bad arguments must give their status code
// without reaching a launcher; valid ones must give TATTN_ERR_HIP (no
// device), again without reaching a launcher. Exits non-zero on the first
// mismatch; the sanitizers abort on any memory or undefined-behaviour error.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "tattn.h"

namespace tattn {
extern int g_stub_launches;
}

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
static float* F(uintptr_t a) { return reinterpret_cast<float*>(a); }
static const int32_t* I(uintptr_t a) { return reinterpret_cast<const int32_t*>(a); }

int main() {
  const float nan = std::nanf("");
  // attn_fwd / attn_fwd_f32
  expect("mha null q", attn_fwd(nullptr, P(16), P(16), P(16), F(16), 1, 1, 8, 8, 128, 0, 0.1f, nullptr),
         TATTN_ERR_INVALID_ARG);
  expect("mha B<0", attn_fwd(P(16), P(16), P(16), P(16), F(16), -1, 1, 8, 8, 128, 0, 0.1f, nullptr),
         TATTN_ERR_INVALID_ARG);
  expect("mha causal 2", attn_fwd(P(16), P(16), P(16), P(16), F(16), 1, 1, 8, 8, 128, 2, 0.1f, nullptr),
         TATTN_ERR_INVALID_ARG);
  expect("mha nan scale", attn_fwd(P(16), P(16), P(16), P(16), F(16), 1, 1, 8, 8, 128, 0, nan, nullptr),
         TATTN_ERR_INVALID_ARG);
  expect("mha D=96", attn_fwd(P(16), P(16), P(16), P(16), F(16), 1, 1, 8, 8, 96, 0, 0.1f, nullptr),
         TATTN_ERR_UNSUPPORTED);
  expect("mha align", attn_fwd(P(24), P(16), P(16), P(16), F(16), 1, 1, 8, 8, 128, 0, 0.1f, nullptr),
         TATTN_ERR_ALIGN);
  expect("mha huge", attn_fwd(P(16), P(16), P(16), P(16), F(16), 1 << 20, 1 << 12, 1 << 20, 8, 128, 0, 0.1f,
                              nullptr),
         TATTN_ERR_UNSUPPORTED);
  expect("mha INT_MAX heads", attn_fwd(P(16), P(16), P(16), P(16), F(16), 2147483647, 2147483647, 2147483647,
                                       2147483647, 128, 1, 0.1f, nullptr),
         TATTN_ERR_UNSUPPORTED);
  expect("mha nothing", attn_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 1, 8, 8, 128, 0, 0.1f, nullptr),
         TATTN_OK);
  expect("mha valid, no device", attn_fwd(P(16), P(16), P(16), P(16), F(16), 1, 1, 8, 8, 128, 0, 0.1f, nullptr),
         TATTN_ERR_HIP);
  expect("f32 D=256", attn_fwd_f32(F(16), F(16), F(16), F(16), F(16), 1, 1, 8, 8, 256, 0, 0.1f, nullptr),
         TATTN_ERR_UNSUPPORTED);
  expect("f32 valid, no device",
         attn_fwd_f32(F(16), F(16), F(16), F(16), F(16), 1, 1, 8, 8, 64, 1, 0.1f, nullptr), TATTN_ERR_HIP);
  // attn_fwd_ex
  expect("ex Hkv 3", attn_fwd_ex(P(16), P(16), P(16), P(16), F(16), 1, 4, 3, 8, 8, 128, 0, 0, nullptr, 0.1f,
                                 nullptr),
         TATTN_ERR_INVALID_ARG);
  expect("ex window<0", attn_fwd_ex(P(16), P(16), P(16), P(16), F(16), 1, 4, 2, 8, 8, 128, 0, -1, nullptr, 0.1f,
                                    nullptr),
         TATTN_ERR_INVALID_ARG);
  expect("ex valid, no device",
         attn_fwd_ex(P(16), P(16), P(16), P(16), F(16), 1, 4, 1, 8, 8, 128, 1, 3, nullptr, 0.1f, nullptr),
         TATTN_ERR_HIP);
  // mla_decode
  expect("mla null ind", mla_decode(P(16), P(16), P(16), P(16), P(16), F(16), 2, 128, nullptr, 0.05f, nullptr),
         TATTN_ERR_INVALID_ARG);
  expect("mla H=129", mla_decode(P(16), P(16), P(16), P(16), P(16), F(16), 2, 129, I(16), 0.05f, nullptr),
         TATTN_ERR_UNSUPPORTED);
  expect("mla align", mla_decode(P(16), P(16), P(40), P(16), P(16), F(16), 2, 128, I(16), 0.05f, nullptr),
         TATTN_ERR_ALIGN);
  expect("mla huge B", mla_decode(P(16), P(16), P(16), P(16), P(16), F(16), 1 << 25, 128, I(16), 0.05f, nullptr),
         TATTN_ERR_UNSUPPORTED);
  expect("mla nothing", mla_decode(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 128, nullptr, 0.05f,
                                   nullptr),
         TATTN_OK);
  expect("mla valid, no device",
         mla_decode(P(16), P(16), P(16), P(16), P(16), F(16), 2, 128, I(16), 0.05f, nullptr), TATTN_ERR_HIP);
  expect("mla no keys (null kv, k_pe), no device",
         mla_decode(P(16), P(16), nullptr, nullptr, P(16), F(16), 2, 128, I(16), 0.05f, nullptr), TATTN_ERR_HIP);
  expect("mla noalloc H=129", mla_decode_noalloc(P(16), P(16), P(16), P(16), P(16), F(16), 2, 129, I(16), 0.05f,
                                                 nullptr),
         TATTN_ERR_UNSUPPORTED);
  expect("mla noalloc null q", mla_decode_noalloc(nullptr, P(16), P(16), P(16), P(16), F(16), 2, 128, I(16),
                                                   0.05f, nullptr),
         TATTN_ERR_INVALID_ARG);
  expect("mla noalloc valid, no device",
         mla_decode_noalloc(P(16), P(16), P(16), P(16), P(16), F(16), 2, 128, I(16), 0.05f, nullptr),
         TATTN_ERR_HIP);
  // ssd_scan
  expect("ssd G 3", ssd_scan(P(16), F(4), F(4), P(16), P(16), P(16), nullptr, nullptr, 2, 100, 8, 3, 64, 128,
                             nullptr),
         TATTN_ERR_INVALID_ARG);
  expect("ssd overlap", ssd_scan(P(16), F(4), F(4), P(16), P(16), P(16), F(4096), F(4096 + 64 * 128 * 4), 2, 100,
                                 8, 1, 64, 128, nullptr),
         TATTN_ERR_INVALID_ARG);
  expect("ssd valid, no device",
         ssd_scan(P(16), F(4), F(4), P(16), P(16), P(16), nullptr, nullptr, 1, 64, 2, 1, 64, 128, nullptr),
         TATTN_ERR_HIP);
  // status strings
  for (int s = -7; s <= 1; ++s) {
    const char* t = tattn_status_str(s);
    if (!t || !std::strlen(t)) {
      std::fprintf(stderr, "FAIL status string %d\n", s);
      ++failures;
    }
  }
  if (tattn::g_stub_launches != 0) {
    std::fprintf(stderr, "FAIL %d launches reached without a device\n", tattn::g_stub_launches);
    ++failures;
  }
  std::printf("%s (%d failures)\n", failures ? "FAILED" : "all statuses as expected", failures);
  return failures ? 1 : 0;
}
