// Host build of the library's correctly rounded binary32 sin/cos (csrc/cr_sincos.h),
// for the CPU test that compares it with extended-precision references. Compiled by
// tests/test_sincos_host.py with g++; not part of the library.
#include <stdint.h>

static int64_t g_fallbacks = 0;
#define ROPE_HD
#define ROPE_TRIG_ON_FALLBACK() (++g_fallbacks)
#include "cr_sincos.h"

extern "C" {

// sin/cos exactly as the kernels evaluate them (fast path, then the double-double
// fallback near a binary32 rounding boundary). fell_back[i] (if not NULL) is set
// to 1 where angle i took the fallback. Returns how many did.
int64_t host_sincos(const float* angle, int64_t n, float* s, float* c, uint8_t* fell_back) {
  int64_t total = 0;
  for (int64_t i = 0; i < n; ++i) {
    g_fallbacks = 0;
    rope_trig::sincos_f32_cr(angle[i], s[i], c[i]);
    total += g_fallbacks;
    if (fell_back) fell_back[i] = (uint8_t)(g_fallbacks != 0);
  }
  return total;
}

// The double-double fallback alone, forced on every angle.
void host_sincos_dd(const float* angle, int64_t n, float* s, float* c) {
  for (int64_t i = 0; i < n; ++i) {
    const rope_trig::sc32 r = rope_trig::sincos_dd_path((double)angle[i]);
    s[i] = r.s;
    c[i] = r.c;
  }
}

}  // extern "C"
