// fast_div.h -- division of a workgroup index by a launch constant, as one
// 32x32->64-bit multiply and a shift (Granlund and Montgomery, "Division by
// invariant integers using multiplication", PLDI 1994, the round-up method).
//
// For a divisor 1 <= d < 2^31 let l = ceil(log2 d), s = 26 + l and
// m = ceil(2^s / d), so m * d = 2^s + e with 0 <= e < d. Then for 0 <= n < 2^26
//   n * m / 2^s = n / d + n * e / (d * 2^s),  and  n * e < 2^26 * 2^l = 2^s,
// so the excess is below 1/d and cannot reach the next integer: the floor of
// n * m / 2^s is floor(n / d). Also m <= 2^(s - l + 1) + 1 = 2^27 + 1 fits in 32
// bits and n * m < 2^54 fits in 64. Workgroup indices satisfy n < 2^26 because a
// dispatch holds fewer than 2^32 work-items and the kernels that use this run
// 64-lane workgroups.
//
// Plain C++ (constexpr functions are callable from device code under hipcc), so
// the host test compiles this header with the system compiler.
#pragma once

#include <stdint.h>

namespace fastdiv {

constexpr uint32_t kMaxDividendBits = 26;

struct FastDiv {
  uint32_t mul;
  uint32_t shift;
};

constexpr FastDiv make(uint32_t d) {
  uint32_t l = 0;
  while (((uint64_t)1 << l) < d) ++l;
  const uint32_t s = kMaxDividendBits + l;
  return FastDiv{(uint32_t)((((uint64_t)1 << s) + d - 1) / d), s};
}

// floor(n / d) for n < 2^26, where f = make(d).
constexpr uint32_t div(uint32_t n, FastDiv f) {
  return (uint32_t)(((uint64_t)n * f.mul) >> f.shift);
}

}  // namespace fastdiv
