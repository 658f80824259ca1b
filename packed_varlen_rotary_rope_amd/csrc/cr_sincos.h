// Correctly rounded binary32 cos/sin of a binary32 angle, for angles in
// [0, 2^31] (the RoPE angles fp32(pos) * inv_freq with pos < 2^31 and
// inv_freq <= 1).
//
// Method (Cody-Waite reduction + Taylor polynomials, then a rounding test):
//  1. Fast path in double. k = rint(x * 2/pi); r = x - k*pi/2 with pi/2 split
//     into three doubles (PIO2_1 + PIO2_2 + PIO2_3). The first step
//     fma(-k, PIO2_1, x) is exact: for x >= pi/4 both x and k*PIO2_1 are
//     multiples of 2^-52 and their difference is below 1 in magnitude. The
//     remaining two steps each round once, so r carries a relative error of
//     about 2^-52. sin r and cos r come from Taylor polynomials through r^15
//     and r^16 (truncation below 2^-53 for |r| <= pi/4), evaluated by Horner's
//     rule with FMA. Total error: a few units in the last place of the double.
//  2. Rounding test. Rounding a double v to binary32 is ambiguous only if v is
//     within the error bound of a binary32 rounding boundary (a midpoint
//     between two floats): in v's bit pattern, the 29 bits below binary32
//     precision are then within that bound of 0x10000000. The test uses a
//     window of 64 double ulps, several times the fast path's error bound, so
//     about one value in 2^22 falls back.
//  3. Fallback in double-double (about 2^-100 relative): reduction with an
//     exact two-product for k*PIO2_2, Horner's rule in double-double with the
//     Taylor coefficients through r^23 / r^22, then an exact rounding of the
//     double-double pair to binary32.
// The result is the binary32 nearest to the exact cos/sin of the fp32 angle,
// apart from inputs whose exact value lies within about 2^-100 of a midpoint.
#pragma once

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "trig_constants.h"

#ifndef ROPE_HD
#define ROPE_HD __host__ __device__
#endif
// A host build may count the fallbacks (the CPU test of this header does).
#ifndef ROPE_TRIG_ON_FALLBACK
#define ROPE_TRIG_ON_FALLBACK()
#endif

namespace rope_trig {

struct dd {
  double hi, lo;
};

struct sc32 {
  float s, c;
};

ROPE_HD inline uint64_t bits_of(double v) {
  uint64_t u;
  memcpy(&u, &v, sizeof u);
  return u;
}

ROPE_HD inline dd two_sum(double a, double b) {
  double s = a + b;
  double bb = s - a;
  double e = (a - (s - bb)) + (b - bb);
  return {s, e};
}

ROPE_HD inline dd fast_two_sum(double a, double b) {  // requires |a| >= |b| or a == 0
  double s = a + b;
  return {s, b - (s - a)};
}

ROPE_HD inline dd two_prod(double a, double b) {
  double p = a * b;
  return {p, fma(a, b, -p)};
}

ROPE_HD inline dd dd_mul(dd a, dd b) {
  dd p = two_prod(a.hi, b.hi);
  p.lo += a.hi * b.lo + a.lo * b.hi;
  return fast_two_sum(p.hi, p.lo);
}

ROPE_HD inline dd dd_add(dd a, dd b) {
  dd s = two_sum(a.hi, b.hi);
  s.lo += a.lo + b.lo;
  return fast_two_sum(s.hi, s.lo);
}

// True if rounding v (carrying a few ulps of error) to binary32 might differ
// from rounding the exact value, or if v is tiny and nonzero (binary32
// subnormal range, where the 29-bit test does not apply).
ROPE_HD inline bool near_f32_boundary(double v) {
  uint64_t u = bits_of(v) & 0x7fffffffffffffffull;
  if (u == 0) return false;
  if (u < (uint64_t)(1023 - 126) << 52) return true;
  int32_t low = (int32_t)(u & 0x1fffffffu) - 0x10000000;
  return low <= 64 && low >= -64;
}

// Exact rounding of hi + lo (|lo| <= ulp(hi)/2) to binary32, ties to even.
ROPE_HD inline float round_dd_to_f32(dd v) {
  float f = (float)v.hi;
  uint64_t u = bits_of(v.hi);
  bool midpoint = (u & 0x1fffffffu) == 0x10000000u;
  if (!midpoint || v.lo == 0.0) return f;
  // hi is exactly halfway between two binary32 values: lo decides the side.
  float up = nextafterf(f, __builtin_inff());
  float down = nextafterf(f, -__builtin_inff());
  float other = ((double)f < v.hi) ? up : down;
  float lo_side = (v.lo > 0.0) == ((double)other > v.hi) ? other : f;
  return lo_side;
}

// Quadrant bookkeeping: with x = k*pi/2 + r and q = k mod 4,
// sin x = {s, c, -s, -c}[q], cos x = {c, -s, -c, s}[q].
ROPE_HD inline void apply_quadrant(int q, double s, double c, double& sx, double& cx) {
  sx = (q & 1) ? c : s;
  cx = (q & 1) ? s : c;
  if (q & 2) sx = -sx;
  if (q == 1 || q == 2) cx = -cx;
}

#if defined(__HIP_DEVICE_COMPILE__)
__device__ __noinline__
#else
inline
#endif
sc32 sincos_dd_path(double x) {
  double k = rint(x * TWO_OVER_PI);
  double r1 = fma(-k, PIO2_1, x);  // exact
  dd kp2 = two_prod(k, PIO2_2);    // exact
  dd s = two_sum(r1, -kp2.hi);     // exact
  double lo = (s.lo - kp2.lo) - k * PIO2_3;
  dd r = fast_two_sum(s.hi, lo);
  dd z = dd_mul(r, r);
  dd ps = {SIN_DD[N_SIN_DD - 1][0], SIN_DD[N_SIN_DD - 1][1]};
  for (int i = N_SIN_DD - 2; i >= 0; --i) ps = dd_add(dd_mul(ps, z), dd{SIN_DD[i][0], SIN_DD[i][1]});
  dd sn = dd_mul(r, ps);
  dd pc = {COS_DD[N_COS_DD - 1][0], COS_DD[N_COS_DD - 1][1]};
  for (int i = N_COS_DD - 2; i >= 0; --i) pc = dd_add(dd_mul(pc, z), dd{COS_DD[i][0], COS_DD[i][1]});
  int q = (int)((int64_t)k & 3);
  dd sx = (q & 1) ? pc : sn;
  dd cx = (q & 1) ? sn : pc;
  if (q & 2) sx = dd{-sx.hi, -sx.lo};
  if (q == 1 || q == 2) cx = dd{-cx.hi, -cx.lo};
  return {round_dd_to_f32(sx), round_dd_to_f32(cx)};
}

ROPE_HD inline void sincos_f32_cr(float angle, float& s_out, float& c_out) {
  double x = (double)angle;
  double k = rint(x * TWO_OVER_PI);
  double r = fma(-k, PIO2_1, x);  // exact
  r = fma(-k, PIO2_2, r);
  r = fma(-k, PIO2_3, r);
  double z = r * r;
  double ps = SIN_C[N_SIN - 1];
#pragma unroll
  for (int i = N_SIN - 2; i >= 1; --i) ps = fma(ps, z, SIN_C[i]);
  double s = fma(r * z, ps, r);  // r + r^3 * (S1 + z*(S2 + ...))
  double pc = COS_C[N_COS - 1];
#pragma unroll
  for (int i = N_COS - 2; i >= 1; --i) pc = fma(pc, z, COS_C[i]);
  double c = fma(z, pc, 1.0);  // 1 + z * (C1 + z*(C2 + ...))
  double sx, cx;
  apply_quadrant((int)((int64_t)k & 3), s, c, sx, cx);
  float so = (float)sx, co = (float)cx;
  if (near_f32_boundary(sx) || near_f32_boundary(cx)) {
    ROPE_TRIG_ON_FALLBACK();
    const sc32 r = sincos_dd_path(x);
    so = r.s;
    co = r.c;
  }
  s_out = so;
  c_out = co;
}

}  // namespace rope_trig
