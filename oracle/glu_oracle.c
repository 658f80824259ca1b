/*
 * glu_oracle.c -- CPU oracle for the gated MLP activations SwiGLU and GeGLU,
 * forward and backward, over 2-D [rows, cols] tensors with row strides.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load or call this library. It shares
 * no code, header, table or constant with the HIP library, and neither side
 * includes or links the other.
 *
 * Plain and slow on purpose: one element at a time, in double precision, each
 * activation written as its textbook definition; outputs are doubles, so the
 * caller rounds once to the storage format it compares against.
 *
 * Source (web page, cited by title and section):
 *  [U-MLP]  Unsloth, "Entrainement des LLM 3 fois plus rapide avec les noyaux
 *           Unsloth + le packing": the opening list says the SwiGLU and GeGLU
 *           MLP kernels were updated with int64 indexing for long contexts, and
 *           section "Indexage int64 pour les kernels Triton" explains why: at a
 *           500K-token context their element offsets overflowed 32 bits, so the
 *           kernels gained a compile-time switch between 32- and 64-bit offsets.
 *           The page names the two activations but does not write them out.
 *
 * Readings (the page is silent on the formulas; each reading is listed in the
 * design notes):
 *  G1 SwiGLU: h = silu(e) * g, silu(e) = e * sigmoid(e), sigmoid(e) = 1/(1+exp(-e))
 *     (Shazeer, "GLU Variants Improve Transformer", 2020). e is the gate
 *     projection, g the up projection, element for element.
 *  G2 GeGLU: h = gelu(e) * g with the exact GELU, gelu(e) = e * Phi(e), Phi the
 *     standard normal CDF, Phi(e) = erfc(-e/sqrt(2)) / 2 (Hendrycks & Gimpel).
 *  G3 GeGLU with the tanh approximation of GELU:
 *     gelu_tanh(e) = e/2 * (1 + tanh(sqrt(2/pi) * (e + 0.044715 e^3))).
 *     Both GELU forms are built, since the page does not say which one.
 *  G4 backward, from upstream dh: dg = dh * act(e), de = dh * g * act'(e)
 *     (chain rule), with act' written out below.
 *  G5 the sums 1 + erf(x) and 1 + tanh(u) are evaluated as erfc(-x) and
 *     2/(1 + exp(-2u)), the same numbers written without cancellation, so the
 *     double result keeps its relative accuracy in the negative tail.
 *  G6 layout: e and g (and de, dg) are [rows, cols] with rows in_stride elements
 *     apart; h and dh have rows out_stride apart. Oracle outputs are dense
 *     [rows, cols] doubles.
 *
 * Parity pins: tests/glu_oracle_checks.py checks every function here against
 * something other than itself (mpmath at high precision with the literal
 * definitions, numerical derivatives, torch's float64 activations and autograd,
 * symmetry identities, printed normal-table values, exact rational rounding).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <time.h>

#define GLU_F32 0
#define GLU_BF16 1
#define GLU_F16 2

#define PI 3.14159265358979323846

#define GLU_SWIGLU 0
#define GLU_GEGLU 1
#define GLU_GEGLU_TANH 2

/* ---- element storage ------------------------------------------------------- */

static double decode_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16; /* bf16 is the upper half of a binary32 */
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double decode_f16(uint16_t h) {
  int neg = (h >> 15) & 1;
  int ex = (h >> 10) & 0x1f;
  int man = h & 0x3ff;
  double v;
  if (ex == 0)
    v = ldexp((double)man, -24); /* subnormal: man * 2^-24 */
  else if (ex == 31)
    v = man ? NAN : INFINITY;
  else
    v = ldexp((double)(man + 1024), ex - 25);
  return neg ? -v : v;
}

static double elem(int32_t dtype, const void* x, int64_t i) {
  if (dtype == GLU_F32) return (double)((const float*)x)[i];
  if (dtype == GLU_BF16) return decode_bf16(((const uint16_t*)x)[i]);
  return decode_f16(((const uint16_t*)x)[i]);
}

/* ---- G1-G3: the activations and their derivatives ---------------------------- */

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Phi(x), the standard normal CDF. */
static double normal_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

/* phi(x), the standard normal density. */
static double normal_pdf(double x) { return exp(-0.5 * x * x) / sqrt(2.0 * PI); }

/* u(x) of the tanh form and its derivative. */
static double tanh_arg(double x) { return sqrt(2.0 / PI) * (x + 0.044715 * x * x * x); }
static double tanh_arg_prime(double x) { return sqrt(2.0 / PI) * (1.0 + 3.0 * 0.044715 * x * x); }

double oracle_glu_act(int32_t kind, double e) {
  switch (kind) {
    case GLU_SWIGLU: return e * sigmoid(e);
    case GLU_GEGLU: return e * normal_cdf(e);
    /* (1 + tanh(u)) / 2 = sigmoid(2u), G5 */
    case GLU_GEGLU_TANH: return e * sigmoid(2.0 * tanh_arg(e));
    default: return NAN;
  }
}

double oracle_glu_grad(int32_t kind, double e) {
  switch (kind) {
    case GLU_SWIGLU: {
      /* d/de [e s(e)] = s + e s (1 - s), with 1 - s(e) = s(-e) */
      double s = sigmoid(e);
      return s + e * s * sigmoid(-e);
    }
    case GLU_GEGLU:
      /* d/de [e Phi(e)] = Phi(e) + e phi(e) */
      return normal_cdf(e) + e * normal_pdf(e);
    case GLU_GEGLU_TANH: {
      /* d/de [e s(2u)] = s(2u) + e s(2u) s(-2u) 2 u'(e) */
      double u = tanh_arg(e);
      double s = sigmoid(2.0 * u);
      return s + e * s * sigmoid(-2.0 * u) * 2.0 * tanh_arg_prime(e);
    }
    default: return NAN;
  }
}

static int bad_args(int32_t kind, int32_t dtype, int64_t rows, int64_t cols) {
  if (kind < GLU_SWIGLU || kind > GLU_GEGLU_TANH) return 1;
  if (dtype < GLU_F32 || dtype > GLU_F16) return 1;
  return rows < 0 || cols < 0;
}

/* ---- G1-G4, G6: whole tensors -------------------------------------------------- */

/* h[r, c] = act(e[r, c]) * g[r, c]; h is dense [rows, cols]. */
int32_t oracle_glu_fwd(int32_t kind, int32_t dtype, const void* e, const void* g, double* h,
                       int64_t rows, int64_t cols, int64_t in_stride, int32_t nthreads) {
  if (bad_args(kind, dtype, rows, cols) || in_stride < cols) return -1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      int64_t i = r * in_stride + c;
      h[r * cols + c] = oracle_glu_act(kind, elem(dtype, e, i)) * elem(dtype, g, i);
    }
  }
  return 0;
}

/* de = dh * g * act'(e), dg = dh * act(e); de and dg are dense [rows, cols]. */
int32_t oracle_glu_bwd(int32_t kind, int32_t dtype, const void* dh, const void* e, const void* g,
                       double* de, double* dg, int64_t rows, int64_t cols, int64_t in_stride,
                       int64_t out_stride, int32_t nthreads) {
  if (bad_args(kind, dtype, rows, cols) || in_stride < cols || out_stride < cols) return -1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      int64_t i = r * in_stride + c;
      double up = elem(dtype, dh, r * out_stride + c);
      double ev = elem(dtype, e, i);
      double gv = elem(dtype, g, i);
      de[r * cols + c] = up * gv * oracle_glu_grad(kind, ev);
      dg[r * cols + c] = up * oracle_glu_act(kind, ev);
    }
  }
  return 0;
}

/* ---- comparison helper: one rounding from double to the storage format ------- */

/* Round x to nearest (ties to even) in a binary format with p significand bits,
 * minimum normal exponent emin and largest finite value max_finite. */
static double round_to_format(double x, int p, int emin, double max_finite) {
  if (x == 0.0 || isnan(x) || isinf(x)) return x;
  int E;
  frexp(x, &E); /* |x| = m 2^E, m in [0.5, 1): the leading bit has weight 2^(E-1) */
  int lead = E - 1 < emin ? emin : E - 1;
  double quantum = ldexp(1.0, lead - (p - 1));
  double r = nearbyint(x / quantum) * quantum; /* default rounding: to nearest, ties even */
  if (fabs(r) > max_finite) return x > 0 ? INFINITY : -INFINITY;
  return r;
}

/* dtype GLU_F32: out is float[n]; GLU_BF16 / GLU_F16: out holds the 16-bit words. */
void oracle_glu_round(int32_t dtype, const double* in, void* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    if (dtype == GLU_F32) {
      ((float*)out)[i] = (float)round_to_format(in[i], 24, -126, 3.4028234663852886e38);
      continue;
    }
    if (dtype == GLU_BF16) {
      double r = round_to_format(in[i], 8, -126, 3.3895313892515355e38);
      float f = (float)r; /* exact: r has at most 8 significant bits */
      uint32_t u;
      memcpy(&u, &f, sizeof u);
      if (isnan(r)) u |= 0x00400000u;
      ((uint16_t*)out)[i] = (uint16_t)(u >> 16);
      continue;
    }
    double r = round_to_format(in[i], 11, -14, 65504.0);
    uint16_t w;
    if (isnan(r)) {
      w = 0x7e00u;
    } else {
      uint16_t sign = signbit(r) ? 0x8000u : 0;
      double a = fabs(r);
      if (isinf(a)) {
        w = sign | 0x7c00u;
      } else if (a < ldexp(1.0, -14)) {
        w = sign | (uint16_t)(a * ldexp(1.0, 24)); /* subnormal: a / 2^-24 */
      } else {
        int E;
        double m = frexp(a, &E); /* a = m 2^E, m in [0.5, 1) */
        uint16_t ex = (uint16_t)(E - 1 + 15);
        uint16_t man = (uint16_t)((m * 2.0 - 1.0) * 1024.0);
        w = sign | (uint16_t)(ex << 10) | man;
      }
    }
    ((uint16_t*)out)[i] = w;
  }
}

/* Wall time (seconds) of one forward plus one backward over the same tensors. */
double oracle_glu_seconds(int32_t kind, int32_t dtype, const void* e, const void* g,
                          const void* dh, double* h, double* de, double* dg, int64_t rows,
                          int64_t cols, int32_t nthreads) {
  struct timespec a, b;
  clock_gettime(CLOCK_MONOTONIC, &a);
  int rc = oracle_glu_fwd(kind, dtype, e, g, h, rows, cols, cols, nthreads);
  rc |= oracle_glu_bwd(kind, dtype, dh, e, g, de, dg, rows, cols, cols, cols, nthreads);
  clock_gettime(CLOCK_MONOTONIC, &b);
  if (rc) return -1.0;
  return (double)(b.tv_sec - a.tv_sec) + 1e-9 * (double)(b.tv_nsec - a.tv_nsec);
}
