/*
 * rope_oracle.c -- CPU oracle for packed variable-length QK rotary position
 * embedding (RoPE), forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load or call this library. It shares
 * no code, header, table or constant with the HIP library, and neither side
 * includes or links the other.
 *
 * It is deliberately plain and slow: one element at a time, in the order of
 * the definition, with double/long double arithmetic wherever the result is a
 * real number that is later rounded once.
 *
 * Sources (web pages, cited by title and section):
 *  [U-RoPE] Unsloth, "Entrainement des LLM 3 fois plus rapide avec les noyaux
 *           Unsloth + le packing", section "Kernel Triton QK RoPE fusionne avec
 *           packing": the rotation is x*cos + rotate_half(x)*sin, which equals
 *           x*cos + (x @ R)*sin with the block matrix R = [[0, I], [-I, 0]]; the
 *           backward pass applies R transposed, i.e. the same map with sin
 *           negated; Q and K are rotated in place.
 *  [U-Pack] same page, section "Packing non contamine": several samples are
 *           packed into one 1-D token tensor and the RoPE positions restart at
 *           each sample.
 *  [DB-Pack] Databricks, "Reduire le temps d'entrainement de Qwen de 6x sur AI
 *           Runtime", section "Mise en lots, tokenisation et padding": per-sample
 *           position ids for a 1-D packed batch.
 *  [TRL-YaRN] TRL guide "Entrainement au-dela de 1 M de jetons", YaRN section:
 *           rope_theta (1e6 for Qwen3) is the frequency base the model ships with.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *  R1 inverse frequencies inv_freq[j] = theta^(-2j/D), j < D/2 (standard RoPE),
 *     rounded once to fp32; cos/sin shared by element j and element j + D/2.
 *  R2 pairing of element j with element j + D/2 (the rotate_half layout that the
 *     block matrix R describes), not interleaved pairs.
 *  R3 positions start at 0 at cu_seqlens[s]; tokens before cu_seqlens[0], at or
 *     after cu_seqlens[num_seqs], or at a position >= seqused[s] are untouched.
 *  R4 the angle is one fp32 multiply, fp32(pos) * inv_freq[j].
 *  R5 cos and sin are the correctly rounded fp32 values of cos/sin of that angle.
 *  R6 the rotation is evaluated exactly (both products are exact in double) and
 *     rounded once to fp32; bf16 outputs are that fp32 value rounded to nearest
 *     even.
 *  R7 explicit positions: token t uses position_ids[t]; a negative id leaves it
 *     untouched (Databricks page above: per-example position ids of a 1-D packed
 *     batch). Per-sequence offsets: position p of sequence s becomes
 *     p + seq_offsets[s]; a result outside [0, 2^31) leaves the token untouched.
 *  R8 linear position interpolation by a factor f >= 1 (TRL guide, YaRN section:
 *     with factor 4, position 100000 is treated as 25000): the fp32 position is
 *     divided by the fp32 factor (one rounding) before the angle multiply.
 *  R9 caller-supplied cos/sin tables: row p of each table holds the fp32 cos /
 *     sin of position p for every frequency; the rotation (R2, R6) uses them as
 *     given, sin negated backward; a token whose position has no row is
 *     untouched.
 *
 * Parity pins: every function here is checked against something other than
 * itself in tests/test_oracle_pins.py (closed forms, mpmath, the block matrix R
 * built with numpy, complex multiplication, invariants, brute force; the storage
 * decodes against the IEEE 754 field layout, all 65536 binary16 words included).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F16 2

/* ---- element storage formats (the oracle's own conversions) ---------------- */

static float bits_to_float(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static uint32_t float_to_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}

/* bf16 is the upper half of an IEEE binary32: widening is exact. */
static float bf16_to_float(uint16_t b) { return bits_to_float((uint32_t)b << 16); }

/* binary16 -> binary32, exact, written from the IEEE 754 field layout. */
static float f16_to_float(uint16_t h) {
  int sign = (h >> 15) & 1;
  int exp = (h >> 10) & 0x1f;
  int man = h & 0x3ff;
  double v;
  if (exp == 0)
    v = ldexp((double)man, -24); /* subnormal: man * 2^-14 * 2^-10 */
  else if (exp == 31)
    v = man ? NAN : INFINITY;
  else
    v = ldexp((double)(man | 0x400), exp - 25); /* (1024 + man) * 2^(exp-15-10) */
  return (float)(sign ? -v : v);
}

static double load_elem(int32_t dtype, const void* x, int64_t i) {
  switch (dtype) {
    case ORACLE_F32: return (double)((const float*)x)[i];
    case ORACLE_BF16: return (double)bf16_to_float(((const uint16_t*)x)[i]);
    default: return (double)f16_to_float(((const uint16_t*)x)[i]);
  }
}

/* ---- R1: inverse frequencies -------------------------------------------------- */

void oracle_inv_freq(double theta, int32_t D, float* out) {
  for (int32_t j = 0; j < D / 2; ++j) {
    long double e = -(2.0L * (long double)j) / (long double)D;
    out[j] = (float)powl((long double)theta, e);
  }
}

/* ---- R4 + R5: angle and fp32 cos/sin for one (position, frequency) ------------ */

static void cos_sin_one(int32_t pos, float scale, float inv_freq_j, float* c, float* s) {
  float p = (float)pos;
  if (scale != 1.0f) p = p / scale;  /* R8: one fp32 division */
  float angle = p * inv_freq_j;      /* one fp32 multiply */
  *c = (float)cosl((long double)angle);
  *s = (float)sinl((long double)angle);
}

/* Table of cos/sin for a list of positions: out[i*(D/2) + j]. */
void oracle_cos_sin_ex(const int32_t* pos, int64_t npos, int32_t D, double theta,
                       double pos_scale, float* cos_out, float* sin_out) {
  float inv_freq[1024];
  oracle_inv_freq(theta, D, inv_freq);
  for (int64_t i = 0; i < npos; ++i)
    for (int32_t j = 0; j < D / 2; ++j)
      cos_sin_one(pos[i], (float)pos_scale, inv_freq[j], &cos_out[i * (D / 2) + j],
                  &sin_out[i * (D / 2) + j]);
}

void oracle_cos_sin(const int32_t* pos, int64_t npos, int32_t D, double theta,
                    float* cos_out, float* sin_out) {
  oracle_cos_sin_ex(pos, npos, D, theta, 1.0, cos_out, sin_out);
}

/* ---- R3: token -> (sequence id, position), by walking the sequences ------------ */

/* Length of sequence s that is rotated: its cu_seqlens span, cut to seqused[s]. */
static int64_t used_len(const int32_t* cu, const int32_t* seqused, int32_t s) {
  int64_t len = (int64_t)cu[s + 1] - (int64_t)cu[s];
  if (seqused && (int64_t)seqused[s] < len) len = seqused[s];
  return len < 0 ? 0 : len;
}

/* Position after the per-sequence offset (R7), or -1 when it leaves [0, 2^31). */
static int32_t shifted(int64_t p, const int32_t* seq_offsets, int32_t s) {
  int64_t q = p + (seq_offsets ? (int64_t)seq_offsets[s] : 0);
  return (q < 0 || q > 2147483647LL) ? -1 : (int32_t)q;
}

/* pos_out[t] / seq_out[t] = position and sequence of token t, or -1 / -1 for a
 * token that is left untouched. Either output may be NULL. With position_ids the
 * sequence ids are all -1. */
void oracle_positions_ex(const int32_t* cu, int32_t num_seqs, const int32_t* seqused,
                         const int32_t* seq_offsets, const int32_t* position_ids, int64_t T,
                         int32_t* pos_out, int32_t* seq_out) {
  for (int64_t t = 0; t < T; ++t) {
    if (pos_out) pos_out[t] = -1;
    if (seq_out) seq_out[t] = -1;
  }
  if (position_ids) {
    for (int64_t t = 0; t < T; ++t)
      if (pos_out) pos_out[t] = position_ids[t] < 0 ? -1 : position_ids[t];
    return;
  }
  for (int32_t s = 0; s < num_seqs; ++s) {
    int64_t len = used_len(cu, seqused, s);
    for (int64_t p = 0; p < len; ++p) {
      int64_t t = (int64_t)cu[s] + p;
      if (t < 0 || t >= T) continue;
      int32_t pe = shifted(p, seq_offsets, s);
      if (pe < 0) continue;
      if (pos_out) pos_out[t] = pe;
      if (seq_out) seq_out[t] = s;
    }
  }
}

void oracle_positions(const int32_t* cu, int32_t num_seqs, const int32_t* seqused, int64_t T,
                      int32_t* pos_out, int32_t* seq_out) {
  oracle_positions_ex(cu, num_seqs, seqused, NULL, NULL, T, pos_out, seq_out);
}

/* Position of one token, or -1 if untouched: the same walk, stopped at t. */
static int32_t position_of(const int32_t* cu, int32_t num_seqs, const int32_t* seqused,
                           const int32_t* seq_offsets, const int32_t* position_ids, int64_t t) {
  if (position_ids) return position_ids[t] < 0 ? -1 : position_ids[t];
  for (int32_t s = 0; s < num_seqs; ++s) {
    int64_t p = t - (int64_t)cu[s];
    if (p >= 0 && p < used_len(cu, seqused, s)) return shifted(p, seq_offsets, s);
  }
  return -1;
}

/* ---- R2 + R6: rotate one (token, head) row ------------------------------------ */

/* x_row / y_row hold D elements. sin is multiplied by dir (+1 forward, -1
 * backward: the transpose of the rotation). */
static void rotate_row(int32_t dtype, const void* x, int64_t row_off, float* y_row, int32_t D,
                       const float* cs, const float* sn, int32_t dir) {
  int32_t half = D / 2;
  for (int32_t j = 0; j < half; ++j) {
    double x1 = load_elem(dtype, x, row_off + j);
    double x2 = load_elem(dtype, x, row_off + j + half);
    double c = (double)cs[j];
    double s = (double)dir * (double)sn[j];
    double y1 = x1 * c - x2 * s; /* first half:  x1*cos + (-x2)*sin */
    double y2 = x2 * c + x1 * s; /* second half: x2*cos + ( x1)*sin */
    y_row[j] = (float)y1;
    y_row[j + half] = (float)y2;
  }
}

static void copy_row(int32_t dtype, const void* x, int64_t row_off, float* y_row, int32_t D) {
  for (int32_t e = 0; e < D; ++e) y_row[e] = (float)load_elem(dtype, x, row_off + e);
}

static int check_args(int32_t dtype, int32_t H, int32_t D) {
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F16) return -1;
  if (H < 0 || D < 2 || (D & 1) || D > 2048) return -1;
  return 0;
}

/* Apply the rotation to a whole packed tensor x[T, H, D] (one of Q, K, dQ, dK).
 * y[T, H, D] receives the fp32 result; untouched tokens receive their input value.
 * Parallel over the positions of each sequence (nthreads <= 0: one thread). */
int32_t oracle_rope_ex(int32_t dtype, const void* x, float* y, int64_t T, int32_t H, int32_t D,
                       const int32_t* cu, int32_t num_seqs, const int32_t* seqused,
                       const int32_t* seq_offsets, const int32_t* position_ids, double theta,
                       double pos_scale, int32_t dir, int32_t nthreads) {
  if (check_args(dtype, H, D) || T < 0 || num_seqs < 0) return -1;
  if (nthreads <= 0) nthreads = 1;
  float inv_freq[1024];
  oracle_inv_freq(theta, D, inv_freq);
  const float scale = (float)pos_scale;
  int64_t row_elems = (int64_t)H * D;

  /* Start from the input: tokens outside every sequence keep their value. */
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int32_t h = 0; h < H; ++h)
      copy_row(dtype, x, t * row_elems + (int64_t)h * D, y + t * row_elems + (int64_t)h * D, D);

  if (position_ids) { /* R7: explicit positions */
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      int32_t pe = position_ids[t];
      if (pe < 0) continue;
      float cs[1024], sn[1024];
      for (int32_t j = 0; j < D / 2; ++j) cos_sin_one(pe, scale, inv_freq[j], &cs[j], &sn[j]);
      for (int32_t h = 0; h < H; ++h) {
        int64_t off = t * row_elems + (int64_t)h * D;
        rotate_row(dtype, x, off, y + off, D, cs, sn, dir);
      }
    }
    return 0;
  }

  for (int32_t s = 0; s < num_seqs; ++s) {
    int64_t len = used_len(cu, seqused, s);
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t p = 0; p < len; ++p) {
      int64_t t = (int64_t)cu[s] + p;
      if (t < 0 || t >= T) continue;
      int32_t pe = shifted(p, seq_offsets, s);
      if (pe < 0) continue;
      float cs[1024], sn[1024];
      for (int32_t j = 0; j < D / 2; ++j) cos_sin_one(pe, scale, inv_freq[j], &cs[j], &sn[j]);
      for (int32_t h = 0; h < H; ++h) {
        int64_t off = t * row_elems + (int64_t)h * D;
        rotate_row(dtype, x, off, y + off, D, cs, sn, dir);
      }
    }
  }
  return 0;
}

/* R9: the same rotation with cos/sin taken from tables cos_tab / sin_tab
 * [tab_rows, D/2] (row p = position p) instead of from theta. Positions and
 * untouched tokens as in oracle_rope_ex; a position >= tab_rows is untouched.
 * One thread, one token at a time. */
int32_t oracle_rope_table(int32_t dtype, const void* x, float* y, int64_t T, int32_t H,
                          int32_t D, const int32_t* cu, int32_t num_seqs, const int32_t* seqused,
                          const int32_t* seq_offsets, const int32_t* position_ids,
                          const float* cos_tab, const float* sin_tab, int64_t tab_rows,
                          int32_t dir) {
  if (check_args(dtype, H, D) || T < 0 || num_seqs < 0 || tab_rows < 1) return -1;
  int64_t row_elems = (int64_t)H * D;
  int32_t half = D / 2;
  for (int64_t t = 0; t < T; ++t) {
    int32_t pe = position_of(cu, num_seqs, seqused, seq_offsets, position_ids, t);
    for (int32_t h = 0; h < H; ++h) {
      int64_t off = t * row_elems + (int64_t)h * D;
      if (pe < 0 || pe >= tab_rows)
        copy_row(dtype, x, off, y + off, D);
      else
        rotate_row(dtype, x, off, y + off, D, cos_tab + (int64_t)pe * half,
                   sin_tab + (int64_t)pe * half, dir);
    }
  }
  return 0;
}

int32_t oracle_rope(int32_t dtype, const void* x, float* y, int64_t T, int32_t H, int32_t D,
                    const int32_t* cu, int32_t num_seqs, const int32_t* seqused, double theta,
                    int32_t dir, int32_t nthreads) {
  return oracle_rope_ex(dtype, x, y, T, H, D, cu, num_seqs, seqused, NULL, NULL, theta, 1.0, dir,
                        nthreads);
}

/* Same result for a list of tokens only. x_rows[n, H, D] holds the input rows of
 * tokens[0..n) (gathered by the caller); y_rows[n, H, D] receives their outputs.
 * The position of each token is found by walking the sequences. */
int32_t oracle_rope_rows_ex(int32_t dtype, const void* x_rows, float* y_rows,
                            const int64_t* tokens, int64_t n, int32_t H, int32_t D,
                            const int32_t* cu, int32_t num_seqs, const int32_t* seqused,
                            const int32_t* seq_offsets, const int32_t* position_ids,
                            double theta, double pos_scale, int32_t dir, int32_t nthreads) {
  if (check_args(dtype, H, D) || n < 0 || num_seqs < 0) return -1;
  if (nthreads <= 0) nthreads = 1;
  float inv_freq[1024];
  oracle_inv_freq(theta, D, inv_freq);
  const float scale = (float)pos_scale;
  int64_t row_elems = (int64_t)H * D;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 16)
  for (int64_t i = 0; i < n; ++i) {
    int32_t p = position_of(cu, num_seqs, seqused, seq_offsets, position_ids, tokens[i]);
    float cs[1024], sn[1024];
    if (p >= 0)
      for (int32_t j = 0; j < D / 2; ++j) cos_sin_one(p, scale, inv_freq[j], &cs[j], &sn[j]);
    for (int32_t h = 0; h < H; ++h) {
      int64_t off = i * row_elems + (int64_t)h * D;
      if (p >= 0)
        rotate_row(dtype, x_rows, off, y_rows + off, D, cs, sn, dir);
      else
        copy_row(dtype, x_rows, off, y_rows + off, D);
    }
  }
  return 0;
}

int32_t oracle_rope_rows(int32_t dtype, const void* x_rows, float* y_rows, const int64_t* tokens,
                         int64_t n, int32_t H, int32_t D, const int32_t* cu, int32_t num_seqs,
                         const int32_t* seqused, double theta, int32_t dir, int32_t nthreads) {
  return oracle_rope_rows_ex(dtype, x_rows, y_rows, tokens, n, H, D, cu, num_seqs, seqused, NULL,
                             NULL, theta, 1.0, dir, nthreads);
}

/* ---- comparison helpers ------------------------------------------------------ */

/* fp32 -> bf16, round to nearest, ties to even; NaN stays a (quiet) NaN. */
void oracle_round_bf16(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u = float_to_bits(in[i]);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) {
      out[i] = (uint16_t)((u >> 16) | 0x0040u);
      continue;
    }
    uint32_t keep = u >> 16;
    uint32_t rest = u & 0xffffu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
    out[i] = (uint16_t)keep;
  }
}

/* Elapsed-time helper for the CPU baseline: fwd on two tensors then bwd on two
 * tensors, as one timed unit (seconds, wall clock). */
#include <time.h>
double oracle_fwd_bwd_seconds(int32_t dtype, const void* q, const void* k, const void* dq,
                              const void* dk, float* yq, float* yk, float* ydq, float* ydk,
                              int64_t T, int32_t Hq, int32_t Hkv, int32_t D, const int32_t* cu,
                              int32_t num_seqs, const int32_t* seqused, double theta,
                              int32_t nthreads) {
  struct timespec a, b;
  clock_gettime(CLOCK_MONOTONIC, &a);
  int rc = 0;
  rc |= oracle_rope(dtype, q, yq, T, Hq, D, cu, num_seqs, seqused, theta, +1, nthreads);
  rc |= oracle_rope(dtype, k, yk, T, Hkv, D, cu, num_seqs, seqused, theta, +1, nthreads);
  rc |= oracle_rope(dtype, dq, ydq, T, Hq, D, cu, num_seqs, seqused, theta, -1, nthreads);
  rc |= oracle_rope(dtype, dk, ydk, T, Hkv, D, cu, num_seqs, seqused, theta, -1, nthreads);
  clock_gettime(CLOCK_MONOTONIC, &b);
  if (rc) return -1.0;
  return (double)(b.tv_sec - a.tv_sec) + 1e-9 * (double)(b.tv_nsec - a.tv_nsec);
}

/* The same for a sample of tokens: forward over the gathered rows of Q and K,
 * backward over those of dQ and dK (oracle_rope_rows each), timed as one unit.
 * For the CPU baseline on inputs too large to process whole. */
double oracle_rows_fwd_bwd_seconds(int32_t dtype, const void* q_rows, const void* k_rows,
                                   const void* dq_rows, const void* dk_rows, float* yq,
                                   float* yk, float* ydq, float* ydk, const int64_t* tokens,
                                   int64_t n, int32_t Hq, int32_t Hkv, int32_t D,
                                   const int32_t* cu, int32_t num_seqs, const int32_t* seqused,
                                   double theta, int32_t nthreads) {
  struct timespec a, b;
  clock_gettime(CLOCK_MONOTONIC, &a);
  int rc = 0;
  rc |= oracle_rope_rows(dtype, q_rows, yq, tokens, n, Hq, D, cu, num_seqs, seqused, theta, +1,
                         nthreads);
  rc |= oracle_rope_rows(dtype, k_rows, yk, tokens, n, Hkv, D, cu, num_seqs, seqused, theta, +1,
                         nthreads);
  rc |= oracle_rope_rows(dtype, dq_rows, ydq, tokens, n, Hq, D, cu, num_seqs, seqused, theta, -1,
                         nthreads);
  rc |= oracle_rope_rows(dtype, dk_rows, ydk, tokens, n, Hkv, D, cu, num_seqs, seqused, theta, -1,
                         nthreads);
  clock_gettime(CLOCK_MONOTONIC, &b);
  if (rc) return -1.0;
  return (double)(b.tv_sec - a.tv_sec) + 1e-9 * (double)(b.tv_nsec - a.tv_nsec);
}
