// rope_qk.hip -- fused, in-place, packed variable-length QK rotary position
// embedding for MI355X (gfx950, CDNA4): kernels and the C ABI of include/rope_qk.h.
//
// Pages followed (cited by title and section):
//  [U-RoPE]  Unsloth, "Entrainement des LLM 3 fois plus rapide avec les noyaux
//            Unsloth + le packing", section "Kernel Triton QK RoPE fusionne avec
//            packing": one kernel for Q and K, fully in place, rotate_half form
//            x*cos + (x @ R)*sin with R = [[0, I], [-I, 0]]; backward = same
//            rotation with sin negated.
//  [U-Pack]  same page, "Packing non contamine": positions restart per sample.
//  [U-int64] same page, "Indexage int64 pour les kernels Triton": 64-bit offsets
//            as a compile-time specialization, chosen only when needed.
//  [U-Group] same page, fused QK RoPE section (history): a workgroup handles a
//            group of heads.
//
// Work decomposition (memory-bound: one read and one write of every Q/K element,
// no MFMA). A lane owns one (token, chunk) pair, where a chunk is VEC
// consecutive elements of the first half of a head row (16 bytes for bf16/f16
// with VEC = 8, fp32 with VEC = 4) together with the matching VEC elements of the
// second half, D/2 further on. The lane
//   1. maps its token to (sequence, position) by binary search over cu_seqlens,
//   2. computes the VEC fp32 cos/sin values of its frequencies once,
//   3. walks the heads of its head group -- Q heads, then K heads -- and for each
//      head loads the two 16-byte chunks, rotates in fp32, rounds to the storage
//      dtype and stores them back in place.
// The lane that reads a pair (j, j + D/2) is the one that writes it, so the
// in-place update needs no synchronization. Per wave, each load instruction
// touches whole 128-byte half-rows (8 lanes x 16 B for D = 128 bf16).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/rope_qk.h"
#include "cr_sincos.h"

namespace {

constexpr int kBlock = 256;     // threads per workgroup (4 waves of 64)
constexpr int kMaxHalf = 256;   // D <= 512
constexpr int kMaxHeads = 4096;
constexpr int kUnroll = 8;      // head rows in flight per lane
// A dispatch's grid size in work-items is a 32-bit field: blocks * kBlock < 2^32.
constexpr int64_t kMaxBlocksX = (int64_t)0xffffffffu / kBlock;

struct RopeParams {
  alignas(16) float inv_freq[kMaxHalf];  // first: 16-byte aligned for vector loads
  void* q;
  void* k;
  int64_t T;
  const int32_t* cu;
  const int32_t* seqused;
  int32_t num_seqs;
  int32_t Hq, Hkv, D;
  int32_t nc;   // chunks per half row: (D/2) / VEC
  int32_t tpb;  // tokens per workgroup: kBlock / nc
  int32_t hpg;  // heads per group (blockIdx.y selects the group)
  float sin_sign;
};

struct CosSinParams {
  float inv_freq[kMaxHalf];
};

// ---- a1: token -> (sequence, position) [U-Pack] ------------------------------------
// Sequence s is the last index with cu[s] <= t (upper bound minus one). The token
// is rotated if 0 <= s < num_seqs and, with seqused, t - cu[s] < seqused[s].
// Returns the position, or -1 for an untouched token (then *seq_out = -1).
__device__ inline int32_t token_position(const int32_t* __restrict__ cu, int32_t num_seqs,
                                         const int32_t* __restrict__ seqused, int64_t t,
                                         int32_t* seq_out) {
  int32_t first = 0;
  int32_t count = num_seqs + 1;
  while (count > 0) {
    const int32_t step = count >> 1;
    const int32_t it = first + step;
    if ((int64_t)cu[it] <= t) {
      first = it + 1;
      count -= step + 1;
    } else {
      count = step;
    }
  }
  const int32_t s = first - 1;
  *seq_out = -1;
  if (s < 0 || s >= num_seqs) return -1;
  const int64_t p = t - (int64_t)cu[s];
  if (seqused != nullptr && p >= (int64_t)seqused[s]) return -1;
  *seq_out = s;
  return (int32_t)p;
}

// ---- a3: the angle, one fp32 multiply --------------------------------------------
__device__ inline float rope_angle(int32_t pos, float inv_freq_j) {
  return __fmul_rn((float)pos, inv_freq_j);
}

// ---- storage <-> fp32 -------------------------------------------------------------
template <typename T, int VEC>
struct alignas(sizeof(T) * VEC <= 16 ? sizeof(T) * VEC : 16) Chunk {
  T v[VEC];
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(__bf16 x) { return (float)x; }
__device__ inline float to_f32(_Float16 x) { return (float)x; }

// Round-to-nearest-even narrowing of a pair (one v_cvt_pk_* on gfx950).
__device__ inline void from_f32_pair(float a, float b, float* out) { out[0] = a; out[1] = b; }
__device__ inline void from_f32_pair(float a, float b, __bf16* out) {
  const bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);
  out[0] = r[0];
  out[1] = r[1];
}
__device__ inline void from_f32_pair(float a, float b, _Float16* out) {
  const f16x2 r = __builtin_convertvector((f32x2){a, b}, f16x2);
  out[0] = r[0];
  out[1] = r[1];
}
__device__ inline float from_f32(float a, float) { return a; }
__device__ inline __bf16 from_f32(float a, __bf16) { return (__bf16)a; }
__device__ inline _Float16 from_f32(float a, _Float16) { return (_Float16)a; }

template <typename T, int VEC>
__device__ inline void narrow(const float (&y)[VEC], Chunk<T, VEC>& out) {
#pragma unroll
  for (int e = 0; e + 1 < VEC; e += 2) from_f32_pair(y[e], y[e + 1], &out.v[e]);
  if constexpr (VEC & 1) out.v[VEC - 1] = from_f32(y[VEC - 1], T());
}

// ---- a4/a5: the rotation of one chunk pair [U-RoPE] ------------------------------
// y1 = x1*c - x2*s and y2 = x2*c + x1*s, each as a 2x2 determinant evaluated with
// Kahan's FMA scheme: w = b*c rounded, e = w - b*c exactly (FMA), f = a*d - w
// rounded (FMA), result = f + e. The fp32 result is within 2 ulps of the exact
// real value even where the two products cancel (Jeannerod, Louvet, Muller,
// Math. Comp. 82 (2013)), so rounding it to bf16 stays within 1 bf16 ulp of the
// exactly rounded result.
template <typename T, int VEC>
__device__ inline void rotate_chunk(Chunk<T, VEC>& lo, Chunk<T, VEC>& hi, const float (&cs)[VEC],
                                    const float (&sn)[VEC]) {
  float y1[VEC], y2[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    const float x1 = to_f32(lo.v[e]);
    const float x2 = to_f32(hi.v[e]);
    const float c = cs[e], s = sn[e];
    const float w1 = x2 * s;
    const float e1 = __builtin_fmaf(-x2, s, w1);
    const float f1 = __builtin_fmaf(x1, c, -w1);
    y1[e] = f1 + e1;
    const float w2 = x1 * s;
    const float e2 = __builtin_fmaf(x1, s, -w2);
    const float f2 = __builtin_fmaf(x2, c, w2);
    y2[e] = f2 + e2;
  }
  narrow(y1, lo);
  narrow(y2, hi);
}

// Rotate `nrows` consecutive head rows starting at row pointer `row` (already
// offset to this lane's chunk): loads for kUnroll rows are issued before any of
// them is used, so each lane keeps 2*kUnroll 16-byte loads in flight.
template <typename T, int VEC>
__device__ inline void rotate_rows(T* __restrict__ base, uint32_t off, int nrows, uint32_t D,
                                   uint32_t half, const float (&cs)[VEC], const float (&sn)[VEC]) {
  using C = Chunk<T, VEC>;
  int r = 0;
  for (; r + kUnroll <= nrows; r += kUnroll) {
    C lo[kUnroll], hi[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t o = off + (uint32_t)(r + u) * D;
      lo[u] = *reinterpret_cast<const C*>(base + o);
      hi[u] = *reinterpret_cast<const C*>(base + o + half);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t o = off + (uint32_t)(r + u) * D;
      rotate_chunk(lo[u], hi[u], cs, sn);
      *reinterpret_cast<C*>(base + o) = lo[u];
      *reinterpret_cast<C*>(base + o + half) = hi[u];
    }
  }
  for (; r < nrows; ++r) {
    const uint32_t o = off + (uint32_t)r * D;
    C lo = *reinterpret_cast<const C*>(base + o);
    C hi = *reinterpret_cast<const C*>(base + o + half);
    rotate_chunk(lo, hi, cs, sn);
    *reinterpret_cast<C*>(base + o) = lo;
    *reinterpret_cast<C*>(base + o + half) = hi;
  }
}

// Pointer to the first row of this workgroup's first token in a [T, H, D] tensor.
// [U-int64]: with LONG_INDEX the workgroup base offset is formed in 64 bits (it is
// uniform, so this is scalar arithmetic); without it, in 32 bits, which the host
// only selects when every offset of the launch fits. Per-lane offsets relative to
// this base are 32-bit in both cases (tpb * H * D < 2^29).
template <typename T, bool LONG_INDEX>
__device__ inline T* block_base(void* p, int64_t t0, int32_t H, int32_t D) {
  if (LONG_INDEX) return static_cast<T*>(p) + t0 * (int64_t)H * (int64_t)D;
  return static_cast<T*>(p) + (uint32_t)((uint32_t)t0 * (uint32_t)H * (uint32_t)D);
}

// ---- the fused QK kernel (a1..a7) ---------------------------------------------------
template <typename T, int VEC, bool LONG_INDEX>
__global__ __launch_bounds__(kBlock) void rope_qk_kernel(const RopeParams p) {
  const int tid = threadIdx.x;
  const int tl = tid / p.nc;  // token within the workgroup
  const int c = tid - tl * p.nc;
  if (tl >= p.tpb) return;
  const int64_t t0 = (int64_t)blockIdx.x * p.tpb;
  const int64_t t = t0 + tl;
  if (t >= p.T) return;
  int32_t seq;
  const int32_t pos = token_position(p.cu, p.num_seqs, p.seqused, t, &seq);
  if (pos < 0) return;

  // This lane's VEC inverse frequencies, fetched together before any sin/cos.
  const Chunk<float, VEC> f = *reinterpret_cast<const Chunk<float, VEC>*>(&p.inv_freq[c * VEC]);
  float cs[VEC], sn[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    rope_trig::sincos_f32_cr(rope_angle(pos, f.v[e]), sn[e], cs[e]);
    sn[e] *= p.sin_sign;  // backward: R transposed = sin negated
  }

  const uint32_t D = (uint32_t)p.D;
  const uint32_t half = D >> 1;
  const int hb = (int)blockIdx.y * p.hpg;  // this group's heads, Q first then K
  const int he = min(p.Hq + p.Hkv, hb + p.hpg);
  if (hb < p.Hq) {
    T* base = block_base<T, LONG_INDEX>(p.q, t0, p.Hq, p.D);
    const uint32_t off = ((uint32_t)tl * (uint32_t)p.Hq + (uint32_t)hb) * D + (uint32_t)(c * VEC);
    rotate_rows<T, VEC>(base, off, min(he, p.Hq) - hb, D, half, cs, sn);
  }
  if (he > p.Hq) {
    const int kb = max(hb, p.Hq) - p.Hq;
    T* base = block_base<T, LONG_INDEX>(p.k, t0, p.Hkv, p.D);
    const uint32_t off = ((uint32_t)tl * (uint32_t)p.Hkv + (uint32_t)kb) * D + (uint32_t)(c * VEC);
    rotate_rows<T, VEC>(base, off, he - p.Hq - kb, D, half, cs, sn);
  }
}

// ---- export hooks (same device functions) --------------------------------------------
__global__ __launch_bounds__(kBlock) void rope_positions_kernel(const int32_t* __restrict__ cu,
                                                                int32_t num_seqs,
                                                                const int32_t* __restrict__ seqused,
                                                                int64_t T, int32_t* pos_out,
                                                                int32_t* seq_out) {
  const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (t >= T) return;
  int32_t seq;
  const int32_t pos = token_position(cu, num_seqs, seqused, t, &seq);
  if (pos_out) pos_out[t] = pos;
  if (seq_out) seq_out[t] = seq;
}

__global__ __launch_bounds__(kBlock) void rope_cos_sin_kernel(const int32_t* __restrict__ positions,
                                                              int64_t n, int32_t half,
                                                              const CosSinParams p, float* cos_out,
                                                              float* sin_out) {
  const int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (idx >= n * half) return;
  const int64_t i = idx / half;
  const int32_t j = (int32_t)(idx - i * half);
  float s, c;
  rope_trig::sincos_f32_cr(rope_angle(positions[i], p.inv_freq[j]), s, c);
  cos_out[idx] = c;
  sin_out[idx] = s;
}

// ---- host side -----------------------------------------------------------------------

// a2: inv_freq[j] = theta^(-2j/D), evaluated in extended precision and rounded once.
void host_inv_freq(double theta, int32_t D, float* out) {
  for (int32_t j = 0; j < D / 2; ++j)
    out[j] = (float)powl((long double)theta, -(2.0L * (long double)j) / (long double)D);
}

bool valid_theta(double theta) { return isfinite(theta) && theta >= 1.0; }
bool valid_D(int32_t D) { return D >= 2 && D <= 2 * kMaxHalf && (D & 1) == 0; }

int32_t elem_size(int32_t dtype) { return dtype == ROPE_F32 ? 4 : 2; }

// Widest chunk (<= 16 bytes) that divides a half row and keeps every access aligned.
int32_t chunk_bytes(int32_t D, int32_t esize, const void* q, const void* k) {
  const int64_t half_bytes = (int64_t)(D / 2) * esize;
  for (int32_t b = 16; b > esize; b >>= 1) {
    if (half_bytes % b) continue;
    if (q && ((uintptr_t)q % b)) continue;
    if (k && ((uintptr_t)k % b)) continue;
    return b;
  }
  return esize;
}

template <typename T, int VEC>
int32_t launch_vec(const RopeParams& p, bool long_index, dim3 grid, hipStream_t stream) {
  if (long_index)
    hipLaunchKernelGGL((rope_qk_kernel<T, VEC, true>), grid, dim3(kBlock), 0, stream, p);
  else
    hipLaunchKernelGGL((rope_qk_kernel<T, VEC, false>), grid, dim3(kBlock), 0, stream, p);
  return hipGetLastError() == hipSuccess ? ROPE_OK : ROPE_ELAUNCH;
}

template <typename T>
int32_t launch_typed(RopeParams& p, int32_t bytes, bool long_index, hipStream_t stream) {
  const int32_t vec = bytes / (int32_t)sizeof(T);
  p.nc = (p.D / 2) / vec;
  if (p.nc > kBlock) return ROPE_EINVAL;  // cannot happen for D <= 512 and vec >= 1
  p.tpb = kBlock / p.nc;
  const int64_t gx = (p.T + p.tpb - 1) / p.tpb;
  const int32_t H = p.Hq + p.Hkv;
  const int64_t gy = (H + p.hpg - 1) / p.hpg;
  if (gx > kMaxBlocksX || gy > 65535) return ROPE_EINVAL;
  const dim3 grid((unsigned)gx, (unsigned)gy);
  switch (vec) {
    case 1: return launch_vec<T, 1>(p, long_index, grid, stream);
    case 2: return launch_vec<T, 2>(p, long_index, grid, stream);
    case 4: return launch_vec<T, 4>(p, long_index, grid, stream);
    default:
      if constexpr (sizeof(T) == 2) return launch_vec<T, 8>(p, long_index, grid, stream);
      return ROPE_EINVAL;
  }
}

}  // namespace

extern "C" {

int32_t rope_qk_apply(void* q, void* k, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                      const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                      double theta, int32_t dtype, int32_t direction, int32_t index_mode,
                      int32_t heads_per_group, void* stream) {
  if (dtype != ROPE_F32 && dtype != ROPE_BF16 && dtype != ROPE_F16) return ROPE_EUNSUPPORTED;
  if (T < 0 || T > ((int64_t)1 << 40)) return ROPE_EINVAL;
  if (Hq < 0 || Hkv < 0 || Hq > kMaxHeads || Hkv > kMaxHeads) return ROPE_EINVAL;
  if (!valid_D(D) || !valid_theta(theta)) return ROPE_EINVAL;
  if (num_seqs < 0 || num_seqs == INT32_MAX) return ROPE_EINVAL;
  if (direction != 1 && direction != -1) return ROPE_EINVAL;
  if (index_mode < ROPE_INDEX_AUTO || index_mode > ROPE_INDEX_64) return ROPE_EINVAL;
  if (heads_per_group < 0) return ROPE_EINVAL;
  const int32_t H = Hq + Hkv;
  if (T > 0 && H == 0) return ROPE_EINVAL;
  if (T == 0 || num_seqs == 0) return ROPE_OK;  // nothing is rotated
  if (cu_seqlens == nullptr) return ROPE_EINVAL;
  if ((Hq > 0 && q == nullptr) || (Hkv > 0 && k == nullptr)) return ROPE_EINVAL;

  const bool needs_long = T * (int64_t)H * (int64_t)D >= ((int64_t)1 << 31);
  if (index_mode == ROPE_INDEX_32 && needs_long) return ROPE_EINVAL;
  const bool long_index = needs_long || index_mode == ROPE_INDEX_64;

  RopeParams p;
  p.q = Hq > 0 ? q : nullptr;
  p.k = Hkv > 0 ? k : nullptr;
  p.T = T;
  p.cu = cu_seqlens;
  p.seqused = seqused;
  p.num_seqs = num_seqs;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.D = D;
  p.hpg = heads_per_group == 0 ? H : (heads_per_group < H ? heads_per_group : H);
  p.sin_sign = direction > 0 ? 1.0f : -1.0f;
  host_inv_freq(theta, D, p.inv_freq);

  const int32_t esize = elem_size(dtype);
  const int32_t bytes = chunk_bytes(D, esize, p.q, p.k);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case ROPE_F32: return launch_typed<float>(p, bytes, long_index, s);
    case ROPE_BF16: return launch_typed<__bf16>(p, bytes, long_index, s);
    default: return launch_typed<_Float16>(p, bytes, long_index, s);
  }
}

int32_t rope_qk_fwd(void* q, void* k, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                    const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                    double theta, int32_t dtype, void* stream) {
  return rope_qk_apply(q, k, T, Hq, Hkv, D, cu_seqlens, num_seqs, seqused, theta, dtype, +1,
                       ROPE_INDEX_AUTO, 0, stream);
}

int32_t rope_qk_bwd(void* dq, void* dk, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                    const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                    double theta, int32_t dtype, void* stream) {
  return rope_qk_apply(dq, dk, T, Hq, Hkv, D, cu_seqlens, num_seqs, seqused, theta, dtype, -1,
                       ROPE_INDEX_AUTO, 0, stream);
}

int32_t rope_positions(const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                       int64_t T, int32_t* pos_out, int32_t* seq_out, void* stream) {
  if (T < 0 || T > ((int64_t)1 << 40)) return ROPE_EINVAL;
  if (num_seqs < 0 || num_seqs == INT32_MAX) return ROPE_EINVAL;
  if (T == 0 || (pos_out == nullptr && seq_out == nullptr)) return ROPE_OK;
  if (cu_seqlens == nullptr) return ROPE_EINVAL;
  const int64_t blocks = (T + kBlock - 1) / kBlock;
  if (blocks > kMaxBlocksX) return ROPE_EINVAL;
  hipLaunchKernelGGL(rope_positions_kernel, dim3((unsigned)blocks), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), cu_seqlens, num_seqs, seqused, T, pos_out,
                     seq_out);
  return hipGetLastError() == hipSuccess ? ROPE_OK : ROPE_ELAUNCH;
}

int32_t rope_cos_sin(const int32_t* positions, int64_t n, int32_t D, double theta,
                     float* cos_out, float* sin_out, void* stream) {
  if (!valid_D(D) || !valid_theta(theta)) return ROPE_EINVAL;
  if (n < 0 || n > ((int64_t)1 << 34)) return ROPE_EINVAL;
  if (n == 0) return ROPE_OK;
  if (positions == nullptr || cos_out == nullptr || sin_out == nullptr) return ROPE_EINVAL;
  CosSinParams p;
  host_inv_freq(theta, D, p.inv_freq);
  const int32_t half = D / 2;
  const int64_t blocks = (n * half + kBlock - 1) / kBlock;
  if (blocks > kMaxBlocksX) return ROPE_EINVAL;
  hipLaunchKernelGGL(rope_cos_sin_kernel, dim3((unsigned)blocks), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), positions, n, half, p, cos_out, sin_out);
  return hipGetLastError() == hipSuccess ? ROPE_OK : ROPE_ELAUNCH;
}

int32_t rope_inv_freq(double theta, int32_t D, float* out) {
  if (!valid_D(D) || !valid_theta(theta) || out == nullptr) return ROPE_EINVAL;
  host_inv_freq(theta, D, out);
  return ROPE_OK;
}

const char* rope_status_str(int32_t status) {
  switch (status) {
    case ROPE_OK: return "ROPE_OK: success";
    case ROPE_EINVAL: return "ROPE_EINVAL: invalid argument";
    case ROPE_EUNSUPPORTED: return "ROPE_EUNSUPPORTED: unsupported dtype";
    case ROPE_ELAUNCH: return "ROPE_ELAUNCH: kernel launch failed";
    default: return "unknown rope status";
  }
}

int32_t rope_abi_version(void) { return ROPE_QK_ABI_VERSION; }

}  // extern "C"
