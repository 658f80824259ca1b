// glu.hip -- SwiGLU / GeGLU forward and backward for MI355X (gfx950, CDNA4):
// kernels and the C ABI of include/glu.h.
//
// Page followed: Unsloth, "Entrainement des LLM 3 fois plus rapide avec les noyaux
// Unsloth + le packing" -- opening list (SwiGLU and GeGLU kernels with int64
// indexing for long contexts) and section "Indexage int64 pour les kernels
// Triton" (64-bit offsets as a compile-time specialization, selected only when an
// offset needs them) [U-int64]. The activations are the standard ones (Shazeer
// 2020; Hendrycks & Gimpel 2016), written out in include/glu.h.
//
// Work decomposition (memory-bound elementwise: one read of each input and one
// write of each output, no reuse, no MFMA). The [rows, cols] index space is cut
// into chunks of VEC consecutive elements of a row (16 bytes when sizes, strides
// and addresses allow: VEC = 8 for bf16/f16, 4 for fp32). A 256-lane workgroup
// takes 4 x 256 consecutive chunks per step: each lane issues the loads of its
// 4 chunks (2 inputs each in the forward, 3 in the backward) before any math,
// then computes in fp32 and stores. Loads and stores are non-temporal. When the
// three tensors are dense the chunk index is the element offset / VEC; otherwise
// a lane splits it into (row, chunk in row) with one division.
//
// Accuracy. sigmoid comes from one exp of -|z| (no overflow, no cancellation:
// sigmoid(z) = 1/(1+t) or t/(1+t), t = exp(-|z|)); Phi(e) comes from
// erfc(|e|/sqrt 2)/2 = s exp(-e^2/2) R(s), s = 1/(2 sqrt 2 + |e|), with a fitted
// polynomial R and (fp32 storage) an exactly split exponent, so it keeps its relative accuracy
// in the negative tail and shares its exp with the density. The derivative act'(e) has a
// root e0 where its direct formula cancels; near e0 it is taken from a Taylor
// polynomial around e0 (glu_constants.h). With fp32 storage every output is then
// within a few fp32 ulps of the exact value (plus, for the tanh form, the
// conditioning of its tail: about |2u(e)| ulps). With bf16 / f16 storage shorter
// polynomials and an unsplit exponent product are used, whose errors (below 2^-16
// relative) stay far under half a 16-bit ulp; either way each output is rounded
// once to the storage dtype.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/glu.h"
#include "glu_constants.h"
#include "storage.h"

namespace {

using namespace storage;
using namespace glu_const;

constexpr int kBlock = 256;
constexpr int kUnroll = 4;                   // chunks per lane whose loads are in flight together
constexpr int64_t kMaxBlocks = 1 << 20;      // beyond this the grid strides
constexpr int64_t kMaxSpan = (int64_t)1 << 48;  // elements

struct GluShape {
  int64_t n_chunks;              // end of this launch's chunks (rows * chunks_per_row for all)
  int64_t chunks_per_row;        // cols / VEC
  int64_t in_stride, out_stride;  // elements between rows (e, g, de, dg / h, dh)
  int64_t begin;                 // first chunk of this launch
};

// ---- activations in fp32 -----------------------------------------------------------

// exp(y) for -150 <= y <= 0 (Cody-Waite style): y log2(e) = n + f with n an
// integer and |f| <= 1/2, exp(y) = 2^f 2^n; 2^f is one v_exp_f32 (1 ulp on
// [-1/2, 1/2]) and the scaling by 2^n one ldexp, which also rounds the subnormal
// results correctly. FULL (fp32 storage): the product y log2(e) is carried as
// ph + pl (FMA split, log2(e) itself in two parts), so f = (ph - n) + pl is exact
// to far below an ulp. Otherwise f = ph - n (exact) and the rounding of ph, at
// most 2^-24 |ph| <= 2^-16.2 for |y| <= 150, moves the result by under 2^-16.7
// relative: far below a 16-bit ulp, and the two FMAs and an add are saved.
template <bool FULL>
__device__ inline float exp_nonpos(float y) {
  const float ph = y * kLog2e;
  const float n = __builtin_rintf(ph);
  float f;
  if constexpr (FULL) {
    const float pl = __builtin_fmaf(y, kLog2eLo, __builtin_fmaf(y, kLog2e, -ph));
    f = (ph - n) + pl;
  } else {
    f = ph - n;
  }
  return __builtin_amdgcn_ldexpf(__builtin_amdgcn_exp2f(f), (int)n);
}

// sigmoid(z) and 1 - sigmoid(z) from t = exp(-|z|): 1/(1+t) and t/(1+t), each the
// larger or the smaller by the sign of z. rcp is within 1 ulp. exp(-150) is 0 in
// fp32, so larger |z| are capped there.
template <bool FULL>
__device__ inline void sigmoid_pair(float z, float& s, float& sc) {
  const float t = exp_nonpos<FULL>(fmaxf(-fabsf(z), -150.0f));
  const float r = __builtin_amdgcn_rcpf(1.0f + t);
  const float small = t * r;
  s = z >= 0.0f ? r : small;
  sc = z >= 0.0f ? small : r;
}

// Phi(e) and exp(-e^2/2) with one exp. With s = 1/(2 sqrt(2) + |e|),
// erfc(|e|/sqrt 2)/2 = s exp(-e^2/2) R(s) for a fitted polynomial R
// (glu_constants.h). Phi(e) is that half-erfc for e < 0 and 1 minus it
// otherwise. |e| is capped at 16, where Phi is 0 or 1 in fp32 and exp(-e^2/2) is
// 0, so nothing overflows. FULL (fp32 storage): the degree-8 R, and e^2 split into
// its rounded value and the exact rounding error (FMA) so that the exponent
// carries no rounding of its own; otherwise the degree-6 R and the rounded e^2,
// whose errors (below 2^-16 relative) vanish in the 16-bit rounding.
template <bool FULL>
__device__ inline void normal_cdf_gauss(float e, float& cdf, float& gauss) {
  const float ec = fminf(fmaxf(e, -16.0f), 16.0f);
  const float s = __builtin_amdgcn_rcpf(kPhiShift + fabsf(ec));
  float r;
  if constexpr (FULL) {
    r = kPhiPoly[kPhiDegree];
#pragma unroll
    for (int k = kPhiDegree - 1; k >= 0; --k) r = __builtin_fmaf(r, s, kPhiPoly[k]);
  } else {
    r = kPhiPoly16[kPhiDegree16];
#pragma unroll
    for (int k = kPhiDegree16 - 1; k >= 0; --k) r = __builtin_fmaf(r, s, kPhiPoly16[k]);
  }
  const float sq = ec * ec;
  const float g0 = exp_nonpos<FULL>(-0.5f * sq);
  if constexpr (FULL) {
    const float sq_err = __builtin_fmaf(ec, ec, -sq);  // e^2 = sq + sq_err exactly
    gauss = __builtin_fmaf(-0.5f * sq_err, g0, g0);   // exp(-sq/2) * (1 - sq_err/2)
  } else {
    gauss = g0;
  }
  const float half_erfc = s * gauss * r;
  cdf = e < 0.0f ? half_erfc : 1.0f - half_erfc;
}

// act'(e0 + d) near the root e0 of the derivative: d * sum_k a[k] d^k, where the
// direct formula cancels. FULL: degree 10 for |d| <= 1/4; otherwise degree 5 for
// |d| <= 1/8 (outside it the direct formula loses at most a factor 8 to
// cancellation, far below a 16-bit ulp).
template <bool FULL, int N16, int N>
__device__ inline float root_poly(float e, float root_hi, float root_lo, const float (&a16)[N16],
                                  const float (&a)[N], float direct) {
  const float d = (e - root_hi) - root_lo;  // e - root_hi is exact inside the window
  if constexpr (FULL) {
    float p = a[N - 1];
#pragma unroll
    for (int k = N - 2; k >= 0; --k) p = __builtin_fmaf(p, d, a[k]);
    return fabsf(d) <= kRootWindow ? p * d : direct;
  } else {
    float p = a16[N16 - 1];
#pragma unroll
    for (int k = N16 - 2; k >= 0; --k) p = __builtin_fmaf(p, d, a16[k]);
    return fabsf(d) <= kRootWindow16 ? p * d : direct;
  }
}

template <int KIND, bool FULL>
__device__ inline float act_fwd(float e) {
  if constexpr (KIND == GLU_SWIGLU) {
    float s, sc;
    sigmoid_pair<FULL>(e, s, sc);
    return e * s;
  } else if constexpr (KIND == GLU_GEGLU) {
    float cdf, gauss;
    normal_cdf_gauss<FULL>(e, cdf, gauss);
    return e * cdf;
  } else {
    // 2u = e (A + B e^2); |e| > 64 gives the same sigmoid (0 or 1) without overflow
    const float ec = fminf(fmaxf(e, -64.0f), 64.0f);
    const float z = ec * __builtin_fmaf(kTanhB, ec * ec, kTanhA);
    float s, sc;
    sigmoid_pair<FULL>(z, s, sc);
    return e * s;
  }
}

// act(e) and act'(e) together (the backward needs both).
template <int KIND, bool FULL>
__device__ inline void act_bwd(float e, float& a, float& da) {
  if constexpr (KIND == GLU_SWIGLU) {
    float s, sc;
    sigmoid_pair<FULL>(e, s, sc);
    a = e * s;
    // s (1 + e (1 - s))
    const float direct = s * __builtin_fmaf(e, sc, 1.0f);
    da = root_poly<FULL>(e, kSiluRootHi, kSiluRootLo, kSiluPoly16, kSiluPoly, direct);
  } else if constexpr (KIND == GLU_GEGLU) {
    float cdf, gauss;
    normal_cdf_gauss<FULL>(e, cdf, gauss);
    const float pdf = gauss * kInvSqrt2Pi;
    a = e * cdf;
    // Phi + e phi
    const float direct = __builtin_fmaf(e, pdf, cdf);
    da = root_poly<FULL>(e, kGeluRootHi, kGeluRootLo, kGeluPoly16, kGeluPoly, direct);
  } else {
    const float ec = fminf(fmaxf(e, -64.0f), 64.0f);
    const float e2 = ec * ec;
    const float z = ec * __builtin_fmaf(kTanhB, e2, kTanhA);
    const float zp = __builtin_fmaf(kTanhC, e2, kTanhA);
    float s, sc;
    sigmoid_pair<FULL>(z, s, sc);
    a = e * s;
    // s (1 + e z' (1 - s))
    const float direct = s * __builtin_fmaf(ec * zp, sc, 1.0f);
    da = root_poly<FULL>(e, kGeluTanhRootHi, kGeluTanhRootLo, kGeluTanhPoly16, kGeluTanhPoly,
                         direct);
  }
}

// ---- the kernel ------------------------------------------------------------------------

// One step of a lane: chunks base + u*kBlock + lane, u < kUnroll. CHECKED = false
// when the whole step is in range (every step but the last): then the loads of all
// kUnroll chunks are unconditional and go out back to back, before any math; a
// per-chunk bounds branch would make the compiler wait for each chunk's loads
// before issuing the next chunk's.
template <typename T, int VEC, int KIND, bool BWD, bool DENSE, bool CHECKED, typename Index>
__device__ __attribute__((always_inline)) inline void glu_step(const T* dh, const T* e, const T* g,
                                                               T* out0, T* out1, const GluShape& s,
                                                               Index base, Index n) {
  using C = Chunk<T, VEC>;
  constexpr bool kFull = sizeof(T) == 4;  // fp32 storage: full-length polynomials
  C ce[kUnroll], cg[kUnroll], cd[kUnroll];
  Index in_off[kUnroll], out_off[kUnroll];
  bool live[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const Index c = base + (Index)(u * kBlock) + (Index)threadIdx.x;
    live[u] = !CHECKED || c < n;
    const Index cc = live[u] ? c : (Index)0;  // chunk 0 always exists: a safe dummy
    if constexpr (DENSE) {
      in_off[u] = cc * VEC;
      out_off[u] = cc * VEC;
    } else {
      const Index row = cc / (Index)s.chunks_per_row;
      const Index col = (cc - row * (Index)s.chunks_per_row) * VEC;
      in_off[u] = row * (Index)s.in_stride + col;
      out_off[u] = row * (Index)s.out_stride + col;
    }
    ce[u] = load_chunk<T, VEC>(e + in_off[u]);
    cg[u] = load_chunk<T, VEC>(g + in_off[u]);
    if constexpr (BWD) cd[u] = load_chunk<T, VEC>(dh + out_off[u]);
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    if constexpr (!BWD) {
      float h[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) h[j] = act_fwd<KIND, kFull>(to_f32(ce[u].v[j])) * to_f32(cg[u].v[j]);
      C ch;
      narrow(h, ch);
      if (live[u]) store_chunk<T, VEC>(out0 + out_off[u], ch);
    } else {
      float de[VEC], dg[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        float a, da;
        act_bwd<KIND, kFull>(to_f32(ce[u].v[j]), a, da);
        const float up = to_f32(cd[u].v[j]);
        de[j] = up * to_f32(cg[u].v[j]) * da;
        dg[j] = up * a;
      }
      C cde, cdg;
      narrow(de, cde);
      narrow(dg, cdg);
      if (live[u]) {
        store_chunk<T, VEC>(out0 + in_off[u], cde);
        store_chunk<T, VEC>(out1 + in_off[u], cdg);
      }
    }
  }
}

// [U-int64]: Index is uint32_t when every offset of the launch is below 2^31 (the
// host checks), int64_t otherwise. No __restrict__: an output may be the memory
// of one of the inputs (in place).
template <typename T, int VEC, int KIND, bool BWD, bool DENSE, typename Index>
__global__ __launch_bounds__(kBlock) void glu_kernel(const T* dh, const T* e, const T* g, T* out0,
                                                     T* out1, const GluShape s) {
  const Index n = (Index)s.n_chunks;
  const Index per_step = (Index)(kBlock * kUnroll);
  const Index step = (Index)gridDim.x * per_step;
  for (Index base = (Index)s.begin + (Index)blockIdx.x * per_step; base < n; base += step) {
    if (n - base >= per_step)  // wave-uniform: the whole step is in range
      glu_step<T, VEC, KIND, BWD, DENSE, false>(dh, e, g, out0, out1, s, base, n);
    else
      glu_step<T, VEC, KIND, BWD, DENSE, true>(dh, e, g, out0, out1, s, base, n);
  }
}

// ---- host side -------------------------------------------------------------------------

int32_t elem_bytes(int32_t dtype) { return dtype == ROPE_F32 ? 4 : 2; }

// Widest access (<= 16 bytes) that divides the row length, every stride and every
// address, in bytes.
int32_t chunk_bytes(int32_t esize, int64_t cols, int64_t in_stride, int64_t out_stride,
                    const void* const* ptrs, int nptr) {
  for (int32_t b = 16; b > esize; b >>= 1) {
    bool ok = (cols * esize) % b == 0 && (in_stride * esize) % b == 0 && (out_stride * esize) % b == 0;
    for (int i = 0; i < nptr && ok; ++i) ok = ((uintptr_t)ptrs[i] % b) == 0;
    if (ok) return b;
  }
  return esize;
}

struct Launch {
  const void* dh;
  const void* e;
  const void* g;
  void* out0;
  void* out1;
  GluShape shape;
  unsigned blocks;
  hipStream_t stream;
};

// Workgroups resident per CU, capped by reserving LDS the kernel does not use
// (lds_per_cu / cap bytes per workgroup): fewer in flight stream HBM faster once a
// launch has many rounds of workgroups. Measured on MI355X, bf16: forward capped
// at 5 (20 waves) 0.7-3% faster on 16384 x 9728 and 65536 x 12288, backward
// capped at 3 (12 waves) up to 4% faster (unchanged for exact GeGLU); on 4096 x
// 4096 (2048 workgroups, 8 per CU) either cap is 2-8% slower, so launches under
// 8192 workgroups run uncapped.
constexpr uint32_t kLdsPerCU = 160 * 1024;
uint32_t glu_dynamic_lds(bool bwd, unsigned blocks) {
  if (blocks < 8192) return 0;
  return kLdsPerCU / (bwd ? 3 : 5);
}

// Long calls as several launches. Workgroup i of a launch runs on XCC i mod 8, and
// over a long launch the eight XCCs drift apart, so that they stream from separate
// address ranges instead of neighbouring ones, which HBM serves more slowly; a
// launch boundary brings them back together (the RoPE kernel's host code measures
// the drift). Calls of 2 * kGluPieceBlocks workgroups or more are issued as
// consecutive launches of about kGluPieceBlocks each, every launch starting at a
// multiple of 8 workgroups so that each step keeps the XCC it has in a single
// launch. Measured on SwiGLU 524288 x 9728 bf16 (row ranges of one call,
// interleaved): one launch 5065 us forward / 8600 us backward, launches of 38912
// workgroups 4784 / 8136, of 19456 workgroups 4774 / 8132, of 77824 4843 / 8217.
constexpr int64_t kGluPieceBlocks = 32768;
int64_t glu_piece_blocks(int64_t blocks) {
  if (blocks < 2 * kGluPieceBlocks) return blocks;
  const int64_t n = (blocks + kGluPieceBlocks - 1) / kGluPieceBlocks;
  return ((blocks + n - 1) / n + 7) / 8 * 8;
}

template <typename T, int VEC, int KIND, bool BWD, bool DENSE, typename Index>
int32_t launch_one(const Launch& L) {
  hipLaunchKernelGGL((glu_kernel<T, VEC, KIND, BWD, DENSE, Index>), dim3(L.blocks), dim3(kBlock),
                     glu_dynamic_lds(BWD, L.blocks),
                     L.stream, static_cast<const T*>(L.dh), static_cast<const T*>(L.e),
                     static_cast<const T*>(L.g), static_cast<T*>(L.out0), static_cast<T*>(L.out1),
                     L.shape);
  return hipGetLastError() == hipSuccess ? ROPE_OK : ROPE_ELAUNCH;
}

template <typename T, int VEC, int KIND, bool BWD>
int32_t launch_layout(const Launch& L, bool dense, bool long_index) {
  if (dense) {
    return long_index ? launch_one<T, VEC, KIND, BWD, true, int64_t>(L)
                      : launch_one<T, VEC, KIND, BWD, true, uint32_t>(L);
  }
  return long_index ? launch_one<T, VEC, KIND, BWD, false, int64_t>(L)
                    : launch_one<T, VEC, KIND, BWD, false, uint32_t>(L);
}

template <typename T, int VEC, bool BWD>
int32_t launch_kind(int32_t kind, const Launch& L, bool dense, bool long_index) {
  switch (kind) {
    case GLU_SWIGLU: return launch_layout<T, VEC, GLU_SWIGLU, BWD>(L, dense, long_index);
    case GLU_GEGLU: return launch_layout<T, VEC, GLU_GEGLU, BWD>(L, dense, long_index);
    default: return launch_layout<T, VEC, GLU_GEGLU_TANH, BWD>(L, dense, long_index);
  }
}

template <typename T, bool BWD>
int32_t launch_vec(int32_t kind, int32_t vec, const Launch& L, bool dense, bool long_index) {
  switch (vec) {
    case 1: return launch_kind<T, 1, BWD>(kind, L, dense, long_index);
    case 2: return launch_kind<T, 2, BWD>(kind, L, dense, long_index);
    case 4: return launch_kind<T, 4, BWD>(kind, L, dense, long_index);
    default:
      if constexpr (sizeof(T) == 2) return launch_kind<T, 8, BWD>(kind, L, dense, long_index);
      return ROPE_EINVAL;
  }
}

int32_t glu_launch(bool bwd, int32_t kind, const void* dh, const void* e, const void* g, void* out0,
                   void* out1, int64_t rows, int64_t cols, int64_t in_stride, int64_t out_stride,
                   int32_t dtype, int32_t index_mode, void* stream) {
  if (dtype != ROPE_F32 && dtype != ROPE_BF16 && dtype != ROPE_F16) return ROPE_EUNSUPPORTED;
  if (kind < GLU_SWIGLU || kind > GLU_GEGLU_TANH) return ROPE_EINVAL;
  if (index_mode < ROPE_INDEX_AUTO || index_mode > ROPE_INDEX_64) return ROPE_EINVAL;
  if (rows < 0 || cols < 0 || in_stride < 0 || out_stride < 0) return ROPE_EINVAL;
  const int64_t is = in_stride == 0 ? cols : in_stride;
  const int64_t os = out_stride == 0 ? cols : out_stride;
  if (is < cols || os < cols) return ROPE_EINVAL;
  if (rows == 0 || cols == 0) return ROPE_OK;
  if (is > kMaxSpan / rows || os > kMaxSpan / rows) return ROPE_EINVAL;
  if (!e || !g || !out0 || (bwd && (!dh || !out1))) return ROPE_EINVAL;

  // [U-int64] 64-bit offsets exactly when the largest element offset reaches 2^31.
  const int64_t lim = (int64_t)1 << 31;
  const bool needs_long = (rows - 1) * is + cols >= lim || (rows - 1) * os + cols >= lim;
  if (index_mode == ROPE_INDEX_32 && needs_long) return ROPE_EINVAL;
  // The tanh-GeGLU backward takes the 64-bit instance under AUTO also where every
  // offset fits: in the 32-bit instance the compiler's schedule waits for a step's
  // first loads before issuing the rest (the 64-bit instance keeps them in flight),
  // measured 262.1 against 254.6 us on 16384 x 9728 bf16. For the other kinds the
  // 32-bit instance is as fast or faster (exact GeGLU 259.0 / 258.4, SwiGLU
  // 251.6 / 254.7), so the offset width itself costs nothing measurable here.
  const bool prefer_long = bwd && kind == GLU_GEGLU_TANH && index_mode == ROPE_INDEX_AUTO;
  const bool long_index = needs_long || index_mode == ROPE_INDEX_64 || prefer_long;

  const int32_t esize = elem_bytes(dtype);
  const void* ptrs[5] = {e, g, out0, bwd ? dh : e, bwd ? out1 : e};
  const int32_t vec = chunk_bytes(esize, cols, is, os, ptrs, 5) / esize;
  const bool dense = is == cols && os == cols;

  Launch L;
  L.dh = dh;
  L.e = e;
  L.g = g;
  L.out0 = out0;
  L.out1 = out1;
  L.shape.chunks_per_row = cols / vec;
  L.shape.in_stride = is;
  L.shape.out_stride = os;
  L.stream = static_cast<hipStream_t>(stream);
  const int64_t total = rows * L.shape.chunks_per_row;
  const int64_t per_block = (int64_t)kBlock * kUnroll;
  const int64_t want = (total + per_block - 1) / per_block;
  const int64_t piece = glu_piece_blocks(want);

  for (int64_t b0 = 0; b0 < want; b0 += piece) {
    const int64_t nb = want - b0 < piece ? want - b0 : piece;
    L.shape.begin = b0 * per_block;
    L.shape.n_chunks = (b0 + nb) * per_block < total ? (b0 + nb) * per_block : total;
    L.blocks = (unsigned)(nb < kMaxBlocks ? nb : kMaxBlocks);
    int32_t st;
    switch (dtype) {
      case ROPE_F32:
        st = bwd ? launch_vec<float, true>(kind, vec, L, dense, long_index)
                 : launch_vec<float, false>(kind, vec, L, dense, long_index);
        break;
      case ROPE_BF16:
        st = bwd ? launch_vec<__bf16, true>(kind, vec, L, dense, long_index)
                 : launch_vec<__bf16, false>(kind, vec, L, dense, long_index);
        break;
      default:
        st = bwd ? launch_vec<_Float16, true>(kind, vec, L, dense, long_index)
                 : launch_vec<_Float16, false>(kind, vec, L, dense, long_index);
    }
    if (st != ROPE_OK) return st;
  }
  return ROPE_OK;
}

}  // namespace

extern "C" {

int32_t glu_fwd(int32_t kind, const void* e, const void* g, void* h, int64_t rows, int64_t cols,
                int64_t in_stride, int64_t out_stride, int32_t dtype, int32_t index_mode,
                void* stream) {
  return glu_launch(false, kind, nullptr, e, g, h, nullptr, rows, cols, in_stride, out_stride,
                    dtype, index_mode, stream);
}

int32_t glu_bwd(int32_t kind, const void* dh, const void* e, const void* g, void* de, void* dg,
                int64_t rows, int64_t cols, int64_t in_stride, int64_t out_stride, int32_t dtype,
                int32_t index_mode, void* stream) {
  return glu_launch(true, kind, dh, e, g, de, dg, rows, cols, in_stride, out_stride, dtype,
                    index_mode, stream);
}

}  // extern "C"
