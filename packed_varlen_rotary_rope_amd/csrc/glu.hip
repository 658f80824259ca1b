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
// sigmoid(z) = 1/(1+t) or t/(1+t), t = exp(-|z|)); Phi(e) = erfc(-e/sqrt 2)/2
// keeps its relative accuracy in the negative tail. The derivative act'(e) has a
// root e0 where its direct formula cancels; within |e - e0| <= 1/4 it is taken
// from a degree-10 Taylor polynomial around e0 (glu_constants.h). Every output is
// then within a few fp32 ulps of the exact value, plus the conditioning of the
// tail (about e^2 ulps for the erfc and tanh forms), before its one rounding to
// the storage dtype.
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
  int64_t n_chunks;              // rows * chunks_per_row
  int64_t chunks_per_row;        // cols / VEC
  int64_t in_stride, out_stride;  // elements between rows (e, g, de, dg / h, dh)
};

// ---- activations in fp32 -----------------------------------------------------------

// sigmoid(z) and 1 - sigmoid(z) from t = exp(-|z|): 1/(1+t) and t/(1+t), each the
// larger or the smaller by the sign of z. rcp is within 1 ulp.
__device__ inline void sigmoid_pair(float z, float& s, float& sc) {
  const float t = expf(-fabsf(z));
  const float r = __builtin_amdgcn_rcpf(1.0f + t);
  const float small = t * r;
  s = z >= 0.0f ? r : small;
  sc = z >= 0.0f ? small : r;
}

// act'(e0 + d) near the root e0 of the derivative: d * sum_{k<K} a[k] d^k.
__device__ inline float root_poly(float e, float root_hi, float root_lo, const float (&a)[kRootDegree],
                                  float direct) {
  const float d = (e - root_hi) - root_lo;  // e - root_hi is exact inside the window
  float p = a[kRootDegree - 1];
#pragma unroll
  for (int k = kRootDegree - 2; k >= 0; --k) p = __builtin_fmaf(p, d, a[k]);
  return fabsf(d) <= kRootWindow ? p * d : direct;
}

template <int KIND>
__device__ inline float act_fwd(float e) {
  if constexpr (KIND == GLU_SWIGLU) {
    float s, sc;
    sigmoid_pair(e, s, sc);
    return e * s;
  } else if constexpr (KIND == GLU_GEGLU) {
    return e * (0.5f * erfcf(-e * kInvSqrt2));
  } else {
    // 2u = e (A + B e^2); |e| > 64 gives the same sigmoid (0 or 1) without overflow
    const float ec = fminf(fmaxf(e, -64.0f), 64.0f);
    const float z = ec * __builtin_fmaf(kTanhB, ec * ec, kTanhA);
    float s, sc;
    sigmoid_pair(z, s, sc);
    return e * s;
  }
}

// act(e) and act'(e) together (the backward needs both).
template <int KIND>
__device__ inline void act_bwd(float e, float& a, float& da) {
  if constexpr (KIND == GLU_SWIGLU) {
    float s, sc;
    sigmoid_pair(e, s, sc);
    a = e * s;
    // s (1 + e (1 - s))
    const float direct = s * __builtin_fmaf(e, sc, 1.0f);
    da = root_poly(e, kSiluRootHi, kSiluRootLo, kSiluPoly, direct);
  } else if constexpr (KIND == GLU_GEGLU) {
    const float cdf = 0.5f * erfcf(-e * kInvSqrt2);
    const float pdf = expf(-0.5f * e * e) * kInvSqrt2Pi;
    a = e * cdf;
    // Phi + e phi
    const float direct = __builtin_fmaf(e, pdf, cdf);
    da = root_poly(e, kGeluRootHi, kGeluRootLo, kGeluPoly, direct);
  } else {
    const float ec = fminf(fmaxf(e, -64.0f), 64.0f);
    const float e2 = ec * ec;
    const float z = ec * __builtin_fmaf(kTanhB, e2, kTanhA);
    const float zp = __builtin_fmaf(kTanhC, e2, kTanhA);
    float s, sc;
    sigmoid_pair(z, s, sc);
    a = e * s;
    // s (1 + e z' (1 - s))
    const float direct = s * __builtin_fmaf(ec * zp, sc, 1.0f);
    da = root_poly(e, kGeluTanhRootHi, kGeluTanhRootLo, kGeluTanhPoly, direct);
  }
}

// ---- the kernel ------------------------------------------------------------------------

// [U-int64]: Index is uint32_t when every offset of the launch is below 2^31 (the
// host checks), int64_t otherwise.
template <typename T, int VEC, int KIND, bool BWD, bool DENSE, typename Index>
// No __restrict__: an output may be the memory of one of the inputs (in place).
__global__ __launch_bounds__(kBlock) void glu_kernel(const T* dh, const T* e, const T* g, T* out0,
                                                     T* out1, const GluShape s) {
  using C = Chunk<T, VEC>;
  const Index n = (Index)s.n_chunks;
  const Index step = (Index)gridDim.x * (Index)(kBlock * kUnroll);
  for (Index base = (Index)blockIdx.x * (Index)(kBlock * kUnroll); base < n; base += step) {
    C ce[kUnroll], cg[kUnroll], cd[kUnroll];
    Index in_off[kUnroll], out_off[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const Index c = base + (Index)(u * kBlock) + (Index)threadIdx.x;
      if (c < n) {
        if constexpr (DENSE) {
          in_off[u] = c * VEC;
          out_off[u] = c * VEC;
        } else {
          const Index row = c / (Index)s.chunks_per_row;
          const Index col = (c - row * (Index)s.chunks_per_row) * VEC;
          in_off[u] = row * (Index)s.in_stride + col;
          out_off[u] = row * (Index)s.out_stride + col;
        }
        ce[u] = load_chunk<T, VEC>(e + in_off[u]);
        cg[u] = load_chunk<T, VEC>(g + in_off[u]);
        if constexpr (BWD) cd[u] = load_chunk<T, VEC>(dh + out_off[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const Index c = base + (Index)(u * kBlock) + (Index)threadIdx.x;
      if (c < n) {
        if constexpr (!BWD) {
          float h[VEC];
#pragma unroll
          for (int j = 0; j < VEC; ++j) h[j] = act_fwd<KIND>(to_f32(ce[u].v[j])) * to_f32(cg[u].v[j]);
          C ch;
          narrow(h, ch);
          store_chunk<T, VEC>(out0 + out_off[u], ch);
        } else {
          float de[VEC], dg[VEC];
#pragma unroll
          for (int j = 0; j < VEC; ++j) {
            float a, da;
            act_bwd<KIND>(to_f32(ce[u].v[j]), a, da);
            const float up = to_f32(cd[u].v[j]);
            de[j] = up * to_f32(cg[u].v[j]) * da;
            dg[j] = up * a;
          }
          C cde, cdg;
          narrow(de, cde);
          narrow(dg, cdg);
          store_chunk<T, VEC>(out0 + in_off[u], cde);
          store_chunk<T, VEC>(out1 + in_off[u], cdg);
        }
      }
    }
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

template <typename T, int VEC, int KIND, bool BWD, bool DENSE, typename Index>
int32_t launch_one(const Launch& L) {
  hipLaunchKernelGGL((glu_kernel<T, VEC, KIND, BWD, DENSE, Index>), dim3(L.blocks), dim3(kBlock), 0,
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
  const bool long_index = needs_long || index_mode == ROPE_INDEX_64;

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
  L.shape.n_chunks = rows * L.shape.chunks_per_row;
  L.shape.in_stride = is;
  L.shape.out_stride = os;
  const int64_t per_block = (int64_t)kBlock * kUnroll;
  const int64_t want = (L.shape.n_chunks + per_block - 1) / per_block;
  L.blocks = (unsigned)(want < kMaxBlocks ? want : kMaxBlocks);
  L.stream = static_cast<hipStream_t>(stream);

  switch (dtype) {
    case ROPE_F32:
      return bwd ? launch_vec<float, true>(kind, vec, L, dense, long_index)
                 : launch_vec<float, false>(kind, vec, L, dense, long_index);
    case ROPE_BF16:
      return bwd ? launch_vec<__bf16, true>(kind, vec, L, dense, long_index)
                 : launch_vec<__bf16, false>(kind, vec, L, dense, long_index);
    default:
      return bwd ? launch_vec<_Float16, true>(kind, vec, L, dense, long_index)
                 : launch_vec<_Float16, false>(kind, vec, L, dense, long_index);
  }
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
