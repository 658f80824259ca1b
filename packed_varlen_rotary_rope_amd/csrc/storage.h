// storage.h -- element storage for the streaming kernels on gfx950: a chunk of
// VEC consecutive elements moved as one (up to 16-byte) non-temporal access,
// widening to fp32, and round-to-nearest-even narrowing back to the storage type.
// Included by the QK-RoPE and the SwiGLU/GeGLU kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace storage {

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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <int BYTES> struct WordOf;
template <> struct WordOf<16> { typedef u32x4 type; };
template <> struct WordOf<8> { typedef u32x2 type; };
template <> struct WordOf<4> { typedef uint32_t type; };
template <> struct WordOf<2> { typedef uint16_t type; };

// Streaming (non-temporal) access to one chunk.
template <typename T, int VEC>
__device__ inline Chunk<T, VEC> load_chunk(const T* p) {
  typedef typename WordOf<VEC * sizeof(T)>::type W;
  return __builtin_bit_cast(Chunk<T, VEC>, __builtin_nontemporal_load(reinterpret_cast<const W*>(p)));
}
template <typename T, int VEC>
__device__ inline void store_chunk(T* p, const Chunk<T, VEC>& c) {
  typedef typename WordOf<VEC * sizeof(T)>::type W;
  __builtin_nontemporal_store(__builtin_bit_cast(W, c), reinterpret_cast<W*>(p));
}

}  // namespace storage
