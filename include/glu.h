/*
 * glu.h -- C ABI of the gated MLP activation kernels (SwiGLU, GeGLU) on MI355X,
 * exported by the same shared library as rope_qk.h (librope_qk.so).
 *
 * Page: Unsloth, "Entrainement des LLM 3 fois plus rapide avec les noyaux Unsloth
 * + le packing" -- the opening list says the SwiGLU and GeGLU MLP kernels gained
 * int64 indexing for long contexts, and section "Indexage int64 pour les kernels
 * Triton" says why and how: at a 500K-token context their element offsets no
 * longer fit 32 bits, so 64-bit offsets are a compile-time specialization,
 * chosen only when needed because they cost time on short inputs. The page names
 * the activations without writing them out; the standard definitions are used:
 *   SwiGLU (Shazeer 2020)      act(e) = e * sigmoid(e)
 *   GeGLU, exact (Hendrycks & Gimpel 2016)  act(e) = e * Phi(e), Phi the normal CDF
 *   GeGLU, tanh approximation  act(e) = e/2 * (1 + tanh(sqrt(2/pi)(e + 0.044715 e^3)))
 * Forward h = act(e) * g; backward from the upstream gradient dh:
 *   de = dh * g * act'(e),  dg = dh * act(e).
 *
 * Tensors are 2-D [rows, cols] in one storage dtype (rope_dtype: f32, bf16 or
 * f16), row-major with contiguous columns; each group of tensors has a row
 * stride in elements (0 = cols, i.e. dense). e and g -- and de, dg in the
 * backward -- share in_stride: they may be two dense [rows, cols] tensors or the
 * two halves of one fused gate/up projection output [rows, 2*cols]
 * (in_stride = 2*cols). h and dh use out_stride. Arithmetic is fp32 with one
 * rounding to the storage dtype per output; the library allocates nothing, keeps
 * no state and never synchronizes. Calls on one stream run in order. A call is one
 * kernel launch, except that a call of 65536 workgroups or more (each covers 1024
 * chunks of 16 bytes or less, e.g. 2^26 bf16 elements per 8192 workgroups) goes
 * out as several launches of about 32768 workgroups, one after another on the same
 * stream, over consecutive ranges of the elements: results are identical, and the
 * shorter launches keep the GPU's eight dies streaming neighbouring addresses.
 *
 * Aliasing: an output may be the same memory as one of its own-shape inputs at
 * the same address and stride (h over e or g in the forward; de over e and dg
 * over g in the backward: a fully in-place backward). Any other overlap is
 * undefined.
 *
 * Errors (host-side validation before any HIP call): ROPE_EINVAL for an unknown
 * kind, rows or cols < 0, a stride below cols, a NULL pointer with rows*cols > 0,
 * a span rows*stride above 2^48 elements, or index_mode ROPE_INDEX_32 when 64-bit
 * offsets are needed; ROPE_EUNSUPPORTED for an unknown dtype; ROPE_ELAUNCH if
 * a launch fails (the earlier ranges of a multi-launch call stay enqueued).
 * rows*cols == 0 returns ROPE_OK without launching.
 *
 * index_mode (rope_index_mode): ROPE_INDEX_AUTO picks 64-bit offsets when some
 * element offset of the call reaches 2^31, and otherwise 32-bit offsets, except
 * for the tanh-GeGLU backward, whose 64-bit instance is the faster one on gfx950
 * even where every offset fits; ROPE_INDEX_32 forces 32-bit offsets (rejected when
 * they do not fit) and ROPE_INDEX_64 64-bit ones. The results are identical either
 * way.
 */
#ifndef GLU_H
#define GLU_H

#include <stdint.h>

#include "rope_qk.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GLU_SWIGLU = 0, GLU_GEGLU = 1, GLU_GEGLU_TANH = 2 } glu_kind;

/* h[r, c] = act(e[r, c]) * g[r, c] for r < rows, c < cols.
 *  e, g       device, read; rows in_stride elements apart (0 = cols)
 *  h          device, written; rows out_stride elements apart (0 = cols)
 *  stream     hipStream_t as void* (NULL = the default stream) */
int32_t glu_fwd(int32_t kind, const void* e, const void* g, void* h, int64_t rows, int64_t cols,
                int64_t in_stride, int64_t out_stride, int32_t dtype, int32_t index_mode,
                void* stream);

/* de = dh * g * act'(e), dg = dh * act(e).
 *  dh         device, read; rows out_stride elements apart (0 = cols)
 *  e, g       device, read; rows in_stride elements apart (0 = cols)
 *  de, dg     device, written with the layout of e and g (in_stride); de may be e
 *             and dg may be g (in place). */
int32_t glu_bwd(int32_t kind, const void* dh, const void* e, const void* g, void* de, void* dg,
                int64_t rows, int64_t cols, int64_t in_stride, int64_t out_stride, int32_t dtype,
                int32_t index_mode, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GLU_H */
