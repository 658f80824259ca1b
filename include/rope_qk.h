/*
 * rope_qk.h -- C ABI of the fused, in-place, packed variable-length QK rotary
 * position embedding (RoPE) library for AMD Instinct MI355X (gfx950).
 *
 * What the operation is (web pages cited by title and section):
 *  - Unsloth, "Entrainement des LLM 3 fois plus rapide avec les noyaux Unsloth +
 *    le packing", section "Kernel Triton QK RoPE fusionne avec packing": one
 *    kernel rotates both Q and K, in place, as x*cos + rotate_half(x)*sin, where
 *    rotate_half(x) = x @ R and R = [[0, I], [-I, 0]]; the backward pass applies
 *    R transposed, which is the same rotation with sin negated. Variable-length
 *    (packed) batches are supported.
 *  - same page, section "Packing non contamine", and Databricks, "Reduire le
 *    temps d'entrainement de Qwen de 6x sur AI Runtime", section "Mise en lots,
 *    tokenisation et padding": samples are packed into one token dimension and
 *    the RoPE positions restart at every sample, so no sample sees another's
 *    positions.
 *  - same Unsloth page, section "Indexage int64 pour les kernels Triton": 64-bit
 *    offsets are compiled in only where the tensors need them.
 *  - TRL guide "Entrainement au-dela de 1 M de jetons", YaRN section: theta is
 *    the model's rope_theta (1e6 for Qwen3).
 *
 * Semantics. Q is [T, Hq, D] and K is [T, Hkv, D], row-major and contiguous, in
 * one dtype. Token t belongs to sequence s when cu_seqlens[s] <= t <
 * cu_seqlens[s+1]; its position is p = t - cu_seqlens[s]. Tokens before
 * cu_seqlens[0], at or after cu_seqlens[num_seqs], or with p >= seqused[s] (when
 * seqused is given) are left bit-for-bit untouched. For every other token,
 * every head and every j < D/2:
 *     inv_freq[j] = theta^(-2j/D) rounded once to fp32
 *     a = fp32(p) * inv_freq[j]                      (one fp32 multiply)
 *     c, s = cos(a), sin(a) correctly rounded to fp32; s is negated backward
 *     x1 = X[t,h,j], x2 = X[t,h,j+D/2]  (widened to fp32)
 *     X[t,h,j]       = round(x1*c - x2*s)
 *     X[t,h,j+D/2]   = round(x2*c + x1*s)
 * where the products are formed with an FMA-compensated (Kahan) scheme, so the
 * fp32 value is within 2 fp32 ulps of the exact real result before it is rounded
 * to the storage dtype (round to nearest even).
 *
 * Ownership and threading. The caller owns every buffer. The library allocates
 * nothing, keeps no state between calls, never synchronizes and never reads
 * device memory from the host. Calls only enqueue work on `stream` (a
 * hipStream_t; NULL means the null stream) and return. Calls on different
 * streams are independent; the library is reentrant. A pass is one kernel launch,
 * except that the default geometry issues a long pass (Q holding at least four
 * times K's head-row groups, 655360 workgroups or more, e.g. 131072 tokens of 32 + 8
 * heads at D = 128) as several launches of the same kernel, one after another on
 * the same stream, over consecutive token ranges: results are identical, and the
 * shorter launches keep the GPU's eight dies streaming neighbouring addresses.
 *
 * Errors. Arguments are validated on the host before any HIP call; a rejected
 * call enqueues nothing. A launch failure reported by hipGetLastError maps to
 * ROPE_ELAUNCH (when a later launch of a multi-launch pass is rejected, the
 * earlier token ranges have been enqueued). Faults during execution surface at
 * the caller's next synchronization. Not validated (undefined behaviour): the
 * contents of cu_seqlens (must be non-decreasing and within [0, T] for meaningful
 * results; any contents stay memory-safe, because a work item only touches its
 * own token's rows), and aliasing between Q and K.
 */
#ifndef ROPE_QK_H
#define ROPE_QK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ROPE_QK_ABI_VERSION 5

/* Storage dtype of Q and K (computation is fp32 in every case). */
typedef enum rope_dtype { ROPE_F32 = 0, ROPE_BF16 = 1, ROPE_F16 = 2 } rope_dtype;

typedef enum rope_status {
  ROPE_OK = 0,
  ROPE_EINVAL = -1,       /* an argument is out of range or a required pointer is NULL */
  ROPE_EUNSUPPORTED = -2, /* unknown dtype */
  ROPE_ELAUNCH = -3       /* the HIP runtime rejected the launch */
} rope_status;

/* Index-width choice for rope_qk_apply. AUTO selects 64-bit offsets exactly when
 * T * (Hq + Hkv) * D >= 2^31 (the int64 specialization), 32-bit otherwise. */
typedef enum rope_index_mode { ROPE_INDEX_AUTO = 0, ROPE_INDEX_32 = 1, ROPE_INDEX_64 = 2 } rope_index_mode;

/* Forward RoPE on Q and K in place, in one kernel launch (a long pass: several, see
 * above).
 *  q, k        device pointers to Q[T, Hq, D] and K[T, Hkv, D]; may be NULL only if
 *              that tensor has no elements (T == 0 or its head count is 0)
 *  T           rows (tokens) of Q and K, >= 0
 *  Hq, Hkv     head counts, 0..4096, not both 0 unless T == 0
 *  D           head size: even, 2..512
 *  cu_seqlens  device int32[num_seqs + 1], cumulative sequence starts
 *  num_seqs    >= 0; with 0 nothing is rotated and cu_seqlens may be NULL
 *  seqused     device int32[num_seqs] or NULL: rotate only the first seqused[s]
 *              tokens of sequence s (padded layouts)
 *  theta       rope_theta, finite and >= 1
 *  dtype       a rope_dtype value
 *  stream      hipStream_t to enqueue on (NULL: null stream)
 * Returns ROPE_OK, ROPE_EINVAL, ROPE_EUNSUPPORTED or ROPE_ELAUNCH. */
int32_t rope_qk_fwd(void* q, void* k, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                    const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                    double theta, int32_t dtype, void* stream);

/* Backward RoPE on the gradients dQ and dK in place: the transpose of the forward
 * rotation, i.e. the forward with sin negated (Unsloth page, fused QK RoPE
 * section). Needs only cu_seqlens and theta, no saved Q or K. Arguments as in
 * rope_qk_fwd, with q, k replaced by dq, dk. */
int32_t rope_qk_bwd(void* dq, void* dk, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                    const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                    double theta, int32_t dtype, void* stream);

/* The general entry point behind rope_qk_fwd / rope_qk_bwd.
 *  direction        +1 forward, -1 backward (anything else: ROPE_EINVAL)
 *  index_mode       a rope_index_mode; ROPE_INDEX_32 is rejected (ROPE_EINVAL)
 *                   when the tensors need 64-bit offsets
 *  tokens_per_wave  launch geometry. 0: the library's default, one 64-lane
 *                   workgroup per token and group of consecutive head rows (8 rows
 *                   for D = 128 in bf16), which evaluates the token's cos/sin once
 *                   per group; one wave per token instead when seqused is given
 *                   (padded layouts skip many rows, which that geometry passes over
 *                   more cheaply; rope_qk_apply_padded spends nothing on them) or
 *                   when the row layout or the grid size rules the row groups out
 *                   (e.g. D = 384 in 16-bit storage: 24 chunks of 16 bytes per half
 *                   row, too few rows per group; half rows that are not whole
 *                   128-byte lines with at most 15 such chunks, e.g. D = 64, 80, 96,
 *                   192, move through LDS in whole lines instead).
 *                   1..1024: each 64-lane wave rotates this many consecutive
 *                   tokens, one at a time, all Q and K heads of each, evaluating
 *                   each token's cos/sin once. Results do not depend on it.
 * Other arguments as in rope_qk_fwd. */
int32_t rope_qk_apply(void* q, void* k, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                      const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                      double theta, int32_t dtype, int32_t direction, int32_t index_mode,
                      int32_t tokens_per_wave, void* stream);

/* The most general entry point: positions from explicit ids or from cu_seqlens
 * with per-sequence offsets, and linear position interpolation.
 *  seq_offsets   device int32[num_seqs] or NULL: added to every position of
 *                sequence s (a context-parallel shard of a longer sequence passes
 *                the global position of its first token). A token whose shifted
 *                position falls outside [0, 2^31) is left untouched.
 *  position_ids  device int32[T] or NULL: when given, token t has position
 *                position_ids[t] and cu_seqlens, num_seqs, seqused and seq_offsets
 *                are ignored (may be NULL / 0); a negative id leaves the token
 *                untouched. This is the per-example position_ids representation of
 *                a 1-D packed batch (Databricks, "Reduire le temps d'entrainement de
 *                Qwen de 6x sur AI Runtime", section "Mise en lots, tokenisation et
 *                padding").
 *  pos_scale     linear position interpolation factor s, rounded to fp32, finite
 *                and >= 1: the angle becomes fp32(fp32(pos) / s) * inv_freq[j], so
 *                position s*p rotates exactly like position p (TRL guide
 *                "Entrainement au-dela de 1 M de jetons", YaRN section: with factor 4,
 *                position 100000 is treated as position 25000). 1 = no scaling.
 *  q_token_stride, k_token_stride
 *                elements from one token's first head to the next token's (0 = Hq*D
 *                resp. Hkv*D, a contiguous [T, H, D] tensor). Heads of one token stay
 *                contiguous; a larger stride lets q and k be views into a fused QKV
 *                projection output [T, (Hq + 2*Hkv)*D], rotated in place with V and
 *                any gaps untouched. q and k must not overlap. A stride below H*D
 *                (tokens would overlap) or with T*stride above 2^48 elements is
 *                ROPE_EINVAL. The widest access the library uses is the largest of
 *                16/8/4 bytes that divides the half row, both base addresses and both
 *                strides in bytes.
 * Other arguments as in rope_qk_apply. */
int32_t rope_qk_apply_ex(void* q, void* k, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                         int64_t q_token_stride, int64_t k_token_stride,
                         const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                         const int32_t* seq_offsets, const int32_t* position_ids, double theta,
                         double pos_scale, int32_t dtype, int32_t direction, int32_t index_mode,
                         int32_t tokens_per_wave, void* stream);

/* rope_qk_apply_ex with caller-supplied cos/sin tables instead of theta: a
 * cos/sin cache computed once and reused across calls, or the tables of a RoPE
 * variant whose frequencies this library does not generate. The rotation, its
 * backward (sin negated), the pairing, the positions and the untouched tokens
 * are those of rope_qk_apply_ex (Unsloth page, fused QK RoPE section; positions
 * per "Packing non contamine").
 *  cos_tab, sin_tab  device float[tab_rows * (D/2)], row-major: row p holds the
 *                    cos / sin of position p for frequencies j < D/2 (the layout
 *                    rope_cos_sin writes with max_pos = tab_rows). Read only.
 *  tab_rows          rows of both tables, >= 1. A token whose position is >=
 *                    tab_rows is left untouched (no row exists for it).
 * There is no theta or pos_scale: the tables already hold the angles' cos/sin.
 * Rotating with the tables rope_cos_sin writes for (theta, D) gives results bit
 * for bit equal to rope_qk_apply_ex with that theta and pos_scale 1.
 * Errors: ROPE_EINVAL if either table is NULL or tab_rows < 1, otherwise as in
 * rope_qk_apply_ex. Other arguments as in rope_qk_apply_ex. */
int32_t rope_qk_apply_table(void* q, void* k, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                            int64_t q_token_stride, int64_t k_token_stride,
                            const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                            const int32_t* seq_offsets, const int32_t* position_ids,
                            const float* cos_tab, const float* sin_tab, int32_t tab_rows,
                            int32_t dtype, int32_t direction, int32_t index_mode,
                            int32_t tokens_per_wave, void* stream);

/* rope_qk_apply_ex for a padded layout whose rotated tokens the caller has
 * counted: the launch covers only those tokens, so padded rows cost no work at
 * all (Unsloth page, section "Pourquoi le remplissage est-il necessaire et gain
 * de vitesse mathematique": padding rows are waste; section "Packing non
 * contamine": positions restart per sample). The tokens rotated, their positions
 * and the results are those of rope_qk_apply_ex with the same cu_seqlens,
 * seqused and seq_offsets, bit for bit, whenever cu_valid and valid_tokens match
 * them; the extra arguments only shape the launch.
 *  cu_valid      device int32[num_seqs + 1]: cu_valid[0] = 0 and cu_valid[s+1] =
 *                cu_valid[s] + used(s), used(s) = min(seqused[s], cu_seqlens[s+1]
 *                - cu_seqlens[s]) clamped at 0 (the sequence length when seqused
 *                is NULL): the running count of rotated tokens, the same for every
 *                layer of a batch. rope_valid_prefix writes it.
 *  valid_tokens  host count of rotated tokens, cu_valid[num_seqs]; 0..T.
 * When they do not match, memory stays safe and no token is rotated twice or
 * with a wrong position, but tokens outside the ranges they describe may be
 * left untouched. Where the row-group geometry does not apply (nc does not
 * divide 64, a token stride of 2^32 elements or more, or a grid beyond the
 * dispatch limit) the call runs the seqused launch of rope_qk_apply_ex instead,
 * which rotates every token seqused describes.
 * Errors: ROPE_EINVAL for valid_tokens < 0 or > T, or a NULL cu_valid with
 * valid_tokens > 0 (valid_tokens == 0 enqueues nothing); otherwise as in
 * rope_qk_apply_ex. Other arguments as in rope_qk_apply_ex. */
int32_t rope_qk_apply_padded(void* q, void* k, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                             int64_t q_token_stride, int64_t k_token_stride,
                             const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                             const int32_t* cu_valid, int64_t valid_tokens,
                             const int32_t* seq_offsets, double theta, double pos_scale,
                             int32_t dtype, int32_t direction, int32_t index_mode, void* stream);

/* Forward / backward RoPE with explicit positions: position_ids is a device
 * int32[T] (required when T > 0); negative ids leave their token untouched.
 * Other arguments as in rope_qk_fwd. */
int32_t rope_qk_fwd_pos(void* q, void* k, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                        const int32_t* position_ids, double theta, int32_t dtype, void* stream);
int32_t rope_qk_bwd_pos(void* dq, void* dk, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                        const int32_t* position_ids, double theta, int32_t dtype, void* stream);

/* Export of the token -> (position, sequence) map the kernels use (test hook,
 * same device code). pos_out, seq_out: device int32[T] (either may be NULL);
 * -1 for tokens that are left untouched. With num_seqs == 0 every token is
 * untouched and cu_seqlens may be NULL (it is not read). Validation as in
 * rope_qk_fwd. */
int32_t rope_positions(const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                       int64_t T, int32_t* pos_out, int32_t* seq_out, void* stream);

/* rope_positions with the position sources of rope_qk_apply_ex (seq_offsets,
 * position_ids). seq_out is -1 for every token when position_ids is given. */
int32_t rope_positions_ex(const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                          const int32_t* seq_offsets, const int32_t* position_ids, int64_t T,
                          int32_t* pos_out, int32_t* seq_out, void* stream);

/* The cu_valid array of rope_qk_apply_padded, on the device: cu_valid_out[0] = 0
 * and cu_valid_out[s+1] = cu_valid_out[s] + min(seqused[s], cu_seqlens[s+1] -
 * cu_seqlens[s]), each term clamped at 0 (the length alone when seqused is NULL),
 * saturated at INT32_MAX. One small launch per batch.
 *  cu_seqlens     device int32[num_seqs + 1] (not read when num_seqs == 0)
 *  seqused        device int32[num_seqs] or NULL
 *  cu_valid_out   device int32[num_seqs + 1], owned by the caller
 * Returns ROPE_OK, ROPE_EINVAL (num_seqs < 0 or INT32_MAX, a NULL output, or a
 * NULL cu_seqlens with num_seqs > 0) or ROPE_ELAUNCH. */
int32_t rope_valid_prefix(const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                          int32_t* cu_valid_out, void* stream);

/* The fp32 cos/sin the kernels use, as a table (same device code; Unsloth page,
 * fused QK RoPE section: the cos and sin of the rotation): for every position
 * p < max_pos and every frequency j < D/2, cos_out[p*(D/2) + j] and
 * sin_out[p*(D/2) + j] receive the correctly rounded fp32 cos and sin of the
 * angle fp32(p) * inv_freq[j]. This is the row layout rope_qk_apply_table reads.
 *  max_pos           rows, >= 0 (0: nothing is written)
 *  D, theta          as in rope_qk_fwd
 *  cos_out, sin_out  device float[max_pos * (D/2)], owned by the caller
 * Returns ROPE_OK, ROPE_EINVAL (max_pos < 0, bad D or theta, a NULL output with
 * max_pos > 0) or ROPE_ELAUNCH. */
int32_t rope_cos_sin(int32_t max_pos, int32_t D, double theta, float* cos_out, float* sin_out,
                     void* stream);

/* The same values for an arbitrary list of positions, with linear position
 * interpolation: row i is position positions[i] (device int32[n], each >= 0),
 * angle fp32(fp32(positions[i]) / pos_scale) * inv_freq[j] (pos_scale as in
 * rope_qk_apply_ex; 1 = none). cos_out, sin_out: device float[n * (D/2)].
 * Errors as in rope_cos_sin, and ROPE_EINVAL for n < 0, a NULL positions array
 * with n > 0, or a bad pos_scale. */
int32_t rope_cos_sin_at(const int32_t* positions, int64_t n, int32_t D, double theta,
                        double pos_scale, float* cos_out, float* sin_out, void* stream);

/* Host-only: the fp32 inverse frequencies theta^(-2j/D), j < D/2, written to the
 * host array out[D/2]. Same validation of D and theta as rope_qk_fwd. */
int32_t rope_inv_freq(double theta, int32_t D, float* out);

/* Static description of a status code. */
const char* rope_status_str(int32_t status);

/* ROPE_QK_ABI_VERSION of the library. */
int32_t rope_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ROPE_QK_H */
