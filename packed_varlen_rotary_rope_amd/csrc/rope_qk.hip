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
// no MFMA). A chunk is VEC consecutive elements of the first half of a head row
// (16 bytes: VEC = 8 for bf16/f16, 4 for fp32) together with the matching VEC
// elements of the second half, D/2 further on; the lane that loads a chunk pair
// rotates it and stores it back, so the in-place update needs no synchronization
// between lanes. Loads and stores are non-temporal: the data is streamed once; the
// row-group kernel's stores also write through L2 at device scope.
// Two kernels, one launch per pass either way (long passes of the row-group kernel
// as several launches over consecutive token ranges, see group_piece_tokens):
//  * rope_qk_group_kernel (the default): one 64-lane workgroup per (token, group
//    of group_rows(nc) head rows: 64 / nc, rounded down, to whole 128-byte lines
//    where that keeps 48 lanes busy), Q's groups then K's; for D = 128 in bf16 a
//    group is 8 rows = 2 KB, one chunk pair per lane. The wave maps its token to (sequence,
//    position) with a wave-uniform binary search over cu_seqlens [U-Pack],
//    issues its row loads, evaluates the token's correctly rounded fp32 cos/sin
//    (one frequency per lane) into a wave-local LDS table while the loads are in
//    flight, rotates in fp32 and stores.
//  * rope_qk_kernel: a 64-lane wave walks whole tokens (tokens_per_wave of them),
//    evaluating each token's cos/sin once and rotating its Q rows then its K rows
//    [U-Group]; used for padded layouts (seqused), head sizes whose chunk count
//    neither divides 64 nor fits the staged instance (16-byte chunks, at most 10
//    per half row), and when the caller chooses tokens per wave.
// Both take cos/sin from caller-supplied tables instead (TABLE instances) for
// rope_qk_apply_table.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/rope_qk.h"
#include "cr_sincos.h"
#include "fast_div.h"
#include "storage.h"

namespace {

using namespace storage;

constexpr int kBlock = 256;     // threads per workgroup of the export kernels
// The token kernel: one wave per workgroup, so a wave whose tokens are all skipped
// (padded rows) frees its slot at once. Measured on padded layouts (bf16, 32 + 8
// heads): 8 x 2048 rows 32.0 us against 33.0 with four waves per workgroup (32.7
// with two); 32 x 4096 rows 263 against 271 us.
constexpr int kTokenBlock = 64;
constexpr int kWaves = kTokenBlock / 64;  // waves per workgroup, one token at a time each
constexpr int kMaxHalf = 256;   // D <= 512
constexpr int kMaxHeads = 4096;
constexpr int kUnroll = 4;      // wave steps (row groups) whose loads are in flight together
constexpr int kMaxTokensPerWave = 1024;
// A dispatch's grid size in work-items is a 32-bit field: blocks * block size < 2^32.
constexpr int64_t kMaxBlocksX = (int64_t)0xffffffffu / kBlock;
constexpr int64_t kMaxTokenBlocks = (int64_t)0xffffffffu / kTokenBlock;

struct RopeParams {
  alignas(16) float inv_freq[kMaxHalf];
  int64_t T;
  int32_t num_seqs;
  int32_t Hq, Hkv, D;
  int64_t q_stride, k_stride;  // elements between consecutive tokens of Q / K
  int32_t nc;   // chunks per half row: (D/2) / VEC
  int32_t tpw;  // tokens per wave
  float sin_sign;
  float pos_scale;  // linear position interpolation: positions divided by this (1 = none)
  // row-group kernel only, set by the host when it launches that kernel
  uint32_t gq, gk;           // row groups of Q and of K per token
  uint32_t nc_shift;         // log2(nc); nc divides 64
  fastdiv::FastDiv groups;   // division by gq + gk
  // caller-supplied cos/sin tables [tab_rows, D/2] (table kernels only)
  const float* tab_cos;
  const float* tab_sin;
  int32_t tab_rows;
};

struct CosSinParams {
  float inv_freq[kMaxHalf];
  float pos_scale;
};

// Where a token's position comes from: explicit position ids, or its offset in its
// cu_seqlens sequence (optionally cut by seqused and shifted by a per-sequence
// offset, as a context-parallel shard of a longer sequence needs). cu_valid is set
// only for compact launches over a padded layout (compact_position).
struct PosSource {
  const int32_t* cu;
  const int32_t* seqused;
  const int32_t* seq_offsets;
  const int32_t* position_ids;
  int32_t num_seqs;
  const int32_t* cu_valid;
};

// ---- a1: token -> (sequence, position) [U-Pack] ------------------------------------
// Sequence s is the last index with cu[s] <= t (upper bound minus one). The token
// is rotated if 0 <= s < num_seqs and, with seqused, t - cu[s] < seqused[s].
// Returns the position, or -1 for an untouched token (then *seq_out = -1).
// I is the token index type: int32_t where every token index of the launch fits
// (the search then compares in 32 bits), int64_t otherwise.
template <typename I>
__device__ inline int32_t token_position(const int32_t* __restrict__ cu, int32_t num_seqs,
                                         const int32_t* __restrict__ seqused, I t,
                                         int32_t* seq_out) {
  int32_t first = 0;
  int32_t count = num_seqs + 1;
  while (count > 0) {
    const int32_t step = count >> 1;
    const int32_t it = first + step;
    if ((I)cu[it] <= t) {
      first = it + 1;
      count -= step + 1;
    } else {
      count = step;
    }
  }
  const int32_t s = first - 1;
  *seq_out = -1;
  if (s < 0 || s >= num_seqs) return -1;
  const int64_t p = (int64_t)t - (int64_t)cu[s];
  if (seqused != nullptr && p >= (int64_t)seqused[s]) return -1;
  *seq_out = s;
  return (int32_t)p;
}

// Position of token t from any source, or -1 (untouched). With explicit ids a
// negative id leaves the token untouched; with per-sequence offsets a shifted
// position outside [0, 2^31) does.
template <typename I>
__device__ inline int32_t resolve_position(const PosSource& ps, I t, int32_t* seq_out) {
  if (ps.position_ids != nullptr) {
    *seq_out = -1;
    const int32_t p = ps.position_ids[t];
    return p < 0 ? -1 : p;
  }
  const int32_t p = token_position(ps.cu, ps.num_seqs, ps.seqused, t, seq_out);
  if (p < 0 || ps.seq_offsets == nullptr) return p;
  const int64_t shifted = (int64_t)p + (int64_t)ps.seq_offsets[*seq_out];
  if (shifted < 0 || shifted > (int64_t)INT32_MAX) {
    *seq_out = -1;
    return -1;
  }
  return (int32_t)shifted;
}

// Compact launches over a padded layout count only the rotated tokens: token index
// v of the launch is the v-th rotated token, sequence by sequence, and
// cu_valid[s] is the number of rotated tokens before sequence s (the running sum
// of min(seqused[s], sequence length)). So v lies in the sequence s with the last
// cu_valid[s] <= v (the search above, over cu_valid), at position p = v -
// cu_valid[s], in row cu[s] + p. Returns the position and sets *row, or returns -1
// when v lies past the rotated tokens, or when the metadata puts the row outside
// sequence s's rotated prefix or outside [0, T): nothing is touched then, so any
// metadata stays memory-safe, and no row is rotated twice (p is one-to-one in v).
// cu_valid is passed on its own (it is a preloaded kernel argument; ps.cu_valid
// holds the same pointer).
__device__ inline int32_t compact_position(const PosSource& ps, const int32_t* __restrict__ cu_valid,
                                           int32_t num_seqs, int32_t v, int64_t T, int64_t* row) {
  int32_t s;
  const int32_t p = token_position(cu_valid, num_seqs, (const int32_t*)nullptr, v, &s);
  if (p < 0) return -1;
  const int64_t start = ps.cu[s];
  const int64_t r = start + p;
  if (start < 0 || r >= (int64_t)ps.cu[s + 1] || r >= T) return -1;
  if (ps.seqused != nullptr && p >= ps.seqused[s]) return -1;
  *row = r;
  if (ps.seq_offsets == nullptr) return p;
  const int64_t shifted = (int64_t)p + (int64_t)ps.seq_offsets[s];
  return shifted < 0 || shifted > (int64_t)INT32_MAX ? -1 : (int32_t)shifted;
}

// ---- a3: the angle --------------------------------------------------------------
// fp32(pos) * inv_freq[j], one fp32 multiply; with linear position interpolation
// by a factor s, the position is first divided by s in fp32 (correctly rounded),
// so that position s*p gets exactly the angles of position p.
__device__ inline float scaled_position(int32_t pos, float pos_scale) {
  const float fp = (float)pos;
  return pos_scale == 1.0f ? fp : __fdiv_rn(fp, pos_scale);
}
__device__ inline float rope_angle(float scaled_pos, float inv_freq_j) {
  return __fmul_rn(scaled_pos, inv_freq_j);
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

// Orders LDS traffic between the lanes of one wave (wave-local table, no s_barrier).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Rotate the H rows of one token. `row0` points at the token's first row. Lane
// items are (row r, chunk c) = (r0 + k*step_r, c0) for k = 0, 1, ...: this is the
// layout when nc divides 64 (step_c == 0), so each lane keeps one chunk and its
// cos/sin in registers for the whole token.
template <typename T, int VEC>
__device__ inline void rotate_rows_fixed_chunk(T* __restrict__ row0, int H, uint32_t D, uint32_t half,
                                               int r0, int c, int step_r, const float (&cs)[VEC],
                                               const float (&sn)[VEC]) {
  using C = Chunk<T, VEC>;
  for (int r = r0; r < H; r += kUnroll * step_r) {
    C lo[kUnroll], hi[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int ru = r + u * step_r;
      if (ru < H) {
        const uint32_t o = (uint32_t)ru * D + (uint32_t)(c * VEC);
        lo[u] = load_chunk<T, VEC>(row0 + o);
        hi[u] = load_chunk<T, VEC>(row0 + o + half);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int ru = r + u * step_r;
      if (ru < H) {
        const uint32_t o = (uint32_t)ru * D + (uint32_t)(c * VEC);
        rotate_chunk(lo[u], hi[u], cs, sn);
        store_chunk<T, VEC>(row0 + o, lo[u]);
        store_chunk<T, VEC>(row0 + o + half, hi[u]);
      }
    }
  }
}

// General layout (nc does not divide 64): lane items advance by 64 (row, chunk)
// pairs in row-major order, so the chunk changes from step to step and cos/sin
// are read from the wave's LDS table per item.
template <typename T, int VEC>
__device__ inline void rotate_rows_general(T* __restrict__ row0, int H, uint32_t D, uint32_t half,
                                           int nc, int r0, int c0, int step_r, int step_c,
                                           const float* cs_tab, const float* sn_tab) {
  using C = Chunk<T, VEC>;
  int r = r0, c = c0;
  while (r < H) {
    C lo[kUnroll], hi[kUnroll];
    int cc[kUnroll], rr[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      rr[u] = r;
      cc[u] = c;
      if (r < H) {
        const uint32_t o = (uint32_t)r * D + (uint32_t)(c * VEC);
        lo[u] = load_chunk<T, VEC>(row0 + o);
        hi[u] = load_chunk<T, VEC>(row0 + o + half);
      }
      r += step_r;
      c += step_c;
      if (c >= nc) {
        c -= nc;
        r += 1;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (rr[u] < H) {
        float cs[VEC], sn[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          cs[e] = cs_tab[cc[u] * VEC + e];
          sn[e] = sn_tab[cc[u] * VEC + e];
        }
        const uint32_t o = (uint32_t)rr[u] * D + (uint32_t)(cc[u] * VEC);
        rotate_chunk(lo[u], hi[u], cs, sn);
        store_chunk<T, VEC>(row0 + o, lo[u]);
        store_chunk<T, VEC>(row0 + o + half, hi[u]);
      }
    }
  }
}

// First row of token t in a [T, H, D] tensor whose tokens are `stride` elements
// apart (H * D when contiguous; more for a view into a fused QKV buffer).
// [U-int64]: with LONG_INDEX the offset is formed in 64 bits; without it, in 32
// bits, which the host selects only when every offset of the launch fits. t is
// wave-uniform, so either way this is scalar arithmetic; per-lane offsets below
// it are 32-bit (H * D < 2^22).
template <typename T, bool LONG_INDEX>
__device__ inline T* token_row0(T* p, int64_t t, int64_t stride) {
  if (LONG_INDEX) return p + t * stride;
  return p + (uint32_t)((uint32_t)t * (uint32_t)stride);
}

// ---- the fused QK kernel (a1..a7) ---------------------------------------------------
// TABLE: cos/sin of position p are row p of the caller's tables (a token whose
// position has no row is left untouched) instead of being evaluated here.
template <typename T, int VEC, bool LONG_INDEX, bool TABLE>
__global__ __launch_bounds__(kTokenBlock) void rope_qk_kernel(T* __restrict__ q, T* __restrict__ k,
                                                         const PosSource ps, const RopeParams p) {
  __shared__ float lds_cs[kWaves][kMaxHalf];
  __shared__ float lds_sn[kWaves][kMaxHalf];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t_begin = ((int64_t)blockIdx.x * kWaves + wave) * p.tpw;
  const uint32_t D = (uint32_t)p.D;
  const uint32_t half = D >> 1;
  const int nc = p.nc;
  // This lane's first (row, chunk) item and the per-step advance over 64 items.
  const int step_r = 64 / nc, step_c = 64 % nc;
  const int r0 = lane < nc ? 0 : lane / nc;
  const int c0 = lane - r0 * nc;
  // This lane's frequencies j = lane + 64*i (same for every token).
  float f[kMaxHalf / 64];
#pragma unroll
  for (int i = 0; i < kMaxHalf / 64; ++i) {
    const uint32_t j = (uint32_t)lane + 64u * i;
    f[i] = j < half ? p.inv_freq[j] : 0.0f;
  }

  for (int it = 0; it < p.tpw; ++it) {
    const int64_t t = t_begin + it;
    if (t >= p.T) break;
    int32_t seq;
    const int32_t pos = resolve_position(ps, t, &seq);  // wave-uniform
    if (pos < 0 || (TABLE && pos >= p.tab_rows)) continue;

    // a3: this token's fp32 cos/sin table, each (token, frequency) computed once.
    if constexpr (TABLE) {
      const float* crow = p.tab_cos + (int64_t)pos * half;
      const float* srow = p.tab_sin + (int64_t)pos * half;
      for (uint32_t j = (uint32_t)lane; j < half; j += 64) {
        lds_cs[wave][j] = crow[j];
        lds_sn[wave][j] = srow[j] * p.sin_sign;
      }
    } else {
      const float spos = scaled_position(pos, p.pos_scale);
#pragma unroll
      for (int i = 0; i < kMaxHalf / 64; ++i) {
        const uint32_t j = (uint32_t)lane + 64u * i;
        if (j < half) {
          float sn, cs;
          rope_trig::sincos_f32_cr(rope_angle(spos, f[i]), sn, cs);
          lds_cs[wave][j] = cs;
          lds_sn[wave][j] = sn * p.sin_sign;  // backward: R transposed = sin negated
        }
      }
    }
    wave_lds_sync();

    // a4/a5: Q rows then K rows of this token, in place.
    T* qrow = token_row0<T, LONG_INDEX>(q, t, p.q_stride);
    T* krow = token_row0<T, LONG_INDEX>(k, t, p.k_stride);
    if (step_c == 0) {
      if (lane < step_r * nc) {
        float cs[VEC], sn[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          cs[e] = lds_cs[wave][c0 * VEC + e];
          sn[e] = lds_sn[wave][c0 * VEC + e];
        }
        rotate_rows_fixed_chunk<T, VEC>(qrow, p.Hq, D, half, r0, c0, step_r, cs, sn);
        rotate_rows_fixed_chunk<T, VEC>(krow, p.Hkv, D, half, r0, c0, step_r, cs, sn);
      }
    } else {
      rotate_rows_general<T, VEC>(qrow, p.Hq, D, half, nc, r0, c0, step_r, step_c,
                                  lds_cs[wave], lds_sn[wave]);
      rotate_rows_general<T, VEC>(krow, p.Hkv, D, half, nc, r0, c0, step_r, step_c,
                                  lds_cs[wave], lds_sn[wave]);
    }
    wave_lds_sync();  // the table is rewritten for the next token
  }
}

// Streaming store of one chunk written through to memory at device scope (cache
// policy sc1 + nt on the gfx950 store), so the line does not stay dirty in the
// XCD's L2. For this in-place update, whose stores follow loads of the same lines,
// that keeps HBM 1-2% busier than store_chunk on the row-group kernel; the token
// kernel is 5% slower with it and the out-of-place GLU kernels 1-2% slower, so
// they keep store_chunk. The compiler has no builtin for these bits on a global
// store, hence the asm, which the compiler does not see as a store: (1) a store
// wider than 8 bytes reads its data registers after issue, and gfx950 needs two
// wait states before a vector instruction may overwrite them, so the asm carries
// them (s_nop 1); (2) the compiler does not count the store among the wave's
// outstanding memory operations, so it is used only where the wave issues no
// further memory operation (the end of the kernel). Other widths use store_chunk.
template <typename T, int VEC>
__device__ inline void store_chunk_through(T* p, const Chunk<T, VEC>& c) {
  if constexpr (sizeof(Chunk<T, VEC>) == 16) {
    const u32x4 w = __builtin_bit_cast(u32x4, c);
    asm volatile("global_store_dwordx4 %0, %1, off nt sc1\n\ts_nop 1" : : "v"(p), "v"(w) : "memory");
  } else {
    store_chunk<T, VEC>(p, c);
  }
}

// Rows per group for nc chunks per half row and `steps` row steps: the 64 * steps
// / nc rows whose chunk pairs the lanes hold, rounded down to a group of whole
// 128-byte lines when at least 5/8 of the 64 * steps lane slots stay busy (16-byte
// chunks, the one size whose groups can end inside a line: rows * nc a multiple of
// 4). A group that ends inside a line shares it with the next group, which runs on
// another XCC, and the two partial writes of that line cost more than the idle
// lanes: D = 112 in bf16 (nc = 7) as 8 rows of 224 bytes (14 lines) instead of 9 ran
// 10-21% faster (interleaved, bit-identical; 32 + 32 heads, 16384 tokens: 92.2 ->
// 72.7 us per pass), D = 48 (nc = 3, 20 rows instead of 21) 4-11%, and with two
// steps D = 176 (nc = 11, 8 rows instead of 11, 88 of 128 slots) 8-18%. For nc = 9
// (D = 144) the aligned one-step group is 4 rows, 36 busy lanes, which measured
// 18-20% slower than 7. Other nc give whole lines already.
__host__ __device__ inline uint32_t group_rows(uint32_t nc, uint32_t steps = 1) {
  const uint32_t r = 64u * steps / nc;
  const uint32_t a = (nc & 1u) != 0 ? r & ~3u : (nc & 3u) == 2u ? r & ~1u : r;
  return 8u * a * nc >= 5u * 64u * steps ? a : r;
}

// ---- the default geometry: one wave per (token, row group) --------------------------
// A 64-lane workgroup owns one group of group_rows(nc) consecutive head rows of
// one token (Q rows first, then K rows; the last group of each may be partial).
// For D = 128 in bf16 that is 8 rows = 2 KB, one 16-byte lo and one 16-byte hi
// chunk per lane. The wave issues its loads first, then evaluates the token's
// cos/sin (one correctly rounded sincos per lane and frequency, into a wave-local
// LDS table), rotates and stores, and ends. Waves that each move one small
// contiguous piece of a token and end keep HBM busier than waves that walk a whole
// token: more short-lived waves overlap the cos/sin evaluation of some with the
// memory traffic of others, and each wave's reads and writes stay within 2 KB.
// The cost is evaluating each (token, frequency) cos/sin once per row group of
// the token instead of once per token.
// TABLE as in rope_qk_kernel. COMPACT: the grid covers only the rotated tokens of
// a padded layout (compact_position), so no workgroup is spent on padded rows.
// STAGED (see the address computation below): row halves that are not whole
// 128-byte lines, e.g. D = 64, 80, 96 or 112 in 16-bit storage, move through LDS
// in whole lines. Otherwise nc is a power of two, the groups are 64 / nc rows and
// the lane split is a shift. STEPS (group_steps, 1 or 2): without STAGED a group
// is STEPS times 64 / nc rows, each lane rotating its chunk pair in STEPS rows
// 64 / nc apart with the one cos/sin table of the token; with STAGED a group is
// group_rows(nc, STEPS) rows, up to 128 * STEPS chunks moved through LDS, each lane
// rotating (row, chunk) pairs lane and lane + 64 of the group.
//
// Everything a wave needs before its first loads leads the argument list as 13
// plain dwords, which the library's build preloads into SGPRs at wave launch
// (the compiler's kernel-argument preload), so the wave does not first wait for
// a load of its arguments: q, k, cu_seqlens (cu_valid for COMPACT: the array the
// position search runs over); q_stride, k_stride (elements between tokens,
// < 2^32); groups_mul, the multiplier of the division of the workgroup index by
// the row groups per token (fast_div.h); geo = gq | gk << 13 | nc_shift << 26 |
// position-source flags << 29 (kFlag*); heads = Hq | Hkv << 13 | (division
// shift - 26) << 26; num_seqs; t_base, the token (COMPACT: rotated token) of
// workgroup 0, nonzero when a long pass is issued as several launches. The rest
// (frequencies, sign, scale, tables, the other position sources) comes from ps
// and p, read after the row loads are issued or only on the paths that need them.
// Unless STAGED, D follows from nc_shift: a half row is 2^nc_shift chunks of VEC
// elements.
constexpr uint32_t kFlagIds = 1, kFlagOffsets = 2, kFlagSeqused = 4;
template <typename T, int VEC, bool LONG_INDEX, bool TABLE, bool COMPACT, bool STAGED, int STEPS>
__global__ __launch_bounds__(64) void rope_qk_group_kernel(
    T* __restrict__ q, T* __restrict__ k, const int32_t* __restrict__ cu, uint32_t q_stride,
    uint32_t k_stride, uint32_t groups_mul, uint32_t geo, uint32_t heads, int32_t num_seqs,
    uint32_t t_base, const PosSource ps, const RopeParams p) {
  __shared__ float lds_cs[kMaxHalf];
  __shared__ float lds_sn[kMaxHalf];
  extern __shared__ __align__(16) unsigned char lds_dyn[];  // the residency cap's reserve
  using C = Chunk<T, VEC>;
  const int lane = threadIdx.x;
  const uint32_t gq = geo & 0x1fffu;
  const uint32_t gk = (geo >> 13) & 0x1fffu;
  const uint32_t ns = (geo >> 26) & 7u;
  const uint32_t flags = geo >> 29;
  const int Hq = (int)(heads & 0x1fffu);
  const int Hkv = (int)((heads >> 13) & 0x1fffu);
  // Workgroup -> (token, row group) with host-made constants: a multiply and a
  // shift instead of integer divisions, so the wave reaches its loads sooner.
  const fastdiv::FastDiv groups{groups_mul, fastdiv::kMaxDividendBits + (heads >> 26)};
  const uint32_t tl = fastdiv::div(blockIdx.x, groups);
  const uint32_t g = blockIdx.x - tl * (gq + gk);
  const uint32_t t = t_base + tl;  // < 2^26; COMPACT: rotated-token index

  // a4/a5 addresses: this lane's row of the group, and its chunk of the row
  // halves. Lanes past the last row of a partial group address row 0 of the same
  // token and tensor (valid memory) and store nothing.
  // STAGED: nc (16-byte chunks per half row) is at most 10 and not 8, so the row
  // halves are not whole 128-byte lines (e.g. D = 64, 80, 96 or 112 in 16-bit
  // storage; staged_geometry). A group is then group_rows(nc) rows
  // and is moved as one contiguous range: two coalesced 16-byte loads and stores
  // per lane cover its up to 128 chunks, and the (lo, hi) pairs meet in LDS, in the
  // dynamic LDS the residency cap reserves anyway. Each lane's row and chunk in
  // the group come from a division by nc (read from p).
  const bool in_q = g < gq;
  uint32_t half;
  int c, r;
  bool live;
  uint32_t rl = 0, g0 = 0, nchunks = 0;  // STAGED: lane's row in the group, first row, chunks
  if constexpr (STAGED) {
    const uint32_t nc = (uint32_t)p.nc;
    const uint32_t rows = group_rows(nc, STEPS);
    rl = (uint32_t)lane / nc;
    c = lane - (int)(rl * nc);
    half = (uint32_t)VEC * nc;
    g0 = (in_q ? g : g - gq) * rows;
    const uint32_t H = (uint32_t)(in_q ? Hq : Hkv);
    const uint32_t grows = H - g0 < rows ? H - g0 : rows;  // >= 1
    nchunks = grows * 2u * nc;                              // <= 128 * STEPS
    r = (int)(g0 + rl);
    live = rl < grows;
  } else {
    c = lane & ((1 << ns) - 1);
    half = (uint32_t)VEC << ns;
    r = (int)((((in_q ? g : g - gq) * (uint32_t)STEPS) << (6 - ns)) + ((uint32_t)lane >> ns));
    live = r < (in_q ? Hq : Hkv);
  }
  [[maybe_unused]] const int H = in_q ? Hq : Hkv;
  const uint32_t D = half << 1;
  // !STAGED: this lane's chunk of its row; STAGED: the group's first element
  T* row = nullptr;
  T* trow = nullptr;  // STEPS > 1: the token's first row in the tensor
  if constexpr (!COMPACT) {
    row = in_q ? token_row0<T, LONG_INDEX>(q, (int64_t)t, (int64_t)q_stride)
               : token_row0<T, LONG_INDEX>(k, (int64_t)t, (int64_t)k_stride);
    trow = row;
    // r * D < 2^22: a 24-bit multiply. (A full 32-bit multiply-add becomes
    // v_mad_u64_u32 with an undefined high addend, which the register allocator
    // may place in a register a pending load writes, forcing a wait on it.)
    if constexpr (STAGED)
      row += __umul24(g0, D);
    else
      row += __umul24((uint32_t)(live ? r : 0), D) + (uint32_t)(c * VEC);
  }

  // Vector-memory loads complete in issue order, so the order of issue below is
  // what lets the cos/sin evaluation overlap the row loads: this lane's inverse
  // frequencies first (from the argument struct; only the 64-entry blocks below
  // D/2, a wave-uniform condition: D = 128 needs one of the four, and skipping the
  // rest measured 0.1-0.6% faster), then the position search (scalar loads), then
  // the two row loads, unconditionally, so that the wait for the frequencies
  // needs no wait for the rows. The schedule barriers keep the compiler from
  // interleaving these phases.
  __builtin_amdgcn_sched_barrier(0);
  float f[kMaxHalf / 64];
#pragma unroll
  for (int i = 0; i < kMaxHalf / 64; ++i)
    f[i] = 64u * i < half ? p.inv_freq[(uint32_t)lane + 64u * i] : 0.0f;
  __builtin_amdgcn_sched_barrier(0);
  int32_t pos;  // wave-uniform
  if constexpr (COMPACT) {
    int64_t tok = 0;
    pos = compact_position(ps, cu, num_seqs, (int32_t)t, p.T, &tok);  // cu: cu_valid
    if (pos < 0) return;
    row = in_q ? token_row0<T, LONG_INDEX>(q, tok, (int64_t)q_stride)
               : token_row0<T, LONG_INDEX>(k, tok, (int64_t)k_stride);
    trow = row;
    if constexpr (STAGED)
      row += __umul24(g0, D);
    else
      row += __umul24((uint32_t)(live ? r : 0), D) + (uint32_t)(c * VEC);
  } else {
    int32_t seq;
    // cu_seqlens alone (the packed default) from the preloaded arguments; the
    // other position sources through ps
    pos = flags == 0 ? token_position(cu, num_seqs, (const int32_t*)nullptr, (int32_t)t, &seq)
                     : resolve_position(ps, (int32_t)t, &seq);
  }
  if (pos < 0 || (TABLE && pos >= p.tab_rows)) return;
  C lo, hi;
  if constexpr (STAGED) {
    // chunks lane and lane + 64 of the group; lanes past its end load its last chunk
    const uint32_t i0 = (uint32_t)lane < nchunks ? (uint32_t)lane : nchunks - 1;
    const uint32_t i1 = (uint32_t)lane + 64u < nchunks ? (uint32_t)lane + 64u : nchunks - 1;
    lo = load_chunk<T, VEC>(row + i0 * VEC);
    hi = load_chunk<T, VEC>(row + i1 * VEC);
  } else {
    lo = load_chunk<T, VEC>(row);
    hi = load_chunk<T, VEC>(row + half);
  }
  // STEPS > 1: the lane's chunk pair in rows r + j * (64 / nc), j = 1 .. STEPS - 1
  // (row 0 of the token for rows past the tensor's last, which store nothing)
  // STAGED with STEPS = 2: chunks lane + 128 and lane + 192 of the group
  C lo_s[STEPS > 1 ? STEPS - 1 : 1], hi_s[STEPS > 1 ? STEPS - 1 : 1];
  if constexpr (STAGED && STEPS > 1) {
    static_assert(STEPS == 2, "staged groups hold at most 256 chunks");
    const uint32_t i2 = (uint32_t)lane + 128u < nchunks ? (uint32_t)lane + 128u : nchunks - 1;
    const uint32_t i3 = (uint32_t)lane + 192u < nchunks ? (uint32_t)lane + 192u : nchunks - 1;
    lo_s[0] = load_chunk<T, VEC>(row + i2 * VEC);
    hi_s[0] = load_chunk<T, VEC>(row + i3 * VEC);
  } else if constexpr (STEPS > 1) {
#pragma unroll
    for (int j = 1; j < STEPS; ++j) {
      const uint32_t rj = (uint32_t)r + ((uint32_t)j << (6 - ns));
      T* pj = trow + __umul24(rj < (uint32_t)H ? rj : 0u, D) + (uint32_t)(c * VEC);
      lo_s[j - 1] = load_chunk<T, VEC>(pj);
      hi_s[j - 1] = load_chunk<T, VEC>(pj + half);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // a3: the token's fp32 cos/sin table
  if constexpr (TABLE) {
    const float* crow = p.tab_cos + (int64_t)pos * half;
    const float* srow = p.tab_sin + (int64_t)pos * half;
    for (uint32_t j = (uint32_t)lane; j < half; j += 64) {
      lds_cs[j] = crow[j];
      lds_sn[j] = srow[j] * p.sin_sign;
    }
  } else {
    const float spos = scaled_position(pos, p.pos_scale);
#pragma unroll
    for (int i = 0; i < kMaxHalf / 64; ++i) {
      const uint32_t j = (uint32_t)lane + 64u * i;
      if (j < half) {
        float sn, cs;
        rope_trig::sincos_f32_cr(rope_angle(spos, f[i]), sn, cs);
        lds_cs[j] = cs;
        lds_sn[j] = sn * p.sin_sign;  // backward: R transposed = sin negated
      }
    }
  }
  if constexpr (STAGED) {
    C* stage = reinterpret_cast<C*>(lds_dyn);
    if ((uint32_t)lane < nchunks) stage[lane] = lo;
    if ((uint32_t)lane + 64u < nchunks) stage[lane + 64] = hi;
    if constexpr (STEPS > 1) {
      if ((uint32_t)lane + 128u < nchunks) stage[lane + 128] = lo_s[0];
      if ((uint32_t)lane + 192u < nchunks) stage[lane + 192] = hi_s[0];
    }
  }
  wave_lds_sync();

  if constexpr (STAGED) {
    C* stage = reinterpret_cast<C*>(lds_dyn);
    if (live) {
      const uint32_t i = rl * 2u * (half / VEC) + (uint32_t)c;  // this lane's lo chunk
      C a = stage[i];
      C b = stage[i + half / VEC];
      float cs[VEC], sn[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        cs[e] = lds_cs[c * VEC + e];
        sn[e] = lds_sn[c * VEC + e];
      }
      rotate_chunk(a, b, cs, sn);
      stage[i] = a;
      stage[i + half / VEC] = b;
    }
    if constexpr (STEPS > 1) {
      // the group's (row, chunk) pair lane + 64
      const uint32_t ncv = half / VEC;
      const uint32_t pi = (uint32_t)lane + 64u;
      const uint32_t prow = pi / ncv;
      const uint32_t pc = pi - prow * ncv;
      if (prow * 2u * ncv < nchunks) {
        const uint32_t i = prow * 2u * ncv + pc;
        C a = stage[i];
        C b = stage[i + ncv];
        float cs[VEC], sn[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          cs[e] = lds_cs[pc * VEC + e];
          sn[e] = lds_sn[pc * VEC + e];
        }
        rotate_chunk(a, b, cs, sn);
        stage[i] = a;
        stage[i + ncv] = b;
      }
    }
    wave_lds_sync();
    // written through to memory, whole lines of the group at a time
    if ((uint32_t)lane < nchunks) store_chunk_through<T, VEC>(row + lane * VEC, stage[lane]);
    if ((uint32_t)lane + 64u < nchunks)
      store_chunk_through<T, VEC>(row + ((uint32_t)lane + 64u) * VEC, stage[lane + 64]);
    if constexpr (STEPS > 1) {
      if ((uint32_t)lane + 128u < nchunks)
        store_chunk_through<T, VEC>(row + ((uint32_t)lane + 128u) * VEC, stage[lane + 128]);
      if ((uint32_t)lane + 192u < nchunks)
        store_chunk_through<T, VEC>(row + ((uint32_t)lane + 192u) * VEC, stage[lane + 192]);
    }
  } else if (live) {
    float cs[VEC], sn[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      cs[e] = lds_cs[c * VEC + e];
      sn[e] = lds_sn[c * VEC + e];
    }
    rotate_chunk(lo, hi, cs, sn);
    // the wave's last memory operations: written through to memory, not left
    // dirty in L2
    store_chunk_through<T, VEC>(row, lo);
    store_chunk_through<T, VEC>(row + half, hi);
    if constexpr (STEPS > 1) {
#pragma unroll
      for (int j = 1; j < STEPS; ++j) {
        const uint32_t rj = (uint32_t)r + ((uint32_t)j << (6 - ns));
        if (rj < (uint32_t)H) {
          T* pj = trow + __umul24(rj, D) + (uint32_t)(c * VEC);
          rotate_chunk(lo_s[j - 1], hi_s[j - 1], cs, sn);
          store_chunk_through<T, VEC>(pj, lo_s[j - 1]);
          store_chunk_through<T, VEC>(pj + half, hi_s[j - 1]);
        }
      }
    }
  }
}

// ---- export hooks (same device functions) --------------------------------------------
__global__ __launch_bounds__(kBlock) void rope_positions_kernel(const PosSource ps, int64_t T,
                                                                int32_t* pos_out,
                                                                int32_t* seq_out) {
  const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (t >= T) return;
  int32_t seq = -1, pos = -1;
  // With no sequences (and no explicit ids) every token is untouched, and
  // cu_seqlens may be NULL: it is not read.
  if (ps.position_ids != nullptr || ps.num_seqs > 0) pos = resolve_position(ps, t, &seq);
  if (pos_out) pos_out[t] = pos;
  if (seq_out) seq_out[t] = seq;
}

// Running count of rotated tokens per sequence, the cu_valid of a compact launch:
// out[0] = 0 and out[s+1] = out[s] + min(seqused[s], cu[s+1] - cu[s]) (the length
// alone without seqused), each term clamped at 0, summed in 64 bits and saturated
// at INT32_MAX. One workgroup; each step scans kBlock sequences in LDS
// (Hillis-Steele) and carries the step's total into the next.
__global__ __launch_bounds__(kBlock) void rope_valid_prefix_kernel(const int32_t* __restrict__ cu,
                                                                   int32_t num_seqs,
                                                                   const int32_t* __restrict__ seqused,
                                                                   int32_t* __restrict__ out) {
  __shared__ int64_t scan[kBlock];
  const int i = threadIdx.x;
  if (i == 0) out[0] = 0;
  int64_t carry = 0;
  for (int64_t base = 0; base < num_seqs; base += kBlock) {
    const int64_t s = base + i;
    int64_t used = 0;
    if (s < num_seqs) {
      const int64_t len = (int64_t)cu[s + 1] - (int64_t)cu[s];
      used = seqused != nullptr && (int64_t)seqused[s] < len ? (int64_t)seqused[s] : len;
      used = used < 0 ? 0 : used;
    }
    scan[i] = used;
    __syncthreads();
    for (int d = 1; d < kBlock; d <<= 1) {
      const int64_t add = i >= d ? scan[i - d] : 0;
      __syncthreads();
      scan[i] += add;
      __syncthreads();
    }
    const int64_t incl = carry + scan[i];
    if (s < num_seqs) out[s + 1] = incl > (int64_t)INT32_MAX ? INT32_MAX : (int32_t)incl;
    carry += scan[kBlock - 1];
    __syncthreads();  // scan[] is rewritten by the next step
  }
}

// Row i of the tables is position positions[i], or position i when positions is
// NULL (the [max_pos, D/2] table of positions 0 .. max_pos-1).
__global__ __launch_bounds__(kBlock) void rope_cos_sin_kernel(const int32_t* __restrict__ positions,
                                                              int64_t n, int32_t half,
                                                              const CosSinParams p, float* cos_out,
                                                              float* sin_out) {
  const int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (idx >= n * half) return;
  const int64_t i = idx / half;
  const int32_t j = (int32_t)(idx - i * half);
  const int32_t pos = positions != nullptr ? positions[i] : (int32_t)i;
  float s, c;
  rope_trig::sincos_f32_cr(rope_angle(scaled_position(pos, p.pos_scale), p.inv_freq[j]), s, c);
  cos_out[idx] = c;
  sin_out[idx] = s;
}

// ---- host side -----------------------------------------------------------------------

// a2: inv_freq[j] = theta^(-2j/D), correctly rounded to fp32.
// Fast path in double: the exponent -2j/D rounds with a relative error of at most
// 2^-53, which moves theta^e by at most |ln theta| * 2^-53 relative (< 2^-43.4 for
// any finite theta), and pow adds under one double ulp: the double result is within
// about 800 double ulps of the exact value. Rounding it to fp32 therefore gives the
// correctly rounded result unless it lies within that distance of a binary32
// midpoint -- its 29 bits below binary32 precision near 0x10000000 -- or below the
// binary32 normal range; those values (about 1 in 65000) are recomputed in
// extended precision (powl with a 64-bit-mantissa exponent), as is the whole
// table on hosts without an 80-bit long double. powl for every entry costs about
// 0.35 us each, more than a short launch's GPU time.
void host_inv_freq(double theta, int32_t D, float* out) {
  constexpr int64_t kWindow = 4096;  // double ulps; 5x the error bound above
  for (int32_t j = 0; j < D / 2; ++j) {
    const double v = pow(theta, -(2.0 * (double)j) / (double)D);
    uint64_t u;
    memcpy(&u, &v, sizeof u);
    const int64_t low = (int64_t)(u & 0x1fffffffu) - 0x10000000;
    const bool safe = v >= 0x1p-126 && (low > kWindow || low < -kWindow);
    out[j] = safe ? (float)v
                  : (float)powl((long double)theta, -(2.0L * (long double)j) / (long double)D);
  }
}

bool valid_theta(double theta) { return isfinite(theta) && theta >= 1.0; }
bool valid_D(int32_t D) { return D >= 2 && D <= 2 * kMaxHalf && (D & 1) == 0; }
// Linear position interpolation factor, applied in fp32: finite and >= 1.
bool valid_scale(double s) { return isfinite(s) && (float)s >= 1.0f && isfinite((float)s); }

int32_t elem_size(int32_t dtype) { return dtype == ROPE_F32 ? 4 : 2; }

// Widest chunk (<= 16 bytes) that divides a half row and keeps every access
// aligned: the base pointers and the token strides must be multiples of it too.
int32_t chunk_bytes(int32_t D, int32_t esize, const void* q, const void* k, int64_t q_stride,
                    int64_t k_stride) {
  const int64_t half_bytes = (int64_t)(D / 2) * esize;
  for (int32_t b = 16; b > esize; b >>= 1) {
    if (half_bytes % b) continue;
    if (q && (((uintptr_t)q % b) || (q_stride * esize) % b)) continue;
    if (k && (((uintptr_t)k % b) || (k_stride * esize) % b)) continue;
    return b;
  }
  return esize;
}

// Workgroups of the row-group kernel resident per CU. Unrestricted, its 64-lane
// workgroups fill every wave slot of a CU (32); fewer in flight move data faster.
// The cap is set by reserving LDS the kernel does not use: each workgroup asks
// for lds_per_cu / cap bytes in all. Measured on MI355X with the write-through
// stores (bf16, D = 128, caps 16-32 and none, interleaved on the same buffers):
// 20 is the best cap, or within 0.5% of it, for 32 + 8, 32 + 4, 16 + 8 and 40 + 8
// heads from 2048 to 524288 tokens (8554 tokens 27.85 us vs 27.95 at 24 and 28.54
// uncapped; 524288 tokens 1609 vs 1637 at 24 and 1750 uncapped); Q-heavy launches
// (64 + 8 heads) of 2^18 workgroups or more do best at 28 (32768 tokens 179.8 vs
// 182.2 us at 24; 65536 and 131072 tokens 2.5-3% better than 24).
constexpr uint32_t kLdsPerCU = 160 * 1024;
constexpr uint32_t kGroupStaticLds = 2 * kMaxHalf * sizeof(float);
// Workgroups that take longer each want more of them in flight. The STAGED
// instances (staged_geometry: the pairs meet in LDS) do best with as many as the
// waves allow, 32 per CU: 12% faster than 20 for D = 96 and D = 160 (32 + 32 and
// 16 + 16 heads, 16384 tokens, 73.6 -> 64.7 and 63.8 -> 56.0 us), 9% for D = 80,
// 1% for D = 64. So do half rows of more than 64 frequencies, whose cos/sin take
// each lane two or four evaluations: D = 256 at 28 (83.1 -> 80.5 us for 16 + 16
// heads, 250.9 -> 240.6 for 16 + 8 heads over 65536 tokens), D = 512 at 32 with
// one row step (109.7 -> 99.7 us for 8 + 8 heads). A workgroup of two row steps
// (group_steps) carries twice the bytes and does best at 20 again: 14-15% faster
// than one step at 32 for D = 512 in bf16, 3% of it from the cap (32 -> 20).
constexpr uint32_t kCap = 20, kCapLongQHeavy = 28, kCapStaged = 32;
uint32_t group_dynamic_lds(unsigned group_blocks, uint32_t gq, uint32_t gk, bool staged,
                           uint32_t half, int32_t steps) {
  const bool long_q_heavy = group_blocks >= (1u << 18) && gq >= 8 * gk;
  const uint32_t cap = steps > 1                   ? kCap
                       : staged || half > 128       ? kCapStaged
                       : half > 64 || long_q_heavy ? kCapLongQHeavy
                                                   : kCap;
  return kLdsPerCU / cap - kGroupStaticLds;
}
// The STAGED instances keep a group's up to 128 16-byte chunks in that reserve.
static_assert(kLdsPerCU / kCapStaged - kGroupStaticLds >= 128 * 16,
              "the residency reserve must hold a staged group");

// The row-group kernel's STAGED instance: 16-byte chunks and row halves that are
// not whole 128-byte lines (nc other than 8), at most 10 chunks per half row so
// that a one-step group holds at least 6 rows (11 to 15 with two steps, below).
// Measured against the token kernel
// (interleaved, bit-identical, bf16, 16384 tokens): D = 32, 64, 80, 96, 112 and 160
// 7-44% faster (D = 96: 96.8 -> 74.4 us per pass for 32 + 32 heads; D = 64: 48.1
// -> 43.2), but D = 192 (12 chunks, 5 rows per group, 16 + 16 heads) 14% slower:
// groups that short spend as much per workgroup on the search and cos/sin as a
// full group for fewer bytes, so from 11 chunks on a staged group takes two steps.
// The staged instance with two steps (a group of group_rows(nc, 2) rows, up to 256
// chunks, four coalesced loads and stores per lane, two (lo, hi) pairs per lane)
// for 11 to 15 chunks per half row, which one step would leave at 4 or 5 rows per
// group. Against the token kernel these head sizes took before (interleaved,
// bit-identical, 16384 tokens, two boxes, per pass): in bf16, 16 + 16 heads, D = 176
// 79.4-79.6 -> 66.2-66.7 us (58% -> 69% of 8 TB/s; 60.0 us, 77%, with 8 rows, above), D = 192 74.0-74.1 -> 68.8-69.2
// (68% -> 73%), D = 208 105.2 -> 68.1 (52% -> 80%), D = 224 101.3 -> 74.3, D = 240
// 111.2 -> 79.9; D = 192 with 32 + 8 heads 95.7-95.9 -> 77.4-78.8 (66% -> 80-81%);
// fp32 D = 96, 32 + 8 heads, 95.2 -> 78.5 (66% -> 80%). For 10 chunks or fewer two
// steps measured slower than one (D = 80 +14%, D = 96 +3 to +6%, D = 112 +1 to +3%;
// D = 144 +5% for 16 + 16 heads, -5% for 32 + 8).
bool staged_two_steps(int32_t nc, int32_t chunk_bytes) {
  return chunk_bytes == 16 && nc >= 11 && nc <= 15;
}
bool staged_geometry(int32_t nc, int32_t chunk_bytes) {
  return (chunk_bytes == 16 && nc <= 10 && nc != 8) || staged_two_steps(nc, chunk_bytes);
}

// Row steps per row-group workgroup: 2 for half rows of more than 128 elements in
// 16-byte chunks (D = 512) and for the staged instance at 11 to 15 chunks per half
// row (staged_two_steps), 1 otherwise. A D = 512 row takes each lane four cos/sin
// evaluations for one chunk pair; a second row step (the lane's chunk pair in the
// row 64 / nc further on, loaded with the first) shares them, so a workgroup moves
// twice the rows (4 instead of 2 in 16-bit storage) for the same VALU work.
// Measured against one step (interleaved, bit-identical, 16384 tokens, two boxes;
// with the cap of 20 that group_dynamic_lds gives stepped launches): D = 512 in
// bf16 11-15% faster (8 + 8 heads 98.4 -> 83.7 and 95.9 -> 85.3 us per pass,
// 68-70% -> 79-80% of 8 TB/s), 16 + 8 heads 12-15%, 32 + 8 heads over 65536
// tokens 12-14%; in fp32 (8 + 8 heads) 5-8%. Four steps gained less (D = 512 in
// bf16 -15 to -17% at the old cap of 32, against -17 to -19% for two), and two
// steps cost 7-8% for D = 256 in fp32 and 1.5-4% in bf16, whose lanes evaluate two
// cos/sin values.
int32_t group_steps(int32_t nc, int32_t half, int32_t chunk_bytes) {
  return (chunk_bytes == 16 && half > 128) || staged_two_steps(nc, chunk_bytes) ? 2 : 1;
}

// Long passes as several launches. Workgroup i of a launch runs on XCC i mod 8
// for the whole launch, and the eight XCCs drift apart as it runs (a probe that
// recorded each workgroup's XCC and start time: on 524288 tokens of 32 + 8 heads
// the spread between the most and the least advanced XCC grows from ~250 to
// ~8600 tokens; within 65536 tokens it stays under ~900). The XCCs then stream
// from separate address ranges instead of neighbouring ones, which HBM serves
// more slowly; a launch boundary brings them back together. Passes of Q-heavy
// shapes (Q holding at least 4x K's row groups) of 2 * kPieceBlocks workgroups or
// more are therefore issued as consecutive launches of about kPieceBlocks each
// over consecutive token ranges, every range starting at a multiple of 8 tokens
// so that each (token, row group) keeps the XCC it has in a single launch (ranges
// one token off that alignment lose most of the gain). Measured, bf16, D = 128,
// one sequence, interleaved, bit-identical: 32 + 8 heads, 524288 tokens 1604.7 ->
// 1576.2 us per pass (8 launches), 262144 tokens -1.1%, 131072 tokens -0.4%;
// 64 + 8 heads, 262144 tokens 1514.6 -> 1427.9 us (8 launches); 40 + 8, 48 + 8 and
// 32 + 4 heads 1.3-4.4% faster. Below the 4x ratio splitting measured neutral or
// slower at every piece count (24 + 8, 16 + 8, 16 + 4, 8 + 8 heads: -0.7 to +6.9%).
constexpr uint32_t kPieceBlocks = 327680;
uint32_t group_piece_tokens(uint32_t rows, uint32_t gq, uint32_t gk) {
  const uint64_t blocks = (uint64_t)rows * (gq + gk);
  if (gq < 4 * gk || blocks < 2ull * kPieceBlocks) return rows;
  const uint64_t n = (blocks + kPieceBlocks - 1) / kPieceBlocks;
  return (uint32_t)(((rows + n - 1) / n + 7) / 8 * 8);
}

// The leading scalar arguments of rope_qk_group_kernel (see there).
struct GroupScalars {
  const int32_t* search;  // cu_seqlens, or cu_valid for a compact launch
  uint32_t q_stride, k_stride, groups_mul, geo, heads;
};
// Field widths of the packed words: head and row-group counts below 2^13 (at most
// kMaxHeads), nc_shift below 8 (nc <= 64), the division shift minus 26 below 16
// (l = ceil(log2(gq + gk)) <= 13), three flag bits.
static_assert(kMaxHeads < (1 << 13), "head counts must fit 13 bits");
static_assert(kMaxHalf <= 256, "nc_shift must fit 3 bits");
GroupScalars group_scalars(const RopeParams& p, const PosSource& ps) {
  const uint32_t flags = (ps.position_ids ? kFlagIds : 0u) | (ps.seq_offsets ? kFlagOffsets : 0u) |
                         (ps.seqused ? kFlagSeqused : 0u);
  GroupScalars g;
  g.search = ps.cu_valid != nullptr ? ps.cu_valid : ps.cu;
  g.q_stride = (uint32_t)p.q_stride;
  g.k_stride = (uint32_t)p.k_stride;
  g.groups_mul = p.groups.mul;
  g.geo = p.gq | p.gk << 13 | p.nc_shift << 26 | flags << 29;
  g.heads = (uint32_t)p.Hq | (uint32_t)p.Hkv << 13 |
            (p.groups.shift - fastdiv::kMaxDividendBits) << 26;
  return g;
}

// One launch of the row-group kernel over tokens [t0, t0 + n) (rotated-token
// indices for a compact launch).
template <typename T, int VEC, bool TABLE, bool STAGED, int STEPS>
void launch_group(T* qt, T* kt, const PosSource& ps, const RopeParams& p, const GroupScalars& s,
                  bool long_index, uint32_t lds, uint32_t t0, uint32_t n, hipStream_t stream) {
  const dim3 grid(n * (p.gq + p.gk));
#define ROPE_GROUP_ARGS                                                                     \
  grid, dim3(64), lds, stream, qt, kt, s.search, s.q_stride, s.k_stride, s.groups_mul,    \
      s.geo, s.heads, ps.num_seqs, t0, ps, p
  if (!TABLE && ps.cu_valid != nullptr) {
    if (long_index)
      hipLaunchKernelGGL((rope_qk_group_kernel<T, VEC, true, false, true, STAGED, STEPS>), ROPE_GROUP_ARGS);
    else
      hipLaunchKernelGGL((rope_qk_group_kernel<T, VEC, false, false, true, STAGED, STEPS>), ROPE_GROUP_ARGS);
  } else if (long_index) {
    hipLaunchKernelGGL((rope_qk_group_kernel<T, VEC, true, TABLE, false, STAGED, STEPS>), ROPE_GROUP_ARGS);
  } else {
    hipLaunchKernelGGL((rope_qk_group_kernel<T, VEC, false, TABLE, false, STAGED, STEPS>), ROPE_GROUP_ARGS);
  }
#undef ROPE_GROUP_ARGS
}

template <typename T, int VEC, bool TABLE>
int32_t launch_vec(void* q, void* k, const PosSource& ps, const RopeParams& p, bool long_index,
                   unsigned blocks, unsigned group_blocks, hipStream_t stream) {
  T* qt = static_cast<T*>(q);
  T* kt = static_cast<T*>(k);
  if (group_blocks > 0) {
    const bool staged = staged_geometry(p.nc, VEC * (int)sizeof(T));
    const int32_t steps = group_steps(p.nc, p.D / 2, VEC * (int)sizeof(T));
    const uint32_t lds =
        group_dynamic_lds(group_blocks, p.gq, p.gk, staged, (uint32_t)p.D / 2, steps);
    const GroupScalars s = group_scalars(p, ps);
    const uint32_t rows = group_blocks / (p.gq + p.gk);
    const uint32_t piece = group_piece_tokens(rows, p.gq, p.gk);
    for (uint32_t t0 = 0; t0 < rows; t0 += piece) {
      const uint32_t n = rows - t0 < piece ? rows - t0 : piece;
      if constexpr (VEC * sizeof(T) == 16) {
        if (staged && steps == 2)
          launch_group<T, VEC, TABLE, true, 2>(qt, kt, ps, p, s, long_index, lds, t0, n, stream);
        else if (staged)
          launch_group<T, VEC, TABLE, true, 1>(qt, kt, ps, p, s, long_index, lds, t0, n, stream);
        else if (steps == 2)
          launch_group<T, VEC, TABLE, false, 2>(qt, kt, ps, p, s, long_index, lds, t0, n, stream);
        else
          launch_group<T, VEC, TABLE, false, 1>(qt, kt, ps, p, s, long_index, lds, t0, n, stream);
      } else {
        launch_group<T, VEC, TABLE, false, 1>(qt, kt, ps, p, s, long_index, lds, t0, n, stream);
      }
      if (hipGetLastError() != hipSuccess) return ROPE_ELAUNCH;
    }
    return ROPE_OK;
  }
  if (long_index)
    hipLaunchKernelGGL((rope_qk_kernel<T, VEC, true, TABLE>), dim3(blocks), dim3(kTokenBlock), 0, stream,
                       qt, kt, ps, p);
  else
    hipLaunchKernelGGL((rope_qk_kernel<T, VEC, false, TABLE>), dim3(blocks), dim3(kTokenBlock), 0, stream,
                       qt, kt, ps, p);
  return hipGetLastError() == hipSuccess ? ROPE_OK : ROPE_ELAUNCH;
}

template <typename T, int VEC>
int32_t launch_vec(void* q, void* k, const PosSource& ps, const RopeParams& p, bool long_index,
                   unsigned blocks, unsigned group_blocks, hipStream_t stream) {
  return p.tab_cos != nullptr
             ? launch_vec<T, VEC, true>(q, k, ps, p, long_index, blocks, group_blocks, stream)
             : launch_vec<T, VEC, false>(q, k, ps, p, long_index, blocks, group_blocks, stream);
}

// Tokens per wave when the caller does not choose: one. Short-lived waves, one per
// token, keep the most loads in flight across the chip (measured on the Qwen3-4B,
// -8B, -32B and 512K-token shapes: one token per wave is fastest or tied). More
// tokens per wave only when the grid would exceed the dispatch size limit.
int32_t auto_tokens_per_wave(int64_t T) {
  const int64_t max_waves = kMaxTokenBlocks * kWaves;
  const int64_t tpw = (T + max_waves - 1) / max_waves;
  return (int32_t)(tpw < 1 ? 1 : tpw);
}

// Grid of the row-group kernel (one 64-lane workgroup per token and row group), or
// 0 when that kernel does not apply: the caller chose tokens per wave, nc neither
// divides 64 nor takes the staged instance (staged_geometry; wide: 16-byte
// chunks), a token stride is 2^32 elements or more, the grid would exceed the
// dispatch size limit, or seqused marks a padded layout and the launch is not
// compact. In that last case many rows are skipped; the row-group kernel spends
// one workgroup per row group of each skipped token where the token kernel spends
// one wave per token, and it measures slower there (Qwen3-8B batch padded to
// 8 x 2048 rows: 34.2-34.4 vs 33.1-33.4 us), so such launches keep the token
// kernel. A compact launch (compact_rows >=
// 0 rotated tokens, cu_valid given) covers only the rotated tokens and takes the
// row-group kernel (28.3 against 32.0 us on that batch).
int64_t group_grid(const RopeParams& p, bool geometry_chosen, bool padded, int64_t compact_rows,
                   bool wide) {
  const bool compact = compact_rows >= 0;
  if (geometry_chosen || (padded && !compact)) return 0;
  if (64 % p.nc != 0 && !staged_geometry(p.nc, wide ? 16 : 0)) return 0;
  // token strides travel as 32-bit kernel arguments
  if (p.q_stride > (int64_t)UINT32_MAX || p.k_stride > (int64_t)UINT32_MAX) return 0;
  const int step_r = (int)group_rows((uint32_t)p.nc, group_steps(p.nc, p.D / 2, wide ? 16 : 0));
  const int64_t groups = (p.Hq + step_r - 1) / step_r + (p.Hkv + step_r - 1) / step_r;
  const int64_t blocks = (compact ? compact_rows : p.T) * groups;
  // < 2^26 workgroups: the dispatch limit, and the range of fastdiv::div
  return blocks <= (int64_t)0xffffffffu / 64 ? blocks : 0;
}

// compact_rows: rotated tokens of a compact launch (ps.cu_valid set), else -1. When
// the row-group kernel does not apply, a compact launch falls back to the token
// kernel over all rows with seqused, which rotates the same tokens.
template <typename T>
int32_t launch_typed(void* q, void* k, PosSource ps, RopeParams& p, int32_t bytes,
                     bool long_index, bool geometry_chosen, int64_t compact_rows,
                     hipStream_t stream) {
  const int32_t vec = bytes / (int32_t)sizeof(T);
  p.nc = (p.D / 2) / vec;
  const int64_t group_blocks = group_grid(p, geometry_chosen, ps.seqused != nullptr,
                                          ps.cu_valid ? compact_rows : -1, bytes == 16);
  if (group_blocks == 0) ps.cu_valid = nullptr;
  if (group_blocks > 0) {
    const int step_r = (int)group_rows((uint32_t)p.nc, group_steps(p.nc, p.D / 2, bytes));
    p.gq = (uint32_t)((p.Hq + step_r - 1) / step_r);
    p.gk = (uint32_t)((p.Hkv + step_r - 1) / step_r);
    p.nc_shift = 0;
    while ((1 << p.nc_shift) < p.nc) ++p.nc_shift;
    p.groups = fastdiv::make(p.gq + p.gk);
  }
  if (group_blocks == 0 && !geometry_chosen) p.tpw = auto_tokens_per_wave(p.T);
  const int64_t waves = (p.T + p.tpw - 1) / p.tpw;
  const int64_t blocks = (waves + kWaves - 1) / kWaves;
  if (group_blocks == 0 && blocks > kMaxTokenBlocks) return ROPE_EINVAL;
  const unsigned b = (unsigned)(group_blocks > 0 ? 0 : blocks);
  const unsigned gb = (unsigned)group_blocks;
  switch (vec) {
    case 1: return launch_vec<T, 1>(q, k, ps, p, long_index, b, gb, stream);
    case 2: return launch_vec<T, 2>(q, k, ps, p, long_index, b, gb, stream);
    case 4: return launch_vec<T, 4>(q, k, ps, p, long_index, b, gb, stream);
    default:
      if constexpr (sizeof(T) == 2)
        return launch_vec<T, 8>(q, k, ps, p, long_index, b, gb, stream);
      return ROPE_EINVAL;
  }
}

}  // namespace

extern "C" {

// Shared by rope_qk_apply_ex (cos/sin evaluated from theta and pos_scale) and
// rope_qk_apply_table (tab_cos != NULL: cos/sin read from the caller's tables;
// theta and pos_scale unused).
// cu_valid / valid_tokens: a compact launch over a padded layout (rope_qk_apply_padded);
// valid_tokens = -1 for every other entry point.
static int32_t apply_impl(void* q, void* k, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                          int64_t q_token_stride, int64_t k_token_stride,
                          const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                          const int32_t* cu_valid, int64_t valid_tokens,
                          const int32_t* seq_offsets, const int32_t* position_ids, double theta,
                          double pos_scale, const float* tab_cos, const float* tab_sin,
                          int32_t tab_rows, int32_t dtype, int32_t direction, int32_t index_mode,
                          int32_t tokens_per_wave, void* stream) {
  const bool table = tab_cos != nullptr;
  if (dtype != ROPE_F32 && dtype != ROPE_BF16 && dtype != ROPE_F16) return ROPE_EUNSUPPORTED;
  if (T < 0 || T > ((int64_t)1 << 40)) return ROPE_EINVAL;
  if (Hq < 0 || Hkv < 0 || Hq > kMaxHeads || Hkv > kMaxHeads) return ROPE_EINVAL;
  if (!valid_D(D)) return ROPE_EINVAL;
  if (table ? (tab_sin == nullptr || tab_rows < 1)
            : (!valid_theta(theta) || !valid_scale(pos_scale)))
    return ROPE_EINVAL;
  if (num_seqs < 0 || num_seqs == INT32_MAX) return ROPE_EINVAL;
  if (direction != 1 && direction != -1) return ROPE_EINVAL;
  if (index_mode < ROPE_INDEX_AUTO || index_mode > ROPE_INDEX_64) return ROPE_EINVAL;
  if (tokens_per_wave < 0 || tokens_per_wave > kMaxTokensPerWave) return ROPE_EINVAL;
  const int32_t H = Hq + Hkv;
  if (T > 0 && H == 0) return ROPE_EINVAL;
  if (T == 0) return ROPE_OK;
  if (position_ids == nullptr) {
    if (num_seqs == 0) return ROPE_OK;  // nothing is rotated
    if (cu_seqlens == nullptr) return ROPE_EINVAL;
  }
  if ((Hq > 0 && q == nullptr) || (Hkv > 0 && k == nullptr)) return ROPE_EINVAL;
  const bool compact = valid_tokens >= 0;
  if (compact) {
    if (valid_tokens > T) return ROPE_EINVAL;
    if (valid_tokens == 0) return ROPE_OK;  // nothing is rotated
    if (cu_valid == nullptr) return ROPE_EINVAL;
  }

  const int64_t qs = q_token_stride == 0 ? (int64_t)Hq * D : q_token_stride;
  const int64_t ks = k_token_stride == 0 ? (int64_t)Hkv * D : k_token_stride;
  if (qs < (int64_t)Hq * D || ks < (int64_t)Hkv * D) return ROPE_EINVAL;  // tokens overlap
  // T * stride is formed only after these bounds rule out overflow (T <= 2^40).
  const int64_t span_max = (int64_t)1 << 48;
  if ((Hq > 0 && qs > span_max / T) || (Hkv > 0 && ks > span_max / T)) return ROPE_EINVAL;

  // [U-int64] 64-bit offsets exactly when some offset of the launch needs them.
  const int64_t lim = (int64_t)1 << 31;
  const bool needs_long = T * (int64_t)H * (int64_t)D >= lim || (Hq > 0 && T * qs >= lim) ||
                          (Hkv > 0 && T * ks >= lim);
  if (index_mode == ROPE_INDEX_32 && needs_long) return ROPE_EINVAL;
  const bool long_index = needs_long || index_mode == ROPE_INDEX_64;

  RopeParams p;
  p.T = T;
  p.num_seqs = num_seqs;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.D = D;
  p.q_stride = qs;
  p.k_stride = ks;
  p.tpw = tokens_per_wave == 0 ? 1 : tokens_per_wave;  // 0: launch_typed picks the geometry
  p.sin_sign = direction > 0 ? 1.0f : -1.0f;
  p.tab_cos = table ? tab_cos : nullptr;
  p.tab_sin = table ? tab_sin : nullptr;
  p.tab_rows = table ? tab_rows : 0;
  if (table) {
    p.pos_scale = 1.0f;
    for (int32_t j = 0; j < kMaxHalf; ++j) p.inv_freq[j] = 0.0f;  // unused
  } else {
    p.pos_scale = (float)pos_scale;
    host_inv_freq(theta, D, p.inv_freq);
  }

  PosSource ps;
  ps.position_ids = position_ids;
  ps.cu = position_ids ? nullptr : cu_seqlens;
  ps.seqused = position_ids ? nullptr : seqused;
  ps.seq_offsets = position_ids ? nullptr : seq_offsets;
  ps.num_seqs = position_ids ? 0 : num_seqs;
  ps.cu_valid = compact ? cu_valid : nullptr;

  void* qp = Hq > 0 ? q : nullptr;
  void* kp = Hkv > 0 ? k : nullptr;
  const int32_t bytes = chunk_bytes(D, elem_size(dtype), qp, kp, qs, ks);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool chosen = tokens_per_wave != 0;
  switch (dtype) {
    case ROPE_F32:
      return launch_typed<float>(qp, kp, ps, p, bytes, long_index, chosen, valid_tokens, s);
    case ROPE_BF16:
      return launch_typed<__bf16>(qp, kp, ps, p, bytes, long_index, chosen, valid_tokens, s);
    default:
      return launch_typed<_Float16>(qp, kp, ps, p, bytes, long_index, chosen, valid_tokens, s);
  }
}

int32_t rope_qk_apply_ex(void* q, void* k, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                         int64_t q_token_stride, int64_t k_token_stride,
                         const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                         const int32_t* seq_offsets, const int32_t* position_ids, double theta,
                         double pos_scale, int32_t dtype, int32_t direction, int32_t index_mode,
                         int32_t tokens_per_wave, void* stream) {
  return apply_impl(q, k, T, Hq, Hkv, D, q_token_stride, k_token_stride, cu_seqlens, num_seqs,
                    seqused, nullptr, -1, seq_offsets, position_ids, theta, pos_scale, nullptr,
                    nullptr, 0, dtype, direction, index_mode, tokens_per_wave, stream);
}

int32_t rope_qk_apply_padded(void* q, void* k, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                             int64_t q_token_stride, int64_t k_token_stride,
                             const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                             const int32_t* cu_valid, int64_t valid_tokens,
                             const int32_t* seq_offsets, double theta, double pos_scale,
                             int32_t dtype, int32_t direction, int32_t index_mode, void* stream) {
  if (valid_tokens < 0) return ROPE_EINVAL;
  return apply_impl(q, k, T, Hq, Hkv, D, q_token_stride, k_token_stride, cu_seqlens, num_seqs,
                    seqused, cu_valid, valid_tokens, seq_offsets, nullptr, theta, pos_scale,
                    nullptr, nullptr, 0, dtype, direction, index_mode, 0, stream);
}

int32_t rope_qk_apply_table(void* q, void* k, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                            int64_t q_token_stride, int64_t k_token_stride,
                            const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                            const int32_t* seq_offsets, const int32_t* position_ids,
                            const float* cos_tab, const float* sin_tab, int32_t tab_rows,
                            int32_t dtype, int32_t direction, int32_t index_mode,
                            int32_t tokens_per_wave, void* stream) {
  if (dtype != ROPE_F32 && dtype != ROPE_BF16 && dtype != ROPE_F16) return ROPE_EUNSUPPORTED;
  if (cos_tab == nullptr || sin_tab == nullptr || tab_rows < 1) return ROPE_EINVAL;
  return apply_impl(q, k, T, Hq, Hkv, D, q_token_stride, k_token_stride, cu_seqlens, num_seqs,
                    seqused, nullptr, -1, seq_offsets, position_ids, 1.0, 1.0, cos_tab, sin_tab,
                    tab_rows, dtype, direction, index_mode, tokens_per_wave, stream);
}

int32_t rope_qk_apply(void* q, void* k, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                      const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                      double theta, int32_t dtype, int32_t direction, int32_t index_mode,
                      int32_t tokens_per_wave, void* stream) {
  return rope_qk_apply_ex(q, k, T, Hq, Hkv, D, 0, 0, cu_seqlens, num_seqs, seqused, nullptr,
                          nullptr, theta, 1.0, dtype, direction, index_mode, tokens_per_wave,
                          stream);
}

int32_t rope_qk_fwd(void* q, void* k, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                    const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                    double theta, int32_t dtype, void* stream) {
  return rope_qk_apply_ex(q, k, T, Hq, Hkv, D, 0, 0, cu_seqlens, num_seqs, seqused, nullptr,
                          nullptr, theta, 1.0, dtype, +1, ROPE_INDEX_AUTO, 0, stream);
}

int32_t rope_qk_bwd(void* dq, void* dk, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                    const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                    double theta, int32_t dtype, void* stream) {
  return rope_qk_apply_ex(dq, dk, T, Hq, Hkv, D, 0, 0, cu_seqlens, num_seqs, seqused, nullptr,
                          nullptr, theta, 1.0, dtype, -1, ROPE_INDEX_AUTO, 0, stream);
}

int32_t rope_qk_fwd_pos(void* q, void* k, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                        const int32_t* position_ids, double theta, int32_t dtype, void* stream) {
  if (T > 0 && position_ids == nullptr) return ROPE_EINVAL;
  return rope_qk_apply_ex(q, k, T, Hq, Hkv, D, 0, 0, nullptr, 0, nullptr, nullptr, position_ids,
                          theta, 1.0, dtype, +1, ROPE_INDEX_AUTO, 0, stream);
}

int32_t rope_qk_bwd_pos(void* dq, void* dk, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                        const int32_t* position_ids, double theta, int32_t dtype, void* stream) {
  if (T > 0 && position_ids == nullptr) return ROPE_EINVAL;
  return rope_qk_apply_ex(dq, dk, T, Hq, Hkv, D, 0, 0, nullptr, 0, nullptr, nullptr, position_ids,
                          theta, 1.0, dtype, -1, ROPE_INDEX_AUTO, 0, stream);
}

int32_t rope_positions_ex(const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                          const int32_t* seq_offsets, const int32_t* position_ids, int64_t T,
                          int32_t* pos_out, int32_t* seq_out, void* stream) {
  if (T < 0 || T > ((int64_t)1 << 40)) return ROPE_EINVAL;
  if (num_seqs < 0 || num_seqs == INT32_MAX) return ROPE_EINVAL;
  if (T == 0 || (pos_out == nullptr && seq_out == nullptr)) return ROPE_OK;
  if (position_ids == nullptr && num_seqs > 0 && cu_seqlens == nullptr) return ROPE_EINVAL;
  const int64_t blocks = (T + kBlock - 1) / kBlock;
  if (blocks > kMaxBlocksX) return ROPE_EINVAL;
  PosSource ps;
  ps.cu_valid = nullptr;
  ps.position_ids = position_ids;
  ps.cu = position_ids ? nullptr : cu_seqlens;
  ps.seqused = position_ids ? nullptr : seqused;
  ps.seq_offsets = position_ids ? nullptr : seq_offsets;
  ps.num_seqs = position_ids ? 0 : num_seqs;
  hipLaunchKernelGGL(rope_positions_kernel, dim3((unsigned)blocks), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), ps, T, pos_out, seq_out);
  return hipGetLastError() == hipSuccess ? ROPE_OK : ROPE_ELAUNCH;
}

int32_t rope_valid_prefix(const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                          int32_t* cu_valid_out, void* stream) {
  if (num_seqs < 0 || num_seqs == INT32_MAX || cu_valid_out == nullptr) return ROPE_EINVAL;
  if (num_seqs > 0 && cu_seqlens == nullptr) return ROPE_EINVAL;
  hipLaunchKernelGGL(rope_valid_prefix_kernel, dim3(1), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), cu_seqlens, num_seqs, seqused, cu_valid_out);
  return hipGetLastError() == hipSuccess ? ROPE_OK : ROPE_ELAUNCH;
}

int32_t rope_positions(const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* seqused,
                       int64_t T, int32_t* pos_out, int32_t* seq_out, void* stream) {
  if (num_seqs > 0 && cu_seqlens == nullptr) return ROPE_EINVAL;
  return rope_positions_ex(cu_seqlens, num_seqs, seqused, nullptr, nullptr, T, pos_out, seq_out,
                           stream);
}

// Shared by rope_cos_sin (positions == NULL: rows are positions 0 .. n-1) and
// rope_cos_sin_at.
static int32_t cos_sin_impl(const int32_t* positions, int64_t n, int32_t D, double theta,
                            double pos_scale, float* cos_out, float* sin_out, void* stream) {
  if (!valid_D(D) || !valid_theta(theta) || !valid_scale(pos_scale)) return ROPE_EINVAL;
  if (n < 0 || n > ((int64_t)1 << 34)) return ROPE_EINVAL;
  if (n == 0) return ROPE_OK;
  if (cos_out == nullptr || sin_out == nullptr) return ROPE_EINVAL;
  CosSinParams p;
  host_inv_freq(theta, D, p.inv_freq);
  p.pos_scale = (float)pos_scale;
  const int32_t half = D / 2;
  const int64_t blocks = (n * half + kBlock - 1) / kBlock;
  if (blocks > kMaxBlocksX) return ROPE_EINVAL;
  hipLaunchKernelGGL(rope_cos_sin_kernel, dim3((unsigned)blocks), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), positions, n, half, p, cos_out, sin_out);
  return hipGetLastError() == hipSuccess ? ROPE_OK : ROPE_ELAUNCH;
}

int32_t rope_cos_sin(int32_t max_pos, int32_t D, double theta, float* cos_out, float* sin_out,
                     void* stream) {
  if (max_pos < 0) return ROPE_EINVAL;
  return cos_sin_impl(nullptr, max_pos, D, theta, 1.0, cos_out, sin_out, stream);
}

int32_t rope_cos_sin_at(const int32_t* positions, int64_t n, int32_t D, double theta,
                        double pos_scale, float* cos_out, float* sin_out, void* stream) {
  if (n > 0 && positions == nullptr) return ROPE_EINVAL;
  return cos_sin_impl(positions, n, D, theta, pos_scale, cos_out, sin_out, stream);
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
