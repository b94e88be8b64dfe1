// Internal helpers shared by the nxattn HIP sources (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>
#include <cstdio>
#include <cstdarg>

#include "nxattn.h"

namespace nx {

// ---- error reporting (thread-local detail string) ----------------------------------
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
int check_launch(const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int64_t esize(int dtype) { return dtype == NXATTN_F32 ? 4 : 2; }

// true if [a, a+na) and [b, b+nb) (bytes) overlap
inline bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  auto x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

// Largest byte extent a tensor argument may span (2^50 bytes, far beyond any device's
// memory). The extents for the overlap checks are formed with overflow checks against
// it, so caller-supplied sizes and strides of any value keep the host arithmetic exact.
constexpr int64_t MAX_SPAN = INT64_C(1) << 50;

// Byte extent of a strided [n0, n1, n2, inner] view of es-byte elements: 0 when a size is
// 0 or less, -1 when a stride is negative or the extent exceeds MAX_SPAN.
inline int64_t span_bytes(const int64_t st[3], int64_t n0, int64_t n1, int64_t n2, int64_t inner, int64_t es) {
  if (n0 <= 0 || n1 <= 0 || n2 <= 0 || inner <= 0) return 0;
  const int64_t n[3] = {n0, n1, n2};
  int64_t e = inner, t = 0;
  for (int i = 0; i < 3; ++i)
    if (st[i] < 0 || __builtin_mul_overflow(n[i] - 1, st[i], &t) || __builtin_add_overflow(e, t, &e)) return -1;
  return (__builtin_mul_overflow(e, es, &e) || e > MAX_SPAN) ? -1 : e;
}

// Bytes of n0 * n1 * n2 * n3 dense es-byte elements (sizes >= 0), -1 beyond MAX_SPAN.
inline int64_t dense_bytes(int64_t n0, int64_t n1, int64_t n2, int64_t n3, int64_t es) {
  const int64_t n[4] = {n0, n1, n2, n3};
  int64_t e = es;
  for (int i = 0; i < 4; ++i)
    if (n[i] < 0 || __builtin_mul_overflow(e, n[i], &e)) return -1;
  return e > MAX_SPAN ? -1 : e;
}

// A stride of s es-byte elements is a whole number of 16-byte units (the unsigned product
// is exact modulo 16 for any s).
inline bool stride16(int64_t s, int64_t es) { return ((uint64_t)s * (uint64_t)es) % 16u == 0; }

// ---- device-side element types ------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// round-to-nearest-even (gfx950 v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = static_cast<__bf16>(lo);
  r[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, r);
}

// ---- RoPE descriptors ---------------------------------------------------------------------
// Checks one nxattn_rope_desc against seq and head_dim (fail() with `who` on error).
int check_rope_desc(const nxattn_rope_desc& d, int64_t seq, int64_t head_dim, const char* who);

// ---- FP8 quantization ----------------------------------------------------------------------
// Running maxima of the quantizers (float bits of non-negative values): AMAX_SLOTS copies of
// the [batch * heads] array, each starting on its own 128-byte line; workgroup w updates
// copy w % AMAX_SLOTS, so that the global atomics of thousands of workgroups on a few
// slices do not all queue on one cache line. The exponent pass reduces over the copies.
constexpr int AMAX_SLOTS = 32;
inline int64_t amax_stride(int64_t n) { return (n + 31) / 32 * 32; }
inline int64_t amax_words(int64_t n) { return AMAX_SLOTS * amax_stride(n); }
// zeroes every copy of the n maxima
void launch_amax_clear(uint32_t* amax, int64_t n, hipStream_t stream);
// exps[i] = fp8_exponent of the largest of the copies of maximum i, i < n
void launch_fp8_exponents(const uint32_t* amax, int8_t* exps, int64_t n, hipStream_t stream);

// smallest integer e with amax <= 448 * 2^e (0 for 0), held at -127 or above (E8M0 range)
__device__ __forceinline__ int fp8_exponent(float amax) {
  if (amax == 0.f) return 0;
  int E;
  const float m = frexpf(amax, &E);          // amax = m * 2^E, 0.5 <= m < 1; 448 = 0.875 * 2^9
  const int e = E - 9 + (m > 0.875f ? 1 : 0);
  return e < -127 ? -127 : e;
}
// 2^-e exactly, for e in [-127, 126]
__device__ __forceinline__ float exp2_neg(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// The tensors of one RoPE launch: they share batch, seq, head_dim, dtype and positions, and
// their heads are laid end to end (tensor t owns heads hoff[t] .. hoff[t+1]-1 of the
// launch; hoff[t] = total heads for t >= n). Rotation in place uses x[0] only; the fp8
// passes read every x and write codes[t] (contiguous [batch, seq, heads_t, head_dim]) and
// either exps[t] ([batch, heads_t]), with the running maxima in amax (AMAX_SLOTS copies of
// [batch * total heads], copy stride astride), or, with blocks set, scales[t] (E8M0
// codes, contiguous [batch, seq, heads_t, head_dim / 32]) in a single pass.
constexpr int ROPE_MAX_TENSORS = NXATTN_MAX_FP8_TENSORS;
struct RopeTensors {
  void* x[ROPE_MAX_TENSORS];
  int64_t sb[ROPE_MAX_TENSORS], ss[ROPE_MAX_TENSORS], sh[ROPE_MAX_TENSORS];
  uint8_t* codes[ROPE_MAX_TENSORS];
  int8_t* exps[ROPE_MAX_TENSORS];
  uint8_t* scales[ROPE_MAX_TENSORS];
  float mult[ROPE_MAX_TENSORS];   // fp8 passes: multiplier of the stored rotated values (1: none)
  int32_t hoff[ROPE_MAX_TENSORS + 1];
  int32_t n;
  uint32_t* amax;
  int64_t astride;
  int32_t blocks;                 // fp8: one scale per 32-element run (head_dim % 64 == 0)
};
enum class RopeMode { Rotate, Max, Codes, Blocks };

// ---- KV relayout ----------------------------------------------------------------------
// Rows of vpr vectors: src viewed as [LC][A][B][vpr], dst as [LC][B][A][vpr] (replay <->
// online, dims 2 and 3 exchanged); this thread moves vectors i0, i0 + step, ... of dst.
template <typename V>
__device__ __forceinline__ void relayout_rows(const V* __restrict__ src, V* __restrict__ dst, int64_t A, int64_t B,
                                              int64_t vpr, int64_t total, int64_t i0, int64_t step) {
  for (int64_t i = i0; i < total; i += step) {
    const int64_t c = i % vpr;
    const int64_t r = i / vpr;        // destination row (lc, b, a)
    const int64_t a = r % A;
    const int64_t t = r / A;
    const int64_t b = t % B;
    const int64_t lc = t / B;
    dst[i] = src[((lc * A + a) * B + b) * vpr + c];
  }
}
// Relayout jobs appended to a RoPE launch (16-byte vectors): job j moves `total` vectors
// with the workgroups blk0[j] .. blk0[j + 1] - 1 after the RoPE workgroups.
struct RelayoutJobs {
  const u32x4* src[NXATTN_MAX_BRANCHES];
  u32x4* dst[NXATTN_MAX_BRANCHES];
  int64_t A[NXATTN_MAX_BRANCHES], B[NXATTN_MAX_BRANCHES], vpr[NXATTN_MAX_BRANCHES], total[NXATTN_MAX_BRANCHES];
  int32_t blk0[NXATTN_MAX_BRANCHES + 1];
  int32_t n;
};
// workgroups a relayout of `total` vectors takes (as its own launch would)
inline int32_t relayout_blocks(int64_t total) {
  const int64_t blocks = (total + 255) / 256;
  return (int32_t)(blocks < 256 * 64 ? blocks : 256 * 64);
}

// Validates the RoPE arguments (errors name `who`; rope and the x pointers and strides of
// every tensor) and launches: with fp8 == false, the in-place rotation of x[0]; with
// fp8 == true (total heads <= 4096), the clear of the maxima, the pass that takes them
// from the rotated values and the pass that writes exponents and codes, or with
// tt.blocks the one pass that writes codes and block scales. The caller checks codes,
// exps, scales and amax. With jobs (rotation only; checked by the caller), the jobs' rows
// move in the same launch.
int rope_launch(const char* who, const RopeTensors& tt, int64_t batch, int64_t seq, int64_t head_dim, int dtype,
                const nxattn_rope_desc* rope, bool fp8, hipStream_t stream, const RelayoutJobs* jobs = nullptr);

// nxattn_rope_quantize_fp8 (validation and launches; errors name `who`) with the running
// maxima in `workspace`.
int rope_quantize(const char* who, const nxattn_fp8_tensor* tensors, int32_t n_tensors, int dtype, int64_t batch,
                  int64_t seq, int64_t head_dim, const nxattn_rope_desc* rope, void* workspace,
                  int64_t workspace_bytes, hipStream_t stream);

// RoPE of q applied on load by the fused attention kernels (axes beyond n_axes have grid
// 1, pairs 0, offset 0)
struct RopeQ {
  int32_t n_axes, interleaved, global_freq;
  int32_t grid[3], pairs[3], offset[3];
  double log2_theta;
};
// Checks `batch` q_rope descriptors (check_rope_desc, and every position below 2^24: the
// rotation on load holds positions as exact fp32 integers) and converts them into out[];
// errors name `who`.
int rope_q_setup(const nxattn_rope_desc* d, int batch, int64_t seq, int64_t head_dim, const char* who, RopeQ* out);

// ---- launchers implemented per kernel file -------------------------------------------
struct FwdProblem {
  int dtype, batch, seq_q, heads_q, heads_kv, head_dim;
  const void* q; const void* k; const void* v; void* o;
  int64_t qs[3], ks[3], os[3];
  const void* prefix[NXATTN_MAX_BRANCHES];
  int32_t plen[NXATTN_MAX_BRANCHES];
  float scale;
  int32_t rope_q;                       // rotate q on load with rq[b]
  RopeQ rq[NXATTN_MAX_BRANCHES];
  float* lse;                           // one pass: [batch, heads_q, seq_q] or NULL
  int32_t prefix_only;                  // keys = prefix rows only
  // Key ranges: work item `split` of a branch covers tiles [split*per, split*per + per)
  // (clipped to the branch; empty ranges do nothing). A branch with at most `per` tiles
  // (every branch when nsplit == 1) is one range and its o (and lse) are written
  // directly; the ranges of a longer branch write normalised fp32 partials part_o
  // [nsplit, batch, seq_q, heads_q, D] and their log-sum-exp part_lse
  // [nsplit, batch, heads_q, seq_q] for the merge pass.
  int32_t nsplit, per;
  float* part_o;
  float* part_lse;
  // branch pairs (bf16, batch 2, one key range): cfg [seq_q, heads_q, D] with strides cs
  // {s, h} receives the guidance combination of the two branches' rounded outputs, and o
  // may be NULL
  void* cfg;
  int64_t cs[2];
  float guidance;
};
constexpr int KEY_TILE = 64;            // keys per tile in both attention kernels
// Launch shape of an attention kernel for a problem: workgroups per key range of one
// branch (all kv heads and query blocks) and workgroups resident per CU.
struct FwdShape { int64_t wgs_per_range; int resident_per_cu; };
FwdShape fwd_shape_bf16(const FwdProblem& p);
FwdShape fwd_shape_f32(const FwdProblem& p);
int launch_fwd_bf16(const FwdProblem& p, hipStream_t stream);
int launch_fwd_f32(const FwdProblem& p, hipStream_t stream);

// Merge of per-part attention results (see nxattn_attn_merge). Part p of batch entry b
// is used for p < nparts[b] (per_branch; rows of a batch entry with one part were
// written directly and are skipped) or p < n_all.
struct MergeProblem {
  const void* po[NXATTN_MAX_SPLITS];
  const float* pl[NXATTN_MAX_SPLITS];
  int32_t n_all, per_branch;
  int32_t nparts[NXATTN_MAX_BRANCHES];
  int in_dtype, out_dtype;
  int64_t batch, seq, heads, head_dim;
  int64_t is[3], os[3];
  void* o;
  float* lse;
};
int launch_merge(const MergeProblem& m, hipStream_t stream);

}  // namespace nx
