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

// RoPE of q applied on load by the fused attention kernel (axes beyond n_axes have grid
// 1, pairs 0, offset 0)
struct RopeQ {
  int32_t n_axes, interleaved, global_freq;
  int32_t grid[3], pairs[3], offset[3];
  float log2_theta;
};

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
