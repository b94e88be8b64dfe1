// Merge of attention results over disjoint key sets into the result over their union,
// the block form of the online-softmax rescale:
//   lse = log sum_p exp(lse_p),   o = sum_p exp(lse_p - lse) * o_p.
// KLiteInfer page, "架构": the softmax between the two GEMMs (over a union of key blocks
// its normaliser is the sum of the blocks' normalisers); NeoPP page: the replay divides
// the work by a sequence-parallel degree, and key blocks computed apart combine this way.
//
// HBM-bound. A row (b, s, h) of head_dim elements is served by a power-of-two group of
// threads inside one wave; each thread owns 8 consecutive elements and reads the same 8
// of every part (16-byte loads; consecutive threads read consecutive memory when rows
// are contiguous) and each part's lse of the row. Bytes per row: parts * (D * in_size +
// 4) + D * out_size (+ 4 for the lse output). Each output element is read (from every
// part) and written by one thread, and a row's lse is read and written inside one wave,
// so an output may be exactly one of the parts (in-place accumulation).
#include <cstring>

#include "nx_internal.h"

namespace nx {

namespace mergek {

constexpr int THREADS = 256;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

struct Args {
  const void* po[NXATTN_MAX_SPLITS];
  const float* pl[NXATTN_MAX_SPLITS];
  int32_t n_all, per_branch;
  int32_t nparts[NXATTN_MAX_BRANCHES];
  uint32_t heads, seq, cpr, tpr_log2;  // chunks of 8 per row; threads per row = 1 << tpr_log2
  uint32_t total;                      // rows << tpr_log2
  int64_t is0, is1, is2, os0, os1, os2;
  void* o;
  float* lse;
};

__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
}
__device__ __forceinline__ void load8(const uint16_t* p, float (&x)[8]) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(v[e] << 16);
    x[2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
  }
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}
__device__ __forceinline__ void store8(uint16_t* p, const float (&x)[8]) {
  *reinterpret_cast<u32x4*>(p) = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                       pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
}

template <typename TI, typename TO>
__global__ __launch_bounds__(THREADS) void merge_kernel(Args a) {
  const uint32_t tid = blockIdx.x * THREADS + threadIdx.x;
  if (tid >= a.total) return;
  const uint32_t row = tid >> a.tpr_log2, c = tid & ((1u << a.tpr_log2) - 1);
  if (c >= a.cpr) return;                       // padding threads of a row
  const uint32_t h = row % a.heads, bs = row / a.heads;
  const uint32_t s = bs % a.seq, b = bs / a.seq;
  // parts of this row (per batch entry for split keys; b < NXATTN_MAX_BRANCHES then)
  int n = a.n_all;
  if (a.per_branch) {
#pragma unroll
    for (int i = 0; i < NXATTN_MAX_BRANCHES; ++i) n = (uint32_t)i == b ? a.nparts[i] : n;
    if (n <= 1) return;                         // written directly by the attention kernel
  }
  const int64_t lrow = ((int64_t)b * a.heads + h) * a.seq + s;
  float lv[NXATTN_MAX_SPLITS];
  float m = -__builtin_inff();
#pragma unroll
  for (int p = 0; p < NXATTN_MAX_SPLITS; ++p) {
    lv[p] = p < n ? a.pl[p][lrow] : -__builtin_inff();
    m = __builtin_fmaxf(m, lv[p]);
  }
  const int64_t ioff = (int64_t)b * a.is0 + (int64_t)s * a.is1 + (int64_t)h * a.is2 + 8 * c;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float sum = 0.f;
#pragma unroll
  for (int p = 0; p < NXATTN_MAX_SPLITS; ++p) {
    if (p < n) {
      float x[8];
      load8(static_cast<const TI*>(a.po[p]) + ioff, x);
      const float wgt = __builtin_amdgcn_exp2f((lv[p] - m) * LOG2E);   // 0 for an empty part
      sum += wgt;
      // an empty part's output is not used (it may hold anything)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = wgt > 0.f ? __builtin_fmaf(wgt, x[e], acc[e]) : acc[e];
    }
  }
  const float inv = 1.0f / sum;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= inv;
  store8(static_cast<TO*>(a.o) + (int64_t)b * a.os0 + (int64_t)s * a.os1 + (int64_t)h * a.os2 + 8 * c, acc);
  if (a.lse && c == 0) a.lse[lrow] = m + LN2 * __builtin_amdgcn_logf(sum);
}

}  // namespace mergek

int launch_merge(const MergeProblem& m, hipStream_t stream) {
  using namespace mergek;
  Args a;
  std::memset(&a, 0, sizeof(a));
  for (int p = 0; p < NXATTN_MAX_SPLITS; ++p) { a.po[p] = m.po[p]; a.pl[p] = m.pl[p]; }
  a.n_all = m.n_all; a.per_branch = m.per_branch;
  for (int b = 0; b < NXATTN_MAX_BRANCHES; ++b) a.nparts[b] = m.nparts[b];
  const int64_t cpr = m.head_dim / 8;
  int lg = 0;
  while ((1 << lg) < cpr) ++lg;
  const int64_t rows = m.batch * m.seq * m.heads;
  const int64_t total = rows << lg;
  if (m.seq > UINT32_MAX / 2 || m.heads > UINT32_MAX / 2 || total > (int64_t)UINT32_MAX - THREADS)
    return fail(NXATTN_ERR_UNSUPPORTED, "merge: problem too large");
  a.heads = (uint32_t)m.heads; a.seq = (uint32_t)m.seq; a.cpr = (uint32_t)cpr;
  a.tpr_log2 = (uint32_t)lg; a.total = (uint32_t)total;
  a.is0 = m.is[0]; a.is1 = m.is[1]; a.is2 = m.is[2];
  a.os0 = m.os[0]; a.os1 = m.os[1]; a.os2 = m.os[2];
  a.o = m.o; a.lse = m.lse;
  const unsigned grid = (unsigned)((total + THREADS - 1) / THREADS);
  const bool fin = m.in_dtype == NXATTN_F32, fout = m.out_dtype == NXATTN_F32;
  if (fin && fout) merge_kernel<float, float><<<grid, THREADS, 0, stream>>>(a);
  else if (fin) merge_kernel<float, uint16_t><<<grid, THREADS, 0, stream>>>(a);
  else if (fout) merge_kernel<uint16_t, float><<<grid, THREADS, 0, stream>>>(a);
  else merge_kernel<uint16_t, uint16_t><<<grid, THREADS, 0, stream>>>(a);
  return check_launch("attention merge");
}

}  // namespace nx

using namespace nx;

extern "C" int nxattn_attn_merge(const void* const* part_o, const float* const* part_lse, int32_t n_parts,
                                 int64_t batch, int64_t seq, int64_t heads, int64_t head_dim,
                                 const int64_t part_strides[3], int dtype, void* o, const int64_t o_strides[3],
                                 float* lse, hipStream_t stream) {
  clear_error();
  if (dtype != NXATTN_F32 && dtype != NXATTN_BF16)
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_attn_merge: dtype %d is not F32 or BF16", dtype);
  if (n_parts < 1 || n_parts > NXATTN_MAX_SPLITS)
    return fail(NXATTN_ERR_INVALID, "nxattn_attn_merge: n_parts %d not in [1, %d]", n_parts, NXATTN_MAX_SPLITS);
  if (batch < 0 || seq < 0 || heads < 0 || head_dim <= 0)
    return fail(NXATTN_ERR_INVALID, "nxattn_attn_merge: bad sizes");
  if (head_dim % 8 != 0 || head_dim > 256)
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_attn_merge: head_dim %lld is not a multiple of 8 in [8, 256]",
                (long long)head_dim);
  if (!part_o || !part_lse || !part_strides || !o_strides)
    return fail(NXATTN_ERR_INVALID, "nxattn_attn_merge: NULL array argument");
  if (batch == 0 || seq == 0 || heads == 0) return NXATTN_OK;
  if (!o) return fail(NXATTN_ERR_INVALID, "nxattn_attn_merge: o is NULL");
  const int64_t es = esize(dtype);
  for (int i = 0; i < 3; ++i) {
    if (part_strides[i] < 0 || o_strides[i] < 0) return fail(NXATTN_ERR_INVALID, "nxattn_attn_merge: negative stride");
    if (!stride16(part_strides[i], es) || !stride16(o_strides[i], es))
      return fail(NXATTN_ERR_ALIGN, "nxattn_attn_merge: strides must be multiples of 16 bytes");
  }
  if (!aligned16(o)) return fail(NXATTN_ERR_ALIGN, "nxattn_attn_merge: o is not 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(NXATTN_ERR_ALIGN, "nxattn_attn_merge: lse is not 4-byte aligned");
  const int64_t ob = span_bytes(o_strides, batch, seq, heads, head_dim, es);
  const int64_t pb = span_bytes(part_strides, batch, seq, heads, head_dim, es);
  const int64_t lb = dense_bytes(batch, heads, seq, 1, 4);
  if (ob < 0 || pb < 0 || lb < 0)
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_attn_merge: sizes or strides span more than 2^50 bytes");
  const bool same_strides = part_strides[0] == o_strides[0] && part_strides[1] == o_strides[1] &&
                            part_strides[2] == o_strides[2];
  for (int p = 0; p < n_parts; ++p) {
    if (!part_o[p] || !part_lse[p]) return fail(NXATTN_ERR_INVALID, "nxattn_attn_merge: part %d is NULL", p);
    if (!aligned16(part_o[p])) return fail(NXATTN_ERR_ALIGN, "nxattn_attn_merge: part_o[%d] misaligned", p);
    if (reinterpret_cast<uintptr_t>(part_lse[p]) & 3u)
      return fail(NXATTN_ERR_ALIGN, "nxattn_attn_merge: part_lse[%d] misaligned", p);
    const bool o_is_part = part_o[p] == o && same_strides;
    if (!o_is_part && overlaps(o, ob, part_o[p], pb))
      return fail(NXATTN_ERR_INVALID, "nxattn_attn_merge: o overlaps part_o[%d] (only exact aliasing is allowed)", p);
    if (overlaps(o, ob, part_lse[p], lb))
      return fail(NXATTN_ERR_INVALID, "nxattn_attn_merge: o overlaps part_lse[%d]", p);
    if (lse) {
      if (part_lse[p] != lse && overlaps(lse, lb, part_lse[p], lb))
        return fail(NXATTN_ERR_INVALID, "nxattn_attn_merge: lse overlaps part_lse[%d] (only exact aliasing is allowed)", p);
      if (overlaps(lse, lb, part_o[p], pb))
        return fail(NXATTN_ERR_INVALID, "nxattn_attn_merge: lse overlaps part_o[%d]", p);
    }
  }
  if (lse && overlaps(lse, lb, o, ob)) return fail(NXATTN_ERR_INVALID, "nxattn_attn_merge: lse overlaps o");

  MergeProblem m;
  std::memset(&m, 0, sizeof(m));
  for (int p = 0; p < n_parts; ++p) { m.po[p] = part_o[p]; m.pl[p] = part_lse[p]; }
  m.n_all = n_parts; m.per_branch = 0;
  m.in_dtype = dtype; m.out_dtype = dtype;
  m.batch = batch; m.seq = seq; m.heads = heads; m.head_dim = head_dim;
  for (int i = 0; i < 3; ++i) { m.is[i] = part_strides[i]; m.os[i] = o_strides[i]; }
  m.o = o; m.lse = lse;
  return launch_merge(m, stream);
}
