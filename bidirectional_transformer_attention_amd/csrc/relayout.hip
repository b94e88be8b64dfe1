// KV relayout between the replay layout [L,2,H,S,D] and the online layout
// [L,2,S,H,D] (NeoPP page, "KV file layout": converting exchanges dims 2 and 3).
//
// Each (l, c, a, b) row of D elements is contiguous in both layouts, so the op is a
// permutation of whole rows. Threads are laid out over the destination (writes fully
// coalesced); each source row is read in full by consecutive lanes. Rows are moved in
// 16-byte vectors when the row size and pointers allow it, else in 4- or 2-byte words.
// HBM-bound: 2 * L*2*H*S*D*esize bytes per call.
#include "nx_internal.h"

namespace nx {

template <typename V>
__global__ __launch_bounds__(256) void relayout_kernel(const V* __restrict__ src, V* __restrict__ dst,
                                                       int64_t A, int64_t B, int64_t vpr, int64_t total) {
  relayout_rows(src, dst, A, B, vpr, total, (int64_t)blockIdx.x * blockDim.x + threadIdx.x,
                (int64_t)gridDim.x * blockDim.x);
}

template <typename V>
static int launch(const void* src, void* dst, int64_t A, int64_t B, int64_t row_bytes, int64_t rows_total,
                  hipStream_t stream) {
  const int64_t vpr = row_bytes / (int64_t)sizeof(V);
  const int64_t total = vpr * rows_total;
  const int grid = relayout_blocks(total);
  relayout_kernel<V><<<grid, 256, 0, stream>>>(static_cast<const V*>(src), static_cast<V*>(dst), A, B, vpr, total);
  return check_launch("nxattn_kv_relayout");
}

}  // namespace nx

using namespace nx;

extern "C" int nxattn_kv_relayout(const void* src, void* dst, int64_t layers, int64_t kv_heads, int64_t seq,
                                  int64_t head_dim, int dtype, int dir, hipStream_t stream) {
  clear_error();
  if (dtype != NXATTN_F32 && dtype != NXATTN_BF16)
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_kv_relayout: dtype %d is not F32 or BF16", dtype);
  if (dir != 0 && dir != 1) return fail(NXATTN_ERR_INVALID, "nxattn_kv_relayout: dir must be 0 or 1");
  if (layers < 0 || kv_heads < 0 || seq < 0 || head_dim < 0)
    return fail(NXATTN_ERR_INVALID, "nxattn_kv_relayout: negative size");
  if (layers == 0 || kv_heads == 0 || seq == 0 || head_dim == 0) return NXATTN_OK;
  if (!src || !dst) return fail(NXATTN_ERR_INVALID, "nxattn_kv_relayout: NULL pointer");
  const int64_t es = esize(dtype);
  if (head_dim > (INT64_C(1) << 20) || kv_heads > (INT64_C(1) << 20) || seq > (INT64_C(1) << 31) ||
      layers > (INT64_C(1) << 20))
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_kv_relayout: size out of range");
  const int64_t bytes = dense_bytes(layers * 2, kv_heads, seq, head_dim, es);
  if (bytes < 0) return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_kv_relayout: the tensor spans more than 2^50 bytes");
  const int64_t rows = layers * 2 * kv_heads * seq;
  const int64_t row_bytes = head_dim * es;
  if (overlaps(src, bytes, dst, bytes))
    return fail(NXATTN_ERR_INVALID, "nxattn_kv_relayout: src and dst overlap");
  // dir 0: src [LC][H][S] -> dst [LC][S][H]; dir 1: src [LC][S][H] -> dst [LC][H][S]
  const int64_t A = dir == 0 ? kv_heads : seq;
  const int64_t B = dir == 0 ? seq : kv_heads;
  const uintptr_t align = reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst);
  if (row_bytes % 16 == 0 && (align & 15u) == 0) return launch<u32x4>(src, dst, A, B, row_bytes, rows, stream);
  if (row_bytes % 4 == 0 && (align & 3u) == 0) return launch<uint32_t>(src, dst, A, B, row_bytes, rows, stream);
  if ((align & 1u) == 0) return launch<uint16_t>(src, dst, A, B, row_bytes, rows, stream);
  return fail(NXATTN_ERR_ALIGN, "nxattn_kv_relayout: pointers must be at least 2-byte aligned");
}
