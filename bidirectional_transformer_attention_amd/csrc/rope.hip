// In-place rotary position embedding over 1, 2 or 3 grid axes (KLiteInfer page,
// section "架构": RoPE / 2-D RoPE / MRoPE operators; NeoPP page: explicit position
// offsets supplied with the KV cache).
//
// One workgroup handles TOK consecutive tokens of one branch. The angle of each
// (token, pair) depends only on the position and the pair, not on the head, so the
// workgroup first evaluates cos/sin once per (token, pair) in fp64 into LDS, then all
// threads rotate every head of those tokens. A thread owns four consecutive rotary
// pairs of one (token, head) and moves them with one or two vector loads. HBM-bound:
// 2 * B*S*H*D*esize bytes per call.
#include <cmath>
#include <cstring>

#include "nx_internal.h"

namespace nx {

constexpr int ROPE_TOK = 4;          // tokens per workgroup
constexpr int ROPE_MAX_HALF = 128;   // head_dim / 2 limit

struct RopeBranch {
  int32_t n_axes, interleaved, global_freq;
  int32_t grid[3], pairs[3], offset[3];
  double log2_theta;
};
struct RopeArgs {
  RopeBranch br[NXATTN_MAX_BRANCHES];
};

template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(T* x, int64_t seq, int64_t heads, int32_t D,
                                                   int64_t sb, int64_t ss, int64_t sh, RopeArgs args) {
  __shared__ float cs[ROPE_TOK][ROPE_MAX_HALF];
  __shared__ float sn[ROPE_TOK][ROPE_MAX_HALF];
  const int half = D / 2;
  const int64_t blocks_per_branch = (seq + ROPE_TOK - 1) / ROPE_TOK;
  const int b = (int)(blockIdx.x / blocks_per_branch);
  const int64_t s0 = (blockIdx.x % blocks_per_branch) * ROPE_TOK;
  const RopeBranch& br = args.br[b];

  // 1. angles: token s -> row-major grid coordinates (+ offset) -> per-pair angle
  for (int idx = threadIdx.x; idx < ROPE_TOK * half; idx += blockDim.x) {
    const int tk = idx / half, j = idx % half;
    const int64_t s = s0 + tk;
    if (s >= seq) continue;
    int64_t coord[3] = {0, 0, 0};
    int64_t rem = s;
    for (int a = br.n_axes - 1; a >= 0; --a) {
      coord[a] = rem % br.grid[a];
      rem /= br.grid[a];
    }
    int axis = 0, u = j;
    while (axis < br.n_axes - 1 && u >= br.pairs[axis]) { u -= br.pairs[axis]; ++axis; }
    const double pos = (double)(coord[axis] + br.offset[axis]);
    // per-section ladder theta^(-2u / (2 pairs_k)), or one ladder theta^(-2j / D)
    const double inv_freq = br.global_freq ? exp2(br.log2_theta * (-2.0 * (double)j / (double)D))
                                           : exp2(br.log2_theta * (-2.0 * (double)u / (2.0 * (double)br.pairs[axis])));
    double sv, cv;
    sincos(pos * inv_freq, &sv, &cv);
    cs[tk][j] = (float)cv;
    sn[tk][j] = (float)sv;
  }
  __syncthreads();

  // 2. rotate: work item = (token, head, quad of 4 pairs)
  const int quads = half / 4;
  const int64_t items = (int64_t)ROPE_TOK * heads * quads;
  for (int64_t it = threadIdx.x; it < items; it += blockDim.x) {
    const int tk = (int)(it / (heads * quads));
    const int64_t r = it % (heads * quads);
    const int64_t h = r / quads;
    const int q4 = (int)(r % quads);
    const int64_t s = s0 + tk;
    if (s >= seq) continue;
    T* row = x + b * sb + s * ss + h * sh;
    const int j0 = 4 * q4;
    float a[4], c[4];
    if (!br.interleaved) {
      // pairs (j, j + D/2) for j = j0 .. j0+3
      if constexpr (sizeof(T) == 2) {
        const u32x2 va = *reinterpret_cast<const u32x2*>(row + j0);
        const u32x2 vb = *reinterpret_cast<const u32x2*>(row + j0 + half);
        a[0] = __uint_as_float(va[0] << 16); a[1] = __uint_as_float(va[0] & 0xffff0000u);
        a[2] = __uint_as_float(va[1] << 16); a[3] = __uint_as_float(va[1] & 0xffff0000u);
        c[0] = __uint_as_float(vb[0] << 16); c[1] = __uint_as_float(vb[0] & 0xffff0000u);
        c[2] = __uint_as_float(vb[1] << 16); c[3] = __uint_as_float(vb[1] & 0xffff0000u);
      } else {
        const f32x4 va = *reinterpret_cast<const f32x4*>(row + j0);
        const f32x4 vb = *reinterpret_cast<const f32x4*>(row + j0 + half);
        for (int e = 0; e < 4; ++e) { a[e] = va[e]; c[e] = vb[e]; }
      }
    } else {
      // pairs (2j, 2j+1) for j = j0 .. j0+3: 8 consecutive elements
      if constexpr (sizeof(T) == 2) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(row + 2 * j0);
        for (int e = 0; e < 4; ++e) { a[e] = __uint_as_float(v[e] << 16); c[e] = __uint_as_float(v[e] & 0xffff0000u); }
      } else {
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(row + 2 * j0);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(row + 2 * j0 + 4);
        a[0] = v0[0]; c[0] = v0[1]; a[1] = v0[2]; c[1] = v0[3];
        a[2] = v1[0]; c[2] = v1[1]; a[3] = v1[2]; c[3] = v1[3];
      }
    }
    float ra[4], rb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float co = cs[tk][j0 + e], si = sn[tk][j0 + e];
      ra[e] = __builtin_fmaf(a[e], co, -c[e] * si);
      rb[e] = __builtin_fmaf(a[e], si, c[e] * co);
    }
    if (!br.interleaved) {
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<u32x2*>(row + j0) = u32x2{pack_bf16x2(ra[0], ra[1]), pack_bf16x2(ra[2], ra[3])};
        *reinterpret_cast<u32x2*>(row + j0 + half) = u32x2{pack_bf16x2(rb[0], rb[1]), pack_bf16x2(rb[2], rb[3])};
      } else {
        *reinterpret_cast<f32x4*>(row + j0) = f32x4{ra[0], ra[1], ra[2], ra[3]};
        *reinterpret_cast<f32x4*>(row + j0 + half) = f32x4{rb[0], rb[1], rb[2], rb[3]};
      }
    } else {
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<u32x4*>(row + 2 * j0) =
            u32x4{pack_bf16x2(ra[0], rb[0]), pack_bf16x2(ra[1], rb[1]), pack_bf16x2(ra[2], rb[2]), pack_bf16x2(ra[3], rb[3])};
      } else {
        *reinterpret_cast<f32x4*>(row + 2 * j0) = f32x4{ra[0], rb[0], ra[1], rb[1]};
        *reinterpret_cast<f32x4*>(row + 2 * j0 + 4) = f32x4{ra[2], rb[2], ra[3], rb[3]};
      }
    }
  }
}

}  // namespace nx

using namespace nx;

int nx::check_rope_desc(const nxattn_rope_desc& d, int64_t seq, int64_t head_dim, const char* who) {
  if (d.n_axes < 1 || d.n_axes > 3) return fail(NXATTN_ERR_INVALID, "%s: n_axes %d not in 1..3", who, d.n_axes);
  int64_t prod = 1, psum = 0;
  for (int a = 0; a < d.n_axes; ++a) {
    if (d.grid[a] < 1 || d.pairs[a] < 1) return fail(NXATTN_ERR_INVALID, "%s: grid and pairs must be >= 1", who);
    prod *= d.grid[a];
    psum += d.pairs[a];
  }
  if (prod != seq) return fail(NXATTN_ERR_INVALID, "%s: grid product %lld != seq %lld", who, (long long)prod, (long long)seq);
  if (2 * psum != head_dim) return fail(NXATTN_ERR_INVALID, "%s: 2*sum(pairs) %lld != head_dim", who, (long long)(2 * psum));
  if (!(d.theta > 1.0) || std::isinf(d.theta)) return fail(NXATTN_ERR_INVALID, "%s: theta must be finite and > 1", who);
  if (d.interleaved != 0 && d.interleaved != 1) return fail(NXATTN_ERR_INVALID, "%s: interleaved must be 0 or 1", who);
  if (d.global_freq != 0 && d.global_freq != 1) return fail(NXATTN_ERR_INVALID, "%s: global_freq must be 0 or 1", who);
  return NXATTN_OK;
}

extern "C" int nxattn_rope_apply(void* x, int64_t batch, int64_t seq, int64_t heads, int64_t head_dim,
                                 const int64_t strides[3], int dtype, const nxattn_rope_desc* rope,
                                 hipStream_t stream) {
  clear_error();
  if (dtype != NXATTN_F32 && dtype != NXATTN_BF16)
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_rope_apply: dtype %d is not F32 or BF16", dtype);
  if (batch < 0 || seq < 0 || heads < 0 || head_dim < 0) return fail(NXATTN_ERR_INVALID, "nxattn_rope_apply: negative size");
  if (batch > NXATTN_MAX_BRANCHES) return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_rope_apply: batch > %d", NXATTN_MAX_BRANCHES);
  if (head_dim % 8 != 0 || head_dim < 8 || head_dim > 2 * ROPE_MAX_HALF)
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_rope_apply: head_dim %lld must be a multiple of 8 in [8, 256]", (long long)head_dim);
  if (seq > INT32_MAX || heads > INT32_MAX) return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_rope_apply: size out of range");
  if (batch == 0 || seq == 0 || heads == 0) return NXATTN_OK;
  if (!x || !strides || !rope) return fail(NXATTN_ERR_INVALID, "nxattn_rope_apply: NULL pointer");
  RopeArgs args;
  memset(&args, 0, sizeof(args));
  for (int64_t b = 0; b < batch; ++b) {
    const nxattn_rope_desc& d = rope[b];
    const int st = check_rope_desc(d, seq, head_dim, "nxattn_rope_apply");
    if (st != NXATTN_OK) return st;
    RopeBranch& r = args.br[b];
    r.n_axes = d.n_axes; r.interleaved = d.interleaved; r.global_freq = d.global_freq;
    r.log2_theta = std::log2(d.theta);
    for (int a = 0; a < 3; ++a) {
      r.grid[a] = a < d.n_axes ? d.grid[a] : 1;
      r.pairs[a] = a < d.n_axes ? d.pairs[a] : 0;
      r.offset[a] = a < d.n_axes ? d.offset[a] : 0;
    }
  }
  const int64_t es = esize(dtype);
  if (!aligned16(x)) return fail(NXATTN_ERR_ALIGN, "nxattn_rope_apply: x must be 16-byte aligned");
  for (int i = 0; i < 3; ++i) {
    if (strides[i] < 0) return fail(NXATTN_ERR_INVALID, "nxattn_rope_apply: negative stride");
    if ((strides[i] * es) % 16 != 0) return fail(NXATTN_ERR_ALIGN, "nxattn_rope_apply: strides must be multiples of 16 bytes");
  }
  const int64_t blocks = batch * ((seq + ROPE_TOK - 1) / ROPE_TOK);
  if (blocks > INT32_MAX) return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_rope_apply: too many tokens");
  if (dtype == NXATTN_BF16)
    rope_kernel<uint16_t><<<(int)blocks, 256, 0, stream>>>(static_cast<uint16_t*>(x), seq, heads, (int32_t)head_dim,
                                                           strides[0], strides[1], strides[2], args);
  else
    rope_kernel<float><<<(int)blocks, 256, 0, stream>>>(static_cast<float*>(x), seq, heads, (int32_t)head_dim,
                                                        strides[0], strides[1], strides[2], args);
  return check_launch("nxattn_rope_apply");
}
