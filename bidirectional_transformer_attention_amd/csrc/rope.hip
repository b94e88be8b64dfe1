// In-place rotary position embedding over 1, 2 or 3 grid axes (KLiteInfer page,
// section "架构": RoPE / 2-D RoPE / MRoPE operators; NeoPP page: explicit position
// offsets supplied with the KV cache).
//
// One workgroup handles TOK consecutive tokens of one branch. The angle of each
// (token, pair) depends only on the position and the pair, not on the head, so the
// workgroup first evaluates cos/sin once per (token, pair) into LDS, then all threads
// rotate every head of those tokens. fp32 data: the angle in fp64 and the library's fp64
// sine and cosine. bf16 data with every position below 2^24: each pair's step in
// revolutions per position is evaluated once in fp64 and split into two fp32 parts,
// and the turn pos * step is formed exactly but for the roundings of small terms
// (below 1e-7 revolutions) and taken by the hardware sine and cosine, far below the bf16
// rounding of the result. A thread owns four consecutive rotary pairs of one
// (token, head) and moves them with one or two vector loads. HBM-bound:
// 2 * B*S*H*D*esize bytes per call.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <type_traits>

#include "nx_internal.h"
#include "rope_turn.h"

namespace nx {

constexpr int ROPE_TOK = 8;          // tokens per workgroup
constexpr int ROPE_MAX_HALF = 128;   // head_dim / 2 limit
constexpr int ROPE_MAX_HEADS = 4096; // heads limit of the fused maximum (LDS)
constexpr int ROPE_UNROLL = 4;       // rows whose loads a thread issues together

struct RopeBranch {
  int32_t n_axes, interleaved, global_freq;
  int32_t grid[3], pairs[3], offset[3];
  double log2_theta;
};
struct RopeArgs {
  RopeBranch br[NXATTN_MAX_BRANCHES];
  int32_t turns;      // bf16 data, every position below 2^24: turns in fp32 revolutions
};

// codes of 4 scaled values; the scaled values of finite inputs lie in [-448, 448], where
// v_cvt_pk_fp8_f32 rounds to nearest even E4M3 (the rotated values of the fused calls are
// finite by contract, so no NaN case)
__device__ __forceinline__ uint32_t fp8x4(float y0, float y1, float y2, float y3) {
  int c = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  c = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, c, true);
  return (uint32_t)c;
}

// maximum over aligned groups of 4 (quad permutations) or 8 lanes (then the mirror of each
// 8-lane half row) through DPP moves, without the LDS crossbar
template <int CTRL>
__device__ __forceinline__ float dpp_max(float m) {
  return __builtin_fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), CTRL, 0xF, 0xF, true)));
}
__device__ __forceinline__ float max4_lanes(float m) {
  m = dpp_max<0xB1>(m);      // quad_perm [1,0,3,2]
  return dpp_max<0x4E>(m);   // quad_perm [2,3,0,1]
}
__device__ __forceinline__ float max8_lanes(float m) { return dpp_max<0x141>(max4_lanes(m)); }  // row_half_mirror

// 4 consecutive elements as loaded and stored (bf16: two words; fp32: one 16-byte vector)
template <typename T>
struct Quad;
template <>
struct Quad<uint16_t> {
  u32x2 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const u32x2*>(p); }
  __device__ __forceinline__ float get(int e) const {
    return (e & 1) ? __uint_as_float(w[e >> 1] & 0xffff0000u) : __uint_as_float(w[e >> 1] << 16);
  }
  __device__ __forceinline__ static void store(uint16_t* p, const float (&v)[4]) {
    *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
};
template <>
struct Quad<float> {
  f32x4 w;
  __device__ __forceinline__ void load(const float* p) { w = *reinterpret_cast<const f32x4*>(p); }
  __device__ __forceinline__ float get(int e) const { return w[e]; }
  __device__ __forceinline__ static void store(float* p, const float (&v)[4]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  }
};

// tensor t's entry of a per-tensor array (t < ROPE_MAX_TENSORS), without dynamic indexing
template <typename V>
__device__ __forceinline__ V pick(const V (&a)[ROPE_MAX_TENSORS], int t) {
  V r = a[0];
#pragma unroll
  for (int i = 1; i < ROPE_MAX_TENSORS; ++i)
    if (t == i) r = a[i];
  return r;
}

// One workgroup: ROPE_TOK tokens of one branch, every head of every tensor (the heads of
// the tensors laid end to end, `heads` in total). MODE Rotate: x[0] is rotated in place.
// MODE Max: x is read only; the largest magnitude of the rotated values as
// nxattn_rope_apply would store them (bf16: after rounding) is taken per (branch, head)
// into copy blockIdx % AMAX_SLOTS of tt.amax (cleared beforehand). MODE Codes: x is read
// only; each workgroup first turns the copies of its branch's maxima into the exponents e
// (the branch's first workgroup also stores them), then writes the E4M3 codes of the
// rotated, rounded values times 2^-e. MODE Blocks: x is read only; each run of 32
// elements of a row takes its exponent from its own maximum, reduced over the lanes that
// hold the run, and the codes and the run's E8M0 scale are written in the same pass.
// The work of one workgroup (block index blk) of the RoPE launch.
template <typename T, RopeMode MODE>
__device__ __forceinline__ void rope_block(const RopeTensors& tt, int32_t seq, int32_t heads, int32_t D,
                                           const RopeArgs& args, int blk) {
  constexpr bool FP8 = MODE != RopeMode::Rotate;
  constexpr bool SLICE = MODE == RopeMode::Max || MODE == RopeMode::Codes;
  __shared__ float cs[ROPE_TOK][ROPE_MAX_HALF];
  __shared__ float sn[ROPE_TOK][ROPE_MAX_HALF];
  __shared__ uint32_t hw[SLICE ? ROPE_MAX_HEADS : 1];   // Max: running maxima; Codes: bits of 2^-e
  const int half = D / 2;
  const int blocks_per_branch = (seq + ROPE_TOK - 1) / ROPE_TOK;
  const int b = blk / blocks_per_branch;
  const int s0 = (blk - b * blocks_per_branch) * ROPE_TOK;
  const RopeBranch& br = args.br[b];
  // tensor of launch head v: the number of tensor starts at or below v
  auto tensor_of = [&](int v) {
    int t = 0;
#pragma unroll
    for (int i = 1; i < ROPE_MAX_TENSORS; ++i) t += v >= tt.hoff[i] ? 1 : 0;
    return t;
  };

  if constexpr (MODE == RopeMode::Max)
    for (int v = threadIdx.x; v < heads; v += blockDim.x) hw[v] = 0u;
  if constexpr (MODE == RopeMode::Codes)
    for (int v = threadIdx.x; v < heads; v += blockDim.x) {
      const uint32_t* am = tt.amax + (int64_t)b * heads + v;
      uint32_t m = 0u;
#pragma unroll
      for (int k = 0; k < AMAX_SLOTS; ++k) m = max(m, am[k * tt.astride]);
      const int e = fp8_exponent(__uint_as_float(m));
      hw[v] = (uint32_t)(127 - e) << 23;                 // 2^-e, e in [-127, 120]
      if (s0 == 0) {
        const int t = tensor_of(v);
        const int ht = tt.hoff[t + 1] - tt.hoff[t];
        pick(tt.exps, t)[(int64_t)b * ht + (v - tt.hoff[t])] = (int8_t)e;
      }
    }
  // 1. angles: token s -> row-major grid coordinates (+ offset) -> per-pair angle. Axes
  // past n_axes have grid 1 and no pairs, so a fixed three-axis unravel and the section
  // bounds p0, p0 + p1 hold for every n_axes (branch values are uniform: no per-lane
  // indexing of the descriptor).
  const int g1 = br.grid[1], g2 = br.grid[2];
  const int p0 = br.pairs[0], p1 = br.pairs[1], p2 = br.pairs[2];
  const int f0 = br.offset[0], f1 = br.offset[1], f2 = br.offset[2];
  if (sizeof(T) == 2 && args.turns) {
    // each pair's step in revolutions per position (fp64, once), as hi + lo in fp32
    __shared__ float st_hi[ROPE_MAX_HALF], st_lo[ROPE_MAX_HALF];
    for (int j = threadIdx.x; j < half; j += blockDim.x) {
      const bool ax1 = j >= p0, ax2 = j >= p0 + p1;
      const int u = j - (ax1 ? p0 : 0) - (ax2 ? p1 : 0);
      const int pk = ax2 ? p2 : ax1 ? p1 : p0;
      const double e = br.global_freq ? -2.0 * (double)j / (double)D : -2.0 * (double)u / (2.0 * (double)pk);
      const double step = exp2_taylor(br.log2_theta * e) * 0.15915494309189535;
      const float hi = (float)step;
      st_hi[j] = hi;
      st_lo[j] = (float)(step - (double)hi);
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < ROPE_TOK * half; idx += blockDim.x) {
      const int tk = idx / half, j = idx - tk * half;
      const int s = s0 + tk;
      if (s >= seq) continue;
      const int s12 = s / g2, c2 = s - s12 * g2;
      const int c0 = s12 / g1, c1 = s12 - c0 * g1;
      const bool ax1 = j >= p0, ax2 = j >= p0 + p1;
      const float pos = (float)(ax2 ? c2 + f2 : ax1 ? c1 + f1 : c0 + f0);   // exact below 2^24
      const float hi = st_hi[j];
      const float rev = pos * hi;
      const float err = __builtin_fmaf(pos, hi, -rev);
      const float f = __builtin_amdgcn_fractf(rev) + __builtin_fmaf(pos, st_lo[j], err);
      cs[tk][j] = __builtin_amdgcn_cosf(f);
      sn[tk][j] = __builtin_amdgcn_sinf(f);
    }
  } else
  for (int idx = threadIdx.x; idx < ROPE_TOK * half; idx += blockDim.x) {
    const int tk = idx / half, j = idx - tk * half;
    const int s = s0 + tk;
    if (s >= seq) continue;
    const int s12 = s / g2, c2 = s - s12 * g2;
    const int c0 = s12 / g1, c1 = s12 - c0 * g1;
    const bool ax1 = j >= p0, ax2 = j >= p0 + p1;
    const int u = j - (ax1 ? p0 : 0) - (ax2 ? p1 : 0);
    const int pk = ax2 ? p2 : ax1 ? p1 : p0;
    const double pos = (double)(ax2 ? c2 + f2 : ax1 ? c1 + f1 : c0 + f0);
    // per-section ladder theta^(-2u / (2 pairs_k)), or one ladder theta^(-2j / D)
    const double inv_freq = br.global_freq ? exp2(br.log2_theta * (-2.0 * (double)j / (double)D))
                                           : exp2(br.log2_theta * (-2.0 * (double)u / (2.0 * (double)pk)));
    double sv, cv;
    sincos(pos * inv_freq, &sv, &cv);
    cs[tk][j] = (float)cv;
    sn[tk][j] = (float)sv;
  }
  __syncthreads();

  // 2. rotate: work item = (token, head, quad of 4 pairs j0 .. j0+3), one tensor after
  // another (the tensor's pointers and strides stay uniform). The item's elements form two
  // groups of 4 at element offsets o1 and o2: (j0, j0 + D/2) for half-split pairs, whose
  // pair e is (lo[e], hi[e]); (2 j0, 2 j0 + 4) for adjacent pairs, whose pairs are
  // (lo0, lo1), (lo2, lo3), (hi0, hi1), (hi2, hi3). A row (token, head) has `quads` items
  // on consecutive lanes; a thread keeps its quad and walks the rows r0, r0 + rstep, ...
  // with (token, head) advanced without divisions, issuing the loads of ROPE_UNROLL rows
  // before it uses them (lanes past the end load row 0 and drop it). The trip count is the
  // same for every thread, so with a power-of-two row width (<= 32 lanes, inside one
  // wave) the lanes of a row combine their maxima with swaps. In MODE Blocks a 32-element
  // run is held by 8 aligned lanes (half-split pairs: the lo groups of quads 8i .. 8i+7
  // form run i, their hi groups run i + half/32) or by 4 (adjacent pairs: quad q holds
  // elements 8q .. 8q+7 of run q/4); head_dim % 64 == 0 keeps runs inside rows and the
  // lane groups aligned, and all lanes of a group share one `in`.
  const int quads = half / 4;
  const bool pow2 = (quads & (quads - 1)) == 0;
  const int rstep = 256 / quads;
  const int q4 = (int)threadIdx.x % quads;
  const int j0 = 4 * q4;
  const int r0 = (int)threadIdx.x / quads;
  const int ntok = min(ROPE_TOK, seq - s0);
  // the pair layout is the branch's (uniform): one specialised walk per layout
  auto walk = [&](auto il_tag) {
  constexpr bool il = decltype(il_tag)::value;
  const int o1 = il ? 2 * j0 : j0, o2 = il ? 2 * j0 + 4 : j0 + half;
  for (int t = 0; t < tt.n; ++t) {
    const int h0 = tt.hoff[t], ht = tt.hoff[t + 1] - h0;
    T* const xt = static_cast<T*>(tt.x[t]) + b * tt.sb[t] + (int64_t)s0 * tt.ss[t];
    const int64_t sst = tt.ss[t], sht = tt.sh[t];
    uint8_t* const ct = FP8 ? tt.codes[t] + ((int64_t)b * seq + s0) * ht * D : nullptr;
    uint8_t* const st = MODE == RopeMode::Blocks ? tt.scales[t] + ((int64_t)b * seq + s0) * ht * (D / 32) : nullptr;
    const float mu = FP8 ? tt.mult[t] : 1.f;
    const int rows = ntok * ht;
    const int hstep = rstep % ht, tstep = rstep / ht;
    int tk = r0 / ht, h = r0 - tk * ht;
    for (int pass = 0; pass < rows; pass += ROPE_UNROLL * rstep) {   // rows pass .. pass + U * rstep - 1
      Quad<T> lo[ROPE_UNROLL], hi[ROPE_UNROLL];
      int hu[ROPE_UNROLL], tku[ROPE_UNROLL];
      bool in[ROPE_UNROLL];
#pragma unroll
      for (int u = 0; u < ROPE_UNROLL; ++u) {
        in[u] = r0 < rstep && pass + u * rstep + r0 < rows;
        hu[u] = in[u] ? h : 0;
        tku[u] = in[u] ? tk : 0;
        const T* row = xt + (int64_t)tku[u] * sst + (int64_t)hu[u] * sht;
        lo[u].load(row + o1);
        hi[u].load(row + o2);
        h += hstep;
        tk += tstep;
        if (h >= ht) { h -= ht; ++tk; }
      }
#pragma unroll
      for (int u = 0; u < ROPE_UNROLL; ++u) {
        float a[4], c[4];
        if constexpr (!il) {
#pragma unroll
          for (int e = 0; e < 4; ++e) { a[e] = lo[u].get(e); c[e] = hi[u].get(e); }
        } else {
          a[0] = lo[u].get(0); c[0] = lo[u].get(1); a[1] = lo[u].get(2); c[1] = lo[u].get(3);
          a[2] = hi[u].get(0); c[2] = hi[u].get(1); a[3] = hi[u].get(2); c[3] = hi[u].get(3);
        }
        float ra[4], rb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float co = cs[tku[u]][j0 + e], si = sn[tku[u]][j0 + e];
          ra[e] = __builtin_fmaf(a[e], co, -c[e] * si);
          rb[e] = __builtin_fmaf(a[e], si, c[e] * co);
        }
        // the two output groups, in the positions of lo and hi
        float wl[4], wh[4];
        if constexpr (!il) {
#pragma unroll
          for (int e = 0; e < 4; ++e) { wl[e] = ra[e]; wh[e] = rb[e]; }
        } else {
          wl[0] = ra[0]; wl[1] = rb[0]; wl[2] = ra[1]; wl[3] = rb[1];
          wh[0] = ra[2]; wh[1] = rb[2]; wh[2] = ra[3]; wh[3] = rb[3];
        }
        float m = 0.f;
        if constexpr (MODE == RopeMode::Rotate) {
          if (in[u]) {
            T* row = xt + (int64_t)tku[u] * sst + (int64_t)hu[u] * sht;
            Quad<T>::store(row + o1, wl);
            Quad<T>::store(row + o2, wh);
          }
        } else {
          // the values as nxattn_rope_apply stores them (bf16: rounded to nearest even),
          // times the tensor's multiplier (one fp32 multiply)
          if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t p = pack_bf16x2(wl[e], wh[e]);
              wl[e] = __uint_as_float(p << 16);
              wh[e] = __uint_as_float(p & 0xffff0000u);
            }
          }
          if (mu != 1.f) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              wl[e] *= mu;
              wh[e] *= mu;
            }
          }
          if constexpr (MODE == RopeMode::Max) {
            if (in[u]) {
#pragma unroll
              for (int e = 0; e < 4; ++e) m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fabsf(wl[e]), __builtin_fabsf(wh[e])));
            }
          } else if constexpr (MODE == RopeMode::Blocks) {
            float ml = 0.f, mh = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ml = __builtin_fmaxf(ml, __builtin_fabsf(wl[e]));
              mh = __builtin_fmaxf(mh, __builtin_fabsf(wh[e]));
            }
            if constexpr (!il) {
              ml = max8_lanes(ml);
              mh = max8_lanes(mh);
            } else {
              ml = max4_lanes(__builtin_fmaxf(ml, mh));
              mh = ml;
            }
            const int el = fp8_exponent(ml), eh = fp8_exponent(mh);
            if (in[u]) {
              const float il2 = exp2_neg(el), ih2 = exp2_neg(eh);
              const int64_t row = (int64_t)tku[u] * ht + hu[u];
              uint8_t* crow = ct + row * D;   // contiguous
              *reinterpret_cast<uint32_t*>(crow + o1) = fp8x4(wl[0] * il2, wl[1] * il2, wl[2] * il2, wl[3] * il2);
              *reinterpret_cast<uint32_t*>(crow + o2) = fp8x4(wh[0] * ih2, wh[1] * ih2, wh[2] * ih2, wh[3] * ih2);
              uint8_t* srow = st + row * (D / 32);
              if constexpr (!il) {
                if ((q4 & 7) == 0) {
                  srow[j0 / 32] = (uint8_t)(el + 127);
                  srow[(j0 + half) / 32] = (uint8_t)(eh + 127);
                }
              } else {
                if ((q4 & 3) == 0) srow[q4 / 4] = (uint8_t)(el + 127);
              }
            }
          } else if (in[u]) {
            const float inv = __uint_as_float(hw[h0 + hu[u]]);
            uint8_t* crow = ct + ((int64_t)tku[u] * ht + hu[u]) * D;   // contiguous
            *reinterpret_cast<uint32_t*>(crow + o1) = fp8x4(wl[0] * inv, wl[1] * inv, wl[2] * inv, wl[3] * inv);
            *reinterpret_cast<uint32_t*>(crow + o2) = fp8x4(wh[0] * inv, wh[1] * inv, wh[2] * inv, wh[3] * inv);
          }
        }
        if constexpr (MODE == RopeMode::Max) {
          // non-negative floats: bit order = value order
          if (pow2) {
            for (int d = 1; d < quads; d <<= 1) m = __builtin_fmaxf(m, __shfl_xor(m, d));
            if (in[u] && q4 == 0) atomicMax(&hw[h0 + hu[u]], __float_as_uint(m));
          } else if (in[u]) {
            atomicMax(&hw[h0 + hu[u]], __float_as_uint(m));
          }
        }
      }
    }
  }
  };
  if (br.interleaved)
    walk(std::true_type{});
  else
    walk(std::false_type{});
  if constexpr (MODE == RopeMode::Max) {
    __syncthreads();
    uint32_t* am = tt.amax + (blk % AMAX_SLOTS) * tt.astride + (int64_t)b * heads;
    for (int w = threadIdx.x; w < heads; w += blockDim.x)
      if (hw[w] != 0u) atomicMax(&am[w], hw[w]);
  }
}

template <typename T, RopeMode MODE>
__global__ __launch_bounds__(256) void rope_kernel(RopeTensors tt, int32_t seq, int32_t heads, int32_t D,
                                                   RopeArgs args) {
  rope_block<T, MODE>(tt, seq, heads, D, args, (int)blockIdx.x);
}

// The RoPE launch with relayout jobs appended: workgroups [0, nrope) rotate, the rest move
// the jobs' rows (job j owns workgroups nrope + blk0[j] .. nrope + blk0[j + 1] - 1).
template <typename T>
__global__ __launch_bounds__(256) void rope_relayout_kernel(RopeTensors tt, int32_t seq, int32_t heads, int32_t D,
                                                            RopeArgs args, int32_t nrope, RelayoutJobs jobs) {
  const int blk = (int)blockIdx.x;
  if (blk < nrope) {
    rope_block<T, RopeMode::Rotate>(tt, seq, heads, D, args, blk);
    return;
  }
  const int r = blk - nrope;
  int j = 0;
  while (j + 1 < jobs.n && r >= jobs.blk0[j + 1]) ++j;
  const int64_t nthreads = (int64_t)(jobs.blk0[j + 1] - jobs.blk0[j]) * 256;
  relayout_rows(jobs.src[j], jobs.dst[j], jobs.A[j], jobs.B[j], jobs.vpr[j], jobs.total[j],
                (int64_t)(r - jobs.blk0[j]) * 256 + threadIdx.x, nthreads);
}

}  // namespace nx

using namespace nx;

int nx::check_rope_desc(const nxattn_rope_desc& d, int64_t seq, int64_t head_dim, const char* who) {
  if (d.n_axes < 1 || d.n_axes > 3) return fail(NXATTN_ERR_INVALID, "%s: n_axes %d not in 1..3", who, d.n_axes);
  int64_t prod = 1, psum = 0;
  for (int a = 0; a < d.n_axes; ++a) {
    if (d.grid[a] < 1 || d.pairs[a] < 1) return fail(NXATTN_ERR_INVALID, "%s: grid and pairs must be >= 1", who);
    if (d.offset[a] < 0 || (int64_t)d.offset[a] + d.grid[a] - 1 > INT32_MAX)
      return fail(NXATTN_ERR_INVALID, "%s: offset[%d] must be >= 0 with offset + grid - 1 in int32", who, a);
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

int nx::rope_launch(const char* who, const RopeTensors& tt, int64_t batch, int64_t seq, int64_t head_dim,
                    int dtype, const nxattn_rope_desc* rope, bool fp8, hipStream_t stream, const RelayoutJobs* jobs) {
  if (dtype != NXATTN_F32 && dtype != NXATTN_BF16)
    return fail(NXATTN_ERR_UNSUPPORTED, "%s: dtype %d is not F32 or BF16", who, dtype);
  const int64_t heads = tt.hoff[tt.n];
  if (batch < 0 || seq < 0 || heads < 0 || head_dim < 0) return fail(NXATTN_ERR_INVALID, "%s: negative size", who);
  if (batch > NXATTN_MAX_BRANCHES) return fail(NXATTN_ERR_UNSUPPORTED, "%s: batch > %d", who, NXATTN_MAX_BRANCHES);
  if (head_dim % 8 != 0 || head_dim < 8 || head_dim > 2 * ROPE_MAX_HALF)
    return fail(NXATTN_ERR_UNSUPPORTED, "%s: head_dim %lld must be a multiple of 8 in [8, 256]", who, (long long)head_dim);
  if (seq > INT32_MAX) return fail(NXATTN_ERR_UNSUPPORTED, "%s: size out of range", who);
  if (fp8 && heads > ROPE_MAX_HEADS) return fail(NXATTN_ERR_UNSUPPORTED, "%s: heads > %d in total", who, ROPE_MAX_HEADS);
  const bool with_jobs = jobs && jobs->n > 0;
  if (batch == 0 || seq == 0 || heads == 0) {
    if (!with_jobs) return NXATTN_OK;
    // relayout jobs alone
    RopeArgs none;
    memset(&none, 0, sizeof(none));
    if (dtype == NXATTN_BF16)
      rope_relayout_kernel<uint16_t><<<jobs->blk0[jobs->n], 256, 0, stream>>>(tt, 1, 1, 8, none, 0, *jobs);
    else
      rope_relayout_kernel<float><<<jobs->blk0[jobs->n], 256, 0, stream>>>(tt, 1, 1, 8, none, 0, *jobs);
    return check_launch(who);
  }
  if (!rope) return fail(NXATTN_ERR_INVALID, "%s: NULL pointer", who);
  RopeArgs args;
  memset(&args, 0, sizeof(args));
  // bf16 data: angles as exact fp32 turns when every position is below 2^24 (fp32 integers)
  int64_t max_pos = 0;
  for (int64_t b = 0; b < batch; ++b) {
    const nxattn_rope_desc& d = rope[b];
    const int st = check_rope_desc(d, seq, head_dim, who);
    if (st != NXATTN_OK) return st;
    for (int a = 0; a < d.n_axes; ++a) max_pos = std::max<int64_t>(max_pos, (int64_t)d.offset[a] + d.grid[a] - 1);
    RopeBranch& r = args.br[b];
    r.n_axes = d.n_axes; r.interleaved = d.interleaved; r.global_freq = d.global_freq;
    r.log2_theta = std::log2(d.theta);
    for (int a = 0; a < 3; ++a) {
      r.grid[a] = a < d.n_axes ? d.grid[a] : 1;
      r.pairs[a] = a < d.n_axes ? d.pairs[a] : 0;
      r.offset[a] = a < d.n_axes ? d.offset[a] : 0;
    }
  }
  args.turns = dtype == NXATTN_BF16 && max_pos < (INT64_C(1) << 24);
  const int64_t es = esize(dtype);
  for (int t = 0; t < tt.n; ++t) {
    if (!tt.x[t]) return fail(NXATTN_ERR_INVALID, "%s: NULL pointer", who);
    if (!aligned16(tt.x[t])) return fail(NXATTN_ERR_ALIGN, "%s: x must be 16-byte aligned", who);
    const int64_t st[3] = {tt.sb[t], tt.ss[t], tt.sh[t]};
    for (int i = 0; i < 3; ++i) {
      if (st[i] < 0) return fail(NXATTN_ERR_INVALID, "%s: negative stride", who);
      if (!stride16(st[i], es)) return fail(NXATTN_ERR_ALIGN, "%s: strides must be multiples of 16 bytes", who);
    }
    if (span_bytes(st, batch, seq, tt.hoff[t + 1] - tt.hoff[t], head_dim, es) < 0)
      return fail(NXATTN_ERR_UNSUPPORTED, "%s: sizes or strides span more than 2^50 bytes", who);
  }
  const int64_t blocks = batch * ((seq + ROPE_TOK - 1) / ROPE_TOK);
  if (blocks + (with_jobs ? jobs->blk0[jobs->n] : 0) > INT32_MAX)
    return fail(NXATTN_ERR_UNSUPPORTED, "%s: too many tokens", who);
  const unsigned grid = (unsigned)blocks;
  if (with_jobs) {
    const unsigned g2 = grid + (unsigned)jobs->blk0[jobs->n];
    if (dtype == NXATTN_BF16)
      rope_relayout_kernel<uint16_t><<<g2, 256, 0, stream>>>(tt, (int32_t)seq, (int32_t)heads, (int32_t)head_dim, args,
                                                              (int32_t)blocks, *jobs);
    else
      rope_relayout_kernel<float><<<g2, 256, 0, stream>>>(tt, (int32_t)seq, (int32_t)heads, (int32_t)head_dim, args,
                                                           (int32_t)blocks, *jobs);
    return check_launch(who);
  }
  auto launch = [&](auto* tp, auto mode_tag) {
    using T = std::remove_pointer_t<decltype(tp)>;
    constexpr RopeMode M = decltype(mode_tag)::value;
    rope_kernel<T, M><<<grid, 256, 0, stream>>>(tt, (int32_t)seq, (int32_t)heads, (int32_t)head_dim, args);
  };
  using Rot = std::integral_constant<RopeMode, RopeMode::Rotate>;
  using Max = std::integral_constant<RopeMode, RopeMode::Max>;
  using Codes = std::integral_constant<RopeMode, RopeMode::Codes>;
  const bool bf = dtype == NXATTN_BF16;
  if (!fp8) {
    if (bf) launch((uint16_t*)nullptr, Rot{}); else launch((float*)nullptr, Rot{});
    return check_launch(who);
  }
  if (tt.blocks) {
    if (head_dim % 64 != 0)
      return fail(NXATTN_ERR_UNSUPPORTED, "%s: block scales need head_dim a multiple of 64", who);
    using Blk = std::integral_constant<RopeMode, RopeMode::Blocks>;
    if (bf) launch((uint16_t*)nullptr, Blk{}); else launch((float*)nullptr, Blk{});
    return check_launch(who);
  }
  // maxima of the rotated values, then exponents and codes
  launch_amax_clear(tt.amax, batch * heads, stream);
  if (bf) launch((uint16_t*)nullptr, Max{}); else launch((float*)nullptr, Max{});
  if (bf) launch((uint16_t*)nullptr, Codes{}); else launch((float*)nullptr, Codes{});
  return check_launch(who);
}

extern "C" int nxattn_rope_apply(void* x, int64_t batch, int64_t seq, int64_t heads, int64_t head_dim,
                                 const int64_t strides[3], int dtype, const nxattn_rope_desc* rope,
                                 hipStream_t stream) {
  clear_error();
  if (heads < 0 || heads > (1 << 28))
    return fail(heads < 0 ? NXATTN_ERR_INVALID : NXATTN_ERR_UNSUPPORTED, "nxattn_rope_apply: heads out of range");
  if (batch > 0 && seq > 0 && heads > 0 && !strides) return fail(NXATTN_ERR_INVALID, "nxattn_rope_apply: NULL pointer");
  RopeTensors tt;
  memset(&tt, 0, sizeof(tt));
  tt.n = 1;
  tt.x[0] = x;
  if (strides) { tt.sb[0] = strides[0]; tt.ss[0] = strides[1]; tt.sh[0] = strides[2]; }
  for (int i = 1; i <= ROPE_MAX_TENSORS; ++i) tt.hoff[i] = (int32_t)heads;
  return rope_launch("nxattn_rope_apply", tt, batch, seq, head_dim, dtype, rope, false, stream);
}

extern "C" int nxattn_rope_apply_relayout(void* x, int64_t batch, int64_t seq, int64_t heads, int64_t head_dim,
                                          const int64_t strides[3], int dtype, const nxattn_rope_desc* rope,
                                          const nxattn_relayout_job* jobs, int32_t n_jobs, hipStream_t stream) {
  static const char* who = "nxattn_rope_apply_relayout";
  clear_error();
  if (heads < 0 || heads > (1 << 28))
    return fail(heads < 0 ? NXATTN_ERR_INVALID : NXATTN_ERR_UNSUPPORTED, "%s: heads out of range", who);
  if (batch > 0 && seq > 0 && heads > 0 && !strides) return fail(NXATTN_ERR_INVALID, "%s: NULL pointer", who);
  if (n_jobs < 0 || n_jobs > NXATTN_MAX_BRANCHES)
    return fail(NXATTN_ERR_INVALID, "%s: n_jobs %d not in [0, %d]", who, n_jobs, NXATTN_MAX_BRANCHES);
  if (n_jobs > 0 && !jobs) return fail(NXATTN_ERR_INVALID, "%s: NULL jobs", who);
  if (dtype != NXATTN_F32 && dtype != NXATTN_BF16)
    return fail(NXATTN_ERR_UNSUPPORTED, "%s: dtype %d is not F32 or BF16", who, dtype);
  const int64_t es = esize(dtype);
  // the rotated tensor's byte extent (for the overlap checks)
  int64_t xb = 0;
  if (batch > 0 && seq > 0 && heads > 0 && head_dim > 0 && strides) {
    for (int i = 0; i < 3; ++i)
      if (strides[i] < 0) return fail(NXATTN_ERR_INVALID, "%s: negative stride", who);
    xb = span_bytes(strides, batch, seq, heads, head_dim, es);
    if (xb < 0) return fail(NXATTN_ERR_UNSUPPORTED, "%s: sizes or strides of x span more than 2^50 bytes", who);
  }
  RelayoutJobs rj;
  memset(&rj, 0, sizeof(rj));
  int64_t jbytes[NXATTN_MAX_BRANCHES] = {0};
  for (int32_t i = 0; i < n_jobs; ++i) {
    const nxattn_relayout_job& j = jobs[i];
    if (j.dir != 0 && j.dir != 1) return fail(NXATTN_ERR_INVALID, "%s: job %d: dir must be 0 or 1", who, i);
    if (j.layers < 0 || j.kv_heads < 0 || j.seq < 0 || j.head_dim < 0)
      return fail(NXATTN_ERR_INVALID, "%s: job %d: negative size", who, i);
    if (j.layers == 0 || j.kv_heads == 0 || j.seq == 0 || j.head_dim == 0) continue;
    if (!j.src || !j.dst) return fail(NXATTN_ERR_INVALID, "%s: job %d: NULL pointer", who, i);
    if (j.head_dim > (INT64_C(1) << 20) || j.kv_heads > (INT64_C(1) << 20) || j.seq > (INT64_C(1) << 31) ||
        j.layers > (INT64_C(1) << 20))
      return fail(NXATTN_ERR_UNSUPPORTED, "%s: job %d: size out of range", who, i);
    const int64_t row_bytes = j.head_dim * es;
    if (row_bytes % 16 != 0 || !aligned16(j.src) || !aligned16(j.dst))
      return fail(NXATTN_ERR_UNSUPPORTED, "%s: job %d: rows and pointers must be 16-byte multiples "
                  "(nxattn_kv_relayout takes the others)", who, i);
    jbytes[i] = dense_bytes(j.layers * 2, j.kv_heads, j.seq, j.head_dim, es);
    if (jbytes[i] < 0) return fail(NXATTN_ERR_UNSUPPORTED, "%s: job %d spans more than 2^50 bytes", who, i);
    const int64_t rows = j.layers * 2 * j.kv_heads * j.seq;
    const int n = rj.n;
    rj.src[n] = static_cast<const u32x4*>(j.src);
    rj.dst[n] = static_cast<u32x4*>(j.dst);
    rj.A[n] = j.dir == 0 ? j.kv_heads : j.seq;
    rj.B[n] = j.dir == 0 ? j.seq : j.kv_heads;
    rj.vpr[n] = row_bytes / 16;
    rj.total[n] = rj.vpr[n] * rows;
    rj.blk0[n + 1] = rj.blk0[n] + relayout_blocks(rj.total[n]);
    ++rj.n;
  }
  // every job's destination must overlap nothing it or the rotation reads or writes
  for (int32_t i = 0; i < n_jobs; ++i) {
    if (!jbytes[i]) continue;
    if (overlaps(jobs[i].dst, jbytes[i], x, xb) || overlaps(jobs[i].src, jbytes[i], x, xb))
      return fail(NXATTN_ERR_INVALID, "%s: job %d overlaps x", who, i);
    for (int32_t k = 0; k < n_jobs; ++k)
      if (jbytes[k] && overlaps(jobs[i].dst, jbytes[i], jobs[k].src, jbytes[k]))
        return fail(NXATTN_ERR_INVALID, "%s: job %d's dst overlaps job %d's src", who, i, k);
    for (int32_t k = 0; k < i; ++k)
      if (jbytes[k] && overlaps(jobs[i].dst, jbytes[i], jobs[k].dst, jbytes[k]))
        return fail(NXATTN_ERR_INVALID, "%s: the dst of jobs %d and %d overlap", who, k, i);
  }
  RopeTensors tt;
  memset(&tt, 0, sizeof(tt));
  tt.n = 1;
  tt.x[0] = x;
  if (strides) { tt.sb[0] = strides[0]; tt.ss[0] = strides[1]; tt.sh[0] = strides[2]; }
  for (int i = 1; i <= ROPE_MAX_TENSORS; ++i) tt.hoff[i] = (int32_t)heads;
  return rope_launch(who, tt, batch, seq, head_dim, dtype, rope, false, stream, &rj);
}
