// FP8 (OCP E4M3) quantization of q or k for the fp8 score GEMM: one power-of-two scale
// per (branch, head), or (nxattn_quantize_fp8_blocks) one per run of 32 elements of a row. The pages name fp8 DiT variants (NeoPP page, "Run the replay
// examples") without a recipe; this one keeps every step exact except the final rounding:
// e = smallest integer with max|x| <= 448 * 2^e over the (branch, head) slice, then each
// element x * 2^-e (an exact power-of-two scaling) is rounded to the nearest E4M3 value,
// ties to the even code.
//
// Four launches. A small one clears the running maxima in the caller's workspace (32
// line-separated copies per (branch, head)); the second reduces |x| over chunks of QCH
// tokens (lanes that share a row combine their maxima with cross-lane swaps, one LDS
// atomic per row, then one global atomic per (workgroup, head) into the workgroup's
// copy); the third turns the largest copy into e; the fourth writes the codes. HBM-bound: the input is read twice, the codes written once. Where the input
// would first be rotated by RoPE, nxattn_rope_quantize_fp8 rotates it inside both reading
// passes instead (the RoPE kernel's maximum and code modes), so the rotated values are
// never stored.
#include <algorithm>
#include <cmath>
#include <cstring>

#include "nx_internal.h"

namespace nx {

namespace quantk {

constexpr int QCH = 16;          // most tokens per workgroup
constexpr int THREADS = 256;
constexpr int MAX_HEADS = 4096;
constexpr int UNROLL = 4;        // items per thread whose loads are issued together

struct Args {
  const void* x;
  uint8_t* codes;
  int8_t* exps;
  uint32_t* amax;                // AMAX_SLOTS copies of [batch, heads] float bits of max |x|
  int64_t astride;               // amax_stride(batch * heads)
  int64_t sb, ss, sh;            // input strides (elements)
  int32_t batch, seq, heads, head_dim, nchunks, tpw;   // tpw: tokens per workgroup
};

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&v)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(w[e] << 16);
    v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
}

// Rows (token, head) of the workgroup's chunk and the 8-element groups in them. With a
// power-of-two row width gpr (<= 64) a thread keeps one group g and walks rows
// rslot, rslot + 256/gpr, ... (its (token, head) advanced without divisions); otherwise
// it walks flat items.
struct RowWalk {
  int g, t, h, rstep, hstep, tstep;
  __device__ __forceinline__ void next(int heads) {
    h += hstep;
    t += tstep;
    if (h >= heads) { h -= heads; ++t; }
  }
};

template <typename T>
__device__ __forceinline__ const T* row_ptr(const Args& a, int b, int t0, int t, int h, int g) {
  return static_cast<const T*>(a.x) + b * a.sb + (int64_t)(t0 + t) * a.ss + (int64_t)h * a.sh + 8 * g;
}

template <typename T>
__global__ __launch_bounds__(THREADS) void amax_kernel(Args a) {
  __shared__ uint32_t smax[MAX_HEADS];
  const int b = blockIdx.x / a.nchunks, ch = blockIdx.x % a.nchunks;
  for (int h = threadIdx.x; h < a.heads; h += THREADS) smax[h] = 0u;
  __syncthreads();
  const int t0 = ch * a.tpw;
  const int nt = min(a.tpw, a.seq - t0);
  const int gpr = a.head_dim / 8;                             // 8-element groups per row
  if ((gpr & (gpr - 1)) == 0 && gpr <= 64) {
    // a row's gpr groups sit on gpr aligned lanes of one wave: combine with lane swaps
    const int rows = nt * a.heads, rstep = THREADS / gpr;
    const int rslot = threadIdx.x / gpr;
    RowWalk w{(int)threadIdx.x % gpr, rslot / a.heads, rslot % a.heads, rstep, rstep % a.heads, rstep / a.heads};
    const int rounds = (rows + rstep * UNROLL - 1) / (rstep * UNROLL);   // uniform over the workgroup
    int r = rslot;
    for (int k = 0; k < rounds; ++k) {
      float v[UNROLL][8];
      RowWalk w0 = w;
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {              // the round's loads first, then the maxima
        if (r + u * rstep < rows) load8<T>(row_ptr<T>(a, b, t0, w.t, w.h, w.g), v[u]);
        w.next(a.heads);
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const bool in = r + u * rstep < rows;
        float m = 0.f;
        if (in) {
#pragma unroll
          for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[u][e]));
        }
        for (int d = 1; d < gpr; d <<= 1) m = __builtin_fmaxf(m, __shfl_xor(m, d));
        if (in && w0.g == 0) atomicMax(&smax[w0.h], __float_as_uint(m));   // non-negative: bit order = value order
        w0.next(a.heads);
      }
      r += rstep * UNROLL;
    }
  } else {
    const int items = nt * a.heads * gpr;
    for (int it = threadIdx.x; it < items; it += THREADS) {
      const int g = it % gpr, rr = it / gpr;
      const int h = rr % a.heads, t = rr / a.heads;
      float v[8];
      load8<T>(row_ptr<T>(a, b, t0, t, h, g), v);
      float m = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[e]));
      atomicMax(&smax[h], __float_as_uint(m));
    }
  }
  __syncthreads();
  for (int h = threadIdx.x; h < a.heads; h += THREADS)
    if (smax[h] != 0u) atomicMax(&a.amax[(blockIdx.x % AMAX_SLOTS) * a.astride + (int64_t)b * a.heads + h], smax[h]);
}

__global__ __launch_bounds__(THREADS) void clear_kernel(uint32_t* amax, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x;
  if (i < n) amax[i] = 0u;
}

// one thread per (branch, head): e from the largest of the maximum's copies
__global__ __launch_bounds__(THREADS) void exp_kernel(const uint32_t* amax, int8_t* exps, int64_t n, int64_t stride) {
  const int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x;   // b * heads + h
  if (i >= n) return;
  uint32_t m = 0u;
#pragma unroll 8
  for (int k = 0; k < AMAX_SLOTS; ++k) m = max(m, amax[k * stride + i]);
  exps[i] = (int8_t)fp8_exponent(__uint_as_float(m));
}

// codes of 8 values scaled by 2^-e. Every scaled value of a finite input lies in
// [-448, 448], where the hardware conversion (v_cvt_pk_fp8_f32) is round-to-nearest-even
// to E4M3 (checked against the integer definition of the rounding on every bf16 value in
// that range and on exact ties); NaN becomes 0x7F.
__device__ __forceinline__ u32x2 codes8(const float (&v)[8], float inv) {
  uint32_t w[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float y0 = v[4 * k] * inv, y1 = v[4 * k + 1] * inv, y2 = v[4 * k + 2] * inv, y3 = v[4 * k + 3] * inv;
    int c = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
    c = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, c, true);
    uint32_t u = (uint32_t)c;
    if (y0 != y0) u = (u & 0xffffff00u) | 0x7Fu;
    if (y1 != y1) u = (u & 0xffff00ffu) | 0x7F00u;
    if (y2 != y2) u = (u & 0xff00ffffu) | 0x7F0000u;
    if (y3 != y3) u = (u & 0x00ffffffu) | 0x7F000000u;
    w[k] = u;
  }
  return u32x2{w[0], w[1]};
}

template <typename T>
__global__ __launch_bounds__(THREADS) void quant_kernel(Args a) {
  __shared__ int8_t sexp[MAX_HEADS];
  const int b = blockIdx.x / a.nchunks, ch = blockIdx.x % a.nchunks;
  for (int h = threadIdx.x; h < a.heads; h += THREADS) sexp[h] = a.exps[(int64_t)b * a.heads + h];
  __syncthreads();
  const int t0 = ch * a.tpw;
  const int nt = min(a.tpw, a.seq - t0);
  const int gpr = a.head_dim / 8;
  auto out = [&](int t, int h, int g) {
    return reinterpret_cast<u32x2*>(a.codes + (((int64_t)b * a.seq + t0 + t) * a.heads + h) * a.head_dim + 8 * g);
  };
  auto inv_of = [&](int h) { return __uint_as_float((uint32_t)(127 - sexp[h]) << 23); };   // 2^-e, exact
  if ((gpr & (gpr - 1)) == 0 && gpr <= 64) {
    const int rows = nt * a.heads, rstep = THREADS / gpr;
    const int rslot = threadIdx.x / gpr;
    RowWalk w{(int)threadIdx.x % gpr, rslot / a.heads, rslot % a.heads, rstep, rstep % a.heads, rstep / a.heads};
    for (int r = rslot; r < rows; r += rstep * UNROLL) {
      float v[UNROLL][8];
      RowWalk w0 = w;
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {              // the round's loads first, then the codes
        if (r + u * rstep < rows) load8<T>(row_ptr<T>(a, b, t0, w.t, w.h, w.g), v[u]);
        w.next(a.heads);
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        if (r + u * rstep < rows) *out(w0.t, w0.h, w0.g) = codes8(v[u], inv_of(w0.h));
        w0.next(a.heads);
      }
    }
  } else {
    const int items = nt * a.heads * gpr;
    for (int it = threadIdx.x; it < items; it += THREADS) {
      const int g = it % gpr, rr = it / gpr;
      const int h = rr % a.heads, t = rr / a.heads;
      float v[8];
      load8<T>(row_ptr<T>(a, b, t0, t, h, g), v);
      *out(t, h, g) = codes8(v, inv_of(h));
    }
  }
}

// Block scaling: one thread per run of 32 consecutive elements of a row (branch, token,
// head): the run's maximum gives its exponent e (the per-slice rule applied to the run),
// then its 32 codes of x * 2^-e and its E8M0 scale e + 127. Rows are read in order, the
// codes (and scales) written contiguously.
struct BlockArgs {
  const void* x;
  uint8_t* codes;
  uint8_t* scales;
  int64_t sb, ss, sh;            // input strides (elements)
  int64_t runs;                  // batch * seq * heads * runs per row
  int32_t seq, heads, rpr;       // rpr: runs per row, head_dim / 32
};

template <typename T>
__global__ __launch_bounds__(THREADS) void block_kernel(BlockArgs a) {
  const int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x;
  if (i >= a.runs) return;
  const int64_t r = i / a.rpr;
  const int k = (int)(i - r * a.rpr);
  const int64_t bs = r / a.heads, h = r - bs * a.heads;
  const int64_t b = bs / a.seq, s = bs - b * a.seq;
  const T* src = static_cast<const T*>(a.x) + b * a.sb + s * a.ss + h * a.sh + 32 * k;
  float v[4][8];
#pragma unroll
  for (int g = 0; g < 4; ++g) load8<T>(src + 8 * g, v[g]);
  float m = 0.f;
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[g][e]));
  const int e = fp8_exponent(m);
  const float inv = exp2_neg(e);
  u32x2* out = reinterpret_cast<u32x2*>(a.codes + i * 32);
#pragma unroll
  for (int g = 0; g < 4; ++g) out[g] = codes8(v[g], inv);
  a.scales[i] = (uint8_t)(e + 127);
}

}  // namespace quantk

void launch_fp8_exponents(const uint32_t* amax, int8_t* exps, int64_t n, hipStream_t stream) {
  using namespace quantk;
  exp_kernel<<<(unsigned)((n + THREADS - 1) / THREADS), THREADS, 0, stream>>>(amax, exps, n, amax_stride(n));
}

void launch_amax_clear(uint32_t* amax, int64_t n, hipStream_t stream) {
  using namespace quantk;
  const int64_t words = amax_words(n);
  clear_kernel<<<(unsigned)((words + THREADS - 1) / THREADS), THREADS, 0, stream>>>(amax, words);
}

}  // namespace nx

using namespace nx;

extern "C" int nxattn_quantize_fp8_workspace_size(int64_t batch, int64_t seq, int64_t heads, int64_t* bytes) {
  clear_error();
  if (!bytes || batch < 0 || seq < 0 || heads < 0)
    return fail(NXATTN_ERR_INVALID, "nxattn_quantize_fp8_workspace_size: bad argument");
  *bytes = amax_words(batch * heads) * 4;
  return NXATTN_OK;
}

namespace {

// Validation and launch geometry shared by both entry points. `empty`: nothing to write.
int quant_setup(const char* who, const void* x, int dtype, int64_t batch, int64_t seq, int64_t heads,
                int64_t head_dim, const int64_t strides[3], uint8_t* codes, int8_t* exps, void* workspace,
                int64_t workspace_bytes, quantk::Args& a, bool& empty) {
  using namespace quantk;
  empty = false;
  if (dtype != NXATTN_F32 && dtype != NXATTN_BF16)
    return fail(NXATTN_ERR_UNSUPPORTED, "%s: dtype %d is not F32 or BF16", who, dtype);
  if (batch < 0 || seq < 0 || heads < 0 || head_dim < 0 || !strides) return fail(NXATTN_ERR_INVALID, "%s: bad sizes", who);
  if (head_dim % 8 != 0 || head_dim > 1024)
    return fail(NXATTN_ERR_UNSUPPORTED, "%s: head_dim must be a multiple of 8 up to 1024", who);
  if (heads > MAX_HEADS) return fail(NXATTN_ERR_UNSUPPORTED, "%s: heads > %d", who, MAX_HEADS);
  if (seq > INT32_MAX / 2 || batch > INT32_MAX / 2) return fail(NXATTN_ERR_UNSUPPORTED, "%s: size out of range", who);
  if (batch == 0 || seq == 0 || heads == 0 || head_dim == 0) {
    empty = true;
    return NXATTN_OK;
  }
  if (!x || !codes || !exps || !workspace) return fail(NXATTN_ERR_INVALID, "%s: NULL pointer", who);
  const int64_t es = esize(dtype);
  for (int i = 0; i < 3; ++i) {
    if (strides[i] < 0) return fail(NXATTN_ERR_INVALID, "%s: negative stride", who);
    if (!stride16(strides[i], es)) return fail(NXATTN_ERR_ALIGN, "%s: strides must be multiples of 16 bytes", who);
  }
  if (!aligned16(x)) return fail(NXATTN_ERR_ALIGN, "%s: x is not 16-byte aligned", who);
  if (reinterpret_cast<uintptr_t>(codes) & 7u) return fail(NXATTN_ERR_ALIGN, "%s: codes not 8-byte aligned", who);
  if (reinterpret_cast<uintptr_t>(workspace) & 3u) return fail(NXATTN_ERR_ALIGN, "%s: workspace not 4-byte aligned", who);
  // tokens per workgroup: QCH, or fewer for short inputs so that ~512 workgroups run
  const int64_t tpw = std::max<int64_t>(1, std::min<int64_t>(QCH, batch * seq / 512));
  const int64_t nchunks = (seq + tpw - 1) / tpw;
  const int64_t need = amax_words(batch * heads) * 4;
  if (workspace_bytes < need)
    return fail(NXATTN_ERR_INVALID, "%s: workspace_bytes %lld < %lld", who, (long long)workspace_bytes, (long long)need);
  if (batch * nchunks > INT32_MAX) return fail(NXATTN_ERR_UNSUPPORTED, "%s: problem too large", who);
  const int64_t xb = span_bytes(strides, batch, seq, heads, head_dim, es);
  const int64_t cb = dense_bytes(batch, seq, heads, head_dim, 1);
  if (xb < 0 || cb < 0) return fail(NXATTN_ERR_UNSUPPORTED, "%s: sizes or strides span more than 2^50 bytes", who);
  if (overlaps(x, xb, codes, cb) || overlaps(x, xb, exps, batch * heads) || overlaps(x, xb, workspace, need) ||
      overlaps(codes, cb, exps, batch * heads) || overlaps(codes, cb, workspace, need) ||
      overlaps(exps, batch * heads, workspace, need))
    return fail(NXATTN_ERR_INVALID, "%s: x, codes, exps and workspace must not overlap", who);
  a.x = x; a.codes = codes; a.exps = exps; a.amax = static_cast<uint32_t*>(workspace);
  a.astride = amax_stride(batch * heads);
  a.sb = strides[0]; a.ss = strides[1]; a.sh = strides[2];
  a.batch = (int32_t)batch; a.seq = (int32_t)seq; a.heads = (int32_t)heads; a.head_dim = (int32_t)head_dim;
  a.nchunks = (int32_t)nchunks; a.tpw = (int32_t)tpw;
  return NXATTN_OK;
}

// exponents from the maxima, then the codes
void launch_exp_quant(const quantk::Args& a, int dtype, hipStream_t stream) {
  using namespace quantk;
  const unsigned grid = (unsigned)((int64_t)a.batch * a.nchunks);
  launch_fp8_exponents(a.amax, a.exps, (int64_t)a.batch * a.heads, stream);
  if (dtype == NXATTN_BF16)
    quant_kernel<uint16_t><<<grid, THREADS, 0, stream>>>(a);
  else
    quant_kernel<float><<<grid, THREADS, 0, stream>>>(a);
}

}  // namespace

extern "C" int nxattn_quantize_fp8(const void* x, int dtype, int64_t batch, int64_t seq, int64_t heads,
                                   int64_t head_dim, const int64_t strides[3], uint8_t* codes, int8_t* exps,
                                   void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  using namespace quantk;
  clear_error();
  Args a;
  bool empty;
  const int st = quant_setup("nxattn_quantize_fp8", x, dtype, batch, seq, heads, head_dim, strides, codes, exps,
                             workspace, workspace_bytes, a, empty);
  if (st != NXATTN_OK || empty) return st;
  const unsigned grid = (unsigned)(batch * a.nchunks);
  launch_amax_clear(a.amax, batch * heads, stream);
  if (dtype == NXATTN_BF16)
    amax_kernel<uint16_t><<<grid, THREADS, 0, stream>>>(a);
  else
    amax_kernel<float><<<grid, THREADS, 0, stream>>>(a);
  launch_exp_quant(a, dtype, stream);
  return check_launch("nxattn_quantize_fp8");
}

extern "C" int nxattn_quantize_fp8_blocks(const void* x, int dtype, int64_t batch, int64_t seq, int64_t heads,
                                          int64_t head_dim, const int64_t strides[3], uint8_t* codes,
                                          uint8_t* scales, hipStream_t stream) {
  using namespace quantk;
  static const char* who = "nxattn_quantize_fp8_blocks";
  clear_error();
  if (dtype != NXATTN_F32 && dtype != NXATTN_BF16)
    return fail(NXATTN_ERR_UNSUPPORTED, "%s: dtype %d is not F32 or BF16", who, dtype);
  if (batch < 0 || seq < 0 || heads < 0 || head_dim < 0 || !strides) return fail(NXATTN_ERR_INVALID, "%s: bad sizes", who);
  if (head_dim % 32 != 0 || head_dim > 1024)
    return fail(NXATTN_ERR_UNSUPPORTED, "%s: head_dim must be a multiple of 32 up to 1024", who);
  if (seq > INT32_MAX / 2 || heads > INT32_MAX / 2 || batch > INT32_MAX / 2)
    return fail(NXATTN_ERR_UNSUPPORTED, "%s: size out of range", who);
  if (batch == 0 || seq == 0 || heads == 0 || head_dim == 0) return NXATTN_OK;
  if (!x || !codes || !scales) return fail(NXATTN_ERR_INVALID, "%s: NULL pointer", who);
  const int64_t es = esize(dtype);
  for (int i = 0; i < 3; ++i) {
    if (strides[i] < 0) return fail(NXATTN_ERR_INVALID, "%s: negative stride", who);
    if (!stride16(strides[i], es)) return fail(NXATTN_ERR_ALIGN, "%s: strides must be multiples of 16 bytes", who);
  }
  if (!aligned16(x)) return fail(NXATTN_ERR_ALIGN, "%s: x is not 16-byte aligned", who);
  if (reinterpret_cast<uintptr_t>(codes) & 7u) return fail(NXATTN_ERR_ALIGN, "%s: codes not 8-byte aligned", who);
  const int64_t runs = dense_bytes(batch, seq, heads, head_dim / 32, 1);
  const int64_t xb = span_bytes(strides, batch, seq, heads, head_dim, es);
  const int64_t cb = dense_bytes(batch, seq, heads, head_dim, 1);
  if (runs < 0 || xb < 0 || cb < 0)
    return fail(NXATTN_ERR_UNSUPPORTED, "%s: sizes or strides span more than 2^50 bytes", who);
  const int64_t grid = (runs + THREADS - 1) / THREADS;
  if (grid > INT32_MAX) return fail(NXATTN_ERR_UNSUPPORTED, "%s: problem too large", who);
  if (overlaps(x, xb, codes, cb) || overlaps(x, xb, scales, runs) || overlaps(codes, cb, scales, runs))
    return fail(NXATTN_ERR_INVALID, "%s: x, codes and scales must not overlap", who);
  BlockArgs a;
  a.x = x; a.codes = codes; a.scales = scales;
  a.sb = strides[0]; a.ss = strides[1]; a.sh = strides[2];
  a.runs = runs;
  a.seq = (int32_t)seq; a.heads = (int32_t)heads; a.rpr = (int32_t)(head_dim / 32);
  if (dtype == NXATTN_BF16)
    block_kernel<uint16_t><<<(unsigned)grid, THREADS, 0, stream>>>(a);
  else
    block_kernel<float><<<(unsigned)grid, THREADS, 0, stream>>>(a);
  return check_launch(who);
}

namespace nx {

// Validation and launches of nxattn_rope_quantize_fp8 with the running maxima in
// `workspace` (the caller's memory, or the static scratch of the no-allocation variant).
int rope_quantize(const char* who, const nxattn_fp8_tensor* tensors, int32_t n_tensors, int dtype, int64_t batch,
                  int64_t seq, int64_t head_dim, const nxattn_rope_desc* rope, void* workspace,
                  int64_t workspace_bytes, hipStream_t stream) {
  if (!tensors || n_tensors < 1 || n_tensors > NXATTN_MAX_FP8_TENSORS)
    return fail(NXATTN_ERR_INVALID, "%s: need 1 to %d tensors", who, NXATTN_MAX_FP8_TENSORS);
  if (dtype != NXATTN_F32 && dtype != NXATTN_BF16)
    return fail(NXATTN_ERR_UNSUPPORTED, "%s: dtype %d is not F32 or BF16", who, dtype);
  if (batch < 0 || seq < 0 || head_dim < 0) return fail(NXATTN_ERR_INVALID, "%s: negative size", who);
  if (batch > NXATTN_MAX_BRANCHES) return fail(NXATTN_ERR_UNSUPPORTED, "%s: batch > %d", who, NXATTN_MAX_BRANCHES);
  if (seq > INT32_MAX) return fail(NXATTN_ERR_UNSUPPORTED, "%s: size out of range", who);
  int64_t total = 0;
  for (int t = 0; t < n_tensors; ++t) {
    if (tensors[t].heads < 0) return fail(NXATTN_ERR_INVALID, "%s: negative heads", who);
    total += tensors[t].heads;
    if (total > quantk::MAX_HEADS) return fail(NXATTN_ERR_UNSUPPORTED, "%s: more than %d heads in total", who, quantk::MAX_HEADS);
  }
  // block scales (every tensor with heads has scales, none exps) or one exponent per
  // slice (every one exps, none scales)
  bool blocks = false;
  for (int t = 0; t < n_tensors; ++t)
    if (tensors[t].heads > 0) { blocks = tensors[t].scales != nullptr; break; }
  for (int t = 0; t < n_tensors; ++t)
    if (tensors[t].heads > 0 && ((tensors[t].scales != nullptr) != blocks || (tensors[t].exps != nullptr) == blocks))
      return fail(NXATTN_ERR_INVALID, "%s: every tensor needs scales (block scaling) or every tensor exps, not both",
                  who);
  if (blocks && head_dim % 64 != 0)
    return fail(NXATTN_ERR_UNSUPPORTED, "%s: block scales need head_dim a multiple of 64", who);
  if (batch == 0 || seq == 0 || total == 0) return NXATTN_OK;
  // the running maxima of the per-slice exponents; block scaling needs none
  const int64_t need = blocks ? 0 : amax_words(batch * total) * 4;
  if (!blocks) {
    if (!workspace) return fail(NXATTN_ERR_INVALID, "%s: NULL workspace", who);
    if (reinterpret_cast<uintptr_t>(workspace) & 3u) return fail(NXATTN_ERR_ALIGN, "%s: workspace not 4-byte aligned", who);
    if (workspace_bytes < need)
      return fail(NXATTN_ERR_INVALID, "%s: workspace_bytes %lld < %lld", who, (long long)workspace_bytes, (long long)need);
  }
  // the tensors with heads, heads laid end to end
  const int64_t es = esize(dtype);
  RopeTensors tt;
  memset(&tt, 0, sizeof(tt));
  struct Span { const void* p; int64_t n; };
  Span xs[NXATTN_MAX_FP8_TENSORS], outs[2 * NXATTN_MAX_FP8_TENSORS + 1];
  int nout = 0;
  if (!blocks) outs[nout++] = {workspace, need};
  for (int t = 0; t < n_tensors; ++t) {
    const nxattn_fp8_tensor& z = tensors[t];
    if (z.heads == 0) continue;
    if (!z.x || !z.codes) return fail(NXATTN_ERR_INVALID, "%s: NULL pointer in tensor %d", who, t);
    if (reinterpret_cast<uintptr_t>(z.codes) & 7u) return fail(NXATTN_ERR_ALIGN, "%s: codes not 8-byte aligned", who);
    for (int i = 0; i < 3; ++i)
      if (z.strides[i] < 0) return fail(NXATTN_ERR_INVALID, "%s: negative stride", who);
    const int64_t zxb = span_bytes(z.strides, batch, seq, z.heads, head_dim, es);
    const int64_t zcb = dense_bytes(batch, seq, z.heads, head_dim, 1);
    if (zxb < 0 || zcb < 0)
      return fail(NXATTN_ERR_UNSUPPORTED, "%s: tensor %d's sizes or strides span more than 2^50 bytes", who, t);
    if (!(z.mult >= 0.f) || std::isinf(z.mult))
      return fail(NXATTN_ERR_INVALID, "%s: mult of tensor %d must be finite and >= 0", who, t);
    if (z.fold_softmax != 0 && z.fold_softmax != 1)
      return fail(NXATTN_ERR_INVALID, "%s: fold_softmax of tensor %d must be 0 or 1", who, t);
    if (z.fold_softmax && head_dim <= 0) return fail(NXATTN_ERR_INVALID, "%s: fold_softmax needs head_dim > 0", who);
    const int k = tt.n++;
    if (z.fold_softmax) {
      // c = softmax scale * log2(e) in fp32, the scale given in mult or 1/sqrt(head_dim)
      // formed as nxattn_fwd and nxattn_fwd_fp8 form their default
      const float sc = z.mult > 0.f ? z.mult : 1.0f / std::sqrt((float)head_dim);
      tt.mult[k] = sc * 1.4426950408889634f;
    } else {
      tt.mult[k] = z.mult == 0.f ? 1.f : z.mult;
    }
    tt.x[k] = const_cast<void*>(z.x);
    tt.sb[k] = z.strides[0]; tt.ss[k] = z.strides[1]; tt.sh[k] = z.strides[2];
    tt.codes[k] = z.codes;
    tt.exps[k] = z.exps;
    tt.scales[k] = z.scales;
    tt.hoff[k + 1] = tt.hoff[k] + (int32_t)z.heads;
    xs[k] = {z.x, zxb};
    outs[nout++] = {z.codes, zcb};
    if (blocks)
      outs[nout++] = {z.scales, batch * seq * z.heads * (head_dim / 32)};
    else
      outs[nout++] = {z.exps, batch * z.heads};
  }
  tt.blocks = blocks ? 1 : 0;
  for (int i = tt.n + 1; i <= ROPE_MAX_TENSORS; ++i) tt.hoff[i] = tt.hoff[tt.n];
  // outputs must not overlap one another, an input or the workspace; inputs may overlap
  // one another but not the workspace
  for (int i = 0; i < nout; ++i) {
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
        return fail(NXATTN_ERR_INVALID, "%s: outputs and workspace must not overlap", who);
    for (int k = 0; k < tt.n; ++k)
      if (overlaps(outs[i].p, outs[i].n, xs[k].p, xs[k].n))
        return fail(NXATTN_ERR_INVALID, "%s: an output or the workspace overlaps an input", who);
  }
  tt.amax = blocks ? nullptr : static_cast<uint32_t*>(workspace);
  tt.astride = amax_stride(batch * total);
  // validates the RoPE arguments and the inputs (head_dim 8..256 among them) before the
  // first launch
  return rope_launch(who, tt, batch, seq, head_dim, dtype, rope, true, stream);
}

}  // namespace nx

extern "C" int nxattn_rope_quantize_fp8(const nxattn_fp8_tensor* tensors, int32_t n_tensors, int dtype,
                                        int64_t batch, int64_t seq, int64_t head_dim, const nxattn_rope_desc* rope,
                                        void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  clear_error();
  return rope_quantize("nxattn_rope_quantize_fp8", tensors, n_tensors, dtype, batch, seq, head_dim, rope, workspace,
                       workspace_bytes, stream);
}

