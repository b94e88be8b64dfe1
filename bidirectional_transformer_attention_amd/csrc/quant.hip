// FP8 (OCP E4M3) quantization of q or k for the fp8 score GEMM: one power-of-two scale
// per (branch, head). The pages name fp8 DiT variants (NeoPP page, "Run the replay
// examples") without a recipe; this one keeps every step exact except the final rounding:
// e = smallest integer with max|x| <= 448 * 2^e over the (branch, head) slice, then each
// element x * 2^-e (an exact power-of-two scaling) is rounded to the nearest E4M3 value,
// ties to the even code.
//
// Four launches. A small one clears one maximum per (branch, head) in the caller's
// workspace; the second reduces |x| over chunks of QCH tokens (lanes that share a row
// combine their maxima with cross-lane swaps, one LDS atomic per row, then one global
// atomic per (workgroup, head)); the third turns each maximum into e; the fourth writes
// the codes. HBM-bound: the input is read twice, the codes written once.
#include <cmath>

#include "nx_internal.h"

namespace nx {

namespace quantk {

constexpr int QCH = 16;          // tokens per workgroup
constexpr int THREADS = 256;
constexpr int MAX_HEADS = 4096;
constexpr int UNROLL = 4;        // items per thread whose loads are issued together

struct Args {
  const void* x;
  uint8_t* codes;
  int8_t* exps;
  uint32_t* amax;                // [batch, heads] float bits of max |x| (non-negative)
  int64_t sb, ss, sh;            // input strides (elements)
  int32_t batch, seq, heads, head_dim, nchunks;
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

// Nearest E4M3 code of y (ties to the even code), saturating at +-448, NaN -> 0x7F; the
// sign of a value that rounds to zero is kept. Integer arithmetic on the fp32 bits.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t s = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7Fu;                          // NaN
  if (a >= 0x43e00000u) return s | 0x7Eu;                     // |y| >= 448
  if (a < 0x3c800000u) {                                      // |y| < 2^-6: step 2^-9
    const float r = __builtin_rintf(__uint_as_float(a) * 512.0f);   // exact scaling, RNE
    return s | (uint32_t)r;                                   // 8 -> 0x08 = 2^-6
  }
  const uint32_t ef = (a >> 23) - 120u;                       // biased exponent 127 -> field 7
  const uint32_t mant = a & 0x7fffffu;
  const uint32_t keep = mant >> 20, rest = mant & 0xfffffu;
  uint32_t c = (ef << 3) + keep;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++c;   // carries into the exponent
  return s | (c > 0x7Eu ? 0x7Eu : c);
}

// smallest integer e with amax <= 448 * 2^e (0 for 0), clamped to the E8M0 range (>= -127)
__device__ __forceinline__ int fp8_exponent(float amax) {
  if (amax == 0.f) return 0;
  int E;
  const float m = frexpf(amax, &E);          // amax = m * 2^E, 0.5 <= m < 1; 448 = 0.875 * 2^9
  const int e = E - 9 + (m > 0.875f ? 1 : 0);
  return e < -127 ? -127 : e;
}

template <typename T>
__global__ __launch_bounds__(THREADS) void amax_kernel(Args a) {
  __shared__ uint32_t smax[MAX_HEADS];
  const int b = blockIdx.x / a.nchunks, ch = blockIdx.x % a.nchunks;
  for (int h = threadIdx.x; h < a.heads; h += THREADS) smax[h] = 0u;
  __syncthreads();
  const int t0 = ch * QCH;
  const int nt = min(QCH, a.seq - t0);
  const int gpr = a.head_dim / 8;                             // 8-element groups per row
  // a power-of-two row width puts each row's gpr groups on gpr aligned lanes of one wave
  const bool pow2 = (gpr & (gpr - 1)) == 0 && gpr <= 64;
  const int items = nt * a.heads * gpr;
  const int span = (items + THREADS * UNROLL - 1) / (THREADS * UNROLL) * (THREADS * UNROLL);  // every lane runs every round
  const T* x = static_cast<const T*>(a.x);
  for (int it0 = threadIdx.x; it0 < span; it0 += THREADS * UNROLL) {
    float v[UNROLL][8];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {              // the round's loads first, then the maxima
      const int it = it0 + u * THREADS;
      const int g = it % gpr, r = it / gpr;
      const int h = r % a.heads, t = r / a.heads;
      if (it < items) load8<T>(x + b * a.sb + (int64_t)(t0 + t) * a.ss + (int64_t)h * a.sh + 8 * g, v[u]);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int it = it0 + u * THREADS;
      const bool in = it < items;
      const int g = it % gpr, h = (it / gpr) % a.heads;
      float m = 0.f;
      if (in) {
#pragma unroll
        for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[u][e]));
      }
      if (pow2) {
        for (int d = 1; d < gpr; d <<= 1) m = __builtin_fmaxf(m, __shfl_xor(m, d));
        if (in && g == 0) atomicMax(&smax[h], __float_as_uint(m));   // non-negative: bit order = value order
      } else if (in) {
        atomicMax(&smax[h], __float_as_uint(m));
      }
    }
  }
  __syncthreads();
  for (int h = threadIdx.x; h < a.heads; h += THREADS)
    if (smax[h] != 0u) atomicMax(&a.amax[(int64_t)b * a.heads + h], smax[h]);
}

__global__ __launch_bounds__(THREADS) void clear_kernel(Args a) {
  const int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x;
  if (i < (int64_t)a.batch * a.heads) a.amax[i] = 0u;
}

// one thread per (branch, head): e from the maximum
__global__ __launch_bounds__(THREADS) void exp_kernel(Args a) {
  const int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x;   // b * heads + h
  if (i < (int64_t)a.batch * a.heads) a.exps[i] = (int8_t)fp8_exponent(__uint_as_float(a.amax[i]));
}

template <typename T>
__global__ __launch_bounds__(THREADS) void quant_kernel(Args a) {
  __shared__ int8_t sexp[MAX_HEADS];
  const int b = blockIdx.x / a.nchunks, ch = blockIdx.x % a.nchunks;
  for (int h = threadIdx.x; h < a.heads; h += THREADS) sexp[h] = a.exps[(int64_t)b * a.heads + h];
  __syncthreads();
  const int t0 = ch * QCH;
  const int nt = min(QCH, a.seq - t0);
  const int gpr = a.head_dim / 8;
  const int items = nt * a.heads * gpr;
  const T* x = static_cast<const T*>(a.x);
  for (int it0 = threadIdx.x; it0 < items; it0 += THREADS * UNROLL) {
    float v[UNROLL][8];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {              // the round's loads first, then the codes
      const int it = it0 + u * THREADS;
      const int g = it % gpr, r = it / gpr;
      const int h = r % a.heads, t = r / a.heads;
      if (it < items) load8<T>(x + b * a.sb + (int64_t)(t0 + t) * a.ss + (int64_t)h * a.sh + 8 * g, v[u]);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int it = it0 + u * THREADS;
      if (it >= items) break;
      const int g = it % gpr, r = it / gpr;
      const int h = r % a.heads, t = r / a.heads;
      const float inv = __uint_as_float((uint32_t)(127 - sexp[h]) << 23);   // 2^-e, exact
      uint32_t lo = 0u, hi = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo |= e4m3_code(v[u][e] * inv) << (8 * e);
        hi |= e4m3_code(v[u][4 + e] * inv) << (8 * e);
      }
      *reinterpret_cast<u32x2*>(a.codes + (((int64_t)b * a.seq + t0 + t) * a.heads + h) * a.head_dim + 8 * g) =
          u32x2{lo, hi};
    }
  }
}

}  // namespace quantk

}  // namespace nx

using namespace nx;

extern "C" int nxattn_quantize_fp8_workspace_size(int64_t batch, int64_t seq, int64_t heads, int64_t* bytes) {
  clear_error();
  if (!bytes || batch < 0 || seq < 0 || heads < 0)
    return fail(NXATTN_ERR_INVALID, "nxattn_quantize_fp8_workspace_size: bad argument");
  *bytes = batch * heads * 4;
  return NXATTN_OK;
}

extern "C" int nxattn_quantize_fp8(const void* x, int dtype, int64_t batch, int64_t seq, int64_t heads,
                                   int64_t head_dim, const int64_t strides[3], uint8_t* codes, int8_t* exps,
                                   void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  using namespace quantk;
  clear_error();
  if (dtype != NXATTN_F32 && dtype != NXATTN_BF16)
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_quantize_fp8: dtype %d is not F32 or BF16", dtype);
  if (batch < 0 || seq < 0 || heads < 0 || head_dim < 0 || !strides)
    return fail(NXATTN_ERR_INVALID, "nxattn_quantize_fp8: bad sizes");
  if (head_dim % 8 != 0 || head_dim > 1024)
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_quantize_fp8: head_dim must be a multiple of 8 up to 1024");
  if (heads > MAX_HEADS) return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_quantize_fp8: heads > %d", MAX_HEADS);
  if (seq > INT32_MAX / 2 || batch > INT32_MAX / 2)
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_quantize_fp8: size out of range");
  if (batch == 0 || seq == 0 || heads == 0 || head_dim == 0) return NXATTN_OK;
  if (!x || !codes || !exps || !workspace) return fail(NXATTN_ERR_INVALID, "nxattn_quantize_fp8: NULL pointer");
  const int64_t es = esize(dtype);
  for (int i = 0; i < 3; ++i) {
    if (strides[i] < 0) return fail(NXATTN_ERR_INVALID, "nxattn_quantize_fp8: negative stride");
    if ((strides[i] * es) % 16 != 0) return fail(NXATTN_ERR_ALIGN, "nxattn_quantize_fp8: strides must be multiples of 16 bytes");
  }
  if (!aligned16(x)) return fail(NXATTN_ERR_ALIGN, "nxattn_quantize_fp8: x is not 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(codes) & 7u) return fail(NXATTN_ERR_ALIGN, "nxattn_quantize_fp8: codes not 8-byte aligned");
  if (reinterpret_cast<uintptr_t>(workspace) & 3u) return fail(NXATTN_ERR_ALIGN, "nxattn_quantize_fp8: workspace not 4-byte aligned");
  const int64_t nchunks = (seq + QCH - 1) / QCH;
  const int64_t need = batch * heads * 4;
  if (workspace_bytes < need)
    return fail(NXATTN_ERR_INVALID, "nxattn_quantize_fp8: workspace_bytes %lld < %lld", (long long)workspace_bytes,
                (long long)need);
  if (batch * nchunks > INT32_MAX) return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_quantize_fp8: problem too large");
  const int64_t xb = ((batch - 1) * strides[0] + (seq - 1) * strides[1] + (heads - 1) * strides[2] + head_dim) * es;
  const int64_t cb = batch * seq * heads * head_dim;
  if (overlaps(x, xb, codes, cb) || overlaps(x, xb, exps, batch * heads) || overlaps(x, xb, workspace, need) ||
      overlaps(codes, cb, exps, batch * heads) || overlaps(codes, cb, workspace, need) ||
      overlaps(exps, batch * heads, workspace, need))
    return fail(NXATTN_ERR_INVALID, "nxattn_quantize_fp8: x, codes, exps and workspace must not overlap");
  Args a;
  a.x = x; a.codes = codes; a.exps = exps; a.amax = static_cast<uint32_t*>(workspace);
  a.sb = strides[0]; a.ss = strides[1]; a.sh = strides[2];
  a.batch = (int32_t)batch; a.seq = (int32_t)seq; a.heads = (int32_t)heads; a.head_dim = (int32_t)head_dim;
  a.nchunks = (int32_t)nchunks;
  const unsigned grid = (unsigned)(batch * nchunks);
  const unsigned egrid = (unsigned)((batch * heads + THREADS - 1) / THREADS);
  clear_kernel<<<egrid, THREADS, 0, stream>>>(a);
  if (dtype == NXATTN_BF16) {
    amax_kernel<uint16_t><<<grid, THREADS, 0, stream>>>(a);
    exp_kernel<<<egrid, THREADS, 0, stream>>>(a);
    quant_kernel<uint16_t><<<grid, THREADS, 0, stream>>>(a);
  } else {
    amax_kernel<float><<<grid, THREADS, 0, stream>>>(a);
    exp_kernel<<<egrid, THREADS, 0, stream>>>(a);
    quant_kernel<float><<<grid, THREADS, 0, stream>>>(a);
  }
  return check_launch("nxattn_quantize_fp8");
}
