// Classifier-free guidance combine: out = uncond + s * (cond - uncond)
// (LingBot-Video page, "Key Parameters": guidance_scale; NeoPP page: two KV branches).
// Elementwise and HBM-bound: 3 * n * esize bytes. Each thread moves 16-byte vectors;
// the math is fp32 fma(s, c - u, u); bf16 results are rounded to nearest even.
#include "nx_internal.h"

namespace nx {

__global__ __launch_bounds__(256) void cfg_bf16_kernel(const uint16_t* c, const uint16_t* u,
                                                       uint16_t* out, int64_t n, float s) {
  const int64_t nv = n / 8;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t i = tid; i < nv; i += step) {
    const u32x4 cv = reinterpret_cast<const u32x4*>(c)[i];
    const u32x4 uv = reinterpret_cast<const u32x4*>(u)[i];
    u32x4 r;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float c0 = __uint_as_float(cv[w] << 16), c1 = __uint_as_float(cv[w] & 0xffff0000u);
      const float u0 = __uint_as_float(uv[w] << 16), u1 = __uint_as_float(uv[w] & 0xffff0000u);
      r[w] = pack_bf16x2(__builtin_fmaf(s, c0 - u0, u0), __builtin_fmaf(s, c1 - u1, u1));
    }
    reinterpret_cast<u32x4*>(out)[i] = r;
  }
  for (int64_t i = nv * 8 + tid; i < n; i += step) {
    const float cf = bf16_bits_to_f32(c[i]), uf = bf16_bits_to_f32(u[i]);
    out[i] = static_cast<uint16_t>(pack_bf16x2(__builtin_fmaf(s, cf - uf, uf), 0.f) & 0xffffu);
  }
}

__global__ __launch_bounds__(256) void cfg_f32_kernel(const float* c, const float* u,
                                                      float* out, int64_t n, float s) {
  const int64_t nv = n / 4;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t i = tid; i < nv; i += step) {
    const f32x4 cv = reinterpret_cast<const f32x4*>(c)[i];
    const f32x4 uv = reinterpret_cast<const f32x4*>(u)[i];
    f32x4 r;
#pragma unroll
    for (int w = 0; w < 4; ++w) r[w] = __builtin_fmaf(s, cv[w] - uv[w], uv[w]);
    reinterpret_cast<f32x4*>(out)[i] = r;
  }
  for (int64_t i = nv * 4 + tid; i < n; i += step) out[i] = __builtin_fmaf(s, c[i] - u[i], u[i]);
}

}  // namespace nx

using namespace nx;

extern "C" int nxattn_cfg_combine(const void* cond, const void* uncond, void* out, int64_t n, float guidance,
                                  int dtype, hipStream_t stream) {
  clear_error();
  if (dtype != NXATTN_F32 && dtype != NXATTN_BF16)
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_cfg_combine: dtype %d is not F32 or BF16", dtype);
  if (n < 0) return fail(NXATTN_ERR_INVALID, "nxattn_cfg_combine: n < 0");
  if (!(guidance == guidance) || __builtin_isinf(guidance))
    return fail(NXATTN_ERR_INVALID, "nxattn_cfg_combine: guidance is not finite");
  if (n == 0) return NXATTN_OK;
  if (!cond || !uncond || !out) return fail(NXATTN_ERR_INVALID, "nxattn_cfg_combine: NULL pointer");
  if (!aligned16(cond) || !aligned16(uncond) || !aligned16(out))
    return fail(NXATTN_ERR_ALIGN, "nxattn_cfg_combine: pointers must be 16-byte aligned");
  const int64_t bytes = n * esize(dtype);
  if ((out != cond && overlaps(out, bytes, cond, bytes)) || (out != uncond && overlaps(out, bytes, uncond, bytes)))
    return fail(NXATTN_ERR_INVALID, "nxattn_cfg_combine: out partially overlaps an input");
  const int64_t per = dtype == NXATTN_BF16 ? 8 : 4;
  const int64_t blocks = (n / per + 255) / 256 + 1;
  const int grid = (int)(blocks < 256 * 32 ? blocks : 256 * 32);
  if (dtype == NXATTN_BF16)
    cfg_bf16_kernel<<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(cond), static_cast<const uint16_t*>(uncond),
                                               static_cast<uint16_t*>(out), n, guidance);
  else
    cfg_f32_kernel<<<grid, 256, 0, stream>>>(static_cast<const float*>(cond), static_cast<const float*>(uncond),
                                              static_cast<float*>(out), n, guidance);
  return check_launch("nxattn_cfg_combine");
}
