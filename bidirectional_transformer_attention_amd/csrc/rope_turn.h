// RoPE angles for the attention kernels that rotate q as they load it (same convention as
// the RoPE kernel: pair j of axis k with local index u turns by pos_k * theta^(-u /
// pairs_k), or with the global ladder by pos_k * theta^(-j / 64); KLiteInfer page, "架构":
// RoPE / 2-D RoPE / MRoPE operators; NeoPP page: explicit position offsets). head_dim 128:
// 64 pairs, one per lane of a wave.
#pragma once

#include "nx_internal.h"

namespace nx {

// 2^x in fp64 for x <= 0 (the RoPE frequency ladder): x = k + r with k = floor(x), 2^r =
// e^(r ln 2) by its Taylor series to degree 13 (remainder below 7e-14 relative for
// r ln 2 < 0.7), scaled by 2^k. Written out so that the kernels call no library routine
// (a call there made the register allocator spill).
__device__ __forceinline__ double exp2_taylor(double x) {
  const double k = __builtin_floor(x);
  const double y = (x - k) * 0.6931471805599453094;
  double t = 1.0;
#pragma unroll
  for (int i = 13; i >= 1; --i) t = __builtin_fma(t, y * (1.0 / i), 1.0);
  return __builtin_ldexp(t, (int)k);
}

// The turns of one token. Lane l evaluates pair l's step in revolutions per position,
// theta^(..) / 2pi, in fp64, rounds it to fp32 with the pair's axis in the two low
// mantissa bits (s) and keeps the remainder lo = step - s in fp32; every lane fetches
// the s and lo of the pairs it rotates with ds_bpermute. The turn pos * step is then
// pos * s, formed exactly as rev + err (err by an fma), plus pos * lo: fract(rev) + (err +
// pos * lo) revolutions, exact but for the roundings of the small terms and of the sum
// (below 1e-7 revolutions for every position under 2^24). The hardware sin/cos take the
// turn in revolutions.
struct RopeTurns {
  uint32_t s, lo;         // this lane's pair: step (axis in the low 2 bits) and remainder
  float p0, p1, p2;       // the token's position on each axis

  __device__ __forceinline__ RopeTurns(const RopeQ& r, int tok, int lane) {
    int c0 = tok, c1 = 0, c2 = 0;
    if (r.n_axes == 2) {
      c0 = tok / r.grid[1];
      c1 = tok - c0 * r.grid[1];
    } else if (r.n_axes == 3) {
      const int hw = r.grid[1] * r.grid[2];
      c0 = tok / hw;
      const int rem = tok - c0 * hw;
      c1 = rem / r.grid[2];
      c2 = rem - c1 * r.grid[2];
    }
    p0 = (float)(c0 + r.offset[0]);
    p1 = (float)(c1 + r.offset[1]);
    p2 = (float)(c2 + r.offset[2]);
    // pair j = lane: its axis (as 0/1 weights, a blend keeps the choice in registers) and
    // its index in the ladder
    const int j = lane, n0 = r.pairs[0], n1 = r.pairs[1], n2 = r.pairs[2];
    const int i0 = j < n0, i1 = (1 - i0) & (j < n0 + n1), i2 = 1 - i0 - i1;
    const int u = r.global_freq ? j : j - i1 * n0 - i2 * (n0 + n1);
    const int n = r.global_freq ? n0 + n1 + n2 : i0 * n0 + i1 * n1 + i2 * n2;
    const double step = exp2_taylor(-(double)u * r.log2_theta / (double)(n > 0 ? n : 1)) * 0.15915494309189535;
    s = (__float_as_uint((float)step) & ~3u) | (uint32_t)(i1 + 2 * i2);
    lo = __float_as_uint((float)(step - (double)__uint_as_float(s)));
  }

  // sin and cos of pair j's turn
  __device__ __forceinline__ void turn(int j, float& sn, float& cs) const {
    const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * j, (int)s);
    const float l = __uint_as_float((uint32_t)__builtin_amdgcn_ds_bpermute(4 * j, (int)lo));
    const uint32_t ax = v & 3u;
    const float st = __uint_as_float(v);
    const float w1 = (float)(ax == 1u), w2 = (float)(ax == 2u), w0 = 1.f - w1 - w2;
    const float pos = w0 * p0 + w1 * p1 + w2 * p2;
    const float rev = pos * st;
    const float err = __builtin_fmaf(pos, st, -rev);
    const float f = __builtin_amdgcn_fractf(rev) + __builtin_fmaf(pos, l, err);
    sn = __builtin_amdgcn_sinf(f);
    cs = __builtin_amdgcn_cosf(f);
  }
};

}  // namespace nx
