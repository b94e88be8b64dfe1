// Fused non-causal attention, fp32 in/out, true fp32 MFMA (v_mfma_f32_32x32x2f32),
// head_dim 64 or 72 (the vision-encoder shape: KLiteInfer page, "架构": bidirectional
// attention of the ViT as two strided-batched fp32 GEMMs plus a softmax, TF32 off).
//
// Work split: a workgroup (4 waves) serves one (branch, kv head) and 4 query blocks of
// 32 rows; query blocks enumerate (q head in the group, 32-token chunk), so every wave
// of a workgroup reads the same K/V tiles. Keys are walked in tiles of 64 over the
// virtual sequence [prefix ++ own] (the concatenation is only index arithmetic), or
// over one key range of it when the keys are split (each range then writes a normalised
// fp32 partial and its log-sum-exp for the merge kernel).
// Each wave keeps S^T = K Q^T in the MFMA accumulator layout (lane = query, registers
// = keys), so the running max and sum are per lane; the P^T accumulator registers feed
// the P V MFMA directly as its B operand (no shuffle). K and V tiles are staged through
// LDS, double-buffered, with the next tile's global loads in flight during compute.
// MFMA-bound: 4*Sq*Skv*Hq*D flops.
#include "nx_internal.h"

namespace nx {

namespace f32k {

constexpr int WAVES = 4;
constexpr int BN = KEY_TILE;    // keys per tile (64)
constexpr int VSTR = 72;        // V row stride in LDS (floats)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float RESCALE_T = 8.0f;   // running max moves only when it grows by > 2^8

struct Args {
  const float* q; const float* k; const float* v; float* o;
  int64_t qs0, qs1, qs2, ks0, ks1, ks2, os0, os1, os2;
  const float* prefix[NXATTN_MAX_BRANCHES];
  int32_t plen[NXATTN_MAX_BRANCHES];
  int32_t batch, seq, heads_q, heads_kv, group, nchunks, nqb, wg_per_group, total_wg;
  float c;  // scale * log2(e)
  float* lse;
  float* part_o;
  float* part_lse;
  int32_t nsplit, per, prefix_only;
};

__device__ __forceinline__ int remap_xcd(int i, int n) {
  // Workgroups are dispatched round-robin over 8 XCDs; give each XCD a contiguous run of
  // logical work so workgroups that share K/V tiles share one L2.
  const int xcd = i & 7, local = i >> 3;
  const int per = n >> 3, rem = n & 7;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(Args a) {
  constexpr int KSTR = D + 1;                 // odd stride: column reads are conflict-free
  constexpr int NDB = (D + 31) / 32;          // 32-wide output blocks (72 -> 3, last one partial)
  constexpr int CH = D / 4;                   // 16-byte chunks per row
  constexpr int LD = (BN * CH + 255) / 256;   // chunks per thread per tensor
  __shared__ float Ks[2][BN * KSTR];
  __shared__ float Vs[2][BN * VSTR];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int w = remap_xcd(blockIdx.x, a.total_wg);
  // (branch, kv head, key range) groups of wg_per_group workgroups
  const int grp = w / a.wg_per_group;
  const int split = grp % a.nsplit, bg = grp / a.nsplit;
  const int b = bg / a.heads_kv, g = bg % a.heads_kv;
  const int rem = w % a.wg_per_group;
  const int qb = rem * WAVES + wave;
  const bool active = qb < a.nqb;
  const int hq = g * a.group + (active ? qb / a.nchunks : 0);
  const int tok = (active ? qb % a.nchunks : 0) * 32 + n;
  const int tokc = tok < a.seq ? tok : a.seq - 1;
  // this work item's keys: tiles [t0, t0 + T) of the virtual sequence, keys below kend
  const int P = a.plen[b];
  const int Skv = P + (a.prefix_only ? 0 : a.seq);
  const int t0 = split * a.per;
  const int Tall = (Skv + BN - 1) / BN;
  const int T = min(a.per, Tall - t0);
  if (T <= 0) return;   // empty key range (uniform over the workgroup, before any barrier)
  // a branch whose keys fit in one range writes its result directly, without a merge
  const bool partial = a.nsplit > 1 && Tall > a.per;
  const int kend = min((t0 + T) * BN, Skv);

  // Q^T operand: k-step s holds Q[tok][hq][2s + hh]
  float qv[D / 2];
  {
    const float* qrow = a.q + b * a.qs0 + (int64_t)tokc * a.qs1 + (int64_t)hq * a.qs2;
#pragma unroll
    for (int s = 0; s < D / 2; ++s) qv[s] = qrow[2 * s + hh];
  }

  // tile loader: thread -> (row, 16-byte chunk) items of K and V
  auto key_rows = [&](int j, const float*& kr, const float*& vr) {
    j = j < kend ? j : kend - 1;
    if (j < P) {
      const float* base = a.prefix[b] + ((int64_t)j * a.heads_kv + g) * D;
      kr = base;
      vr = base + (int64_t)P * a.heads_kv * D;
    } else {
      const int64_t off = b * a.ks0 + (int64_t)(j - P) * a.ks1 + (int64_t)g * a.ks2;
      kr = a.k + off;
      vr = a.v + off;
    }
  };
  f32x4 stk[LD], stv[LD];
  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const int it = threadIdx.x + i * 256;
      if (it < BN * CH) {
        const int r = it / CH, c = it % CH;
        const float *kr, *vr;
        key_rows(t * BN + r, kr, vr);
        stk[i] = *reinterpret_cast<const f32x4*>(kr + 4 * c);
        stv[i] = *reinterpret_cast<const f32x4*>(vr + 4 * c);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const int it = threadIdx.x + i * 256;
      if (it < BN * CH) {
        const int r = it / CH, c = it % CH;
        float* kd = &Ks[buf][r * KSTR + 4 * c];
        kd[0] = stk[i][0]; kd[1] = stk[i][1]; kd[2] = stk[i][2]; kd[3] = stk[i][3];
        *reinterpret_cast<f32x4*>(&Vs[buf][r * VSTR + 4 * c]) = stv[i];
      }
    }
  };

  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
  float m = -__builtin_inff(), l = 0.f;

  gload(t0);
  lstore(0);
  __syncthreads();

  for (int t = t0; t < t0 + T; ++t) {
    const int buf = (t - t0) & 1;
    if (t + 1 < t0 + T) gload(t + 1);
    const float* kb_ = Ks[buf];
    const float* vb_ = Vs[buf];

    // S^T = K Q^T for two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const float* krow = kb_ + (kb * 32 + n) * KSTR + hh;
#pragma unroll
      for (int st = 0; st < D / 2; ++st)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * st], qv[st], s[kb], 0, 0, 0);
    }
    // mask keys past the end (only the last tile can have them)
    const int valid = kend - t * BN;
    if (valid < BN) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (key >= valid) s[kb][i] = -__builtin_inff();
        }
    }
    // online softmax (base 2, scale folded into one fma per score)
    float tmax = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = __builtin_fmaxf(tmax, s[kb][i]);
    {
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(tmax), __float_as_int(tmax), false, false);
      tmax = __builtin_fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1]));
    }
    const float cand = tmax * a.c;
    const bool grow = cand > m + RESCALE_T;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float mnew = grow ? cand : m;
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc_o[db][i] *= alpha;
      m = mnew;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], a.c, -m));
        s[kb][i] = p;
        l += p;
      }
    // O^T += V^T P^T: accumulator register i of key block kb is the B operand of one step
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = db * 32 + n < D ? db * 32 + n : D - 1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vb_[key * VSTR + d], s[kb][i], acc_o[db], 0, 0, 0);
        }
    }
    if (t + 1 < t0 + T) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: combine the two lane halves' partial sums, normalise, store
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(l), __float_as_int(l), false, false);
    l = __int_as_float(sw[0]) + __int_as_float(sw[1]);
  }
  if (!active || tok >= a.seq) return;
  const float inv = 1.0f / l;
  // log-sum-exp: sum_j exp2(c s_j - m) = l, so lse = ln2 * (m + log2 l)  (l >= 1)
  const float lse = LN2 * (m + __builtin_amdgcn_logf(l));
  float* orow;
  if (partial) {
    orow = a.part_o + ((((int64_t)split * a.batch + b) * a.seq + tok) * a.heads_q + hq) * D;
    if (hh == 0) a.part_lse[(((int64_t)split * a.batch + b) * a.heads_q + hq) * a.seq + tok] = lse;
  } else {
    orow = a.o + b * a.os0 + (int64_t)tok * a.os1 + (int64_t)hq * a.os2;
    if (a.lse && hh == 0) a.lse[((int64_t)b * a.heads_q + hq) * a.seq + tok] = lse;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = db * 32 + 8 * i4 + 4 * hh;
      if (d < D)
        *reinterpret_cast<f32x4*>(orow + d) = f32x4{acc_o[db][4 * i4] * inv, acc_o[db][4 * i4 + 1] * inv,
                                                    acc_o[db][4 * i4 + 2] * inv, acc_o[db][4 * i4 + 3] * inv};
    }
}

}  // namespace f32k

FwdShape fwd_shape_f32(const FwdProblem& p) {
  using namespace f32k;
  // resident workgroups per CU of the variant that will run (queried on each call: the
  // library keeps no state)
  int n = 0;
  const hipError_t e = p.head_dim == 64 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_f32_kernel<64>, 256, 0)
                                        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_f32_kernel<72>, 256, 0);
  const int64_t nqb = (int64_t)(p.heads_q / p.heads_kv) * ((p.seq_q + 31) / 32);
  return FwdShape{(nqb + WAVES - 1) / WAVES * p.heads_kv, (e != hipSuccess || n < 1) ? 1 : n};
}

int launch_fwd_f32(const FwdProblem& p, hipStream_t stream) {
  using namespace f32k;
  Args a;
  a.q = static_cast<const float*>(p.q); a.k = static_cast<const float*>(p.k);
  a.v = static_cast<const float*>(p.v); a.o = static_cast<float*>(p.o);
  a.qs0 = p.qs[0]; a.qs1 = p.qs[1]; a.qs2 = p.qs[2];
  a.ks0 = p.ks[0]; a.ks1 = p.ks[1]; a.ks2 = p.ks[2];
  a.os0 = p.os[0]; a.os1 = p.os[1]; a.os2 = p.os[2];
  for (int b = 0; b < NXATTN_MAX_BRANCHES; ++b) { a.prefix[b] = static_cast<const float*>(p.prefix[b]); a.plen[b] = p.plen[b]; }
  a.batch = p.batch; a.seq = p.seq_q; a.heads_q = p.heads_q; a.heads_kv = p.heads_kv;
  a.group = p.heads_q / p.heads_kv;
  a.nchunks = (p.seq_q + 31) / 32;
  const int64_t nqb = (int64_t)a.group * a.nchunks;
  const int64_t wpg = (nqb + WAVES - 1) / WAVES;
  const int64_t total = wpg * p.heads_kv * p.batch * p.nsplit;
  if (total > INT32_MAX / 2) return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd: problem too large");
  a.nqb = (int)nqb; a.wg_per_group = (int)wpg; a.total_wg = (int)total;
  a.c = p.scale * LOG2E;
  a.lse = p.lse; a.part_o = p.part_o; a.part_lse = p.part_lse;
  a.nsplit = p.nsplit; a.per = p.per; a.prefix_only = p.prefix_only;
  if (p.prefix_only) {  // own keys are never read: keep valid (unused) base pointers
    a.k = a.q; a.v = a.q;
    a.ks0 = a.ks1 = a.ks2 = 0;
  }
  if (p.head_dim == 64)
    fwd_f32_kernel<64><<<a.total_wg, 256, 0, stream>>>(a);
  else
    fwd_f32_kernel<72><<<a.total_wg, 256, 0, stream>>>(a);
  return check_launch("nxattn_fwd(f32)");
}

}  // namespace nx
