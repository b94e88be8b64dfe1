// Fused non-causal attention, fp32 in/out, true fp32 MFMA (v_mfma_f32_16x16x4f32),
// head_dim 64 or 72 (the vision-encoder shape: KLiteInfer page, "架构": bidirectional
// attention of the ViT as two strided-batched fp32 GEMMs plus a softmax, TF32 off).
//
// Work split: a workgroup (4 waves) serves one (branch, kv head) and 4 query blocks of
// 32 rows; query blocks enumerate (q head in the group, 32-token chunk), so every wave
// of a workgroup reads the same K/V tiles. Keys are walked in tiles of 64 over the
// virtual sequence [prefix ++ own] (the concatenation is only index arithmetic), or
// over one key range of it when the keys are split (each range then writes a normalised
// fp32 partial and its log-sum-exp for the merge kernel).
//
// 16x16 tiles. A wave's 32 queries are two sub-blocks of 16 (lane l: queries l % 16 and
// 16 + l % 16). S^T = K Q^T is kept as 4 x 2 blocks of 16 keys x 16 queries (lane l:
// keys 4(l / 16) .. + 3 of a block), so each K fragment read from LDS feeds both
// sub-blocks, and one 16-byte read feeds four k-steps. For P V, register j of key block kb is directly the B operand (P^T) of one
// 16x16x4 step over keys 16kb + 4k + j (k = 0..3), with the V^T operand read in the same
// key order: no shuffle of P. The output is O^T in blocks of 16 head dims, so head_dim
// 72 takes 5 blocks (80 columns, 10 % padding) rather than three of 32 (96 columns).
// LDS rows are unpadded with 16-byte chunks permuted so that the fragment reads are free
// of bank conflicts (see kslot / vcol). K and V tiles are double-buffered and loaded
// straight into LDS, the next tile's loads in flight during compute; two workgroups
// share a CU, so one wave's softmax overlaps another's MFMAs.
// MFMA-bound: 4*Sq*Skv*Hq*D flops.
#include "nx_internal.h"

namespace nx {

namespace f32k {

constexpr int WAVES = 4;
constexpr int BN = KEY_TILE;    // keys per tile (64)
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

// LDS placement (banks: 32 of 4 bytes; a 32-bit read is served per half-wave, a 128-bit
// read per group of 8 lanes). Tiles arrive by 16-byte chunks, so only whole chunks move.
// K row r, chunk c sits at chunk kslot(r, c) of the row. A score step group reads chunk
// 4G + l / 16 of rows 16kb + l % 16 with one ds_read_b128: each 8-lane group reads one
// chunk column of 8 consecutive rows, which must start on 8 different bank quads (D = 64:
// chunk XOR r & 7; D = 72, rows 18 chunks = 2 quads apart: rows with bit 2 set move by
// one chunk).
template <int D>
__device__ __forceinline__ int kslot(int r, int c) {
  if constexpr (D == 64) return c ^ (r & 7);
  else { const int x = c + ((r >> 2) & 1); return x < D / 4 ? x : x - D / 4; }
}
// V row r (a key), column d at float vcol(r, d) of the row. A P V step reads keys
// 16kb + 4g + j (g = l / 16) at columns 16db + l % 16; a half-wave holds g = 0, 1 (or 2,
// 3), whose rows differ in bit 2 and must fall on complementary 16-bank halves (D = 64: a
// row stride of 64 floats repeats the banks, so the 16-column group is XORed with bit 2
// of the key; D = 72: rows with bit 2 set are rotated by 16 columns). Columns past D (the
// padded output block) wrap inside the row.
template <int D>
__device__ __forceinline__ int vcol(int r, int d) {
  if constexpr (D == 64) return d ^ (16 * ((r >> 2) & 1));
  else { const int x = d + 16 * ((r >> 2) & 1); return x < D ? x : x - D; }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_f32_kernel(Args a) {
  constexpr int CH = D / 4;                   // 16-byte chunks per row
  constexpr int NS = D / 4;                   // k-steps of a score block
  constexpr int NG = D / 16;                  // groups of four steps read as 16-byte chunks
  constexpr int NDB = (D + 15) / 16;          // 16-wide output blocks (72 -> 5, the last partial)
  __shared__ __attribute__((aligned(1024))) float Ks[2][BN * D];
  __shared__ __attribute__((aligned(1024))) float Vs[2][BN * D];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int a16 = lane & 15, grp4 = lane >> 4;
  const int w = remap_xcd(blockIdx.x, a.total_wg);
  // (branch, kv head, key range) groups of wg_per_group workgroups
  const int grp = w / a.wg_per_group;
  const int split = grp % a.nsplit, bg = grp / a.nsplit;
  const int b = bg / a.heads_kv, g = bg % a.heads_kv;
  const int rem = w % a.wg_per_group;
  const int qb = rem * WAVES + wave;
  const bool active = qb < a.nqb;
  const int hq = g * a.group + (active ? qb / a.nchunks : 0);
  // the lane's two queries: sub-block qs holds token chunk*32 + 16qs + l % 16
  const int tok0 = (active ? qb % a.nchunks : 0) * 32 + a16;
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

  // Q^T operand of sub-block qs. Score steps come in groups G of four: step 4G + w takes
  // head dims 16G + 4k + w (k = l / 16, the MFMA's k index), so that a lane's K operands
  // for the group are one 16-byte chunk (one ds_read_b128). With head_dim 72 the last 8
  // dims form two single steps, 64 + 4t + k (t = 0, 1).
  float qv[2][NS];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int tk = tok0 + 16 * qs < a.seq ? tok0 + 16 * qs : a.seq - 1;
    const float* qrow = a.q + b * a.qs0 + (int64_t)tk * a.qs1 + (int64_t)hq * a.qs2;
#pragma unroll
    for (int G = 0; G < NG; ++G) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(qrow + 16 * G + 4 * grp4);
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) qv[qs][4 * G + w4] = x[w4];
    }
#pragma unroll
    for (int t2 = 0; t2 < NS - 4 * NG; ++t2) qv[qs][4 * NG + t2] = qrow[16 * NG + 4 * t2 + grp4];
  }

  // Tile loads go straight to LDS (global_load_lds, 16 bytes a lane, 1 KB an
  // instruction at consecutive LDS slots): slot x of a tile is row x / CH, chunk position
  // x % CH, and its lane fetches the global chunk that kslot / vcol place there. The CH
  // instructions per tensor are dealt round-robin to the 4 waves.
  const int64_t pstride = (int64_t)a.heads_kv * D;
  auto tile_dma = [&](int t, int buf) {
    constexpr int NI = BN * CH / 64;
#pragma unroll
    for (int ii = 0; ii < (NI + WAVES - 1) / WAVES; ++ii) {
      const int ins = ii * WAVES + wave;
      if (ins < NI) {
        const int x = ins * 64 + lane;
        const int r = x / CH, cp = x - r * CH;
        int jk = t * BN + r;
        jk = jk < kend ? jk : kend - 1;
        const float *kr, *vr;
        if (jk < P) {
          kr = a.prefix[b] + (int64_t)jk * pstride + (int64_t)g * D;
          vr = kr + (int64_t)P * pstride;
        } else {
          const int64_t off = b * a.ks0 + (int64_t)(jk - P) * a.ks1 + (int64_t)g * a.ks2;
          kr = a.k + off;
          vr = a.v + off;
        }
        // inverse permutations: the global chunk whose LDS position is cp
        int ck, cv;
        if constexpr (D == 64) {
          ck = cp ^ (r & 7);
          cv = cp ^ (4 * ((r >> 2) & 1));
        } else {
          ck = cp - ((r >> 2) & 1);
          ck = ck < 0 ? ck + CH : ck;
          cv = cp - 4 * ((r >> 2) & 1);
          cv = cv < 0 ? cv + CH : cv;
        }
        __builtin_amdgcn_global_load_lds(kr + 4 * ck, (__attribute__((address_space(3))) void*)&Ks[buf][ins * 256],
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds(vr + 4 * cv, (__attribute__((address_space(3))) void*)&Vs[buf][ins * 256],
                                         16, 0, 0);
      }
    }
  };
  auto wait_tiles = [&]() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
  };

  f32x4 acc_o[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db][0] = acc_o[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-__builtin_inff(), -__builtin_inff()}, l[2] = {0.f, 0.f};

  tile_dma(t0, 0);
  wait_tiles();

  for (int t = t0; t < t0 + T; ++t) {
    const int buf = (t - t0) & 1;
    if (t + 1 < t0 + T) tile_dma(t + 1, buf ^ 1);
    const float* kb_ = Ks[buf];
    const float* vb_ = Vs[buf];

    // S^T = K Q^T: key block kb, query sub-block qs; one K fragment per (kb, step)
    f32x4 s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb][0] = s[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = 16 * kb + a16;
      const float* krow = kb_ + r * D;
#pragma unroll
      for (int G = 0; G < NG; ++G) {
        const f32x4 kf = *reinterpret_cast<const f32x4*>(krow + 4 * kslot<D>(r, 4 * G + grp4));
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          s[kb][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[w4], qv[0][4 * G + w4], s[kb][0], 0, 0, 0);
          s[kb][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[w4], qv[1][4 * G + w4], s[kb][1], 0, 0, 0);
        }
      }
#pragma unroll
      for (int t2 = 0; t2 < NS - 4 * NG; ++t2) {
        const float kf = krow[4 * kslot<D>(r, 4 * NG + t2) + grp4];
        s[kb][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf, qv[0][4 * NG + t2], s[kb][0], 0, 0, 0);
        s[kb][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf, qv[1][4 * NG + t2], s[kb][1], 0, 0, 0);
      }
    }
    // mask keys past the end (only the last tile can have them): register j of block
    // kb is key 16kb + 4(l / 16) + j
    const int valid = kend - t * BN;
    if (valid < BN) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (16 * kb + 4 * grp4 + j >= valid) s[kb][0][j] = s[kb][1][j] = -__builtin_inff();
    }
    // online softmax per query (base 2, scale folded into one fma per score); a row's
    // keys are spread over the four 16-lane groups
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      float tmax = s[0][qs][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) tmax = __builtin_fmaxf(tmax, s[kb][qs][j]);
      {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(tmax), __float_as_int(tmax), false, false);
        tmax = __builtin_fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1]));
      }
      tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 16));
      const float cand = tmax * a.c;
      const bool grow = cand > m[qs] + RESCALE_T;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float mnew = grow ? cand : m[qs];
        const float alpha = __builtin_amdgcn_exp2f(m[qs] - mnew);
        l[qs] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc_o[db][qs] *= alpha;
        m[qs] = mnew;
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qs][j], a.c, -m[qs]));
          s[kb][qs][j] = p;
          l[qs] += p;
        }
    }
    // O^T += V^T P^T: step (kb, j) covers keys 16kb + 4k + j (k = l / 16 in both operands)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * kb + 4 * grp4 + j;
          const float vf = vb_[r * D + vcol<D>(r, 16 * db + a16)];
          acc_o[db][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf, s[kb][0][j], acc_o[db][0], 0, 0, 0);
          acc_o[db][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf, s[kb][1][j], acc_o[db][1], 0, 0, 0);
        }
    wait_tiles();
  }

  // epilogue: combine the four lane groups' partial sums, normalise, store (lane l holds
  // head dims 16db + 4(l / 16) .. + 3 of its two queries)
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(l[qs]), __float_as_int(l[qs]), false, false);
    l[qs] = __int_as_float(sw[0]) + __int_as_float(sw[1]);
    l[qs] += __shfl_xor(l[qs], 16);
  }
  if (!active) return;
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int tok = tok0 + 16 * qs;
    if (tok >= a.seq) continue;
    const float inv = 1.0f / l[qs];
    // log-sum-exp: sum_j exp2(c s_j - m) = l, so lse = ln2 * (m + log2 l)  (l >= 1)
    const float lse = LN2 * (m[qs] + __builtin_amdgcn_logf(l[qs]));
    float* orow;
    if (partial) {
      orow = a.part_o + ((((int64_t)split * a.batch + b) * a.seq + tok) * a.heads_q + hq) * D;
      if (grp4 == 0) a.part_lse[(((int64_t)split * a.batch + b) * a.heads_q + hq) * a.seq + tok] = lse;
    } else {
      orow = a.o + b * a.os0 + (int64_t)tok * a.os1 + (int64_t)hq * a.os2;
      if (a.lse && grp4 == 0) a.lse[((int64_t)b * a.heads_q + hq) * a.seq + tok] = lse;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = 16 * db + 4 * grp4;
      if (d < D) *reinterpret_cast<f32x4*>(orow + d) = acc_o[db][qs] * inv;
    }
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
