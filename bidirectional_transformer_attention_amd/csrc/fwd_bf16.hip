// Fused non-causal GQA attention, bf16 in/out, head_dim 128, bf16 MFMA
// (v_mfma_f32_32x32x16_bf16) with fp32 accumulation and an fp32 online softmax.
// KLiteInfer page, "架构": bidirectional attention = scores GEMM + softmax + output GEMM
// (prior art materialises the score matrix; here it never leaves the registers).
// NeoPP page: the DiT attends to [conditioning KV prefix ++ own tokens], one CFG branch
// per batch entry, prefix in the online layout [2, P, kv_heads, D].
//
// Work split. A workgroup of 8 waves serves one (branch, kv head) and 8 query blocks of
// 32 rows; query blocks enumerate (q head within the GQA group, 32-token chunk), so all
// 8 waves read the same K/V tiles from LDS (one tile load feeds G heads). Keys are
// walked in tiles of 64 over the virtual sequence [prefix ++ own].
//
// Per wave: S^T = K Q^T lives in the 32x32 accumulator layout (lane = query row, 16
// registers = keys), so row max / row sum are in-lane plus one permlane32 swap; the
// accumulator registers, rounded to bf16, are directly the B operand (P^T) of
// O^T += V^T P^T. The V^T operand comes from row-major V in LDS through the gfx950
// transposing read ds_read_b64_tr_b16, so K and V are both stored row-major.
//
// Ping-pong. Waves 0-3 and 4-7 (one of each per SIMD) run the same program half a
// tile apart: while one group issues the MFMAs of tile t (scores of t+1 and P V of t),
// the other group runs the exp2/max/sum of its softmax, so matrix cores and VALU of a
// SIMD overlap. Each half-iteration ends at a workgroup barrier.
//
// LDS: K and V double-buffered, 64 rows x 256 B each, 16-byte chunks XOR-swizzled per
// row (K: chunk ^ (row & 15), V: chunk ^ 4*(row & 3)) so the row-parallel K reads and
// the 4-row transposing V reads are free of bank conflicts. 64 KB per workgroup.
// MFMA-bound: 4*Sq*Skv*Hq*D flops per launch.
#include "nx_internal.h"

namespace nx {

namespace bf16k {

constexpr int D = 128;
constexpr int BN = 64;            // keys per tile
constexpr int WAVES = 8;
constexpr int THREADS = WAVES * 64;
constexpr int ROWB = D * 2;       // bytes per K/V row
constexpr int TILEB = BN * ROWB;  // bytes per K or V tile (16 KB)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_T = 8.0f; // running max moves only when it grows by > 2^8

struct Args {
  const uint16_t* q; const uint16_t* k; const uint16_t* v; uint16_t* o;
  int64_t qs0, qs1, qs2, ks0, ks1, ks2, os0, os1, os2;
  const uint16_t* prefix[NXATTN_MAX_BRANCHES];
  int32_t plen[NXATTN_MAX_BRANCHES];
  int32_t batch, seq, heads_q, heads_kv, group, nchunks, nqb, wg_per_group, total_wg;
  float c;  // scale * log2(e)
};

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ int remap_xcd(int i, int n) {
  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a contiguous
  // run of logical work so workgroups sharing K/V tiles share one L2.
  const int xcd = i & 7, local = i >> 3;
  const int per = n >> 3, rem = n & 7;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

__device__ __forceinline__ int kslot(int row, int chunk) { return chunk ^ (row & 15); }
__device__ __forceinline__ int vslot(int row, int chunk) { return chunk ^ ((row & 3) << 2); }

__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

struct Wave {
  // per-wave state of one 32-row query block
  bf16x8 qf[8];       // Q^T operand, k-step ks: Q[row][16ks + 8hh .. +7]
  f32x16 o[4];        // O^T accumulators, d-block db: rows d = 32db + ..., lane = query
  f32x16 s[2];        // S^T accumulators of the tile being scored (2 key blocks of 32)
  bf16x8 p[4];        // P^T operand of the tile being accumulated, step (kb, half)
  float m, l;
};

// S^T = K_tile Q^T for the tile in LDS buffer kbuf.
__device__ __forceinline__ void gemm_s(Wave& w, const lds_u8* kbuf, int n, int hh) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int r = kb * 32 + n;
    const lds_u8* rowp = kbuf + r * ROWB;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const u32x4 kv = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(rowp + 16 * kslot(r, 2 * ks + hh));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), w.qf[ks], acc, 0, 0, 0);
    }
    w.s[kb] = acc;
  }
}

// O^T += V_tile^T P^T for the tile in LDS buffer vbuf.
__device__ __forceinline__ void gemm_pv(Wave& w, const lds_u8* vbuf, int lane) {
  const int q = lane >> 4, j = lane & 15;
  const int hq = q >> 1;                 // lane half of the reading group
  const int rsub = j >> 2;               // row within the 4-row group this lane addresses
  const int csub = 4 * (j & 3);          // first column this lane addresses
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      const int r0 = kb * 32 + 16 * hs + 4 * hq + rsub;   // rows of elements 0..3
      const int r1 = r0 + 8;                              // rows of elements 4..7
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int col = 32 * db + 16 * (q & 1) + csub;
        const lds_u8* a0 = vbuf + r0 * ROWB + 16 * vslot(r0, col >> 3) + 2 * (col & 7);
        const lds_u8* a1 = vbuf + r1 * ROWB + 16 * vslot(r1, col >> 3) + 2 * (col & 7);
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)a0);
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)a1);
        const bf16x8 vf = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        w.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, w.p[2 * kb + hs], w.o[db], 0, 0, 0);
      }
    }
}

// Online softmax of w.s (tile with `valid` keys, < BN only for the last tile) -> w.p.
__device__ __forceinline__ void softmax(Wave& w, float c, int valid, int hh) {
  if (valid < BN) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
        if (key >= valid) w.s[kb][i] = -__builtin_inff();
      }
  }
  float t0 = __builtin_fmaxf(w.s[0][0], w.s[0][1]);
  float t1 = __builtin_fmaxf(w.s[1][0], w.s[1][1]);
#pragma unroll
  for (int i = 2; i < 16; ++i) {
    t0 = __builtin_fmaxf(t0, w.s[0][i]);
    t1 = __builtin_fmaxf(t1, w.s[1][i]);
  }
  float tmax = __builtin_fmaxf(t0, t1);
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(tmax), __float_as_int(tmax), false, false);
    tmax = __builtin_fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1]));
  }
  const float cand = tmax * c;
  const bool grow = cand > w.m + RESCALE_T;
  if (__builtin_amdgcn_ballot_w64(grow)) {
    const float mnew = grow ? cand : w.m;
    const float alpha = __builtin_amdgcn_exp2f(w.m - mnew);
    w.l *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) w.o[db][i] *= alpha;
    w.m = mnew;
  }
  const float nm = -w.m;
  float l0 = 0.f, l1 = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(w.s[kb][8 * hs + 2 * e], c, nm));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(w.s[kb][8 * hs + 2 * e + 1], c, nm));
        l0 += p0;
        l1 += p1;
        pk[e] = pack_bf16x2(p0, p1);
      }
      w.p[2 * kb + hs] = as_bf16x8(pk);
    }
  w.l += l0 + l1;
}

__global__ __launch_bounds__(THREADS) void fwd_bf16_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * TILEB];   // K0 K1 V0 V1
  lds_u8* lds = (lds_u8*)smem;
  lds_u8* kbufs[2] = {lds, lds + TILEB};
  lds_u8* vbufs[2] = {lds + 2 * TILEB, lds + 3 * TILEB};

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const bool grpA = wave < 4;

  const int wg = remap_xcd(blockIdx.x, a.total_wg);
  const int b = wg / (a.heads_kv * a.wg_per_group);
  const int rem = wg % (a.heads_kv * a.wg_per_group);
  const int g = rem / a.wg_per_group;
  const int qb = (rem % a.wg_per_group) * WAVES + wave;
  const bool active = qb < a.nqb;
  const int hq = g * a.group + (active ? qb / a.nchunks : 0);
  const int tok = (active ? qb % a.nchunks : 0) * 32 + n;
  const int tokc = tok < a.seq ? tok : a.seq - 1;
  const int P = a.plen[b];
  const int Skv = P + a.seq;
  const int T = (Skv + BN - 1) / BN;
  const float c = a.c;

  Wave w;
  {
    const uint16_t* qrow = a.q + b * a.qs0 + (int64_t)tokc * a.qs1 + (int64_t)hq * a.qs2;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) w.qf[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * hh));
  }
#pragma unroll
  for (int db = 0; db < 4; ++db) w.o[db] = f32x16{};
  w.m = -__builtin_inff();
  w.l = 0.f;

  // Tile loads: thread -> two 16-byte chunks of K and two of V (row = it / 16, chunk = it % 16).
  const uint16_t* kprefix = a.prefix[b] ? a.prefix[b] + (int64_t)g * D : nullptr;
  const int64_t pstride = (int64_t)a.heads_kv * D;
  const uint16_t* kown = a.k + b * a.ks0 + (int64_t)g * a.ks2;
  const uint16_t* vown = a.v + b * a.ks0 + (int64_t)g * a.ks2;
  auto row_ptrs = [&](int j, const uint16_t*& kr, const uint16_t*& vr) {
    j = j < Skv ? j : Skv - 1;
    if (j < P) {
      kr = kprefix + (int64_t)j * pstride;
      vr = kr + (int64_t)P * pstride;
    } else {
      kr = kown + (int64_t)(j - P) * a.ks1;
      vr = vown + (int64_t)(j - P) * a.ks1;
    }
  };
  u32x4 stg_k[2], stg_v[2];
  auto load_k = [&](int t) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int it = tid + i * THREADS;
      const uint16_t *kr, *vr;
      row_ptrs(t * BN + (it >> 4), kr, vr);
      stg_k[i] = *reinterpret_cast<const u32x4*>(kr + 8 * (it & 15));
    }
  };
  auto load_v = [&](int t) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int it = tid + i * THREADS;
      const uint16_t *kr, *vr;
      row_ptrs(t * BN + (it >> 4), kr, vr);
      stg_v[i] = *reinterpret_cast<const u32x4*>(vr + 8 * (it & 15));
    }
  };
  auto store_k = [&](lds_u8* buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int it = tid + i * THREADS, r = it >> 4, ch = it & 15;
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(buf + r * ROWB + 16 * kslot(r, ch)) = stg_k[i];
    }
  };
  auto store_v = [&](lds_u8* buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int it = tid + i * THREADS, r = it >> 4, ch = it & 15;
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(buf + r * ROWB + 16 * vslot(r, ch)) = stg_v[i];
    }
  };

  // ---- prologue: K_0, V_0, K_1 resident; both groups score tile 0; group A also
  // ---- runs its softmax, so that A leads B by half a tile from here on.
  load_k(0);
  load_v(0);
  store_k(kbufs[0]);
  store_v(vbufs[0]);
  if (T > 1) {
    load_k(1);
    store_k(kbufs[1]);
  }
  barrier_lds();
  gemm_s(w, kbufs[0], n, hh);
  if (grpA) softmax(w, c, Skv < BN ? Skv : BN, hh);
  barrier_only();

  for (int t = 0; t < T; ++t) {
    const bool more = t + 1 < T;
    const int valid_next = Skv - (t + 1) * BN;
    // slot 2t: loads for tile t+2 (K) / t+1 (V) go out; A multiplies, B normalises.
    if (t + 2 < T) load_k(t + 2);
    if (more) load_v(t + 1);
    if (grpA) {
      gemm_pv(w, vbufs[t & 1], lane);
      if (more) gemm_s(w, kbufs[(t + 1) & 1], n, hh);
    } else {
      softmax(w, c, Skv - t * BN < BN ? Skv - t * BN : BN, hh);
    }
    barrier_only();
    // slot 2t+1: A normalises tile t+1, B multiplies; staged tiles land in LDS.
    if (grpA) {
      if (more) softmax(w, c, valid_next < BN ? valid_next : BN, hh);
    } else {
      gemm_pv(w, vbufs[t & 1], lane);
      if (more) gemm_s(w, kbufs[(t + 1) & 1], n, hh);
    }
    if (t + 2 < T) store_k(kbufs[t & 1]);
    if (more) store_v(vbufs[(t + 1) & 1]);
    barrier_lds();
  }

  // ---- epilogue: total row sum (both lane halves), normalise, round, store
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(w.l), __float_as_int(w.l), false, false);
    w.l = __int_as_float(sw[0]) + __int_as_float(sw[1]);
  }
  if (!active || tok >= a.seq) return;
  const float inv = 1.0f / w.l;
  uint16_t* orow = a.o + b * a.os0 + (int64_t)tok * a.os1 + (int64_t)hq * a.os2;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = 32 * db + 8 * i4 + 4 * hh;
      *reinterpret_cast<u32x2*>(orow + d) =
          u32x2{pack_bf16x2(w.o[db][4 * i4] * inv, w.o[db][4 * i4 + 1] * inv),
                pack_bf16x2(w.o[db][4 * i4 + 2] * inv, w.o[db][4 * i4 + 3] * inv)};
    }
}

}  // namespace bf16k

int launch_fwd_bf16(const FwdProblem& p, hipStream_t stream) {
  using namespace bf16k;
  Args a;
  a.q = static_cast<const uint16_t*>(p.q); a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.v); a.o = static_cast<uint16_t*>(p.o);
  a.qs0 = p.qs[0]; a.qs1 = p.qs[1]; a.qs2 = p.qs[2];
  a.ks0 = p.ks[0]; a.ks1 = p.ks[1]; a.ks2 = p.ks[2];
  a.os0 = p.os[0]; a.os1 = p.os[1]; a.os2 = p.os[2];
  for (int b = 0; b < NXATTN_MAX_BRANCHES; ++b) { a.prefix[b] = static_cast<const uint16_t*>(p.prefix[b]); a.plen[b] = p.plen[b]; }
  a.batch = p.batch; a.seq = p.seq_q; a.heads_q = p.heads_q; a.heads_kv = p.heads_kv;
  a.group = p.heads_q / p.heads_kv;
  a.nchunks = (p.seq_q + 31) / 32;
  const int64_t nqb = (int64_t)a.group * a.nchunks;
  const int64_t wpg = (nqb + WAVES - 1) / WAVES;
  const int64_t total = wpg * p.heads_kv * p.batch;
  if (total > INT32_MAX / 2) return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd: problem too large");
  a.nqb = (int)nqb; a.wg_per_group = (int)wpg; a.total_wg = (int)total;
  a.c = p.scale * LOG2E;
  fwd_bf16_kernel<<<a.total_wg, THREADS, 0, stream>>>(a);
  return check_launch("nxattn_fwd(bf16)");
}

}  // namespace nx
