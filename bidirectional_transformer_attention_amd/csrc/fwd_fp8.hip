// Fused non-causal GQA attention with an FP8 score GEMM: q and k are OCP E4M3 codes with
// one power-of-two scale per (branch, head), v and the output are bf16, head_dim 128.
// The scores come from v_mfma_scale_f32_32x32x64_f8f6f4, whose per-lane E8M0 scale
// operands apply the (power-of-two) dequantisation exactly inside the matrix core: the
// key rows take the scale of the tensor they come from (prefix or own keys), the query
// columns the scale of their head. Softmax, P (bf16) and O^T += V^T P^T are the bf16
// kernel's. KLiteInfer page, "架构": scores GEMM, softmax, output GEMM; NeoPP page: the
// DiT attends to [conditioning prefix ++ own tokens], and it names fp8 DiT variants
// without a recipe (the recipe here is the quantisation of q and k in quant.hip).
//
// The structure follows the bf16 kernel (8 waves, two ping-pong groups half a tile apart,
// a workgroup per (branch, kv head) and 8 query blocks of 32 rows, direct-to-LDS tile
// loads by waves 0-3 interleaved with the score MFMAs, the straddling tile processed
// last). What changes: K tiles are 64 rows x 128 B of fp8 (16-byte chunks swizzled
// chunk ^ (row & 7)); a score step is one 32x32x64 MFMA, so a tile needs 4 score MFMAs
// next to its 16 P V MFMAs; q stays in registers as 16 VGPRs of codes.
// MFMA-bound: 4*Sq*Skv*Hq*D flops per launch, half on the fp8 and half on the bf16 unit.
#include <cmath>
#include <type_traits>

#include "nx_internal.h"

namespace nx {

namespace fp8k {

typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int D = 128;
constexpr int BN = KEY_TILE;       // keys per tile (64)
constexpr int WAVES = 8;
constexpr int THREADS = WAVES * 64;
constexpr int VROWB = D * 2;       // bytes per V row (bf16)
constexpr int KROWB = D;           // bytes per K row (fp8)
constexpr int VTILEB = BN * VROWB; // 16 KB
constexpr int KTILEB = BN * KROWB; // 8 KB
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float RESCALE_T = 8.0f;  // running max moves only when it grows by > 2^8
constexpr float RESCALE_LIM = 256.0f;  // 2^RESCALE_T
constexpr int BUF_RECORDS = 0x7fffffff;
constexpr int BUF_FLAGS = 0x00020000;

struct Args {
  const uint8_t* q8; const uint8_t* k8; const uint16_t* v; uint16_t* o;
  const int8_t* q_exp; const int8_t* k_exp; const int8_t* pk_exp;
  int64_t vs0, vs1, vs2, os0, os1, os2;
  const uint8_t* pk8[NXATTN_MAX_BRANCHES];
  const uint16_t* pv[NXATTN_MAX_BRANCHES];
  int32_t plen[NXATTN_MAX_BRANCHES];
  int32_t batch, seq, heads_q, heads_kv, group, nchunks, nqb, wg_per_group, total_wg;
  float c;  // scale * log2(e)
  float* lse;
};

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ int remap_xcd(int i, int n) {
  const int xcd = i & 7, local = i >> 3;
  const int per = n >> 3, rem = n & 7;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

__device__ __forceinline__ void barrier_only() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
// No wave priorities here (unlike the bf16 kernel): with the fp8 score GEMM the softmax,
// not the matrix core, sets the pace, and same-box runs were 1.7 % faster at the 1K DiT
// shape (0.2 % slower at 2K) without them. The iteration's one barrier is the one after
// the tile loads land (the second slot reads only buffers no load of the iteration writes).
__device__ __forceinline__ void wait_dma_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// LDS: K (fp8) and V (bf16) tiles, double-buffered, as four distinct objects
__shared__ __attribute__((aligned(1024))) uint8_t lds_k0[KTILEB];
__shared__ __attribute__((aligned(1024))) uint8_t lds_k1[KTILEB];
__shared__ __attribute__((aligned(1024))) uint8_t lds_v0[VTILEB];
__shared__ __attribute__((aligned(1024))) uint8_t lds_v1[VTILEB];
template <int PAR> __device__ __forceinline__ uint8_t* kbuf() { return PAR ? lds_k1 : lds_k0; }
template <int PAR> __device__ __forceinline__ uint8_t* vbuf() { return PAR ? lds_v1 : lds_v0; }

// Steady-state tile loads of one wave (rows 16ws .. 16ws+15 of a tile): K in 2
// instructions of 8 rows (lane -> row rl8 = lane/8, slot lane%8), V in 4 of 4 rows
// (lane -> row lane/16, slot lane%16). Global address = the raw buffer's base (row 16ws of
// the tile) + the lane offset + the instruction's row step.
struct DmaPlan {
  __amdgpu_buffer_rsrc_t krsrc, vrsrc;
  uint32_t krs, vrs;      // 8-row (K) / 4-row (V) step in bytes
  uint32_t koff, voff;    // lane offsets in bytes (row and swizzled chunk)
  int ws;
};

struct Wave {
  v8i q8[2];          // Q^T operand, k-step ks: codes Q[row][64ks + 32hh .. +31]
  f32x16 o[4];        // O^T accumulators, d-block db
  f32x16 s[2];        // S^T accumulators of the tile being scored (2 key blocks of 32)
  bf16x8 p[4];        // P^T operand of the tile being accumulated
  float m, l;
  bool primed;        // FOLD: a first tile has set m (weights may be taken before the max)
  float thr;          // FOLD: row max of the shifted scores above which m moves (-inf before
                      // the first tile); else (m + RESCALE_T) / c on raw scores
  f32x16 negm;        // FOLD: -m in every register, the score accumulators' start value
  int kbase, kxh;     // K fragment (kb, ks, half e): kbase + kb*32*KROWB + ((64ks + 16e) ^ kxh)
  int vbase, vy;      // V^T fragment of d-block db at vbase + (64db ^ vy)
  int qsc;            // E8M0 scale of the wave's q head (B operand)
};

__device__ __forceinline__ u32x4 lds_read_b128(const uint8_t* smem, int byte) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>((const lds_u8*)smem + byte);
}
__device__ __forceinline__ bf16x4 lds_read_tr(const uint8_t* smem, int byte) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)((const lds_u8*)smem + byte));
}
__device__ __forceinline__ v8i kfrag(const uint8_t* ksm, const Wave& w, int kb, int ks) {
  const int base = w.kbase + kb * 32 * KROWB;
  const u32x4 a = lds_read_b128(ksm, base + ((64 * ks) ^ w.kxh));
  const u32x4 b = lds_read_b128(ksm, base + ((64 * ks + 16) ^ w.kxh));
  return __builtin_bit_cast(v8i, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ f32x16 mfma_s(v8i k, v8i q, f32x16 acc, int ksc, int qsc) {
  // formats 0 / 0: E4M3 for both operands; E8M0 scales from the low byte of ksc / qsc
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k, q, acc, 0, 0, 0, ksc, 0, qsc);
}

// One GEMM phase: O^T += V_t^T P_t^T (16 bf16 MFMAs), then S^T = K_{t+1} Q^T (4 fp8
// MFMAs, key blocks kb with E8M0 scales ksc0 / ksc1). V fragments are read three MFMAs
// ahead; the 4 K fragments are read during the last P V steps.
template <int I, int N>
__device__ __forceinline__ void sched8_reads() {
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    sched8_reads<I + 1, N>();
  }
}
template <int I, bool DMA>
__device__ __forceinline__ void sched8_steps() {
  if constexpr (I < 20) {
    // reads issued before MFMA I: V step I+3 (2 reads) while I + 3 < 16, then K
    // fragments (2 reads each) for the score steps
    if constexpr (I + 3 < 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    else if constexpr (I + 3 < 20) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    if constexpr (DMA && I >= 16) __builtin_amdgcn_sched_group_barrier(0x010, I < 18 ? 2 : 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    sched8_steps<I + 1, DMA>();
  }
}

template <int VPAR, int KPAR, bool FOLD, bool DMA = false>
__device__ __forceinline__ void gemm_phase(Wave& w, int ksc0, int ksc1, const DmaPlan* plan = nullptr) {
  const uint8_t* vsm = vbuf<VPAR>();
  const uint8_t* ksm = kbuf<KPAR>();
  constexpr int DIST = 3;
  auto vread = [&](int i) -> bf16x8 {
    const int kbhs = i >> 2, db = i & 3;
    const int rbase = (kbhs >> 1) * 32 + (kbhs & 1) * 16;
    const int off = w.vbase + ((64 * db) ^ w.vy);
    const bf16x4 a = lds_read_tr(vsm, rbase * VROWB + off);
    const bf16x4 b = lds_read_tr(vsm, (rbase + 8) * VROWB + off);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // DMA d: 0-1 K rows 16ws + 8d .. into K buffer KPAR^1, 2-5 V rows 16ws + 4(d-2) ..
  // into V buffer VPAR^1 (both last read in the previous iteration)
  auto dma = [&](int d) {
    if (d < 2) {
      uint8_t* dst = kbuf<KPAR ^ 1>() + (16 * plan->ws + 8 * d) * KROWB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(plan->krsrc, (__attribute__((address_space(3))) void*)(lds_u8*)dst, 16,
                                               plan->koff, d * plan->krs, 0, 0);
    } else {
      const int i = d - 2;
      uint8_t* dst = vbuf<VPAR ^ 1>() + (16 * plan->ws + 4 * i) * VROWB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(plan->vrsrc, (__attribute__((address_space(3))) void*)(lds_u8*)dst, 16,
                                               plan->voff, i * plan->vrs, 0, 0);
    }
  };
  bf16x8 ring[DIST + 1];
  v8i kf[4];
#pragma unroll
  for (int i = 0; i < DIST; ++i) ring[i] = vread(i);
#pragma unroll
  for (int i = 0; i < 20; ++i) {
    if (i + DIST < 16) ring[(i + DIST) % (DIST + 1)] = vread(i + DIST);
    else if (i + DIST < 20) { const int j = i + DIST - 16; kf[j] = kfrag(ksm, w, j & 1, j >> 1); }
    if constexpr (DMA) {
      if (i == 16) { dma(0); dma(1); }
      if (i == 17) { dma(2); dma(3); }
      if (i == 18) dma(4);
      if (i == 19) dma(5);
    }
    if (i < 16) {
      const int kbhs = i >> 2, db = i & 3;
      w.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % (DIST + 1)], w.p[kbhs], w.o[db], 0, 0, 0);
    } else {
      const int j = i - 16, ks = j >> 1, kb = j & 1;
      w.s[kb] = mfma_s(kf[j], w.q8[ks], ks == 0 ? (FOLD ? w.negm : f32x16{}) : w.s[kb], kb ? ksc1 : ksc0, w.qsc);
    }
  }
  sched8_reads<0, DIST>();
  sched8_steps<0, DMA>();
}

// S^T only (prologue).
template <int KPAR, bool FOLD>
__device__ __forceinline__ void gemm_s_only(Wave& w, int ksc0, int ksc1) {
  const uint8_t* ksm = kbuf<KPAR>();
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      w.s[kb] = mfma_s(kfrag(ksm, w, kb, ks), w.q8[ks], ks == 0 ? (FOLD ? w.negm : f32x16{}) : w.s[kb],
                       kb ? ksc1 : ksc0, w.qsc);
}

// Row max of the tile; rows whose max exceeds their threshold move m (rescaling l, O).
template <bool FOLD>
__device__ __forceinline__ void max_update(Wave& w, float c) {
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
  const bool grow = tmax > w.thr;
  if constexpr (FOLD) {
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float d = grow ? tmax : 0.f;
      const float alpha = __builtin_amdgcn_exp2f(-d);
      w.l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) w.o[db][i] *= alpha;
      w.m += d;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        w.s[0][i] -= d;
        w.s[1][i] -= d;
      }
      w.thr = RESCALE_T;
    }
  } else {
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float mnew = grow ? tmax * c : w.m;
      const float alpha = __builtin_amdgcn_exp2f(w.m - mnew);
      w.l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) w.o[db][i] *= alpha;
      w.m = mnew;
      w.thr = (mnew + RESCALE_T) / c;
    }
  }
}

// Weights of the tile against the current m, rounded to bf16 into w.p; returns this
// lane's (unrounded) sum of them.
template <bool FOLD>
__device__ __forceinline__ float weights(Wave& w, float c) {
  const float nm = -w.m;
  float l0 = 0.f, l1 = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = w.s[kb][8 * hs + 2 * e], x1 = w.s[kb][8 * hs + 2 * e + 1];
        const float p0 = __builtin_amdgcn_exp2f(FOLD ? x0 : __builtin_fmaf(x0, c, nm));
        const float p1 = __builtin_amdgcn_exp2f(FOLD ? x1 : __builtin_fmaf(x1, c, nm));
        l0 += p0;
        l1 += p1;
        pk[e] = pack_bf16x2(p0, p1);
      }
      w.p[2 * kb + hs] = as_bf16x8(pk);
    }
  return l0 + l1;
}

// Online softmax of w.s (the tile holds `valid` keys, < BN only for the last tile of a
// branch) -> w.p. MASK = false: the tile is known to be whole. FOLD: q's codes carry
// c = scale * log2(e) and the score accumulators start at -m, so w.s holds c s - m and each
// weight is one exp2 (a rescale moves m by the tile max d and shifts the tile by -d);
// otherwise w.s holds the raw scores and each weight is exp2(fma(s, c, -m)).
template <bool MASK, bool FOLD>
__device__ __forceinline__ void softmax(Wave& w, float c, int valid, int hh) {
  if (MASK && valid < BN) {
    const int lim = valid - 4 * hh;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kb * 32 + 8 * (i >> 2) + (i & 3) >= lim) w.s[kb][i] = -__builtin_inff();
  }
  if constexpr (FOLD) {
    // weights first against the current m; the row max only when some lane's sum of
    // them exceeds 2^RESCALE_T (then every weight might have, and m may have to move),
    // or before a first tile has set m. One copy of the weight code in a loop that is
    // never unrolled.
    float lt = 0.f;
#pragma nounroll
    for (int pass = w.primed ? 0 : 1; pass < 2; ++pass) {
      if (pass == 1) {
        max_update<FOLD>(w, c);
        w.primed = true;
      }
      lt = weights<FOLD>(w, c);
      if (pass == 1 || !__builtin_amdgcn_ballot_w64(!(lt <= RESCALE_LIM))) break;
    }
    w.l += lt;
#pragma unroll
    for (int i = 0; i < 16; ++i) w.negm[i] = -w.m;
  } else {
    max_update<FOLD>(w, c);
    w.l += weights<FOLD>(w, c);
  }
}

template <bool GROUP_A, bool FOLD>
__device__ __forceinline__ void wave_program(const Args& a, int lane, int wave) {
  const int n = lane & 31, hh = lane >> 5;
  const int wg = remap_xcd(blockIdx.x, a.total_wg);
  const int grp = wg / a.wg_per_group;
  const int g = grp / a.batch, b = grp % a.batch;
  const int qb = (wg % a.wg_per_group) * WAVES + wave;
  const bool active = qb < a.nqb;
  const int hq = g * a.group + (active ? qb / a.nchunks : 0);
  const int tok = (active ? qb % a.nchunks : 0) * 32 + n;
  const int tokc = tok < a.seq ? tok : a.seq - 1;
  const int P = a.plen[b];
  const int Skv = P + a.seq;
  const int T = (Skv + BN - 1) / BN;
  const float c = a.c;
  // E8M0 scales: key rows of the prefix / own keys, and this wave's q head
  const int sc_own = 127 + (int)a.k_exp[b * a.heads_kv + g];
  const int sc_pre = P > 0 ? 127 + (int)a.pk_exp[b * a.heads_kv + g] : sc_own;

  Wave w;
  {
    const uint8_t* qrow = a.q8 + (((int64_t)b * a.seq + tokc) * a.heads_q + hq) * D;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(qrow + 64 * ks + 32 * hh);
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(qrow + 64 * ks + 32 * hh + 16);
      w.q8[ks] = __builtin_bit_cast(v8i, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
  w.qsc = 127 + (int)a.q_exp[b * a.heads_q + hq];
#pragma unroll
  for (int db = 0; db < 4; ++db) w.o[db] = f32x16{};
  // FOLD: m starts at 0 (the accumulators start at -m = 0) and the first tile always
  // moves it to its row max
  w.m = FOLD ? 0.f : -__builtin_inff();
  w.primed = false;
  w.thr = -__builtin_inff();
  w.l = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) w.negm[i] = 0.f;
  // K fragment of key block kb, k-step ks, half e: row kb*32 + n, 16-byte chunk
  // 4ks + 2hh + e at slot chunk ^ (n & 7): byte n*KROWB + ((64ks + 16e) ^ (32hh ^ 16(n&7)))
  w.kbase = n * KROWB;
  w.kxh = (32 * hh) ^ (16 * (n & 7));
  {
    const int q = lane >> 4, j = lane & 15;
    const int rsub = j >> 2, csub = 4 * (j & 3);
    const int r = 4 * (q >> 1) + rsub;
    const int e = 2 * (q & 1) + (csub >> 3);
    w.vbase = r * VROWB + 16 * e + 2 * (csub & 7);
    w.vy = 64 * rsub;
  }

  // per-lane clamped direct-to-LDS loads (prologue, the straddling and the ragged tile)
  const uint8_t* kpre = a.pk8[b] ? a.pk8[b] + (int64_t)g * D : nullptr;
  const uint16_t* vpre = a.pv[b] ? a.pv[b] + (int64_t)g * D : nullptr;
  const int64_t krow = (int64_t)a.heads_kv * D;          // bytes between key rows (prefix and own)
  const int64_t pvrow = (int64_t)a.heads_kv * D;         // elements between prefix V rows
  const uint8_t* kown = a.k8 + (int64_t)b * a.seq * krow + (int64_t)g * D;
  const uint16_t* vown = a.v + b * a.vs0 + (int64_t)g * a.vs2;
  const int64_t vs1 = a.vs1;
  auto dma_k = [&](int t, uint8_t* dst, int ws, auto nw) {
    constexpr int NW = decltype(nw)::value;
    constexpr int ROWS = BN / NW;
#pragma unroll
    for (int i = 0; i < ROWS / 8; ++i) {
      const int r = ROWS * ws + 8 * i + (lane >> 3);
      const int chunk = (lane & 7) ^ (r & 7);
      int j = t * BN + r;
      j = j < Skv ? j : Skv - 1;
      const uint8_t* src = j < P ? kpre + (int64_t)j * krow : kown + (int64_t)(j - P) * krow;
      __builtin_amdgcn_global_load_lds(src + 16 * chunk,
                                       (__attribute__((address_space(3))) void*)((lds_u8*)dst + (ROWS * ws + 8 * i) * KROWB),
                                       16, 0, 0);
    }
  };
  auto dma_v = [&](int t, uint8_t* dst, int ws, auto nw) {
    constexpr int NW = decltype(nw)::value;
    constexpr int ROWS = BN / NW;
#pragma unroll
    for (int i = 0; i < ROWS / 4; ++i) {
      const int r = ROWS * ws + 4 * i + (lane >> 4);
      const int chunk = (lane & 15) ^ ((r & 3) << 2);
      int j = t * BN + r;
      j = j < Skv ? j : Skv - 1;
      const uint16_t* src = j < P ? vpre + (int64_t)j * pvrow : vown + (int64_t)(j - P) * vs1;
      __builtin_amdgcn_global_load_lds(src + 8 * chunk,
                                       (__attribute__((address_space(3))) void*)((lds_u8*)dst + (ROWS * ws + 4 * i) * VROWB),
                                       16, 0, 0);
    }
  };
  using All = std::integral_constant<int, 8>;
  using Half = std::integral_constant<int, 4>;

  // key tiles in natural order, the tile straddling the prefix end (unless last) moved
  // to the end; positions [0, nwhole) hold whole tiles wholly inside prefix or own keys
  const int sb = (P % BN != 0 && P / BN < T - 1) ? P / BN : -1;
  auto tile_at = [&](int pos) { return (sb < 0 || pos < sb) ? pos : (pos < T - 1 ? pos + 1 : sb); };
  auto valid_at = [&](int pos) { const int r = Skv - tile_at(pos) * BN; return r < BN ? r : BN; };
  const bool last_whole = T * BN <= Skv && ((T - 1) * BN >= P || T * BN <= P);
  const int nwhole = T - (sb >= 0 ? 1 : 0) - (last_whole ? 0 : 1);
  // E8M0 scale of this lane's key row in key block kb of tile t
  auto ksc = [&](int t, int kb) { return t * BN + kb * 32 + n < P ? sc_pre : sc_own; };

  const int rl8 = lane >> 3, rl4 = lane >> 4;
  const uint32_t koff = (uint32_t)(rl8 * krow) + 16u * (uint32_t)((lane & 7) ^ rl8);
  const uint32_t voff_pre = (uint32_t)(rl4 * pvrow * 2) + 16u * (uint32_t)((lane & 15) ^ (rl4 << 2));
  const uint32_t voff_own = (uint32_t)(rl4 * vs1 * 2) + 16u * (uint32_t)((lane & 15) ^ (rl4 << 2));
  auto plan_of = [&](int t) {
    DmaPlan pl;
    const int jk = tile_at(t + 2) * BN + 16 * wave, jv = tile_at(t + 1) * BN + 16 * wave;
    const bool kp = jk < P, vp = jv < P;
    const uint8_t* kb_ = kp ? kpre + (int64_t)jk * krow : kown + (int64_t)(jk - P) * krow;
    const uint16_t* vb_ = vp ? vpre + (int64_t)jv * pvrow : vown + (int64_t)(jv - P) * vs1;
    pl.krsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kb_), 0, BUF_RECORDS, BUF_FLAGS);
    pl.vrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vb_), 0, BUF_RECORDS, BUF_FLAGS);
    pl.krs = (uint32_t)(8 * krow);
    pl.vrs = (uint32_t)(8 * (vp ? pvrow : vs1));
    pl.koff = koff;
    pl.voff = vp ? voff_pre : voff_own;
    pl.ws = wave;
    return pl;
  };

  // ---- prologue (as in the bf16 kernel)
  dma_k(tile_at(0), kbuf<0>(), wave, All{});
  dma_v(tile_at(0), vbuf<0>(), wave, All{});
  if (T > 1) dma_k(tile_at(1), kbuf<1>(), wave, All{});
  wait_dma_barrier();
  gemm_s_only<0, FOLD>(w, ksc(tile_at(0), 0), ksc(tile_at(0), 1));
  if (GROUP_A) softmax<true, FOLD>(w, c, valid_at(0), hh);
  barrier_only();

  auto iter_a = [&](int t, auto par, auto fast) {
    constexpr int PAR = decltype(par)::value;
    constexpr bool FAST = decltype(fast)::value;
    asm volatile("" : "+v"(w.kbase), "+v"(w.kxh), "+v"(w.vbase), "+v"(w.vy));
    const int ts = t + 1 < T ? tile_at(t + 1) : 0;
    if constexpr (FAST) {
      const DmaPlan pl = plan_of(t);
      gemm_phase<PAR, PAR ^ 1, FOLD, true>(w, ksc(ts, 0), ksc(ts, 1), &pl);
    } else {
      gemm_phase<PAR, PAR ^ 1, FOLD>(w, ksc(ts, 0), ksc(ts, 1));
      if (t + 2 < T) dma_k(tile_at(t + 2), kbuf<PAR>(), wave, Half{});
      if (t + 1 < T) dma_v(tile_at(t + 1), vbuf<PAR ^ 1>(), wave, Half{});
    }
    __builtin_amdgcn_sched_barrier(0);   // the GEMM phase's work stays ahead of the softmax
    if (t + 1 < T) softmax<!FAST, FOLD>(w, c, valid_at(t + 1), hh);
    wait_dma_barrier();
  };
  auto iter_b = [&](int t, auto par, auto mask) {
    constexpr int PAR = decltype(par)::value;
    asm volatile("" : "+v"(w.kbase), "+v"(w.kxh), "+v"(w.vbase), "+v"(w.vy));
    softmax<decltype(mask)::value, FOLD>(w, c, valid_at(t), hh);
    __builtin_amdgcn_sched_barrier(0);
    const int ts = t + 1 < T ? tile_at(t + 1) : 0;
    gemm_phase<PAR, PAR ^ 1, FOLD>(w, ksc(ts, 0), ksc(ts, 1));
    wait_dma_barrier();
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using Fast = std::true_type;
  using Slow = std::false_type;
  using Mask = std::true_type;
  using NoMask = std::false_type;
  int t = 0;
  if (GROUP_A) {
    const int nfast = nwhole - 2;
    for (; t + 1 < nfast; t += 2) {
      iter_a(t, P0{}, Fast{});
      iter_a(t + 1, P1{}, Fast{});
    }
    for (; t + 1 < T; t += 2) {
      iter_a(t, P0{}, Slow{});
      iter_a(t + 1, P1{}, Slow{});
    }
    if (t < T) iter_a(t, P0{}, Slow{});
  } else {
    for (; t + 1 < nwhole; t += 2) {
      iter_b(t, P0{}, NoMask{});
      iter_b(t + 1, P1{}, NoMask{});
    }
    for (; t + 1 < T; t += 2) {
      iter_b(t, P0{}, Mask{});
      iter_b(t + 1, P1{}, Mask{});
    }
    if (t < T) iter_b(t, P0{}, Mask{});
  }

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
  if (a.lse && hh == 0) a.lse[((int64_t)b * a.heads_q + hq) * a.seq + tok] = LN2 * (w.m + __builtin_amdgcn_logf(w.l));
}

template <bool FOLD>
__global__ __launch_bounds__(THREADS) void fwd_fp8_kernel(Args a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave < 4) wave_program<true, FOLD>(a, lane, wave);
  else wave_program<false, FOLD>(a, lane, wave);
}

}  // namespace fp8k

}  // namespace nx

using namespace nx;

extern "C" int nxattn_fwd_fp8(const nxattn_fwd_fp8_args* p, hipStream_t stream) {
  using namespace fp8k;
  clear_error();
  if (!p) return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: args is NULL");
  if (p->batch < 0 || p->seq_q < 0 || p->heads_q <= 0 || p->heads_kv <= 0 || p->head_dim <= 0)
    return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: bad sizes");
  if (p->head_dim != D) return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd_fp8: head_dim must be 128, got %d", p->head_dim);
  if (p->batch > NXATTN_MAX_BRANCHES)
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd_fp8: batch %d > %d", p->batch, NXATTN_MAX_BRANCHES);
  if (p->heads_q % p->heads_kv != 0) return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: heads_q %% heads_kv != 0");
  if (p->heads_q > 4096) return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd_fp8: heads_q > 4096");
  if (!(p->scale == p->scale) || std::isinf(p->scale)) return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: scale is not finite");
  bool any_prefix = false;
  for (int b = 0; b < p->batch; ++b) {
    if (p->prefix_len[b] < 0) return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: prefix_len[%d] < 0", b);
    const bool has = p->prefix_len[b] > 0;
    if (has != (p->prefix_k8[b] != nullptr) || has != (p->prefix_v[b] != nullptr))
      return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: prefix_k8[%d] / prefix_v[%d] must be non-NULL iff prefix_len > 0", b, b);
    if ((int64_t)p->prefix_len[b] + p->seq_q > INT32_MAX)
      return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd_fp8: prefix_len[%d] + seq_q overflows int32", b);
    any_prefix |= has;
  }
  if (p->batch == 0 || p->seq_q == 0) return NXATTN_OK;
  if (!p->q8 || !p->k8 || !p->v || !p->o || !p->q_exp || !p->k_exp || (any_prefix && !p->prefix_k_exp))
    return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: NULL pointer");
  for (int i = 0; i < 3; ++i) {
    if (p->v_strides[i] < 0 || p->o_strides[i] < 0) return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: negative stride");
    if ((p->v_strides[i] * 2) % 16 != 0 || (p->o_strides[i] * 2) % 16 != 0)
      return fail(NXATTN_ERR_ALIGN, "nxattn_fwd_fp8: strides must be multiples of 16 bytes");
  }
  if (!aligned16(p->q8) || !aligned16(p->k8) || !aligned16(p->v) || !aligned16(p->o))
    return fail(NXATTN_ERR_ALIGN, "nxattn_fwd_fp8: q8/k8/v/o must be 16-byte aligned");
  for (int b = 0; b < p->batch; ++b)
    if ((p->prefix_k8[b] && !aligned16(p->prefix_k8[b])) || (p->prefix_v[b] && !aligned16(p->prefix_v[b])))
      return fail(NXATTN_ERR_ALIGN, "nxattn_fwd_fp8: prefix_k8[%d] / prefix_v[%d] misaligned", b, b);
  if (p->lse && (reinterpret_cast<uintptr_t>(p->lse) & 3u)) return fail(NXATTN_ERR_ALIGN, "nxattn_fwd_fp8: lse misaligned");
  // outputs must not overlap any input
  const int64_t B = p->batch, S = p->seq_q, Hq = p->heads_q, Hkv = p->heads_kv;
  const int64_t ob = ((B - 1) * p->o_strides[0] + (S - 1) * p->o_strides[1] + (Hq - 1) * p->o_strides[2] + D) * 2;
  const int64_t vb = ((B - 1) * p->v_strides[0] + (S - 1) * p->v_strides[1] + (Hkv - 1) * p->v_strides[2] + D) * 2;
  const int64_t lb = p->lse ? B * Hq * S * 4 : 0;
  struct Span { const void* ptr; int64_t n; };
  Span ins[6 + 2 * NXATTN_MAX_BRANCHES] = {{p->q8, B * S * Hq * D}, {p->k8, B * S * Hkv * D}, {p->v, vb},
                                           {p->q_exp, B * Hq}, {p->k_exp, B * Hkv},
                                           {p->prefix_k_exp, any_prefix ? B * Hkv : 0}};
  int nin = 6;
  for (int b = 0; b < p->batch; ++b) {
    ins[nin++] = Span{p->prefix_k8[b], (int64_t)p->prefix_len[b] * Hkv * D};
    ins[nin++] = Span{p->prefix_v[b], (int64_t)p->prefix_len[b] * Hkv * D * 2};
  }
  for (int i = 0; i < nin; ++i)
    if (ins[i].ptr && (overlaps(p->o, ob, ins[i].ptr, ins[i].n) || (p->lse && overlaps(p->lse, lb, ins[i].ptr, ins[i].n))))
      return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: o or lse overlaps an input");
  if (p->lse && overlaps(p->lse, lb, p->o, ob)) return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: lse overlaps o");

  Args a;
  a.q8 = p->q8; a.k8 = p->k8; a.v = static_cast<const uint16_t*>(p->v); a.o = static_cast<uint16_t*>(p->o);
  a.q_exp = p->q_exp; a.k_exp = p->k_exp; a.pk_exp = p->prefix_k_exp ? p->prefix_k_exp : p->k_exp;
  a.vs0 = p->v_strides[0]; a.vs1 = p->v_strides[1]; a.vs2 = p->v_strides[2];
  a.os0 = p->o_strides[0]; a.os1 = p->o_strides[1]; a.os2 = p->o_strides[2];
  for (int b = 0; b < NXATTN_MAX_BRANCHES; ++b) {
    const bool in = b < p->batch;
    a.pk8[b] = in ? p->prefix_k8[b] : nullptr;
    a.pv[b] = in ? static_cast<const uint16_t*>(p->prefix_v[b]) : nullptr;
    a.plen[b] = in ? p->prefix_len[b] : 0;
  }
  a.batch = p->batch; a.seq = p->seq_q; a.heads_q = p->heads_q; a.heads_kv = p->heads_kv;
  a.group = p->heads_q / p->heads_kv;
  a.nchunks = (p->seq_q + 31) / 32;
  const int64_t nqb = (int64_t)a.group * a.nchunks;
  const int64_t wpg = (nqb + WAVES - 1) / WAVES;
  const int64_t total = wpg * p->heads_kv * p->batch;
  if (total > INT32_MAX / 2) return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd_fp8: problem too large");
  a.nqb = (int)nqb; a.wg_per_group = (int)wpg; a.total_wg = (int)total;
  const float scale = p->scale > 0.f ? p->scale : 1.0f / std::sqrt((float)D);
  a.c = scale * LOG2E;
  a.lse = p->lse;
  if (p->q_folded)
    fwd_fp8_kernel<true><<<a.total_wg, THREADS, 0, stream>>>(a);
  else
    fwd_fp8_kernel<false><<<a.total_wg, THREADS, 0, stream>>>(a);
  return check_launch("nxattn_fwd_fp8");
}
