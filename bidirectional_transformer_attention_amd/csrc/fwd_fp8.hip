// Fused non-causal GQA attention with an FP8 score GEMM: q and k are OCP E4M3 codes with
// one power-of-two scale per (branch, head) or, with BLOCK, one per run of 32 head_dim
// elements of a row; v and the output are bf16, head_dim 128. The scores come from
// v_mfma_scale_f32_32x32x64_f8f6f4, whose per-lane E8M0 scale operands apply the
// (power-of-two) dequantisation exactly inside the matrix core: for row (or column) r,
// lane r's scale covers bytes 0-15 of lanes r and r + 32 and lane r + 32's scale bytes
// 16-31 of both. Per slice, the key rows take the scale of the tensor they come from
// (prefix or own keys) and the query columns that of their head; with BLOCK each lane
// takes the scale of the run whose codes that placement puts under it. Softmax, P (bf16) and O^T += V^T P^T are the bf16
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
#include <algorithm>
#include <cmath>
#include <cstring>
#include <type_traits>

#include "nx_internal.h"
#include "rope_turn.h"

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
  const uint8_t* q_sc; const uint8_t* k_sc;     // BLOCK: E8M0 codes [.., heads, 4] per row
  const uint8_t* pk_sc[NXATTN_MAX_BRANCHES];
  int64_t vs0, vs1, vs2, os0, os1, os2;
  const uint8_t* pk8[NXATTN_MAX_BRANCHES];
  const uint16_t* pv[NXATTN_MAX_BRANCHES];
  int32_t plen[NXATTN_MAX_BRANCHES];
  int32_t batch, seq, heads_q, heads_kv, group, nchunks, nqb, wg_per_group, total_wg;
  float c;  // scale * log2(e)
  float* lse;
  // QROPE: q as bf16 (element strides), rotated, folded and block-quantized on load
  const uint16_t* q;
  int64_t qs0, qs1, qs2;
  RopeQ rq[NXATTN_MAX_BRANCHES];
  uint8_t* q8_out;      // QROPE, optional: the codes [B, S, Hq, 128] and run scales [B, S, Hq, 4]
  uint8_t* qsc_out;     // formed on load
  // branch pairs: out[i, h] = bf16(fma(guidance, c - u, u)) with c, u the bf16 outputs of
  // branches 0 and 1 (o may then be NULL: branch outputs not stored)
  uint16_t* cfg;
  int64_t cs0, cs1;
  float guidance;
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
// The wait is the builtin (every counter to zero), not inline asm: the compiler's own wait
// insertion sees it and knows that the tile loads and the block-scale loads issued before
// it have landed, so it adds no waits for them after the barrier (behind an asm wait it
// assumed them outstanding and waited on the next iteration's fresh scale loads).
__device__ __forceinline__ void wait_dma_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// A wave-uniform pointer stated as such (read back from the first lane), so that the buffer
// descriptors built from it stay in scalar registers: under the register pressure of the
// branch-pair kernels the compiler otherwise computed some in vector registers and
// wrapped every tile load in a loop over the distinct values.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// LDS: K (fp8) and V (bf16) tiles, double-buffered, as four distinct objects
__shared__ __attribute__((aligned(1024))) uint8_t lds_k0[KTILEB];
__shared__ __attribute__((aligned(1024))) uint8_t lds_k1[KTILEB];
__shared__ __attribute__((aligned(1024))) uint8_t lds_v0[VTILEB];
__shared__ __attribute__((aligned(1024))) uint8_t lds_v1[VTILEB];
template <int PAR> __device__ __forceinline__ uint8_t* kbuf() { return PAR ? lds_k1 : lds_k0; }
template <int PAR> __device__ __forceinline__ uint8_t* vbuf() { return PAR ? lds_v1 : lds_v0; }
// BLOCK: the four run scales (E8M0 codes) of each key row of a K tile, beside the tile
__shared__ __attribute__((aligned(256))) uint8_t lds_s0[BN * 4];
__shared__ __attribute__((aligned(256))) uint8_t lds_s1[BN * 4];
// Branch pairs: the first branch's rounded output, held until the second branch's epilogue
// (entry (wave, j, lane)); only the pair kernels use it. 16-byte aligned so that it is
// placed after the tile buffers, whose LDS offsets then fit the reads' immediate field.
__shared__ __attribute__((aligned(16))) u32x2 lds_keep[WAVES * 16 * 64];
template <int PAR> __device__ __forceinline__ uint8_t* sbuf() { return PAR ? lds_s1 : lds_s0; }

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
  v8i q8[2];          // Q^T operand, k-step ks: codes Q[row][64ks + 16hh + 32e .. +15], e = 0, 1
  f32x16 o[4];        // O^T accumulators, d-block db
  f32x16 s[2];        // S^T accumulators of the tile being scored (2 key blocks of 32)
  bf16x8 p[4];        // P^T operand of the tile being accumulated
  float m, l;
  bool primed;        // FOLD: a first tile has set m (weights may be taken before the max)
  float thr;          // FOLD: row max of the shifted scores above which m moves (-inf before
                      // the first tile); else (m + RESCALE_T) / c on raw scores
  f32x16 negm;        // FOLD: -m in every register, the score accumulators' start value
  int kbase, kxh;     // K fragment (kb, ks, half e): kbase + kb*32*KROWB + ((64ks + 32e) ^ kxh)
  int vbase, vy;      // V^T fragment of d-block db at vbase + (64db ^ vy)
  int qsc;            // E8M0 scale of the B operand: the q head's, or (BLOCK) the row's run
                      // scales shifted so that k-step ks finds its own in byte 2ks
  uint32_t qrun;      // QROPE: the row's four run scales in run order (for q_scales_out)
};

// Byte of the scale operands that k-step ks uses: per slice the value itself (byte 0);
// with BLOCK byte 2ks of a row's four run scales shifted right by 8 * (lane half), i.e.
// run 2ks + half, the run whose codes the lane's scale covers in that step
template <bool BLOCK, int KS>
constexpr int scale_byte() { return BLOCK ? 2 * KS : 0; }

__device__ __forceinline__ u32x4 lds_read_b128(const uint8_t* smem, int byte) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>((const lds_u8*)smem + byte);
}
__device__ __forceinline__ bf16x4 lds_read_tr(const uint8_t* smem, int byte) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)((const lds_u8*)smem + byte));
}
__device__ __forceinline__ v8i kfrag(const uint8_t* ksm, const Wave& w, int kb, int ks) {
  const int base = w.kbase + kb * 32 * KROWB;
  const u32x4 a = lds_read_b128(ksm, base + ((64 * ks) ^ w.kxh));
  const u32x4 b = lds_read_b128(ksm, base + ((64 * ks + 32) ^ w.kxh));
  return __builtin_bit_cast(v8i, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
// formats 0 / 0: E4M3 for both operands; the E8M0 scales are byte SEL of ksc / qsc (op_sel
// picks the byte: measured)
template <int SEL>
__device__ __forceinline__ f32x16 mfma_s(v8i k, v8i q, f32x16 acc, int ksc, int qsc) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k, q, acc, 0, 0, SEL, ksc, SEL, qsc);
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

template <int VPAR, int KPAR, bool FOLD, bool BLOCK, bool DMA = false>
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
      if (ks == 0)
        w.s[kb] = mfma_s<scale_byte<BLOCK, 0>()>(kf[j], w.q8[0], FOLD ? w.negm : f32x16{}, kb ? ksc1 : ksc0, w.qsc);
      else
        w.s[kb] = mfma_s<scale_byte<BLOCK, 1>()>(kf[j], w.q8[1], w.s[kb], kb ? ksc1 : ksc0, w.qsc);
    }
  }
  sched8_reads<0, DIST>();
  sched8_steps<0, DMA>();
}

// S^T only (prologue).
template <int KPAR, bool FOLD, bool BLOCK>
__device__ __forceinline__ void gemm_s_only(Wave& w, int ksc0, int ksc1) {
  const uint8_t* ksm = kbuf<KPAR>();
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
    w.s[kb] = mfma_s<scale_byte<BLOCK, 0>()>(kfrag(ksm, w, kb, 0), w.q8[0], FOLD ? w.negm : f32x16{},
                                             kb ? ksc1 : ksc0, w.qsc);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
    w.s[kb] = mfma_s<scale_byte<BLOCK, 1>()>(kfrag(ksm, w, kb, 1), w.q8[1], w.s[kb], kb ? ksc1 : ksc0, w.qsc);
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
      // the score accumulators' start block follows m; kept between rescales
#pragma unroll
      for (int i = 0; i < 16; ++i) w.negm[i] = -w.m;
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
  // the two partial sums start from the first weights (the same values as 0 + p, since a
  // weight is never -0, without the two adds)
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
        l0 = (kb | hs | e) ? l0 + p0 : p0;
        l1 = (kb | hs | e) ? l1 + p1 : p1;
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
  } else {
    max_update<FOLD>(w, c);
    w.l += weights<FOLD>(w, c);
  }
}

// QROPE: this lane's q codes and run scales formed in registers. The lane holds dims
// 64ks + 32e + 16hh + i (k-step ks, half e, i < 16) of its query row, as bf16. They are
// rotated with the branch's RoPE (RopeTurns; half-split pairs (j, j + 64) are ks 0 and 1
// at the same (e, i), adjacent pairs neighbouring i) and multiplied by c, both in fp32
// (no bf16 rounding in between). Run 2ks + e (32 dims) is half e of k-step ks in both lane
// halves, so its maximum is the larger of this lane's and its partner's (lane ^ 32), and
// both form the same exponent (smallest e with max <= 448 * 2^e, at least -127); the codes
// are the values times 2^-e rounded to nearest even E4M3. The lane's scale for k-step ks is
// that of run 2ks + hh, in byte 2ks of w.qsc (the layout the score MFMAs' op_sel reads).
// The lane's bf16 q values (loaded at the start of the work item, before the first tiles'
// DMA, so that waiting for them never waits for the DMA): raw[ks][e][h] holds dims
// 64ks + 32e + 16hh + 8h .. +7.
struct QRaw {
  u32x4 raw[2][2][2];
};
__device__ __forceinline__ QRaw q_rope_load(const Args& a, int b, int tokc, int hq, int hh) {
  const uint16_t* qrow = a.q + b * a.qs0 + (int64_t)tokc * a.qs1 + (int64_t)hq * a.qs2;
  QRaw r;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8)
        r.raw[ks][e][h8] = *reinterpret_cast<const u32x4*>(qrow + 64 * ks + 32 * e + 16 * hh + 8 * h8);
  return r;
}

__device__ __forceinline__ void q_rope_quantize(Wave& w, const Args& a, const QRaw& qr, int b, int tokc,
                                                int lane) {
  const int hh = lane >> 5;
  float x[2][2][16];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const u32x4 v = qr.raw[ks][e][h8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[ks][e][8 * h8 + 2 * k] = __uint_as_float(v[k] << 16);
          x[ks][e][8 * h8 + 2 * k + 1] = __uint_as_float(v[k] & 0xffff0000u);
        }
      }
  const RopeQ& r = a.rq[b];
  const RopeTurns rt(r, tokc, lane);
  const float c = a.c;
  if (!r.interleaved) {
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float sn, cs;
        rt.turn(32 * e + 16 * hh + i, sn, cs);
        const float xa = x[0][e][i], xb = x[1][e][i];
        x[0][e][i] = (xa * cs - xb * sn) * c;
        x[1][e][i] = (xa * sn + xb * cs) * c;
      }
  } else {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          float sn, cs;
          rt.turn((64 * ks + 32 * e + 16 * hh + i) >> 1, sn, cs);
          const float xa = x[ks][e][i], xb = x[ks][e][i + 1];
          x[ks][e][i] = (xa * cs - xb * sn) * c;
          x[ks][e][i + 1] = (xa * sn + xb * cs) * c;
        }
  }
  int sc[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    u32x4 cw[2];        // half e of the k-step's operand: bytes 16e .. 16e + 15
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(x[ks][e][i]));
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(m), __float_as_int(m), false, false);
      m = __builtin_fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1]));
      const int ex = fp8_exponent(m);
      sc[ks][e] = ex + 127;
      const float inv = exp2_neg(ex);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        int cc = __builtin_amdgcn_cvt_pk_fp8_f32(x[ks][e][4 * k] * inv, x[ks][e][4 * k + 1] * inv, 0, false);
        cc = __builtin_amdgcn_cvt_pk_fp8_f32(x[ks][e][4 * k + 2] * inv, x[ks][e][4 * k + 3] * inv, cc, true);
        cw[e][k] = (uint32_t)cc;
      }
    }
    w.q8[ks] = __builtin_bit_cast(v8i, __builtin_shufflevector(cw[0], cw[1], 0, 1, 2, 3, 4, 5, 6, 7));
  }
  w.qsc = (hh ? sc[0][1] : sc[0][0]) | ((hh ? sc[1][1] : sc[1][0]) << 16);
  w.qrun = (uint32_t)sc[0][0] | ((uint32_t)sc[0][1] << 8) | ((uint32_t)sc[1][0] << 16) | ((uint32_t)sc[1][1] << 24);
}

// PAIR: the workgroup runs branch 0 and then branch 1 of its query blocks (two inlined
// passes), keeps branch 0's rounded output in LDS and writes the guidance combination.
template <bool GROUP_A, bool FOLD, bool BLOCK, bool QROPE, bool PAIR>
__device__ __forceinline__ void wave_program(const Args& a, int lane, int wave) {
  const int n = lane & 31, hh = lane >> 5;
  const int wg = remap_xcd(blockIdx.x, a.total_wg);
  const int grp = wg / a.wg_per_group;
  const int g = PAIR ? grp : grp / a.batch, b0 = PAIR ? 0 : grp % a.batch;
  const int qb = (wg % a.wg_per_group) * WAVES + wave;
  const bool active = qb < a.nqb;
  const int hq = g * a.group + (active ? qb / a.nchunks : 0);
  const int tok = (active ? qb % a.nchunks : 0) * 32 + n;
  const int tokc = tok < a.seq ? tok : a.seq - 1;
  auto pass = [&](auto bic) {
  constexpr int bi = decltype(bic)::value;
  const int b = PAIR ? bi : b0;
  const int P = a.plen[b];
  const int Skv = P + a.seq;
  const int T = (Skv + BN - 1) / BN;
  const float c = a.c;
  // E8M0 scales, per slice: key rows of the prefix / own keys, and this wave's q head
  const int sc_own = BLOCK ? 0 : 127 + (int)a.k_exp[b * a.heads_kv + g];
  const int sc_pre = BLOCK ? 0 : (P > 0 ? 127 + (int)a.pk_exp[b * a.heads_kv + g] : sc_own);

  Wave w;
  QRaw qraw;
  if constexpr (QROPE) {
    qraw = q_rope_load(a, b, tokc, hq, hh);
  } else {
    const uint8_t* qrow = a.q8 + (((int64_t)b * a.seq + tokc) * a.heads_q + hq) * D;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(qrow + 64 * ks + 16 * hh);
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(qrow + 64 * ks + 16 * hh + 32);
      w.q8[ks] = __builtin_bit_cast(v8i, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
  // QROPE: the codes formed from q (after the first tiles' DMA is issued) and, if asked
  // for, copied out
  auto q_rope_codes = [&]() {
    q_rope_quantize(w, a, qraw, b, tokc, lane);
    if (a.q8_out && active && tok < a.seq) {
      // the codes and run scales formed here, for callers that check or reuse them
      const int64_t row = ((int64_t)b * a.seq + tok) * a.heads_q + hq;
      uint8_t* orow = a.q8_out + row * D;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const v8i v = w.q8[ks];
        *reinterpret_cast<u32x4*>(orow + 64 * ks + 16 * hh) = u32x4{(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]};
        *reinterpret_cast<u32x4*>(orow + 64 * ks + 32 + 16 * hh) =
            u32x4{(uint32_t)v[4], (uint32_t)v[5], (uint32_t)v[6], (uint32_t)v[7]};
      }
      if (hh == 0) *reinterpret_cast<uint32_t*>(a.qsc_out + row * 4) = w.qrun;
    }
  };
  if constexpr (QROPE) {
  } else if constexpr (BLOCK) {
    const uint32_t qs = *reinterpret_cast<const uint32_t*>(a.q_sc + (((int64_t)b * a.seq + tokc) * a.heads_q + hq) * 4);
    w.qsc = (int)(qs >> (8 * hh));
  } else {
    w.qsc = 127 + (int)a.q_exp[b * a.heads_q + hq];
  }
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
  // 4ks + 2e + hh at slot chunk ^ (n & 7): byte n*KROWB + ((64ks + 32e) ^ (16hh ^ 16(n&7))).
  // The matrix core scales bytes 0-15 of lanes r and r + 32 (one 32-wide k block) by lane
  // r's scale and bytes 16-31 of both by lane r + 32's (measured), so half e of k-step ks
  // holds 16 codes of run 2ks + e: lane half hh its elements 16hh .. 16hh + 15, and the
  // lane's scale is that of run 2ks + hh. q's fragments are placed the same way.
  w.kbase = n * KROWB;
  w.kxh = (16 * hh) ^ (16 * (n & 7));
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
  // E8M0 scale of this lane's key row in key block kb of tile t (per slice)
  auto ksc = [&](int t, int kb) { return t * BN + kb * 32 + n < P ? sc_pre : sc_own; };
  // BLOCK: the four run scales of the 64 key rows of a tile travel into LDS with the K
  // tile (sbuf<p> beside kbuf<p>): one 4-byte direct-to-LDS load per lane (lane = row)
  // from wave 0, instead of every wave gathering its rows from memory (which cost 9 % at
  // the 1K DiT shape). A whole tile lies inside the prefix or inside the own keys, so its
  // rows are one buffer (uniform), a uniform row offset and the lane's row; the
  // straddling and the ragged tile take per-lane addresses (rows past the keys read the
  // last key's: their scores are masked).
  const uint8_t* ksc_pre = BLOCK && P > 0 ? a.pk_sc[b] + (int64_t)g * 4 : nullptr;
  const uint8_t* ksc_own = BLOCK ? a.k_sc + ((int64_t)b * a.seq * a.heads_kv + g) * 4 : nullptr;
  const uint32_t ksc_row = (uint32_t)a.heads_kv * 4;               // bytes between key rows
  const uint32_t ksc_lane = (uint32_t)lane * ksc_row;
  const __amdgpu_buffer_rsrc_t ksr_own =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(const_cast<uint8_t*>(ksc_own)), 0, BUF_RECORDS, BUF_FLAGS);
  const __amdgpu_buffer_rsrc_t ksr_pre =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(const_cast<uint8_t*>(P > 0 ? ksc_pre : ksc_own)), 0, BUF_RECORDS,
                                        BUF_FLAGS);
  // the scales of the tile at position pos into dst (wave 0 only; WHOLE: pos < nwhole)
  auto dma_s = [&](int pos, uint8_t* dst, auto whole) {
    if constexpr (BLOCK) {
      if (wave != 0) return;
      const int t = tile_at(pos);
      if (decltype(whole)::value || pos < nwhole) {
        const int j0 = t * BN;
        const bool pre = j0 < P;
        const uint32_t soff = (uint32_t)(pre ? j0 : j0 - P) * ksc_row;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(pre ? ksr_pre : ksr_own,
                                                 (__attribute__((address_space(3))) void*)(lds_u8*)dst, 4, ksc_lane,
                                                 soff, 0, 0);
      } else {
        int j = t * BN + lane;
        j = j < Skv ? j : Skv - 1;
        const uint8_t* src = j < P ? ksc_pre + (int64_t)j * ksc_row : ksc_own + (int64_t)(j - P) * ksc_row;
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds_u8*)dst, 4, 0, 0);
      }
    }
  };
  // scale operands of key block kb for the tile in sbuf<PAR> (BLOCK: this lane's row's
  // four run scales, shifted right by 8 * (lane half)) or of tile t (per slice)
  auto kop = [&](auto par, int t, int kb) -> int {
    if constexpr (BLOCK) {
      const uint32_t v = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(
          (const lds_u8*)sbuf<decltype(par)::value>() + (32 * kb + n) * 4);
      return (int)(v >> (8 * hh));
    } else {
      return ksc(t, kb);
    }
  };

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
    pl.krsrc = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(const_cast<uint8_t*>(kb_)), 0, BUF_RECORDS, BUF_FLAGS);
    pl.vrsrc = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(const_cast<uint16_t*>(vb_)), 0, BUF_RECORDS, BUF_FLAGS);
    pl.krs = (uint32_t)(8 * krow);
    pl.vrs = (uint32_t)(8 * (vp ? pvrow : vs1));
    pl.koff = koff;
    pl.voff = vp ? voff_pre : voff_own;
    pl.ws = wave;
    return pl;
  };

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using Whole = std::true_type;
  using AnyTile = std::false_type;

  // ---- prologue (as in the bf16 kernel)
  dma_s(0, sbuf<0>(), AnyTile{});
  if (T > 1) dma_s(1, sbuf<1>(), AnyTile{});
  dma_k(tile_at(0), kbuf<0>(), wave, All{});
  dma_v(tile_at(0), vbuf<0>(), wave, All{});
  if (T > 1) dma_k(tile_at(1), kbuf<1>(), wave, All{});
  if constexpr (QROPE) q_rope_codes();    // while the first tiles are in flight
  wait_dma_barrier();
  gemm_s_only<0, FOLD, BLOCK>(w, kop(P0{}, tile_at(0), 0), kop(P0{}, tile_at(0), 1));
  if (GROUP_A) softmax<true, FOLD>(w, c, valid_at(0), hh);
  barrier_only();

  auto iter_a = [&](int t, auto par, auto fast) {
    constexpr int PAR = decltype(par)::value;
    constexpr bool FAST = decltype(fast)::value;
    asm volatile("" : "+v"(w.kbase), "+v"(w.kxh), "+v"(w.vbase), "+v"(w.vy));
    const int ts = t + 1 < T ? tile_at(t + 1) : 0;
    // tile t+1 (scored now) sits in kbuf / sbuf PAR ^ 1; tile t+2 goes to PAR
    using KP = std::integral_constant<int, PAR ^ 1>;
    const int s0 = kop(KP{}, ts, 0), s1 = kop(KP{}, ts, 1);
    if constexpr (FAST) {
      dma_s(t + 2, sbuf<PAR>(), Whole{});
      const DmaPlan pl = plan_of(t);
      gemm_phase<PAR, PAR ^ 1, FOLD, BLOCK, true>(w, s0, s1, &pl);
    } else {
      if (t + 2 < T) dma_s(t + 2, sbuf<PAR>(), AnyTile{});
      gemm_phase<PAR, PAR ^ 1, FOLD, BLOCK>(w, s0, s1);
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
    using KP = std::integral_constant<int, PAR ^ 1>;
    gemm_phase<PAR, PAR ^ 1, FOLD, BLOCK>(w, kop(KP{}, ts, 0), kop(KP{}, ts, 1));
    wait_dma_barrier();
  };
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
  uint16_t* orow = a.o ? a.o + b * a.os0 + (int64_t)tok * a.os1 + (int64_t)hq * a.os2 : nullptr;
  uint16_t* crow = PAIR ? a.cfg + (int64_t)tok * a.cs0 + (int64_t)hq * a.cs1 : nullptr;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = 32 * db + 8 * i4 + 4 * hh;
      const u32x2 r = u32x2{pack_bf16x2(w.o[db][4 * i4] * inv, w.o[db][4 * i4 + 1] * inv),
                            pack_bf16x2(w.o[db][4 * i4 + 2] * inv, w.o[db][4 * i4 + 3] * inv)};
      if (!PAIR || orow) *reinterpret_cast<u32x2*>(orow + d) = r;
      if constexpr (PAIR) {
        __attribute__((address_space(3))) u32x2* kp =
            (__attribute__((address_space(3))) u32x2*)&lds_keep[(wave * 16 + 4 * db + i4) * 64 + lane];
        if constexpr (bi == 0) {
          *kp = r;
        } else {
          // the arithmetic of the combine pass on the two rounded outputs: c = branch 0,
          // u = branch 1, fma(guidance, c - u, u) in fp32, rounded to nearest even
          const u32x2 cv = *kp;
          u32x2 o2;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t cw = cv[e], uw = r[e];
            const float c0 = __uint_as_float(cw << 16), c1 = __uint_as_float(cw & 0xffff0000u);
            const float u0 = __uint_as_float(uw << 16), u1 = __uint_as_float(uw & 0xffff0000u);
            o2[e] = pack_bf16x2(__builtin_fmaf(a.guidance, c0 - u0, u0), __builtin_fmaf(a.guidance, c1 - u1, u1));
          }
          *reinterpret_cast<u32x2*>(crow + d) = o2;
        }
      }
    }
  if (a.lse && hh == 0) a.lse[((int64_t)b * a.heads_q + hq) * a.seq + tok] = LN2 * (w.m + __builtin_amdgcn_logf(w.l));
  };
  if constexpr (PAIR) {
    pass(std::integral_constant<int, 0>{});
    // the second branch's first loads refill buffers that group B may still be reading
    // for the first branch's last tile
    barrier_only();
    pass(std::integral_constant<int, 1>{});
  } else {
    pass(std::integral_constant<int, 0>{});
  }
}

template <bool FOLD, bool BLOCK, bool QROPE, bool PAIR>
__global__ __launch_bounds__(THREADS) void fwd_fp8_kernel(Args a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave < 4) wave_program<true, FOLD, BLOCK, QROPE, PAIR>(a, lane, wave);
  else wave_program<false, FOLD, BLOCK, QROPE, PAIR>(a, lane, wave);
}

// launch of the instantiation that matches the call
template <bool PAIR>
static void launch_fp8(const Args& a, bool qrope, bool block, bool folded, hipStream_t stream) {
  if (qrope) {
    fwd_fp8_kernel<true, true, true, PAIR><<<a.total_wg, THREADS, 0, stream>>>(a);
  } else if (block) {
    if (folded)
      fwd_fp8_kernel<true, true, false, PAIR><<<a.total_wg, THREADS, 0, stream>>>(a);
    else
      fwd_fp8_kernel<false, true, false, PAIR><<<a.total_wg, THREADS, 0, stream>>>(a);
  } else {
    if (folded)
      fwd_fp8_kernel<true, false, false, PAIR><<<a.total_wg, THREADS, 0, stream>>>(a);
    else
      fwd_fp8_kernel<false, false, false, PAIR><<<a.total_wg, THREADS, 0, stream>>>(a);
  }
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
  // q: codes (q8 with q_exp, or with q_scales) or, with q_rope, bf16 q rotated, folded and
  // block-quantized on load; keys: block scales (k_scales and each prefix's scales) with
  // q_scales or q_rope, one exponent per slice otherwise
  const bool qrope = p->q_rope != nullptr;
  const bool block = p->q_scales != nullptr || qrope;
  if (qrope && (p->q8 || p->q_scales || p->q_exp))
    return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: q_rope takes bf16 q: q8, q_scales and q_exp must be NULL");
  if (qrope && p->q_folded)
    return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: q_rope folds the softmax scale itself: q_folded must be 0");
  if (!qrope && p->q) return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: q given without q_rope");
  if ((p->q8_out != nullptr) != (p->q_scales_out != nullptr) || (!qrope && p->q8_out))
    return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: q8_out and q_scales_out go together, with q_rope only");
  if (p->q8_out && (!aligned16(p->q8_out) || (reinterpret_cast<uintptr_t>(p->q_scales_out) & 3u)))
    return fail(NXATTN_ERR_ALIGN, "nxattn_fwd_fp8: q8_out must be 16-byte and q_scales_out 4-byte aligned");
  if (block && (p->q_exp || p->k_exp || p->prefix_k_exp))
    return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: block scales exclude q_exp, k_exp and prefix_k_exp");
  if (!block && p->k_scales) return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: k_scales given without q_scales");
  bool any_prefix = false;
  for (int b = 0; b < p->batch; ++b) {
    if (p->prefix_len[b] < 0) return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: prefix_len[%d] < 0", b);
    const bool has = p->prefix_len[b] > 0;
    if (has != (p->prefix_k8[b] != nullptr) || has != (p->prefix_v[b] != nullptr))
      return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: prefix_k8[%d] / prefix_v[%d] must be non-NULL iff prefix_len > 0", b, b);
    if ((block && has) != (p->prefix_k_scales[b] != nullptr))
      return fail(NXATTN_ERR_INVALID,
                  "nxattn_fwd_fp8: prefix_k_scales[%d] must be non-NULL iff block scales and prefix_len > 0", b);
    if ((int64_t)p->prefix_len[b] + p->seq_q > INT32_MAX)
      return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd_fp8: prefix_len[%d] + seq_q overflows int32", b);
    any_prefix |= has;
  }
  // branch pairs: the guidance combination written by the attention kernel itself
  const bool pair = p->cfg_out != nullptr;
  if (pair) {
    if (p->batch != 2) return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: cfg_out needs batch 2 (cond, uncond), got %d", p->batch);
    if (!(p->guidance == p->guidance) || std::isinf(p->guidance))
      return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: guidance is not finite");
    for (int i = 0; i < 2; ++i) {
      if (p->cfg_strides[i] < 0) return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: negative cfg stride");
      if (!stride16(p->cfg_strides[i], 2))
        return fail(NXATTN_ERR_ALIGN, "nxattn_fwd_fp8: cfg stride %lld is not a multiple of 16 bytes", (long long)p->cfg_strides[i]);
    }
    if (!aligned16(p->cfg_out)) return fail(NXATTN_ERR_ALIGN, "nxattn_fwd_fp8: cfg_out must be 16-byte aligned");
  }
  if (p->batch == 0 || p->seq_q == 0) return NXATTN_OK;
  if (!(qrope ? p->q : p->q8) || !p->k8 || !p->v || (!p->o && !pair))
    return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: NULL pointer");
  if (block ? !p->k_scales : (!p->q_exp || !p->k_exp || (any_prefix && !p->prefix_k_exp)))
    return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: NULL pointer (exponents or scales)");
  if (block) {
    // the key-scale rows of a whole tile are read with 32-bit buffer offsets
    int64_t rows = p->seq_q;
    for (int b = 0; b < p->batch; ++b) rows = std::max<int64_t>(rows, p->prefix_len[b]);
    if (rows * p->heads_kv * 4 > INT32_MAX)
      return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd_fp8: block scales of one branch exceed 2 GiB");
    auto al4 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 3u) == 0; };
    bool ok = al4(p->q_scales) && al4(p->k_scales);
    for (int b = 0; b < p->batch; ++b) ok = ok && al4(p->prefix_k_scales[b]);
    if (!ok) return fail(NXATTN_ERR_ALIGN, "nxattn_fwd_fp8: scales must be 4-byte aligned");
  }
  for (int i = 0; i < 3; ++i) {
    const int64_t os = p->o ? p->o_strides[i] : 0;
    if (p->v_strides[i] < 0 || os < 0) return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: negative stride");
    if (!stride16(p->v_strides[i], 2) || !stride16(os, 2))
      return fail(NXATTN_ERR_ALIGN, "nxattn_fwd_fp8: strides must be multiples of 16 bytes");
  }
  // V tiles (64 rows) are fetched through raw buffers with 32-bit byte offsets
  if (p->v_strides[1] > INT32_MAX / (2 * KEY_TILE))
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd_fp8: v token stride %lld elements spans 2 GiB or more per %d rows",
                (long long)p->v_strides[1], KEY_TILE);
  if (!aligned16(qrope ? p->q : p->q8) || !aligned16(p->k8) || !aligned16(p->v) || (p->o && !aligned16(p->o)))
    return fail(NXATTN_ERR_ALIGN, "nxattn_fwd_fp8: q8 (or q)/k8/v/o must be 16-byte aligned");
  if (qrope)
    for (int i = 0; i < 3; ++i) {
      if (p->q_strides[i] < 0) return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: negative stride");
      if (!stride16(p->q_strides[i], 2)) return fail(NXATTN_ERR_ALIGN, "nxattn_fwd_fp8: strides must be multiples of 16 bytes");
    }
  for (int b = 0; b < p->batch; ++b)
    if ((p->prefix_k8[b] && !aligned16(p->prefix_k8[b])) || (p->prefix_v[b] && !aligned16(p->prefix_v[b])))
      return fail(NXATTN_ERR_ALIGN, "nxattn_fwd_fp8: prefix_k8[%d] / prefix_v[%d] misaligned", b, b);
  if (p->lse && (reinterpret_cast<uintptr_t>(p->lse) & 3u)) return fail(NXATTN_ERR_ALIGN, "nxattn_fwd_fp8: lse misaligned");
  // outputs must not overlap any input
  const int64_t B = p->batch, S = p->seq_q, Hq = p->heads_q, Hkv = p->heads_kv;
  const int64_t cst[3] = {0, p->cfg_strides[0], p->cfg_strides[1]};
  const int64_t ob = p->o ? span_bytes(p->o_strides, B, S, Hq, D, 2) : 0;
  const int64_t cb = pair ? span_bytes(cst, 1, S, Hq, D, 2) : 0;
  const int64_t vb = span_bytes(p->v_strides, B, S, Hkv, D, 2);
  const int64_t lb = p->lse ? B * Hq * S * 4 : 0;
  const int64_t qb = qrope ? span_bytes(p->q_strides, B, S, Hq, D, 2) : B * S * Hq * D;
  if (ob < 0 || cb < 0 || vb < 0 || qb < 0)
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd_fp8: q, v, o or cfg_out strides span more than 2^50 bytes");
  struct Span { const void* ptr; int64_t n; };
  Span ins[8 + 3 * NXATTN_MAX_BRANCHES] = {{qrope ? p->q : p->q8, qb}, {p->k8, B * S * Hkv * D}, {p->v, vb},
                                           {p->q_exp, B * Hq}, {p->k_exp, B * Hkv},
                                           {p->prefix_k_exp, any_prefix ? B * Hkv : 0},
                                           {p->q_scales, B * S * Hq * 4}, {p->k_scales, B * S * Hkv * 4}};
  int nin = 8;
  for (int b = 0; b < p->batch; ++b) {
    ins[nin++] = Span{p->prefix_k8[b], (int64_t)p->prefix_len[b] * Hkv * D};
    ins[nin++] = Span{p->prefix_v[b], (int64_t)p->prefix_len[b] * Hkv * D * 2};
    ins[nin++] = Span{p->prefix_k_scales[b], (int64_t)p->prefix_len[b] * Hkv * 4};
  }
  // outputs: o, lse, (with q_rope) the codes and scales formed on load, the guided output
  const Span outs[5] = {{p->o, ob}, {p->lse, lb}, {p->q8_out, p->q8_out ? B * S * Hq * D : 0},
                        {p->q_scales_out, p->q_scales_out ? B * S * Hq * 4 : 0}, {p->cfg_out, cb}};
  for (int j = 0; j < 5; ++j) {
    if (!outs[j].ptr) continue;
    for (int i = 0; i < nin; ++i)
      if (ins[i].ptr && overlaps(outs[j].ptr, outs[j].n, ins[i].ptr, ins[i].n))
        return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: an output overlaps an input");
    for (int i = j + 1; i < 5; ++i)
      if (outs[i].ptr && overlaps(outs[j].ptr, outs[j].n, outs[i].ptr, outs[i].n))
        return fail(NXATTN_ERR_INVALID, "nxattn_fwd_fp8: outputs overlap");
  }

  Args a;
  a.q8 = p->q8; a.k8 = p->k8; a.v = static_cast<const uint16_t*>(p->v); a.o = static_cast<uint16_t*>(p->o);
  a.q_exp = p->q_exp; a.k_exp = p->k_exp; a.pk_exp = p->prefix_k_exp ? p->prefix_k_exp : p->k_exp;
  a.q_sc = p->q_scales; a.k_sc = p->k_scales;
  a.q8_out = p->q8_out; a.qsc_out = p->q_scales_out;
  a.q = static_cast<const uint16_t*>(p->q);
  a.qs0 = p->q_strides[0]; a.qs1 = p->q_strides[1]; a.qs2 = p->q_strides[2];
  std::memset(a.rq, 0, sizeof(a.rq));
  if (qrope) {
    const int st = rope_q_setup(p->q_rope, p->batch, p->seq_q, D, "nxattn_fwd_fp8 (q_rope)", a.rq);
    if (st != NXATTN_OK) return st;
  }
  a.vs0 = p->v_strides[0]; a.vs1 = p->v_strides[1]; a.vs2 = p->v_strides[2];
  a.os0 = p->o_strides[0]; a.os1 = p->o_strides[1]; a.os2 = p->o_strides[2];
  for (int b = 0; b < NXATTN_MAX_BRANCHES; ++b) {
    const bool in = b < p->batch;
    a.pk8[b] = in ? p->prefix_k8[b] : nullptr;
    a.pv[b] = in ? static_cast<const uint16_t*>(p->prefix_v[b]) : nullptr;
    a.plen[b] = in ? p->prefix_len[b] : 0;
    a.pk_sc[b] = in ? p->prefix_k_scales[b] : nullptr;
  }
  a.batch = p->batch; a.seq = p->seq_q; a.heads_q = p->heads_q; a.heads_kv = p->heads_kv;
  a.group = p->heads_q / p->heads_kv;
  a.nchunks = (p->seq_q + 31) / 32;
  const int64_t nqb = (int64_t)a.group * a.nchunks;
  const int64_t wpg = (nqb + WAVES - 1) / WAVES;
  // branch pairs: one workgroup per (kv head, query blocks) serves both branches
  const int64_t total = wpg * p->heads_kv * (pair ? 1 : p->batch);
  if (total > INT32_MAX / 2) return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd_fp8: problem too large");
  a.nqb = (int)nqb; a.wg_per_group = (int)wpg; a.total_wg = (int)total;
  const float scale = p->scale > 0.f ? p->scale : 1.0f / std::sqrt((float)D);
  a.c = scale * LOG2E;
  a.lse = p->lse;
  a.cfg = static_cast<uint16_t*>(p->cfg_out);
  a.cs0 = pair ? p->cfg_strides[0] : 0;
  a.cs1 = pair ? p->cfg_strides[1] : 0;
  a.guidance = pair ? p->guidance : 0.f;
  if (pair) launch_fp8<true>(a, qrope, block, p->q_folded != 0, stream);
  else launch_fp8<false>(a, qrope, block, p->q_folded != 0, stream);
  return check_launch("nxattn_fwd_fp8");
}
