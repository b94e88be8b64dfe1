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
// walked in tiles of 64 over the virtual sequence [prefix ++ own], or over one range of
// whole tiles of it when the keys are split across workgroups (each range then writes a
// normalised fp32 partial and its log-sum-exp, combined by the merge kernel).
//
// Per wave: S^T = K Q^T lives in the 32x32 accumulator layout (lane = query row, 16
// registers = keys), so row max / row sum are in-lane plus one permlane32 swap. When q
// is rotated on load it is also multiplied by scale*log2(e) before its one rounding to
// bf16, and the score accumulators start at -m (the running row max): the MFMAs then
// deliver the exponent c s - m itself and the softmax needs no per-score FMA. The
// weights, rounded to bf16 in the accumulator layout, are directly the B operand (P^T) of
// O^T += V^T P^T. The V^T operand comes from row-major V in LDS through the gfx950
// transposing read ds_read_b64_tr_b16, so K and V are both stored row-major.
//
// Ping-pong. Waves 0-3 and 4-7 (one of each per SIMD) run the same program half a
// tile apart: while one group issues the MFMAs of tile t (scores of t+1 and P V of t),
// the other group runs the exp2/max/sum of its softmax, so matrix cores and VALU of a
// SIMD overlap. Each iteration ends at one workgroup barrier (after the tile loads have
// landed); inside it the groups pace themselves, since no LDS buffer read in the second
// half is written in the first. The wave that issues MFMAs in a half-iteration runs at
// the higher s_setprio level (the issue arbiter otherwise favours the older wave, which
// starves the second group's GEMM).
//
// Tile loads. Direct-to-LDS loads issued by waves 0-3 and interleaved with their
// score MFMAs. Tiles wholly inside the prefix or the own keys use buffer loads
// (buffer_load_dwordx4 ... lds) from a per-tile raw buffer with fixed per-lane offsets;
// the tile straddling the prefix end is processed last and, with the ragged last tile,
// uses per-lane clamped global_load_lds addresses after the GEMM phase. K and V buffers are distinct LDS objects, so the compiler does not make
// the score reads of one K buffer wait for loads into the other.
//
// Work order. Workgroups enumerate (kv head, branch, query blocks) kv-head-major and
// are remapped so that each XCD runs a contiguous range: the workgroups that stream
// the same K/V share an L2, and every XCD gets a mix of CFG branches (whose key
// counts differ).
//
// LDS: K and V double-buffered, 64 rows x 256 B each, 16-byte chunks XOR-swizzled per
// row (K: chunk ^ (row & 15), V: chunk ^ 4*(row & 3)) so the row-parallel K reads and
// the 4-row transposing V reads are free of bank conflicts. 64 KB per workgroup.
// MFMA-bound: 4*Sq*Skv*Hq*D flops per launch.
#include <type_traits>

#include "nx_internal.h"
#include "rope_turn.h"

namespace nx {

namespace bf16k {

constexpr int D = 128;
constexpr int BN = KEY_TILE;      // keys per tile (64)
constexpr int WAVES = 8;
constexpr int THREADS = WAVES * 64;
constexpr int ROWB = D * 2;       // bytes per K/V row
constexpr int TILEB = BN * ROWB;  // bytes per K or V tile (16 KB)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float RESCALE_T = 8.0f; // running max moves only when it grows by > 2^8
constexpr float RESCALE_LIM = 256.0f;  // 2^RESCALE_T
// raw buffer descriptors for the tile loads: no stride, bounds check effectively off
// (every steady-state tile lies inside its tensor), 32-bit data format
constexpr int BUF_RECORDS = 0x7fffffff;
constexpr int BUF_FLAGS = 0x00020000;

struct Args {
  const uint16_t* q; const uint16_t* k; const uint16_t* v; uint16_t* o;
  int64_t qs0, qs1, qs2, ks0, ks1, ks2, os0, os1, os2;
  const uint16_t* prefix[NXATTN_MAX_BRANCHES];
  int32_t plen[NXATTN_MAX_BRANCHES];
  int32_t batch, seq, heads_q, heads_kv, group, nchunks, nqb, wg_per_group, total_wg;
  float c;  // scale * log2(e)
  int32_t rope_q;
  RopeQ rq[NXATTN_MAX_BRANCHES];
  float* lse;
  float* part_o;
  float* part_lse;
  int32_t nsplit, per, prefix_only;
  // branch pairs: out[i, h] = bf16(fma(guidance, c - u, u)) with c, u the bf16 outputs of
  // branches 0 and 1 (o may then be NULL: branch outputs not stored)
  uint16_t* cfg;
  int64_t cs0, cs1;
  float guidance;
};

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ int remap_xcd(int i, int n) {
  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a contiguous
  // run of logical work so workgroups sharing K/V tiles share one L2.
  const int xcd = i & 7, local = i >> 3;
  const int per = n >> 3, rem = n & 7;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// LDS placement of 16-byte chunk `chunk` of tile row `row`
__device__ __forceinline__ int kslot(int row, int chunk) { return chunk ^ (row & 15); }
__device__ __forceinline__ int vslot(int row, int chunk) { return chunk ^ ((row & 3) << 2); }

// Workgroup barriers that also fence the instruction scheduler: nothing (not even pure
// ALU work) may move across, so each half-iteration's work stays in its slot.
__device__ __forceinline__ void barrier_only() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
// s_setprio around a barrier: the wave that issues MFMAs in the coming slot gets
// priority over its SIMD partner's softmax VALU (the issue arbiter would otherwise
// favour the older wave).
template <int BEFORE, int AFTER>
__device__ __forceinline__ void barrier_prio() {
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (BEFORE >= 0) asm volatile("s_setprio %0" :: "n"(BEFORE));
  asm volatile("s_barrier" ::: "memory");
  if constexpr (AFTER >= 0) asm volatile("s_setprio %0" :: "n"(AFTER));
  __builtin_amdgcn_sched_barrier(0);
}
// s_setprio alone (the half-iteration boundary inside an iteration): a second barrier
// there cost about 100 cycles per tile and guards no LDS hazard
template <int PRIO>
__device__ __forceinline__ void prio_only() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_setprio %0" :: "n"(PRIO));
  __builtin_amdgcn_sched_barrier(0);
}
template <int BEFORE, int AFTER>
__device__ __forceinline__ void wait_dma_barrier_prio() {
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (BEFORE >= 0) asm volatile("s_setprio %0" :: "n"(BEFORE));
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if constexpr (AFTER >= 0) asm volatile("s_setprio %0" :: "n"(AFTER));
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void wait_dma_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// LDS: K and V tiles, double-buffered, as four distinct objects (TILEB bytes each), so
// the compiler can tell a direct-to-LDS load into one buffer from a read of another and
// does not serialise them.
__shared__ __attribute__((aligned(1024))) uint8_t lds_k0[TILEB];
__shared__ __attribute__((aligned(1024))) uint8_t lds_k1[TILEB];
__shared__ __attribute__((aligned(1024))) uint8_t lds_v0[TILEB];
__shared__ __attribute__((aligned(1024))) uint8_t lds_v1[TILEB];
template <int PAR> __device__ __forceinline__ uint8_t* kbuf() { return PAR ? lds_k1 : lds_k0; }
template <int PAR> __device__ __forceinline__ uint8_t* vbuf() { return PAR ? lds_v1 : lds_v0; }
// Branch pairs: the first branch's rounded output, held until the second branch's epilogue
// (entry (wave, j, lane): 16 words-pairs per lane). Only the pair kernels use it; one
// workgroup per CU runs at a time (two waves per SIMD at these register counts), so
// 64 KB more fit beside the tiles.
__shared__ __attribute__((aligned(16))) u32x2 lds_keep[WAVES * 16 * 64];

// Direct-to-LDS tile load plan of a wave for one iteration: K tile t+2 and V tile t+1,
// each wholly inside the prefix or wholly inside the own keys. Instruction i (0-3: K,
// 4-7: V) moves rows 16ws + 4(i%4) .. +3: global address = row base (wave-uniform) +
// lane offset; LDS address = the buffer + the same rows.
struct DmaPlan {
  __amdgpu_buffer_rsrc_t krsrc, vrsrc;    // raw buffers based at row 16ws of the K / V tile
  uint32_t krs, vrs;                      // 4-row step in bytes
  uint32_t krp, vrp;                      // lane row offset (rl * row stride) in bytes
  uint32_t ck[4], cv;                     // lane chunk offsets (swizzled) in bytes
  int ws;
};

struct Wave {
  bf16x8 qf[8];       // Q^T operand, k-step ks: Q[row][16ks + 8hh .. +7]
  f32x16 o[4];        // O^T accumulators, d-block db (lane = query, registers = d)
  f32x16 s[2];        // S^T accumulators of the tile being scored (2 key blocks of 32)
  bf16x8 p[4];        // P^T operand of the tile being accumulated, step (kb, half)
  float m, l;
  float thr;          // FOLD: row max of the shifted scores above which m moves (-inf
                      // before the first tile); else (m + RESCALE_T) / c on raw scores
  f32x16 negm;        // FOLD: -m in every register, the score accumulators' start value
  bool primed;        // m has been set by a first tile (wave-uniform)
  // lane parts of the LDS byte addresses: K fragment of k-step ks at kbase + (32ks ^ kx),
  // V^T fragment of d-block db at vbase + (64db ^ vy)
  int kbase, kx, vbase, vy;
};

__device__ __forceinline__ u32x4 lds_read_b128(const uint8_t* smem, int byte) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>((const lds_u8*)smem + byte);
}
__device__ __forceinline__ bf16x4 lds_read_tr(const uint8_t* smem, int byte) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)((const lds_u8*)smem + byte));
}

// Scheduling-group helpers (compile-time sequences for __builtin_amdgcn_sched_group_barrier):
// With scores, steps 0-15 are score steps (one b128 read each) and steps 16-31 P V steps
// (two transposed halves each); without, all 16 steps are P V steps.
template <bool SCORE>
constexpr int reads_of(int i) { return SCORE ? (i < 16 ? 1 : 2) : 2; }
template <int I, int N, bool SCORE>
__device__ __forceinline__ void sched_reads() {
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(0x100, reads_of<SCORE>(I), 0);
    sched_reads<I + 1, N, SCORE>();
  }
}
template <int I, int N, int DIST, bool DMA, bool SCORE>
__device__ __forceinline__ void sched_steps() {
  if constexpr (I < N) {
    if constexpr (I + DIST < N) __builtin_amdgcn_sched_group_barrier(0x100, reads_of<SCORE>(I + DIST), 0);
    if constexpr (DMA && I >= 16 && ((I - 16) & 1) == 0) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    sched_steps<I + 1, N, DIST, DMA, SCORE>();
  }
}

// One GEMM phase of a wave: if `score`, S^T = K_{t+1} Q^T (16 MFMAs, issued first), and
// O^T += V_t^T P_t^T (16 MFMAs). Fragments are read from LDS three MFMAs ahead so the
// matrix core never waits on LDS latency; consecutive MFMAs target different
// accumulators. VPAR / KPAR select the V and K buffers (compile-time LDS offsets).
template <int VPAR, int KPAR, bool SCORE, bool FOLD, bool DMA = false>
__device__ __forceinline__ void gemm_phase(Wave& w, const DmaPlan* plan = nullptr) {
  const uint8_t* vsm = vbuf<VPAR>();
  const uint8_t* ksm = kbuf<KPAR>();
  constexpr int DIST = 3;
  constexpr int nsteps = SCORE ? 32 : 16;
  // with SCORE: step i < 16: S, (ks = i/2, kb = i%2); step i >= 16: PV, (kbhs = (i-16)/4,
  // db = (i-16)%4). Scores first: the next softmax's inputs are complete when the phase
  // ends, and only the P V MFMAs are still in flight.
  auto is_pv = [&](int i) { return SCORE ? i >= 16 : true; };
  auto pv_of = [&](int i) { return SCORE ? i - 16 : i; };
  auto read = [&](int i) -> bf16x8 {
    if (is_pv(i)) {
      const int ip = pv_of(i);
      const int kbhs = ip >> 2, db = ip & 3;
      const int rbase = (kbhs >> 1) * 32 + (kbhs & 1) * 16;   // kb*32 + 16*hs
      const int off = w.vbase + ((64 * db) ^ w.vy);
      const bf16x4 a = lds_read_tr(vsm, rbase * ROWB + off);
      const bf16x4 b = lds_read_tr(vsm, (rbase + 8) * ROWB + off);
      return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    const int j = i, ks = j >> 1, kb = j & 1;
    return as_bf16x8(lds_read_b128(ksm, kb * 32 * ROWB + w.kbase + ((32 * ks) ^ w.kx)));
  };
  // DMA instruction d (during the P V steps, after the phase's last K read): K_{t+2}
  // into K buffer KPAR^1, V_{t+1} into V buffer VPAR^1, both last read in the previous
  // iteration
  auto dma = [&](int d) {
    const int i = d & 3;
    const bool isv = d >= 4;
    uint8_t* dst = (isv ? vbuf<VPAR ^ 1>() : kbuf<KPAR ^ 1>()) + (16 * plan->ws + 4 * i) * ROWB;
    // buffer (MUBUF) form: unlike the flat-encoded global form, the compiler does not
    // count it as a possible LDS access under lgkmcnt, so the LDS fragment reads around
    // it keep their partial waits
    if (isv)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(plan->vrsrc, (__attribute__((address_space(3))) void*)(lds_u8*)dst, 16,
                                               plan->vrp + plan->cv, i * plan->vrs, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(plan->krsrc, (__attribute__((address_space(3))) void*)(lds_u8*)dst, 16,
                                               plan->krp + plan->ck[i], i * plan->krs, 0, 0);
  };
  bf16x8 ring[DIST + 1];
#pragma unroll
  for (int i = 0; i < DIST; ++i) ring[i] = read(i);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    if (i < nsteps) {
      if (i + DIST < nsteps) ring[(i + DIST) % (DIST + 1)] = read(i + DIST);
      if constexpr (DMA) {
        if (i >= 16 && ((i - 16) & 1) == 0) dma((i - 16) >> 1);
      }
      const bf16x8 f = ring[i % (DIST + 1)];
      if (is_pv(i)) {
        const int ip = pv_of(i);
        const int kbhs = ip >> 2, db = ip & 3;
        w.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, w.p[kbhs], w.o[db], 0, 0, 0);
      } else {
        const int j = i, ks = j >> 1, kb = j & 1;
        if (ks == 0) w.s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, w.qf[ks], FOLD ? w.negm : f32x16{}, 0, 0, 0);
        else w.s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, w.qf[ks], w.s[kb], 0, 0, 0);
      }
    }
  }
  // keep the issue order: the first DIST fragments' reads, then per step the reads of
  // step i+DIST followed by MFMA i
  sched_reads<0, DIST, SCORE>();
  sched_steps<0, nsteps, DIST, DMA, SCORE>();
}

// S^T only (prologue).
template <int KPAR, bool FOLD>
__device__ __forceinline__ void gemm_s_only(Wave& w) {
  const uint8_t* ksm = kbuf<KPAR>();
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 f = as_bf16x8(lds_read_b128(ksm, kb * 32 * ROWB + w.kbase + ((32 * ks) ^ w.kx)));
      if (ks == 0) w.s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, w.qf[ks], FOLD ? w.negm : f32x16{}, 0, 0, 0);
      else w.s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, w.qf[ks], w.s[kb], 0, 0, 0);
    }
}

// RoPE of this lane's q values on load, with the turns of RopeTurns (rope_turn.h), times
// sc; results rounded to bf16 (RNE). Lane data: qf[ks][e] = q[16 ks + 8 hh + e].
__device__ __forceinline__ void rotate_q(bf16x8* qf, const RopeQ& r, int tok, int lane, float sc) {
  const int hh = lane >> 5;
  const RopeTurns rt(r, tok, lane);
  auto turn = [&](int j, float& sn, float& cs) { rt.turn(j, sn, cs); };
  if (!r.interleaved) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float sn, cs;
        turn(16 * ks + 8 * hh + e, sn, cs);
        const float xa = (float)qf[ks][e], xb = (float)qf[ks + 4][e];
        qf[ks][e] = (__bf16)((xa * cs - xb * sn) * sc);
        qf[ks + 4][e] = (__bf16)((xa * sn + xb * cs) * sc);
      }
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float sn, cs;
        turn((16 * ks + 8 * hh + e) >> 1, sn, cs);
        const float xa = (float)qf[ks][e], xb = (float)qf[ks][e + 1];
        qf[ks][e] = (__bf16)((xa * cs - xb * sn) * sc);
        qf[ks][e + 1] = (__bf16)((xa * sn + xb * cs) * sc);
      }
  }
}

// Weights of the tile against the current m, rounded to bf16 into w.p (the B operand of
// the P V step); returns this lane's sum of them (unrounded).
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
        const float p0 = FOLD ? __builtin_amdgcn_exp2f(w.s[kb][8 * hs + 2 * e])
                              : __builtin_amdgcn_exp2f(__builtin_fmaf(w.s[kb][8 * hs + 2 * e], c, nm));
        const float p1 = FOLD ? __builtin_amdgcn_exp2f(w.s[kb][8 * hs + 2 * e + 1])
                              : __builtin_amdgcn_exp2f(__builtin_fmaf(w.s[kb][8 * hs + 2 * e + 1], c, nm));
        l0 = (kb | hs | e) ? l0 + p0 : p0;
        l1 = (kb | hs | e) ? l1 + p1 : p1;
        pk[e] = pack_bf16x2(p0, p1);
      }
      w.p[2 * kb + hs] = as_bf16x8(pk);
    }
  return l0 + l1;
}

// FOLD: -m into every register of the score accumulators' start block. The block is
// kept across tiles and rebuilt only when m moves (the score MFMAs read it, never write
// it); rebuilding it after every softmax cost 8 moves per half-tile (same-box: 0.5 %
// at the 1K DiT shape, 0.8 % at 2K).
template <bool FOLD>
__device__ __forceinline__ void set_negm(Wave& w) {
  if constexpr (FOLD) {
#pragma unroll
    for (int i = 0; i < 16; ++i) w.negm[i] = -w.m;
  }
}

// The full softmax update: row max of the tile; rows whose max exceeds their threshold
// move m (rescaling l and O).
template <bool FOLD>
__device__ __forceinline__ void full_update(Wave& w, float c) {
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
    // the scores arrive as c s - m: a row moves its max by d = tmax, and this tile's
    // scores by -d
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
      set_negm<FOLD>(w);
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
  w.primed = true;
}

// Online softmax of w.s (tile with `valid` keys, < BN only for the last tile) -> w.p.
// FOLD: w.s already holds c s - m (q pre-scaled, accumulators started at -m).
//
// FOLD: the weights first, the max only when needed. m moves only when a row's tile max
// exceeds m by more than RESCALE_T (in log2 units), i.e. when some weight 2^(c s - m)
// exceeds 2^RESCALE_T. Once a first tile has set m, the weights are taken against the
// current m with no max: they are non-negative, so when every lane's sum of them is at
// most 2^RESCALE_T, every weight is too, m would not have moved, and the weights stand
// (bit for bit what the full update computes in that case). A larger sum (or inf or NaN)
// anywhere in the wave sends it through the full update and the weights again (one copy
// of the weight code, in a loop that is never unrolled: two inlined copies made the
// register allocator spill). With a stored q (an FMA per score in front of each exp) the
// two-pass form measured slower, so that variant keeps the single pass.
template <bool MASK, bool FOLD>
__device__ __forceinline__ void softmax(Wave& w, float c, int valid, int hh) {
  // MASK = false: the tile is known to be whole (no per-key compare/select is compiled)
  if (MASK && valid < BN) {
    // key of register i in block kb is kb*32 + 8(i/4) + 4hh + (i%4): compare the
    // compile-time part against valid - 4hh
    const int lim = valid - 4 * hh;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kb * 32 + 8 * (i >> 2) + (i & 3) >= lim) w.s[kb][i] = -__builtin_inff();
  }
  float lt = 0.f;
  if constexpr (FOLD) {
#pragma nounroll
    for (int pass = w.primed ? 0 : 1; pass < 2; ++pass) {
      if (pass == 1) full_update<FOLD>(w, c);
      lt = weights<FOLD>(w, c);
      if (pass == 1 || !__builtin_amdgcn_ballot_w64(!(lt <= RESCALE_LIM))) break;
    }
  } else {
    full_update<FOLD>(w, c);
    lt = weights<FOLD>(w, c);
  }
  w.l += lt;
}

// The per-wave program. Group A (waves 0-3) and group B (waves 4-7) run it half a tile
// apart; both execute the same sequence of workgroup barriers. PAIR: the workgroup runs
// branch 0 and then branch 1 of its query blocks, keeps branch 0's rounded output in
// registers and writes the guidance combination of the two.
template <bool GROUP_A, bool FOLD, bool PAIR>
__device__ __forceinline__ void wave_program(const Args& a, int lane, int wave) {
  const int n = lane & 31, hh = lane >> 5;
  const int wg = remap_xcd(blockIdx.x, a.total_wg);
  // (kv head, branch, key range) groups in kv-head-major order: each XCD's contiguous
  // share mixes the CFG branches, whose key counts differ (PAIR: (kv head) groups)
  const int grp = wg / a.wg_per_group;
  const int split = grp % a.nsplit, gb = grp / a.nsplit;
  const int g = PAIR ? gb : gb / a.batch, b0 = PAIR ? 0 : gb % a.batch;
  const int qb = (wg % a.wg_per_group) * WAVES + wave;
  const bool active = qb < a.nqb;
  const int hq = g * a.group + (active ? qb / a.nchunks : 0);
  const int tok = (active ? qb % a.nchunks : 0) * 32 + n;
  const int tokc = tok < a.seq ? tok : a.seq - 1;
  // one branch (PAIR: branch bi of the pair, the two passes inlined one after the other)
  auto pass = [&](auto bic) {
  constexpr int bi = decltype(bic)::value;
  const int b = PAIR ? bi : b0;
  // this work item's keys: tiles [t0, t0 + T) of the virtual sequence, keys below kend
  const int P = a.plen[b];
  const int Skv = P + (a.prefix_only ? 0 : a.seq);
  const int t0 = split * a.per;
  const int Tall = (Skv + BN - 1) / BN;
  const int T = min(a.per, Tall - t0);
  if (T <= 0) return;   // empty key range (uniform over the workgroup, before any barrier;
                        // PAIR launches have one range per branch and T >= 1)
  // a branch whose keys fit in one range writes its result directly, without a merge
  const bool partial = a.nsplit > 1 && Tall > a.per;
  const int kend = min((t0 + T) * BN, Skv);
  const float c = a.c;

  Wave w;
  {
    const uint16_t* qrow = a.q + b * a.qs0 + (int64_t)tokc * a.qs1 + (int64_t)hq * a.qs2;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) w.qf[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * hh));
  }
#pragma unroll
  for (int db = 0; db < 4; ++db) w.o[db] = f32x16{};
  // FOLD: m starts at 0 (the accumulators start at -m = 0) and the first tile always
  // moves it to its row max
  w.m = FOLD ? 0.f : -__builtin_inff();
  w.thr = -__builtin_inff();
  w.primed = false;
#pragma unroll
  for (int i = 0; i < 16; ++i) w.negm[i] = 0.f;
  w.l = 0.f;
  // lane parts of the LDS read addresses. K: row n, chunk 2ks+hh at slot
  // (2ks+hh) ^ (n & 15), i.e. byte n*ROWB + 16*(hh ^ (n&1)) + (32ks ^ 16*(n & 14)).
  // V (transposing read): row r = 4*(q>>1) + rsub, column col = 32db + 16(q&1) + csub,
  // chunk col>>3 = 4db + e at slot (4db + e) ^ 4rsub, i.e. byte
  // r*ROWB + 16e + 2*(csub&7) + (64db ^ 64rsub).
  // The fragment addresses these give are the same for every tile: the compiler keeps
  // them in registers (20 more VGPRs, 234 in the branch-pair kernel, no spills), so the
  // main loop does no address arithmetic for its LDS reads.
  w.kbase = n * ROWB + 16 * (hh ^ (n & 1));
  w.kx = 16 * (n & 14);
  {
    const int q = lane >> 4, j = lane & 15;
    const int rsub = j >> 2, csub = 4 * (j & 3);
    const int r = 4 * (q >> 1) + rsub;                 // row within a 16-row step (+ 8 for elements 4..7)
    const int e = 2 * (q & 1) + (csub >> 3);
    w.vbase = r * ROWB + 16 * e + 2 * (csub & 7);
    w.vy = 64 * rsub;
  }

  // DMA tile loads (global_load_lds, 1 KB = 4 rows per instruction). With NW waves
  // taking part, wave slot ws fills rows (64/NW)*ws .. ; lane -> (row, LDS slot), and it
  // fetches the global chunk that the swizzle places in that slot.
  const uint16_t* kprefix = a.prefix[b] ? a.prefix[b] + (int64_t)g * D : nullptr;
  const int64_t pstride = (int64_t)a.heads_kv * D;
  const uint16_t* kown = a.k + b * a.ks0 + (int64_t)g * a.ks2;
  const uint16_t* vown = a.v + b * a.ks0 + (int64_t)g * a.ks2;
  const int64_t ks1 = a.ks1;
  auto dma_tile = [&](int t, bool isv, uint8_t* dst, int ws, auto nw) {
    constexpr int NW = decltype(nw)::value;
    constexpr int ROWS = BN / NW;
#pragma unroll
    for (int i = 0; i < ROWS / 4; ++i) {
      const int r = ROWS * ws + 4 * i + (lane >> 4);
      const int slot = lane & 15;
      const int chunk = isv ? (slot ^ ((r & 3) << 2)) : (slot ^ (r & 15));
      int j = t * BN + r;
      j = j < kend ? j : kend - 1;
      const uint16_t* src;
      if (j < P) src = (isv ? kprefix + (int64_t)P * pstride : kprefix) + (int64_t)j * pstride;
      else src = (isv ? vown : kown) + (int64_t)(j - P) * ks1;
      __builtin_amdgcn_global_load_lds(src + 8 * chunk,
                                       (__attribute__((address_space(3))) void*)((lds_u8*)dst + (ROWS * ws + 4 * i) * ROWB),
                                       16, 0, 0);
    }
  };
  using All = std::integral_constant<int, 8>;
  using Half = std::integral_constant<int, 4>;

  // Key tiles are processed in natural order, except that a tile straddling the end of
  // the prefix (when it is not also the range's last tile) moves to the end: the online
  // softmax does not depend on the order. Positions [0, nwhole) then hold only whole
  // tiles, wholly inside the prefix or wholly inside the own keys.
  const int tl = t0 + T - 1;
  const int sb = (P % BN != 0 && P / BN >= t0 && P / BN < tl) ? P / BN : -1;
  auto tile_at = [&](int pos) {
    const int t = t0 + pos;
    return (sb < 0 || t < sb) ? t : (pos < T - 1 ? t + 1 : sb);
  };
  auto valid_at = [&](int pos) { const int r = kend - tile_at(pos) * BN; return r < BN ? r : BN; };
  const bool last_whole = (tl + 1) * BN <= kend && (tl * BN >= P || (tl + 1) * BN <= P);
  const int nwhole = T - (sb >= 0 ? 1 : 0) - (last_whole ? 0 : 1);

  // Steady-state loads of whole tiles (4 waves x 16 rows): a wave-uniform row base in
  // scalar registers plus a per-lane 32-bit byte offset. Lane (rl = lane/16, slot =
  // lane%16) of instruction i fills row 16ws + 4i + rl, whose K swizzle is
  // slot ^ (4i + rl) and whose V swizzle is slot ^ 4rl.
  const int rl = lane >> 4, lslot = lane & 15;
  const uint32_t rp_pre = (uint32_t)(rl * pstride * 2), rp_own = (uint32_t)(rl * ks1 * 2);
  uint32_t ck[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) ck[i] = 16u * (uint32_t)(lslot ^ (4 * i + rl));
  const uint32_t cv = 16u * (uint32_t)(lslot ^ (rl << 2));
  auto plan_of = [&](int t) {
    DmaPlan pl;
    const int jk = tile_at(t + 2) * BN + 16 * wave, jv = tile_at(t + 1) * BN + 16 * wave;
    const bool kpre = jk < P, vpre = jv < P;
    const uint16_t* kb = kpre ? kprefix + (int64_t)jk * pstride : kown + (int64_t)(jk - P) * ks1;
    const uint16_t* vb = vpre ? kprefix + (int64_t)(P + jv) * pstride : vown + (int64_t)(jv - P) * ks1;
    pl.krsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kb), 0, BUF_RECORDS, BUF_FLAGS);
    pl.vrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vb), 0, BUF_RECORDS, BUF_FLAGS);
    pl.krs = (uint32_t)(8 * (kpre ? pstride : ks1));
    pl.vrs = (uint32_t)(8 * (vpre ? pstride : ks1));
    pl.krp = kpre ? rp_pre : rp_own;
    pl.vrp = vpre ? rp_pre : rp_own;
#pragma unroll
    for (int i = 0; i < 4; ++i) pl.ck[i] = ck[i];
    pl.cv = cv;
    pl.ws = wave;
    return pl;
  };

  // ---- prologue: the first K tile, V tile and second K tile resident; both groups
  // ---- score position 0; group A also runs its softmax, so that A leads B by half a
  // ---- tile from here on.
  dma_tile(tile_at(0), false, kbuf<0>(), wave, All{});
  dma_tile(tile_at(0), true, vbuf<0>(), wave, All{});
  if (T > 1) dma_tile(tile_at(1), false, kbuf<1>(), wave, All{});
  // q's RoPE (if requested) while the first tiles are in flight
  if (FOLD) rotate_q(w.qf, a.rq[b], tokc, lane, c);
  else if (a.rope_q) rotate_q(w.qf, a.rq[b], tokc, lane, 1.0f);
  wait_dma_barrier();
  gemm_s_only<0, FOLD>(w);
  if (GROUP_A) softmax<true, FOLD>(w, c, valid_at(0), hh);
  if (GROUP_A) barrier_prio<-1, 2>();
  else barrier_only();

  // Iteration t: slot 2t (A multiplies, B normalises), slot 2t+1 (swapped). Each GEMM
  // phase accumulates P V of position t and scores position t+1 (the last iteration
  // scores a stale K buffer that is never used: one code path keeps the register
  // allocation of S and P straight). The multiplying wave holds the higher priority.
  // Group A fetches K of position t+2 into K buffer t&1 and V of position t+1 into V
  // buffer (t+1)&1, both last read in the previous iteration; the loads land before
  // the barrier that ends slot 2t+1, the iteration's only barrier (slot 2t+1 reads V
  // buffer t&1 and K buffer (t+1)&1, which no load of the iteration writes). FAST: both
  // are whole tiles, and the loads are interleaved with the score MFMAs (after the
  // phase's last V read).
  auto iter_a = [&](int t, auto par, auto fast) {
    constexpr int PAR = decltype(par)::value;        // t & 1
    constexpr bool FAST = decltype(fast)::value;
    if constexpr (FAST) {
      const DmaPlan pl = plan_of(t);
      gemm_phase<PAR, PAR ^ 1, true, FOLD, true>(w, &pl);
    } else {
      gemm_phase<PAR, PAR ^ 1, true, FOLD>(w);
      if (t + 2 < T) dma_tile(tile_at(t + 2), false, kbuf<PAR>(), wave, Half{});
      if (t + 1 < T) dma_tile(tile_at(t + 1), true, vbuf<PAR ^ 1>(), wave, Half{});
    }
    prio_only<0>();
    // a fast iteration's next position is a whole tile
    if (t + 1 < T) softmax<!FAST, FOLD>(w, c, valid_at(t + 1), hh);
    wait_dma_barrier_prio<-1, 2>();
  };
  // MASK: the position may be the range's last, possibly ragged, tile
  auto iter_b = [&](int t, auto par, auto mask) {
    constexpr int PAR = decltype(par)::value;
    softmax<decltype(mask)::value, FOLD>(w, c, valid_at(t), hh);
    prio_only<2>();
    gemm_phase<PAR, PAR ^ 1, true, FOLD>(w);
    wait_dma_barrier_prio<0, -1>();
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
    // positions [0, nwhole) are whole tiles; a ragged tile can sit at T - 2 when the
    // straddling tile is moved to T - 1
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

  if (GROUP_A) asm volatile("s_setprio 0");
  // ---- epilogue: total row sum (both lane halves), normalise, round, store
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(w.l), __float_as_int(w.l), false, false);
    w.l = __int_as_float(sw[0]) + __int_as_float(sw[1]);
  }
  if (PAIR) {
    // no early exit: every wave takes part in the second branch's barriers
    if constexpr (bi == 0) {
      if (active && tok < a.seq) {
        const float inv = 1.0f / w.l;
        if (a.lse && hh == 0) a.lse[((int64_t)b * a.heads_q + hq) * a.seq + tok] = LN2 * (w.m + __builtin_amdgcn_logf(w.l));
        uint16_t* orow = a.o ? a.o + b * a.os0 + (int64_t)tok * a.os1 + (int64_t)hq * a.os2 : nullptr;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int d = 32 * db + 8 * i4 + 4 * hh;
            const u32x2 r = u32x2{pack_bf16x2(w.o[db][4 * i4] * inv, w.o[db][4 * i4 + 1] * inv),
                                  pack_bf16x2(w.o[db][4 * i4 + 2] * inv, w.o[db][4 * i4 + 3] * inv)};
            if (orow) *reinterpret_cast<u32x2*>(orow + d) = r;
            *(__attribute__((address_space(3))) u32x2*)&lds_keep[(wave * 16 + 4 * db + i4) * 64 + lane] = r;
          }
      }
    } else if (active) {
      // The wave's 32 rows: this lane's row half of branch 0 (kept in LDS) in registers
      // first; then the guided values go back into the same 8 KB, row-major with the 16-byte
      // chunk c of row n at chunk c ^ (n & 15), and leave as whole 256-byte rows (16 lanes
      // per row) instead of 8-byte pieces of 32 rows per store.
      const bool valid = tok < a.seq;
      const float inv = 1.0f / w.l;
      if (valid && a.lse && hh == 0) a.lse[((int64_t)b * a.heads_q + hq) * a.seq + tok] = LN2 * (w.m + __builtin_amdgcn_logf(w.l));
      uint16_t* orow = (valid && a.o) ? a.o + b * a.os0 + (int64_t)tok * a.os1 + (int64_t)hq * a.os2 : nullptr;
      typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
      typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
      lds_u32x2* keep = (lds_u32x2*)&lds_keep[wave * 16 * 64];
      u32x2 cv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) cv[j] = keep[j * 64 + lane];
      lds_u8* stage = (lds_u8*)&lds_keep[wave * 16 * 64];
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d = 32 * db + 8 * i4 + 4 * hh, ch = 4 * db + i4;
          const u32x2 r = u32x2{pack_bf16x2(w.o[db][4 * i4] * inv, w.o[db][4 * i4 + 1] * inv),
                                pack_bf16x2(w.o[db][4 * i4 + 2] * inv, w.o[db][4 * i4 + 3] * inv)};
          if (orow) *reinterpret_cast<u32x2*>(orow + d) = r;
          // the arithmetic of the combine pass on the two rounded outputs: c = branch 0,
          // u = branch 1, fma(guidance, c - u, u) in fp32, rounded to nearest even
          u32x2 o2;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t cw = cv[ch][e], uw = r[e];
            const float c0 = __uint_as_float(cw << 16), c1 = __uint_as_float(cw & 0xffff0000u);
            const float u0 = __uint_as_float(uw << 16), u1 = __uint_as_float(uw & 0xffff0000u);
            o2[e] = pack_bf16x2(__builtin_fmaf(a.guidance, c0 - u0, u0), __builtin_fmaf(a.guidance, c1 - u1, u1));
          }
          *(lds_u32x2*)(stage + n * ROWB + 16 * (ch ^ (n & 15)) + 8 * hh) = o2;
        }
      // lane L writes chunk L % 16 of rows L / 16 + 4k (the wave's own LDS writes above
      // are ordered before these reads)
      const int ch = lane & 15, tok0 = tok - n;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int nr = (lane >> 4) + 4 * k;
        const u32x4 v = *(lds_u32x4*)(stage + nr * ROWB + 16 * (ch ^ (nr & 15)));
        if (tok0 + nr < a.seq)
          *reinterpret_cast<u32x4*>(a.cfg + (int64_t)(tok0 + nr) * a.cs0 + (int64_t)hq * a.cs1 + 8 * ch) = v;
      }
    }
    return;
  }
  if (!active || tok >= a.seq) return;
  const float inv = 1.0f / w.l;
  // log-sum-exp of the scaled scores: sum_j exp2(c s_j - m) = l, so in natural log
  // lse = ln2 * (m + log2 l)  (l >= 1: the key that set m contributes 1)
  const float lse = LN2 * (w.m + __builtin_amdgcn_logf(w.l));
  if (partial) {
    // normalised fp32 partial of this key range, and its log-sum-exp
    const int64_t row = ((int64_t)split * a.batch + b) * a.seq + tok;
    float* prow = a.part_o + (row * a.heads_q + hq) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * db + 8 * i4 + 4 * hh;
        *reinterpret_cast<f32x4*>(prow + d) = f32x4{w.o[db][4 * i4] * inv, w.o[db][4 * i4 + 1] * inv,
                                                    w.o[db][4 * i4 + 2] * inv, w.o[db][4 * i4 + 3] * inv};
      }
    if (hh == 0) a.part_lse[(((int64_t)split * a.batch + b) * a.heads_q + hq) * a.seq + tok] = lse;
    return;
  }
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
  if (a.lse && hh == 0) a.lse[((int64_t)b * a.heads_q + hq) * a.seq + tok] = lse;
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

template <bool FOLD, bool PAIR>
__global__ __launch_bounds__(THREADS) void fwd_bf16_kernel(Args a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave < 4) wave_program<true, FOLD, PAIR>(a, lane, wave);
  else wave_program<false, FOLD, PAIR>(a, lane, wave);
}

}  // namespace bf16k

FwdShape fwd_shape_bf16(const FwdProblem& p) {
  using namespace bf16k;
  // resident workgroups per CU (registers and LDS bound it) of the variant that will run,
  // queried on each call: the library keeps no state
  int n = 0;
  const hipError_t e = p.rope_q ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_bf16_kernel<true, false>, THREADS, 0)
                                : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_bf16_kernel<false, false>, THREADS, 0);
  const int64_t nqb = (int64_t)(p.heads_q / p.heads_kv) * ((p.seq_q + 31) / 32);
  return FwdShape{(nqb + WAVES - 1) / WAVES * p.heads_kv, (e != hipSuccess || n < 1) ? 1 : n};
}

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
  const bool pair = p.cfg != nullptr;   // one workgroup per (kv head, query blocks), both branches
  const int64_t total = wpg * p.heads_kv * (pair ? 1 : p.batch * p.nsplit);
  if (total > INT32_MAX / 2) return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd: problem too large");
  a.nqb = (int)nqb; a.wg_per_group = (int)wpg; a.total_wg = (int)total;
  a.c = p.scale * LOG2E;
  a.rope_q = p.rope_q;
  for (int b = 0; b < NXATTN_MAX_BRANCHES; ++b) a.rq[b] = p.rq[b];
  a.lse = p.lse; a.part_o = p.part_o; a.part_lse = p.part_lse;
  a.nsplit = p.nsplit; a.per = p.per; a.prefix_only = p.prefix_only;
  if (p.prefix_only) {  // own keys are never read: keep valid (unused) base pointers
    a.k = a.q; a.v = a.q;
    a.ks0 = a.ks1 = a.ks2 = 0;
  }
  a.cfg = static_cast<uint16_t*>(p.cfg);
  a.cs0 = p.cs[0]; a.cs1 = p.cs[1];
  a.guidance = p.guidance;
  if (pair) {
    if (a.rope_q) fwd_bf16_kernel<true, true><<<a.total_wg, THREADS, 0, stream>>>(a);
    else fwd_bf16_kernel<false, true><<<a.total_wg, THREADS, 0, stream>>>(a);
  } else {
    if (a.rope_q) fwd_bf16_kernel<true, false><<<a.total_wg, THREADS, 0, stream>>>(a);
    else fwd_bf16_kernel<false, false><<<a.total_wg, THREADS, 0, stream>>>(a);
  }
  return check_launch("nxattn_fwd(bf16)");
}

}  // namespace nx
