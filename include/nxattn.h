/*
 * nxattn — non-causal (bidirectional) grouped-query attention over a conditioning
 * KV prefix plus the model's own tokens, with RoPE at explicit position offsets,
 * for AMD Instinct MI355X (gfx950). C ABI: plain pointers, sizes and a HIP stream.
 *
 * Conventions shared by every entry point
 *  - Device pointers are owned by the caller; the library allocates no device memory,
 *    keeps no state except a thread-local error message (and, for
 *    nxattn_rope_quantize_fp8_noalloc alone, its static device scratch and that
 *    scratch's address per GPU), and never synchronises: work is enqueued on `stream`
 *    (NULL = the default stream) and the call returns.
 *  - Every argument is validated on the host before anything is enqueued; on error
 *    nothing is launched and the return value is a nonzero nxattn_status. The detail
 *    of the last failing call on this thread is in nxattn_last_error().
 *  - Zero-size problems return NXATTN_OK without launching.
 *  - Element types: NXATTN_F32 (IEEE binary32) or NXATTN_BF16 (bfloat16, stored as
 *    16-bit words). Every float -> bf16 conversion rounds to nearest even.
 *  - Strides are in elements; the innermost (head_dim) dimension is contiguous.
 *  - Base pointers must be 16-byte aligned and every stride must keep rows 16-byte
 *    aligned (NXATTN_ERR_ALIGN otherwise).
 *  - No tensor argument's sizes and strides may span more than 2^50 bytes (far beyond
 *    any device's memory): such calls return NXATTN_ERR_UNSUPPORTED, whatever values
 *    the sizes and strides take (the host arithmetic that checks them cannot overflow).
 */
#ifndef NXATTN_H
#define NXATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NXATTN_OK = 0,
  NXATTN_ERR_INVALID = 1,      /* NULL pointer, negative size, inconsistent shape   */
  NXATTN_ERR_UNSUPPORTED = 2,  /* valid but outside the supported set (dtype, D, …)  */
  NXATTN_ERR_ALIGN = 3,        /* pointer or stride breaks the 16-byte rule          */
  NXATTN_ERR_HIP = 4           /* the HIP runtime reported an error at launch        */
} nxattn_status;

typedef enum { NXATTN_F32 = 0, NXATTN_BF16 = 1 } nxattn_dtype;

#define NXATTN_MAX_BRANCHES 8
#define NXATTN_MAX_SPLITS 16

/*
 * KV relayout between the replay-file layout and the online layout.
 * Defined by the NeoPP page ("NeoPP: LightLLM integration and KV replay"), section
 * "KV file layout": the online cache is [layers, 2, seq, kv_heads, head_dim], replay
 * files hold [layers, 2, kv_heads, seq, head_dim], and converting between them
 * exchanges dimensions 2 and 3 (index 0 of the size-2 dimension is K, 1 is V).
 *
 *   dir 0: src replay [L,2,H,S,D]  -> dst online [L,2,S,H,D]
 *   dir 1: src online [L,2,S,H,D]  -> dst replay [L,2,H,S,D]
 *
 * Both buffers are contiguous device memory of L*2*H*S*D elements of `dtype`; they
 * must not overlap (NXATTN_ERR_INVALID). The copy is bit-exact.
 */
int nxattn_kv_relayout(const void* src, void* dst, int64_t layers, int64_t kv_heads, int64_t seq,
                       int64_t head_dim, int dtype, int dir, hipStream_t stream);

/*
 * Rotary position embedding descriptor of one branch (batch entry).
 * KLiteInfer page, section "架构" (architecture): RoPE, 2-D RoPE (vision) and MRoPE
 * operators; NeoPP page, intro and "KV file layout": position offsets are supplied
 * with the KV cache and never inferred from tensor sizes.
 *
 * Own token s in [0, seq) is unravelled row-major over grid[0..n_axes) (axis 0
 * slowest); the position on axis k is its coordinate plus offset[k]. The head_dim/2
 * rotary pairs are split into contiguous sections, pairs[k] of them for axis k in
 * axis order (sum == head_dim/2). Pair j with local index u in section k rotates by
 * angle pos_k * theta^(-2u / (2*pairs[k])) (global_freq == 0: a frequency ladder per
 * section), or by pos_k * theta^(-2j / head_dim) (global_freq == 1: one ladder over
 * all pairs, the sections only choose the axis; the MRoPE of the KLiteInfer page's
 * ERNIE decoder):
 *   a' = a cos - b sin,  b' = a sin + b cos,
 * with (a, b) = (x[j], x[j + head_dim/2]) (interleaved == 0) or (x[2j], x[2j+1]).
 */
typedef struct {
  int32_t n_axes;        /* 1, 2 or 3                                   */
  int32_t grid[3];       /* grid extents; product == seq                */
  int32_t pairs[3];      /* rotary pairs per axis; sum == head_dim / 2  */
  int32_t offset[3];     /* position offset per axis (>= 0)             */
  double theta;          /* frequency base (> 1), 10000 in the configs  */
  int32_t interleaved;   /* 0 = half-split pairs, 1 = adjacent pairs    */
  int32_t global_freq;   /* 0 = ladder per axis section, 1 = one ladder */
} nxattn_rope_desc;

/*
 * In-place RoPE on x[b, s, h, :] for b < batch, s < seq, h < heads.
 * strides = {stride_b, stride_s, stride_h} in elements; the head_dim elements of a
 * row are contiguous. rope points to `batch` host descriptors (one per branch, so the
 * two CFG branches may use different offsets); batch <= NXATTN_MAX_BRANCHES.
 * The rotation is computed in fp32. F32 data: from an fp64 angle and fp64 sine and
 * cosine. BF16 data (every position below 2^24): each pair's step in revolutions is
 * evaluated in fp64 and the turn position * step formed exactly in fp32 but for the
 * roundings of small terms (below 1e-7 revolutions), then taken by the hardware sine and
 * cosine, as q_rope in nxattn_fwd does; bf16 results are rounded to nearest even.
 * Supported: head_dim a multiple of 8, 8 <= head_dim <= 256, dtype F32 or BF16.
 */
int nxattn_rope_apply(void* x, int64_t batch, int64_t seq, int64_t heads, int64_t head_dim,
                      const int64_t strides[3], int dtype, const nxattn_rope_desc* rope,
                      hipStream_t stream);

/*
 * The RoPE of x (exactly nxattn_rope_apply, same arguments and checks) and n_jobs KV
 * relayouts (each exactly nxattn_kv_relayout of its job: replay <-> online layout, NeoPP
 * page, "KV file layout") in one launch: a DiT step's rotation of k and the relayout of
 * each branch's prefix then cost one kernel boundary instead of 1 + n_jobs. The jobs run
 * in workgroups appended after the rotation's; the results are bit for bit those of the
 * separate calls.
 *   jobs: host array of n_jobs (0 .. NXATTN_MAX_BRANCHES) descriptors, read during the
 *   call; each job's src and dst hold layers*2*kv_heads*seq rows of head_dim elements of
 *   x's dtype. Rows and pointers must be 16-byte multiples (NXATTN_ERR_UNSUPPORTED
 *   otherwise: nxattn_kv_relayout takes the rest). No job's src or dst may overlap x, a
 *   job's dst may not overlap any job's src or another job's dst (NXATTN_ERR_INVALID).
 *   Jobs with a zero size are skipped; with no rotation work (batch, seq or heads zero;
 *   head_dim is still checked), the jobs alone run.
 */
typedef struct {
  const void* src;
  void* dst;
  int64_t layers, kv_heads, seq, head_dim;
  int32_t dir;                       /* 0: replay -> online, 1: online -> replay */
} nxattn_relayout_job;

int nxattn_rope_apply_relayout(void* x, int64_t batch, int64_t seq, int64_t heads, int64_t head_dim,
                               const int64_t strides[3], int dtype, const nxattn_rope_desc* rope,
                               const nxattn_relayout_job* jobs, int32_t n_jobs, hipStream_t stream);

/*
 * Fused non-causal attention over [prefix ++ own] for every branch of a CFG batch.
 * KLiteInfer page, section "架构": bidirectional attention is scores GEMM, softmax,
 * output GEMM (here fused, the score matrix never leaves the chip); NeoPP page:
 * the DiT attends to the injected conditioning KV (one branch per CFG side).
 *
 * For branch b, q head h (kv head g = h / (heads_q / heads_kv)), own query i:
 *   keys j in [0, P_b + seq_q): K_j = prefix K row j for j < P_b, else own k row j-P_b
 *   (same for V); s_j = scale * <q_i, K_j>; o = sum_j softmax(s)_j V_j.
 * k must already be rotated (nxattn_rope_apply); q too, unless q_rope is given (see
 * below); prefix keys are used as stored. Layouts (element strides {b, s, h},
 * head_dim contiguous):
 *   q [batch, seq_q, heads_q, D]     k, v [batch, seq_q, heads_kv, D]
 *   o [batch, seq_q, heads_q, D]     (written, must not overlap the inputs)
 *   prefix_kv[b]: one layer slice of the online cache, contiguous [2, P_b, heads_kv, D]
 *                 (K at offset 0, V at offset P_b*heads_kv*D); NULL iff P_b == 0.
 * scale <= 0 selects 1/sqrt(head_dim). Accumulation is fp32; P is rounded to bf16
 * before the P*V product on the bf16 path; the output is rounded to nearest even.
 * Supported: BF16 with head_dim 128; F32 with head_dim 64 or 72 (true fp32 MFMA, no
 * reduced-precision inputs); heads_q % heads_kv == 0; batch <= 8; seq_q >= 1; a token
 * stride kv_strides[1] under 2^31 bytes per 64 rows (key tiles are fetched through
 * 32-bit offsets), NXATTN_ERR_UNSUPPORTED otherwise.
 *
 * q_rope (optional, host memory, `batch` descriptors; NULL: q is used as stored):
 * rotate q on load with the RoPE of nxattn_rope_apply (same descriptor meaning and
 * checks, grid product == seq_q), inside the attention kernel, so that no separate
 * pass over q is needed; the q buffer is not modified. Positions (grid coordinate plus
 * offset) must stay below 2^24 (NXATTN_ERR_UNSUPPORTED otherwise). Each pair's step
 * theta^(..)/2pi is evaluated in fp64 and carried as two fp32 parts, and position * step
 * is formed exactly but for the roundings of small terms: the turn is accurate to about
 * 1e-7 revolutions at every supported position, far below the bf16 rounding of the
 * rotated value, and the hardware sine and cosine take it. The rotated value is
 * multiplied by scale * log2(e) (the units of the kernel's base-2 softmax) and rounded
 * once to bf16, nearest even: the q used
 * is that rounding divided by scale * log2(e), as close to the rotated q as a stored
 * bf16 q would be, but rounded at a different point.
 * BF16 only: F32 with q_rope returns NXATTN_ERR_UNSUPPORTED (rotate with
 * nxattn_rope_apply, whose fp64 angles keep the fp32 path exact to 1e-4).
 *
 * The fields after q_rope are off when zero (a zero-initialised struct keeps the
 * behaviour above). They are the softmax normaliser of the same attention (KLiteInfer
 * page, "架构": the softmax between the two GEMMs) and the block form of its online
 * rescale, which a key range split over workgroups, or over devices (the NeoPP
 * replay's sequence-parallel degree), needs.
 *
 * lse (optional, device, fp32 [batch, heads_q, seq_q] contiguous, 4-byte aligned):
 *   lse[b, h, i] = log sum_j exp(s_j), natural log, over the keys of query (b, h, i),
 *   s_j including the scale; then softmax(s)_j = exp(s_j - lse). Must not overlap o or
 *   any input. With it, results over disjoint key sets combine with nxattn_attn_merge.
 * prefix_only (0 or 1): 1 = the keys are the prefix rows alone (every prefix_len[b] >= 1;
 *   k, v and kv_strides are not read and may be NULL / zero). Attention over the own
 *   keys alone is a call with no prefix; the two merge into the full result.
 * num_splits (0 or 1: one pass; 2 .. NXATTN_MAX_SPLITS): the most key ranges a branch
 *   may be cut into. Ranges are `per` whole 64-key tiles long, with
 *     per = max(ceil(max_b tiles_b / num_splits), ceil(W * sum_b tiles_b / slots)),
 *   W the workgroups one key range of one branch takes (all kv heads and query blocks)
 *   and slots the workgroups the GPU holds at once: no range is shorter than a fair
 *   share of the whole problem's work per slot. A branch of at most `per` tiles runs as
 *   one range and writes o (and lse) directly; if that holds for every branch the call
 *   is one pass. The ranges of a longer branch write fp32 partial outputs and
 *   log-sum-exps into the workspace, and a second kernel on the same stream merges them
 *   (the arithmetic of nxattn_attn_merge) into o, and into lse if given. For problems
 *   with too few workgroups to fill the GPU (a short query against a long prefix) or
 *   with branches of very different key counts.
 * workspace, workspace_bytes: with num_splits > 1, 16-byte aligned device memory of at
 *   least nxattn_fwd_workspace_size() bytes, overlapping nothing else; its contents on
 *   entry do not matter and it is busy until the merge kernel has run on `stream`.
 *
 * cfg_out (optional, device; off when NULL): classifier-free guidance folded into the
 * attention call (LingBot-Video page, "Key Parameters": guidance_scale; NeoPP page: the
 * cond and uncond KV branches). BF16, batch 2 (branch 0 cond, branch 1 uncond), and one
 * key range (num_splits 0 or 1) only; NXATTN_ERR_UNSUPPORTED / _INVALID otherwise.
 *   cfg_out[i, h, :] = nxattn_cfg_combine of the two branches' outputs, bit for bit:
 *   fma(guidance, c - u, u) in fp32 on c = o[0, i, h, :] and u = o[1, i, h, :] as rounded
 *   to bf16, rounded to nearest even. Layout [seq_q, heads_q, head_dim], element strides
 *   cfg_strides {s, h} (multiples of 8, head_dim contiguous), 16-byte aligned; it must
 *   not overlap the inputs, o, lse or the workspace. guidance must be finite.
 *   One workgroup serves both branches of its query rows, so no combine pass and no
 *   second reading of the branch outputs is needed. o may be NULL: the branch outputs
 *   are then not stored (lse, if given, is still written for both branches).
 */
typedef struct {
  int32_t dtype;
  int32_t batch;       /* CFG branches                                  */
  int32_t seq_q;       /* own tokens (queries and own keys/values)      */
  int32_t heads_q;
  int32_t heads_kv;
  int32_t head_dim;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t q_strides[3];
  int64_t kv_strides[3];
  int64_t o_strides[3];
  const void* prefix_kv[NXATTN_MAX_BRANCHES];
  int32_t prefix_len[NXATTN_MAX_BRANCHES];
  float scale;
  const nxattn_rope_desc* q_rope;   /* NULL, or batch descriptors (see above)        */
  float* lse;                       /* NULL, or [batch, heads_q, seq_q] fp32 output  */
  int32_t prefix_only;              /* 1: keys = prefix rows only                     */
  int32_t num_splits;               /* 0/1: one pass; 2..NXATTN_MAX_SPLITS key ranges */
  void* workspace;                  /* num_splits > 1: caller's device scratch        */
  int64_t workspace_bytes;
  void* cfg_out;                    /* NULL, or the guidance combination (see above)  */
  int64_t cfg_strides[2];           /* cfg_out element strides {s, h}                 */
  float guidance;
} nxattn_fwd_args;

int nxattn_fwd(const nxattn_fwd_args* args, hipStream_t stream);

/*
 * Workspace bytes that nxattn_fwd needs for args->num_splits (0 when num_splits <= 1):
 * num_splits * batch * seq_q * heads_q * (head_dim + 1) * 4 plus 256 bytes of alignment.
 * Checks only the sizes it reads (NXATTN_ERR_INVALID if negative or out of range).
 */
int nxattn_fwd_workspace_size(const nxattn_fwd_args* args, int64_t* bytes);

/*
 * Merge attention results over disjoint key sets into the result over their union:
 *   lse = log sum_p exp(lse_p),   o = sum_p exp(lse_p - lse) * o_p.
 * The softmax of the KLiteInfer page's "架构" attention over a union of key blocks is
 * the weighted sum of the blocks' normalised outputs (the online-softmax rescale); the
 * NeoPP replay splits work over a sequence-parallel degree, whose key blocks combine
 * this way. Typical use: nxattn_fwd with lse over the own keys (no prefix) and again
 * with prefix_only over each prefix block, then one merge.
 *
 * part_o:   host array of n_parts device pointers, each [batch, seq, heads, head_dim]
 *           of `dtype` with part_strides (elements {b, s, h}; head_dim contiguous).
 * part_lse: host array of n_parts device pointers, each fp32 [batch, heads, seq]
 *           contiguous; -inf marks an empty part (its o_p is then not used). Every row
 *           needs one finite lse_p; a row with none gets NaN.
 * o:        output [batch, seq, heads, head_dim] of `dtype` with o_strides; it may be
 *           exactly one of the parts (same pointer and strides: in-place accumulation).
 * lse:      NULL, or fp32 [batch, heads, seq] contiguous output; it may be exactly one
 *           of part_lse. Any other overlap between outputs and inputs is
 *           NXATTN_ERR_INVALID.
 * Arithmetic in fp32; bf16 output rounded to nearest even. 1 <= n_parts <=
 * NXATTN_MAX_SPLITS; head_dim a multiple of 8, at most 256; dtype F32 or BF16.
 */
int nxattn_attn_merge(const void* const* part_o, const float* const* part_lse, int32_t n_parts,
                      int64_t batch, int64_t seq, int64_t heads, int64_t head_dim,
                      const int64_t part_strides[3], int dtype, void* o, const int64_t o_strides[3],
                      float* lse, hipStream_t stream);

/*
 * FP8 score GEMM. The pages name fp8 variants of the DiT (NeoPP page, "Run the
 * replay examples") without a recipe; the one here: q and k (own and prefix keys) are OCP
 * FP8 E4M3 codes with one power-of-two scale 2^e per (branch, head); the scores are the
 * dot products of the decoded codes times both scales (exact inside the fp8 MFMA, whose
 * E8M0 scale operands carry 2^e); softmax, P (bf16) and the P*V product with bf16 V are
 * those of nxattn_fwd.
 *
 * E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is subnormal
 * (m/8 * 2^-6); S.1111.111 is NaN; the largest finite magnitude is 448.
 *
 * nxattn_quantize_fp8: x [batch, seq, heads, head_dim] of dtype (F32 or BF16; strides
 * {b, s, h} in elements, multiples of 16 bytes; head_dim contiguous, a multiple of 8, at
 * most 1024; heads <= 4096) ->
 *   exps  int8 [batch, heads]: e = the smallest integer with max|x[b, :, h, :]| <= 448 * 2^e,
 *         0 for an all-zero slice, at least -127 (the E8M0 range);
 *   codes uint8 [batch, seq, heads, head_dim] contiguous: the nearest E4M3 value of
 *         x * 2^-e (an exact scaling), ties to the even code; the sign of a value that
 *         rounds to zero is kept; NaN -> 0x7F. x must not hold infinities.
 * workspace: device memory of nxattn_quantize_fp8_workspace_size() bytes (32 running
 * maxima per slice on separate 128-byte lines, 4-byte aligned: 128 * ceil(batch * heads /
 * 32) * 32 bytes; its contents on entry do not matter); x, codes, exps and workspace must
 * not overlap (NXATTN_ERR_INVALID). Four launches on
 * `stream`; bit-exact by construction.
 */
int nxattn_quantize_fp8_workspace_size(int64_t batch, int64_t seq, int64_t heads, int64_t* bytes);
int nxattn_quantize_fp8(const void* x, int dtype, int64_t batch, int64_t seq, int64_t heads, int64_t head_dim,
                        const int64_t strides[3], uint8_t* codes, int8_t* exps, void* workspace,
                        int64_t workspace_bytes, hipStream_t stream);

/*
 * Block scaling, a finer reading of the same recipe: the scale is shared by each run of 32
 * consecutive head_dim elements of one (branch, token, head) row, the block size and scale
 * format of the OCP Microscaling (MX) formats. Inside a run the rule is the one above (e =
 * the smallest integer with max|run| <= 448 * 2^e, 0 for an all-zero run, at least -127;
 * codes of x * 2^-e, nearest even), and the scale is stored as its E8M0 code e + 127
 * (value 2^(code - 127)), the form the fp8 matrix core takes. One scale per run needs no
 * reduction across the tensor, so one pass writes codes and scales.
 *
 * nxattn_quantize_fp8_blocks: x as in nxattn_quantize_fp8 with head_dim a multiple of 32 up
 * to 1024 -> codes uint8 [batch, seq, heads, head_dim] contiguous (8-byte aligned) and
 * scales uint8 [batch, seq, heads, head_dim / 32] contiguous. x, codes and scales must not
 * overlap (NXATTN_ERR_INVALID). One launch on `stream`, no workspace.
 */
int nxattn_quantize_fp8_blocks(const void* x, int dtype, int64_t batch, int64_t seq, int64_t heads,
                               int64_t head_dim, const int64_t strides[3], uint8_t* codes, uint8_t* scales,
                               hipStream_t stream);

/*
 * RoPE and FP8 quantization together, for tensors that share positions (the q and k of
 * the own tokens): for each tensor t, codes_t and exps_t are exactly what
 * nxattn_quantize_fp8 gives for x_t after nxattn_rope_apply(x_t, rope), bit for bit, but
 * x_t is only read. For the fp8 score GEMM the rotated q and k are needed only as codes,
 * so the rotation is evaluated inside the two reading passes (the maxima, then the codes)
 * and never stored, and one evaluation of the angles per token serves the heads of every
 * tensor.
 *
 * tensors[0 .. n_tensors) (host memory, 1 <= n_tensors <= NXATTN_MAX_FP8_TENSORS):
 *   x       [batch, seq, heads, head_dim] of dtype, element strides {b, s, h} (multiples
 *           of 16 bytes; head_dim contiguous), 16-byte aligned; read only (tensors may
 *           share or overlap their x);
 *   codes   out, uint8 [batch, seq, heads, head_dim] contiguous, 8-byte aligned;
 *   exps    out, int8 [batch, heads] (one exponent per slice), or NULL with scales;
 *   scales  out, uint8 [batch, seq, heads, head_dim / 32] E8M0 codes (block scaling, as
 *           nxattn_quantize_fp8_blocks gives for the rotated values), or NULL with exps.
 *           Either every tensor of a call has exps or every one has scales
 *           (NXATTN_ERR_INVALID otherwise); block scaling needs head_dim % 64 == 0, takes
 *           one launch and no workspace (workspace may be NULL, workspace_bytes 0);
 *   mult    with fold_softmax == 0: 0 or 1: none; else a finite multiplier > 0 applied
 *           (fp32 multiply) to each rotated value as stored in dtype before quantization,
 *           so that the codes are those of mult * rope(x).
 *   fold_softmax  0 or 1. 1: the multiplier is c = s * log2(e), formed by the library in
 *           fp32 as fl(s * fl(log2 e)), with s = mult when mult > 0, else the default
 *           softmax scale fl(1 / fl(sqrt(head_dim))) of nxattn_fwd and nxattn_fwd_fp8.
 *           These are the codes of q that nxattn_fwd_fp8 takes with q_folded != 0 (the
 *           scores then arrive in base-2 units), so a caller never forms c itself.
 * Shared: dtype F32 or BF16; head_dim a multiple of 8 in [8, 256]; batch <=
 * NXATTN_MAX_BRANCHES; rope as in nxattn_rope_apply (grid product == seq); the total of
 * the heads at most 4096. workspace (per-slice exponents only):
 * nxattn_quantize_fp8_workspace_size(batch, seq, total heads) bytes, 4-byte aligned,
 * contents on entry irrelevant. No output may overlap an x, another output or the
 * workspace, and no x the workspace (NXATTN_ERR_INVALID). The rotated values must be
 * finite. Three launches on `stream` (one with block scaling).
 */
#define NXATTN_MAX_FP8_TENSORS 4
typedef struct {
  const void* x;
  int64_t heads;
  int64_t strides[3];
  uint8_t* codes;
  int8_t* exps;
  float mult;
  int32_t fold_softmax;
  uint8_t* scales;
} nxattn_fp8_tensor;

int nxattn_rope_quantize_fp8(const nxattn_fp8_tensor* tensors, int32_t n_tensors, int dtype, int64_t batch,
                             int64_t seq, int64_t head_dim, const nxattn_rope_desc* rope, void* workspace,
                             int64_t workspace_bytes, hipStream_t stream);

/*
 * nxattn_rope_quantize_fp8 for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments and
 * results, bit for bit, without the workspace: the running maxima live in a static device
 * array of the library (256 KiB per GPU, held from the first call on a GPU until the
 * process ends), so batch * (total heads) must be at most 2048 (NXATTN_ERR_UNSUPPORTED
 * otherwise). No call allocates. Every call on one GPU shares that GPU's array: calls
 * that overlap in time on one GPU (several streams, or several host threads) race and
 * must be ordered by the caller; the array's contents between calls do not matter (each
 * call clears what it uses with a kernel, no memset). The device is the calling thread's
 * current one; stream must belong to it. Block scaling (tensors with scales) needs no
 * maxima: such a call does not touch the array and has no slice limit.
 */
int nxattn_rope_quantize_fp8_noalloc(const nxattn_fp8_tensor* tensors, int32_t n_tensors, int dtype, int64_t batch,
                                     int64_t seq, int64_t head_dim, const nxattn_rope_desc* rope, hipStream_t stream);

/*
 * Attention of nxattn_fwd with the fp8 score GEMM above (head_dim 128, heads_q % heads_kv
 * == 0, batch <= 8). For branch b, q head h (kv head g = h / (heads_q / heads_kv)):
 *   keys j < P_b: prefix row j (codes prefix_k8[b], exponent prefix_k_exp[b, g]; value
 *   prefix_v[b]), else own row j - P_b (codes k8, exponent k_exp[b, g]; value v);
 *   s_j = scale * 2^(q_exp[b, h] + e_j) * <dec(q8), dec(k8_j)>, o = softmax(s) . V.
 * Layouts: q8 [batch, seq_q, heads_q, 128] and k8 [batch, seq_q, heads_kv, 128] contiguous
 * E4M3 (as nxattn_quantize_fp8 writes them); v, o bf16 with element strides {b, s, h};
 * prefix_k8[b] E4M3 [P_b, heads_kv, 128] contiguous; prefix_v[b] bf16 [P_b, heads_kv, 128]
 * contiguous (the V half of one layer slice of the online cache); exponents int8 in
 * device memory. lse as in nxattn_fwd. Outputs must not overlap inputs. scale <= 0 selects
 * 1/sqrt(128). v's token stride v_strides[1] must span under 2^31 bytes per 64 rows
 * (NXATTN_ERR_UNSUPPORTED otherwise).
 *
 * q_folded != 0: q8 holds the codes of c * q with c = scale * log2(e), as
 * nxattn_rope_quantize_fp8 writes them with fold_softmax = 1. The products then are the scores
 * in base-2 units, s_j * log2(e) = 2^(q_exp + e_j) <dec(q8), dec(k8_j)>, `scale` is not
 * used, and the kernel's softmax takes one exp2 per score with no multiply in front
 * (its score accumulators start at minus the running max), the bf16 kernel's q_rope fold.
 *
 * Block scales (q_scales != NULL): q8, k8 and the prefix codes carry one E8M0 scale per run
 * of 32 head_dim elements of each row, as nxattn_quantize_fp8_blocks and the block mode of
 * nxattn_rope_quantize_fp8 write them, and the dot products sum the runs' products each
 * times its two scales: s_j = scale * sum_r 2^(eq_r + ek_jr) <dec(q8_r), dec(k8_jr)>.
 * q_scales uint8 [batch, seq_q, heads_q, 4], k_scales uint8 [batch, seq_q, heads_kv, 4] and
 * prefix_k_scales[b] uint8 [P_b, heads_kv, 4] (non-NULL iff prefix_len[b] > 0), contiguous
 * and 4-byte aligned; q_exp, k_exp and prefix_k_exp must then be NULL. Without q_scales
 * (or q_rope), k_scales and every prefix_k_scales[b] must be NULL.
 *
 * q rotated and quantized on load (q_rope != NULL, `batch` descriptors in host memory, as
 * nxattn_fwd's q_rope, positions below 2^24): q is bf16 [batch, seq_q, heads_q, 128] with
 * element strides q_strides {b, s, h} (multiples of 16 bytes, 16-byte aligned) and is only
 * read. The kernel rotates each row with the turns of nxattn_fwd's q_rope, multiplies it
 * by c = scale * log2(e) (both in fp32, with no bf16 rounding in between) and forms the
 * codes and run scales of block scaling from those values in registers; the keys take
 * block scales (k_scales, prefix_k_scales). q8, q_scales and q_exp must be NULL and
 * q_folded 0 (the fold is implied). Without q_rope, q must be NULL. Optionally (both
 * non-NULL or both NULL, with q_rope only) the kernel also writes the codes it formed to
 * q8_out (uint8 [batch, seq_q, heads_q, 128] contiguous, 16-byte aligned) and the run
 * scales to q_scales_out (uint8 E8M0 [batch, seq_q, heads_q, 4], 4-byte aligned), as
 * nxattn_fwd_fp8 with q_scales would take them. No output may overlap an input or another
 * output.
 *
 * cfg_out, cfg_strides, guidance (off when cfg_out is NULL): the guidance combination of
 * the two branches written by this call, exactly as in nxattn_fwd (batch 2, branch 0
 * cond; bit for bit nxattn_cfg_combine of the two branches' rounded outputs); o may then
 * be NULL.
 */
typedef struct {
  int32_t batch;
  int32_t seq_q;
  int32_t heads_q;
  int32_t heads_kv;
  int32_t head_dim;                                   /* 128 */
  const uint8_t* q8;
  const uint8_t* k8;
  const int8_t* q_exp;                                /* [batch, heads_q]  */
  const int8_t* k_exp;                                /* [batch, heads_kv] */
  const void* v;
  void* o;
  int64_t v_strides[3];
  int64_t o_strides[3];
  const uint8_t* prefix_k8[NXATTN_MAX_BRANCHES];      /* NULL iff prefix_len[b] == 0 */
  const void* prefix_v[NXATTN_MAX_BRANCHES];          /* NULL iff prefix_len[b] == 0 */
  int32_t prefix_len[NXATTN_MAX_BRANCHES];
  const int8_t* prefix_k_exp;                         /* [batch, heads_kv]; needed if any prefix */
  float scale;
  float* lse;                                         /* NULL, or [batch, heads_q, seq_q] fp32 */
  int32_t q_folded;                                   /* see above */
  const uint8_t* q_scales;                            /* block scales, see above */
  const uint8_t* k_scales;
  const uint8_t* prefix_k_scales[NXATTN_MAX_BRANCHES];
  const void* q;                                      /* q_rope: bf16 q, see above */
  int64_t q_strides[3];
  const nxattn_rope_desc* q_rope;
  uint8_t* q8_out;                                    /* q_rope, optional: codes formed on load */
  uint8_t* q_scales_out;
  void* cfg_out;                                      /* NULL, or the guidance combination      */
  int64_t cfg_strides[2];                             /* (as in nxattn_fwd_args)                */
  float guidance;
} nxattn_fwd_fp8_args;

int nxattn_fwd_fp8(const nxattn_fwd_fp8_args* args, hipStream_t stream);

/*
 * Classifier-free guidance: out = uncond + guidance * (cond - uncond) over n elements.
 * LingBot-Video page, "Key Parameters": guidance_scale, guidance active above 1.0;
 * NeoPP page: the two KV branches (cond, uncond). The combination is evaluated in
 * fp32 as fma(guidance, cond - uncond, uncond). out may alias cond or uncond exactly
 * (any other overlap is NXATTN_ERR_INVALID).
 */
int nxattn_cfg_combine(const void* cond, const void* uncond, void* out, int64_t n, float guidance,
                       int dtype, hipStream_t stream);

/* Static description of a status code. */
const char* nxattn_status_string(int status);
/* Detail of the last failing call on the calling thread ("" if none). */
const char* nxattn_last_error(void);
/* Library version, e.g. "0.1.0". */
const char* nxattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NXATTN_H */
