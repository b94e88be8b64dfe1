// Host side of the nxattn C ABI: error reporting, status strings and the validation
// and dispatch of nxattn_fwd (the relayout, RoPE and CFG entry points live beside
// their kernels).
#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>

#include "nx_internal.h"

namespace nx {

static thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

void clear_error() { g_last_error.clear(); }

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(NXATTN_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return NXATTN_OK;
}

// Workspace of a split-key nxattn_fwd: fp32 partial outputs, then (256-byte aligned)
// their log-sum-exp. Returns false if the sizes are out of range.
struct SplitLayout { int64_t o_bytes, lse_offset, total; };
static bool split_layout(int64_t ns, int64_t batch, int64_t seq, int64_t heads, int64_t d, SplitLayout* L) {
  if (ns < 0 || batch < 0 || seq < 0 || heads < 0 || d < 0) return false;
  if (ns <= 1) { *L = SplitLayout{0, 0, 0}; return true; }
  const double approx = (double)ns * batch * seq * heads * (d + 1) * 4.0;
  if (approx > 4.0e18) return false;
  const int64_t rows = ns * batch * seq * heads;
  L->o_bytes = rows * d * 4;
  L->lse_offset = (L->o_bytes + 255) / 256 * 256;
  L->total = L->lse_offset + rows * 4 + 256;
  return true;
}

}  // namespace nx

using namespace nx;

extern "C" const char* nxattn_status_string(int status) {
  switch (status) {
    case NXATTN_OK: return "ok";
    case NXATTN_ERR_INVALID: return "invalid argument";
    case NXATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case NXATTN_ERR_ALIGN: return "misaligned pointer or stride";
    case NXATTN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

extern "C" const char* nxattn_last_error(void) { return g_last_error.c_str(); }

extern "C" const char* nxattn_version(void) { return "0.1.0"; }

extern "C" int nxattn_fwd_workspace_size(const nxattn_fwd_args* a, int64_t* bytes) {
  clear_error();
  if (!a || !bytes) return fail(NXATTN_ERR_INVALID, "nxattn_fwd_workspace_size: NULL argument");
  if (a->num_splits < 0 || a->num_splits > NXATTN_MAX_SPLITS)
    return fail(NXATTN_ERR_INVALID, "nxattn_fwd_workspace_size: num_splits %d not in [0, %d]", a->num_splits,
                NXATTN_MAX_SPLITS);
  SplitLayout L;
  if (!split_layout(a->num_splits, a->batch, a->seq_q, a->heads_q, a->head_dim, &L))
    return fail(NXATTN_ERR_INVALID, "nxattn_fwd_workspace_size: bad sizes");
  *bytes = L.total;
  return NXATTN_OK;
}

extern "C" int nxattn_fwd(const nxattn_fwd_args* a, hipStream_t stream) {
  clear_error();
  if (!a) return fail(NXATTN_ERR_INVALID, "nxattn_fwd: args is NULL");
  if (a->dtype != NXATTN_F32 && a->dtype != NXATTN_BF16)
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd: dtype %d is not F32 or BF16", a->dtype);
  if (a->batch < 0 || a->seq_q < 0 || a->heads_q <= 0 || a->heads_kv <= 0 || a->head_dim <= 0)
    return fail(NXATTN_ERR_INVALID, "nxattn_fwd: bad sizes batch=%d seq_q=%d heads_q=%d heads_kv=%d head_dim=%d",
                a->batch, a->seq_q, a->heads_q, a->heads_kv, a->head_dim);
  if (a->batch > NXATTN_MAX_BRANCHES)
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd: batch %d > %d", a->batch, NXATTN_MAX_BRANCHES);
  if (a->heads_q % a->heads_kv != 0)
    return fail(NXATTN_ERR_INVALID, "nxattn_fwd: heads_q %d is not a multiple of heads_kv %d", a->heads_q, a->heads_kv);
  if (a->heads_q > 4096) return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd: heads_q %d > 4096", a->heads_q);
  if (a->dtype == NXATTN_BF16 && a->head_dim != 128)
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd: bf16 supports head_dim 128, got %d", a->head_dim);
  if (a->dtype == NXATTN_F32 && a->head_dim != 64 && a->head_dim != 72)
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd: f32 supports head_dim 64 or 72, got %d", a->head_dim);
  if (!(a->scale == a->scale) || std::isinf(a->scale)) return fail(NXATTN_ERR_INVALID, "nxattn_fwd: scale is not finite");
  if (a->prefix_only != 0 && a->prefix_only != 1)
    return fail(NXATTN_ERR_INVALID, "nxattn_fwd: prefix_only must be 0 or 1, got %d", a->prefix_only);
  if (a->num_splits < 0 || a->num_splits > NXATTN_MAX_SPLITS)
    return fail(NXATTN_ERR_INVALID, "nxattn_fwd: num_splits %d not in [0, %d]", a->num_splits, NXATTN_MAX_SPLITS);
  for (int b = 0; b < a->batch; ++b) {
    if (a->prefix_len[b] < 0) return fail(NXATTN_ERR_INVALID, "nxattn_fwd: prefix_len[%d] < 0", b);
    if (a->prefix_only && a->prefix_len[b] == 0)
      return fail(NXATTN_ERR_INVALID, "nxattn_fwd: prefix_only needs prefix_len[%d] >= 1", b);
    if ((a->prefix_len[b] > 0) != (a->prefix_kv[b] != nullptr))
      return fail(NXATTN_ERR_INVALID, "nxattn_fwd: prefix_kv[%d] must be non-NULL iff prefix_len[%d] > 0", b, b);
    if ((int64_t)a->prefix_len[b] + a->seq_q > INT32_MAX)
      return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd: prefix_len[%d] + seq_q overflows int32", b);
  }
  if (a->q_rope && a->dtype != NXATTN_BF16)
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd: q_rope is supported for BF16 only");
  // branch pairs: the guidance combination written by the attention kernel itself
  const bool pair = a->cfg_out != nullptr;
  if (pair) {
    if (a->dtype != NXATTN_BF16) return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd: cfg_out is supported for BF16 only");
    if (a->batch != 2) return fail(NXATTN_ERR_INVALID, "nxattn_fwd: cfg_out needs batch 2 (cond, uncond), got %d", a->batch);
    if (a->num_splits > 1) return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd: cfg_out with num_splits > 1");
    if (!(a->guidance == a->guidance) || std::isinf(a->guidance))
      return fail(NXATTN_ERR_INVALID, "nxattn_fwd: guidance is not finite");
    for (int i = 0; i < 2; ++i) {
      if (a->cfg_strides[i] < 0) return fail(NXATTN_ERR_INVALID, "nxattn_fwd: negative cfg stride");
      if ((a->cfg_strides[i] * 2) % 16 != 0)
        return fail(NXATTN_ERR_ALIGN, "nxattn_fwd: cfg stride %lld is not a multiple of 16 bytes", (long long)a->cfg_strides[i]);
    }
    if (!aligned16(a->cfg_out)) return fail(NXATTN_ERR_ALIGN, "nxattn_fwd: cfg_out must be 16-byte aligned");
  }
  if (a->batch == 0 || a->seq_q == 0) return NXATTN_OK;
  RopeQ rq[NXATTN_MAX_BRANCHES];
  std::memset(rq, 0, sizeof(rq));
  if (a->q_rope) {
    const int st = rope_q_setup(a->q_rope, a->batch, a->seq_q, a->head_dim, "nxattn_fwd (q_rope)", rq);
    if (st != NXATTN_OK) return st;
  }
  // own k and v are not read with prefix_only
  const bool own = !a->prefix_only;
  if (!a->q || (!a->o && !pair) || (own && (!a->k || !a->v))) return fail(NXATTN_ERR_INVALID, "nxattn_fwd: NULL q/k/v/o");
  const int64_t es = esize(a->dtype);
  const int64_t* sts[3] = {a->q_strides, a->kv_strides, a->o_strides};
  for (int t = 0; t < 3; ++t)
    for (int i = 0; i < 3; ++i) {
      if ((t == 1 && !own) || (t == 2 && !a->o)) continue;
      if (sts[t][i] < 0) return fail(NXATTN_ERR_INVALID, "nxattn_fwd: negative stride");
      if (!stride16(sts[t][i], es)) return fail(NXATTN_ERR_ALIGN, "nxattn_fwd: stride %lld is not a multiple of 16 bytes", (long long)sts[t][i]);
    }
  // key tiles (64 rows) are fetched through raw buffers with 32-bit byte offsets
  if (own && a->kv_strides[1] > INT32_MAX / (es * KEY_TILE))
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd: kv token stride %lld elements spans 2 GiB or more per %d rows",
                (long long)a->kv_strides[1], KEY_TILE);
  if (!aligned16(a->q) || (a->o && !aligned16(a->o)) || (own && (!aligned16(a->k) || !aligned16(a->v))))
    return fail(NXATTN_ERR_ALIGN, "nxattn_fwd: q/k/v/o must be 16-byte aligned");
  for (int b = 0; b < a->batch; ++b)
    if (a->prefix_kv[b] && !aligned16(a->prefix_kv[b])) return fail(NXATTN_ERR_ALIGN, "nxattn_fwd: prefix_kv[%d] misaligned", b);
  if (a->lse && (reinterpret_cast<uintptr_t>(a->lse) & 3u))
    return fail(NXATTN_ERR_ALIGN, "nxattn_fwd: lse is not 4-byte aligned");
  // outputs (o, lse, workspace) must not overlap any input or each other
  const int64_t D = a->head_dim;
  const int64_t ob = a->o ? span_bytes(a->o_strides, a->batch, a->seq_q, a->heads_q, D, es) : 0;
  const int64_t qb = span_bytes(a->q_strides, a->batch, a->seq_q, a->heads_q, D, es);
  const int64_t kb = own ? span_bytes(a->kv_strides, a->batch, a->seq_q, a->heads_kv, D, es) : 0;
  const int64_t lb = a->lse ? (int64_t)a->batch * a->heads_q * a->seq_q * 4 : 0;
  int ns = a->num_splits > 1 ? a->num_splits : 1;
  SplitLayout L;
  if (!split_layout(ns, a->batch, a->seq_q, a->heads_q, D, &L)) return fail(NXATTN_ERR_INVALID, "nxattn_fwd: bad sizes");
  if (ns > 1) {
    if (!a->workspace) return fail(NXATTN_ERR_INVALID, "nxattn_fwd: num_splits > 1 needs a workspace");
    if (!aligned16(a->workspace)) return fail(NXATTN_ERR_ALIGN, "nxattn_fwd: workspace is not 16-byte aligned");
    if (a->workspace_bytes < L.total)
      return fail(NXATTN_ERR_INVALID, "nxattn_fwd: workspace_bytes %lld < %lld needed for %d splits",
                  (long long)a->workspace_bytes, (long long)L.total, ns);
  }
  const int64_t wb = ns > 1 ? L.total : 0;
  const int64_t cst[3] = {0, a->cfg_strides[0], a->cfg_strides[1]};
  const int64_t cb = pair ? span_bytes(cst, 1, a->seq_q, a->heads_q, D, es) : 0;
  if (ob < 0 || qb < 0 || kb < 0 || cb < 0)
    return fail(NXATTN_ERR_UNSUPPORTED, "nxattn_fwd: q, k, v, o or cfg_out strides span more than 2^50 bytes");
  struct Span { const void* p; int64_t n; const char* name; };
  const Span outs[4] = {{a->o, ob, "o"}, {a->lse, lb, "lse"}, {a->workspace, wb, "workspace"}, {a->cfg_out, cb, "cfg_out"}};
  for (int i = 0; i < 4; ++i) {
    const Span& x = outs[i];
    if (!x.p || x.n == 0) continue;
    if (overlaps(x.p, x.n, a->q, qb) || overlaps(x.p, x.n, a->k, kb) || overlaps(x.p, x.n, a->v, kb))
      return fail(NXATTN_ERR_INVALID, "nxattn_fwd: %s overlaps q, k or v", x.name);
    for (int b = 0; b < a->batch; ++b)
      if (a->prefix_kv[b] && overlaps(x.p, x.n, a->prefix_kv[b], 2LL * a->prefix_len[b] * a->heads_kv * D * es))
        return fail(NXATTN_ERR_INVALID, "nxattn_fwd: %s overlaps prefix_kv[%d]", x.name, b);
    for (int j = 0; j < i; ++j)
      if (outs[j].p && overlaps(x.p, x.n, outs[j].p, outs[j].n))
        return fail(NXATTN_ERR_INVALID, "nxattn_fwd: %s overlaps %s", x.name, outs[j].name);
  }

  FwdProblem p;
  p.dtype = a->dtype; p.batch = a->batch; p.seq_q = a->seq_q; p.heads_q = a->heads_q;
  p.heads_kv = a->heads_kv; p.head_dim = a->head_dim;
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->o;
  for (int i = 0; i < 3; ++i) { p.qs[i] = a->q_strides[i]; p.ks[i] = a->kv_strides[i]; p.os[i] = a->o_strides[i]; }
  for (int b = 0; b < NXATTN_MAX_BRANCHES; ++b) {
    p.prefix[b] = b < a->batch ? a->prefix_kv[b] : nullptr;
    p.plen[b] = b < a->batch ? a->prefix_len[b] : 0;
  }
  p.scale = a->scale > 0.f ? a->scale : 1.0f / std::sqrt((float)a->head_dim);
  p.rope_q = a->q_rope != nullptr;
  std::memcpy(p.rq, rq, sizeof(p.rq));
  p.cfg = a->cfg_out;
  p.cs[0] = pair ? a->cfg_strides[0] : 0;
  p.cs[1] = pair ? a->cfg_strides[1] : 0;
  p.guidance = pair ? a->guidance : 0.f;
  // Key ranges of `per` whole tiles. The range length is at least ceil(max tiles /
  // num_splits) and at least the tile work per resident workgroup slot of the GPU
  // (sum over branches of tiles * workgroups per range, over the workgroups the GPU
  // holds at once): ranges no shorter than a fair share leave no slot idle while one
  // runs, and a branch shorter than a range stays whole (no partial, no merge). With
  // per >= every branch's tiles the call is one pass.
  int64_t tmax = 0, tsum = 0;
  int32_t tiles[NXATTN_MAX_BRANCHES] = {0};
  for (int b = 0; b < a->batch; ++b) {
    const int64_t skv = (int64_t)a->prefix_len[b] + (own ? a->seq_q : 0);
    tiles[b] = (int32_t)((skv + KEY_TILE - 1) / KEY_TILE);
    if (tiles[b] > tmax) tmax = tiles[b];
    tsum += tiles[b];
  }
  p.prefix_only = a->prefix_only;
  int64_t per = tmax;
  if (ns > 1) {
    const FwdShape sh = a->dtype == NXATTN_BF16 ? fwd_shape_bf16(p) : fwd_shape_f32(p);
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      return fail(NXATTN_ERR_HIP, "nxattn_fwd: cannot query the device's compute units");
    const int64_t slots = (int64_t)cus * sh.resident_per_cu;
    const int64_t fair = (sh.wgs_per_range * tsum + slots - 1) / slots;
    per = std::max<int64_t>((tmax + ns - 1) / ns, fair);
    if (per >= tmax) { per = tmax; ns = 1; }
    else ns = (int)((tmax + per - 1) / per);
  }
  p.lse = a->lse;
  p.nsplit = ns;
  p.per = (int32_t)per;
  p.part_o = ns > 1 ? static_cast<float*>(a->workspace) : nullptr;
  p.part_lse = ns > 1 ? reinterpret_cast<float*>(static_cast<char*>(a->workspace) + L.lse_offset) : nullptr;
  const int st = a->dtype == NXATTN_BF16 ? launch_fwd_bf16(p, stream) : launch_fwd_f32(p, stream);
  if (st != NXATTN_OK || ns == 1) return st;

  // merge the key ranges of each branch into o (and lse)
  MergeProblem m;
  std::memset(&m, 0, sizeof(m));
  const int64_t part_rows = (int64_t)a->batch * a->seq_q * a->heads_q;
  for (int s = 0; s < ns; ++s) {
    m.po[s] = p.part_o + s * part_rows * D;
    m.pl[s] = p.part_lse + s * part_rows;
  }
  m.per_branch = 1;
  for (int b = 0; b < a->batch; ++b) m.nparts[b] = (tiles[b] + p.per - 1) / p.per;
  m.in_dtype = NXATTN_F32; m.out_dtype = a->dtype;
  m.batch = a->batch; m.seq = a->seq_q; m.heads = a->heads_q; m.head_dim = D;
  m.is[0] = (int64_t)a->seq_q * a->heads_q * D; m.is[1] = (int64_t)a->heads_q * D; m.is[2] = D;
  for (int i = 0; i < 3; ++i) m.os[i] = a->o_strides[i];
  m.o = a->o; m.lse = a->lse;
  return launch_merge(m, stream);
}

int nx::rope_q_setup(const nxattn_rope_desc* d, int batch, int64_t seq, int64_t head_dim, const char* who,
                     RopeQ* out) {
  for (int b = 0; b < batch; ++b) {
    const int st = check_rope_desc(d[b], seq, head_dim, who);
    if (st != NXATTN_OK) return st;
    for (int ax = 0; ax < d[b].n_axes; ++ax)
      if ((int64_t)d[b].offset[ax] + d[b].grid[ax] - 1 >= (1 << 24))
        return fail(NXATTN_ERR_UNSUPPORTED, "%s: positions must stay below 2^24 (rotate q with nxattn_rope_apply "
                    "instead)", who);
    RopeQ& r = out[b];
    r.n_axes = d[b].n_axes; r.interleaved = d[b].interleaved; r.global_freq = d[b].global_freq;
    r.log2_theta = std::log2(d[b].theta);
    for (int ax = 0; ax < 3; ++ax) {
      r.grid[ax] = ax < d[b].n_axes ? d[b].grid[ax] : 1;
      r.pairs[ax] = ax < d[b].n_axes ? d[b].pairs[ax] : 0;
      r.offset[ax] = ax < d[b].n_axes ? d[b].offset[ax] : 0;
    }
  }
  return NXATTN_OK;
}
