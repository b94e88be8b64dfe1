// The no-allocation variant of nxattn_rope_quantize_fp8, for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops, harnesses that
// forbid hipMalloc): the running maxima that the caller's workspace holds in the plain
// entry point live in a static device array of this file instead.
#include <mutex>

#include "nx_internal.h"

namespace {

using namespace nx;

// The no-allocation variant's scratch: the running maxima of at most NOALLOC_SLICES
// (branch, head) slices (AMAX_SLOTS line-separated copies each, 256 KiB). Every GPU that
// runs the variant holds its own copy until the process ends. In host code `scratch` only
// names the variable: its device address on the current GPU comes from
// hipGetSymbolAddress, looked up once per device and kept in g_scratch.
constexpr int64_t NOALLOC_SLICES = 2048;
constexpr int64_t NOALLOC_WORDS = AMAX_SLOTS * NOALLOC_SLICES;
static __device__ __align__(256) uint32_t scratch[NOALLOC_WORDS];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch[MAX_DEVICES] = {};

// Device address of `scratch` on the current device (looked up on the first call there).
int scratch_address(const char* who, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
    return fail(NXATTN_ERR_HIP, "%s: cannot query the current device", who);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(NXATTN_ERR_HIP, "%s: hipGetSymbolAddress of the scratch failed: %s", who, hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return NXATTN_OK;
}

}  // namespace

using namespace nx;

extern "C" int nxattn_rope_quantize_fp8_noalloc(const nxattn_fp8_tensor* tensors, int32_t n_tensors, int dtype,
                                                int64_t batch, int64_t seq, int64_t head_dim,
                                                const nxattn_rope_desc* rope, hipStream_t stream) {
  static const char* who = "nxattn_rope_quantize_fp8_noalloc";
  clear_error();
  if (!tensors || n_tensors < 1 || n_tensors > NXATTN_MAX_FP8_TENSORS)
    return fail(NXATTN_ERR_INVALID, "%s: need 1 to %d tensors", who, NXATTN_MAX_FP8_TENSORS);
  if (batch < 0) return fail(NXATTN_ERR_INVALID, "%s: negative size", who);
  if (batch > NXATTN_MAX_BRANCHES) return fail(NXATTN_ERR_UNSUPPORTED, "%s: batch > %d", who, NXATTN_MAX_BRANCHES);
  int64_t total = 0;
  for (int t = 0; t < n_tensors; ++t) {
    if (tensors[t].heads < 0) return fail(NXATTN_ERR_INVALID, "%s: negative heads", who);
    total += tensors[t].heads;
  }
  // block scaling keeps no running maxima: the scratch is not used (rope_quantize checks
  // that every tensor with heads has the same kind of scale)
  bool blocks = false;
  for (int t = 0; t < n_tensors; ++t)
    if (tensors[t].heads > 0) { blocks = tensors[t].scales != nullptr; break; }
  if (blocks)
    return rope_quantize(who, tensors, n_tensors, dtype, batch, seq, head_dim, rope, nullptr, 0, stream);
  if (batch * total > NOALLOC_SLICES)
    return fail(NXATTN_ERR_UNSUPPORTED,
                "%s: batch * total heads = %lld exceeds the %lld (branch, head) slices of the static scratch; "
                "use nxattn_rope_quantize_fp8 with a workspace", who, (long long)(batch * total),
                (long long)NOALLOC_SLICES);
  void* ws = nullptr;
  const int st = scratch_address(who, &ws);
  if (st != NXATTN_OK) return st;
  // the maxima are cleared by the call's first launch, so whatever an earlier call left
  // in the scratch does not matter
  return rope_quantize(who, tensors, n_tensors, dtype, batch, seq, head_dim, rope, ws, NOALLOC_WORDS * 4, stream);
}
