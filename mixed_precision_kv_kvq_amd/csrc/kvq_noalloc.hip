// Decode attention for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): the same two launches as
// kvq_decode_attention, with the split partial rows kept in a file-scope device array instead
// of a caller-provided workspace.
//
// The array is a module global: every GPU the library runs on holds its own copy, at its own
// address, from the first call on that GPU until the process ends.  In host code `scratch` is
// only a stand-in for the symbol, not a device address, so the address of each device's copy
// is looked up once per device (hipGetSymbolAddress, with that device current) and only that
// address is ever handed to a kernel.  The partial rows need no initial contents (every row the
// merge reads is written by the split kernel of the same call), so nothing is cleared.  Calls
// on one GPU share its array: calls that overlap in time on that GPU (different streams, no
// ordering between them) race on it.
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/kvq.h"

namespace {

static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_ptr[kMaxDevices] = {};

// Address of `scratch` on device `dev` (looked up once per device, with that device current).
hipError_t scratch_address(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_ptr[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" kvq_status kvq_decode_attention_noalloc(const kvq_params *params, const kvq_cache *cache,
                                                   const int32_t *seq_lens, int64_t max_seq_len, const void *q,
                                                   int32_t q_dtype, void *out, int32_t out_dtype, float softmax_scale,
                                                   hipStream_t stream) {
  if (!cache) return KVQ_EINVAL;
  const size_t need = kvq_decode_workspace_bytes(params, cache->batch, max_seq_len);
  if (need == 0) {
    // invalid parameters: let the regular entry point report which status applies
    return kvq_decode_attention(params, cache, seq_lens, max_seq_len, q, q_dtype, out, out_dtype, softmax_scale,
                                nullptr, 0, stream);
  }
  if (need > (size_t)KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ENOSPACE;
  int dev = -1;
  if (stream) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return KVQ_EHIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return KVQ_EHIP;
  }
  void *ws = nullptr;
  if (scratch_address(dev, &ws) != hipSuccess) return KVQ_EHIP;
  return kvq_decode_attention(params, cache, seq_lens, max_seq_len, q, q_dtype, out, out_dtype, softmax_scale, ws,
                              (size_t)KVQ_NOALLOC_SCRATCH_BYTES, stream);
}
