// Host-side stand-ins for the device launches and the two HIP runtime calls of the C-ABI front end,
// for a sanitized host-only build of kvq_api.cpp (no GPU, no HIP runtime).  Each launch records
// that it happened and touches the first and the last element its kernels would address in the
// caller's workspace, using the kernels' own index formulas, so that AddressSanitizer reports a
// workspace whose documented size is too small.  The workspaces of these runs are host buffers of
// exactly the documented size; every other pointer is a stand-in never dereferenced.
#include <stdio.h>
#include <stdlib.h>

#include "../../mixed_precision_kv_kvq_amd/csrc/kvq_extras.h"

int stub_launches = 0;
int stub_last_splits = 0;

static void touch(const float *base, size_t n) {
  if (n == 0) return;
  volatile float sink = base[0];
  sink = base[n - 1];
  (void)sink;
}

hipError_t kvq_launch_append(const KvqAppendArgs &a, hipStream_t) {
  ++stub_launches;
  if (a.n_new <= 0 || a.Hkv <= 0) abort();
  return hipSuccess;
}

hipError_t kvq_launch_attention(const KvqAttnArgs &a, int g, int q_parts, hipStream_t) {
  ++stub_launches;
  stub_last_splits = a.splits;
  if (a.splits < 1 || a.grid < 1 || g < 1 || q_parts < 1 || q_parts > 2) abort();
  // write_partial: row ((b * Hq + h) * splits + split) of KVQ_PART_STRIDE floats
  touch(a.partials, (size_t)a.cache.batch * a.Hq * a.splits * KVQ_PART_STRIDE);
  return hipSuccess;
}

hipError_t kvq_launch_combine(const KvqCombineArgs &a, hipStream_t) {
  ++stub_launches;
  if (a.splits < 1) abort();
  touch(a.partials, (size_t)a.B * a.Hq * a.splits * KVQ_PART_STRIDE);
  return hipSuccess;
}

hipError_t kvq_launch_debug(const KvqDebugArgs &a, hipStream_t) {
  ++stub_launches;
  if (a.n < 0) abort();
  return hipSuccess;
}

hipError_t kvq_launch_dequantize_dense(const KvqDenseArgs &a, hipStream_t) {
  ++stub_launches;
  if (a.B < 1) abort();
  return hipSuccess;
}

hipError_t kvq_launch_dense_partials(const KvqDenseArgs &a, int g, hipStream_t) {
  ++stub_launches;
  stub_last_splits = a.splits;
  if (a.splits < 1 || g < 1) abort();
  touch(a.partials, (size_t)a.B * a.Hq * a.splits * KVQ_PART_STRIDE);
  return hipSuccess;
}

// The error-budget kernels' plan constants, as the kernels define them: up to 4 query heads per
// workgroup, 2112-float items, score rows of whole 16-position pages.
int kvq_errbudget_heads_per_group(int g) { return g < 4 ? g : 4; }
size_t kvq_errbudget_item_floats() { return 2112; }
size_t kvq_errbudget_score_stride(int64_t max_len) { return (size_t)((max_len + 15) / 16) * 16; }

hipError_t kvq_launch_errbudget(const KvqErrArgs &a, hipStream_t) {
  ++stub_launches;
  stub_last_splits = a.splits;
  const int g = a.Hq / a.Hkv, ngrp = g / kvq_errbudget_heads_per_group(g);
  if (a.splits < 1 || ngrp < 1) abort();
  const size_t items = (size_t)a.B * a.Hkv * ngrp * a.splits;
  touch(a.ws, items * kvq_errbudget_item_floats() + (size_t)a.B * a.Hq * kvq_errbudget_score_stride(a.max_len) * 2);
  return hipSuccess;
}

extern "C" hipError_t hipMemcpyAsync(void *dst, const void *, size_t n, hipMemcpyKind, hipStream_t) {
  if (n == sizeof(uint32_t)) *(uint32_t *)dst = 0;
  return hipSuccess;
}
extern "C" hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
