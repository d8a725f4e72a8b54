// Launch interface of the kernels beside the decode path: the unfused baseline and the
// error-budget diagnostics.
#pragma once
#include "kvq_internal.h"

// Unfused baseline: dense bf16 cache [B][Hkv][max_len][128] and dense decode attention over it.
struct KvqDenseArgs {
  KvqLayout lay;
  KvqCacheDev cache;
  const int32_t *seq_lens;
  uint16_t *k_out, *v_out;           // dequantize: written
  const uint16_t *k_in, *v_in;       // attention: read
  const void *q;
  float *partials;                   // [B][Hq][S][KVQ_PART_STRIDE]
  int64_t max_len;
  int32_t B, Hq, Hkv, R, kv_f32, q_f32, rotation, value_rotation, splits;
  float sigma;                       // softmax scale * log2(e)
};
#define KVQ_DENSE_SPLIT 256  // tokens per split of the dense attention
hipError_t kvq_launch_dequantize_dense(const KvqDenseArgs &a, hipStream_t s);
hipError_t kvq_launch_dense_partials(const KvqDenseArgs &a, int g, hipStream_t s);

// Error-budget diagnostics against the original keys and values.
struct KvqErrArgs {
  KvqLayout lay;
  KvqCacheDev cache;
  const int32_t *seq_lens;
  const uint16_t *k_ref, *v_ref;  // bf16 [B][max_len][Hkv][128]
  const void *q;
  float *head_stats, *unit_stats;
  int64_t max_len;
  int32_t B, Hq, Hkv, R, q_f32;
  int32_t rotation, value_rotation;  // stored keys / values are rotated
  float scale;
  float *ws;       // workspace: kvq_errbudget_item_floats() floats per (unit, head group, range)
  int32_t splits;  // ranges of pages per sequence
};
int kvq_errbudget_heads_per_group(int g);
size_t kvq_errbudget_item_floats();
size_t kvq_errbudget_score_stride(int64_t max_len);  // positions per row of the stored scores
hipError_t kvq_launch_errbudget(const KvqErrArgs &a, hipStream_t s);
