// Internal launch interface between the C-ABI front end and the kernels.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/kvq.h"
#include "kvq_layout.h"

// 2^-3.5 rounded to fp64 (the normalization of the 128-point Hadamard transform).
#define KVQ_WHT_C 0x1.6a09e667f3bcdp-4

struct KvqCacheDev {
  uint8_t *pages;
  uint8_t *k_win, *v_win;
  const int32_t *block_table;
  int32_t batch, mbps;
  int64_t pages_per_seq;  // contiguous mode
  int64_t pool_pages;     // paged mode: pages in the pool
  int paged;
};

struct KvqAppendArgs {
  KvqLayout lay;
  KvqCacheDev cache;
  const int32_t *seq_lens_before;
  const int32_t *n_new_per_seq;
  const uint8_t *k_new, *v_new;
  int32_t n_new, Hkv, R, rotation, kv_f32;
};

struct KvqAttnArgs {
  KvqLayout lay;
  KvqCacheDev cache;
  const int32_t *seq_lens;
  const void *q;
  float *partials;  // [B][Hq][S][KVQ_PART_STRIDE]
  int32_t q_f32, kv_f32, Hq, Hkv, R, rotation;
  int32_t splits, pages_per_split;  // all splits; quantized pages per quantized split
  int32_t wsplits;                   // leading splits that cover the recent window, KVQ_WIN_PAGES pages each
  int32_t max_len;  // host-validated upper bound of seq_lens (device lengths are clamped to it)
  float sigma_u;  // softmax_scale * log2(e) * 2^33
};

struct KvqCombineArgs {
  const float *partials;
  void *out;
  int32_t out_f32, B, Hq, splits;
};

struct KvqDebugArgs {
  KvqLayout lay;
  KvqCacheDev cache;
  const int32_t *seq_lens;
  int32_t seq, Hkv, R, kv_f32;
  int64_t t0, n;
  uint8_t *k_codes, *v_codes;
  uint16_t *k_meta, *v_meta;
  float *k_hat, *v_hat;
};

#define KVQ_PART_STRIDE 132
#define KVQ_WIN_PAGES 8  // window pages (128 tokens) per window split

// Waves per SIMD the split kernel is compiled for (register budget 512 / KVQ_WPE).
#ifndef KVQ_WPE
#define KVQ_WPE 3
#endif

#define KVQ_LDS_PER_CU (160 * 1024)

// Page-pair slots of the split kernel's LDS prefetch ring for a given pair size:
// as many as fit in the LDS share of one wave at the compiled occupancy, 2..4.
__host__ __device__ constexpr int kvq_ring_slots(int pair_bytes) {
  return (KVQ_LDS_PER_CU / (4 * KVQ_WPE)) / pair_bytes < 2
             ? 2
             : ((KVQ_LDS_PER_CU / (4 * KVQ_WPE)) / pair_bytes > 4 ? 4 : (KVQ_LDS_PER_CU / (4 * KVQ_WPE)) / pair_bytes);
}

// LDS bytes of one split-kernel workgroup (one wave) for key/value bit widths and value groups.
__host__ __device__ constexpr int kvq_attn_lds_bytes(int kb, int vb, int nvg) {
  return (2 * (((16 * kb + 16 + 16 * vb + 4 * nvg) + 63) / 64) * 1024) * kvq_ring_slots(2 * (((16 * kb + 16 + 16 * vb + 4 * nvg) + 63) / 64) * 1024) >
                 (2 * 8 * 128 + 8 * 4) * 4
             ? (2 * (((16 * kb + 16 + 16 * vb + 4 * nvg) + 63) / 64) * 1024) *
                   kvq_ring_slots(2 * (((16 * kb + 16 + 16 * vb + 4 * nvg) + 63) / 64) * 1024)
             : (2 * 8 * 128 + 8 * 4) * 4;
}

// Resident split-kernel waves per CU: the register limit or the LDS limit.
__host__ __device__ constexpr int kvq_attn_waves_per_cu(int kb, int vb, int nvg) {
  return (4 * KVQ_WPE) < (KVQ_LDS_PER_CU / kvq_attn_lds_bytes(kb, vb, nvg)) ? 4 * KVQ_WPE
                                                                           : KVQ_LDS_PER_CU / kvq_attn_lds_bytes(kb, vb, nvg);
}  // floats per partial: m, l, pad, pad, acc[128]

hipError_t kvq_launch_append(const KvqAppendArgs &a, hipStream_t s);
hipError_t kvq_launch_attention(const KvqAttnArgs &a, int g, int q_parts, hipStream_t s);
hipError_t kvq_launch_combine(const KvqCombineArgs &a, hipStream_t s);
hipError_t kvq_launch_debug(const KvqDebugArgs &a, hipStream_t s);
bool kvq_attention_supported(int kb, int vb, int g, int q_parts, int nvg);
