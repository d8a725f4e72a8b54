// Internal launch interface between the C-ABI front end and the kernels.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/kvq.h"
#include "kvq_layout.h"

// 2^-3.5 rounded to fp64 (the normalization of the 128-point Hadamard transform).
#define KVQ_WHT_C 0x1.6a09e667f3bcdp-4

// Normalized 128-point Walsh-Hadamard transform of a row held two channels per lane (lane l:
// channels 2l, 2l + 1) in fp64: butterflies in stage order 1, 2, ..., 64, then the multiply
// by KVQ_WHT_C.  The matrix is symmetric and orthogonal, so the transform is its own inverse.
__device__ inline void kvq_wht128_fp64(double &x0, double &x1, int lane) {
#pragma clang fp contract(off)
  {
    const double a = x0, b = x1;
    x0 = a + b;
    x1 = a - b;
  }
  for (int h = 2; h < 128; h <<= 1) {
    const int pl = h >> 1;
    const double p0 = __shfl_xor(x0, pl), p1 = __shfl_xor(x1, pl);
    if ((lane & pl) == 0) {
      x0 = x0 + p0;
      x1 = x1 + p1;
    } else {
      x0 = p0 - x0;
      x1 = p1 - x1;
    }
  }
  x0 = x0 * KVQ_WHT_C;
  x1 = x1 * KVQ_WHT_C;
}

struct KvqCacheDev {
  uint8_t *pages;
  uint8_t *k_win, *v_win;
  const int32_t *block_table;
  int32_t batch, mbps;
  int64_t pages_per_seq;  // contiguous mode
  int64_t pool_pages;     // paged mode: pages in the pool
  int paged;
  uint32_t *err;          // optional device error word (kvq_cache::error_flags), or null
};

// OR `flag` into the cache's device error word (when there is one) from the active lanes that
// saw the condition: one atomic per wave, issued by the lowest such lane.
__device__ inline void kvq_raise(const KvqCacheDev &c, bool cond, uint32_t flag) {
  if (!c.err) return;
  const uint64_t m = __ballot(cond);
  if (m && (int)__lane_id() == __ffsll((unsigned long long)m) - 1) atomicOr(c.err, flag);
}

// Record of (sequence b, kv head h, logical page p), with an out-of-range block-table entry
// clamped into the pool and reported as KVQ_DEV_TABLE_ENTRY.
__device__ inline int64_t kvq_record_index_dev(const KvqCacheDev &c, int Hkv, int b, int h, int64_t p) {
  if (c.paged) {
    const int64_t e = c.block_table[(int64_t)b * c.mbps + p];
    kvq_raise(c, e < 0 || e >= c.pool_pages, KVQ_DEV_TABLE_ENTRY);
  }
  return kvq_record_index(c.paged, c.block_table, c.mbps, (int64_t)c.batch * Hkv, c.pool_pages, Hkv, b, h, p);
}

struct KvqAppendArgs {
  KvqLayout lay;
  KvqCacheDev cache;
  const int32_t *seq_lens_before;
  const int32_t *n_new_per_seq;
  const uint8_t *k_new, *v_new;
  int32_t n_new, Hkv, R, rotation, kv_f32;
  int32_t value_rotation;
};

struct KvqAttnArgs {
  KvqLayout lay;
  KvqCacheDev cache;
  const int32_t *seq_lens;
  const void *q;
  float *partials;  // [B][Hq][S][KVQ_PART_STRIDE]
  int32_t q_f32, kv_f32, Hq, Hkv, R, rotation;
  // Split plan (computed per sequence on the device from the lengths, see the split kernel):
  int32_t splits;     // row stride S_max of the partial rows: no sequence gets more splits
  int32_t ws;         // leading splits of every unit that cover the recent window, KVQ_WIN_PAGES pages each
  int32_t target_q;   // quantized waves to share out over the batch, in proportion to its pages
  int32_t cap_max;    // most quantized splits of one unit
  int32_t fixed_per;  // > 0: pages per quantized split fixed instead (KVQ_PAGES_PER_SPLIT)
  int64_t grid;       // waves launched (an upper bound of the plan's total; the rest exit)
  int32_t max_len;  // host-validated upper bound of seq_lens (device lengths are clamped to it)
  float sigma_u;  // softmax_scale * log2(e) * 2^33
  // Fused decode step (fuse = 1; bf16 rings, window > 0): seq_lens are the lengths before the
  // step, k_new / v_new [B][1][Hkv][128] bf16 the appended token, attended at length + 1.
  const uint8_t *k_new, *v_new;
  int32_t fuse;
  int32_t len_plus1;  // attend at seq_lens[b] + 1 (a decode step; set whenever fuse is)
};


struct KvqCombineArgs {
  const float *partials;
  void *out;
  int32_t out_f32, B, Hq, splits;
  int32_t eager;  // entries whose rows are read together with the headers (the rest once seen live)
  int32_t value_rotation;  // the partials are over rotated values: rotate the merged row back
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

#define KVQ_PART_STRIDE KVQ_PART_FLOATS  // floats per partial row: m, l, pad, pad, acc[128]
#define KVQ_WIN_PAGES 8  // window pages (128 tokens) per window split

// Waves per SIMD each split-kernel instantiation is compiled for (register budget
// 512 / waves): 2 for every one.  With 8 waves per CU each wave gets an LDS ring of up to 8
// pages (6 in flight while a pair is processed, the same bytes in flight per CU as 16 waves
// with 3 each), and the 32k batch-16 K4V2 launch measured 91 µs against 94 µs at 4 waves per
// SIMD (3 waves per SIMD measured 114 µs, 1 wave 143 µs).  With the score operand laid out as
// (head, query part) rows when there are 8 or 16 of them, the widest instantiations (8 heads
// per kv head, query in hi and lo parts) need 188-195 registers.  No instantiation spills at
// its budget (the build checks this).
__host__ __device__ constexpr int kvq_attn_wpe(int, int, int, int, int) { return 2; }

#define KVQ_LDS_PER_CU (160 * 1024)

// Page records of the split kernel's LDS prefetch ring: as many as fit in the LDS
// share of one wave at the compiled occupancy after its weight-exchange buffers
// (KVQ_XCHG_BYTES per value group), at least 3 (the pair in use plus one page ahead)
// and at most KVQ_RING_MAX.  Slots are sized for the largest record of the bit widths (key
// groups of 32): rec16 16-byte units, rounded up to whole 1 KiB DMAs (64 lanes x 16 B)
// when KVQ_RING_MAX such slots still fit, so that every lane of every DMA lands inside its slot.
#define KVQ_XCHG_BYTES 1024  // 16 rows x 32 bf16 weights: the A operand of one value contraction
#ifndef KVQ_RING_MAX
#define KVQ_RING_MAX 8  // most ring slots per wave
#endif
#define KVQ_NUM_CUS 256  // MI355X: 256 compute units, 4 SIMDs each
// Split-kernel waves dispatched after every SIMD already holds one (block index >= the SIMD
// count) run their first KVQ_SLOT_PRIO eighths of page pairs at raised issue priority (0 = off).
#ifndef KVQ_SLOT_PRIO
#define KVQ_SLOT_PRIO 5
#endif
#ifndef KVQ_SLOT_PAD
#define KVQ_SLOT_PAD 1  // pad slots to whole DMAs when KVQ_RING_MAX of them still fit
#endif
__host__ __device__ constexpr int kvq_rec16(int kb, int vb, int nvg) { return 16 * kb + 16 + 16 * vb + 4 * nvg; }
__host__ __device__ constexpr int kvq_lds_share(int wpe, int nvg) {
  return KVQ_LDS_PER_CU / (4 * wpe) - KVQ_XCHG_BYTES * nvg;
}
__host__ __device__ constexpr int kvq_slot_padded(int kb, int vb, int nvg) { return 1024 * ((kvq_rec16(kb, vb, nvg) + 63) / 64); }
__host__ __device__ constexpr bool kvq_slot_pad(int kb, int vb, int nvg, int wpe) {
  return KVQ_SLOT_PAD && kvq_lds_share(wpe, nvg) / kvq_slot_padded(kb, vb, nvg) >= KVQ_RING_MAX;
}
__host__ __device__ constexpr int kvq_slot_bytes(int kb, int vb, int nvg, int wpe) {
  return kvq_slot_pad(kb, vb, nvg, wpe) ? kvq_slot_padded(kb, vb, nvg) : 16 * kvq_rec16(kb, vb, nvg);
}
__host__ __device__ constexpr int kvq_ring_pages(int slot_bytes, int wpe, int nvg) {
  return kvq_lds_share(wpe, nvg) / slot_bytes < 3
             ? 3
             : (kvq_lds_share(wpe, nvg) / slot_bytes > KVQ_RING_MAX ? KVQ_RING_MAX
                                                                   : kvq_lds_share(wpe, nvg) / slot_bytes);
}
#define KVQ_STAGE_BYTES ((2 * 8 * 128 + 8 * 4) * 4)  // query / accumulator staging area

// LDS bytes of one split-kernel workgroup (one wave): the ring, then the exchange buffers.
__host__ __device__ constexpr int kvq_attn_ring_bytes(int kb, int vb, int nvg, int wpe) {
  return kvq_slot_bytes(kb, vb, nvg, wpe) * kvq_ring_pages(kvq_slot_bytes(kb, vb, nvg, wpe), wpe, nvg);
}
__host__ __device__ constexpr int kvq_attn_lds_bytes(int kb, int vb, int nvg, int wpe) {
  return kvq_attn_ring_bytes(kb, vb, nvg, wpe) + KVQ_XCHG_BYTES * nvg > KVQ_STAGE_BYTES
             ? kvq_attn_ring_bytes(kb, vb, nvg, wpe) + KVQ_XCHG_BYTES * nvg
             : KVQ_STAGE_BYTES;
}

// Resident split-kernel waves per CU: the register limit or the LDS limit.
__host__ __device__ constexpr int kvq_attn_waves_per_cu(int kb, int vb, int nvg, int g, int p) {
  return (4 * kvq_attn_wpe(kb, vb, g, p, nvg)) < (KVQ_LDS_PER_CU / kvq_attn_lds_bytes(kb, vb, nvg, kvq_attn_wpe(kb, vb, g, p, nvg)))
             ? 4 * kvq_attn_wpe(kb, vb, g, p, nvg)
             : KVQ_LDS_PER_CU / kvq_attn_lds_bytes(kb, vb, nvg, kvq_attn_wpe(kb, vb, g, p, nvg));
}

hipError_t kvq_launch_append(const KvqAppendArgs &a, hipStream_t s);
hipError_t kvq_launch_attention(const KvqAttnArgs &a, int g, int q_parts, hipStream_t s);
hipError_t kvq_launch_combine(const KvqCombineArgs &a, hipStream_t s);
hipError_t kvq_launch_debug(const KvqDebugArgs &a, hipStream_t s);

bool kvq_attention_supported(int kb, int vb, int g, int q_parts, int nvg);
