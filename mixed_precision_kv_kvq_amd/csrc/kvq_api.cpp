// C-ABI front end: host-side validation, sizing and launch.
#include <math.h>
#include <stdlib.h>

#include "kvq_extras.h"

namespace {

constexpr int kNumCUs = KVQ_NUM_CUS;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// 1..6 and 8 bits (the split kernel is instantiated for these widths)
bool bits_ok(int b) { return b >= 1 && b <= 8 && b != 7; }

kvq_status check_params(const kvq_params *p) {
  if (!p) return KVQ_EINVAL;
  if (p->num_q_heads <= 0 || p->num_kv_heads <= 0 || p->num_q_heads % p->num_kv_heads) return KVQ_EINVAL;
  if (p->window < 0 || p->key_rotation < 0 || p->key_rotation > 1) return KVQ_EINVAL;
  // bounds that keep every size and plan product far inside 64 bits
  if (p->num_q_heads > KVQ_MAX_HEADS || p->window > KVQ_MAX_WINDOW) return KVQ_EUNSUPPORTED;
  if (p->value_rotation < 0 || p->value_rotation > 1) return KVQ_EINVAL;
  if (p->kv_dtype != KVQ_F32 && p->kv_dtype != KVQ_BF16) return KVQ_EINVAL;
  if (p->head_dim != KVQ_D) return KVQ_EUNSUPPORTED;
  const int g = p->num_q_heads / p->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return KVQ_EUNSUPPORTED;
  if (!bits_ok(p->k_bits) || !bits_ok(p->v_bits)) return KVQ_EUNSUPPORTED;
  if (p->k_group != 32 && p->k_group != 64 && p->k_group != 128) return KVQ_EUNSUPPORTED;
  if (p->v_group != 64 && p->v_group != 128) return KVQ_EUNSUPPORTED;
  if (p->block_size != 0 && p->block_size != KVQ_PAGE) return KVQ_EUNSUPPORTED;
  // rotated values cannot share one accumulator with the window's unrotated ones
  if (p->value_rotation && p->window > 0) return KVQ_EUNSUPPORTED;
  return KVQ_OK;
}

kvq_status check_cache(const kvq_params *p, const kvq_cache *c) {
  if (!c || c->batch <= 0 || c->capacity <= 0) return KVQ_EINVAL;
  if (!c->pages || !aligned16(c->pages)) return KVQ_EINVAL;
  if (((uintptr_t)c->error_flags & 3u)) return KVQ_EINVAL;
  if (p->window > 0) {
    if (!c->k_win || !c->v_win || !aligned16(c->k_win) || !aligned16(c->v_win)) return KVQ_EINVAL;
  }
  if (p->block_size) {
    if (!c->block_table || ((uintptr_t)c->block_table & 3u) || c->max_blocks_per_seq <= 0) return KVQ_EINVAL;
  }
  return KVQ_OK;
}

KvqCacheDev dev_cache(const kvq_params *p, const kvq_cache *c) {
  KvqCacheDev d;
  d.pages = (uint8_t *)c->pages;
  d.k_win = (uint8_t *)c->k_win;
  d.v_win = (uint8_t *)c->v_win;
  d.block_table = c->block_table;
  d.batch = c->batch;
  d.mbps = c->max_blocks_per_seq;
  d.paged = p->block_size != 0;
  d.pages_per_seq = d.paged ? 0 : kvq_pages_per_seq(c->capacity);
  d.pool_pages = d.paged ? c->capacity : 0;
  d.err = c->error_flags;
  return d;
}

KvqLayout layout_of(const kvq_params *p) { return kvq_make_layout(p->k_bits, p->k_group, p->v_bits, p->v_group); }

// Split plan.  Every (sequence, kv head) unit gets `ws` window splits (KVQ_WIN_PAGES pages of the
// recent window each) and a number of quantized splits that the split kernel works out per sequence
// from the device lengths: the launch's quantized waves (target_q, sized so that every wave of the
// launch is resident at once) are shared out over the sequences in proportion to their quantized
// pages, at most cap_max per unit.  The host only knows max_seq_len, so it sizes the launch (grid)
// and the partial rows (S_max) for the worst case; waves past the plan's total exit at once.
struct SplitPlan {
  int ws, S_max, target_q, cap_max, fixed_per;
  int eager;  // entries the merge reads eagerly: the splits of a unit with an equal share
  int64_t grid;
};

SplitPlan split_plan(const kvq_params *p, int32_t batch, int64_t max_seq_len, int q_parts) {
  if (max_seq_len > INT32_MAX) max_seq_len = INT32_MAX;  // device lengths are int32 (the launch clamps too)
  const int R = p->window;
  const int64_t nq = max_seq_len > R ? max_seq_len - R : 0;
  const int64_t nw = max_seq_len < R ? max_seq_len : R;
  const int64_t qpmax = (nq + KVQ_PAGE - 1) / KVQ_PAGE;
  const int64_t wpages = (nw + KVQ_PAGE - 1) / KVQ_PAGE;
  const int64_t units = (int64_t)batch * p->num_kv_heads;
  SplitPlan sp = {};
  sp.ws = (int)((wpages + KVQ_WIN_PAGES - 1) / KVQ_WIN_PAGES);
  int64_t per = 0;
  if (const char *env = getenv("KVQ_PAGES_PER_SPLIT")) per = atoll(env);
  int64_t qs_max;
  if (per > 0) {  // fixed pages per quantized split
    per = per < 2 ? 2 : (per + 1) & ~int64_t(1);
    sp.fixed_per = (int)per;
    qs_max = (qpmax + per - 1) / per;
    if (qs_max < 1) qs_max = 1;
    sp.grid = units * (sp.ws + qs_max);
  } else {
    const int g = p->num_q_heads / p->num_kv_heads;
    int64_t target = (int64_t)kNumCUs * kvq_attn_waves_per_cu(p->k_bits, p->v_bits, KVQ_D / p->v_group, g, q_parts);
    if (const char *env = getenv("KVQ_TARGET_WAVES")) target = atoll(env) > 0 ? atoll(env) : target;
    int64_t tq = target - units * sp.ws;
    if (tq < units) tq = units;
    // a unit may take up to twice the equal share of the launch
    int64_t cap = 2 * ((target + units - 1) / units);
    sp.target_q = (int)tq;
    sp.cap_max = (int)cap;
    qs_max = (qpmax + 1) / 2 < cap ? (qpmax + 1) / 2 : cap;
    if (qs_max < 1) qs_max = 1;
    // sum over units of the quantized splits <= tq + units (each unit's share rounds down, then up to >= 1)
    sp.grid = units * sp.ws + tq + units;
  }
  // with an even Hkv the waves of the two kv heads of a pair sit 8 apart in groups of 16: up to 14
  // waves at the end of the last group hold no item
  if (p->num_kv_heads % 2 == 0) sp.grid += 16;
  sp.S_max = (int)(sp.ws + qs_max);
  // the merge reads the headers and rows of a unit's equal share at once (exactly the split count
  // of every unit when the lengths are equal)
  if (sp.fixed_per) {
    sp.eager = sp.S_max;
  } else {
    const int64_t share = sp.target_q / units;
    sp.eager = (int)(sp.ws + (share > 1 ? share : 1));
  }
  if (sp.eager > sp.S_max) sp.eager = sp.S_max;
  return sp;
}

kvq_status hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_EHIP; }

}  // namespace

extern "C" {

kvq_status kvq_cache_sizes(const kvq_params *params, int32_t batch, int64_t capacity, kvq_sizes *out) {
  if (kvq_status st = check_params(params)) return st;
  if (!out || batch <= 0 || capacity <= 0) return KVQ_EINVAL;
  const KvqLayout lay = layout_of(params);
  // byte counts that do not fit size_t are reported as invalid arguments
  size_t pages, pb, wb;
  if (params->block_size)
    pages = (size_t)capacity;
  else if (__builtin_mul_overflow((size_t)batch, (size_t)kvq_pages_per_seq(capacity), &pages))
    return KVQ_EINVAL;
  if (__builtin_mul_overflow(pages, (size_t)params->num_kv_heads * (size_t)lay.record, &pb)) return KVQ_EINVAL;
  if (__builtin_mul_overflow((size_t)batch * params->num_kv_heads,
                             (size_t)params->window * KVQ_D * (params->kv_dtype == KVQ_F32 ? 4 : 2), &wb))
    return KVQ_EINVAL;
  out->record_bytes = (size_t)lay.record;
  out->pages_bytes = pb;
  out->window_bytes = wb;
  return KVQ_OK;
}

kvq_status kvq_quantize_append(const kvq_params *params, const kvq_cache *cache, const int32_t *seq_lens_before,
                               const int32_t *n_new_per_seq, const void *k_new, const void *v_new, int32_t n_new,
                               hipStream_t stream) {
  if (kvq_status st = check_params(params)) return st;
  if (kvq_status st = check_cache(params, cache)) return st;
  if (!seq_lens_before || n_new < 0) return KVQ_EINVAL;
  if (n_new == 0) return KVQ_OK;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return KVQ_EINVAL;
  KvqAppendArgs a;
  a.lay = layout_of(params);
  a.cache = dev_cache(params, cache);
  a.seq_lens_before = seq_lens_before;
  a.n_new_per_seq = n_new_per_seq;
  a.k_new = (const uint8_t *)k_new;
  a.v_new = (const uint8_t *)v_new;
  a.n_new = n_new;
  a.Hkv = params->num_kv_heads;
  a.R = params->window;
  a.rotation = params->key_rotation;
  a.value_rotation = params->value_rotation;
  a.kv_f32 = params->kv_dtype == KVQ_F32;
  return hip_status(kvq_launch_append(a, stream));
}

size_t kvq_decode_workspace_bytes(const kvq_params *params, int32_t batch, int64_t max_seq_len) {
  if (check_params(params) != KVQ_OK || batch <= 0 || max_seq_len < 0) return 0;
  // The query dtype is not known here: cover both query-part counts.  S_max never decreases as
  // max_seq_len grows (ws, the quantized pages and the caps are all non-decreasing in it).
  int bound = 0;
  for (int parts = 1; parts <= 2; ++parts) {
    const SplitPlan sp = split_plan(params, batch, max_seq_len, parts);
    bound = sp.S_max > bound ? sp.S_max : bound;
  }
  return (size_t)batch * params->num_q_heads * (size_t)bound * KVQ_PART_STRIDE * sizeof(float);
}

}  // extern "C"

namespace {

// Decode steps fuse their append into the attention launch for bf16 rings (window > 0) with the
// window in splits of its own; otherwise the append kernel runs first.
bool step_fusable(const kvq_params *p) { return p->window > 0 && p->kv_dtype == KVQ_BF16; }

// The split-kernel launch of kvq_decode_partials (step = 0) or of a decode step (step = 1: lengths
// before the step, attended at length + 1; k_new / v_new appended in the same launch when fuse).
kvq_status partials_impl(const kvq_params *params, const kvq_cache *cache, const int32_t *seq_lens,
                         int64_t max_seq_len, const void *q, int32_t q_dtype, float softmax_scale, void *workspace,
                         size_t workspace_bytes, int step, const void *k_new, const void *v_new, bool fuse,
                         hipStream_t stream, bool validate_only = false) {
  if (kvq_status st = check_params(params)) return st;
  if (kvq_status st = check_cache(params, cache)) return st;
  if (!seq_lens || !q || !workspace || max_seq_len < 0) return KVQ_EINVAL;
  if (!aligned16(q) || !aligned16(workspace)) return KVQ_EINVAL;
  if (q_dtype != KVQ_F32 && q_dtype != KVQ_BF16) return KVQ_EINVAL;
  if (!(softmax_scale >= 0.f) || isinf(softmax_scale)) return KVQ_EINVAL;
  const int64_t nq_max = max_seq_len > params->window ? max_seq_len - params->window : 0;
  if (params->block_size) {
    if ((nq_max + KVQ_PAGE - 1) / KVQ_PAGE > cache->max_blocks_per_seq) return KVQ_ENOSPACE;
  } else if (nq_max > cache->capacity) {
    return KVQ_ENOSPACE;
  }
  if (workspace_bytes < kvq_decode_workspace_bytes(params, cache->batch, max_seq_len)) return KVQ_ENOSPACE;

  KvqAttnArgs a;
  a.lay = layout_of(params);
  a.cache = dev_cache(params, cache);
  a.seq_lens = seq_lens;
  a.q = q;
  a.partials = (float *)workspace;
  a.q_f32 = q_dtype == KVQ_F32;
  a.kv_f32 = params->kv_dtype == KVQ_F32;
  a.Hq = params->num_q_heads;
  a.Hkv = params->num_kv_heads;
  a.R = params->window;
  a.rotation = params->key_rotation;
  const int q_parts = (q_dtype == KVQ_BF16 && !params->key_rotation) ? 1 : 2;
  const SplitPlan sp = split_plan(params, cache->batch, max_seq_len, q_parts);
  a.splits = sp.S_max;
  a.ws = sp.ws;
  a.target_q = sp.target_q;
  a.cap_max = sp.cap_max;
  a.fixed_per = sp.fixed_per;
  a.grid = sp.grid;
  a.max_len = (int32_t)(max_seq_len < INT32_MAX ? max_seq_len : INT32_MAX);
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)KVQ_D);
  a.sigma_u = (float)((double)scale * 1.4426950408889634 * 8589934592.0);  // * log2(e) * 2^33
  a.k_new = (const uint8_t *)k_new;
  a.v_new = (const uint8_t *)v_new;
  a.fuse = fuse ? 1 : 0;
  a.len_plus1 = step;
  if (step && max_seq_len < 1) return KVQ_EINVAL;
  if (validate_only) return KVQ_OK;
  const int g = params->num_q_heads / params->num_kv_heads;
  return hip_status(kvq_launch_attention(a, g, q_parts, stream));
}

// Validation and launches of a decode step up to (not including) the merge.
kvq_status step_impl(const kvq_params *params, const kvq_cache *cache, const int32_t *seq_lens_before,
                     const void *k_new, const void *v_new, int64_t max_seq_len, const void *q, int32_t q_dtype,
                     float softmax_scale, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (kvq_status st = check_params(params)) return st;
  if (kvq_status st = check_cache(params, cache)) return st;
  if (!seq_lens_before || !k_new || !v_new || !aligned16(k_new) || !aligned16(v_new) || max_seq_len < 1)
    return KVQ_EINVAL;
  if (step_fusable(params))
    return partials_impl(params, cache, seq_lens_before, max_seq_len, q, q_dtype, softmax_scale, workspace,
                         workspace_bytes, 1, k_new, v_new, true, stream);
  // Validate the attention half before the append launches anything.
  if (kvq_status st = partials_impl(params, cache, seq_lens_before, max_seq_len, q, q_dtype, softmax_scale,
                                    workspace, workspace_bytes, 1, nullptr, nullptr, false, stream, true))
    return st;
  if (kvq_status st = kvq_quantize_append(params, cache, seq_lens_before, nullptr, k_new, v_new, 1, stream)) return st;
  return partials_impl(params, cache, seq_lens_before, max_seq_len, q, q_dtype, softmax_scale, workspace,
                       workspace_bytes, 1, nullptr, nullptr, false, stream);
}

}  // namespace

extern "C" {

kvq_status kvq_decode_partials(const kvq_params *params, const kvq_cache *cache, const int32_t *seq_lens,
                               int64_t max_seq_len, const void *q, int32_t q_dtype, float softmax_scale,
                               void *workspace, size_t workspace_bytes, hipStream_t stream) {
  return partials_impl(params, cache, seq_lens, max_seq_len, q, q_dtype, softmax_scale, workspace, workspace_bytes,
                       0, nullptr, nullptr, false, stream);
}

kvq_status kvq_decode_step_partials(const kvq_params *params, const kvq_cache *cache, const int32_t *seq_lens_before,
                                    const void *k_new, const void *v_new, int64_t max_seq_len, const void *q,
                                    int32_t q_dtype, float softmax_scale, void *workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  return step_impl(params, cache, seq_lens_before, k_new, v_new, max_seq_len, q, q_dtype, softmax_scale, workspace,
                   workspace_bytes, stream);
}

kvq_status kvq_decode_step(const kvq_params *params, const kvq_cache *cache, const int32_t *seq_lens_before,
                           const void *k_new, const void *v_new, int64_t max_seq_len, const void *q, int32_t q_dtype,
                           void *out, int32_t out_dtype, float softmax_scale, void *workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  if (!out || !aligned16(out) || (out_dtype != KVQ_F32 && out_dtype != KVQ_BF16)) {
    if (kvq_status st = check_params(params)) return st;
    return KVQ_EINVAL;
  }
  if (kvq_status st = step_impl(params, cache, seq_lens_before, k_new, v_new, max_seq_len, q, q_dtype, softmax_scale,
                                workspace, workspace_bytes, stream))
    return st;
  return kvq_decode_combine(params, cache->batch, max_seq_len, q_dtype, workspace, out, out_dtype, stream);
}

int32_t kvq_decode_splits(const kvq_params *params, int32_t batch, int64_t max_seq_len, int32_t q_dtype) {
  if (check_params(params) != KVQ_OK || batch <= 0 || max_seq_len < 0) return 0;
  if (q_dtype != KVQ_F32 && q_dtype != KVQ_BF16) return 0;
  const int q_parts = (q_dtype == KVQ_BF16 && !params->key_rotation) ? 1 : 2;
  return split_plan(params, batch, max_seq_len, q_parts).S_max;
}

kvq_status kvq_decode_combine(const kvq_params *params, int32_t batch, int64_t max_seq_len, int32_t q_dtype,
                              const void *workspace, void *out, int32_t out_dtype, hipStream_t stream) {
  if (kvq_status st = check_params(params)) return st;
  if (batch <= 0 || !workspace || !out || max_seq_len < 0) return KVQ_EINVAL;
  if (!aligned16(workspace) || !aligned16(out)) return KVQ_EINVAL;
  if ((q_dtype != KVQ_F32 && q_dtype != KVQ_BF16) || (out_dtype != KVQ_F32 && out_dtype != KVQ_BF16))
    return KVQ_EINVAL;
  const int q_parts = (q_dtype == KVQ_BF16 && !params->key_rotation) ? 1 : 2;
  KvqCombineArgs c;
  c.partials = (const float *)workspace;
  c.out = out;
  c.out_f32 = out_dtype == KVQ_F32;
  c.B = batch;
  c.Hq = params->num_q_heads;
  const SplitPlan sp = split_plan(params, batch, max_seq_len, q_parts);
  c.splits = sp.S_max;
  c.eager = sp.eager;
  c.value_rotation = params->value_rotation;
  return hip_status(kvq_launch_combine(c, stream));
}

kvq_status kvq_decode_attention(const kvq_params *params, const kvq_cache *cache, const int32_t *seq_lens,
                                int64_t max_seq_len, const void *q, int32_t q_dtype, void *out, int32_t out_dtype,
                                float softmax_scale, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!out || !aligned16(out) || (out_dtype != KVQ_F32 && out_dtype != KVQ_BF16)) {
    if (kvq_status st = check_params(params)) return st;
    return KVQ_EINVAL;
  }
  if (kvq_status st = kvq_decode_partials(params, cache, seq_lens, max_seq_len, q, q_dtype, softmax_scale, workspace,
                                          workspace_bytes, stream))
    return st;
  return kvq_decode_combine(params, cache->batch, max_seq_len, q_dtype, workspace, out, out_dtype, stream);
}

kvq_status kvq_dequantize_debug(const kvq_params *params, const kvq_cache *cache, const int32_t *seq_lens,
                                int32_t seq, int64_t t0, int64_t n, uint8_t *k_codes, uint8_t *v_codes,
                                uint16_t *k_meta, uint16_t *v_meta, float *k_hat, float *v_hat,
                                hipStream_t stream) {
  if (kvq_status st = check_params(params)) return st;
  if (kvq_status st = check_cache(params, cache)) return st;
  if (!seq_lens || seq < 0 || seq >= cache->batch || t0 < 0 || n < 0) return KVQ_EINVAL;
  if (n == 0) return KVQ_OK;
  KvqDebugArgs a;
  a.lay = layout_of(params);
  a.cache = dev_cache(params, cache);
  a.seq_lens = seq_lens;
  a.seq = seq;
  a.Hkv = params->num_kv_heads;
  a.R = params->window;
  a.kv_f32 = params->kv_dtype == KVQ_F32;
  a.t0 = t0;
  a.n = n;
  a.k_codes = k_codes;
  a.v_codes = v_codes;
  a.k_meta = k_meta;
  a.v_meta = v_meta;
  a.k_hat = k_hat;
  a.v_hat = v_hat;
  return hip_status(kvq_launch_debug(a, stream));
}

static int dense_splits(int64_t max_seq_len) {
  const int64_t s = (max_seq_len + KVQ_DENSE_SPLIT - 1) / KVQ_DENSE_SPLIT;
  return s < 1 ? 1 : (int)s;
}

kvq_status kvq_dequantize_dense(const kvq_params *params, const kvq_cache *cache, const int32_t *seq_lens,
                                int64_t max_seq_len, uint16_t *k_out, uint16_t *v_out, hipStream_t stream) {
  if (kvq_status st = check_params(params)) return st;
  if (kvq_status st = check_cache(params, cache)) return st;
  if (!seq_lens || max_seq_len < 0 || max_seq_len > INT32_MAX) return KVQ_EINVAL;
  if (!k_out || !v_out || !aligned16(k_out) || !aligned16(v_out)) return KVQ_EINVAL;
  KvqDenseArgs a = {};
  a.lay = layout_of(params);
  a.cache = dev_cache(params, cache);
  a.seq_lens = seq_lens;
  a.k_out = k_out;
  a.v_out = v_out;
  a.max_len = max_seq_len;
  a.B = cache->batch;
  a.Hkv = params->num_kv_heads;
  a.R = params->window;
  a.kv_f32 = params->kv_dtype == KVQ_F32;
  a.rotation = params->key_rotation;
  a.value_rotation = params->value_rotation;
  return hip_status(kvq_launch_dequantize_dense(a, stream));
}

size_t kvq_dense_workspace_bytes(const kvq_params *params, int32_t batch, int64_t max_seq_len) {
  if (check_params(params) != KVQ_OK || batch <= 0 || max_seq_len < 0 || max_seq_len > INT32_MAX) return 0;
  return (size_t)batch * params->num_q_heads * (size_t)dense_splits(max_seq_len) * KVQ_PART_STRIDE * sizeof(float);
}

kvq_status kvq_dense_decode_attention(const kvq_params *params, int32_t batch, const uint16_t *k, const uint16_t *v,
                                      const int32_t *seq_lens, int64_t max_seq_len, const void *q, int32_t q_dtype,
                                      void *out, int32_t out_dtype, float softmax_scale, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  if (kvq_status st = check_params(params)) return st;
  if (batch <= 0 || !seq_lens || max_seq_len < 0 || max_seq_len > INT32_MAX) return KVQ_EINVAL;
  if (!k || !v || !q || !out || !workspace) return KVQ_EINVAL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(q) || !aligned16(out) || !aligned16(workspace)) return KVQ_EINVAL;
  if ((q_dtype != KVQ_F32 && q_dtype != KVQ_BF16) || (out_dtype != KVQ_F32 && out_dtype != KVQ_BF16))
    return KVQ_EINVAL;
  if (!(softmax_scale >= 0.f) || isinf(softmax_scale)) return KVQ_EINVAL;
  if (workspace_bytes < kvq_dense_workspace_bytes(params, batch, max_seq_len)) return KVQ_ENOSPACE;
  KvqDenseArgs a = {};
  a.seq_lens = seq_lens;
  a.k_in = k;
  a.v_in = v;
  a.q = q;
  a.partials = (float *)workspace;
  a.max_len = max_seq_len;
  a.B = batch;
  a.Hq = params->num_q_heads;
  a.Hkv = params->num_kv_heads;
  a.q_f32 = q_dtype == KVQ_F32;
  a.splits = dense_splits(max_seq_len);
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)KVQ_D);
  a.sigma = (float)((double)scale * 1.4426950408889634);  // * log2(e)
  if (hipError_t e = kvq_launch_dense_partials(a, params->num_q_heads / params->num_kv_heads, stream))
    return hip_status(e);
  KvqCombineArgs c = {};
  c.partials = a.partials;
  c.out = out;
  c.out_f32 = out_dtype == KVQ_F32;
  c.B = batch;
  c.Hq = a.Hq;
  c.splits = a.splits;
  c.eager = a.splits;  // every dense split is written
  c.value_rotation = 0;  // the dense cache is in the original domain
  return hip_status(kvq_launch_combine(c, stream));
}

}  // extern "C"

namespace {

// Ranges of pages per sequence for the error-budget passes: about two workgroups per CU over all
// (unit, head group, range) items (the scores pass holds two per CU), at least one page per wave
// of a range.
int errbudget_splits(const kvq_params *p, int32_t batch, int64_t max_seq_len) {
  const int g = p->num_q_heads / p->num_kv_heads, ngrp = g / kvq_errbudget_heads_per_group(g);
  const int64_t items = (int64_t)batch * p->num_kv_heads * ngrp;
  const int64_t pages = (max_seq_len + KVQ_PAGE - 1) / KVQ_PAGE;
  int64_t s = (2 * kNumCUs + items - 1) / items;
  const int64_t smax = (pages + 7) / 8;
  if (s > smax) s = smax;
  return s < 1 ? 1 : (int)s;
}

}  // namespace

extern "C" {

size_t kvq_error_budget_workspace_bytes(const kvq_params *params, int32_t batch, int64_t max_seq_len) {
  if (check_params(params) != KVQ_OK || batch <= 0 || max_seq_len < 0 || max_seq_len > INT32_MAX) return 0;
  const int g = params->num_q_heads / params->num_kv_heads, ngrp = g / kvq_errbudget_heads_per_group(g);
  const size_t items = (size_t)batch * params->num_kv_heads * ngrp * errbudget_splits(params, batch, max_seq_len);
  // the items, then both scores of every (sequence, query head, position), rows padded to whole pages
  return items * kvq_errbudget_item_floats() * sizeof(float) +
         (size_t)batch * params->num_q_heads * kvq_errbudget_score_stride(max_seq_len) * 2 * sizeof(float);
}

kvq_status kvq_error_budget(const kvq_params *params, const kvq_cache *cache, const int32_t *seq_lens,
                            int64_t max_seq_len, const uint16_t *k_ref, const uint16_t *v_ref, const void *q,
                            int32_t q_dtype, float softmax_scale, float *head_stats, float *unit_stats,
                            void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (kvq_status st = check_params(params)) return st;
  if (kvq_status st = check_cache(params, cache)) return st;
  if (!seq_lens || max_seq_len < 0 || max_seq_len > INT32_MAX) return KVQ_EINVAL;
  if (!k_ref || !v_ref || !q || !head_stats || !unit_stats || !workspace) return KVQ_EINVAL;
  if (!aligned16(k_ref) || !aligned16(v_ref) || !aligned16(q) || !aligned16(head_stats) || !aligned16(unit_stats) ||
      !aligned16(workspace))
    return KVQ_EINVAL;
  if (q_dtype != KVQ_F32 && q_dtype != KVQ_BF16) return KVQ_EINVAL;
  if (!(softmax_scale >= 0.f) || isinf(softmax_scale)) return KVQ_EINVAL;
  if (workspace_bytes < kvq_error_budget_workspace_bytes(params, cache->batch, max_seq_len)) return KVQ_ENOSPACE;
  KvqErrArgs a = {};
  a.lay = layout_of(params);
  a.cache = dev_cache(params, cache);
  a.seq_lens = seq_lens;
  a.k_ref = k_ref;
  a.v_ref = v_ref;
  a.q = q;
  a.head_stats = head_stats;
  a.unit_stats = unit_stats;
  a.max_len = max_seq_len;
  a.B = cache->batch;
  a.Hq = params->num_q_heads;
  a.Hkv = params->num_kv_heads;
  a.R = params->window;
  a.q_f32 = q_dtype == KVQ_F32;
  a.rotation = params->key_rotation;
  a.value_rotation = params->value_rotation;
  a.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)KVQ_D);
  a.ws = (float *)workspace;
  a.splits = errbudget_splits(params, cache->batch, max_seq_len);
  return hip_status(kvq_launch_errbudget(a, stream));
}

kvq_status kvq_device_status(const kvq_cache *cache, uint32_t *flags, hipStream_t stream) {
  if (!cache || !cache->error_flags || !flags) return KVQ_EINVAL;
  uint32_t v = 0;
  if (hipMemcpyAsync(&v, cache->error_flags, sizeof(v), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return KVQ_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return KVQ_EHIP;
  *flags = v;
  return v ? KVQ_EDEVICE : KVQ_OK;
}

const char *kvq_status_str(kvq_status status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_EINVAL: return "invalid argument (null or misaligned pointer, inconsistent shapes)";
    case KVQ_EUNSUPPORTED: return "unsupported parameter";
    case KVQ_ENOSPACE: return "workspace too small or length beyond the cache capacity";
    case KVQ_EHIP: return "HIP runtime error at launch";
    case KVQ_EDEVICE: return "device-side input error (block-table entry, capacity, length or count out of range)";
  }
  return "unknown status";
}

}  // extern "C"
