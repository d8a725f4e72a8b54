/*
 * kvq.h — decode attention over a group-wise, asymmetrically quantized KV cache
 * on AMD Instinct MI355X (gfx950).  C ABI; plain pointers and sizes only.
 *
 * The method (sources are cited by page title and section):
 *   [P1] nalar.dev, "Kuantisasi KV cache mengganggu attention melalui key dan
 *        value tersimpan": attention of one head over stored keys and values,
 *        s = q K^T / sqrt(d), a = softmax(s), o = a V (section "Error pada key
 *        masuk sebelum softmax"); groups of values sharing a scale and a zero
 *        point or offset (section "Granularitas kuantisasi menentukan nilai yang
 *        berbagi scale"); recent tokens kept at higher precision, dequantization
 *        fused into the attention kernel (section "Pertumbuhan cache mengubah
 *        trade pada serving").
 *   [P3] gist.science summary of arXiv 2502.15075, "Quantize What Counts: More
 *        for Keys, Less for Values": separate bit widths for keys and values
 *        (section "Probleemstelling"), 4-bit keys with 2-bit values (section
 *        "Belangrijkste Bijdragen"), key groups of 32 and value groups of 64/128,
 *        key-only rotation (section "Resultaten").
 *
 * Quantizer (per token, per kv head, per group of G consecutive channels):
 *   zero  = largest fp16 <= min(group)
 *   scale = smallest fp16 s with zero + (2^b - 1) * s >= max(group)
 *   code  = clamp(round_half_even((x - zero) / scale), 0, 2^b - 1) in fp64
 *           (all codes 0 when scale == 0);  x_hat = zero + code * scale.
 * With key rotation on, keys are first multiplied by the normalized 128-point
 * Walsh-Hadamard matrix (fp64 butterflies in stage order 1, 2, ..., 64, then a
 * multiply by RN64(2^-3.5)); the query is rotated the same way before scoring.
 * Tokens t >= L - window of a length-L sequence stay unquantized in a ring
 * buffer (slot t mod window); older tokens live in the quantized store.
 * Query head h reads kv head h / (num_q_heads / num_kv_heads).
 *
 * Storage.  Quantized tokens are kept in 16-token pages.  One page of one kv
 * head is a record of
 *     [K codes 256*k_bits B][K meta 64*(128/k_group) B]
 *     [V codes 256*v_bits B][V meta 64*(128/v_group) B]
 * whose internal order matches the register layout of the attention kernel;
 * kvq_dequantize_debug reads it back in logical order.  Metadata entries are
 * {fp16 scale, fp16 zero} pairs.  Codes of 3, 5 and 6 bits are stored as bit
 * planes of 4, 2 and 1 bits (the binary digits of the width), each plane an area
 * of its own in the layout of a code of that width, so the code areas still take
 * 256 bits-per-code bytes: a record holds exactly the payload and the metadata.
 *   block_size == 0 (contiguous, page-major): page p of kv head h of sequence b is
 *       record p * (batch * num_kv_heads) + b * num_kv_heads + h, for
 *       p < ceil(capacity / 16); the records of one (sequence, kv head) are spread
 *       evenly over the whole allocation.
 *   block_size == 16 (paged): page p of sequence b is pool page
 *       block_table[b * max_blocks_per_seq + p]; its kv head h is record
 *       pool_page * num_kv_heads + h.
 * Window buffers k_win, v_win: [batch][num_kv_heads][window][128] of kv_dtype.
 *
 * Conventions.
 *   - All tensor pointers are device pointers owned by the caller.  The library
 *     never allocates, frees or synchronizes; work is enqueued on `stream`.
 *   - Arguments are validated on the host before anything is launched.  On any
 *     error nothing is launched and no memory is touched.
 *   - Device pointers must be 16-byte aligned.
 *   - Sequence lengths are read on the device; the library never writes them.
 *     The caller advances them between append and attention.
 *   - Inputs must be finite with |x| < 2^15; non-finite inputs give unspecified (but
 *     memory-safe) results.  The fp16 metadata is then finite for 2- to 8-bit codes.  With
 *     1-bit codes a group whose range (max - zero) exceeds 65504 has no finite fp16 scale:
 *     it gets scale +inf and all codes 0, as the quantizer's definition gives, and its
 *     dequantized values (and any attention over them) are NaN; |x| < 2^14 (or bf16 inputs,
 *     whose largest value below 2^15 is 32640) keeps 1-bit metadata finite.
 *   - Calls on different streams touching different caches may run concurrently.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A status crosses the ABI as a 32-bit int; in C++ the enum has that underlying type, so any
 * value a caller passes (kvq_status_str) is a valid object of it. */
typedef enum
#ifdef __cplusplus
    : int32_t
#endif
{
  KVQ_OK = 0,
  KVQ_EINVAL = 1,       /* null or misaligned pointer, inconsistent shapes       */
  KVQ_EUNSUPPORTED = 2, /* a parameter outside the supported set (see below)      */
  KVQ_ENOSPACE = 3,     /* workspace too small, or lengths beyond the capacity     */
  KVQ_EHIP = 4,         /* the HIP runtime reported an error at launch            */
  KVQ_EDEVICE = 5       /* kernels met device-side inputs they could not honour
                         * (reported by kvq_device_status, see kvq_cache)          */
} kvq_status;

typedef enum { KVQ_F32 = 0, KVQ_BF16 = 1 } kvq_dtype;
typedef enum { KVQ_ROT_NONE = 0, KVQ_ROT_WHT = 1 } kvq_rotation;

/* Supported: head_dim == 128; num_q_heads / num_kv_heads in {1, 2, 4, 8};
 * k_bits, v_bits in {1, 2, 3, 4, 5, 6, 8} (gist.science summary of "Quantize What
 * Counts", section "Resultaten": bit widths from 1 to 8 for keys and values
 * separately; 7 is not offered);
 * k_group in {32, 64, 128}; v_group in {64, 128};
 * 0 <= window <= KVQ_MAX_WINDOW; num_q_heads <= KVQ_MAX_HEADS; block_size in {0, 16};
 * value_rotation only with window == 0. */
#define KVQ_MAX_HEADS 4096
#define KVQ_MAX_WINDOW (1 << 20)
typedef struct {
  int32_t head_dim;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t k_bits, k_group;
  int32_t v_bits, v_group;
  int32_t window;       /* R: most recent tokens kept unquantized                */
  int32_t key_rotation; /* kvq_rotation                                           */
  int32_t kv_dtype;     /* kvq_dtype of appended K/V and of the window buffers    */
  int32_t block_size;   /* 0 = contiguous, 16 = paged                             */
  int32_t value_rotation; /* kvq_rotation of the values (a variant of [P3] "Resultaten"):
                           * values are rotated before they are quantized and the
                           * attention output is rotated back by the merge            */
} kvq_params;

typedef struct {
  void *pages;                /* page records (see Storage)                        */
  void *k_win, *v_win;        /* NULL iff window == 0                              */
  const int32_t *block_table; /* device [batch][max_blocks_per_seq]; NULL iff block_size == 0 */
  int32_t batch;
  int32_t max_blocks_per_seq; /* paged: table row length (ignored when contiguous) */
  int64_t capacity;           /* contiguous: tokens per sequence; paged: pages in the pool */
  uint32_t *error_flags;      /* optional device word (NULL: none), caller-owned and cleared by
                               * the caller; kernels OR in KVQ_DEV_* flags below             */
} kvq_cache;

/* Device-side input errors.  Inputs that only the device sees (lengths, per-sequence counts,
 * block-table entries) cannot be validated before launch.  The kernels keep every access inside
 * the buffers regardless (clamping or dropping as described below), so such inputs give wrong
 * results for the affected sequences but never touch memory outside the cache; when
 * cache->error_flags is set they also OR the matching flag into that word:
 *   KVQ_DEV_TABLE_ENTRY  a block-table entry read for a page holding data lies outside
 *                        [0, pool pages): the page read or written is the nearest pool page;
 *   KVQ_DEV_CAPACITY     an append reached a page beyond the cache (contiguous: capacity;
 *                        paged: max_blocks_per_seq): those quantized tokens were dropped;
 *   KVQ_DEV_LENGTH       a sequence length outside [0, max_seq_len] (attention, read-back,
 *                        diagnostics) or negative (append), or a length whose quantized part
 *                        exceeds the cache: it was clamped;
 *   KVQ_DEV_COUNT        an n_new_per_seq entry outside [0, n_new]: it was clamped. */
#define KVQ_DEV_TABLE_ENTRY 1u
#define KVQ_DEV_CAPACITY 2u
#define KVQ_DEV_LENGTH 4u
#define KVQ_DEV_COUNT 8u

/* Waits for the work queued on `stream` (a synchronizing call: not for use under graph
 * capture), then copies cache->error_flags into *flags.  Returns KVQ_EDEVICE if any flag is
 * set, KVQ_OK otherwise; KVQ_EINVAL without an error word or output pointer; KVQ_EHIP if the
 * copy fails.  The word is not cleared. */
kvq_status kvq_device_status(const kvq_cache *cache, uint32_t *flags, hipStream_t stream);

typedef struct {
  size_t record_bytes; /* one page of one kv head                                 */
  size_t pages_bytes;  /* whole quantized store for (batch, capacity)             */
  size_t window_bytes; /* each of k_win and v_win                                 */
} kvq_sizes;

/* Byte sizes of the buffers of a cache with `batch` sequences and `capacity`
 * (tokens per sequence when contiguous, pages in the pool when paged).
 * Memory accounting of payload plus metadata follows [P1] "Pertumbuhan cache
 * mengubah trade pada serving".  Returns KVQ_EINVAL / KVQ_EUNSUPPORTED for bad
 * parameters. */
kvq_status kvq_cache_sizes(const kvq_params *params, int32_t batch, int64_t capacity, kvq_sizes *out);

/* Append up to n_new tokens per sequence and quantize what leaves the window
 * ([P1] "Granularitas ..." for the quantizer, "Pertumbuhan cache ..." for the
 * window; [P3] "Resultaten" for key-only rotation).
 *   seq_lens_before: device int32 [batch], current lengths L_b.
 *   n_new_per_seq:   device int32 [batch] (each <= n_new), or NULL for n_new everywhere.
 *   k_new, v_new:    device [batch][n_new][num_kv_heads][128] of kv_dtype; token i of
 *                    sequence b becomes position L_b + i.
 * Afterwards positions t < L_b + n_b - window are in the quantized store and the
 * rest in the ring buffers.  The caller must size the cache for L_b + n_b tokens
 * (contiguous) and fill the block table for those pages (paged). */
kvq_status kvq_quantize_append(const kvq_params *params, const kvq_cache *cache, const int32_t *seq_lens_before,
                               const int32_t *n_new_per_seq, const void *k_new, const void *v_new, int32_t n_new,
                               hipStream_t stream);

/* Workspace bytes that kvq_decode_attention needs for this batch and maximum length.
 * Never decreases as max_seq_len grows, so a workspace sized for the largest length
 * serves every shorter one.  Returns 0 for invalid or unsupported parameters. */
size_t kvq_decode_workspace_bytes(const kvq_params *params, int32_t batch, int64_t max_seq_len);

/* Decode attention of one new query per sequence over its whole cache, with
 * dequantization fused into the kernel ([P1] "Error pada key masuk sebelum
 * softmax" for the computation, "Pertumbuhan cache ..." for the fusion).
 *   seq_lens:    device int32 [batch], lengths after the append (each <= max_seq_len).
 *   max_seq_len: host upper bound of seq_lens (sizes the launch; must fit the capacity).
 *   q:           device [batch][num_q_heads][128] of q_dtype.
 *   out:         device [batch][num_q_heads][128] of out_dtype; fp32 accumulation.
 *   softmax_scale: 0 means 1/sqrt(128).
 *   workspace:   device scratch of at least kvq_decode_workspace_bytes(...) bytes, 16-byte
 *                aligned, owned by the caller; no initial contents needed.  Calls that share
 *                a workspace must be ordered (same stream).
 * Two kernel launches: the split-K kernel writes per-split partial results into the
 * workspace, a second kernel merges them into `out`.
 * A sequence of length 0 gets an all-zero output.  Errors: KVQ_EINVAL (null or misaligned
 * pointers, bad dtype or scale), KVQ_ENOSPACE (workspace too small, max_seq_len beyond
 * the capacity), KVQ_EUNSUPPORTED (parameters outside the supported set), KVQ_EHIP
 * (launch failure); nothing is launched on an error. */
kvq_status kvq_decode_attention(const kvq_params *params, const kvq_cache *cache, const int32_t *seq_lens,
                                int64_t max_seq_len, const void *q, int32_t q_dtype, void *out, int32_t out_dtype,
                                float softmax_scale, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* The two launches of kvq_decode_attention, for callers that merge the partial results
 * themselves or schedule the two phases apart.  kvq_decode_partials takes the arguments of
 * kvq_decode_attention except out/out_dtype and leaves in the workspace, for every
 * (sequence, query head) row, entries s = 0 .. S-1 of KVQ_PART_FLOATS fp32 values
 * {m_s, l_s, n, 0, acc_s[128]}.  The first n entries of a row hold its splits (n is the same in
 * all of them, 1 <= n <= S; entries from n on are not written and hold garbage).  For a split, m_s is
 * a running maximum of its scores in log2 units (score * softmax_scale * log2(e)), l_s the sum of
 * 2^(score_log2 - m_s) and acc_s the matching unnormalised sum of values, l_s and acc_s scaled by
 * one common power of two; an empty split has m_s = -inf (its l_s and acc_s are 0).  With
 * M = max_s m_s over the split entries the attention output is
 * sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s ([P1] "Error pada key masuk sebelum softmax").
 * With value_rotation the acc_s are sums over rotated values: the merged row must then be
 * multiplied by the normalized 128-point Walsh-Hadamard matrix (kvq_decode_combine does this).
 * Rows are [batch][num_q_heads][S].  S (kvq_decode_splits) depends on (params, batch, max_seq_len,
 * q_dtype) and on the environment variables KVQ_PAGES_PER_SPLIT / KVQ_TARGET_WAVES, which must not
 * change between the two calls.  The split kernel sizes each sequence's splits from the lengths on
 * the device: the launch's waves are shared out over the sequences in proportion to their stored
 * pages (at most twice an equal share per (sequence, kv head)), so n differs between sequences of
 * different lengths.  kvq_decode_combine computes that merge into `out`
 * ([batch][num_q_heads][128] of out_dtype) from a workspace filled by kvq_decode_partials
 * with the same params, batch, max_seq_len and q_dtype.  Errors as for kvq_decode_attention. */
#define KVQ_PART_FLOATS 132
/* Row stride S (entries per row) of the partial results for these arguments (0 for invalid ones). */
int32_t kvq_decode_splits(const kvq_params *params, int32_t batch, int64_t max_seq_len, int32_t q_dtype);
kvq_status kvq_decode_partials(const kvq_params *params, const kvq_cache *cache, const int32_t *seq_lens,
                               int64_t max_seq_len, const void *q, int32_t q_dtype, float softmax_scale,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);
kvq_status kvq_decode_combine(const kvq_params *params, int32_t batch, int64_t max_seq_len, int32_t q_dtype,
                              const void *workspace, void *out, int32_t out_dtype, hipStream_t stream);

/* One decode step: append one token per sequence, then decode attention over the cache including
 * it -- the same results as kvq_quantize_append(n_new = 1) followed by kvq_decode_attention at
 * the lengths plus one, in fewer launches ([P1] "Pertumbuhan cache mengubah trade pada serving":
 * the recent window, and dequantization fused into the attention kernel).
 *   seq_lens_before: device int32 [batch], lengths L_b before the step (not modified; the caller
 *                    advances them afterwards).
 *   k_new, v_new:    device [batch][1][num_kv_heads][128] of kv_dtype, the token at position L_b.
 *   max_seq_len:     host upper bound of L_b + 1 (sizes the launch, as for kvq_decode_attention).
 *   q, out, softmax_scale, workspace: as for kvq_decode_attention (the same workspace size).
 * With a bf16 window (window > 0) the append runs inside the split-K launch: the split holding
 * the new token's ring slot quantizes the token leaving the window, stores it, attends it and
 * writes the new token into the ring, while the other splits read the stored tokens before the
 * step; then the merge launch.  Otherwise (no window, or fp32 rings) the append kernel runs
 * first, then the split-K and merge launches.
 * kvq_decode_step_partials stops before the merge: kvq_decode_combine(params, batch, max_seq_len,
 * q_dtype, ...) completes it.  Errors as for kvq_decode_attention, plus KVQ_EINVAL for null or
 * misaligned k_new / v_new; nothing is launched on an error. */
kvq_status kvq_decode_step(const kvq_params *params, const kvq_cache *cache, const int32_t *seq_lens_before,
                           const void *k_new, const void *v_new, int64_t max_seq_len, const void *q, int32_t q_dtype,
                           void *out, int32_t out_dtype, float softmax_scale, void *workspace, size_t workspace_bytes,
                           hipStream_t stream);
kvq_status kvq_decode_step_partials(const kvq_params *params, const kvq_cache *cache, const int32_t *seq_lens_before,
                                    const void *k_new, const void *v_new, int64_t max_seq_len, const void *q,
                                    int32_t q_dtype, float softmax_scale, void *workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* Decode attention that allocates nothing, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and launches as kvq_decode_attention, with the partial rows kept in a
 * device array inside the library instead of a caller workspace.  Arguments as for
 * kvq_decode_attention without workspace/workspace_bytes.
 *   Limit: kvq_decode_workspace_bytes(params, batch, max_seq_len) must not exceed
 *   KVQ_NOALLOC_SCRATCH_BYTES (16 MiB: every workload up to batch 64 x 64 query heads x 131072
 *   tokens fits); larger calls return KVQ_ENOSPACE and launch nothing.
 *   Each GPU holds one copy of the array from the first call on it until the process ends; the
 *   first call on a GPU looks up that copy's address (no allocation).  All calls on one GPU
 *   share the array and keep nothing from one call to the next, so calls that may overlap in
 *   time on one GPU (different streams without ordering) race and must not be issued.
 *   The stream's device is the device used (the current device for the null stream).  Errors as
 *   for kvq_decode_attention, KVQ_EHIP also when the array's address cannot be obtained. */
#define KVQ_NOALLOC_SCRATCH_BYTES (16u << 20)
kvq_status kvq_decode_attention_noalloc(const kvq_params *params, const kvq_cache *cache, const int32_t *seq_lens,
                                        int64_t max_seq_len, const void *q, int32_t q_dtype, void *out,
                                        int32_t out_dtype, float softmax_scale, hipStream_t stream);

/* Read back n positions [t0, t0 + n) of sequence `seq` in logical order (debug
 * and verification).  Any output pointer may be NULL.
 *   k_codes, v_codes: device uint8 [n][num_kv_heads][128]; 0xFF for window tokens and t >= L.
 *   k_meta:  device uint16 [n][num_kv_heads][128/k_group][2] fp16 bits {scale, zero};
 *   v_meta:  device uint16 [n][num_kv_heads][128/v_group][2]; 0xFFFF for non-quantized positions.
 *   k_hat, v_hat: device fp32 [n][num_kv_heads][128]: round-to-fp32 of zero + code*scale for
 *            quantized positions (rotated domain for keys with rotation on), the stored
 *            value for window positions, NaN for t >= L. */
kvq_status kvq_dequantize_debug(const kvq_params *params, const kvq_cache *cache, const int32_t *seq_lens,
                                int32_t seq, int64_t t0, int64_t n, uint8_t *k_codes, uint8_t *v_codes,
                                uint16_t *k_meta, uint16_t *v_meta, float *k_hat, float *v_hat,
                                hipStream_t stream);

/* Unfused baseline ([P1] "Pertumbuhan cache mengubah trade pada serving": dequantizing into
 * temporary storage instead of inside the attention kernel).  It exists to measure what the
 * fused path gains; the fused entry points above do not use it.
 *
 * kvq_dequantize_dense writes positions t < min(seq_lens[b], max_seq_len) of every sequence b
 * and kv head h into dense bf16 arrays k_out, v_out, each [batch][num_kv_heads][max_seq_len][128]
 * (device, caller-owned, 16-byte aligned, max_seq_len <= 2^31 - 1): a quantized position as
 * round-to-nearest-even of zero + code * scale evaluated exactly in fp64, rotated back to the
 * original domain first when its tensor is rotated (the transform is its own inverse); a window
 * position as its stored value (fp32 rounded to nearest even).  Positions t >= seq_lens[b] are not
 * written; positions beyond the cache capacity are written as zeros.  Errors as for
 * kvq_dequantize_debug.
 *
 * kvq_dense_decode_attention computes, for every sequence b and query head h, the softmax
 * attention of q[b][h] over positions t < min(seq_lens[b], max_seq_len) of dense bf16 k, v laid
 * out as above (query head h reads kv head h / (num_q_heads / num_kv_heads); all-zero output for
 * an empty sequence), in fp32 with splits of 256 positions merged as in kvq_decode_combine.
 * Only num_q_heads / num_kv_heads of params are used (params must still be valid).  q, out,
 * softmax_scale as for kvq_decode_attention; workspace (device, 16-byte aligned) of at least
 * kvq_dense_workspace_bytes(params, batch, max_seq_len) bytes.  Errors: KVQ_EINVAL for null or
 * misaligned pointers or bad dtypes or scale, KVQ_ENOSPACE for a short workspace. */
kvq_status kvq_dequantize_dense(const kvq_params *params, const kvq_cache *cache, const int32_t *seq_lens,
                                int64_t max_seq_len, uint16_t *k_out, uint16_t *v_out, hipStream_t stream);
size_t kvq_dense_workspace_bytes(const kvq_params *params, int32_t batch, int64_t max_seq_len);
kvq_status kvq_dense_decode_attention(const kvq_params *params, int32_t batch, const uint16_t *k, const uint16_t *v,
                                      const int32_t *seq_lens, int64_t max_seq_len, const void *q, int32_t q_dtype,
                                      void *out, int32_t out_dtype, float softmax_scale, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* Error-budget diagnostics ([P1] "Error pada key masuk sebelum softmax", "Error pada value masuk
 * setelah bobot attention terbentuk", "Evaluasi harus sesuai dengan besaran yang ingin
 * dipertahankan"; [P2]'s entries on separate key and value error budgets).  Compares the cache
 * with the original keys and values k_ref, v_ref (device bf16 [batch][max_seq_len][num_kv_heads]
 * [128], the rows that were appended; 16-byte aligned) for the query q (as for
 * kvq_decode_attention).  For sequence b, query head h, over positions t < min(seq_lens[b],
 * max_seq_len), with exact scores s_t = scale * q.k_t, quantized scores s'_t = scale * q.k_hat_t,
 * a = softmax(s), a' = softmax(s') and window positions exact (k_hat = k, v_hat = v there),
 * head_stats[b][h][0..7] (device fp32, 16-byte aligned) receives
 *   {max_t |s'_t - s_t|, sqrt(mean_t (s'_t - s_t)^2), sum_t |a'_t - a_t| / 2,
 *    |a V_hat - a V| (value error alone), |a' V - a V| (key error alone),
 *    |a' V_hat - a V| (both), |a V|, 0}     (Euclidean norms over the 128 channels),
 * and unit_stats[b][kv][0..7] (device fp32, 16-byte aligned) the reconstruction errors over the
 * quantized positions {sum (k_hat - k)^2, sum (v_hat - v)^2, max |k_hat - k|, max |v_hat - v|,
 *    sum k^2, sum v^2, number of quantized positions, 0}.
 * fp32 arithmetic, reconstructions zero + code * scale rounded to fp32.  Reconstructions of
 * rotated keys or values are rotated back first: every error is taken in the original domain.
 * The query is taken as bf16 hi + lo parts (exact for a bf16 query; about 16 significant bits of
 * an fp32 one) and must stay below 2^27 in magnitude.  workspace (device, 16-byte aligned) of at
 * least kvq_error_budget_workspace_bytes(params, cache->batch, max_seq_len) bytes (about
 * 8 * batch * num_q_heads * max_seq_len) holds what the three launches pass on: per range of each
 * sequence, the score statistics and the weighted sums, and both scores of every position; its
 * contents are not needed between calls.  Errors as for kvq_decode_attention, and KVQ_ENOSPACE
 * for a short workspace. */
#define KVQ_EB_HEAD 8
#define KVQ_EB_UNIT 8
size_t kvq_error_budget_workspace_bytes(const kvq_params *params, int32_t batch, int64_t max_seq_len);
kvq_status kvq_error_budget(const kvq_params *params, const kvq_cache *cache, const int32_t *seq_lens,
                            int64_t max_seq_len, const uint16_t *k_ref, const uint16_t *v_ref, const void *q,
                            int32_t q_dtype, float softmax_scale, float *head_stats, float *unit_stats,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Static description of a status code. */
const char *kvq_status_str(kvq_status status);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
