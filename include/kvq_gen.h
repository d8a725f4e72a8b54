/*
 * kvq_gen.h — device-side seeded input generator (test and benchmark
 * infrastructure; not part of the attention method).
 *
 * Same definition as workloads/__init__.py: element idx of the stream with
 * 64-bit key `key` is SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) at state
 * key + (idx + 1) * 0x9E3779B97F4A7C15; its top 16 bits index `table` (65536
 * fp32 standard-normal quantiles); the value is fp32(sigma * z), rounded to bf16
 * (nearest even) when out_f32 == 0.
 */
#ifndef KVQ_GEN_H
#define KVQ_GEN_H
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* K or V rows for tokens [t0, t0 + n) of every sequence and kv head:
 * out [B][n][Hkv][d]; element (b, h, t, c) has idx ((b*Hkv + h) * 2^24 + t) * d + c
 * and sigma = sigma[h * d + c] (device fp32 [Hkv][d]). Returns a hipError_t. */
int kvq_gen_kv(void *out, int out_f32, uint64_t key, const float *sigma, const float *table, int B, int n, int Hkv,
               int64_t t0, int d, hipStream_t stream);

/* Queries of one decode step: out [B][Hq][d]; idx ((step*B + b)*Hq + h)*d + c, sigma 1. */
int kvq_gen_q(void *out, int out_f32, uint64_t key, const float *table, int B, int Hq, int d, int step,
              hipStream_t stream);

/* Benchmark ceiling: read floor(bytes / 16) 16-byte words of device buffer `buf` (16-byte
 * aligned) once, with `blocks` workgroups of 256 lanes, plain or non-temporal loads; `sink`
 * (device, >= 256 uint32) is written only in the unlikely case that the xor of all words a lane
 * read equals 0x9E3779B9.  Returns a hipError_t. */
int kvq_gen_stream_read(const void *buf, size_t bytes, uint32_t *sink, int blocks, int nontemporal,
                        hipStream_t stream);

/* Counter calibration: copy floor(bytes / 16) 16-byte words from `src` to `dst` (device, 16-byte
 * aligned, not overlapping), a kernel whose HBM traffic is known exactly (that many bytes read
 * and written).  Returns a hipError_t. */
int kvq_gen_stream_copy(void *dst, const void *src, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif
