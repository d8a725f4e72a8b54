// Read-back of stored positions in logical order (verification and debugging).
// Dequantization follows nalar.dev "Kuantisasi KV cache mengganggu attention
// melalui key dan value tersimpan", section "Granularitas kuantisasi menentukan
// nilai yang berbagi scale": x_hat = zero + code * scale (offset convention),
// evaluated in fp64 and rounded once to fp32.
#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace {

__global__ __launch_bounds__(64) void kvq_debug_kernel(KvqDebugArgs a) {
  const int lane = threadIdx.x, h = blockIdx.y, Hkv = a.Hkv;
  const int64_t idx = blockIdx.x, t = a.t0 + idx;
  const int L = a.seq_lens[a.seq];
  const int R = a.R;
  int64_t nq = L > R ? (int64_t)L - R : 0;
  const int64_t cap_tokens = (a.cache.paged ? (int64_t)a.cache.mbps : a.cache.pages_per_seq) * KVQ_PAGE;
  kvq_raise(a.cache, idx == 0 && h == 0 && (L < 0 || nq > cap_tokens), KVQ_DEV_LENGTH);
  if (nq > cap_tokens) nq = cap_tokens;  // lengths beyond the cache read nothing
  const KvqLayout &lay = a.lay;
  const int64_t ob = idx * Hkv + h;  // output row
  const float qnan = __builtin_nanf("");
  for (int e = 0; e < 2; ++e) {
    const int c = 2 * lane + e;
    uint32_t kc = 0xFF, vc = 0xFF;
    float kh = qnan, vh = qnan;
    if (t < nq) {
      const int64_t rec_idx = kvq_record_index_dev(a.cache, Hkv, a.seq, h, t / KVQ_PAGE);
      const uint8_t *rec = a.cache.pages + (size_t)rec_idx * lay.record;
      const int n = (int)(t % KVQ_PAGE);
      kc = kvq_k_code(rec + lay.k_codes_off, lay.kb, n, c);
      vc = kvq_v_code(rec + lay.v_codes_off, lay.vb, n, c);
      const uint32_t km = reinterpret_cast<const uint32_t *>(rec + lay.k_meta_off)[kvq_meta_dword(lay.nkg, n, c / lay.kg)];
      const uint32_t vm = reinterpret_cast<const uint32_t *>(rec + lay.v_meta_off)[kvq_meta_dword(lay.nvg, n, c / lay.vg)];
      kh = (float)(kvq_f16_bits_to_f64(km >> 16) + (double)kc * kvq_f16_bits_to_f64(km & 0xFFFF));
      vh = (float)(kvq_f16_bits_to_f64(vm >> 16) + (double)vc * kvq_f16_bits_to_f64(vm & 0xFFFF));
      if (e == 0 && lane < lay.nkg && a.k_meta) {
        const uint32_t m = reinterpret_cast<const uint32_t *>(rec + lay.k_meta_off)[kvq_meta_dword(lay.nkg, n, lane)];
        a.k_meta[(ob * lay.nkg + lane) * 2] = (uint16_t)(m & 0xFFFF);
        a.k_meta[(ob * lay.nkg + lane) * 2 + 1] = (uint16_t)(m >> 16);
      }
      if (e == 0 && lane < lay.nvg && a.v_meta) {
        const uint32_t m = reinterpret_cast<const uint32_t *>(rec + lay.v_meta_off)[kvq_meta_dword(lay.nvg, n, lane)];
        a.v_meta[(ob * lay.nvg + lane) * 2] = (uint16_t)(m & 0xFFFF);
        a.v_meta[(ob * lay.nvg + lane) * 2 + 1] = (uint16_t)(m >> 16);
      }
    } else {
      if (t < L && R > 0) {
        const int esz = a.kv_f32 ? 4 : 2;
        const size_t off = (((size_t)a.seq * Hkv + h) * R + (size_t)(t % R)) * KVQ_D * esz;
        if (a.kv_f32) {
          kh = reinterpret_cast<const float *>(a.cache.k_win + off)[c];
          vh = reinterpret_cast<const float *>(a.cache.v_win + off)[c];
        } else {
          kh = kvq_bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(a.cache.k_win + off)[c]);
          vh = kvq_bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(a.cache.v_win + off)[c]);
        }
      }
      if (e == 0 && a.k_meta && lane < lay.nkg) {
        a.k_meta[(ob * lay.nkg + lane) * 2] = 0xFFFF;
        a.k_meta[(ob * lay.nkg + lane) * 2 + 1] = 0xFFFF;
      }
      if (e == 0 && a.v_meta && lane < lay.nvg) {
        a.v_meta[(ob * lay.nvg + lane) * 2] = 0xFFFF;
        a.v_meta[(ob * lay.nvg + lane) * 2 + 1] = 0xFFFF;
      }
    }
    if (a.k_codes) a.k_codes[ob * KVQ_D + c] = (uint8_t)kc;
    if (a.v_codes) a.v_codes[ob * KVQ_D + c] = (uint8_t)vc;
    if (a.k_hat) a.k_hat[ob * KVQ_D + c] = kh;
    if (a.v_hat) a.v_hat[ob * KVQ_D + c] = vh;
  }
}

}  // namespace

hipError_t kvq_launch_debug(const KvqDebugArgs &a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  dim3 grid((unsigned)a.n, (unsigned)a.Hkv);
  (void)hipGetLastError();  // drop a stale error left by an earlier, unrelated call
  hipLaunchKernelGGL(kvq_debug_kernel, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}
