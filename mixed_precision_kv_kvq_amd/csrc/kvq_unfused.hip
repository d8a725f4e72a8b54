// Unfused baseline: dequantize the whole quantized store into a dense bf16 cache, then run a
// plain decode attention over that cache.  nalar.dev "Kuantisasi KV cache mengganggu attention
// melalui key dan value tersimpan", section "Pertumbuhan cache mengubah trade pada serving",
// names dequantization into temporary storage as the alternative to dequantizing inside the
// attention kernel, and warns that a smaller cache does not settle latency by itself; this path
// measures what the fused kernel gains.  Dequantization follows section "Granularitas kuantisasi
// menentukan nilai yang berbagi scale" (x_hat = zero + code * scale); attention follows section
// "Error pada key masuk sebelum softmax" (s = q K^T / sqrt(d), a = softmax(s), o = a V).
#include "kvq_extras.h"

#pragma clang fp contract(off)

namespace {

// Round-to-nearest-even of a finite fp64 value to bf16 bits.  The callers' values are zero or
// of magnitude between 2^-40 and 2^40, inside bf16's normal range.
__device__ inline uint32_t f64_to_bf16_rne(double x) {
  uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t sign = (uint32_t)(u >> 63) << 15;
  u &= 0x7FFFFFFFFFFFFFFFull;
  if (u == 0) return sign;
  u += 0xFFFFFFFFFFFull + ((u >> 45) & 1u);  // drop 45 of the 52 fraction bits, ties to even
  const int e = (int)(u >> 52) - 1023;
  return sign | ((uint32_t)(e + 127) << 7) | (uint32_t)((u >> 45) & 0x7Fu);
}

__device__ inline float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);  // exact
}

// bf16 bits of zero + code * scale, rounded once to nearest even, in fp32 arithmetic: the
// product is exact (an 8-bit code times an 11-bit fp16 scale); the sum s and its exact error
// err come from TwoSum; s is turned into the round-to-odd value of the exact sum (truncate
// toward zero, then set the last bit when inexact), whose 24 bits round to bf16's 8 exactly
// as the exact sum would (round-to-odd followed by a rounding at least two bits shorter).
__device__ inline uint32_t affine_bf16(float zero, float scale, uint32_t code) {
  const float p = (float)code * scale;
  const float s = zero + p;
  const float bv = s - zero;
  const float err = (zero - (s - bv)) + (p - bv);
  uint32_t u = __builtin_bit_cast(uint32_t, s);
  if (err != 0.f) {
    if ((err > 0.f) != (s > 0.f)) u -= 1u;  // the exact sum is closer to zero than s
    u |= 1u;
  }
  return kvq_f32_to_bf16_rne(__builtin_bit_cast(float, u));
}

// One wave per (page, kv head, sequence): the page's 16 positions, lane l holding channels
// 2l and 2l + 1.  The page record is staged in LDS once; each position's two codes per lane
// are read from there.  Unrotated tensors: affine_bf16.  Rotated tensors: x_hat = zero + code *
// scale exact in fp64, rotated back in fp64 (the transform is its own inverse), rounded once to
// bf16.  Window positions copy their stored values.
__global__ __launch_bounds__(64) void kvq_dequantize_dense_kernel(KvqDenseArgs a) {
  constexpr int kMaxRecord16 = (256 * 8 + 64 * 4 + 256 * 8 + 64 * 2) / 16;
  __shared__ uint4 rec_s[kMaxRecord16];
  const int lane = threadIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t page = blockIdx.x;
  const int Hkv = a.Hkv, R = a.R;
  int64_t L = a.seq_lens[b];
  kvq_raise(a.cache, page == 0 && h == 0 && (L < 0 || L > a.max_len), KVQ_DEV_LENGTH);
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  const int64_t t_first = page * KVQ_PAGE;
  if (t_first >= L) return;
  int64_t nq = L > R ? L - R : 0;
  const int64_t cap_tokens = (a.cache.paged ? (int64_t)a.cache.mbps : a.cache.pages_per_seq) * KVQ_PAGE;
  if (nq > cap_tokens) nq = cap_tokens;  // lengths beyond the cache read nothing
  const int64_t wstart = L > R ? L - R : 0;  // first window position
  const KvqLayout &lay = a.lay;
  if (t_first < nq) {
    const int64_t rec_idx = kvq_record_index_dev(a.cache, Hkv, b, h, page);
    const uint4 *rec = reinterpret_cast<const uint4 *>(a.cache.pages + (size_t)rec_idx * lay.record);
    for (int c = lane; c < lay.record / 16; c += 64) rec_s[c] = rec[c];
    __syncthreads();
  }
  const uint8_t *rs = reinterpret_cast<const uint8_t *>(rec_s);
  const size_t row0 = ((size_t)b * Hkv + h) * (size_t)a.max_len;
  const int esz = a.kv_f32 ? 4 : 2;
  if (!a.rotation && !a.value_rotation) {
    // Lane 16 r + c8 writes channels [8 c8, 8 c8 + 8) of position 4 it + r: one 16-byte store
    // per tensor, four whole 256-byte rows per store instruction.
    const int r = lane >> 4, c8 = lane & 15;
#pragma unroll
    for (int it = 0; it < KVQ_PAGE / 4; ++it) {
      const int n = 4 * it + r;
      const int64_t t = t_first + n;
      if (t >= L) break;
      uint32_t ko[4], vo[4];
      if (t < nq) {
        const uint32_t km = reinterpret_cast<const uint32_t *>(rs + lay.k_meta_off)[kvq_meta_dword(lay.nkg, n, (8 * c8) / lay.kg)];
        const uint32_t vm = reinterpret_cast<const uint32_t *>(rs + lay.v_meta_off)[kvq_meta_dword(lay.nvg, n, (8 * c8) / lay.vg)];
        const float kz = f16_bits_to_f32(km >> 16), ks = f16_bits_to_f32(km & 0xFFFF);
        const float vz = f16_bits_to_f32(vm >> 16), vs = f16_bits_to_f32(vm & 0xFFFF);
        uint32_t kc[8], vc[8];
        if ((lay.kb & (lay.kb - 1)) == 0)
          kvq_k_codes8_one(rs + lay.k_codes_off, lay.kb, n, c8, kc);
        else
          kvq_k_codes8(rs + lay.k_codes_off, lay.kb, n, c8, kc);
        if ((lay.vb & (lay.vb - 1)) == 0)
          kvq_v_codes8_one(rs + lay.v_codes_off, lay.vb, n, c8, vc);
        else
          kvq_v_codes8(rs + lay.v_codes_off, lay.vb, n, c8, vc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ko[i] = affine_bf16(kz, ks, kc[2 * i]) | (affine_bf16(kz, ks, kc[2 * i + 1]) << 16);
          vo[i] = affine_bf16(vz, vs, vc[2 * i]) | (affine_bf16(vz, vs, vc[2 * i + 1]) << 16);
        }
      } else if (t < wstart) {  // beyond the cache: not stored
#pragma unroll
        for (int i = 0; i < 4; ++i) ko[i] = vo[i] = 0u;
      } else {  // recent window: ring slot t mod R
        const size_t off = (((size_t)b * Hkv + h) * R + (size_t)(t % R)) * KVQ_D * esz;
        if (a.kv_f32) {
          const float4 *kf = reinterpret_cast<const float4 *>(a.cache.k_win + off) + 2 * c8;
          const float4 *vf = reinterpret_cast<const float4 *>(a.cache.v_win + off) + 2 * c8;
          const float4 k0 = kf[0], k1 = kf[1], v0 = vf[0], v1 = vf[1];
          ko[0] = kvq_f32_to_bf16_rne(k0.x) | (kvq_f32_to_bf16_rne(k0.y) << 16);
          ko[1] = kvq_f32_to_bf16_rne(k0.z) | (kvq_f32_to_bf16_rne(k0.w) << 16);
          ko[2] = kvq_f32_to_bf16_rne(k1.x) | (kvq_f32_to_bf16_rne(k1.y) << 16);
          ko[3] = kvq_f32_to_bf16_rne(k1.z) | (kvq_f32_to_bf16_rne(k1.w) << 16);
          vo[0] = kvq_f32_to_bf16_rne(v0.x) | (kvq_f32_to_bf16_rne(v0.y) << 16);
          vo[1] = kvq_f32_to_bf16_rne(v0.z) | (kvq_f32_to_bf16_rne(v0.w) << 16);
          vo[2] = kvq_f32_to_bf16_rne(v1.x) | (kvq_f32_to_bf16_rne(v1.y) << 16);
          vo[3] = kvq_f32_to_bf16_rne(v1.z) | (kvq_f32_to_bf16_rne(v1.w) << 16);
        } else {
          const uint4 kw = reinterpret_cast<const uint4 *>(a.cache.k_win + off)[c8];
          const uint4 vw = reinterpret_cast<const uint4 *>(a.cache.v_win + off)[c8];
          ko[0] = kw.x; ko[1] = kw.y; ko[2] = kw.z; ko[3] = kw.w;
          vo[0] = vw.x; vo[1] = vw.y; vo[2] = vw.z; vo[3] = vw.w;
        }
      }
      reinterpret_cast<uint4 *>(a.k_out + (row0 + (size_t)t) * KVQ_D)[c8] = make_uint4(ko[0], ko[1], ko[2], ko[3]);
      reinterpret_cast<uint4 *>(a.v_out + (row0 + (size_t)t) * KVQ_D)[c8] = make_uint4(vo[0], vo[1], vo[2], vo[3]);
    }
    return;
  }
  // Rotated keys or values: lane l holds channels 2l, 2l + 1 of one position at a time, the
  // layout of the cross-lane transform.
#pragma unroll 4
  for (int n = 0; n < KVQ_PAGE; ++n) {
    const int64_t t = t_first + n;
    if (t >= L) break;
    uint32_t kout, vout;
    if (t < nq) {
      // channels 2 lane and 2 lane + 1 (both in one group)
      const uint32_t kc0 = kvq_k_code(rs + lay.k_codes_off, lay.kb, n, 2 * lane);
      const uint32_t kc1 = kvq_k_code(rs + lay.k_codes_off, lay.kb, n, 2 * lane + 1);
      const uint32_t vc0 = kvq_v_code(rs + lay.v_codes_off, lay.vb, n, 2 * lane);
      const uint32_t vc1 = kvq_v_code(rs + lay.v_codes_off, lay.vb, n, 2 * lane + 1);
      const uint32_t km = reinterpret_cast<const uint32_t *>(rs + lay.k_meta_off)[kvq_meta_dword(lay.nkg, n, (2 * lane) / lay.kg)];
      const uint32_t vm = reinterpret_cast<const uint32_t *>(rs + lay.v_meta_off)[kvq_meta_dword(lay.nvg, n, (2 * lane) / lay.vg)];
      if (a.rotation) {
        const double z = kvq_f16_bits_to_f64(km >> 16), sc = kvq_f16_bits_to_f64(km & 0xFFFF);
        double x0 = z + (double)kc0 * sc, x1 = z + (double)kc1 * sc;
        kvq_wht128_fp64(x0, x1, lane);
        kout = f64_to_bf16_rne(x0) | (f64_to_bf16_rne(x1) << 16);
      } else {
        const float z = f16_bits_to_f32(km >> 16), sc = f16_bits_to_f32(km & 0xFFFF);
        kout = affine_bf16(z, sc, kc0) | (affine_bf16(z, sc, kc1) << 16);
      }
      if (a.value_rotation) {
        const double z = kvq_f16_bits_to_f64(vm >> 16), sc = kvq_f16_bits_to_f64(vm & 0xFFFF);
        double x0 = z + (double)vc0 * sc, x1 = z + (double)vc1 * sc;
        kvq_wht128_fp64(x0, x1, lane);
        vout = f64_to_bf16_rne(x0) | (f64_to_bf16_rne(x1) << 16);
      } else {
        const float z = f16_bits_to_f32(vm >> 16), sc = f16_bits_to_f32(vm & 0xFFFF);
        vout = affine_bf16(z, sc, vc0) | (affine_bf16(z, sc, vc1) << 16);
      }
    } else if (t < wstart) {  // beyond the cache: not stored
      kout = 0u;
      vout = 0u;
    } else {  // recent window: ring slot t mod R
      const size_t off = (((size_t)b * Hkv + h) * R + (size_t)(t % R)) * KVQ_D * esz;
      if (a.kv_f32) {
        const float2 kf = reinterpret_cast<const float2 *>(a.cache.k_win + off)[lane];
        const float2 vf = reinterpret_cast<const float2 *>(a.cache.v_win + off)[lane];
        kout = kvq_f32_to_bf16_rne(kf.x) | (kvq_f32_to_bf16_rne(kf.y) << 16);
        vout = kvq_f32_to_bf16_rne(vf.x) | (kvq_f32_to_bf16_rne(vf.y) << 16);
      } else {
        kout = reinterpret_cast<const uint32_t *>(a.cache.k_win + off)[lane];
        vout = reinterpret_cast<const uint32_t *>(a.cache.v_win + off)[lane];
      }
    }
    reinterpret_cast<uint32_t *>(a.k_out + (row0 + (size_t)t) * KVQ_D)[lane] = kout;
    reinterpret_cast<uint32_t *>(a.v_out + (row0 + (size_t)t) * KVQ_D)[lane] = vout;
  }
}

__device__ inline void bf16x8_to_f32(const uint4 w, float *x) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = kvq_bf16_bits_to_f32(ws[i] & 0xFFFFu);
    x[2 * i + 1] = kvq_bf16_bits_to_f32(ws[i] >> 16);
  }
}

// Dense decode attention, one wave per (split of KVQ_DENSE_SPLIT positions, kv head, sequence)
// for the G query heads of the kv head.  Lane 16 r + c reads channels [8c, 8c + 8) of
// position 4i + r (four 256-byte rows per load).  Scores (log2 units) go to LDS, are turned
// into weights 2^(s - m) with the split's maximum m, and the weighted value rows are summed;
// the partial row {m, l, 0, 0, acc[128]} of each head is merged by the combine kernel.
template <int G>
__global__ __launch_bounds__(64) void kvq_dense_partials_kernel(KvqDenseArgs a) {
  constexpr int T = KVQ_DENSE_SPLIT;
  __shared__ float w_s[G][T];
  const int lane = threadIdx.x, s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int r = lane >> 4, c = lane & 15;
  int64_t L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  const int64_t t0 = (int64_t)s * T;
  const int n = L - t0 <= 0 ? 0 : (L - t0 >= T ? T : (int)(L - t0));
  const size_t row0 = ((size_t)b * a.Hkv + h) * (size_t)a.max_len;
  const float ninf = -__builtin_inff();
  if (n == 0) {
    for (int hh = 0; hh < G; ++hh) {
      float *pr = a.partials + (((size_t)b * a.Hq + h * G + hh) * a.splits + s) * KVQ_PART_STRIDE;
      reinterpret_cast<float2 *>(pr + 4)[lane] = make_float2(0.f, 0.f);
      if (lane == 0) *reinterpret_cast<float4 *>(pr) = make_float4(ninf, 0.f, (float)a.splits, 0.f);
    }
    return;
  }
  // query channels [8c, 8c + 8) of each head, scaled to log2 units
  float qr[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const size_t qrow = ((size_t)b * a.Hq + h * G + hh) * KVQ_D + 8 * c;
    if (a.q_f32) {
      const float4 *qp = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.q) + qrow);
      const float4 x = qp[0], y = qp[1];
      const float v[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) qr[hh][e] = v[e] * a.sigma;
    } else {
      float v[8];
      bf16x8_to_f32(*reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a.q) + qrow), v);
#pragma unroll
      for (int e = 0; e < 8; ++e) qr[hh][e] = v[e] * a.sigma;
    }
  }
  // scores: four loads in flight per lane, then the dot products
  constexpr int U = 4;
  for (int i0 = 0; i0 < n; i0 += 4 * U) {
    uint4 kw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = i0 + 4 * u + r;
      kw[u] = j < n ? reinterpret_cast<const uint4 *>(a.k_in + (row0 + (size_t)(t0 + j)) * KVQ_D)[c]
                    : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = i0 + 4 * u + r;
      float k[8];
      bf16x8_to_f32(kw[u], k);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = __builtin_fmaf(qr[hh][e], k[e], d);
        d += __shfl_xor(d, 1);
        d += __shfl_xor(d, 2);
        d += __shfl_xor(d, 4);
        d += __shfl_xor(d, 8);
        if (c == 0 && j < T) w_s[hh][j] = j < n ? d : ninf;
      }
    }
  }
  __syncthreads();
  // per head: split maximum, weights 2^(s - m), their sum
  float m[G], l[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float mx = ninf;
    for (int j = lane; j < n; j += 64) mx = __builtin_fmaxf(mx, w_s[hh][j]);
    for (int off = 32; off >= 1; off >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, off));
    float sum = 0.f;
    for (int j = lane; j < n; j += 64) {
      const float p = __builtin_amdgcn_exp2f(w_s[hh][j] - mx);
      w_s[hh][j] = p;
      sum += p;
    }
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    m[hh] = mx;
    l[hh] = sum;
  }
  __syncthreads();
  // weighted value rows
  float acc[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
  for (int i0 = 0; i0 < n; i0 += 4 * U) {
    uint4 vw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = i0 + 4 * u + r;
      vw[u] = j < n ? reinterpret_cast<const uint4 *>(a.v_in + (row0 + (size_t)(t0 + j)) * KVQ_D)[c]
                    : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = i0 + 4 * u + r;
      float v[8];
      bf16x8_to_f32(vw[u], v);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float p = j < n ? w_s[hh][j] : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = __builtin_fmaf(p, v[e], acc[hh][e]);
      }
    }
  }
  // sum over the four position classes r (lanes c, c + 16, c + 32, c + 48), then lanes 0..15
  // write channels [8c, 8c + 8) of each head
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[hh][e] += __shfl_xor(acc[hh][e], 16);
      acc[hh][e] += __shfl_xor(acc[hh][e], 32);
    }
    float *pr = a.partials + (((size_t)b * a.Hq + h * G + hh) * a.splits + s) * KVQ_PART_STRIDE;
    if (r == 0) {
      float4 *dst = reinterpret_cast<float4 *>(pr + 4 + 8 * c);
      dst[0] = make_float4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]);
      dst[1] = make_float4(acc[hh][4], acc[hh][5], acc[hh][6], acc[hh][7]);
    }
    if (lane == 0) *reinterpret_cast<float4 *>(pr) = make_float4(m[hh], l[hh], (float)a.splits, 0.f);  // every entry written
  }
}

}  // namespace

hipError_t kvq_launch_dequantize_dense(const KvqDenseArgs &a, hipStream_t s) {
  if (a.B <= 0 || a.max_len <= 0) return hipSuccess;
  (void)hipGetLastError();  // drop a stale error left by an earlier, unrelated call
  const dim3 grid((unsigned)((a.max_len + KVQ_PAGE - 1) / KVQ_PAGE), (unsigned)a.Hkv, (unsigned)a.B);
  hipLaunchKernelGGL(kvq_dequantize_dense_kernel, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t kvq_launch_dense_partials(const KvqDenseArgs &a, int g, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  (void)hipGetLastError();
  const dim3 grid((unsigned)a.splits, (unsigned)a.Hkv, (unsigned)a.B);
  switch (g) {
    case 1: hipLaunchKernelGGL(kvq_dense_partials_kernel<1>, grid, dim3(64), 0, s, a); break;
    case 2: hipLaunchKernelGGL(kvq_dense_partials_kernel<2>, grid, dim3(64), 0, s, a); break;
    case 4: hipLaunchKernelGGL(kvq_dense_partials_kernel<4>, grid, dim3(64), 0, s, a); break;
    case 8: hipLaunchKernelGGL(kvq_dense_partials_kernel<8>, grid, dim3(64), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
