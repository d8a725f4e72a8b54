// Cross-split combine of flash-decoding partials and dispatch of the split kernel.
//
// Each split s of a (sequence, query head) holds its own max m_s (log2 units),
// sum l_s of 2^(score - m_s) and unnormalized output acc_s.  With M = max m_s the
// softmax of nalar.dev "Kuantisasi KV cache mengganggu attention melalui key dan
// value tersimpan", section "Error pada key masuk sebelum softmax", is
//   o = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
#include "kvq_internal.h"

namespace kvq_attn {
hipError_t launch_k1v1(const KvqAttnArgs &a, int g, int p, int nvg, hipStream_t s);
hipError_t launch_k1v2(const KvqAttnArgs &a, int g, int p, int nvg, hipStream_t s);
hipError_t launch_k1v4(const KvqAttnArgs &a, int g, int p, int nvg, hipStream_t s);
hipError_t launch_k1v8(const KvqAttnArgs &a, int g, int p, int nvg, hipStream_t s);
hipError_t launch_k2v1(const KvqAttnArgs &a, int g, int p, int nvg, hipStream_t s);
hipError_t launch_k2v2(const KvqAttnArgs &a, int g, int p, int nvg, hipStream_t s);
hipError_t launch_k2v4(const KvqAttnArgs &a, int g, int p, int nvg, hipStream_t s);
hipError_t launch_k2v8(const KvqAttnArgs &a, int g, int p, int nvg, hipStream_t s);
hipError_t launch_k4v1(const KvqAttnArgs &a, int g, int p, int nvg, hipStream_t s);
hipError_t launch_k4v2(const KvqAttnArgs &a, int g, int p, int nvg, hipStream_t s);
hipError_t launch_k4v4(const KvqAttnArgs &a, int g, int p, int nvg, hipStream_t s);
hipError_t launch_k4v8(const KvqAttnArgs &a, int g, int p, int nvg, hipStream_t s);
hipError_t launch_k8v1(const KvqAttnArgs &a, int g, int p, int nvg, hipStream_t s);
hipError_t launch_k8v2(const KvqAttnArgs &a, int g, int p, int nvg, hipStream_t s);
hipError_t launch_k8v4(const KvqAttnArgs &a, int g, int p, int nvg, hipStream_t s);
hipError_t launch_k8v8(const KvqAttnArgs &a, int g, int p, int nvg, hipStream_t s);
}  // namespace kvq_attn

namespace {

// One wave per (sequence, query head).  Splits are taken 32 at a time: the
// headers (lane s holds split s) and all 32 accumulator rows are requested
// before any is used, so a chunk costs one memory round trip; chunks are
// merged online (running max M, sum l and output o rescaled as M grows).
constexpr int kChunk = 32;

__global__ __launch_bounds__(64) void kvq_combine_kernel(KvqCombineArgs a) {
  const int lane = threadIdx.x;
  const size_t bh = blockIdx.x;
  const float *base = a.partials + bh * (size_t)a.splits * KVQ_PART_STRIDE;
  const float ninf = -__builtin_inff();
  float M = ninf, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s0 = 0; s0 < a.splits; s0 += kChunk) {
    const int n = (a.splits - s0) < kChunk ? (a.splits - s0) : kChunk;
    const float *cb = base + (size_t)s0 * KVQ_PART_STRIDE;
    const bool mine = lane < n;
    const float ms = mine ? cb[(size_t)lane * KVQ_PART_STRIDE] : ninf;
    const float ls = mine ? cb[(size_t)lane * KVQ_PART_STRIDE + 1] : 0.f;
    float2 acc[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u)
      acc[u] = u < n ? reinterpret_cast<const float2 *>(cb + (size_t)u * KVQ_PART_STRIDE + 4)[lane]
                     : make_float2(0.f, 0.f);
    float Mc = ms;
    for (int off = 32; off >= 1; off >>= 1) Mc = __builtin_fmaxf(Mc, __shfl_xor(Mc, off));
    if (Mc == ninf) continue;  // every split of this chunk is empty
    const float Mn = __builtin_fmaxf(M, Mc);
    const float r = (M == ninf) ? 0.f : __builtin_amdgcn_exp2f(M - Mn);  // rescale what came before
    const float w = (ms == ninf) ? 0.f : __builtin_amdgcn_exp2f(ms - Mn);
    float lc = ls * w;
    for (int off = 32; off >= 1; off >>= 1) lc += __shfl_xor(lc, off);
    l = __builtin_fmaf(l, r, lc);
    o0 *= r;
    o1 *= r;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), u));
      o0 = __builtin_fmaf(acc[u].x, wj, o0);
      o1 = __builtin_fmaf(acc[u].y, wj, o1);
    }
    M = Mn;
  }
  if (M != ninf) {
    o0 = o0 / l;
    o1 = o1 / l;
  }
  if (a.value_rotation) {
    // Normalized 128-point Walsh-Hadamard transform of the row (it is its own inverse);
    // lane holds channels 2*lane and 2*lane+1, so channel distance h >= 2 is lane distance h/2.
    const float x = o0, y = o1;
    o0 = x + y;
    o1 = x - y;
    for (int h = 2; h < KVQ_D; h <<= 1) {
      const int pl = h >> 1;
      const float p0 = __shfl_xor(o0, pl), p1 = __shfl_xor(o1, pl);
      const bool upper = (lane & pl) != 0;
      o0 = upper ? p0 - o0 : o0 + p0;
      o1 = upper ? p1 - o1 : o1 + p1;
    }
    o0 *= (float)KVQ_WHT_C;
    o1 *= (float)KVQ_WHT_C;
  }
  if (a.out_f32) {
    reinterpret_cast<float2 *>(a.out)[bh * 64 + lane] = make_float2(o0, o1);
  } else {
    reinterpret_cast<uint32_t *>(a.out)[bh * 64 + lane] = kvq_f32_to_bf16_rne(o0) | (kvq_f32_to_bf16_rne(o1) << 16);
  }
}

}  // namespace

hipError_t kvq_launch_combine(const KvqCombineArgs &a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  (void)hipGetLastError();  // drop a stale error left by an earlier, unrelated call
  hipLaunchKernelGGL(kvq_combine_kernel, dim3((unsigned)((int64_t)a.B * a.Hq)), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t kvq_launch_attention(const KvqAttnArgs &a, int g, int q_parts, hipStream_t s) {
  if (a.cache.batch <= 0) return hipSuccess;
  const int nvg = a.lay.nvg;
  switch (a.lay.kb * 16 + a.lay.vb) {
    case 17: return kvq_attn::launch_k1v1(a, g, q_parts, nvg, s);
    case 18: return kvq_attn::launch_k1v2(a, g, q_parts, nvg, s);
    case 20: return kvq_attn::launch_k1v4(a, g, q_parts, nvg, s);
    case 24: return kvq_attn::launch_k1v8(a, g, q_parts, nvg, s);
    case 33: return kvq_attn::launch_k2v1(a, g, q_parts, nvg, s);
    case 34: return kvq_attn::launch_k2v2(a, g, q_parts, nvg, s);
    case 36: return kvq_attn::launch_k2v4(a, g, q_parts, nvg, s);
    case 40: return kvq_attn::launch_k2v8(a, g, q_parts, nvg, s);
    case 65: return kvq_attn::launch_k4v1(a, g, q_parts, nvg, s);
    case 66: return kvq_attn::launch_k4v2(a, g, q_parts, nvg, s);
    case 68: return kvq_attn::launch_k4v4(a, g, q_parts, nvg, s);
    case 72: return kvq_attn::launch_k4v8(a, g, q_parts, nvg, s);
    case 129: return kvq_attn::launch_k8v1(a, g, q_parts, nvg, s);
    case 130: return kvq_attn::launch_k8v2(a, g, q_parts, nvg, s);
    case 132: return kvq_attn::launch_k8v4(a, g, q_parts, nvg, s);
    case 136: return kvq_attn::launch_k8v8(a, g, q_parts, nvg, s);
  }
  return hipErrorInvalidValue;
}
