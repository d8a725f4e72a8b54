// Cross-split combine of flash-decoding partials and dispatch of the split kernel.
//
// Each split s of a (sequence, query head) holds its own max m_s (log2 units),
// sum l_s of 2^(score - m_s) and unnormalized output acc_s.  With M = max m_s the
// softmax of nalar.dev "Kuantisasi KV cache mengganggu attention melalui key dan
// value tersimpan", section "Error pada key masuk sebelum softmax", is
//   o = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
#include "kvq_internal.h"

namespace kvq_attn {
// Every (key bits, value bits) pair of widths 1..6 and 8 (kvq_attn_inst.hip compiled once per pair).
#define KVQ_FOR_VBITS(X, kb) X(kb, 1) X(kb, 2) X(kb, 3) X(kb, 4) X(kb, 5) X(kb, 6) X(kb, 8)
#define KVQ_FOR_ALL_BITS(X)                                                                             \
  KVQ_FOR_VBITS(X, 1) KVQ_FOR_VBITS(X, 2) KVQ_FOR_VBITS(X, 3) KVQ_FOR_VBITS(X, 4) KVQ_FOR_VBITS(X, 5) \
  KVQ_FOR_VBITS(X, 6) KVQ_FOR_VBITS(X, 8)
#define KVQ_DECLARE_LAUNCH(kb, vb) \
  hipError_t launch_k##kb##v##vb(const KvqAttnArgs &a, int g, int p, int nvg, hipStream_t s);
KVQ_FOR_ALL_BITS(KVQ_DECLARE_LAUNCH)
#undef KVQ_DECLARE_LAUNCH
}  // namespace kvq_attn

namespace {

// One wave per (sequence, query head).  Entries are taken 64 at a time (lane s holds entry s's
// header), accumulator rows in halves of 32.  Every written header holds the number n of entries
// of its row that hold splits; entries from n on are never written.  The first group reads the
// headers and rows of its first `eager` entries together (the equal share of the launch: with equal
// lengths every row has exactly that many entries, all just written and cache-resident), so such a
// row costs one memory round trip and touches no unwritten line; headers of entries [eager, n) and
// rows of later live entries are read once n and the headers are known.  An empty split has
// m = -inf and is not accumulated (rows read for unwritten or empty entries are skipped, not
// multiplied by 0).  Groups are merged online (running max M, sum l and output o rescaled as M
// grows).
constexpr int kHalf = 32;

__global__ __launch_bounds__(64) void kvq_combine_kernel(KvqCombineArgs a) {
  const int lane = threadIdx.x;
  const size_t bh = blockIdx.x;
  const float *base = a.partials + bh * (size_t)a.splits * KVQ_PART_STRIDE;
  const float ninf = -__builtin_inff();
  auto header = [&](int e) { return *reinterpret_cast<const float4 *>(base + (size_t)e * KVQ_PART_STRIDE); };
  float M = ninf, l = 0.f, o0 = 0.f, o1 = 0.f;
  // first group: headers and rows of the eager entries
  int eager = a.eager < a.splits ? a.eager : a.splits;
  eager = eager < 1 ? 1 : (eager > 2 * kHalf ? 2 * kHalf : eager);
  float4 hd = lane < eager ? header(lane) : make_float4(ninf, 0.f, 0.f, 0.f);
  float2 acc[kHalf];
#pragma unroll
  for (int u = 0; u < kHalf; ++u)
    acc[u] = u < eager ? reinterpret_cast<const float2 *>(base + (size_t)u * KVQ_PART_STRIDE + 4)[lane]
                       : make_float2(0.f, 0.f);
  int nrow;
  {
    const int c = (int)__builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, hd.z)));
    nrow = c < 1 ? 1 : (c < a.splits ? c : a.splits);
  }
  for (int s0 = 0; s0 < nrow; s0 += 2 * kHalf) {
    const int n = (nrow - s0) < 2 * kHalf ? (nrow - s0) : 2 * kHalf;
    const int pre = s0 == 0 ? (eager < n ? eager : n) : 0;  // entries whose header (and row, below 32) is read
    if (pre < n) {
      const float4 h2 = (lane >= pre && lane < n) ? header(s0 + lane) : make_float4(ninf, 0.f, 0.f, 0.f);
      if (lane >= pre) hd = h2;
    }
    const float ms = lane < n ? hd.x : ninf;
    const float ls = lane < n ? hd.y : 0.f;
    const uint64_t live = __ballot(ms != ninf);
    if (live) {
      float Mc = ms;
      for (int off = 32; off >= 1; off >>= 1) Mc = __builtin_fmaxf(Mc, __shfl_xor(Mc, off));
      const float Mn = __builtin_fmaxf(M, Mc);
      const float r = (M == ninf) ? 0.f : __builtin_amdgcn_exp2f(M - Mn);  // rescale what came before
      const float w = (ms == ninf) ? 0.f : __builtin_amdgcn_exp2f(ms - Mn);
      float lc = ls * w;
      for (int off = 32; off >= 1; off >>= 1) lc += __shfl_xor(lc, off);
      l = __builtin_fmaf(l, r, lc);
      o0 *= r;
      o1 *= r;
      const float *cb = base + (size_t)s0 * KVQ_PART_STRIDE;
      for (int hf = 0; hf < 2; ++hf) {
        const uint32_t hmask = (uint32_t)(live >> (kHalf * hf));
        if (!hmask) continue;
        const int got = hf == 0 ? (pre < kHalf ? pre : kHalf) : 0;  // rows already read
        const uint32_t late = got >= kHalf ? 0u : hmask & ~((1u << got) - 1u);
        const float *hb = cb + (size_t)(kHalf * hf) * KVQ_PART_STRIDE;
#pragma unroll
        for (int u = 0; u < kHalf; ++u)
          if ((late >> u) & 1) acc[u] = reinterpret_cast<const float2 *>(hb + (size_t)u * KVQ_PART_STRIDE + 4)[lane];
#pragma unroll
        for (int u = 0; u < kHalf; ++u) {
          if (!((hmask >> u) & 1)) continue;  // wave-uniform
          const float wj =
              __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), kHalf * hf + u));
          o0 = __builtin_fmaf(acc[u].x, wj, o0);
          o1 = __builtin_fmaf(acc[u].y, wj, o1);
        }
      }
      M = Mn;
    }
    hd = make_float4(ninf, 0.f, 0.f, 0.f);
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
#define KVQ_LAUNCH_CASE(kb, vb) \
  case kb * 16 + vb:            \
    return kvq_attn::launch_k##kb##v##vb(a, g, q_parts, nvg, s);
    KVQ_FOR_ALL_BITS(KVQ_LAUNCH_CASE)
#undef KVQ_LAUNCH_CASE
  }
  return hipErrorInvalidValue;
}
