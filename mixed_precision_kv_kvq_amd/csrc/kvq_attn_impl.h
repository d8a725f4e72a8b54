// Split-K decode attention over the quantized page store, with dequantization
// fused into MFMA contractions on gfx950.
//
// Computation of nalar.dev "Kuantisasi KV cache mengganggu attention melalui
// key dan value tersimpan", section "Error pada key masuk sebelum softmax":
// s = q K^T / sqrt(d), a = softmax(s), o = a V, for every query head over its
// kv head's stored tokens (quantized pages, then the unquantized recent window
// of section "Pertumbuhan cache mengubah trade pada serving", which also names
// dequantization fused into the attention kernel).
//
// Factorized form used here.  With a key group k_hat = zero + c * scale (codes
// c exact), a group's contribution to q . k_hat is
//     scale * (q . c) + zero * sum(q),
// and with per-token value metadata the output numerator is
//     sum_t (p_t * scale_t) * c_t  +  sum_t p_t * zero_t.
// Both dot products with codes are dense contractions run on
// v_mfma_f32_16x16x32_bf16 with the codes as exact bf16 operands (a code read
// as a bf16 bit pattern is c * 2^-133) and the other operand exact (bf16
// queries) or split into hi + lo bf16 parts (rotated / fp32 queries, and
// always the softmax weights p * scale).  Scale, zero, exponent and max
// bookkeeping stays in fp32 on the VALU.
//
// One 64-lane wave per (sequence, kv head, split); a split is a run of
// 16-token pages.  Per pair of pages (32 tokens):
//   K: 4 MFMAs per page, A = codes (rows = 16 tokens, k = 32 channels of one
//      chunk), B = query matrix whose 16 columns hold the g heads replicated
//      16/g times; replica slots carry different 32-channel chunks (and the hi
//      and lo parts of the query), zero elsewhere, so one accumulator collects
//      per-chunk partial dots that a row-rotation DPP all-reduce sums.
//   V: 8 MFMAs (one per 16-channel tile), A = softmax weights (rows = hi/lo
//      part x head, k = 32 tokens), B = value codes (k = tokens, col = channel).
// Every operand comes from one coalesced load per lane (see kvq_layout.h).
#pragma once
#include "kvq_internal.h"

#ifndef KVQ_WPE
#define KVQ_WPE 4
#endif

namespace kvq_attn {

typedef short bf16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float EXP2_M66 = 0x1p-66f;
constexpr float EXP2_M67 = 0x1p-67f;  // 2^-66 * 2^-67 = 2^-133
constexpr float EXP2_EQ = 0x1p100f;   // query operand scale
constexpr float EXP2_EW = 0x1p100f;   // weight operand scale
constexpr float EXP2_OUT = 0x1p33f;   // 2^(133 - 100): value accumulators back to real units
constexpr float EXP2_WIN_W = 0x1p-33f;

template <int N>
struct Words {
  uint32_t w[N];
};

template <int N>
__device__ __forceinline__ Words<N> load_words(const uint8_t *p) {
  Words<N> r;
  if constexpr (N == 1) {
    r.w[0] = *reinterpret_cast<const uint32_t *>(p);
  } else if constexpr (N == 2) {
    const uint2 v = *reinterpret_cast<const uint2 *>(p);
    r.w[0] = v.x;
    r.w[1] = v.y;
  } else if constexpr (N == 4) {
    const uint4 v = *reinterpret_cast<const uint4 *>(p);
    r.w[0] = v.x;
    r.w[1] = v.y;
    r.w[2] = v.z;
    r.w[3] = v.w;
  } else {
    const uint4 v0 = reinterpret_cast<const uint4 *>(p)[0];
    const uint4 v1 = reinterpret_cast<const uint4 *>(p)[1];
    r.w[0] = v0.x;
    r.w[1] = v0.y;
    r.w[2] = v0.z;
    r.w[3] = v0.w;
    r.w[4] = v1.x;
    r.w[5] = v1.y;
    r.w[6] = v1.z;
    r.w[7] = v1.w;
  }
  return r;
}

template <int N>
__device__ __forceinline__ Words<N> zero_words() {
  Words<N> r;
#pragma unroll
  for (int i = 0; i < N; ++i) r.w[i] = 0;
  return r;
}

__device__ __forceinline__ uint4 load_u4(const uint8_t *p) { return *reinterpret_cast<const uint4 *>(p); }

__device__ __forceinline__ uint32_t u4_get(const uint4 &v, int r) {
  return r == 0 ? v.x : (r == 1 ? v.y : (r == 2 ? v.z : v.w));
}

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ bf16x8 pack8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ uint32_t bf16_rne(float f) { return kvq_f32_to_bf16_rne(f); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

__device__ __forceinline__ float ror_add(float v, int sh) {
  int r;
  switch (sh) {
    case 8: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false); break;
    case 4: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false); break;
    default: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false); break;
  }
  return v + __builtin_bit_cast(float, r);
}

template <int G>
__device__ __forceinline__ float replica_allreduce(float v) {
#pragma unroll
  for (int sh = 8; sh >= G; sh >>= 1) v = ror_add(v, sh);
  return v;
}

// Per-wave running state of the online softmax.
template <int G, int NVG>
struct State {
  f32x4 acc[8];     // value MFMA accumulators (rows = part x head, col = channel)
  float m;          // running max of this lane's head, in score units
  float l;          // this lane's partial sum of p
  float zacc[NVG];  // this lane's partial sum of p * zero_v per value group
  float ow[G][2];   // window contribution for channels 2*lane, 2*lane+1 (real units)
};

template <int KB, int VB, int G, int P, int NVG>
struct Kern {
  static constexpr int REP = 16 / G;                 // replicas of each head in the 16 columns
  static constexpr int X = REP / P;                  // chunk slots per query part
  static constexpr int XE = X < 4 ? X : 4;           // chunk slots in use
  static constexpr int NACC = 4 / XE;                // score accumulators
  static constexpr int PERK = 16 / KB;
  static constexpr uint32_t MASKK = ((1u << KB) - 1u) * 0x00010001u;
  static constexpr uint32_t MASKV = ((1u << VB) - 1u) * 0x00010001u;

  struct Ctx {
    bf16x8 qB[4];    // query operand per 32-channel chunk
    float Qs[NACC];  // sum of this column's query operand per accumulator, x 2^-133
    int kmeta_off[NACC];
    int vmeta_off[NVG];
    int lane, col, quad, rowpart;
    float sig;  // softmax scale in score units (log2 domain)
  };

  // Build the query operand from q (fp32, [G][128] in LDS).
  static __device__ __forceinline__ void build_q(Ctx &cx, const float *qs) {
    const int y = cx.col / G, h = cx.col % G;
    const int part = y / X, x = y % X;
    const bool valid = x < XE;
    float qsum[NACC];
#pragma unroll
    for (int a = 0; a < NACC; ++a) qsum[a] = 0.f;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      uint32_t w[4];
      const bool use = valid && (kc % XE) == x;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t pr = 0;
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          const int ch = 32 * kc + 8 * cx.quad + 2 * i + e2;
          uint32_t bits = 0;
          if (use) {
            const float v = qs[h * KVQ_D + ch] * EXP2_EQ;
            const uint32_t hb = bf16_rne(v);
            if (P == 1 || part == 0) {
              bits = hb;
            } else {
              bits = bf16_rne(v - kvq_bf16_bits_to_f32(hb));
            }
            qsum[kc / XE] += kvq_bf16_bits_to_f32(bits);
          }
          pr |= bits << (16 * e2);
        }
        w[i] = pr;
      }
      cx.qB[kc] = pack8(w[0], w[1], w[2], w[3]);
    }
#pragma unroll
    for (int a = 0; a < NACC; ++a) {
      float s = qsum[a];
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      cx.Qs[a] = s * EXP2_M66 * EXP2_M67;
    }
  }

  static __device__ __forceinline__ void init_meta(Ctx &cx, const KvqLayout &lay) {
    const int y = cx.col / G, x = y % X;
    const bool valid = x < XE;
#pragma unroll
    for (int a = 0; a < NACC; ++a) {
      const int grp = valid ? ((a * XE + x) * 32) / lay.kg : 0;
      cx.kmeta_off[a] = lay.k_meta_off + 16 * (cx.quad * lay.nkg + grp);
    }
#pragma unroll
    for (int v = 0; v < NVG; ++v) cx.vmeta_off[v] = lay.v_meta_off + 16 * (cx.quad * NVG + v);
  }

  struct PageData {
    Words<KB> kc;
    uint4 km[NACC];
    Words<VB> vc;
    uint4 vm[NVG];
  };

  static __device__ __forceinline__ void load_page(PageData &pd, const Ctx &cx, const uint8_t *rec,
                                                   const KvqLayout &lay) {
    pd.kc = load_words<KB>(rec + lay.k_codes_off + cx.lane * 4 * KB);
#pragma unroll
    for (int a = 0; a < NACC; ++a) pd.km[a] = load_u4(rec + cx.kmeta_off[a]);
    pd.vc = load_words<VB>(rec + lay.v_codes_off + cx.lane * 4 * VB);
#pragma unroll
    for (int v = 0; v < NVG; ++v) pd.vm[v] = load_u4(rec + cx.vmeta_off[v]);
  }

  static __device__ __forceinline__ void zero_page(PageData &pd) {
    pd.kc = zero_words<KB>();
    pd.vc = zero_words<VB>();
#pragma unroll
    for (int a = 0; a < NACC; ++a) pd.km[a] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < NVG; ++v) pd.vm[v] = make_uint4(0, 0, 0, 0);
  }

  // Scores of the 16 tokens of one page for this lane's head: s[r] for token 4*quad + r.
  static __device__ __forceinline__ void page_scores(const Ctx &cx, const PageData &pd, float s[4]) {
    f32x4 D[NACC];
#pragma unroll
    for (int a = 0; a < NACC; ++a) D[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int u = 4 * kc + i;
        w[i] = (pd.kc.w[u / PERK] >> (KB * (u % PERK))) & MASKK;
      }
      D[kc / XE] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pack8(w[0], w[1], w[2], w[3]), cx.qB[kc], D[kc / XE], 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int a = 0; a < NACC; ++a) {
        const uint32_t md = u4_get(pd.km[a], r);
        acc = __builtin_fmaf(h2f(md >> 16), cx.Qs[a], acc);
        acc = __builtin_fmaf(D[a][r], h2f(md & 0xFFFF), acc);
      }
      s[r] = replica_allreduce<G>(acc);
    }
  }

  // Online-softmax update with the 8 scores of a page pair; returns p in place.
  template <bool MASKED>
  static __device__ __forceinline__ void softmax_update(const Ctx &cx, State<G, NVG> &st, float s0[4], float s1[4]) {
    float t = s0[0];
#pragma unroll
    for (int r = 1; r < 4; ++r) t = __builtin_fmaxf(t, s0[r]);
#pragma unroll
    for (int r = 0; r < 4; ++r) t = __builtin_fmaxf(t, s1[r]);
    t = __builtin_fmaxf(t, __shfl_xor(t, 16));
    t = __builtin_fmaxf(t, __shfl_xor(t, 32));
    const float mnew = __builtin_fmaxf(st.m, t);
    if (__builtin_amdgcn_ballot_w64(mnew > st.m)) {
      const float alpha = (mnew > st.m) ? __builtin_amdgcn_exp2f(cx.sig * (st.m - mnew)) : 1.0f;
      // st.m == -inf gives alpha = 0 (nothing accumulated yet).
      st.l *= alpha;
#pragma unroll
      for (int v = 0; v < NVG; ++v) st.zacc[v] *= alpha;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * cx.quad + r;
        const float ar = __shfl(alpha, (cx.quad << 4) + (row % G));
#pragma unroll
        for (int m = 0; m < 8; ++m) st.acc[m][r] *= ar;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ah = __shfl(alpha, h);
        st.ow[h][0] *= ah;
        st.ow[h][1] *= ah;
      }
      st.m = mnew;
    }
    const float nb = -cx.sig * st.m;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], cx.sig, nb));
      float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], cx.sig, nb));
      if (MASKED) {
        p0 = (s0[r] == -__builtin_inff()) ? 0.f : p0;
        p1 = (s1[r] == -__builtin_inff()) ? 0.f : p1;
      }
      s0[r] = p0;
      s1[r] = p1;
      st.l += p0 + p1;
    }
  }

  // Weights operand (A of the value MFMA) for value group v from per-token weights.
  static __device__ __forceinline__ bf16x8 weights_operand(const Ctx &cx, const float w0[4], const float w1[4]) {
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a0 = (i < 2) ? w0[2 * i] : w1[2 * i - 4];
      float a1 = (i < 2) ? w0[2 * i + 1] : w1[2 * i - 3];
      if (cx.rowpart == 1) {
        a0 = a0 - kvq_bf16_bits_to_f32(bf16_rne(a0));
        a1 = a1 - kvq_bf16_bits_to_f32(bf16_rne(a1));
      } else if (cx.rowpart > 1) {
        a0 = 0.f;
        a1 = 0.f;
      }
      o[i] = pack_bf16x2(a0, a1);
    }
    return pack8(o[0], o[1], o[2], o[3]);
  }

  // Value contraction of a page pair with probabilities p0 (page A) and p1 (page B).
  template <bool MASKED>
  static __device__ __forceinline__ void pair_values(const Ctx &cx, State<G, NVG> &st, const PageData &A,
                                                     const PageData &B, const float p0[4], const float p1[4],
                                                     int validA, int validB) {
    bf16x8 Aop[NVG];
#pragma unroll
    for (int v = 0; v < NVG; ++v) {
      float w0[4], w1[4];
      float z = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t ma = u4_get(A.vm[v], r), mb = u4_get(B.vm[v], r);
        float za = p0[r] * h2f(ma >> 16), zb = p1[r] * h2f(mb >> 16);
        w0[r] = p0[r] * h2f(ma & 0xFFFF) * EXP2_EW;
        w1[r] = p1[r] * h2f(mb & 0xFFFF) * EXP2_EW;
        if (MASKED) {
          const bool va = 4 * cx.quad + r < validA, vb = 4 * cx.quad + r < validB;
          za = va ? za : 0.f;
          zb = vb ? zb : 0.f;
          w0[r] = va ? w0[r] : 0.f;
          w1[r] = vb ? w1[r] : 0.f;
        }
        z += za + zb;
      }
      st.zacc[v] += z;
      Aop[v] = weights_operand(cx, w0, w1);
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int il = i & 1;
        const int pos = il * 8 * VB + m * VB;
        const uint32_t word = (i < 2) ? A.vc.w[pos >> 4] : B.vc.w[pos >> 4];
        w[i] = (word >> (pos & 15)) & MASKV;
      }
      st.acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Aop[m / (8 / NVG)], pack8(w[0], w[1], w[2], w[3]), st.acc[m], 0, 0, 0);
    }
  }

  template <bool MASKED>
  static __device__ __forceinline__ void process_pair(const Ctx &cx, State<G, NVG> &st, const PageData &A,
                                                      const PageData &B, int validA, int validB) {
    float s0[4], s1[4];
    page_scores(cx, A, s0);
    page_scores(cx, B, s1);
    if (MASKED) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s0[r] = (4 * cx.quad + r < validA) ? s0[r] : -__builtin_inff();
        s1[r] = (4 * cx.quad + r < validB) ? s1[r] : -__builtin_inff();
      }
    }
    softmax_update<MASKED>(cx, st, s0, s1);
    pair_values<MASKED>(cx, st, A, B, s0, s1, validA, validB);
  }

  // Window tokens [w0, w0 + 32) of the ring (valid below wend): scores on MFMA, values on the VALU.
  static __device__ __forceinline__ void window_chunk(const Ctx &cx, State<G, NVG> &st, const uint8_t *kwin,
                                                      const uint8_t *vwin, int kv_f32, int w0, int wend) {
    float s[2][4];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int slot = w0 + 16 * sub + cx.col;  // A-operand row = token
      const bool ok = slot < wend;
      f32x4 D[NACC];
#pragma unroll
      for (int a = 0; a < NACC; ++a) D[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const int ch = 32 * kc + 8 * cx.quad;
        uint32_t hi[4] = {0, 0, 0, 0}, lo[4] = {0, 0, 0, 0};
        if (ok) {
          if (kv_f32) {
            const float *rp = reinterpret_cast<const float *>(kwin) + (size_t)slot * KVQ_D + ch;
            const float4 f0 = reinterpret_cast<const float4 *>(rp)[0];
            const float4 f1 = reinterpret_cast<const float4 *>(rp)[1];
            const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t h0 = bf16_rne(f[2 * i]), h1 = bf16_rne(f[2 * i + 1]);
              hi[i] = h0 | (h1 << 16);
              lo[i] = pack_bf16x2(f[2 * i] - kvq_bf16_bits_to_f32(h0), f[2 * i + 1] - kvq_bf16_bits_to_f32(h1));
            }
          } else {
            const uint4 v = *reinterpret_cast<const uint4 *>(kwin + ((size_t)slot * KVQ_D + ch) * 2);
            hi[0] = v.x;
            hi[1] = v.y;
            hi[2] = v.z;
            hi[3] = v.w;
          }
        }
        D[kc / XE] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pack8(hi[0], hi[1], hi[2], hi[3]), cx.qB[kc], D[kc / XE], 0, 0, 0);
        if (kv_f32)
          D[kc / XE] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pack8(lo[0], lo[1], lo[2], lo[3]), cx.qB[kc], D[kc / XE], 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int a = 0; a < NACC; ++a) acc += D[a][r];
        acc = replica_allreduce<G>(acc * EXP2_M66 * EXP2_M67);
        s[sub][r] = (w0 + 16 * sub + 4 * cx.quad + r < wend) ? acc : -__builtin_inff();
      }
    }
    softmax_update<true>(cx, st, s[0], s[1]);
    // Values: this lane owns channels 2*lane, 2*lane+1; p of (head h, token) lives in lane 16*quad + h.
    const int nval = (wend - w0) < 32 ? (wend - w0) : 32;
    for (int tk = 0; tk < nval; ++tk) {
      const int sub = tk >> 4, tq = (tk & 15) >> 2, r = tk & 3;
      float v0, v1;
      if (kv_f32) {
        const float2 f = reinterpret_cast<const float2 *>(vwin + (size_t)(w0 + tk) * KVQ_D * 4)[cx.lane];
        v0 = f.x;
        v1 = f.y;
      } else {
        const uint32_t u = reinterpret_cast<const uint32_t *>(vwin + (size_t)(w0 + tk) * KVQ_D * 2)[cx.lane];
        v0 = kvq_bf16_bits_to_f32(u & 0xFFFF);
        v1 = kvq_bf16_bits_to_f32(u >> 16);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float pv;
        switch (r) {
          case 0: pv = sub ? s[1][0] : s[0][0]; break;
          case 1: pv = sub ? s[1][1] : s[0][1]; break;
          case 2: pv = sub ? s[1][2] : s[0][2]; break;
          default: pv = sub ? s[1][3] : s[0][3]; break;
        }
        const float p = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pv), 16 * tq + h));
        st.ow[h][0] = __builtin_fmaf(p, v0, st.ow[h][0]);
        st.ow[h][1] = __builtin_fmaf(p, v1, st.ow[h][1]);
      }
    }
  }

  static __device__ void run(const KvqAttnArgs &args, float *lds) {
    const int lane = threadIdx.x;
    const int64_t wave = blockIdx.x;
    const int S = args.splits;
    const int64_t unit = wave / S;
    const int split = (int)(wave % S);
    const int Hkv = args.Hkv;
    const int kvh = (int)(unit % Hkv), b = (int)(unit / Hkv);
    if (b >= args.cache.batch) return;
    const KvqLayout &lay = args.lay;
    const int R = args.R;
    int L = args.seq_lens[b];
    L = L < 0 ? 0 : (L > args.max_len ? args.max_len : L);
    const int nq = L > R ? L - R : 0;
    const int nw = L < R ? L : R;
    const int qpages = (nq + KVQ_PAGE - 1) / KVQ_PAGE;
    const int wpages = (nw + KVQ_PAGE - 1) / KVQ_PAGE;
    const int vp_total = qpages + wpages;
    const int v0 = split * args.pages_per_split;
    int v1 = v0 + args.pages_per_split;
    if (v1 > vp_total) v1 = vp_total;

    Ctx cx;
    cx.lane = lane;
    cx.col = lane & 15;
    cx.quad = lane >> 4;
    cx.rowpart = cx.col / G;
    cx.sig = args.sigma_u;

    // Query of the G heads of this kv head -> LDS (fp32), rotated when keys are.
    float *qraw = lds;               // [G][128]
    float *qrot = lds + G * KVQ_D;   // [G][128]
    const int hq0 = kvh * G;
    for (int i = lane; i < G * KVQ_D; i += 64) {
      const size_t gi = ((size_t)b * args.Hq + hq0) * KVQ_D + i;
      qraw[i] = args.q_f32 ? reinterpret_cast<const float *>(args.q)[gi]
                           : kvq_bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(args.q)[gi]);
    }
    __syncthreads();
    if (args.rotation) {
      for (int i = lane; i < G * KVQ_D; i += 64) qrot[i] = qraw[i];
      __syncthreads();
      for (int hs = 1; hs < KVQ_D; hs <<= 1) {
        for (int pidx = lane; pidx < G * KVQ_D / 2; pidx += 64) {
          const int hh = pidx / (KVQ_D / 2), pp = pidx % (KVQ_D / 2);
          const int i0 = (pp / hs) * 2 * hs + (pp % hs);
          float *row = qrot + hh * KVQ_D;
          const float x0 = row[i0], x1 = row[i0 + hs];
          row[i0] = x0 + x1;
          row[i0 + hs] = x0 - x1;
        }
        __syncthreads();
      }
      for (int i = lane; i < G * KVQ_D; i += 64) qrot[i] *= (float)KVQ_WHT_C;
      __syncthreads();
      build_q(cx, qrot);
    } else {
      build_q(cx, qraw);
    }
    init_meta(cx, lay);

    State<G, NVG> st;
#pragma unroll
    for (int m = 0; m < 8; ++m) st.acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m = -__builtin_inff();
    st.l = 0.f;
#pragma unroll
    for (int v = 0; v < NVG; ++v) st.zacc[v] = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) st.ow[h][0] = st.ow[h][1] = 0.f;

    const int full_pages = nq / KVQ_PAGE;  // pages with all 16 tokens quantized
    const int qend = v1 < qpages ? v1 : qpages;
    auto rec_ptr = [&](int p) -> const uint8_t * {
      const int64_t ri = kvq_record_index(args.cache.paged, args.cache.block_table, args.cache.mbps,
                                          args.cache.pages_per_seq, args.cache.pool_pages, Hkv, b, kvh, p);
      return args.cache.pages + (size_t)ri * lay.record;
    };
    int p = v0;
    // Fast path: pairs of full pages.
    if (p + 1 < qend && p + 1 < full_pages) {
      PageData A, B;
      load_page(A, cx, rec_ptr(p), lay);
      load_page(B, cx, rec_ptr(p + 1), lay);
      while (true) {
        const int pn = p + 2;
        const bool more = (pn + 1 < qend) && (pn + 1 < full_pages);
        PageData An, Bn;
        if (more) {
          load_page(An, cx, rec_ptr(pn), lay);
          load_page(Bn, cx, rec_ptr(pn + 1), lay);
        }
        process_pair<false>(cx, st, A, B, 16, 16);
        p = pn;
        if (!more) break;
        A = An;
        B = Bn;
      }
    }
    // Remaining quantized pages (partial page or an odd page): masked pairs.
    while (p < qend) {
      PageData A, B;
      const int va = (nq - p * KVQ_PAGE) < KVQ_PAGE ? (nq - p * KVQ_PAGE) : KVQ_PAGE;
      load_page(A, cx, rec_ptr(p), lay);
      int vb = 0;
      if (p + 1 < qend) {
        vb = (nq - (p + 1) * KVQ_PAGE) < KVQ_PAGE ? (nq - (p + 1) * KVQ_PAGE) : KVQ_PAGE;
        load_page(B, cx, rec_ptr(p + 1), lay);
      } else {
        zero_page(B);
      }
      process_pair<true>(cx, st, A, B, va, vb);
      p += 2;
    }
    // Window pages of this split.
    const int wv0 = (v0 > qpages ? v0 : qpages) - qpages;
    const int wv1 = v1 - qpages;
    if (wv1 > wv0) {
      if (args.rotation) build_q(cx, qraw);  // window keys are stored unrotated
      const size_t win_off = ((size_t)b * Hkv + kvh) * R * KVQ_D * (args.kv_f32 ? 4 : 2);
      const int wend = (wv1 * KVQ_PAGE) < nw ? wv1 * KVQ_PAGE : nw;
      for (int w = wv0 * KVQ_PAGE; w < wend; w += 32)
        window_chunk(cx, st, args.cache.k_win + win_off, args.cache.v_win + win_off, args.kv_f32, w, wend);
    }

    // ---- reduce and write this split's partial result -------------------------
    float l = st.l;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    float z[NVG];
#pragma unroll
    for (int v = 0; v < NVG; ++v) {
      z[v] = st.zacc[v];
      z[v] += __shfl_xor(z[v], 16);
      z[v] += __shfl_xor(z[v], 32);
    }
    __syncthreads();
    float *accs = lds;                   // [2G][128]
    float *hdr = lds + 2 * G * KVQ_D;    // [G][4]: m, l, z0, z1
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * cx.quad + r;
        if (row < 2 * G) accs[row * KVQ_D + 16 * m + cx.col] = st.acc[m][r];
      }
    }
    if (lane < G) {
      hdr[lane * 4 + 0] = st.m * cx.sig;  // log2 units
      hdr[lane * 4 + 1] = l;
#pragma unroll
      for (int v = 0; v < NVG; ++v) hdr[lane * 4 + 2 + v] = z[v];
    }
    __syncthreads();
    const int vshift = (NVG == 1) ? 7 : 6;  // channel -> value group
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float *dst = args.partials + (((size_t)b * args.Hq + hq0 + h) * S + split) * KVQ_PART_STRIDE;
      float o[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int c = 2 * lane + e;
        const float a = accs[h * KVQ_D + c] + accs[(G + h) * KVQ_D + c];
        o[e] = __builtin_fmaf(a, EXP2_OUT, hdr[h * 4 + 2 + (c >> vshift)]) + st.ow[h][e];
      }
      reinterpret_cast<float2 *>(dst + 4)[lane] = make_float2(o[0], o[1]);
      if (lane == 0) {
        dst[0] = hdr[h * 4 + 0];
        dst[1] = hdr[h * 4 + 1];
        dst[2] = 0.f;
        dst[3] = 0.f;
      }
    }
  }
};

template <int KB, int VB, int G, int P, int NVG>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(KVQ_WPE))) void kvq_attn_split_kernel(KvqAttnArgs args) {
  __shared__ float lds[2 * 8 * KVQ_D + 8 * 4];
  Kern<KB, VB, G, P, NVG>::run(args, lds);
}

}  // namespace kvq_attn
