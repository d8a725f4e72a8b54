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
// One 64-lane wave per (sequence, kv head, split).  A quantized split takes every
// S_q-th pair of 16-token pages of its sequence and kv head (the page records are
// streamed into an LDS ring, see stream_pairs); a window split takes 128 tokens of
// the recent window.  Per pair of pages (32 tokens):
//   K: 4 MFMAs per page, A = codes (rows = 16 tokens, k = 32 channels of one
//      chunk), B = query matrix whose 16 columns hold the g heads replicated
//      16/g times; replica slots carry different 32-channel chunks (and the hi
//      and lo parts of the query), zero elsewhere, so one accumulator collects
//      per-chunk partial dots that a row-rotation DPP all-reduce sums.
//   V: 8 MFMAs (one per 16-channel tile), A = softmax weights (rows = hi/lo
//      part x head, k = 32 tokens), B = value codes (k = tokens, col = channel).
// Every operand comes from one 4- to 16-byte read per lane of the page record (see
// kvq_layout.h for the order of the record's words).
#pragma once
#include "kvq_internal.h"

namespace kvq_attn {

typedef short bf16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float EXP2_M66 = 0x1p-66f;
constexpr float EXP2_M67 = 0x1p-67f;  // 2^-66 * 2^-67 = 2^-133
constexpr float EXP2_EQ = 0x1p100f;  // query operand scale
// Softmax weights are carried as p * 2^64 (l, the zero-point sums, the value
// accumulators and the window sums all share that factor, which cancels in the
// final normalization).  Value MFMA products are (p 2^64 scale)(c 2^s 2^-133)
// for tile scale s, so an accumulator D is brought to the common scale by
// 2^(133 - s) = 2^69 * 2^(64 - s), applied as two exact multiplies.
constexpr float P_BIAS_LOG2 = 64.0f;
constexpr float EXP2_OUT = 0x1p69f;

// Position of a b-bit field within a 16-bit half when extracted without a full
// shift: fields whose bits end inside the low byte are read in place (a bf16
// bit pattern x in the low byte is the value x * 2^-133, so a field at bit s
// reads as code * 2^s); higher fields are first shifted down by 8.
template <int B>
__device__ __forceinline__ constexpr int field_scale_log2(int bit) {
  return (bit + B <= 8) ? bit : bit - 8;
}
// Extract the field of both 16-bit halves at `bit` as a bf16 pair, scaled by 2^field_scale_log2.
template <int B>
__device__ __forceinline__ uint32_t field_pair(uint32_t word, uint32_t word_sh8, int bit) {
  constexpr uint32_t m = ((1u << B) - 1u) * 0x00010001u;
  return (bit + B <= 8) ? (word & (m << bit)) : (word_sh8 & (m << (bit - 8)));
}

template <int N>
struct Words {
  uint32_t w[N];
};

#define KVQ_GLOBAL __attribute__((address_space(1)))

// Loads through global-address-space pointers (global_load_*, not flat_load_*).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2e __attribute__((ext_vector_type(2)));
typedef float f32x4e __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T gload(const void *p) {
  return *(const KVQ_GLOBAL T *)(p);
}

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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t bf16_rne(float f) { return pack_bf16x2(f, 0.f) & 0xFFFFu; }

__device__ __forceinline__ float bf16lo_f32(uint32_t pair) { return __builtin_bit_cast(float, pair << 16); }
__device__ __forceinline__ float bf16hi_f32(uint32_t pair) { return __builtin_bit_cast(float, pair & 0xFFFF0000u); }

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

// Reductions over the four 16-lane rows of the wave (lanes l, l^16, l^32, l^48)
// with v_permlane16_swap / v_permlane32_swap: swapping a value with itself
// leaves the xor-16 (xor-32) partner pair in the two results.
__device__ __forceinline__ float rows_max(float v) {
  const int b = __builtin_bit_cast(int, v);
  auto p16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  v = __builtin_fmaxf(__builtin_bit_cast(float, (int)p16[0]), __builtin_bit_cast(float, (int)p16[1]));
  const int c = __builtin_bit_cast(int, v);
  auto p32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return __builtin_fmaxf(__builtin_bit_cast(float, (int)p32[0]), __builtin_bit_cast(float, (int)p32[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  const int b = __builtin_bit_cast(int, v);
  auto p16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  v = __builtin_bit_cast(float, (int)p16[0]) + __builtin_bit_cast(float, (int)p16[1]);
  const int c = __builtin_bit_cast(int, v);
  auto p32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return __builtin_bit_cast(float, (int)p32[0]) + __builtin_bit_cast(float, (int)p32[1]);
}

template <int G>
__device__ __forceinline__ float replica_allreduce(float v) {
#pragma unroll
  for (int sh = 8; sh >= G; sh >>= 1) v = ror_add(v, sh);
  return v;
}

// ---------------------------------------------------------------------------
// Page prefetch ring in LDS.  In the steady-state loop every page record is
// copied verbatim into a per-wave LDS slot with direct-to-LDS loads
// (buffer_load_dwordx4 ... lds: lane l writes 16 bytes at slot + 16*l), a few page
// pairs ahead of use, and read back with ds_read when processed.  In-flight
// data therefore never occupies a VGPR.  The waits are explicit: vmcnt counts
// vector-memory operations in issue order, so after N newer loads,
// s_waitcnt vmcnt(N) means every older load has landed in LDS.  Every DMA
// instruction has active lanes (lanes past the end of a shorter record re-read an
// in-range chunk into the slot's padding; only lanes past the slot itself are
// idle), so each one is counted, and no other vector-memory load is issued inside
// that loop.
// ---------------------------------------------------------------------------
template <int CNT>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CNT) : "memory");
}

typedef __attribute__((address_space(3))) void *lds_vptr;

template <int N>
struct RawWords;
template <>
struct RawWords<1> {
  uint32_t v;
  __device__ __forceinline__ uint32_t w(int) const { return v; }
};
template <>
struct RawWords<2> {
  u32x2 v;
  __device__ __forceinline__ uint32_t w(int i) const { return v[i]; }
};
template <>
struct RawWords<4> {
  u32x4 v;
  __device__ __forceinline__ uint32_t w(int i) const { return v[i]; }
};
template <>
struct RawWords<8> {
  u32x4 a, b;
  __device__ __forceinline__ uint32_t w(int i) const { return i < 4 ? a[i] : b[i - 4]; }
};

// Per-wave running state of the online softmax.
template <int NVG>
struct State {
  f32x4 acc[8];     // value MFMA accumulators (rows = part x head, col = channel)
  float m;          // running max of this lane's head, in score units
  float l;          // this lane's partial sum of p
  float zacc[NVG];  // this lane's partial sum of p * zero_v per value group
};

template <int KB, int VB, int G, int P, int NVG>
struct Kern {
  static constexpr int REP = 16 / G;        // replicas of each head in the 16 columns
  static constexpr int X = REP / P;         // chunk slots per query part
  static constexpr int XE = X < 4 ? X : 4;  // chunk slots in use
  static constexpr int NACC = 4 / XE;       // score accumulators
  static constexpr int PERK = 16 / KB;
  static constexpr uint32_t MASKK = ((1u << KB) - 1u) * 0x00010001u;
  static constexpr uint32_t MASKV = ((1u << VB) - 1u) * 0x00010001u;

  struct Ctx {
    bf16x8 qB[4];    // query operand per 32-channel chunk
    float Qs[NACC];  // sum of this column's query operand per accumulator, x 2^-133
    int kmeta_off[NACC];
    int vmeta_off[NVG];
    int lane, col, quad;
    float sig;     // softmax scale in score units (log2 domain)
    float tau;     // lazy-max margin in score units (16 in log2 units)
    float sel_lo;  // 1 for rows that carry the low bf16 part of the weights
  };

  // Scale (log2) at which the key codes of chunk kc, pair slot i are read (see field_pair).
  static __device__ __forceinline__ constexpr int kslot_scale(int kc, int i) {
    return field_scale_log2<KB>(KB * ((4 * kc + i) % PERK));
  }

  // Build the query operand from q (fp32, [G][128] in LDS).  For code operands
  // (code_scaled), entries of slots whose codes are read scaled by 2^k are
  // divided by 2^k (exact); raw window keys need the unscaled operand.
  static __device__ __forceinline__ void build_q(Ctx &cx, const float *qs, bool code_scaled = true) {
    const int h = cx.col % G;
    build_q_with(cx, [&](int, int, int ch) { return qs[h * KVQ_D + ch]; }, code_scaled);
  }

  // This lane's query channels 32 kc + 8 quad + j (j < 8, all four kc) of its head, straight
  // from global memory: 16-byte loads, fp32 or bf16 as stored.
  struct QRegs {
    u32x4 v[4][2];
  };
  static __device__ __forceinline__ void load_q_regs(QRegs &qr, const KvqAttnArgs &args, const Ctx &cx, int b,
                                                     int hq0) {
    const uint8_t *row =
        (const uint8_t *)args.q + ((size_t)b * args.Hq + hq0 + cx.col % G) * KVQ_D * (args.q_f32 ? 4 : 2);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int ch = 32 * kc + 8 * cx.quad;
      if (args.q_f32) {
        qr.v[kc][0] = gload<u32x4>(row + 4 * ch);
        qr.v[kc][1] = gload<u32x4>(row + 4 * ch + 16);
      } else {
        qr.v[kc][0] = gload<u32x4>(row + 2 * ch);
      }
    }
  }
  static __device__ __forceinline__ void build_q_regs(Ctx &cx, const QRegs &qr, bool q_f32) {
    build_q_with(
        cx,
        [&](int kc, int j, int) {
          // (copy the vector element out first: a bit cast of the element lvalue itself
          // reads the vector's first element)
          const uint32_t u = qr.v[kc][j >> 2][j & 3];
          if (q_f32) return __builtin_bit_cast(float, u);
          const uint32_t w = qr.v[kc][0][j >> 1];
          return kvq_bf16_bits_to_f32((j & 1) ? (w >> 16) : (w & 0xFFFF));
        },
        true);
  }

  // Shared body: getq(kc, j, ch) returns this lane's head's query (fp32) at channel
  // ch = 32 kc + 8 quad + j.
  template <class GetQ>
  static __device__ __forceinline__ void build_q_with(Ctx &cx, GetQ getq, bool code_scaled) {
    const int y = cx.col / G;
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
        const int ch = 32 * kc + 8 * cx.quad + 2 * i;
        const float v0 = use ? getq(kc, 2 * i, ch) * EXP2_EQ : 0.f;
        const float v1 = use ? getq(kc, 2 * i + 1, ch + 1) * EXP2_EQ : 0.f;
        uint32_t pr = pack_bf16x2(v0, v1);
        if (P == 2) {
          const uint32_t lo = pack_bf16x2(v0 - bf16lo_f32(pr), v1 - bf16hi_f32(pr));
          pr = part ? lo : pr;
        }
        const float e0 = bf16lo_f32(pr), e1 = bf16hi_f32(pr);
        qsum[kc / XE] += e0 + e1;
        const float f = code_scaled ? __builtin_amdgcn_ldexpf(1.0f, -kslot_scale(kc, i)) : 1.0f;
        w[i] = pack_bf16x2(e0 * f, e1 * f);  // exact: power-of-two scaling of bf16 values
      }
      cx.qB[kc] = pack8(w[0], w[1], w[2], w[3]);
    }
#pragma unroll
    for (int a = 0; a < NACC; ++a) {
      cx.Qs[a] = rows_sum(qsum[a]) * EXP2_M66 * EXP2_M67;
    }
  }

  static __device__ __forceinline__ void init_ctx(Ctx &cx, const KvqLayout &lay, float sig) {
    cx.lane = threadIdx.x;
    cx.col = cx.lane & 15;
    cx.quad = cx.lane >> 4;
    cx.sig = sig;
    cx.tau = 16.0f / sig;
    const int rowpart = cx.col / G;  // A-operand row of the value MFMA: 0 = hi, 1 = lo, else unused
    cx.sel_lo = rowpart == 1 ? 1.f : 0.f;
    const int x = (cx.col / G) % X;
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

  // Key codes of chunk kc of one page as the A operand (slot scales per kslot_scale).
  static __device__ __forceinline__ bf16x8 key_operand(const PageData &pd, int kc) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = 4 * kc + i;
      const uint32_t word = pd.kc.w[u / PERK];
      w[i] = field_pair<KB>(word, word >> 8, KB * (u % PERK));
    }
    return pack8(w[0], w[1], w[2], w[3]);
  }

  static __device__ __forceinline__ float score_epilogue(const Ctx &cx, const PageData &pd, const f32x4 *D, int r) {
    float acc = 0.f;
#pragma unroll
    for (int a = 0; a < NACC; ++a) {
      const uint32_t md = u4_get(pd.km[a], r);
      acc = __builtin_fmaf(h2f(md >> 16), cx.Qs[a], acc);
      acc = __builtin_fmaf(D[a][r], h2f(md & 0xFFFF), acc);
    }
    return replica_allreduce<G>(acc);
  }

  // Scores of the 32 tokens of a page pair for this lane's head: s0[r] / s1[r] for token 4*quad + r.
  static __device__ __forceinline__ void pair_scores(const Ctx &cx, const PageData &A, const PageData &B,
                                                     float s0[4], float s1[4]) {
    f32x4 DA[NACC], DB[NACC];
#pragma unroll
    for (int a = 0; a < NACC; ++a) {
      DA[a] = f32x4{0.f, 0.f, 0.f, 0.f};
      DB[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      DA[kc / XE] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(key_operand(A, kc), cx.qB[kc], DA[kc / XE], 0, 0, 0);
      DB[kc / XE] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(key_operand(B, kc), cx.qB[kc], DB[kc / XE], 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s0[r] = score_epilogue(cx, A, DA, r);
      s1[r] = score_epilogue(cx, B, DB, r);
    }
  }

  // Online-softmax update with the 8 scores of a page pair; returns p * 2^64 in place.
  // Lazy running max: weights are formed against the running max m, which is
  // only raised (with the cross-lane tile max and a rescale of everything
  // accumulated so far) when some lane sees a score more than 16 (log2 units)
  // above it, so weights stay below 2^(64+16).  m is always the same in every
  // lane that holds a given head.
  template <bool MASKED, bool WIN>
  static __device__ __forceinline__ void softmax_update(const Ctx &cx, State<NVG> &st, float s0[4], float s1[4],
                                                        float (*ow)[2]) {
    float t = __builtin_fmaxf(__builtin_fmaxf(s0[0], s0[1]), __builtin_fmaxf(s0[2], s0[3]));
    t = __builtin_fmaxf(t, __builtin_fmaxf(__builtin_fmaxf(s1[0], s1[1]), __builtin_fmaxf(s1[2], s1[3])));
    if (__builtin_amdgcn_ballot_w64(t > st.m + cx.tau)) {
      t = rows_max(t);  // tile max of this lane's head
      const float mnew = __builtin_fmaxf(st.m, t);
      // st.m == -inf gives alpha = 0 (nothing accumulated yet).
      const float alpha = (mnew > st.m) ? __builtin_amdgcn_exp2f(cx.sig * (st.m - mnew)) : 1.0f;
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
      if constexpr (WIN) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float ah = __shfl(alpha, h);
          ow[h][0] *= ah;
          ow[h][1] *= ah;
        }
      }
      st.m = mnew;
    }
    const float nb = __builtin_fmaf(-cx.sig, st.m, P_BIAS_LOG2);
    float lsum = 0.f;
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
      lsum += p0 + p1;
    }
    st.l += lsum;
  }

  // Weights operand (A of the value MFMA): rows 0..G-1 carry bf16(w), rows G..2G-1 bf16(w - bf16(w));
  // rows 2G.. (unused) carry bf16(w) too, which only reaches accumulator rows that are never read.
  static __device__ __forceinline__ bf16x8 weights_operand(const Ctx &cx, const float w0[4], const float w1[4]) {
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a0 = (i < 2) ? w0[2 * i] : w1[2 * i - 4];
      const float a1 = (i < 2) ? w0[2 * i + 1] : w1[2 * i - 3];
      const uint32_t hp = pack_bf16x2(a0, a1);
      o[i] = pack_bf16x2(__builtin_fmaf(-cx.sel_lo, bf16lo_f32(hp), a0),
                         __builtin_fmaf(-cx.sel_lo, bf16hi_f32(hp), a1));
    }
    return pack8(o[0], o[1], o[2], o[3]);
  }

  // Scale (log2) at which the value codes of tile m are read (independent of the pair slot).
  static __device__ __forceinline__ constexpr int vtile_scale(int m) { return field_scale_log2<VB>((m * VB) & 15); }

  // Value contraction of a page pair with weights p0 (page A) and p1 (page B), both carried as p * 2^64.
  template <bool MASKED>
  static __device__ __forceinline__ void pair_values(const Ctx &cx, State<NVG> &st, const PageData &A,
                                                     const PageData &B, const float p0[4], const float p1[4],
                                                     int validA, int validB) {
    bf16x8 Aop[NVG];
#pragma unroll
    for (int v = 0; v < NVG; ++v) {
      float w0[4], w1[4];
      float z = st.zacc[v];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t ma = u4_get(A.vm[v], r), mb = u4_get(B.vm[v], r);
        float sa = h2f(ma & 0xFFFF), za = h2f(ma >> 16), sb = h2f(mb & 0xFFFF), zb = h2f(mb >> 16);
        if (MASKED) {  // metadata of invalid tokens may be anything, keep it out
          const bool va = 4 * cx.quad + r < validA, vb = 4 * cx.quad + r < validB;
          sa = va ? sa : 0.f;
          za = va ? za : 0.f;
          sb = vb ? sb : 0.f;
          zb = vb ? zb : 0.f;
        }
        w0[r] = __builtin_fmaf(p0[r], sa, 0.f);
        w1[r] = __builtin_fmaf(p1[r], sb, 0.f);
        z = __builtin_fmaf(p0[r], za, z);
        z = __builtin_fmaf(p1[r], zb, z);
      }
      st.zacc[v] = z;
      Aop[v] = weights_operand(cx, w0, w1);
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = (i & 1) * 8 * VB + m * VB;
        const uint32_t word = (i < 2) ? A.vc.w[pos >> 4] : B.vc.w[pos >> 4];
        w[i] = field_pair<VB>(word, word >> 8, pos & 15);
      }
      st.acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Aop[m / (8 / NVG)], pack8(w[0], w[1], w[2], w[3]), st.acc[m], 0, 0, 0);
    }
  }

  // ---- LDS ring -------------------------------------------------------------
  static constexpr int MAX_REC16 = kvq_rec16(KB, VB, NVG);  // record in 16-byte units (k_group 32)
  static constexpr int REC_BYTES = 16 * MAX_REC16;              // ring slot stride
  static constexpr int DMAS_PER_PAGE = (MAX_REC16 + 63) / 64;
  static constexpr int WPE = kvq_attn_wpe(KB, VB, G, P, NVG);       // waves per SIMD
  static constexpr int NPS = kvq_ring_pages(REC_BYTES, WPE);   // page slots
  static constexpr int AHEAD = NPS - 2;                         // pages in flight while a pair is processed
  static constexpr int LDS_BYTES = kvq_attn_lds_bytes(KB, VB, NVG, WPE);
  static_assert(LDS_BYTES >= NPS * REC_BYTES && LDS_BYTES >= KVQ_STAGE_BYTES, "LDS sizing");
  static_assert(AHEAD * DMAS_PER_PAGE <= 63, "vmcnt range");

  // Copy one page record into an LDS slot: DMAS_PER_PAGE wave-wide DMAs, lane l of DMA k writing
  // slot chunk 64k + l, through a buffer resource spanning just the record (scalar base and size),
  // with 32-bit lane offsets (16-byte chunks, clamped into the record) and the slot given as an
  // LDS byte address (base: the low 32 bits of the slot's shared-aperture address); lanes past
  // the slot stay idle.  The resource's range check also keeps every lane inside the record.
  static __device__ __forceinline__ void dma_page_buf(uint32_t slot_lds, const uint8_t *rec, int rec_bytes,
                                                      const uint32_t (&loff)[DMAS_PER_PAGE], int lane) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)rec, 0, rec_bytes, 0x00020000);
#pragma unroll
    for (int k = 0; k < DMAS_PER_PAGE; ++k) {
      if (k + 1 < DMAS_PER_PAGE || lane < MAX_REC16 - 64 * k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_vptr)(size_t)(slot_lds + 1024u * k), 16, loff[k], 0, 0, 0);
    }
  }

  // Read one page of a ring slot.  The reads are inline asm: the compiler cannot
  // tell that they do not alias the ring's in-flight DMAs and would otherwise
  // drain every outstanding load before them.  A single lgkmcnt(0) wait ties
  // every read result, and nothing touches a result before that wait.
  template <int N>
  static __device__ __forceinline__ void ds_read_words(RawWords<N> &d, uint32_t addr) {
    if constexpr (N == 1) {
      asm volatile("ds_read_b32 %0, %1" : "=v"(d.v) : "v"(addr));
    } else if constexpr (N == 2) {
      asm volatile("ds_read_b64 %0, %1" : "=v"(d.v) : "v"(addr));
    } else if constexpr (N == 4) {
      asm volatile("ds_read_b128 %0, %1" : "=v"(d.v) : "v"(addr));
    } else {
      asm volatile("ds_read_b128 %0, %1" : "=v"(d.a) : "v"(addr));
      asm volatile("ds_read_b128 %0, %1 offset:16" : "=v"(d.b) : "v"(addr));
    }
  }

  static __device__ __forceinline__ void read_page_at(PageData &pd, const Ctx &cx, uint32_t base,
                                                      const KvqLayout &lay) {
    RawWords<KB> rk;
    RawWords<VB> rv;
    u32x4 km[NACC], vm[NVG];
    ds_read_words(rk, base + lay.k_codes_off + cx.lane * 4 * KB);
#pragma unroll
    for (int a = 0; a < NACC; ++a) {
      const uint32_t addr = base + cx.kmeta_off[a];
      asm volatile("ds_read_b128 %0, %1" : "=v"(km[a]) : "v"(addr));
    }
    ds_read_words(rv, base + lay.v_codes_off + cx.lane * 4 * VB);
#pragma unroll
    for (int v = 0; v < NVG; ++v) {
      const uint32_t addr = base + cx.vmeta_off[v];
      asm volatile("ds_read_b128 %0, %1" : "=v"(vm[v]) : "v"(addr));
    }
    if constexpr ((KB == 8) == false && (VB == 8) == false && NACC == 1 && NVG == 1)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.v), "+v"(km[0]), "+v"(rv.v), "+v"(vm[0])::"memory");
    if constexpr ((KB == 8) == false && (VB == 8) == false && NACC == 1 && NVG == 2)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.v), "+v"(km[0]), "+v"(rv.v), "+v"(vm[0]), "+v"(vm[1])::"memory");
    if constexpr ((KB == 8) == false && (VB == 8) == false && NACC == 2 && NVG == 1)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.v), "+v"(km[0]), "+v"(km[1]), "+v"(rv.v), "+v"(vm[0])::"memory");
    if constexpr ((KB == 8) == false && (VB == 8) == false && NACC == 2 && NVG == 2)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.v), "+v"(km[0]), "+v"(km[1]), "+v"(rv.v), "+v"(vm[0]), "+v"(vm[1])::"memory");
    if constexpr ((KB == 8) == false && (VB == 8) == false && NACC == 4 && NVG == 1)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.v), "+v"(km[0]), "+v"(km[1]), "+v"(km[2]), "+v"(km[3]), "+v"(rv.v), "+v"(vm[0])::"memory");
    if constexpr ((KB == 8) == false && (VB == 8) == false && NACC == 4 && NVG == 2)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.v), "+v"(km[0]), "+v"(km[1]), "+v"(km[2]), "+v"(km[3]), "+v"(rv.v), "+v"(vm[0]), "+v"(vm[1])::"memory");
    if constexpr ((KB == 8) == false && (VB == 8) == true && NACC == 1 && NVG == 1)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.v), "+v"(km[0]), "+v"(rv.a), "+v"(rv.b), "+v"(vm[0])::"memory");
    if constexpr ((KB == 8) == false && (VB == 8) == true && NACC == 1 && NVG == 2)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.v), "+v"(km[0]), "+v"(rv.a), "+v"(rv.b), "+v"(vm[0]), "+v"(vm[1])::"memory");
    if constexpr ((KB == 8) == false && (VB == 8) == true && NACC == 2 && NVG == 1)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.v), "+v"(km[0]), "+v"(km[1]), "+v"(rv.a), "+v"(rv.b), "+v"(vm[0])::"memory");
    if constexpr ((KB == 8) == false && (VB == 8) == true && NACC == 2 && NVG == 2)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.v), "+v"(km[0]), "+v"(km[1]), "+v"(rv.a), "+v"(rv.b), "+v"(vm[0]), "+v"(vm[1])::"memory");
    if constexpr ((KB == 8) == false && (VB == 8) == true && NACC == 4 && NVG == 1)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.v), "+v"(km[0]), "+v"(km[1]), "+v"(km[2]), "+v"(km[3]), "+v"(rv.a), "+v"(rv.b), "+v"(vm[0])::"memory");
    if constexpr ((KB == 8) == false && (VB == 8) == true && NACC == 4 && NVG == 2)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.v), "+v"(km[0]), "+v"(km[1]), "+v"(km[2]), "+v"(km[3]), "+v"(rv.a), "+v"(rv.b), "+v"(vm[0]), "+v"(vm[1])::"memory");
    if constexpr ((KB == 8) == true && (VB == 8) == false && NACC == 1 && NVG == 1)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.a), "+v"(rk.b), "+v"(km[0]), "+v"(rv.v), "+v"(vm[0])::"memory");
    if constexpr ((KB == 8) == true && (VB == 8) == false && NACC == 1 && NVG == 2)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.a), "+v"(rk.b), "+v"(km[0]), "+v"(rv.v), "+v"(vm[0]), "+v"(vm[1])::"memory");
    if constexpr ((KB == 8) == true && (VB == 8) == false && NACC == 2 && NVG == 1)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.a), "+v"(rk.b), "+v"(km[0]), "+v"(km[1]), "+v"(rv.v), "+v"(vm[0])::"memory");
    if constexpr ((KB == 8) == true && (VB == 8) == false && NACC == 2 && NVG == 2)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.a), "+v"(rk.b), "+v"(km[0]), "+v"(km[1]), "+v"(rv.v), "+v"(vm[0]), "+v"(vm[1])::"memory");
    if constexpr ((KB == 8) == true && (VB == 8) == false && NACC == 4 && NVG == 1)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.a), "+v"(rk.b), "+v"(km[0]), "+v"(km[1]), "+v"(km[2]), "+v"(km[3]), "+v"(rv.v), "+v"(vm[0])::"memory");
    if constexpr ((KB == 8) == true && (VB == 8) == false && NACC == 4 && NVG == 2)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.a), "+v"(rk.b), "+v"(km[0]), "+v"(km[1]), "+v"(km[2]), "+v"(km[3]), "+v"(rv.v), "+v"(vm[0]), "+v"(vm[1])::"memory");
    if constexpr ((KB == 8) == true && (VB == 8) == true && NACC == 1 && NVG == 1)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.a), "+v"(rk.b), "+v"(km[0]), "+v"(rv.a), "+v"(rv.b), "+v"(vm[0])::"memory");
    if constexpr ((KB == 8) == true && (VB == 8) == true && NACC == 1 && NVG == 2)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.a), "+v"(rk.b), "+v"(km[0]), "+v"(rv.a), "+v"(rv.b), "+v"(vm[0]), "+v"(vm[1])::"memory");
    if constexpr ((KB == 8) == true && (VB == 8) == true && NACC == 2 && NVG == 1)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.a), "+v"(rk.b), "+v"(km[0]), "+v"(km[1]), "+v"(rv.a), "+v"(rv.b), "+v"(vm[0])::"memory");
    if constexpr ((KB == 8) == true && (VB == 8) == true && NACC == 2 && NVG == 2)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.a), "+v"(rk.b), "+v"(km[0]), "+v"(km[1]), "+v"(rv.a), "+v"(rv.b), "+v"(vm[0]), "+v"(vm[1])::"memory");
    if constexpr ((KB == 8) == true && (VB == 8) == true && NACC == 4 && NVG == 1)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.a), "+v"(rk.b), "+v"(km[0]), "+v"(km[1]), "+v"(km[2]), "+v"(km[3]), "+v"(rv.a), "+v"(rv.b), "+v"(vm[0])::"memory");
    if constexpr ((KB == 8) == true && (VB == 8) == true && NACC == 4 && NVG == 2)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rk.a), "+v"(rk.b), "+v"(km[0]), "+v"(km[1]), "+v"(km[2]), "+v"(km[3]), "+v"(rv.a), "+v"(rv.b), "+v"(vm[0]), "+v"(vm[1])::"memory");
#pragma unroll
    for (int i = 0; i < KB; ++i) pd.kc.w[i] = rk.w(i);
#pragma unroll
    for (int i = 0; i < VB; ++i) pd.vc.w[i] = rv.w(i);
#pragma unroll
    for (int a = 0; a < NACC; ++a) pd.km[a] = make_uint4(km[a].x, km[a].y, km[a].z, km[a].w);
#pragma unroll
    for (int v = 0; v < NVG; ++v) pd.vm[v] = make_uint4(vm[v].x, vm[v].y, vm[v].z, vm[v].w);
  }

  template <bool MASKED>
  static __device__ __forceinline__ void process_pair(const Ctx &cx, State<NVG> &st, const PageData &A,
                                                      const PageData &B, int validA, int validB) {
    float s0[4], s1[4];
    pair_scores(cx, A, B, s0, s1);
    if (MASKED) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s0[r] = (4 * cx.quad + r < validA) ? s0[r] : -__builtin_inff();
        s1[r] = (4 * cx.quad + r < validB) ? s1[r] : -__builtin_inff();
      }
    }
    softmax_update<MASKED, false>(cx, st, s0, s1, nullptr);
    pair_values<MASKED>(cx, st, A, B, s0, s1, validA, validB);
  }

  // Window tokens [w0, w0 + 32) of the ring (valid below wend), scores on MFMA.  The values of
  // a bf16 ring go through MFMA as well (exact bf16 B operand, weights as the hi/lo A operand
  // of the quantized path, accumulated in st.acc); those of an fp32 ring are accumulated on the
  // VALU in ow.  Value data is requested before the scores are computed, so its latency overlaps
  // the key loads and the MFMAs.
  template <bool F32>
  static __device__ __forceinline__ void window_chunk(const Ctx &cx, State<NVG> &st, float (*ow)[2],
                                                      const uint8_t *kwin, const uint8_t *vwin, int w0, int wend) {
    const int nval = (wend - w0) < 32 ? (wend - w0) : 32;
    // fp32: this lane's two channels of value row w0 + t (rows past the end re-read row w0)
    constexpr int VT = 16;
    auto vload = [&](int t) -> f32x2e {
      return gload<f32x2e>(vwin + ((size_t)(w0 + (t < nval ? t : 0)) * KVQ_D + 2 * cx.lane) * 4);
    };
    f32x2e vr[F32 ? VT : 1];
    // bf16: B operand of value tile m for this lane = channel 16 m + col of the 8 tokens of its k
    // slots (slot j: token 4 quad + j for j < 4, 16 + 4 quad + j - 4 after; the order in which
    // weights_operand places the weights), packed in pairs.
    uint32_t vb[F32 ? 1 : 8][4];
    if constexpr (F32) {
#pragma unroll
      for (int t = 0; t < VT; ++t) vr[t] = vload(t);
    } else {
      const uint16_t *vrow[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        int t = j < 4 ? 4 * cx.quad + j : 16 + 4 * cx.quad + (j - 4);
        t = t < nval ? t : 0;  // rows past the end re-read row w0 (their weight is 0)
        vrow[j] = reinterpret_cast<const uint16_t *>(vwin) + (size_t)(w0 + t) * KVQ_D + cx.col;
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = gload<uint16_t>(vrow[2 * i] + 16 * m);
          const uint32_t hi = gload<uint16_t>(vrow[2 * i + 1] + 16 * m);
          vb[m][i] = lo | (hi << 16);
        }
      }
    }
    float s[2][4];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      int slot = w0 + 16 * sub + cx.col;  // A-operand row = token
      const bool ok = slot < wend;
      slot = ok ? slot : w0;
      f32x4 D[NACC];
#pragma unroll
      for (int a = 0; a < NACC; ++a) D[a] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (F32) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const uint8_t *rp = kwin + ((size_t)slot * KVQ_D + 32 * kc + 8 * cx.quad) * 4;
          const f32x4e f0 = gload<f32x4e>(rp);
          const f32x4e f1 = gload<f32x4e>(rp + 16);
          const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
          uint32_t hi[4], lo[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            hi[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
            lo[i] = pack_bf16x2(f[2 * i] - bf16lo_f32(hi[i]), f[2 * i + 1] - bf16hi_f32(hi[i]));
          }
          D[kc / XE] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pack8(hi[0], hi[1], hi[2], hi[3]), cx.qB[kc], D[kc / XE], 0, 0, 0);
          D[kc / XE] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pack8(lo[0], lo[1], lo[2], lo[3]), cx.qB[kc], D[kc / XE], 0, 0, 0);
        }
      } else {
        u32x4 kr[4];
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) kr[kc] = gload<u32x4>(kwin + ((size_t)slot * KVQ_D + 32 * kc + 8 * cx.quad) * 2);
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
          D[kc / XE] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pack8(kr[kc].x, kr[kc].y, kr[kc].z, kr[kc].w), cx.qB[kc], D[kc / XE], 0, 0, 0);
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
    if constexpr (F32) {
      softmax_update<true, true>(cx, st, s[0], s[1], ow);
      // Values: this lane owns channels 2*lane, 2*lane+1; p of (head h, token) lives in lane 16*quad + h.
#pragma unroll
      for (int half = 0; half < 32 / VT; ++half) {
        if (half > 0) {
#pragma unroll
          for (int t = 0; t < VT; ++t) vr[t] = vload(VT * half + t);
        }
        // Tokens past the end carry p = 0 (their scores were -inf), so the loop runs in full.
#pragma unroll
        for (int t = 0; t < VT; ++t) {
          const int tk = VT * half + t;
          const int sub = tk >> 4, tq = (tk & 15) >> 2, r = tk & 3;
          const float pv = s[sub][r];
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float p = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pv), 16 * tq + h));
            ow[h][0] = __builtin_fmaf(p, vr[t].x, ow[h][0]);
            ow[h][1] = __builtin_fmaf(p, vr[t].y, ow[h][1]);
          }
        }
      }
    } else {
      softmax_update<true, false>(cx, st, s[0], s[1], nullptr);
      const bf16x8 Aop = weights_operand(cx, s[0], s[1]);
#pragma unroll
      for (int m = 0; m < 8; ++m)
        st.acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Aop, pack8(vb[m][0], vb[m][1], vb[m][2], vb[m][3]), st.acc[m], 0, 0, 0);
    }
  }

  // Queries of the G heads of kv head kvh -> LDS (fp32 [G][128]); rotated when `rotate`.
  static __device__ __forceinline__ void stage_q(const KvqAttnArgs &args, float *qs, int b, int hq0, bool rotate) {
    const int lane = threadIdx.x;
    __syncthreads();
    for (int i = lane; i < G * KVQ_D; i += 64) {
      const size_t gi = ((size_t)b * args.Hq + hq0) * KVQ_D + i;
      qs[i] = args.q_f32 ? gload<float>((const float *)args.q + gi)
                         : kvq_bf16_bits_to_f32(gload<uint16_t>((const uint16_t *)args.q + gi));
    }
    __syncthreads();
    if (rotate) {
      for (int hs = 1; hs < KVQ_D; hs <<= 1) {
        for (int pidx = lane; pidx < G * KVQ_D / 2; pidx += 64) {
          const int hh = pidx / (KVQ_D / 2), pp = pidx % (KVQ_D / 2);
          const int i0 = (pp / hs) * 2 * hs + (pp % hs);
          float *row = qs + hh * KVQ_D;
          const float x0 = row[i0], x1 = row[i0 + hs];
          row[i0] = x0 + x1;
          row[i0 + hs] = x0 - x1;
        }
        __syncthreads();
      }
      for (int i = lane; i < G * KVQ_D; i += 64) qs[i] *= (float)KVQ_WHT_C;
      __syncthreads();
    }
  }

  static __device__ void run(const KvqAttnArgs &args, uint8_t *smem) {
    float *lds = reinterpret_cast<float *>(smem);
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
    // Window splits first, then quantized splits (see the host split plan).
    const bool win_split = split < args.wsplits;
    int wv0 = 0, wv1 = 0;
    if (win_split) {
      wv0 = split * KVQ_WIN_PAGES;
      wv1 = wv0 + KVQ_WIN_PAGES < wpages ? wv0 + KVQ_WIN_PAGES : wpages;
    }

    Ctx cx;
    init_ctx(cx, lay, args.sigma_u);
    const int hq0 = kvh * G;
    State<NVG> st;
#pragma unroll
    for (int m = 0; m < 8; ++m) st.acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m = -__builtin_inff();
    st.l = 0.f;
#pragma unroll
    for (int v = 0; v < NVG; ++v) st.zacc[v] = 0.f;

    if (win_split) {
      // Window pages: raw (and unrotated) keys, scored with the raw, unscaled query operand.
      float ow[G][2];
#pragma unroll
      for (int h = 0; h < G; ++h) ow[h][0] = ow[h][1] = 0.f;
      if (wv1 > wv0) {
        stage_q(args, lds, b, hq0, false);
        build_q(cx, lds, false);
        const size_t win_off = ((size_t)b * Hkv + kvh) * R * KVQ_D * (args.kv_f32 ? 4 : 2);
        const int wend = (wv1 * KVQ_PAGE) < nw ? wv1 * KVQ_PAGE : nw;
        for (int w = wv0 * KVQ_PAGE; w < wend; w += 32) {
          if (args.kv_f32)
            window_chunk<true>(cx, st, ow, args.cache.k_win + win_off, args.cache.v_win + win_off, w, wend);
          else
            window_chunk<false>(cx, st, ow, args.cache.k_win + win_off, args.cache.v_win + win_off, w, wend);
        }
      }
      if (args.kv_f32)
        write_partial<PART_WIN_VALU>(args, cx, st, ow, lds, b, kvh, split);
      else
        write_partial<PART_WIN_ACC>(args, cx, st, ow, lds, b, kvh, split);
      return;
    }

    // Quantized splits take full-page pairs round-robin: pair sq, sq + SQ, sq + 2 SQ, ... so that at
    // any moment the waves of one unit read neighbouring pairs.
    const int SQ = S - args.wsplits, sq = split - args.wsplits;
    const int full_pages = nq / KVQ_PAGE;  // pages with all 16 tokens quantized
    const int tp = full_pages / 2;         // full pairs of this sequence
    // Pairs of full pages, next pairs prefetched while the current one is processed.  The 1-2
    // pages after the last full pair (an odd full page and/or the partial page) form one masked
    // pair; it goes to the split next in the rotation, whose cursor reaches it right after its
    // full pairs, so it streams through the same ring.
    const int npairs = tp > sq ? (tp - sq + SQ - 1) / SQ : 0;
    const bool tail = sq == tp % SQ && 2 * tp < qpages;
    if (npairs > 0 || tail) {
      int tail_va = 0, tail_vb = 0;
      if (tail) {
        const int p = 2 * tp;
        tail_va = (nq - p * KVQ_PAGE) < KVQ_PAGE ? (nq - p * KVQ_PAGE) : KVQ_PAGE;
        tail_vb = p + 1 < qpages ? ((nq - (p + 1) * KVQ_PAGE) < KVQ_PAGE ? (nq - (p + 1) * KVQ_PAGE) : KVQ_PAGE) : 0;
      }
      // The query operand is built while the first pages stream in: without rotation the
      // query loads are issued before the prologue DMAs (vmcnt retires them first); with
      // rotation the query is staged and rotated through LDS before the ring is used.
      QRegs qr;
      if (args.rotation) {
        stage_q(args, lds, b, hq0, true);
        build_q(cx, lds);
        __syncthreads();  // the staging area is reused by the prefetch ring
      } else {
        load_q_regs(qr, args, cx, b, hq0);
      }
      stream_pairs(args, cx, st, smem, qr, b, kvh, sq, SQ, npairs, tail, tail_va, tail_vb);
    }
    write_partial<PART_CODES>(args, cx, st, nullptr, lds, b, kvh, split);
  }

  // Pairs sq, sq + SQ, ... (npairs of them) of one unit through the wave's LDS ring of NPS page
  // slots: local page k (pair k / 2) lives in slot k mod NPS.  The first AHEAD pages are requested
  // up front; processing pair i first requests pages 2i + AHEAD and 2i + AHEAD + 1 (the slots of
  // pair i - 1, already read), then waits until those two are the only pages still in flight
  // behind pair i.  Requests follow a cursor that steps through the pairs in order (the parity of
  // every request site is fixed, so the cursor moves by constant strides), and the slot addresses
  // rotate through the ring, so the loop does no index arithmetic beyond those steps.
  static __device__ __forceinline__ void stream_pairs(const KvqAttnArgs &args, Ctx &cx, State<NVG> &st, uint8_t *smem,
                                                      const QRegs &qr, int b, int kvh, int sq, int SQ, int npairs,
                                                      bool tail, int tail_va, int tail_vb) {
    const KvqLayout &lay = args.lay;
    const int lane = cx.lane, Hkv = args.Hkv;
    const int rec = lay.record, rec16 = rec / 16;
    uint32_t loff[DMAS_PER_PAGE];  // this lane's 16-byte chunk of each DMA, clamped into the record
#pragma unroll
    for (int k = 0; k < DMAS_PER_PAGE; ++k) {
      const int c = 64 * k + lane;
      loff[k] = (uint32_t)(c < rec16 ? c : rec16 - 1) << 4;
    }
    // Cursor: the pair holding the next page to request.
    const uint8_t *pages = args.cache.pages;
    const size_t page_stride = (size_t)args.cache.batch * Hkv * rec;  // contiguous: page p -> p + 1
    const size_t pair_step = 2 * (size_t)SQ * page_stride;            // contiguous: pair j -> j + SQ
    const uint8_t *cur = pages + ((size_t)b * Hkv + kvh) * rec + 2 * (size_t)sq * page_stride;
    // Block-table entries are wave-uniform: read them with scalar loads (constant address space) so
    // that waiting for one never drains the vector-memory queue of requested pages.
    typedef const __attribute__((address_space(4))) int32_t *const_i32p;
    const_i32p tcur = (const_i32p)args.cache.block_table + (int64_t)b * args.cache.mbps + 2 * sq;
    const int pool_last = (int)(args.cache.pool_pages - 1);
    const bool paged = args.cache.paged != 0;
    const uint32_t ring0 = (uint32_t)(uintptr_t)smem, ring_end = ring0 + NPS * REC_BYTES;
    uint32_t wslot = ring0, rslot = ring0;
    auto next_slot = [&](uint32_t sl) { return sl + REC_BYTES == ring_end ? ring0 : sl + REC_BYTES; };
    const int npages = 2 * (npairs + (tail ? 1 : 0));
    // A masked pair with no second page requests its first page twice (never past the cache).
    const bool dup_last = tail && tail_vb == 0;
    auto issue = [&](bool odd, int k) {
      const bool dup = odd && dup_last && k == npages - 1;
      const uint8_t *src;
      if (paged) {
        int e = tcur[(odd && !dup) ? 1 : 0];
        e = e < 0 ? 0 : (e > pool_last ? pool_last : e);
        src = pages + ((size_t)e * Hkv + kvh) * rec;
        if (odd) tcur += 2 * SQ;
      } else {
        src = (odd && !dup) ? cur + page_stride : cur;
        if (odd) cur += pair_step;
      }
      dma_page_buf(wslot, src, rec, loff, lane);
      wslot = next_slot(wslot);
    };
#pragma unroll
    for (int k = 0; k < AHEAD; ++k)
      if (k < npages) issue((k & 1) != 0, k);
    if (!args.rotation) build_q_regs(cx, qr, args.q_f32);
    constexpr bool FIRST_ODD = (AHEAD & 1) != 0;  // parity of page 2i + AHEAD
    for (int i = 0; i < npairs; ++i) {
      const int k0 = 2 * i + AHEAD;
      if (k0 + 1 < npages) {  // steady state: two requests, AHEAD pages stay in flight
        issue(FIRST_ODD, k0);
        issue(!FIRST_ODD, k0 + 1);
        wait_vmcnt<AHEAD * DMAS_PER_PAGE>();
      } else {  // the last pairs: at most one more request, then drain
        if (k0 < npages) issue(FIRST_ODD, k0);
        wait_vmcnt<0>();
      }
      PageData A, B;
      read_page_at(A, cx, rslot, lay);
      rslot = next_slot(rslot);
      read_page_at(B, cx, rslot, lay);
      rslot = next_slot(rslot);
      process_pair<false>(cx, st, A, B, 16, 16);
    }
    if (tail) {  // its pages were requested with the others
      wait_vmcnt<0>();
      PageData A, B;
      read_page_at(A, cx, rslot, lay);
      rslot = next_slot(rslot);
      read_page_at(B, cx, rslot, lay);
      process_pair<true>(cx, st, A, B, tail_va, tail_vb);
    }
  }

  // Reduce the state across rows/replicas and write this split's partial result:
  // [m (log2 units), l, 0, 0, o[128]] per query head, o unnormalised.
  // MODE: PART_CODES (quantized pages: value-code scales and zero-point sums apply),
  // PART_WIN_ACC (bf16 window: MFMA accumulators hold the output as is), PART_WIN_VALU (fp32
  // window: the output is in ow).
  static constexpr int PART_CODES = 0, PART_WIN_ACC = 1, PART_WIN_VALU = 2;
  template <int MODE>
  static __device__ __forceinline__ void write_partial(const KvqAttnArgs &args, const Ctx &cx, const State<NVG> &st,
                                                       float (*ow)[2], float *lds, int b, int kvh, int split) {
    constexpr bool WIN = MODE != PART_CODES;
    const int lane = threadIdx.x;
    const int hq0 = kvh * G;
    const float l = rows_sum(st.l);
    float z[NVG];
#pragma unroll
    for (int v = 0; v < NVG; ++v) z[v] = WIN ? 0.f : rows_sum(st.zacc[v]);
    __syncthreads();
    float *accs = lds;                 // [2G][128]
    float *hdr = lds + 2 * G * KVQ_D;  // [G][4]: m, l, z0, z1
    if constexpr (MODE != PART_WIN_VALU) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 4 * cx.quad + r;
          if (row < 2 * G) accs[row * KVQ_D + 16 * m + cx.col] = st.acc[m][r];
        }
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
    const int S = args.splits;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float *dst = args.partials + (((size_t)b * args.Hq + hq0 + h) * S + split) * KVQ_PART_STRIDE;
      float o[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int c = 2 * lane + e;
        if constexpr (MODE == PART_WIN_VALU) {
          o[e] = ow[h][e];
        } else if constexpr (MODE == PART_WIN_ACC) {
          o[e] = accs[h * KVQ_D + c] + accs[(G + h) * KVQ_D + c];
        } else {
          const float a = accs[h * KVQ_D + c] + accs[(G + h) * KVQ_D + c];
          const float outscale = __builtin_amdgcn_ldexpf(1.0f, (int)P_BIAS_LOG2 - vtile_scale(c >> 4));
          o[e] = __builtin_fmaf(a * EXP2_OUT, outscale, hdr[h * 4 + 2 + (c >> vshift)]);
        }
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
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(kvq_attn_wpe(KB, VB, G, P, NVG), kvq_attn_wpe(KB, VB, G, P, NVG)))) void kvq_attn_split_kernel(KvqAttnArgs args) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[Kern<KB, VB, G, P, NVG>::LDS_BYTES];
  Kern<KB, VB, G, P, NVG>::run(args, smem);
}

}  // namespace kvq_attn
