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
//   K: per page and 32-channel chunk, one MFMA per score accumulator with
//      A = query rows (head slot q, chunk j; only rows of the chunk being
//      contracted are non-zero) and B = codes (k = 32 channels, col = 16 tokens).
//      Lane 16 q + t then holds, in accumulator row r, head q's partial dot with
//      chunk r of token t, so the group scales and zero points are applied and the
//      chunks summed inside the lane: one score per (token, head) per lane, no
//      cross-lane reduction and no replicated softmax work.  With 8 or 16 (head,
//      query part) rows (8 heads, or hi + lo query parts) the A rows are those
//      pairs over a whole chunk instead: one MFMA per chunk into its own
//      accumulator, lane 16 q + t holding head q + 4 hb's rows of token t, the
//      chunk's scale applied per token in the lane (4 MFMAs per page instead of
//      up to 16).
//   V: 8 MFMAs (one per 16-channel tile), A = softmax weights (rows = hi/lo
//      part x head, k = 32 tokens), B = value codes (k = tokens, col = channel).
//      The weights reach the A-operand layout through a small per-wave LDS
//      exchange buffer (four 2-byte writes and one 16-byte read per lane).
// Every code and metadata operand comes from one 4- to 16-byte read per lane of the
// page record (see kvq_layout.h for the order of the record's words).
#pragma once
#include "kvq_quant.h"

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

// Scale (log2) at which a b-bit code is read when its lowest plane's field sits at bit `bit` of a
// 16-bit half: in place when the whole code then ends inside the low byte (a bf16 bit pattern x
// in the low byte is the value x * 2^-133, so a code moved to bit s reads as code * 2^s); after
// a shift by 8 when that is enough; else moved down to bit 0.  The other planes' values are moved
// next to it (plane at code offset o to bit s + o).
__host__ __device__ constexpr int code_read_scale(int b, int bit) {
  return bit + b <= 8 ? bit : ((bit >= 8 && bit - 8 + b <= 8) ? bit - 8 : 0);
}
// The field of width w at `bit` of both 16-bit halves of `word`, moved to bit `to` of each half
// (word_sh8 = word >> 8, shared by the fields a shift by 8 brings into place).  Masking after the
// shift keeps exactly the field's own bits: the target bits [to, to + w) of each half receive
// source bits [bit, bit + w) of the same half.
__device__ __forceinline__ uint32_t field_move(uint32_t word, uint32_t word_sh8, int w, int bit, int to) {
  const uint32_t m = (((1u << w) - 1u) * 0x00010001u) << to;
  const int d = bit - to;
  if (d == 0) return word & m;
  if (d == 8) return word_sh8 & m;
  return d > 0 ? ((word >> d) & m) : ((word << -d) & m);
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

// Sum over the four 16-lane rows of the wave (lanes l, l^16, l^32, l^48) with
// v_permlane16_swap / v_permlane32_swap: swapping a value with itself leaves the
// xor-16 (xor-32) partner pair in the two results.
__device__ __forceinline__ float rows_sum(float v) {
  const int b = __builtin_bit_cast(int, v);
  auto p16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  v = __builtin_bit_cast(float, (int)p16[0]) + __builtin_bit_cast(float, (int)p16[1]);
  const int c = __builtin_bit_cast(int, v);
  auto p32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return __builtin_bit_cast(float, (int)p32[0]) + __builtin_bit_cast(float, (int)p32[1]);
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

// Reductions over the 16 lanes of one row of the wave (lanes 16q .. 16q + 15): row
// rotations by 8, 4, 2, 1 leave the full result in every lane of the row.
__device__ __forceinline__ float row_ror(float v, int sh) {
  int r;
  switch (sh) {
    case 8: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false); break;
    case 4: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false); break;
    default: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false); break;
  }
  return __builtin_bit_cast(float, r);
}
__device__ __forceinline__ float row16_sum(float v) {
#pragma unroll
  for (int sh = 8; sh >= 1; sh >>= 1) v += row_ror(v, sh);
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
#pragma unroll
  for (int sh = 8; sh >= 1; sh >>= 1) v = __builtin_fmaxf(v, row_ror(v, sh));
  return v;
}

// Per-wave running state of the online softmax.  Score-side values (m, l, z) live in the
// score layout: lane 16 q + t holds token column t of heads q + 4 hb.
template <int HB, int NVG>
struct State {
  f32x4 acc[8];        // value MFMA accumulators (rows = part x head, col = channel)
  float m[HB];         // running max of head q + 4 hb, in score units (uniform in the row)
  float l[HB];         // this lane's partial sum of p
  float z[HB][NVG];    // this lane's partial sum of p * zero_v per value group
};

template <int KB, int VB, int G, int P, int NVG>
struct Kern {
  static constexpr int HB = (G + 3) / 4;   // head blocks: row q of the score layout holds heads q + 4 hb
  static constexpr int HSN = G < 4 ? G : 4;  // rows of the score layout in use
  static constexpr int NACC = HB;           // score accumulators (both query parts add into one)
  // Query layout of the score contraction.  With at most 4 (head, part) rows (G * P <= 4) the A
  // rows are (head slot, chunk) and one accumulator per head block collects every chunk's partial
  // dot in its own row (build_q_with).  With 8 or 16 such rows (ROWQ) that layout would repeat the
  // contraction once per part and head block with three quarters of the A rows zero; instead the A
  // rows are (head, part) over a whole chunk, one MFMA per chunk covers every head and part, and
  // each chunk has its own accumulator (build_q_rows).
  static constexpr bool ROWQ = G * P >= 8;
  static constexpr int QAP = ROWQ ? 1 : P, QAH = ROWQ ? 1 : HB;
  // Row of a ROWQ score accumulator (lane 16 q + t: rows 4 q .. 4 q + 3) holding head q + 4 hb,
  // query part `part`.
  static __device__ __forceinline__ constexpr int qrow(int hb, int part) { return P == 2 ? 2 * hb + part : hb; }
  static constexpr int NPK = kvq_nplanes(KB), NPV = kvq_nplanes(VB);  // bit planes of a code
  // plane widths and offsets as constants (a width of 1 for planes a code does not have)
  static constexpr int KW0 = kvq_plane_width(KB, 0), VW0 = kvq_plane_width(VB, 0);
  static constexpr int KW1 = NPK > 1 ? kvq_plane_width(KB, 1) : 1, KW2 = NPK > 2 ? kvq_plane_width(KB, 2) : 1;
  static constexpr int VW1 = NPV > 1 ? kvq_plane_width(VB, 1) : 1, VW2 = NPV > 2 ? kvq_plane_width(VB, 2) : 1;
  static constexpr int KO1 = KW0, KO2 = KW0 + KW1, VO1 = VW0, VO2 = VW0 + VW1;
  static __device__ __forceinline__ constexpr int kpw(int p) { return p == 0 ? KW0 : (p == 1 ? KW1 : KW2); }
  static __device__ __forceinline__ constexpr int vpw(int p) { return p == 0 ? VW0 : (p == 1 ? VW1 : VW2); }
  static __device__ __forceinline__ constexpr int kpo(int p) { return p == 0 ? 0 : (p == 1 ? KO1 : KO2); }
  static __device__ __forceinline__ constexpr int vpo(int p) { return p == 0 ? 0 : (p == 1 ? VO1 : VO2); }
  typedef State<HB, NVG> St;

  struct Ctx {
    bf16x8 qA[QAP][QAH][4];  // query operand per 32-channel chunk (per part and head block unless ROWQ)
    float Qc[HB][4];     // sum of the query operand over chunk r of head quad + 4 hb, x 2^-133
    uint32_t xw;         // exchange-buffer address of this lane's (head row, page-A slot)
    uint32_t xr;         // exchange-buffer address of this lane's A-operand row segment
    int lane, col, quad;
    float sig;  // softmax scale in score units (log2 domain)
    float tau;  // lazy-max margin in score units (16 in log2 units)
  };

  // Scale (log2) at which the key codes of chunk kc, pair slot i are read (see code_read_scale).
  static __device__ __forceinline__ constexpr int kslot_scale(int kc, int i) {
    return code_read_scale(KB, KW0 * ((4 * kc + i) % (16 / KW0)));
  }

  // The query operand (A of the score contraction).  Row rho = 4 hs + j of head block hb
  // holds head hs + 4 hb (part: hi or lo bf16 part of q * 2^100, both contracted into the
  // same accumulator) restricted to chunk j: in the contraction of chunk kc only rows with j == kc are
  // non-zero, so D row 4 q + r (lane 16 q + t) collects head q's partial dot with
  // chunk r of token t.  getq(hb, e) returns the fp32 query of head (lane & 15) / 4 + 4 hb
  // at channel 32 ((lane & 15) % 4) + 8 (lane / 16) + e.  For code operands
  // (code_scaled) the entries of slots whose codes are read scaled by 2^k are divided
  // by 2^k (exact); raw window keys need the unscaled operand.
  template <class GetQ>
  static __device__ __forceinline__ void build_q_with(Ctx &cx, GetQ getq, bool code_scaled) {
    const int rho = cx.lane & 15, hs = rho >> 2, j = rho & 3;
    const bool live = hs < HSN;
    float qsum[P][HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = live ? getq(hb, e) * EXP2_EQ : 0.f;
#pragma unroll
      for (int part = 0; part < P; ++part) {
        float e0[4], e1[4];
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t pr = pack_bf16x2(v[2 * i], v[2 * i + 1]);
          if (part == 1) pr = pack_bf16x2(v[2 * i] - bf16lo_f32(pr), v[2 * i + 1] - bf16hi_f32(pr));
          e0[i] = bf16lo_f32(pr);
          e1[i] = bf16hi_f32(pr);
          s += e0[i] + e1[i];
        }
        qsum[part][hb] = s;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          uint32_t w[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float f = code_scaled ? __builtin_amdgcn_ldexpf(1.0f, -kslot_scale(kc, i)) : 1.0f;
            w[i] = kc == j ? pack_bf16x2(e0[i] * f, e1[i] * f) : 0u;  // exact: power-of-two scaling
          }
          cx.qA[part][hb][kc] = pack8(w[0], w[1], w[2], w[3]);
        }
      }
    }
    // Chunk sums: the four lanes of a row rho (one per channel octet) hold its 32 channels.
#pragma unroll
    for (int part = 0; part < P; ++part) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) qsum[part][hb] = rows_sum(qsum[part][hb]) * EXP2_M66 * EXP2_M67;
    }
    // Lane 16 q + t needs the sums of rows 4 q + r (its head, chunk r), both parts.
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float q = 0.f;
#pragma unroll
        for (int part = 0; part < P; ++part) q += __shfl(qsum[part][hb], 4 * cx.quad + r);
        cx.Qc[hb][r] = q;
      }
    }
  }

  // ROWQ query operand.  Row rho = 4 hs + r holds head hs + 4 hb, part `part` (r = qrow(hb, part)),
  // over all 32 channels of each chunk: qA[0][0][kc] is the A operand of chunk kc (lane 16 c + rho:
  // channels 32 kc + 8 c + e), so D row 4 q + qrow(hb, part) of chunk kc's accumulator (lane
  // 16 q + t) is head q + 4 hb's partial dot with chunk kc of token t for that part.  getq(kc, e)
  // returns the fp32 query of the lane's row head at channel 32 kc + 8 (lane / 16) + e.  Code
  // operands divide each pair slot by its read scale as in build_q_with.
  template <class GetQ>
  static __device__ __forceinline__ void build_q_rows(Ctx &cx, GetQ getq, bool code_scaled) {
    const int rho = cx.lane & 15, hs = rho >> 2, r = rho & 3;
    const int hb = P == 2 ? (r >> 1) : r, part = P == 2 ? (r & 1) : 0;
    const bool live = hs < HSN && hb < HB;
    float qsum[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = live ? getq(kc, e) * EXP2_EQ : 0.f;
      uint32_t w[4];
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t hi = pack_bf16x2(v[2 * i], v[2 * i + 1]);
        const uint32_t lo = pack_bf16x2(v[2 * i] - bf16lo_f32(hi), v[2 * i + 1] - bf16hi_f32(hi));
        const uint32_t pr = part ? lo : hi;
        const float e0 = bf16lo_f32(pr), e1 = bf16hi_f32(pr);
        sum += e0 + e1;
        const float f = code_scaled ? __builtin_amdgcn_ldexpf(1.0f, -kslot_scale(kc, i)) : 1.0f;
        w[i] = pack_bf16x2(e0 * f, e1 * f);  // exact: power-of-two scaling
      }
      qsum[kc] = sum;
      cx.qA[0][0][kc] = pack8(w[0], w[1], w[2], w[3]);
    }
    // Chunk sums of each row (its four lanes hold the chunk's 32 channels), then for lane 16 q + t
    // the sums of its heads q + 4 hb over both parts.
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) qsum[kc] = rows_sum(qsum[kc]) * EXP2_M66 * EXP2_M67;
#pragma unroll
    for (int h = 0; h < HB; ++h) {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        float q = 0.f;
#pragma unroll
        for (int pp = 0; pp < P; ++pp) q += __shfl(qsum[kc], 4 * cx.quad + qrow(h, pp));
        cx.Qc[h][kc] = q;
      }
    }
  }

  // Query from LDS (fp32 [G][128]).
  static __device__ __forceinline__ void build_q(Ctx &cx, const float *qs, bool code_scaled = true) {
    if constexpr (ROWQ) {
      const int rho = cx.lane & 15, r = rho & 3, hb = P == 2 ? (r >> 1) : r;
      const int h = ((rho >> 2) < HSN && hb < HB) ? (rho >> 2) + 4 * hb : 0;
      build_q_rows(cx, [&](int kc, int e) { return qs[h * KVQ_D + 32 * kc + 8 * cx.quad + e]; }, code_scaled);
    } else {
      const int rho = cx.lane & 15, hs = (rho >> 2) < HSN ? (rho >> 2) : 0, ch0 = 32 * (rho & 3) + 8 * cx.quad;
      build_q_with(cx, [&](int hb, int e) { return qs[(hs + 4 * hb) * KVQ_D + ch0 + e]; }, code_scaled);
    }
  }

  // This lane's query channels (one octet of one chunk per head block), straight from global
  // memory: 16-byte loads, fp32 or bf16 as stored.
  // (ROWQ: one octet of every chunk of the lane's row head.)
  static constexpr int QRN = ROWQ ? 4 : HB;
  struct QRegs {
    u32x4 v[QRN][2];
  };
  static __device__ __forceinline__ void load_q_regs(QRegs &qr, const KvqAttnArgs &args, const Ctx &cx, int b,
                                                     int hq0) {
    if constexpr (ROWQ) {
      const int rho = cx.lane & 15, r = rho & 3, hb = P == 2 ? (r >> 1) : r;
      const int h = ((rho >> 2) < HSN && hb < HB) ? (rho >> 2) + 4 * hb : 0;
      const uint8_t *row = (const uint8_t *)args.q + ((size_t)b * args.Hq + hq0 + h) * KVQ_D * (args.q_f32 ? 4 : 2);
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const int ch0 = 32 * kc + 8 * cx.quad;
        if (args.q_f32) {
          qr.v[kc][0] = gload<u32x4>(row + 4 * ch0);
          qr.v[kc][1] = gload<u32x4>(row + 4 * ch0 + 16);
        } else {
          qr.v[kc][0] = gload<u32x4>(row + 2 * ch0);
        }
      }
      return;
    }
    const int rho = cx.lane & 15, hs = (rho >> 2) < HSN ? (rho >> 2) : 0, ch0 = 32 * (rho & 3) + 8 * cx.quad;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const uint8_t *row =
          (const uint8_t *)args.q + ((size_t)b * args.Hq + hq0 + hs + 4 * hb) * KVQ_D * (args.q_f32 ? 4 : 2);
      if (args.q_f32) {
        qr.v[hb][0] = gload<u32x4>(row + 4 * ch0);
        qr.v[hb][1] = gload<u32x4>(row + 4 * ch0 + 16);
      } else {
        qr.v[hb][0] = gload<u32x4>(row + 2 * ch0);
      }
    }
  }
  static __device__ __forceinline__ void build_q_regs(Ctx &cx, const QRegs &qr, bool q_f32, bool code_scaled = true) {
    // (copy the vector element out first: a bit cast of the element lvalue itself reads the
    // vector's first element)
    auto get = [&](int i, int e) {
      const uint32_t u = qr.v[i][e >> 2][e & 3];
      if (q_f32) return __builtin_bit_cast(float, u);
      const uint32_t w = qr.v[i][0][e >> 1];
      return kvq_bf16_bits_to_f32((e & 1) ? (w >> 16) : (w & 0xFFFF));
    };
    if constexpr (ROWQ)
      build_q_rows(cx, get, code_scaled);
    else
      build_q_with(cx, get, code_scaled);
  }

  static __device__ __forceinline__ void init_ctx(Ctx &cx, float sig, uint32_t xbase) {
    cx.lane = threadIdx.x;
    cx.col = cx.lane & 15;
    cx.quad = cx.lane >> 4;
    cx.sig = sig;
    cx.tau = 16.0f / sig;
    // Weights exchange buffer per value group: [16 rows][32 k slots] bf16, row = part * G + head,
    // slot 8 q' + e: page-A token 4 q' + e (e < 4), page-B token 4 q' + e - 4 (e >= 4).
    cx.xw = xbase + 64 * cx.quad + 2 * (8 * (cx.col >> 2) + (cx.col & 3));
    cx.xr = xbase + 64 * cx.col + 16 * cx.quad;
  }

  template <int KS>
  struct PageData {
    static constexpr int NKM = 4 >> KS;  // key groups per token
    Words<KB> kc;
    uint32_t km[NKM];  // this lane's token: {scale, zero} per key group
    Words<VB> vc;
    uint32_t vm[NVG];  // this lane's token: {scale, zero} per value group
  };

  // Key codes of chunk kc of one page as the B operand (slot scales per kslot_scale): per pair
  // slot, the value of each bit plane moved into place and OR-ed (one plane: masked in place or
  // after the shared shift by 8).
  template <int KS>
  static __device__ __forceinline__ bf16x8 key_operand(const PageData<KS> &pd, int kc) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = 4 * kc + i, sc = kslot_scale(kc, i);
      uint32_t v = 0;
#pragma unroll
      for (int p = 0; p < NPK; ++p) {
        const int pw = kpw(p), po = kpo(p), per = 16 / pw;
        const uint32_t word = pd.kc.w[po + u / per];
        v |= field_move(word, word >> 8, pw, pw * (u % per), sc + po);
      }
      w[i] = v;
    }
    return pack8(w[0], w[1], w[2], w[3]);
  }

  // Score of this lane's token for head quad + 4 hb: sum over chunks r of
  // scale_g(r) * (q . c) + sum over groups g of zero_g * sum(q over g).
  template <int KS>
  static __device__ __forceinline__ float score_one(const PageData<KS> &pd, const f32x4 *D, const float (*Qg)[4],
                                                    int hb) {
    float acc = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc = __builtin_fmaf(D[hb][r], h2f(pd.km[r >> KS] & 0xFFFF), acc);
#pragma unroll
    for (int g = 0; g < (4 >> KS); ++g) acc = __builtin_fmaf(h2f(pd.km[g] >> 16), Qg[hb][g], acc);
    return acc;
  }

  // Online-softmax update with the scores of two 16-token column sets (a page pair, or
  // two window halves); returns p * 2^64 in place.  Lazy running max: weights are formed
  // against the running max m, which is only raised (with the row's tile max and a rescale
  // of everything accumulated so far) when some lane sees a score more than 16 (log2
  // units) above it, so weights stay below 2^(64+16).
  template <bool MASKED, bool WINF32>
  static __device__ __forceinline__ void softmax_update(const Ctx &cx, St &st, float sA[HB], float sB[HB],
                                                        float (*ow)[2]) {
    float t[HB];
    bool up = false;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      t[hb] = __builtin_fmaxf(sA[hb], sB[hb]);
      up = up || (t[hb] > st.m[hb] + cx.tau);
    }
    if (__builtin_amdgcn_ballot_w64(up)) {
      float alpha[HB];  // per lane, uniform in the row
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const float tm = row16_max(t[hb]);
        const float mnew = __builtin_fmaxf(st.m[hb], tm);
        // st.m == -inf gives alpha = 0 (nothing accumulated yet).
        alpha[hb] = (mnew > st.m[hb]) ? __builtin_amdgcn_exp2f(cx.sig * (st.m[hb] - mnew)) : 1.0f;
        st.l[hb] *= alpha[hb];
#pragma unroll
        for (int v = 0; v < NVG; ++v) st.z[hb][v] *= alpha[hb];
        st.m[hb] = mnew;
      }
      // alpha of head h, wave-uniform: row h mod 4 of the score layout, register h / 4.
      auto head_alpha = [&](int h) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha[h >> 2]), 16 * (h & 3)));
      };
      // Value accumulator row 4 quad + r is (part, head (4 quad + r) mod G).
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float ar;
        if constexpr (G == 8) {
          const float a0 = head_alpha(r), a1 = head_alpha(4 + r);
          ar = (cx.quad & 1) ? a1 : a0;
        } else {
          ar = head_alpha(r % G);
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) st.acc[m][r] *= ar;
      }
      if constexpr (WINF32) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float ah = head_alpha(h);
          ow[h][0] *= ah;
          ow[h][1] *= ah;
        }
      }
    }
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const float nb = __builtin_fmaf(-cx.sig, st.m[hb], P_BIAS_LOG2);
      float pA = __builtin_amdgcn_exp2f(__builtin_fmaf(sA[hb], cx.sig, nb));
      float pB = __builtin_amdgcn_exp2f(__builtin_fmaf(sB[hb], cx.sig, nb));
      if (MASKED) {
        pA = (sA[hb] == -__builtin_inff()) ? 0.f : pA;
        pB = (sB[hb] == -__builtin_inff()) ? 0.f : pB;
      }
      st.l[hb] += pA + pB;
      sA[hb] = pA;
      sB[hb] = pB;
    }
  }

  // Weights of this lane's tokens (page A, page B) for head quad + 4 hb -> exchange buffer v as
  // bf16 hi part (row head) and lo part (row G + head).  Rows of heads beyond G are not written.
  static __device__ __forceinline__ void xchg_put(const Ctx &cx, int v, int hb, float wA, float wB) {
    const uint32_t hi = pack_bf16x2(wA, wB);
    const uint32_t lo = pack_bf16x2(wA - bf16lo_f32(hi), wB - bf16hi_f32(hi));
    if (HSN == 4 || cx.quad < HSN) {
      const uint32_t addr = cx.xw + KVQ_XCHG_BYTES * v + 256 * hb;
      asm volatile("ds_write_b16 %0, %1" ::"v"(addr), "v"(hi));
      asm volatile("ds_write_b16_d16_hi %0, %1 offset:8" ::"v"(addr), "v"(hi));
      asm volatile("ds_write_b16 %0, %1 offset:%2" ::"v"(addr), "v"(lo), "n"(64 * G));
      asm volatile("ds_write_b16_d16_hi %0, %1 offset:%2" ::"v"(addr), "v"(lo), "n"(64 * G + 8));
    }
  }
  // A operand of the value contraction for value group v (LDS operations of a wave complete in
  // order, so this read sees the writes above).
  static __device__ __forceinline__ u32x4 xchg_get(const Ctx &cx, int v) {
    u32x4 x;
    asm volatile("ds_read_b128 %0, %1" : "=v"(x) : "v"(cx.xr + KVQ_XCHG_BYTES * v));
    return x;
  }

  // Scale (log2) at which the value codes of tile m are read (independent of the pair slot).
  static __device__ __forceinline__ constexpr int vtile_scale(int m) { return code_read_scale(VB, (m * VW0) & 15); }

  // Value contraction of a page pair: weights p (carried as p * 2^64) times the value scale of
  // each token go through the exchange buffer into the A operand, the masked codes are B.
  template <int KS, bool MASKED>
  static __device__ __forceinline__ void pair_values(const Ctx &cx, St &st, const PageData<KS> &A,
                                                     const PageData<KS> &B, const float pA[HB], const float pB[HB],
                                                     int validA, int validB) {
#pragma unroll
    for (int v = 0; v < NVG; ++v) {
      float sa = h2f(A.vm[v] & 0xFFFF), za = h2f(A.vm[v] >> 16), sb = h2f(B.vm[v] & 0xFFFF),
            zb = h2f(B.vm[v] >> 16);
      if (MASKED) {  // metadata of invalid tokens may be anything, keep it out
        const bool va = cx.col < validA, vb = cx.col < validB;
        sa = va ? sa : 0.f;
        za = va ? za : 0.f;
        sb = vb ? sb : 0.f;
        zb = vb ? zb : 0.f;
      }
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        st.z[hb][v] = __builtin_fmaf(pB[hb], zb, __builtin_fmaf(pA[hb], za, st.z[hb][v]));
        xchg_put(cx, v, hb, pA[hb] * sa, pB[hb] * sb);
      }
    }
    u32x4 xa[NVG];
#pragma unroll
    for (int v = 0; v < NVG; ++v) xa[v] = xchg_get(cx, v);
    if constexpr (NVG == 1) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(xa[0])::"memory");
    if constexpr (NVG == 2) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(xa[0]), "+v"(xa[1])::"memory");
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t v = 0;
#pragma unroll
        for (int p = 0; p < NPV; ++p) {
          const int pw = vpw(p), po = vpo(p);
          const int pos = (i & 1) * 8 * pw + m * pw;
          const uint32_t word = (i < 2) ? A.vc.w[po + (pos >> 4)] : B.vc.w[po + (pos >> 4)];
          v |= field_move(word, word >> 8, pw, pos & 15, vtile_scale(m) + po);
        }
        w[i] = v;
      }
      const u32x4 x = xa[m / (8 / NVG)];
      st.acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x), pack8(w[0], w[1], w[2], w[3]),
                                                          st.acc[m], 0, 0, 0);
    }
  }

  // ---- LDS ring -------------------------------------------------------------
  static constexpr int MAX_REC16 = kvq_rec16(KB, VB, NVG);  // record in 16-byte units (k_group 32)
  static constexpr int DMAS_PER_PAGE = (MAX_REC16 + 63) / 64;
  static constexpr int WPE = kvq_attn_wpe(KB, VB, G, P, NVG);       // waves per SIMD
  static constexpr bool PAD = kvq_slot_pad(KB, VB, NVG, WPE);       // slots of whole DMAs: all lanes land
  static constexpr int REC_BYTES = kvq_slot_bytes(KB, VB, NVG, WPE);  // ring slot stride
  static constexpr int NPS = kvq_ring_pages(REC_BYTES, WPE, NVG);  // page slots
  static constexpr int AHEAD = NPS - 2;                             // pages in flight while a pair is processed
  static constexpr int XCHG_OFF = NPS * REC_BYTES;                  // exchange buffers after the ring
  static constexpr int LDS_BYTES = kvq_attn_lds_bytes(KB, VB, NVG, WPE);
  static_assert(LDS_BYTES >= XCHG_OFF + KVQ_XCHG_BYTES * NVG && LDS_BYTES >= KVQ_STAGE_BYTES, "LDS sizing");
  static_assert(AHEAD * DMAS_PER_PAGE <= 63, "vmcnt range");

  // Copy one page record into an LDS slot: DMAS_PER_PAGE wave-wide DMAs, lane l of DMA k writing
  // slot chunk 64k + l, through a buffer resource spanning just the record (scalar base and size),
  // with 32-bit lane offsets (16-byte chunks, clamped into the record) and the slot given as an
  // LDS byte address (base: the low 32 bits of the slot's shared-aperture address); lanes past
  // the slot stay idle (none when slots are padded to whole DMAs: lanes past the record re-read
  // its last chunk into the padding).  The resource's range check also keeps every lane inside
  // the record.
  static __device__ __forceinline__ void dma_page_buf(uint32_t slot_lds, const uint8_t *rec, int rec_bytes,
                                                      const uint32_t (&loff)[DMAS_PER_PAGE], int lane) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)rec, 0, rec_bytes, 0x00020000);
#pragma unroll
    for (int k = 0; k < DMAS_PER_PAGE; ++k) {
      if (PAD || k + 1 < DMAS_PER_PAGE || lane < MAX_REC16 - 64 * k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_vptr)(size_t)(slot_lds + 1024u * k), 16, loff[k], 0, 0, 0);
    }
  }

  // Read one page of a ring slot.  The reads are inline asm: the compiler cannot
  // tell that they do not alias the ring's in-flight DMAs and would otherwise
  // drain every outstanding load before them.  One lgkmcnt(0) wait follows them, and
  // every result passes through an empty asm statement placed after that wait before
  // anything uses it.
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
  template <int N>
  static __device__ __forceinline__ void tie(RawWords<N> &d) {
    if constexpr (N == 8)
      asm volatile("" : "+v"(d.a), "+v"(d.b));
    else
      asm volatile("" : "+v"(d.v));
  }

  // Offsets of this lane's operands inside a record.
  // Offsets of this lane's operands inside a record (codes: one per bit plane).
  struct RecOff {
    uint32_t kc[NPK], km, vc[NPV], vm;
  };
  template <int KS>
  static __device__ __forceinline__ RecOff rec_offsets(const Ctx &cx, const KvqLayout &lay) {
    RecOff o;
#pragma unroll
    for (int p = 0; p < NPK; ++p)
      o.kc[p] = lay.k_codes_off + 256 * kpo(p) + cx.lane * 4 * kpw(p);
    o.km = lay.k_meta_off + cx.col * 4 * (4 >> KS);
#pragma unroll
    for (int p = 0; p < NPV; ++p)
      o.vc[p] = lay.v_codes_off + 256 * vpo(p) + cx.lane * 4 * vpw(p);
    o.vm = lay.v_meta_off + cx.col * 4 * NVG;
    return o;
  }

  template <int KS>
  static __device__ __forceinline__ void read_page_at(PageData<KS> &pd, uint32_t base, const RecOff &o) {
    constexpr int NKM = 4 >> KS;
    RawWords<KW0> rk0;
    RawWords<KW1> rk1;
    RawWords<KW2> rk2;
    RawWords<NKM> rkm;
    RawWords<VW0> rv0;
    RawWords<VW1> rv1;
    RawWords<VW2> rv2;
    RawWords<NVG> rvm;
    ds_read_words(rk0, base + o.kc[0]);
    if constexpr (NPK > 1) ds_read_words(rk1, base + o.kc[NPK > 1 ? 1 : 0]);
    if constexpr (NPK > 2) ds_read_words(rk2, base + o.kc[NPK > 2 ? 2 : 0]);
    ds_read_words(rkm, base + o.km);
    ds_read_words(rv0, base + o.vc[0]);
    if constexpr (NPV > 1) ds_read_words(rv1, base + o.vc[NPV > 1 ? 1 : 0]);
    if constexpr (NPV > 2) ds_read_words(rv2, base + o.vc[NPV > 2 ? 2 : 0]);
    ds_read_words(rvm, base + o.vm);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    tie(rk0);
    if constexpr (NPK > 1) tie(rk1);
    if constexpr (NPK > 2) tie(rk2);
    tie(rkm);
    tie(rv0);
    if constexpr (NPV > 1) tie(rv1);
    if constexpr (NPV > 2) tie(rv2);
    tie(rvm);
#pragma unroll
    for (int i = 0; i < KW0; ++i) pd.kc.w[i] = rk0.w(i);
    if constexpr (NPK > 1) {
#pragma unroll
      for (int i = 0; i < KW1; ++i) pd.kc.w[KO1 + i] = rk1.w(i);
    }
    if constexpr (NPK > 2) {
#pragma unroll
      for (int i = 0; i < KW2; ++i) pd.kc.w[KO2 + i] = rk2.w(i);
    }
#pragma unroll
    for (int i = 0; i < NKM; ++i) pd.km[i] = rkm.w(i);
#pragma unroll
    for (int i = 0; i < VW0; ++i) pd.vc.w[i] = rv0.w(i);
    if constexpr (NPV > 1) {
#pragma unroll
      for (int i = 0; i < VW1; ++i) pd.vc.w[VO1 + i] = rv1.w(i);
    }
    if constexpr (NPV > 2) {
#pragma unroll
      for (int i = 0; i < VW2; ++i) pd.vc.w[VO2 + i] = rv2.w(i);
    }
#pragma unroll
    for (int v = 0; v < NVG; ++v) pd.vm[v] = rvm.w(v);
  }

  // Scores of this lane's token of one page for its heads quad + 4 hb.
  template <int KS>
  static __device__ __forceinline__ void page_scores(const Ctx &cx, const float (*Qg)[4], const PageData<KS> &pd,
                                                     float s[HB]) {
    if constexpr (ROWQ) {
      // one MFMA per chunk into its own accumulator; the chunk's group scale applies per token
      f32x4 Dk[4];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
        Dk[kc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cx.qA[0][0][kc], key_operand(pd, kc),
                                                         f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        float acc = 0.f;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const float d = P == 2 ? Dk[kc][qrow(hb, 0)] + Dk[kc][qrow(hb, 1)] : Dk[kc][qrow(hb, 0)];
          acc = __builtin_fmaf(d, h2f(pd.km[kc >> KS] & 0xFFFF), acc);
        }
#pragma unroll
        for (int g = 0; g < (4 >> KS); ++g) acc = __builtin_fmaf(h2f(pd.km[g] >> 16), Qg[hb][g], acc);
        s[hb] = acc;
      }
      return;
    }
    f32x4 D[NACC];
#pragma unroll
    for (int a = 0; a < NACC; ++a) D[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const bf16x8 k = key_operand(pd, kc);
#pragma unroll
      for (int part = 0; part < P; ++part) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
          D[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cx.qA[part][hb][kc], k, D[hb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) s[hb] = score_one(pd, D, Qg, hb);
  }

  template <int KS, bool MASKED>
  static __device__ __forceinline__ void process_pair(const Ctx &cx, St &st, const float (*Qg)[4],
                                                      const PageData<KS> &A, const PageData<KS> &B, int validA,
                                                      int validB) {
    float sA[HB], sB[HB];
    page_scores(cx, Qg, A, sA);
    page_scores(cx, Qg, B, sB);
    if (MASKED) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        sA[hb] = cx.col < validA ? sA[hb] : -__builtin_inff();
        sB[hb] = cx.col < validB ? sB[hb] : -__builtin_inff();
      }
    }
    softmax_update<MASKED, false>(cx, st, sA, sB, nullptr);
    pair_values<KS, MASKED>(cx, st, A, B, sA, sB, validA, validB);
  }

  // Window tokens [w0, w0 + 32) of the ring (valid below wend), scores on MFMA with the raw
  // keys as the B operand.  The values of a bf16 ring go through MFMA as well (exact bf16 B
  // operand, weights through the exchange buffer as for the quantized pages, accumulated in
  // st.acc); those of an fp32 ring are accumulated on the VALU in ow.  Value data is requested
  // before the scores are computed, so its latency overlaps the key loads and the MFMAs.
  // s_new >= 0 (bf16 rings only): ring slot whose token is read from knew / vnew instead (the
  // token appended by a fused decode step, written to that slot by this launch).
  template <bool F32>
  static __device__ __forceinline__ void window_chunk(const Ctx &cx, St &st, float (*ow)[2], const uint8_t *kwin,
                                                      const uint8_t *vwin, int w0, int wend, int s_new = -1,
                                                      const uint8_t *knew = nullptr,
                                                      const uint8_t *vnew = nullptr) {
    const int nval = (wend - w0) < 32 ? (wend - w0) : 32;
    // fp32: this lane's two channels of value row w0 + t (rows past the end re-read row w0)
    constexpr int VT = G * P >= 16 ? 8 : 16;  // value rows in registers at a time
    auto vload = [&](int t) -> f32x2e {
      return gload<f32x2e>(vwin + ((size_t)(w0 + (t < nval ? t : 0)) * KVQ_D + 2 * cx.lane) * 4);
    };
    f32x2e vr[F32 ? VT : 1];
    // bf16: B operand of value tile m for this lane = channel 16 m + col of the 8 tokens of its k
    // slots (slot j: token 4 quad + j for j < 4, 16 + 4 quad + j - 4 after), packed in pairs.
    uint32_t vb[F32 ? 1 : 8][4];
    auto load_vb = [&]() {
      const uint16_t *vrow[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        int t = j < 4 ? 4 * cx.quad + j : 16 + 4 * cx.quad + (j - 4);
        t = t < nval ? t : 0;  // rows past the end re-read row w0 (their weight is 0)
        vrow[j] = (w0 + t == s_new) ? reinterpret_cast<const uint16_t *>(vnew) + cx.col
                                    : reinterpret_cast<const uint16_t *>(vwin) + (size_t)(w0 + t) * KVQ_D + cx.col;
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
    };
    // With 16 query rows (8 heads, hi/lo parts) the value rows are fetched after the scores, which
    // keeps the register footprint inside the occupancy budget.
    constexpr bool EARLY_V = G * P < 16;
    if constexpr (F32) {
#pragma unroll
      for (int t = 0; t < VT; ++t) vr[t] = vload(t);
    } else if constexpr (EARLY_V) {
      load_vb();
    }
    float s[2][HB];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      int slot = w0 + 16 * sub + cx.col;  // B-operand column = token
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
          const bf16x8 kh = pack8(hi[0], hi[1], hi[2], hi[3]), kl = pack8(lo[0], lo[1], lo[2], lo[3]);
#pragma unroll
          for (int part = 0; part < QAP; ++part) {
#pragma unroll
            for (int hb = 0; hb < QAH; ++hb) {
              D[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cx.qA[part][hb][kc], kh, D[hb], 0, 0, 0);
              D[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cx.qA[part][hb][kc], kl, D[hb], 0, 0, 0);
            }
          }
        }
      } else {
        u32x4 kr[4];
        const uint8_t *krow = slot == s_new ? knew : kwin + (size_t)slot * KVQ_D * 2;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) kr[kc] = gload<u32x4>(krow + (32 * kc + 8 * cx.quad) * 2);
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
          for (int part = 0; part < QAP; ++part) {
#pragma unroll
            for (int hb = 0; hb < QAH; ++hb)
              D[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cx.qA[part][hb][kc], __builtin_bit_cast(bf16x8, kr[kc]),
                                                              D[hb], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        // ROWQ: one accumulator, rows (head, part); else one per head block, rows (head, chunk)
        const float acc = ROWQ ? (P == 2 ? D[0][qrow(hb, 0)] + D[0][qrow(hb, 1)] : D[0][qrow(hb, 0)])
                               : (D[hb][0] + D[hb][1]) + (D[hb][2] + D[hb][3]);
        s[sub][hb] = ok ? acc * EXP2_M66 * EXP2_M67 : -__builtin_inff();
      }
    }
    softmax_update<true, F32>(cx, st, s[0], s[1], ow);
    if constexpr (F32) {
      // Values: this lane owns channels 2*lane, 2*lane+1; p of (head h, token tk) lives in lane
      // 16 (h mod 4) + tk mod 16, register s[tk / 16][h / 4].
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
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float pv = s[tk >> 4][h >> 2];
            const float p = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pv), 16 * (h & 3) + (tk & 15)));
            ow[h][0] = __builtin_fmaf(p, vr[t].x, ow[h][0]);
            ow[h][1] = __builtin_fmaf(p, vr[t].y, ow[h][1]);
          }
        }
      }
    } else {
      if constexpr (!EARLY_V) load_vb();
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) xchg_put(cx, 0, hb, s[0][hb], s[1][hb]);
      u32x4 xa = xchg_get(cx, 0);
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(xa)::"memory");
      const bf16x8 Aop = __builtin_bit_cast(bf16x8, xa);
#pragma unroll
      for (int m = 0; m < 8; ++m)
        st.acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Aop, pack8(vb[m][0], vb[m][1], vb[m][2], vb[m][3]), st.acc[m], 0, 0, 0);
    }
  }

  // ---- fused decode step ---------------------------------------------------------------
  // LDS of a window split beyond the staged query ([G][128] fp32): a page record holding only the
  // token that leaves the window (at token slot 0), then that token's codes and metadata words.
  static constexpr int VREC_OFF = G * KVQ_D * 4;
  static constexpr int QSCR_OFF = VREC_OFF + 16 * MAX_REC16;
  static_assert(QSCR_OFF + 2 * KVQ_D + 4 * 4 + 2 * 4 <= XCHG_OFF, "fused-step scratch overlaps the exchange buffer");

  // The append of a fused decode step, by the window split whose range holds the new token's ring
  // slot s_new = Lb mod R (Lb = length before the step).  When the ring is full (Lb >= R) the
  // token in that slot, position Lb - R, leaves the window: it is read from the ring (before the
  // slot is overwritten: same lanes, same addresses, its loads waited for), rotated if keys are,
  // quantized with the append kernels' fp64 sequence, written into its page record (token slot
  // (Lb - R) mod 16; other splits of this launch read that page only with the token masked out)
  // and into a one-token record at VREC_OFF for evicted_pair.  The new token is written to slot
  // s_new.  Returns whether a token left the window.
  static __device__ __forceinline__ bool fused_append(const KvqAttnArgs &args, uint8_t *smem, int b, int kvh, int Lb,
                                                      int s_new) {
    const int lane = threadIdx.x, R = args.R, Hkv = args.Hkv;
    const KvqLayout &lay = args.lay;
    const size_t row = (size_t)KVQ_D * 2, unit = (size_t)b * Hkv + kvh;
    uint8_t *kslot = args.cache.k_win + (unit * R + s_new) * row;
    uint8_t *vslot = args.cache.v_win + (unit * R + s_new) * row;
    const bool evict = Lb >= R;
    uint32_t ko = 0, vo = 0;
    if (evict) {
      ko = gload<uint32_t>(kslot + 4 * lane);
      vo = gload<uint32_t>(vslot + 4 * lane);
    }
    const uint32_t kn = gload<uint32_t>(args.k_new + unit * row + 4 * lane);
    const uint32_t vn = gload<uint32_t>(args.v_new + unit * row + 4 * lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the old token is in registers before the slot is written
    *reinterpret_cast<uint32_t *>(kslot + 4 * lane) = kn;
    *reinterpret_cast<uint32_t *>(vslot + 4 * lane) = vn;
    if (!evict) return false;
    double k0 = (double)kvq_bf16_bits_to_f32(ko & 0xFFFFu), k1 = (double)kvq_bf16_bits_to_f32(ko >> 16);
    const double v0 = (double)kvq_bf16_bits_to_f32(vo & 0xFFFFu), v1 = (double)kvq_bf16_bits_to_f32(vo >> 16);
    if (args.rotation) kvq_wht128_fp64(k0, k1, lane);
    uint32_t a0, a1, am, b0, b1, bm;
    kvq_quant::quantize_pair(k0, k1, lay.kb, lay.kg, &a0, &a1, &am);
    kvq_quant::quantize_pair(v0, v1, lay.vb, lay.vg, &b0, &b1, &bm);
    uint8_t *ck = smem + QSCR_OFF, *cv = ck + KVQ_D;
    uint32_t *mk = reinterpret_cast<uint32_t *>(cv + KVQ_D), *mv = mk + 4;
    ck[2 * lane] = (uint8_t)a0;
    ck[2 * lane + 1] = (uint8_t)a1;
    cv[2 * lane] = (uint8_t)b0;
    cv[2 * lane + 1] = (uint8_t)b1;
    if (((2 * lane) % lay.kg) == 0) mk[(2 * lane) / lay.kg] = am;
    if (((2 * lane) % lay.vg) == 0) mv[(2 * lane) / lay.vg] = bm;
    uint32_t *vrec = reinterpret_cast<uint32_t *>(smem + VREC_OFF);
    for (int w = lane; w < lay.record / 4; w += 64) vrec[w] = 0u;
    __syncthreads();
    const int64_t t_ev = (int64_t)Lb - R, page = t_ev / KVQ_PAGE;
    if (page < (args.cache.paged ? (int64_t)args.cache.mbps : args.cache.pages_per_seq)) {
      const int64_t ri = kvq_record_index_dev(args.cache, Hkv, b, kvh, page);
      kvq_quant::kvq_write_token(args.cache.pages + (size_t)ri * lay.record, lay, (int)(t_ev % KVQ_PAGE), ck, cv, mk,
                                 mv, lane);
    } else {
      kvq_raise(args.cache, true, KVQ_DEV_CAPACITY);  // not stored (still attended below)
    }
    kvq_quant::kvq_write_token(smem + VREC_OFF, lay, 0, ck, cv, mk, mv, lane);
    __syncthreads();
    return true;
  }

  // Attention over the token that left the window (the one-token record at VREC_OFF), on top of
  // the window tokens already in st: the value accumulators are brought from the window's scale
  // to the scale of the code contractions (tile m: 2^(s_m - 133), exact power-of-two multiplies),
  // the code-scaled query operand (rotated when keys are) is built, and the record goes
  // through the masked pair path with one valid token.
  template <int KS>
  static __device__ __forceinline__ void evicted_pair(const KvqAttnArgs &args, Ctx &cx, St &st, uint8_t *smem,
                                                      int b, int hq0) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float f = __builtin_amdgcn_ldexpf(1.0f, vtile_scale(m) - 66);
#pragma unroll
      for (int r = 0; r < 4; ++r) st.acc[m][r] = st.acc[m][r] * f * EXP2_M67;
    }
    float *lds = reinterpret_cast<float *>(smem);
    stage_q(args, lds, b, hq0, args.rotation != 0);
    build_q(cx, lds);
    float Qg[HB][4];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) Qg[hb][g] = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) Qg[hb][r >> KS] += cx.Qc[hb][r];
    }
    const RecOff ro = rec_offsets<KS>(cx, args.lay);
    PageData<KS> A;
    read_page_at(A, (uint32_t)(uintptr_t)smem + VREC_OFF, ro);
    process_pair<KS, true>(cx, st, Qg, A, A, 1, 0);
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

  // ---- per-sequence split plan ------------------------------------------------------------
  // Quantized splits of each kv head of a sequence with qp quantized pages, out of Q pages over
  // the batch: a share of the launch's quantized waves proportional to its pages (at most cap_max,
  // at least 1), pages per split even (whole pairs) and at least 2.  With equal lengths this is
  // the same count for every sequence.  The share is floor(target_q * qp / (Hkv * Q)) taken in fp64:
  // both products are integers below 2^50, so a non-integer quotient lies at least 1 / (Hkv * Q)
  // from an integer, far above the rounding of the division, and the floor is exact.
  static __device__ __forceinline__ int plan_qsplits(const KvqAttnArgs &a, int qp, double Q) {
    int per;
    if (a.fixed_per > 0) {
      per = a.fixed_per;
    } else {
      int cap = Q > 0.0 ? (int)__builtin_floor((double)a.target_q * (double)qp / ((double)a.Hkv * Q)) : 1;
      cap = cap < 1 ? 1 : (cap > a.cap_max ? a.cap_max : cap);
      per = (qp + cap - 1) / cap;
    }
    per = per < 2 ? 2 : per;
    per = (per + 1) & ~1;
    const int s = (qp + per - 1) / per;
    return s < 1 ? 1 : s;
  }
  // Work items of the launch, sequence after sequence: S_b = window splits + plan_qsplits for each
  // kv head of sequence b.  Blocks go to the 8 XCDs round-robin (block mod 8), and the page
  // records of kv heads 2i and 2i + 1 are adjacent (a 1856-byte K4V2 record is 14.5 cache lines
  // of 128 bytes, so the two share a line): with an even Hkv the items are pair items (kv-head
  // pair, split), and pair item k runs on waves 16 (k / 8) + k mod 8 (kv head 2i) and that + 8
  // (kv head 2i + 1), so both halves of every shared line are fetched into one XCD's L2 whatever
  // the split counts (up to 14 waves at the end of the grid stay idle).  With an odd Hkv an item
  // is one (kv head, split) per wave.  Within a unit the split index is rotated by the unit pair,
  // which spreads each split index (the window splits in particular, which carry less work)
  // evenly over the XCDs.  Computed by the whole wave from the device lengths (lane i handles
  // sequences i, i + 64, ...; for batches up to 64 the lengths are loaded once).  Returns false
  // for a wave past the last item.  Results are wave-uniform (read with readlane), so everything
  // derived from them stays scalar; len_out is the sequence's length as stored in seq_lens (not
  // clamped).
  static __device__ __forceinline__ bool plan_wave(const KvqAttnArgs &a, int wave, int &b_out, int &kvh_out,
                                                   int &split_out, int &S_out, int &len_out) {
    const int lane = threadIdx.x, B = a.cache.batch, R = a.R;
    const int lmax = a.max_len - a.len_plus1;
    int raw0 = 0;  // lane's length in the first chunk of 64 sequences
    auto qpages_of = [&](int raw) {
      int L = raw < 0 ? 0 : (raw > lmax ? lmax : raw);
      L += a.len_plus1;
      return ((L > R ? L - R : 0) + KVQ_PAGE - 1) / KVQ_PAGE;
    };
    double Q = 0.0;  // exact: a sum of integers below 2^53
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int raw = b0 + lane < B ? a.seq_lens[b0 + lane] : 0;
      if (b0 == 0) raw0 = raw;
      double v = b0 + lane < B ? (double)qpages_of(raw) : 0.0;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
      Q += v;
    }
    const bool paired = (a.Hkv & 1) == 0;
    const int item = paired ? 8 * (wave >> 4) + (wave & 7) : wave;
    const int member = paired ? (wave >> 3) & 1 : 0;
    const int per_seq = paired ? a.Hkv / 2 : a.Hkv;  // items per split index of a sequence
    int base = 0;  // items of the sequences before this chunk of 64
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int b = b0 + lane;
      const int raw = b0 == 0 ? raw0 : (b < B ? a.seq_lens[b] : 0);
      const int Sb = b < B ? a.ws + plan_qsplits(a, qpages_of(raw), Q) : 0;
      const int nw_b = per_seq * Sb;
      int incl = nw_b;  // inclusive prefix over the lanes
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
      }
      const int lo = base + incl - nw_b;
      const uint64_t m = __ballot(b < B && item >= lo && item < lo + nw_b);
      if (m) {
        const int src = __ffsll((unsigned long long)m) - 1;
        const int bb = __builtin_amdgcn_readlane(b, src), S = __builtin_amdgcn_readlane(Sb, src);
        const int idx = item - __builtin_amdgcn_readlane(lo, src);
        const int kvh = paired ? 2 * (idx / S) + member : idx / S;
        const int unit = bb * a.Hkv + kvh;
        b_out = bb;
        kvh_out = kvh;
        split_out = (idx % S + unit / 2) % S;
        S_out = S;
        len_out = __builtin_amdgcn_readlane(raw, src);
        return true;
      }
      base += __builtin_amdgcn_readlane(incl, 63);
    }
    return false;
  }

  static __device__ __forceinline__ void run(const KvqAttnArgs &args, uint8_t *smem) {
    float *lds = reinterpret_cast<float *>(smem);
    const int lane = threadIdx.x;
    const int Hkv = args.Hkv;
    int b, kvh, split, S, Lraw;
    if (!plan_wave(args, (int)blockIdx.x, b, kvh, split, S, Lraw)) return;
    const KvqLayout &lay = args.lay;
    const int R = args.R;
    // a length outside [0, max_len] is clamped (reported once per unit, by its split 0); in a decode
    // step the lengths are those before the appended token: [0, max_len - 1]
    // (the same clamp as the plan's)
    int L = Lraw;
    const int lmax = args.max_len - args.len_plus1;
    kvq_raise(args.cache, split == 0 && (L < 0 || L > lmax), KVQ_DEV_LENGTH);
    L = L < 0 ? 0 : (L > lmax ? lmax : L);
    const int Lb = L;  // decode step: length before the step
    L += args.len_plus1;
    const int nq = L > R ? L - R : 0;
    const int nw = L < R ? L : R;
    const int wpages = (nw + KVQ_PAGE - 1) / KVQ_PAGE;
    // Window splits first, then quantized splits.
    const bool win_split = split < args.ws;
    int wv0 = 0, wv1 = 0;
    if (win_split) {
      wv0 = split * KVQ_WIN_PAGES;
      wv1 = wv0 + KVQ_WIN_PAGES < wpages ? wv0 + KVQ_WIN_PAGES : wpages;
    }

    // Exchange buffers start zeroed: rows no lane writes (heads beyond G) then stay finite.
    const uint32_t xbase = (uint32_t)(uintptr_t)smem + XCHG_OFF;
#pragma unroll
    for (int v = 0; v < NVG; ++v) {
      const uint32_t addr = xbase + KVQ_XCHG_BYTES * v + 16 * lane;
      asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(u32x4{0u, 0u, 0u, 0u}));
    }

    Ctx cx;
    init_ctx(cx, args.sigma_u, xbase);
    const int hq0 = kvh * G;
    St st;
#pragma unroll
    for (int m = 0; m < 8; ++m) st.acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      st.m[hb] = -__builtin_inff();
      st.l[hb] = 0.f;
#pragma unroll
      for (int v = 0; v < NVG; ++v) st.z[hb][v] = 0.f;
    }

    if (win_split) {
      // Window pages: raw (and unrotated) keys, scored with the raw, unscaled query operand.
      float ow[G][2];
#pragma unroll
      for (int h = 0; h < G; ++h) ow[h][0] = ow[h][1] = 0.f;
      // Fused step: the new token sits in ring slot s_new; it is read from k_new / v_new (this
      // launch writes the slot), and the split holding that slot also does the append.
      int s_new = -1;
      bool evicted = false;
      const uint8_t *knew = nullptr, *vnew = nullptr;
      if (args.fuse) {
        s_new = Lb % R;
        knew = args.k_new + ((size_t)b * Hkv + kvh) * KVQ_D * 2;
        vnew = args.v_new + ((size_t)b * Hkv + kvh) * KVQ_D * 2;
        if (split == s_new / (KVQ_WIN_PAGES * KVQ_PAGE)) evicted = fused_append(args, smem, b, kvh, Lb, s_new);
      }
      if (wv1 > wv0) {
        stage_q(args, lds, b, hq0, false);
        build_q(cx, lds, false);
        const size_t win_off = ((size_t)b * Hkv + kvh) * R * KVQ_D * (args.kv_f32 ? 4 : 2);
        const int wend = (wv1 * KVQ_PAGE) < nw ? wv1 * KVQ_PAGE : nw;
        for (int w = wv0 * KVQ_PAGE; w < wend; w += 32) {
          if (args.kv_f32)
            window_chunk<true>(cx, st, ow, args.cache.k_win + win_off, args.cache.v_win + win_off, w, wend);
          else
            window_chunk<false>(cx, st, ow, args.cache.k_win + win_off, args.cache.v_win + win_off, w, wend, s_new,
                                knew, vnew);
        }
      }
      if (evicted) {
        if (lay.kg == 32)
          evicted_pair<0>(args, cx, st, smem, b, hq0);
        else if (lay.kg == 64)
          evicted_pair<1>(args, cx, st, smem, b, hq0);
        else
          evicted_pair<2>(args, cx, st, smem, b, hq0);
        write_partial<PART_CODES>(args, cx, st, nullptr, lds, b, kvh, split, S);
        return;
      }
      if (args.kv_f32)
        write_partial<PART_WIN_VALU>(args, cx, st, ow, lds, b, kvh, split, S);
      else
        write_partial<PART_WIN_ACC>(args, cx, st, ow, lds, b, kvh, split, S);
      return;
    }

    // Quantized splits take full-page pairs round-robin: pair sq, sq + SQ, sq + 2 SQ, ... so that at
    // any moment the waves of one unit read neighbouring pairs.
    const int SQ = S - args.ws, sq = split - args.ws;
    // Fused step: the token leaving the window is stored and attended by the window split; the
    // quantized splits cover the tokens stored before the step.
    const int nqs = args.fuse ? (Lb > R ? Lb - R : 0) : nq;
    const int qpages_s = (nqs + KVQ_PAGE - 1) / KVQ_PAGE;
    const int full_pages = nqs / KVQ_PAGE;  // pages with all 16 tokens quantized
    const int tp = full_pages / 2;         // full pairs of this sequence
    // Pairs of full pages, next pairs prefetched while the current one is processed.  The 1-2
    // pages after the last full pair (an odd full page and/or the partial page) form one masked
    // pair; it goes to the split next in the rotation, whose cursor reaches it right after its
    // full pairs, so it streams through the same ring.
    const int npairs = tp > sq ? (tp - sq + SQ - 1) / SQ : 0;
    const bool tail = sq == tp % SQ && 2 * tp < qpages_s;
    if (npairs > 0 || tail) {
      int tail_va = 0, tail_vb = 0;
      if (tail) {
        const int p = 2 * tp;
        tail_va = (nqs - p * KVQ_PAGE) < KVQ_PAGE ? (nqs - p * KVQ_PAGE) : KVQ_PAGE;
        tail_vb = p + 1 < qpages_s ? ((nqs - (p + 1) * KVQ_PAGE) < KVQ_PAGE ? (nqs - (p + 1) * KVQ_PAGE) : KVQ_PAGE)
                                   : 0;
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
      if (lay.kg == 32)
        stream_pairs<0>(args, cx, st, smem, qr, b, kvh, sq, SQ, npairs, tail, tail_va, tail_vb);
      else if (lay.kg == 64)
        stream_pairs<1>(args, cx, st, smem, qr, b, kvh, sq, SQ, npairs, tail, tail_va, tail_vb);
      else
        stream_pairs<2>(args, cx, st, smem, qr, b, kvh, sq, SQ, npairs, tail, tail_va, tail_vb);
    }
    write_partial<PART_CODES>(args, cx, st, nullptr, lds, b, kvh, split, S);
  }

  // Pairs sq, sq + SQ, ... (npairs of them) of one unit through the wave's LDS ring of NPS page
  // slots: local page k (pair k / 2) lives in slot k mod NPS.  The first AHEAD pages are requested
  // up front; processing pair i first requests pages 2i + AHEAD and 2i + AHEAD + 1 (the slots of
  // pair i - 1, already read), then waits until those two are the only pages still in flight
  // behind pair i.  Requests follow a cursor that steps through the pairs in order (the parity of
  // every request site is fixed, so the cursor moves by constant strides), and the slot addresses
  // rotate through the ring, so the loop does no index arithmetic beyond those steps.
  // KS = log2(key group / 32).
  template <int KS>
  static __device__ __forceinline__ void stream_pairs(const KvqAttnArgs &args, Ctx &cx, St &st, uint8_t *smem,
                                                      const QRegs &qr, int b, int kvh, int sq,
                                                      int SQ, int npairs, bool tail, int tail_va, int tail_vb) {
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
    const size_t units = (size_t)args.cache.batch * Hkv;
    const size_t unit_idx = (size_t)b * Hkv + kvh;
    const size_t page_stride = units * rec;                  // contiguous: page p -> p + 1
    const size_t pair_step = 2 * (size_t)SQ * page_stride;   // contiguous: pair j -> j + SQ
    const uint8_t *unit_first = pages + unit_idx * rec;      // the unit's page 0
    const uint8_t *cur = unit_first + 2 * (size_t)sq * page_stride;
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
      if (k >= npages) {  // prologue filler: the unit's first page (always allocated), never read
        src = paged ? pages + (size_t)kvh * rec : unit_first;
      } else if (paged) {
        int e = tcur[(odd && !dup) ? 1 : 0];
        if ((uint32_t)e > (uint32_t)pool_last) {  // outside the pool: clamped and reported
          kvq_raise(args.cache, true, KVQ_DEV_TABLE_ENTRY);
          e = e < 0 ? 0 : pool_last;
        }
        src = pages + ((size_t)e * Hkv + kvh) * rec;
        if (odd) tcur += 2 * SQ;
      } else {
        src = (odd && !dup) ? cur + page_stride : cur;
        if (odd) cur += pair_step;
      }
      dma_page_buf(wslot, src, rec, loff, lane);
      wslot = next_slot(wslot);
    };
    // The prologue always issues AHEAD pages (fillers past the split's own pages), so the number
    // of DMAs in flight is fixed.
#pragma unroll
    for (int k = 0; k < AHEAD; ++k) issue((k & 1) != 0, k);
    if (!args.rotation) build_q_regs(cx, qr, args.q_f32);
    // Zero-point query sums per key group.
    float Qg[HB][4];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) Qg[hb][g] = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) Qg[hb][r >> KS] += cx.Qc[hb][r];
    }
    const RecOff ro = rec_offsets<KS>(cx, lay);
    constexpr bool FIRST_ODD = (AHEAD & 1) != 0;  // parity of page 2i + AHEAD
#if KVQ_SLOT_PRIO
    // With two waves per SIMD the dispatcher gives every SIMD one wave before any gets a second
    // (blocks 0 .. SIMDs - 1 first), and the older wave wins instruction arbitration: measured per
    // wave at the 32k batch-16 launch, the second waves ended ≈9 µs after the first and set the
    // kernel's end.  The second waves therefore issue at priority 1 for the first 5/8 of their
    // pairs (measured best of 0, 2/8, 4/8, 5/8, 6/8 and all: 86.6 µs against 93.0 µs).  Timing
    // only: which pages a wave reads, and so the result, does not change.
    const bool late = WPE == 2 && blockIdx.x >= 4 * KVQ_NUM_CUS;
    const int prio_until = (KVQ_SLOT_PRIO * npairs) / 8;
    if (late) __builtin_amdgcn_s_setprio(1);
#endif
    for (int i = 0; i < npairs; ++i) {
#if KVQ_SLOT_PRIO
      if (late && i == prio_until) __builtin_amdgcn_s_setprio(0);
#endif
      const int k0 = 2 * i + AHEAD;
      if (k0 + 1 < npages) {  // steady state: two requests, AHEAD pages stay in flight
        issue(FIRST_ODD, k0);
        issue(!FIRST_ODD, k0 + 1);
        wait_vmcnt<AHEAD * DMAS_PER_PAGE>();
      } else {  // the last pairs: at most one more request, then drain
        if (k0 < npages) issue(FIRST_ODD, k0);
        wait_vmcnt<0>();
      }
      PageData<KS> A, B;
      read_page_at(A, rslot, ro);
      rslot = next_slot(rslot);
      read_page_at(B, rslot, ro);
      rslot = next_slot(rslot);
      process_pair<KS, false>(cx, st, Qg, A, B, 16, 16);
    }
    if (tail) {  // its pages were requested with the others
      wait_vmcnt<0>();
      PageData<KS> A, B;
      read_page_at(A, rslot, ro);
      rslot = next_slot(rslot);
      read_page_at(B, rslot, ro);
      process_pair<KS, true>(cx, st, Qg, A, B, tail_va, tail_vb);
    }
    wait_vmcnt<0>();  // no DMA (fillers included) may still be writing the ring when the wave ends
  }

  // Reduce the state across lanes and write this split's partial result:
  // [m (log2 units), l, nsplits, 0, o[128]] per query head, o unnormalised, nsplits the number of
  // entries of the row that hold splits.
  // MODE: PART_CODES (quantized pages: value-code scales and zero-point sums apply),
  // PART_WIN_ACC (bf16 window: MFMA accumulators hold the output as is), PART_WIN_VALU (fp32
  // window: the output is in ow).
  static constexpr int PART_CODES = 0, PART_WIN_ACC = 1, PART_WIN_VALU = 2;
  template <int MODE>
  static __device__ __forceinline__ void write_partial(const KvqAttnArgs &args, const Ctx &cx, const St &st,
                                                       float (*ow)[2], float *lds, int b, int kvh, int split,
                                                       int nsplits) {
    constexpr bool WIN = MODE != PART_CODES;
    const int lane = threadIdx.x;
    const int hq0 = kvh * G;
    float lt[HB], zt[HB][NVG];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      lt[hb] = row16_sum(st.l[hb]);
#pragma unroll
      for (int v = 0; v < NVG; ++v) zt[hb][v] = WIN ? 0.f : row16_sum(st.z[hb][v]);
    }
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
    if (cx.col == 0 && cx.quad < HSN) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const int h = 4 * hb + cx.quad;
        hdr[h * 4 + 0] = st.m[hb] * cx.sig;  // log2 units
        hdr[h * 4 + 1] = lt[hb];
#pragma unroll
        for (int v = 0; v < NVG; ++v) hdr[h * 4 + 2 + v] = zt[hb][v];
      }
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
        dst[2] = (float)nsplits;  // entries [nsplits, splits) of the row are not written
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
