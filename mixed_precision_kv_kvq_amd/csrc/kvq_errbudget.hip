// Error-budget diagnostics of a quantized cache against the original keys and values.
// nalar.dev "Kuantisasi KV cache mengganggu attention melalui key dan value tersimpan":
// section "Error pada key masuk sebelum softmax" (a key error E_K shifts the scores by
// q E_K^T / sqrt(d) before the softmax), section "Error pada value masuk setelah bobot attention
// terbentuk" (a value error E_V moves the output by a E_V after the weights are formed), and
// section "Evaluasi harus sesuai dengan besaran yang ingin dipertahankan" (judge the attention
// quantities, not only reconstruction error); the nalar.dev tag page's entries on separate key
// and value error budgets.
#include "kvq_extras.h"

#pragma clang fp contract(off)

namespace {

__device__ __attribute__((always_inline)) inline void bf16x8(const uint4 w, float *x) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = kvq_bf16_bits_to_f32(ws[i] & 0xFFFFu);
    x[2 * i + 1] = kvq_bf16_bits_to_f32(ws[i] >> 16);
  }
}

__device__ inline float f16f(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

// Sum over the 16 lanes of a lane row, in every lane of the row: row rotations by 8, 4, 2, 1 (DPP,
// no LDS round trip).
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
__device__ inline float row16_sum(float v) {
#pragma unroll
  for (int sh = 8; sh >= 1; sh >>= 1) v += row_ror(v, sh);
  return v;
}

// Normalized 128-point Walsh-Hadamard transform of a row held as 8 channels [8c, 8c + 8) in
// each of the 16 lanes of a lane row (c = lane mod 16), fp32: butterflies in stage order 1, 2,
// 4 inside the lane, then 8, 16, 32, 64 across lanes c ^ 1, c ^ 2, c ^ 4, c ^ 8.  Every lane of
// the wave must take part (cross-lane reads); rows whose `apply` is false (the same in the 16
// lanes of the row) keep their values.
__device__ __attribute__((always_inline)) inline void row_wht(float *x, int c, bool apply) {
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = x[e];
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if ((e & h) == 0) {
        const float u = y[e], v = y[e + h];
        y[e] = u + v;
        y[e + h] = u - v;
      }
    }
  }
#pragma unroll
  for (int lx = 1; lx < 16; lx <<= 1) {
    const bool upper = (c & lx) != 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __shfl_xor(y[e], lx);
      y[e] = upper ? p - y[e] : y[e] + p;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = apply ? y[e] * (float)KVQ_WHT_C : x[e];
}

// The same transform for a row held as channels 2l, 2l + 1 in lane l of the wave: stage 1 inside
// the lane, stages 2 .. 64 across lanes l ^ (h / 2).
__device__ __attribute__((always_inline)) inline void pair_wht(float &x0, float &x1, int lane) {
  {
    const float u = x0, v = x1;
    x0 = u + v;
    x1 = u - v;
  }
#pragma unroll
  for (int h = 2; h < KVQ_D; h <<= 1) {
    const int lx = h >> 1;
    const float p0 = __shfl_xor(x0, lx), p1 = __shfl_xor(x1, lx);
    const bool upper = (lane & lx) != 0;
    x0 = upper ? p0 - x0 : x0 + p0;
    x1 = upper ? p1 - x1 : x1 + p1;
  }
  x0 *= (float)KVQ_WHT_C;
  x1 *= (float)KVQ_WHT_C;
}

// The bit planes of a code width b (1..6 or 8), widest first: at most two (w1 = 0: one plane).
// Plane 0 sits at offset 0 of a code area with its fields at bit 0 of the code; plane 1 at byte
// 256 w0 with its fields at bit w0.
struct EbPlanes {
  int w0, w1;
};
__device__ __forceinline__ EbPlanes eb_planes(int b) {
  const int w0 = b == 8 ? 8 : (b >= 4 ? 4 : (b >= 2 ? 2 : 1));
  return {w0, b - w0};
}
// Both 16-bit halves of pair slot u of a slot of one plane (width w, the slot's bytes at s): the
// w-bit fields at bit u w mod 16 of word u w / 16 of each half, moved to bit 0.
__device__ __forceinline__ uint32_t plane_pair(const uint8_t *s, int u, int w) {
  const int bit = u * w;
  const uint32_t word = *reinterpret_cast<const uint32_t *>(s + 4 * (bit >> 4));
  return (word >> (bit & 15)) & (((1u << w) - 1u) * 0x00010001u);
}
// Pair slot u of slot `slot` of a code area, both planes combined: two codes, one per 16-bit half.
// K: slot 16 j + n holds token n's channel octet j of each 32-channel chunk kc, pair slot
// u = 4 kc + i its channels 32 kc + 8 j + 2 i (low half) and + 1 (high half).  V: slot 16 jj + c16
// holds channel 16 m + c16 of tokens 4 jj .. 4 jj + 3, pair slot u = 8 i + m its tokens 4 jj + 2 i
// (low half) and + 1 (high half).
__device__ __forceinline__ uint32_t eb_pair(const uint8_t *area, int slot, int u, EbPlanes P) {
  uint32_t v = plane_pair(area + slot * 4 * P.w0, u, P.w0);
  if (P.w1) v |= plane_pair(area + 256 * P.w0 + slot * 4 * P.w1, u, P.w1) << P.w0;
  return v;
}

// The reconstruction of 8 channels [8c, 8c + 8) of token n of a page record staged in LDS (keys
// or values), zero + code * scale rounded once to fp32 (fused multiply-add).
template <bool KEYS>
__device__ __attribute__((always_inline)) inline void decode8(const KvqLayout &lay, EbPlanes P, const uint8_t *rs,
                                                              int n, int c, float *xh) {
  const uint32_t m = reinterpret_cast<const uint32_t *>(rs + (KEYS ? lay.k_meta_off : lay.v_meta_off))
      [kvq_meta_dword(KEYS ? lay.nkg : lay.nvg, n, (8 * c) / (KEYS ? lay.kg : lay.vg))];
  const float zero = f16f(m >> 16), scale = f16f(m & 0xFFFF);
  uint32_t code[8];
  if (KEYS) {  // channels 8 c + 2 i, + 1: pair slot 4 (c / 4) + i of slot 16 (c mod 4) + n
    const uint8_t *area = rs + lay.k_codes_off;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t v = eb_pair(area, 16 * (c & 3) + n, 4 * (c >> 2) + i, P);
      code[2 * i] = v & 0xFFFFu;
      code[2 * i + 1] = v >> 16;
    }
  } else {  // channel 8 c + e: slot 16 (n / 4) + 8 (c mod 2) + e, pair slot 8 ((n mod 4) / 2) + c / 2
    const uint8_t *area = rs + lay.v_codes_off;
    const int hs = 16 * (n & 1);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      code[e] = (eb_pair(area, 16 * (n >> 2) + 8 * (c & 1) + e, 8 * ((n & 3) >> 1) + (c >> 1), P) >> hs) & 0xFFFFu;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) xh[e] = __builtin_fmaf((float)code[e], scale, zero);
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;
typedef short eb_s8 __attribute__((__vector_size__(8 * sizeof(short))));  // 8 bf16: 16x16x32 operand
typedef short eb_s4 __attribute__((ext_vector_type(4)));                   // 4 bf16: 16x16x16 operand
typedef float eb_f4 __attribute__((ext_vector_type(4)));
typedef uint32_t eb_u4 __attribute__((ext_vector_type(4)));
typedef uint32_t eb_u2 __attribute__((ext_vector_type(2)));
typedef __bf16 eb_bf2 __attribute__((ext_vector_type(2)));
typedef uint16_t eb_h2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  eb_bf2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ eb_s8 pack8s(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3) {
  eb_u4 u;
  u[0] = a0;
  u[1] = a1;
  u[2] = a2;
  u[3] = a3;
  return __builtin_bit_cast(eb_s8, u);
}
__device__ __forceinline__ eb_s4 pack4s(uint32_t a0, uint32_t a1) {
  eb_u2 u;
  u[0] = a0;
  u[1] = a1;
  return __builtin_bit_cast(eb_s4, u);
}
__device__ __forceinline__ float bf_lo(uint32_t p) { return __builtin_bit_cast(float, p << 16); }
__device__ __forceinline__ float bf_hi(uint32_t p) { return __builtin_bit_cast(float, p & 0xFFFF0000u); }
// hi and lo bf16 parts of two fp32 values (x = hi + lo to about 2^-16 relative)
__device__ __forceinline__ void split2(float x0, float x1, uint32_t &hi, uint32_t &lo) {
  hi = pk_bf16(x0, x1);
  lo = pk_bf16(x0 - bf_lo(hi), x1 - bf_hi(hi));
}
__device__ __forceinline__ float row16_max(float v) {
#pragma unroll
  for (int sh = 8; sh >= 1; sh >>= 1) v = __builtin_fmaxf(v, row_ror(v, sh));
  return v;
}

// A code of b bits read as a bf16 bit pattern is code * 2^-133 (c < 256).

constexpr int EB_WAVES = 8;
constexpr int EB_K16 = (256 * 8 + 64 * 4) / 16;  // largest key part of a record, 16-byte units
constexpr int EB_V16 = (256 * 8 + 64 * 2) / 16;  // largest value part
constexpr float EB_Q = 0x1p100f;                 // query operand scale
// Rows staged in LDS are 17 x 16 bytes apart: the 16 positions of a B operand (same channels), the
// 16 octets of a row, and 4 positions x 16 channels all fall in distinct banks, and every offset
// within a page is a constant added to a per-lane base.
constexpr int EB_ROW16 = 17;

// Work items: one workgroup of EB_WAVES waves per (group of HS <= 4 query heads of one kv head and
// sequence, range): range `split` of S near-equal ranges of the sequence's pages.  The head groups
// of a range run on workgroups 8 apart (one XCD), so the second to read a page finds it in that
// XCD's L2.  Wave w of an item takes pages p0 + w, p0 + w + EB_WAVES, ...: a page's original rows
// and record part are loaded while the wave computes the page before, then stored to the wave's
// LDS region.
//
// Workspace: one item of EB_W_ITEM floats per (kv head unit, head group, range), then the scores
// [batch][query head][max_len rounded up to 16][2] (exact, quantized; dot units) that pass 1
// writes for pass 2.  An item holds the pass-1 statistics of each head {M0, Z0, M1, Z1,
// max |ds|, sum ds^2}, the key reconstruction sums {sum e^2, max |e|, sum k^2}, then the pass-2
// sums [sum][head][channel] of a V, a V_hat, a' V, a' V_hat, the total variation of each head and
// the value reconstruction sums.
constexpr int EB_W_STATS = 0;
constexpr int EB_W_KREC = 24;
constexpr int EB_W_SUMS = 32;
constexpr int EB_W_TV = EB_W_SUMS + 4 * 4 * KVQ_D;
constexpr int EB_W_VREC = EB_W_TV + 4;
constexpr int EB_W_ITEM = (EB_W_VREC + 4 + 31) / 32 * 32;  // whole 128-byte lines

// Positions per (sequence, query head) row of the stored scores: a whole number of pages, so each
// page's 16 scores of a head are one aligned 128-byte segment.
__host__ __device__ inline size_t eb_score_stride(int64_t max_len) { return (size_t)((max_len + 15) / 16) * 16; }

struct EbItem {
  int unit, grp, split, b, h, hq0, L, nq, pbeg, pend;
  float *ws;
};
// workgroup -> item: work unit wu = unit S + range; the head groups of wu at blocks
// 8 ngrp (wu / 8) + 8 grp + wu mod 8.  False for the padding after the last group of 8 work units.
template <int HS>
__device__ __forceinline__ bool eb_item(const KvqErrArgs &a, EbItem &it) {
  const int Hkv = a.Hkv, g = a.Hq / a.Hkv, ngrp = g / HS, S = a.splits;
  const int blk = blockIdx.x / (8 * ngrp), rem = blockIdx.x % (8 * ngrp);
  it.grp = rem / 8;
  const int wu = 8 * blk + rem % 8;
  if (wu >= a.B * Hkv * S) return false;
  it.unit = wu / S;
  it.split = wu % S;
  it.b = it.unit / Hkv;
  it.h = it.unit % Hkv;
  it.hq0 = it.h * g + it.grp * HS;
  it.ws = a.ws + (size_t)((it.unit * ngrp + it.grp) * S + it.split) * EB_W_ITEM;
  int L = (int)a.seq_lens[it.b];
  L = L < 0 ? 0 : ((int64_t)L > a.max_len ? (int)a.max_len : L);
  int nq = L > a.R ? L - a.R : 0;
  const int64_t cap_tokens = (a.cache.paged ? (int64_t)a.cache.mbps : a.cache.pages_per_seq) * KVQ_PAGE;
  if ((int64_t)nq > cap_tokens) nq = (int)cap_tokens;
  it.L = L;
  it.nq = nq;
  const int npages = (L + KVQ_PAGE - 1) / KVQ_PAGE;
  const int per = (npages + S - 1) / S;
  it.pbeg = it.split * per < npages ? it.split * per : npages;
  it.pend = it.pbeg + per < npages ? it.pbeg + per : npages;
  return true;
}

// DMA of bytes [from, from + 16 n16) of page pg's record into LDS at dst (per wave; every lane of
// the wave takes part, nothing for a page without quantized positions).
__device__ __forceinline__ void eb_load_rec(const KvqErrArgs &a, const EbItem &it, int pg, int from, int n16,
                                            uint32_t dst, int lane, int max16) {
  if (pg * KVQ_PAGE >= it.nq) return;
  const int64_t rec_idx = kvq_record_index_dev(a.cache, a.Hkv, it.b, it.h, pg);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.cache.pages + (size_t)rec_idx * a.lay.record + from), 0, 16 * n16, 0x00020000);
  for (int i = 0; i < (max16 + 63) / 64; ++i) {
    if (64 * i < n16 && lane + 64 * i < n16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(size_t)(dst + 1024u * i), 16, 16 * (lane + 64 * i), 0,
                                               0, 0);
  }
}

// PASS 1, scores and their statistics.  Scores on MFMA (16x16x32 bf16): the query, scaled by 2^100
// and split into bf16 hi and lo parts, is the A operand (row 4 hs + j: head hs restricted to
// 32-channel chunk j); the B operand is the page's original keys (exact bf16) for the exact scores
// and its key codes (code * 2^-133) for the quantized ones, so D row 4 q + r of lane 16 q + t holds
// head q's dot with chunk r of token t.  The quantized score applies the token's group scales and
// zero points: s' = sum_r scale_r (q . c)_r + sum_g zero_g sum(q over g).  With rotated keys the
// code scores use the rotated query (the normalized transform is orthogonal); window tokens are
// stored exact (s' = s).  Lane 16 q + t then holds both scores of token t for head q: written to the
// workspace, and folded into online maxima and sums (log2 units) and the score-error statistics,
// merged over the 16 lanes of a head and the waves.  Head group 0 also takes the key
// reconstruction errors: from the code and key operands of the score contraction (32 channels of
// one position per lane), or, with rotated keys, from whole rows rotated back (8 channels of a
// position per lane).
template <int HS>
__global__ __launch_bounds__(64 * EB_WAVES, 4) void kvq_eb_scores_kernel(KvqErrArgs a) {  // two workgroups per CU
  __shared__ float red[EB_WAVES][6 * HS];
  __shared__ float ured[EB_WAVES][3];
  __shared__ float qg[HS][4];                    // sums of the code query over each key group
  __shared__ uint4 recs[EB_WAVES][2][EB_K16];    // key parts of page records (the next one lands meanwhile)
  __shared__ uint4 rows[EB_WAVES][KVQ_PAGE * EB_ROW16];  // the page's original key rows
  // before the page loop: the group's queries (raw, and the one the codes are scored with)
  float(*qs)[HS][KVQ_D] = reinterpret_cast<float(*)[HS][KVQ_D]>(&rows[0][0]);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: page loop and record addresses in SGPRs
  const int r = lane >> 4, c = lane & 15;  // element layout: row r, 8 channels [8c, 8c + 8)
  const int q = lane >> 4, t = lane & 15;  // score layout: head q, token t
  EbItem it;
  if (!eb_item<HS>(a, it)) return;
  const int b = it.b, h = it.h, L = it.L, nq = it.nq, pbeg = it.pbeg, pend = it.pend;
  {
    const int raw = (int)a.seq_lens[b];
    kvq_raise(a.cache, it.hq0 == 0 && it.split == 0 && (raw < 0 || (int64_t)raw > a.max_len), KVQ_DEV_LENGTH);
  }
  const bool krec = it.grp == 0;
  const float ninf = -__builtin_inff();
  const KvqLayout &lay = a.lay;
  const EbPlanes KP = eb_planes(lay.kb);
  const bool qlive = q < HS;  // score-layout lanes of a head of the group

  // ---- queries: raw and code-scoring (rotated when keys are) rows, and the group sums ----
  if (w == 0) {
    float x[8];
    if (r < HS) {
      const size_t qrow = ((size_t)b * a.Hq + it.hq0 + r) * KVQ_D + 8 * c;
      if (a.q_f32) {
        const float4 *qp = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.q) + qrow);
        const float4 u0 = qp[0], u1 = qp[1];
        x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w;
        x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
      } else {
        bf16x8(*reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a.q) + qrow), x);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    float xr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) xr[e] = x[e];
    row_wht(xr, c, a.rotation != 0);  // every lane takes part
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) part += xr[e];
    // sum over the lanes of one key group (kg / 8 lanes: 4, 8 or 16)
    for (int sh = 1; sh < lay.kg / 8; sh <<= 1) part += __shfl_xor(part, sh);
    if (r < HS) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qs[0][r][8 * c + e] = x[e];
        qs[1][r][8 * c + e] = xr[e];
      }
      if ((8 * c) % lay.kg == 0) qg[r][(8 * c) / lay.kg] = part;
    }
  }
  __syncthreads();
  // A operands of the score contractions: row 4 hs + j = head hs restricted to chunk j, so the
  // operand of chunk kc is the lane's data where kc = j and zero elsewhere (applied per page).
  // qd[set][part]: set 0 the raw query, 1 the code-scoring one; parts hi and lo (lo = 0 for a bf16
  // query scored against unrotated codes).
  eb_u4 qd[2][2];
  float qgl[4];
  const int jrow = lane & 3;  // the chunk of the lane's A row
  const bool lo0 = a.q_f32 != 0, lo1 = a.q_f32 != 0 || a.rotation != 0;
  {
    const int rho = lane & 15, hs = rho >> 2, oct = lane >> 4;
#pragma unroll
    for (int set = 0; set < 2; ++set) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v0 = hs < HS ? qs[set][hs < HS ? hs : 0][32 * jrow + 8 * oct + 2 * i] * EB_Q : 0.f;
        const float v1 = hs < HS ? qs[set][hs < HS ? hs : 0][32 * jrow + 8 * oct + 2 * i + 1] * EB_Q : 0.f;
        uint32_t hi, lo;
        split2(v0, v1, hi, lo);
        qd[set][0][i] = hi;
        qd[set][1][i] = lo;
      }
    }
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) qgl[gi] = (qlive && gi < lay.nkg) ? qg[qlive ? q : 0][gi] : 0.f;
  }
  __syncthreads();  // the queries' LDS becomes page rows

  // the next page's rows in flight: pk_i = this lane's 8 channels of position 4 i + r (clamped to
  // L - 1 on the last page), from a uniform page base and a 32-bit per-lane offset
  const uint32_t row_elems = (uint32_t)a.Hkv * KVQ_D;  // elements between consecutive positions
  uint4 pk0, pk1, pk2, pk3;
  auto load_rows = [&](int pg) __attribute__((always_inline)) {
    const int t0 = pg * KVQ_PAGE;
    const uint16_t *kp = a.k_ref + ((size_t)b * a.max_len + (size_t)t0) * row_elems + (size_t)h * KVQ_D;
    const int last = L - 1 - t0;
    auto off = [&](int i) { return (uint32_t)(4 * i + r < last ? 4 * i + r : last) * row_elems + 8 * c; };
    pk0 = *reinterpret_cast<const uint4 *>(kp + off(0));
    pk1 = *reinterpret_cast<const uint4 *>(kp + off(1));
    pk2 = *reinterpret_cast<const uint4 *>(kp + off(2));
    pk3 = *reinterpret_cast<const uint4 *>(kp + off(3));
  };
  auto store_rows = [&]() __attribute__((always_inline)) {
    rows[w][(0 + r) * EB_ROW16 + c] = pk0;
    rows[w][(4 + r) * EB_ROW16 + c] = pk1;
    rows[w][(8 + r) * EB_ROW16 + c] = pk2;
    rows[w][(12 + r) * EB_ROW16 + c] = pk3;
  };
  const int kpart16 = lay.v_codes_off / 16;  // the record's key codes and key metadata
  auto load_rec = [&](int pg, int buf) __attribute__((always_inline)) {
    eb_load_rec(a, it, pg, 0, kpart16, (uint32_t)(uintptr_t)&recs[w][buf][0], lane, EB_K16);
  };
  const float sl2 = a.scale * 1.4426950408889634f;  // softmax scale in log2 units
  const uint8_t *krow = reinterpret_cast<const uint8_t *>(rows[w]);
  float2 *scores = reinterpret_cast<float2 *>(a.ws + (size_t)a.B * a.Hkv * (a.Hq / a.Hkv / HS) * a.splits * EB_W_ITEM) +
                   ((size_t)b * a.Hq + it.hq0 + (qlive ? q : 0)) * eb_score_stride(a.max_len);

  float m0 = ninf, z0 = 0.f, m1 = ninf, z1 = 0.f, ds_max = 0.f, ds_sq = 0.f;
  float ek_sq = 0.f, ek_max = 0.f, k_sq = 0.f;  // key reconstruction error (head group 0)
  int buf = 0;
  if (pbeg + w < pend) {
    load_rows(pbeg + w);
    load_rec(pbeg + w, 0);
  }
  for (int pg = pbeg + w; pg < pend; pg += EB_WAVES, buf ^= 1) {
    const int t0 = pg * KVQ_PAGE;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this page's rows and record have landed
    store_rows();
    if (pg + EB_WAVES < pend) {
      load_rows(pg + EB_WAVES);
      load_rec(pg + EB_WAVES, buf ^ 1);
    }
    const uint8_t *rs = reinterpret_cast<const uint8_t *>(recs[w][buf]);
    // exact and quantized dots (dot units, no softmax scale) of token t of the page for head q
    float s0, s1;
    {
      eb_f4 D0 = {0.f, 0.f, 0.f, 0.f}, D1 = {0.f, 0.f, 0.f, 0.f};
      const int n = lane & 15, oct = lane >> 4;  // B operand: token n, channel octet oct of each chunk
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        uint32_t mk = kc == jrow ? ~0u : 0u;
        asm volatile("" : "+v"(mk));  // keeps the masked operands in the loop (no 48 registers of zeros)
        const eb_u4 kv = *reinterpret_cast<const eb_u4 *>(krow + 16 * (n * EB_ROW16 + 4 * kc + oct));
        const eb_s8 bk = __builtin_bit_cast(eb_s8, kv);
        D0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(eb_s8, qd[0][0] & mk), bk, D0, 0, 0, 0);
        if (lo0) D0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(eb_s8, qd[0][1] & mk), bk, D0, 0, 0, 0);
      }
      s0 = (D0[0] + D0[1] + D0[2] + D0[3]) * 0x1p-100f;
      s1 = s0;
      if (t0 < nq) {  // the page holds quantized tokens
        const uint8_t *kcodes = rs + lay.k_codes_off;
        const uint32_t *kmn = reinterpret_cast<const uint32_t *>(rs + lay.k_meta_off) + n * lay.nkg;
        const bool kerr = krec && !a.rotation && t0 + n < nq;  // errors in the operand layout (lane: token n)
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          uint32_t mk = kc == jrow ? ~0u : 0u;
          asm volatile("" : "+v"(mk));
          const uint32_t p0 = eb_pair(kcodes, 16 * oct + n, 4 * kc + 0, KP), p1 = eb_pair(kcodes, 16 * oct + n, 4 * kc + 1, KP);
          const uint32_t p2 = eb_pair(kcodes, 16 * oct + n, 4 * kc + 2, KP), p3 = eb_pair(kcodes, 16 * oct + n, 4 * kc + 3, KP);
          const eb_s8 bc = pack8s(p0, p1, p2, p3);
          D1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(eb_s8, qd[1][0] & mk), bc, D1, 0, 0, 0);
          if (lo1) D1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(eb_s8, qd[1][1] & mk), bc, D1, 0, 0, 0);
          if (kerr) {  // channels 32 kc + 8 oct + e of token n: one key group (groups of 32 or more)
            const uint32_t mm = kmn[(32 * kc) / lay.kg];
            const float ksc = f16f(mm & 0xFFFF), kz = f16f(mm >> 16);
            const eb_u4 kv = *reinterpret_cast<const eb_u4 *>(krow + 16 * (n * EB_ROW16 + 4 * kc + oct));
            const uint32_t pc[4] = {p0, p1, p2, p3};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint32_t cw = (e & 1) ? (pc[e >> 1] >> 16) : (pc[e >> 1] & 0xFFFFu);
              const uint32_t kw = (e & 1) ? (kv[e >> 1] & 0xFFFF0000u) : (kv[e >> 1] << 16);
              const float x = __builtin_bit_cast(float, kw);
              const float err = __builtin_fmaf((float)cw, ksc, kz) - x;
              ek_sq = __builtin_fmaf(err, err, ek_sq);
              ek_max = __builtin_fmaxf(ek_max, __builtin_fabsf(err));
              k_sq = __builtin_fmaf(x, x, k_sq);
            }
          }
        }
        if (t0 + t < nq) {
          const uint32_t *km = reinterpret_cast<const uint32_t *>(rs + lay.k_meta_off) + t * lay.nkg;
          float acc = 0.f;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) acc = __builtin_fmaf(D1[rr] * 0x1p33f, f16f(km[(32 * rr) / lay.kg] & 0xFFFF), acc);
#pragma unroll
          for (int gi = 0; gi < 4; ++gi)
            if (gi < lay.nkg) acc = __builtin_fmaf(f16f(km[gi] >> 16), qgl[gi], acc);
          s1 = acc;
        }
      }
    }
    if (qlive && t0 + t < L) {
      scores[t0 + t] = make_float2(s0, s1);
      const float x0 = s0 * sl2, x1 = s1 * sl2;
      const float n0 = __builtin_fmaxf(m0, x0), n1 = __builtin_fmaxf(m1, x1);
      z0 = z0 * __builtin_amdgcn_exp2f(m0 - n0) + __builtin_amdgcn_exp2f(x0 - n0);
      z1 = z1 * __builtin_amdgcn_exp2f(m1 - n1) + __builtin_amdgcn_exp2f(x1 - n1);
      m0 = n0;
      m1 = n1;
      const float ds = (s1 - s0) * a.scale;
      ds_max = __builtin_fmaxf(ds_max, __builtin_fabsf(ds));
      ds_sq = __builtin_fmaf(ds, ds, ds_sq);
    }
    if (krec && a.rotation && t0 < nq) {  // rotated keys: whole rows rotated back, 8 channels of positions 4 i + r
#pragma unroll 1
      for (int ii = 0; ii < 4; ++ii) {
        const int n = 4 * ii + r;
        const bool quant = t0 + n < nq;  // (positions past L are not quantized either)
        float k[8], kh[8];
        bf16x8(rows[w][n * EB_ROW16 + c], k);
#pragma unroll
        for (int e = 0; e < 8; ++e) kh[e] = 0.f;
        if (quant) decode8<true>(lay, KP, rs, n, c, kh);
        if (a.rotation) row_wht(kh, c, quant);  // back to the original domain
        if (quant) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float err = kh[e] - k[e];
            ek_sq = __builtin_fmaf(err, err, ek_sq);
            ek_max = __builtin_fmaxf(ek_max, __builtin_fabsf(err));
            k_sq = __builtin_fmaf(k[e], k[e], k_sq);
          }
        }
      }
    }
  }
  // merge the 16 tokens of a head (one lane row), then the waves
  {
    const float M0 = row16_max(m0), M1 = row16_max(m1);
    const float Z0 = row16_sum(M0 == ninf ? 0.f : z0 * __builtin_amdgcn_exp2f(m0 - M0));
    const float Z1 = row16_sum(M1 == ninf ? 0.f : z1 * __builtin_amdgcn_exp2f(m1 - M1));
    const float dmx = row16_max(ds_max), dsq = row16_sum(ds_sq);
    if (qlive && t == 0) {
      red[w][6 * q + 0] = M0;
      red[w][6 * q + 1] = Z0;
      red[w][6 * q + 2] = M1;
      red[w][6 * q + 3] = Z1;
      red[w][6 * q + 4] = dmx;
      red[w][6 * q + 5] = dsq;
    }
  }
  if (krec) {
    for (int off = 1; off <= 32; off <<= 1) {
      ek_sq += __shfl_xor(ek_sq, off);
      k_sq += __shfl_xor(k_sq, off);
      ek_max = __builtin_fmaxf(ek_max, __shfl_xor(ek_max, off));
    }
    if (lane == 0) {
      ured[w][0] = ek_sq;
      ured[w][1] = ek_max;
      ured[w][2] = k_sq;
    }
  }
  __syncthreads();
  if (w == 0 && lane < HS) {  // lane j: head j's statistics over the item's pages
    const int j = lane;
    float M0 = ninf, M1 = ninf;
    for (int i = 0; i < EB_WAVES; ++i) {
      M0 = __builtin_fmaxf(M0, red[i][6 * j + 0]);
      M1 = __builtin_fmaxf(M1, red[i][6 * j + 2]);
    }
    float Z0 = 0.f, Z1 = 0.f, dmx = 0.f, dsq = 0.f;
    for (int i = 0; i < EB_WAVES; ++i) {
      if (red[i][6 * j + 0] != ninf) Z0 += red[i][6 * j + 1] * __builtin_amdgcn_exp2f(red[i][6 * j + 0] - M0);
      if (red[i][6 * j + 2] != ninf) Z1 += red[i][6 * j + 3] * __builtin_amdgcn_exp2f(red[i][6 * j + 2] - M1);
      dmx = __builtin_fmaxf(dmx, red[i][6 * j + 4]);
      dsq += red[i][6 * j + 5];
    }
    float *st = it.ws + EB_W_STATS + 6 * j;
    st[0] = M0;
    st[1] = Z0;
    st[2] = M1;
    st[3] = Z1;
    st[4] = dmx;
    st[5] = dsq;
  }
  if (krec && w == 0 && lane == 0) {
    float e0 = 0.f, e1 = 0.f, e2 = 0.f;
    for (int i = 0; i < EB_WAVES; ++i) {
      e0 += ured[i][0];
      e1 = __builtin_fmaxf(e1, ured[i][1]);
      e2 += ured[i][2];
    }
    it.ws[EB_W_KREC + 0] = e0;
    it.ws[EB_W_KREC + 1] = e1;
    it.ws[EB_W_KREC + 2] = e2;
  }
}

// PASS 2, weights and weighted sums.  The maxima and sums of all ranges merged; the weights a
// (exact keys) and a' (quantized keys) from the stored scores, their total variation, and the four
// weighted sums on MFMA (16x16x16 bf16, k = the page's 16 tokens): A rows 8 set + 4 part + q hold
// the weights of set a / a' (hi and lo parts) of head q, through a per-wave LDS exchange buffer;
// B is the original values (exact bf16: a V, a' V) or the value codes (a V_hat, a' V_hat;
// A = weight * scale * 2^64, window tokens take their exact values as B with A = weight * 2^-69,
// so every product carries 2^-69), plus the weighted zero points.  The B operands of the original
// values are read as 16-bit elements from the staged rows.  The range's sums go to the workspace: the weights
// are final, so the ranges' sums add.  The last head group also takes the value reconstruction
// errors, in the same layout as the B operands (4 positions x 8 channels per lane).
template <int HS>
__global__ __launch_bounds__(64 * EB_WAVES) void kvq_eb_sums_kernel(KvqErrArgs a) {
  __shared__ float red[EB_WAVES][HS];             // total variation per wave and head
  __shared__ float ured[EB_WAVES][3];
  __shared__ float zred[EB_WAVES][2][HS][2];      // weighted zero points (set, head, value group)
  __shared__ uint4 recs[EB_WAVES][2][EB_V16];     // value parts of page records (the next one lands meanwhile)
  __shared__ uint4 vt[EB_WAVES][KVQ_PAGE * EB_ROW16];  // the page's original value rows
  __shared__ uint32_t xbuf[EB_WAVES][3][16][8];   // value A operands: [raw, code v0, code v1][row][16 bf16]
  // after the page loop: the four weighted sums of the workgroup
  float(*accs)[HS][KVQ_D] = reinterpret_cast<float(*)[HS][KVQ_D]>(&vt[0][0]);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane >> 4, c = lane & 15;  // row loads: positions 4 r .. 4 r + 3, channels [8c, 8c + 8)
  const int q = lane >> 4, t = lane & 15;  // weight layout: head q, token t
  const int kk = lane >> 4, col = lane & 15;  // B operands: positions 4 kk .. + 3, channel 16 m + col
  EbItem it;
  if (!eb_item<HS>(a, it)) return;
  const int Hkv = a.Hkv, ngrp = a.Hq / a.Hkv / HS, S = a.splits;
  const int b = it.b, h = it.h, L = it.L, nq = it.nq, pbeg = it.pbeg, pend = it.pend;
  const bool vrec = it.grp == ngrp - 1;
  const float ninf = -__builtin_inff();
  const KvqLayout &lay = a.lay;
  const EbPlanes VP = eb_planes(lay.vb);
  const bool qlive = q < HS;
  const int nvg = lay.nvg;
  const int vmeta = lay.v_meta_off - lay.v_codes_off;  // value metadata in the staged part

  if (HS < 4) {
    for (int i = threadIdx.x; i < 3 * 16 * 8 * EB_WAVES; i += 64 * EB_WAVES)
      (&xbuf[0][0][0][0])[i] = 0u;  // rows of heads beyond HS stay zero
  }
  // the head's maxima and sums over all ranges of the sequence
  float M0 = ninf, M1 = ninf, iZ0 = 0.f, iZ1 = 0.f;
  {
    const float *st0 = a.ws + (size_t)(it.unit * ngrp + it.grp) * S * EB_W_ITEM + EB_W_STATS + 6 * (qlive ? q : 0);
    for (int s = 0; s < S; ++s) {
      M0 = __builtin_fmaxf(M0, st0[(size_t)s * EB_W_ITEM + 0]);
      M1 = __builtin_fmaxf(M1, st0[(size_t)s * EB_W_ITEM + 2]);
    }
    float Z0 = 0.f, Z1 = 0.f;
    for (int s = 0; s < S; ++s) {
      const float *st = st0 + (size_t)s * EB_W_ITEM;
      if (st[0] != ninf) Z0 += st[1] * __builtin_amdgcn_exp2f(st[0] - M0);
      if (st[2] != ninf) Z1 += st[3] * __builtin_amdgcn_exp2f(st[2] - M1);
    }
    iZ0 = Z0 > 0.f ? 1.f / Z0 : 0.f;
    iZ1 = Z1 > 0.f ? 1.f / Z1 : 0.f;
  }
  __syncthreads();  // xbuf cleared

  const uint32_t row_elems = (uint32_t)Hkv * KVQ_D;
  const float2 *scores = reinterpret_cast<const float2 *>(a.ws + (size_t)a.B * Hkv * ngrp * S * EB_W_ITEM) +
                         ((size_t)b * a.Hq + it.hq0 + (qlive ? q : 0)) * eb_score_stride(a.max_len);
  // the next page in flight: pv_i = 8 channels of position 4 i + r (clamped to L - 1), its scores
  uint4 pv0, pv1, pv2, pv3;
  float2 psc;
  auto load_page = [&](int pg) __attribute__((always_inline)) {
    const int t0 = pg * KVQ_PAGE;
    const uint16_t *vp = a.v_ref + ((size_t)b * a.max_len + (size_t)t0) * row_elems + (size_t)h * KVQ_D;
    const int last = L - 1 - t0;
    auto off = [&](int i) { return (uint32_t)(4 * i + r < last ? 4 * i + r : last) * row_elems + 8 * c; };
    pv0 = *reinterpret_cast<const uint4 *>(vp + off(0));
    pv1 = *reinterpret_cast<const uint4 *>(vp + off(1));
    pv2 = *reinterpret_cast<const uint4 *>(vp + off(2));
    pv3 = *reinterpret_cast<const uint4 *>(vp + off(3));
    psc = scores[t0 + t < L ? t0 + t : L - 1];
  };
  auto store_page = [&]() __attribute__((always_inline)) {
    vt[w][(0 + r) * EB_ROW16 + c] = pv0;
    vt[w][(4 + r) * EB_ROW16 + c] = pv1;
    vt[w][(8 + r) * EB_ROW16 + c] = pv2;
    vt[w][(12 + r) * EB_ROW16 + c] = pv3;
  };
  const int vpart16 = (lay.record - lay.v_codes_off) / 16;  // the record's value codes and metadata
  auto load_rec = [&](int pg, int bf) __attribute__((always_inline)) {
    eb_load_rec(a, it, pg, lay.v_codes_off, vpart16, (uint32_t)(uintptr_t)&recs[w][bf][0], lane, EB_V16);
  };
  const float sl2 = a.scale * 1.4426950408889634f;

  float tv = 0.f;
  float zs[2][2] = {{0.f, 0.f}, {0.f, 0.f}};  // weighted zero points: set x value group (this lane's head)
  eb_f4 Dr[8], Dc[8];                        // value sums per 16-channel tile: original values, codes
#pragma unroll
  for (int m = 0; m < 8; ++m) Dr[m] = Dc[m] = eb_f4{0.f, 0.f, 0.f, 0.f};
  float ev_sq = 0.f, ev_max = 0.f, v_sq = 0.f;
  int buf = 0;
  if (pbeg + w < pend) {
    load_page(pbeg + w);
    load_rec(pbeg + w, 0);
  }
  for (int pg = pbeg + w; pg < pend; pg += EB_WAVES, buf ^= 1) {
    const int t0 = pg * KVQ_PAGE;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    store_page();
    const float2 sc = psc;
    if (pg + EB_WAVES < pend) {
      load_page(pg + EB_WAVES);
      load_rec(pg + EB_WAVES, buf ^ 1);
    }
    const uint8_t *rs = reinterpret_cast<const uint8_t *>(recs[w][buf]);  // value codes at 0
    const bool valid = qlive && t0 + t < L, quant = t0 + t < nq;
    const float w0 = valid ? __builtin_amdgcn_exp2f(sc.x * sl2 - M0) * iZ0 : 0.f;
    const float w1 = valid ? __builtin_amdgcn_exp2f(sc.y * sl2 - M1) * iZ1 : 0.f;
    tv += __builtin_fabsf(w1 - w0);
    // A operands: raw rows take the weights; code rows the weights times the token's value scale
    // (times 2^64) for quantized tokens, the weights times 2^-69 for window tokens
    if (qlive) {
      const uint32_t *vm = reinterpret_cast<const uint32_t *>(rs + vmeta) + t * nvg;
      uint16_t *xr = reinterpret_cast<uint16_t *>(&xbuf[w][0][0][0]);
      uint32_t hi, lo;
      split2(w0, w1, hi, lo);
      xr[(0 + q) * 16 + t] = (uint16_t)hi;          // set 0, hi
      xr[(4 + q) * 16 + t] = (uint16_t)lo;          // set 0, lo
      xr[(8 + q) * 16 + t] = (uint16_t)(hi >> 16);  // set 1, hi
      xr[(12 + q) * 16 + t] = (uint16_t)(lo >> 16); // set 1, lo
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        if (v >= nvg) break;
        float f0, f1;
        if (quant) {
          const float vs = f16f(vm[v] & 0xFFFF) * 0x1p64f, zr = f16f(vm[v] >> 16);
          f0 = w0 * vs;
          f1 = w1 * vs;
          zs[0][v] = __builtin_fmaf(w0, zr, zs[0][v]);
          zs[1][v] = __builtin_fmaf(w1, zr, zs[1][v]);
        } else {
          f0 = w0 * 0x1p-69f;
          f1 = w1 * 0x1p-69f;
        }
        split2(f0, f1, hi, lo);
        uint16_t *xc = reinterpret_cast<uint16_t *>(&xbuf[w][1 + v][0][0]);
        xc[(0 + q) * 16 + t] = (uint16_t)hi;
        xc[(4 + q) * 16 + t] = (uint16_t)lo;
        xc[(8 + q) * 16 + t] = (uint16_t)(hi >> 16);
        xc[(12 + q) * 16 + t] = (uint16_t)(lo >> 16);
      }
    }
    // A operand of lane l: row l mod 16, tokens 4 (l / 16) .. + 3 (LDS operations of a wave complete in order)
    const eb_s4 ar = __builtin_bit_cast(eb_s4, *reinterpret_cast<const eb_u2 *>(&xbuf[w][0][lane & 15][2 * (lane >> 4)]));
    const eb_s4 ac0 = __builtin_bit_cast(eb_s4, *reinterpret_cast<const eb_u2 *>(&xbuf[w][1][lane & 15][2 * (lane >> 4)]));
    const eb_s4 ac1 = __builtin_bit_cast(eb_s4, *reinterpret_cast<const eb_u2 *>(&xbuf[w][2][lane & 15][2 * (lane >> 4)]));
    const int tq = nq - t0;  // tokens of the page below it are quantized
    const uint16_t *vtb = reinterpret_cast<const uint16_t *>(vt[w]) + (col & 7);
    // value reconstruction in the B layout: the metadata of positions 4 kk + i, group v
    float rsc[2][4], rzr[2][4];
    const bool vr_on = vrec && tq > 0 && !a.value_rotation;
    if (vr_on) {
#pragma unroll
      for (int v = 0; v < 2; ++v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t mm = v < nvg ? reinterpret_cast<const uint32_t *>(rs + vmeta)[(4 * kk + i) * nvg + v] : 0u;
          rsc[v][i] = f16f(mm & 0xFFFF);
          rzr[v][i] = f16f(mm >> 16);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      // positions 4 kk + i, channel 16 m + col: octet 2 m + col / 8
      eb_h2 h01, h23;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 4 * kk + i;
        const uint16_t x = vtb[8 * (n * EB_ROW16 + 2 * m + (col >> 3))];
        if (i == 0) h01[0] = x;
        if (i == 1) h01[1] = x;
        if (i == 2) h23[0] = x;
        if (i == 3) h23[1] = x;
      }
      const uint32_t r0 = __builtin_bit_cast(uint32_t, h01), r1 = __builtin_bit_cast(uint32_t, h23);
      Dr[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ar, pack4s(r0, r1), Dr[m], 0, 0, 0);
      uint32_t c0 = r0, c1 = r1;  // window tokens: exact values
      if (tq > 0) {
        const uint32_t q0 = eb_pair(rs, lane, m, VP), q1 = eb_pair(rs, lane, 8 + m, VP);
        if (tq >= KVQ_PAGE) {
          c0 = q0;
          c1 = q1;
        } else {
          const int tb = 4 * kk;  // first token of the lane's four
          c0 = (tb + 0 < tq ? (q0 & 0xFFFFu) : (r0 & 0xFFFFu)) | (tb + 1 < tq ? (q0 & 0xFFFF0000u) : (r0 & 0xFFFF0000u));
          c1 = (tb + 2 < tq ? (q1 & 0xFFFFu) : (r1 & 0xFFFFu)) | (tb + 3 < tq ? (q1 & 0xFFFF0000u) : (r1 & 0xFFFF0000u));
        }
        if (vr_on) {  // errors of the quantized positions among 4 kk + i, channel 16 m + col
          const int v = (nvg == 2 && m >= 4) ? 1 : 0;
          const uint32_t cw[4] = {q0 & 0xFFFFu, q0 >> 16, q1 & 0xFFFFu, q1 >> 16};
          const uint32_t rw[4] = {r0 << 16, r0 & 0xFFFF0000u, r1 << 16, r1 & 0xFFFF0000u};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (4 * kk + i < tq) {
              const float x = __builtin_bit_cast(float, rw[i]);
              const float err = __builtin_fmaf((float)cw[i], rsc[v][i], rzr[v][i]) - x;
              ev_sq = __builtin_fmaf(err, err, ev_sq);
              ev_max = __builtin_fmaxf(ev_max, __builtin_fabsf(err));
              v_sq = __builtin_fmaf(x, x, v_sq);
            }
          }
        }
      }
      Dc[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k((m < 4 || nvg == 1) ? ac0 : ac1, pack4s(c0, c1), Dc[m], 0, 0, 0);
    }
    if (vrec && a.value_rotation && tq > 0) {  // rotated values: whole rows rotated back
#pragma unroll 1
      for (int ii = 0; ii < 4; ++ii) {
        const int n = 4 * ii + r;
        const bool qn = t0 + n < nq;
        float v[8], vh[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          vh[e] = 0.f;
        }
        bf16x8(vt[w][n * EB_ROW16 + c], v);
        if (qn) decode8<false>(lay, VP, rs - lay.v_codes_off, n, c, vh);
        row_wht(vh, c, qn);
        if (qn) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float err = vh[e] - v[e];
            ev_sq = __builtin_fmaf(err, err, ev_sq);
            ev_max = __builtin_fmaxf(ev_max, __builtin_fabsf(err));
            v_sq = __builtin_fmaf(v[e], v[e], v_sq);
          }
        }
      }
    }
  }

  // ---- merge: TV and weighted zero points per head, value sums per head and channel ----
  {
    const float tvt = row16_sum(tv);
    float zt[2][2];
#pragma unroll
    for (int set = 0; set < 2; ++set) {
#pragma unroll
      for (int v = 0; v < 2; ++v) zt[set][v] = row16_sum(zs[set][v]);
    }
    if (qlive && t == 0) {
      red[w][q] = tvt;
#pragma unroll
      for (int set = 0; set < 2; ++set) {
#pragma unroll
        for (int v = 0; v < 2; ++v) zred[w][set][q][v] = zt[set][v];
      }
    }
  }
  if (vrec) {
    for (int off = 1; off <= 32; off <<= 1) {
      ev_sq += __shfl_xor(ev_sq, off);
      v_sq += __shfl_xor(v_sq, off);
      ev_max = __builtin_fmaxf(ev_max, __shfl_xor(ev_max, off));
    }
    if (lane == 0) {
      ured[w][0] = ev_sq;
      ured[w][1] = ev_max;
      ured[w][2] = v_sq;
    }
  }
  __syncthreads();  // every wave is past its pages: the values' LDS becomes the sums
  for (int i = threadIdx.x; i < 4 * HS * KVQ_D; i += 64 * EB_WAVES) (&accs[0][0][0])[i] = 0.f;
  __syncthreads();
  // value sums: D row 4 (l / 16) + r of lane l = (set, part, head r) = (l / 32, (l / 16) mod 2, r);
  // the hi and lo parts are added across lanes l and l ^ 16; one wave at a time into LDS
  {
    const int G4 = lane >> 4, set = G4 >> 1;
    for (int i = 0; i < EB_WAVES; ++i) {
      if (w == i) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int vg = (nvg == 2 && m >= 4) ? 1 : 0;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const float dr = Dr[m][rr] + __shfl_xor(Dr[m][rr], 16);
            const float dc = Dc[m][rr] + __shfl_xor(Dc[m][rr], 16);
            if ((G4 & 1) == 0 && rr < HS) {
              const int ch = 16 * m + col;
              accs[set == 0 ? 0 : 2][rr][ch] += dr;
              accs[set == 0 ? 1 : 3][rr][ch] += __builtin_fmaf(dc, 0x1p69f, zred[i][set][rr][vg]);
            }
          }
        }
      }
      __syncthreads();
    }
  }
  // the item's sums, total variation and value reconstruction to the workspace
  for (int i = threadIdx.x; i < 4 * HS * KVQ_D; i += 64 * EB_WAVES) {
    const int s = i / (HS * KVQ_D), j = (i / KVQ_D) % HS, ch = i % KVQ_D;
    it.ws[EB_W_SUMS + (4 * s + j) * KVQ_D + ch] = accs[s][j][ch];
  }
  if (w == 0 && lane < HS) {
    float tvj = 0.f;
    for (int i = 0; i < EB_WAVES; ++i) tvj += red[i][lane];
    it.ws[EB_W_TV + lane] = tvj;
  }
  if (vrec && w == 0 && lane == 0) {
    float e0 = 0.f, e1 = 0.f, e2 = 0.f;
    for (int i = 0; i < EB_WAVES; ++i) {
      e0 += ured[i][0];
      e1 = __builtin_fmaxf(e1, ured[i][1]);
      e2 += ured[i][2];
    }
    it.ws[EB_W_VREC + 0] = e0;
    it.ws[EB_W_VREC + 1] = e1;
    it.ws[EB_W_VREC + 2] = e2;
  }
}

// One workgroup of HS waves per (kv head unit, head group): wave j adds the S ranges' sums of head
// j (lane l: channels 2l, 2l + 1) and writes its statistics; the unit's reconstruction errors come
// from head group 0 (keys) and the last head group (values).
template <int HS>
__global__ __launch_bounds__(64 * HS) void kvq_errbudget_final_kernel(KvqErrArgs a) {
  const int lane = threadIdx.x & 63, j = threadIdx.x >> 6;
  const int Hkv = a.Hkv, g = a.Hq / a.Hkv, ngrp = g / HS, S = a.splits;
  const int unit = blockIdx.x / ngrp, grp = blockIdx.x % ngrp;
  const int b = unit / Hkv, h = unit % Hkv;
  const int hq0 = h * g + grp * HS;
  int L = (int)a.seq_lens[b];
  L = L < 0 ? 0 : ((int64_t)L > a.max_len ? (int)a.max_len : L);
  int nq = L > a.R ? L - a.R : 0;
  const int64_t cap_tokens = (a.cache.paged ? (int64_t)a.cache.mbps : a.cache.pages_per_seq) * KVQ_PAGE;
  if ((int64_t)nq > cap_tokens) nq = (int)cap_tokens;
  const float *it0 = a.ws + (size_t)(unit * ngrp + grp) * S * EB_W_ITEM;
  float o2[2] = {0.f, 0.f}, v2[2] = {0.f, 0.f}, k2[2] = {0.f, 0.f}, j2[2] = {0.f, 0.f};
  float tvj = 0.f, dmx = 0.f, dsq = 0.f;
  for (int s = 0; s < S; ++s) {
    const float *it = it0 + (size_t)s * EB_W_ITEM;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int ch = 2 * lane + e;
      o2[e] += it[EB_W_SUMS + (4 * 0 + j) * KVQ_D + ch];
      v2[e] += it[EB_W_SUMS + (4 * 1 + j) * KVQ_D + ch];
      k2[e] += it[EB_W_SUMS + (4 * 2 + j) * KVQ_D + ch];
      j2[e] += it[EB_W_SUMS + (4 * 3 + j) * KVQ_D + ch];
    }
    tvj += it[EB_W_TV + j];
    dmx = __builtin_fmaxf(dmx, it[EB_W_STATS + 6 * j + 4]);
    dsq += it[EB_W_STATS + 6 * j + 5];
  }
  // sums over rotated values are in the rotated domain: rotated back
  if (a.value_rotation) {
    pair_wht(v2[0], v2[1], lane);
    pair_wht(j2[0], j2[1], lane);
  }
  float nv = 0.f, nk = 0.f, nj = 0.f, no = 0.f;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const float oo = o2[e];
    const float dv = v2[e] - oo, dk = k2[e] - oo, dj = j2[e] - oo;
    nv = __builtin_fmaf(dv, dv, nv);
    nk = __builtin_fmaf(dk, dk, nk);
    nj = __builtin_fmaf(dj, dj, nj);
    no = __builtin_fmaf(oo, oo, no);
  }
  for (int off = 1; off <= 32; off <<= 1) {
    nv += __shfl_xor(nv, off);
    nk += __shfl_xor(nk, off);
    nj += __shfl_xor(nj, off);
    no += __shfl_xor(no, off);
  }
  float *hs = a.head_stats + ((size_t)b * a.Hq + hq0 + j) * KVQ_EB_HEAD;
  if (lane == 0) {
    const float n = (float)L;
    hs[0] = dmx;
    hs[1] = L > 0 ? sqrtf(dsq / n) : 0.f;
    hs[2] = 0.5f * tvj;
    hs[3] = sqrtf(nv);
    hs[4] = sqrtf(nk);
    hs[5] = sqrtf(nj);
    hs[6] = sqrtf(no);
    hs[7] = 0.f;
  }
  if (grp == 0 && j == 0 && lane == 0) {
    const float *kit = a.ws + (size_t)(unit * ngrp + 0) * S * EB_W_ITEM;
    const float *vit = a.ws + (size_t)(unit * ngrp + ngrp - 1) * S * EB_W_ITEM;
    float s[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < S; ++sp) {
      const float *kr = kit + (size_t)sp * EB_W_ITEM + EB_W_KREC, *vr = vit + (size_t)sp * EB_W_ITEM + EB_W_VREC;
      s[0] += kr[0];
      s[2] = __builtin_fmaxf(s[2], kr[1]);
      s[4] += kr[2];
      s[1] += vr[0];
      s[3] = __builtin_fmaxf(s[3], vr[1]);
      s[5] += vr[2];
    }
    float *us = a.unit_stats + ((size_t)b * Hkv + h) * KVQ_EB_UNIT;
    us[0] = s[0];
    us[1] = s[1];
    us[2] = s[2];
    us[3] = s[3];
    us[4] = s[4];
    us[5] = s[5];
    us[6] = (float)nq;
    us[7] = 0.f;
  }
}

template <int HS>
void launch_eb(const KvqErrArgs &a, int ngrp, hipStream_t s) {
  const int wus = a.B * a.Hkv * a.splits;
  // groups of 8 work units, each group's head groups 8 workgroups apart (padding after the last)
  const dim3 grid((unsigned)(((wus + 7) / 8) * 8 * ngrp)), block(64 * EB_WAVES);
  hipLaunchKernelGGL((kvq_eb_scores_kernel<HS>), grid, block, 0, s, a);
  hipLaunchKernelGGL((kvq_eb_sums_kernel<HS>), grid, block, 0, s, a);
  hipLaunchKernelGGL((kvq_errbudget_final_kernel<HS>), dim3((unsigned)(a.B * a.Hkv * ngrp)), dim3(64 * HS), 0, s, a);
}

}  // namespace

int kvq_errbudget_heads_per_group(int g) { return g < 4 ? g : 4; }
size_t kvq_errbudget_item_floats() { return EB_W_ITEM; }
size_t kvq_errbudget_score_stride(int64_t max_len) { return eb_score_stride(max_len); }

hipError_t kvq_launch_errbudget(const KvqErrArgs &a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  (void)hipGetLastError();  // drop a stale error left by an earlier, unrelated call
  const int g = a.Hq / a.Hkv, hs = kvq_errbudget_heads_per_group(g);
  switch (hs) {
    case 1: launch_eb<1>(a, g / hs, s); break;
    case 2: launch_eb<2>(a, g / hs, s); break;
    default: launch_eb<4>(a, g / hs, s); break;
  }
  return hipGetLastError();
}
