// Page-record layout of the quantized KV store and small numeric helpers.
//
// One page holds 16 consecutive tokens of one kv head:
//   [K codes 256*kb B][K meta 64*nkg B][V codes 256*vb B][V meta 64*nvg B]
// Everything inside a record is ordered so that each lane of a 64-wide wave
// fetches, with one 16-byte (or smaller) load, exactly the operand bits that
// the gfx950 16x16x32 bf16 MFMA expects in that lane:
//   A operand of v_mfma_f32_16x16x32_bf16: lane l holds row l%16, k = 8*(l/16) + e (e = 0..7)
//   B operand:                              lane l holds col l%16, k = 8*(l/16) + e
//   D (4 x fp32):                          lane l holds col l%16, rows 4*(l/16) + r (r = 0..3)
//
// Codes of b bits are stored as bit planes: b = 8, 4, 2, 1 is one plane; any other b in 1..7
// is split into the binary digits of b from the highest (3 = 2 + 1, 5 = 4 + 1, 6 = 4 + 2,
// 7 = 4 + 2 + 1).  Plane p of width w holds bits [off, off + w) of every code (off = the
// widths of the planes before it) and is an area of its own, 256 * w bytes, in the layout of a
// w-bit code; the areas follow each other in plane order (plane p at byte 256 * off of the code
// area).  So a b-bit code area is 256 * b bytes for every b, and within each plane:
// K codes: lane-slot l = 16*j + n (token n of the page, channel octet j).  The
//   slot has w 32-bit words holding, for the four 32-channel chunks kc, the
//   channels 32*kc + 8*j + e.  Channel e = 2*i + h of chunk kc has index
//   u = 4*kc + i; it sits in word u / (16/w) at bit 16*h + w*(u % (16/w)).
//   So (word >> w*s) & mask(w, both halves) is one bf16 pair of plane values.
// K meta: entry (token n, group g) at dword n*nkg + g (a token's groups are
//   contiguous, so one lane reads all of them with one load):
//   low half = fp16 scale, high half = fp16 zero.
// V codes: lane-slot l = 16*jj + c16 (channels c16 + 16*m, m = 0..7; tokens
//   4*jj + r, r = 0..3).  The slot has w words.  Token r = 2*i + h, tile m:
//   position p = i*8*w + m*w in the half-word stream h, i.e. word p / 16,
//   bit 16*h + p % 16.  A token's bits in one slot never share a byte with
//   another token's, so tokens of a page can be written concurrently.
// V meta: entry (token n, group g) at dword n*nvg + g.
//
// A code c read as a bf16 bit pattern is the value c * 2^-133 for every c in
// 0..255 (subnormal below 128, continuing into the first normal binade), so
// masking the packed word (and, for several planes, OR-ing the planes' values
// into place) gives exact, offset-free MFMA operands.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

#define KVQ_PAGE 16
#define KVQ_D 128
// Pages per sequence of a contiguous store of `capacity` tokens.
__host__ __device__ inline int64_t kvq_pages_per_seq(int64_t capacity) {
  return capacity / KVQ_PAGE + (capacity % KVQ_PAGE != 0);  // (no overflow near INT64_MAX)
}

struct KvqLayout {
  int kb, kg, vb, vg;
  int nkg, nvg;
  int k_codes_off, k_meta_off, v_codes_off, v_meta_off, record;
};

__host__ __device__ inline KvqLayout kvq_make_layout(int kb, int kg, int vb, int vg) {
  KvqLayout L;
  L.kb = kb;
  L.kg = kg;
  L.vb = vb;
  L.vg = vg;
  L.nkg = KVQ_D / kg;
  L.nvg = KVQ_D / vg;
  L.k_codes_off = 0;
  L.k_meta_off = 256 * kb;
  L.v_codes_off = L.k_meta_off + 64 * L.nkg;
  L.v_meta_off = L.v_codes_off + 256 * vb;
  L.record = L.v_meta_off + 64 * L.nvg;
  return L;
}

// Bit planes of a b-bit code (see above): their number, the width of plane p and its offset
// (bit offset inside the code = word offset of its lane-slot words = its area's offset / 256).
__host__ __device__ constexpr int kvq_nplanes(int b) {
  return b == 8 ? 1 : ((b >> 2) & 1) + ((b >> 1) & 1) + (b & 1);
}
__host__ __device__ constexpr int kvq_plane_width(int b, int p) {
  if (b == 8) return 8;
  for (int w = 4; w >= 1; w >>= 1) {
    if (b & w) {
      if (p == 0) return w;
      --p;
    }
  }
  return 0;
}
__host__ __device__ constexpr int kvq_plane_off(int b, int p) {
  int o = 0;
  for (int q = 0; q < p; ++q) o += kvq_plane_width(b, q);
  return o;
}

// Byte offset (within a w-bit plane area) and bit of the K plane value of (token n, channel ch).
__host__ __device__ inline void kvq_k_code_pos(int w, int n, int ch, int *byte_off, int *bit) {
  const int kc = ch >> 5, x = ch & 31, j = x >> 3, e = x & 7;
  const int i = e >> 1, h = e & 1;
  const int u = 4 * kc + i, per = 16 / w;
  const int word = u / per, s = u % per;
  *byte_off = (16 * j + n) * 4 * w + 4 * word;
  *bit = 16 * h + w * s;
}

// Byte offset (within a w-bit plane area of the V codes) and bit of the V plane value of
// (token tt, channel ch).
__host__ __device__ inline void kvq_v_code_pos(int w, int tt, int ch, int *byte_off, int *bit) {
  const int jj = tt >> 2, r = tt & 3, i = r >> 1, h = r & 1;
  const int m = ch >> 4, c16 = ch & 15;
  const int p = i * 8 * w + m * w;
  *byte_off = (16 * jj + c16) * 4 * w + 4 * (p >> 4);
  *bit = 16 * h + (p & 15);
}

// The b-bit K code of (token n, channel ch) from a record's K code area (all planes: the candidate
// widths 8, 4, 2, 1 in plane order, a width present when it is a plane of b).
__host__ __device__ inline uint32_t kvq_k_code(const uint8_t *kcodes, int b, int n, int ch) {
  uint32_t c = 0;
  int sh = 0;
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1) {
    if (b == 8 ? w == 8 : (w < 8 && (b & w) != 0)) {
      int off, bit;
      kvq_k_code_pos(w, n, ch, &off, &bit);
      const uint32_t word = *reinterpret_cast<const uint32_t *>(kcodes + 256 * sh + off);
      c |= ((word >> bit) & ((1u << w) - 1u)) << sh;
      sh += w;
    }
  }
  return c;
}

// The b-bit V code of (token tt, channel ch) from a record's V code area (all planes).
__host__ __device__ inline uint32_t kvq_v_code(const uint8_t *vcodes, int b, int tt, int ch) {
  uint32_t c = 0;
  int sh = 0;
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1) {
    if (b == 8 ? w == 8 : (w < 8 && (b & w) != 0)) {
      int off, bit;
      kvq_v_code_pos(w, tt, ch, &off, &bit);
      const uint32_t word = *reinterpret_cast<const uint32_t *>(vcodes + 256 * sh + off);
      c |= ((word >> bit) & ((1u << w) - 1u)) << sh;
      sh += w;
    }
  }
  return c;
}

// The b-bit K codes of channels [8c, 8c + 8) of token n (c < 16) from a record's K code area, one
// bit plane at a time: in each plane of width up to 4 they sit in one word of slot 16 (c mod 4) + n
// (two words at width 8).
__host__ __device__ inline void kvq_k_codes8(const uint8_t *kcodes, int b, int n, int c, uint32_t code[8]) {
  const int kc = c >> 2, j = c & 3;
  for (int e = 0; e < 8; ++e) code[e] = 0;
  int sh = 0;
#pragma unroll 1
  for (int lw = 3; lw >= 0; --lw) {
    const int w = 1 << lw;
    if (!(b == 8 ? w == 8 : (w < 8 && (b & w) != 0))) continue;  // not a plane of b
    const int lper = 4 - lw;  // log2 of the channel pairs per word
    const uint32_t mask = (1u << w) - 1u;
    const uint32_t *slot = reinterpret_cast<const uint32_t *>(kcodes + 256 * sh + (16 * j + n) * 4 * w);
    const uint32_t wa = slot[(4 * kc) >> lper], wb = slot[(4 * kc + 2) >> lper];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int u = 4 * kc + (e >> 1);
      const uint32_t word = (e >> 2) ? wb : wa;
      code[e] |= ((word >> (16 * (e & 1) + w * (u & ((1 << lper) - 1)))) & mask) << sh;
    }
    sh += w;
  }
}

// The b-bit V codes of channels [8c, 8c + 8) of token tt (c < 16) from a record's V code area, one
// bit plane at a time: in each plane they sit in the same word of value slots 16 (tt / 4) + 8 (c
// mod 2) + e, e = 0..7.
__host__ __device__ inline void kvq_v_codes8(const uint8_t *vcodes, int b, int tt, int c, uint32_t code[8]) {
  const int jj = tt >> 2, i = (tt & 3) >> 1, h = tt & 1, m = c >> 1;
  for (int e = 0; e < 8; ++e) code[e] = 0;
  int sh = 0;
#pragma unroll 1
  for (int lw = 3; lw >= 0; --lw) {
    const int w = 1 << lw;
    if (!(b == 8 ? w == 8 : (w < 8 && (b & w) != 0))) continue;  // not a plane of b
    const uint32_t mask = (1u << w) - 1u;
    const int p = i * 8 * w + m * w, bit = 16 * h + (p & 15);
    const uint8_t *base = vcodes + 256 * sh + (16 * jj + 8 * (c & 1)) * 4 * w + 4 * (p >> 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) code[e] |= ((*reinterpret_cast<const uint32_t *>(base + e * 4 * w) >> bit) & mask) << sh;
    sh += w;
  }
}

// The same for a single-plane width b (1, 2, 4 or 8): no plane offsets to apply.
__host__ __device__ inline void kvq_k_codes8_one(const uint8_t *kcodes, int b, int n, int c, uint32_t code[8]) {
  const int kc = c >> 2, j = c & 3, per = 16 / b;
  const uint32_t mask = (1u << b) - 1u;
  const uint32_t *slot = reinterpret_cast<const uint32_t *>(kcodes + (16 * j + n) * 4 * b);
  const uint32_t wa = slot[(4 * kc) / per], wb = slot[(4 * kc + 2) / per];
  for (int e = 0; e < 8; ++e) {
    const int u = 4 * kc + (e >> 1);
    code[e] = (((e >> 2) ? wb : wa) >> (16 * (e & 1) + b * (u % per))) & mask;
  }
}
__host__ __device__ inline void kvq_v_codes8_one(const uint8_t *vcodes, int b, int tt, int c, uint32_t code[8]) {
  const int jj = tt >> 2, i = (tt & 3) >> 1, h = tt & 1, m = c >> 1;
  const uint32_t mask = (1u << b) - 1u;
  const int p = i * 8 * b + m * b, bit = 16 * h + (p & 15);
  const uint8_t *base = vcodes + (16 * jj + 8 * (c & 1)) * 4 * b + 4 * (p >> 4);
  for (int e = 0; e < 8; ++e) code[e] = (*reinterpret_cast<const uint32_t *>(base + e * 4 * b) >> bit) & mask;
}

__host__ __device__ inline int kvq_meta_dword(int ngroups, int tt, int grp) { return tt * ngroups + grp; }

// Record index of (sequence b, kv head h, logical page p).  Contiguous mode is page-major:
// page p of every (sequence, kv head) unit, then page p + 1, ..., so each unit's pages are
// spread evenly over the whole allocation (units = batch * Hkv).  Callers keep p below
// pages_per_seq (contiguous) or mbps (paged); a block-table entry outside [0, pool_pages)
// is clamped so that a bad table cannot address memory outside the pool.
__host__ __device__ inline int64_t kvq_record_index(int paged, const int32_t *block_table, int mbps,
                                                    int64_t units, int64_t pool_pages, int Hkv, int b, int h,
                                                    int64_t p) {
  if (paged) {
    int64_t e = block_table[(int64_t)b * mbps + p];
    e = e < 0 ? 0 : (e >= pool_pages ? pool_pages - 1 : e);
    return e * Hkv + h;
  }
  return p * units + ((int64_t)b * Hkv + h);
}

// ---------------------------------------------------------------------------
// fp16 directed rounding of fp64 values, by bit manipulation (finite |x| < 65504).
// ---------------------------------------------------------------------------
// Largest fp16 <= a for a >= 0; *exact tells whether a is itself an fp16 value.
__device__ inline uint32_t kvq_f16_trunc_pos(double a, bool *exact) {
  if (a == 0.0) {
    *exact = true;
    return 0u;
  }
  if (a < 6.103515625e-05) {  // below 2^-14: subnormal fp16 m * 2^-24
    const double y = a * 16777216.0;
    const double fl = __builtin_floor(y);
    *exact = (fl == y);
    return (uint32_t)fl;
  }
  const uint64_t u = (uint64_t)__builtin_bit_cast(uint64_t, a);
  const int e = (int)((u >> 52) & 0x7FF) - 1023;
  const uint64_t man = u & 0xFFFFFFFFFFFFFull;
  *exact = (man & ((1ull << 42) - 1)) == 0;
  return ((uint32_t)(e + 15) << 10) | (uint32_t)(man >> 42);
}

__device__ inline uint32_t kvq_f16_round_down(double x) {
  if (x >= 0.0) {
    bool ex;
    return kvq_f16_trunc_pos(x, &ex);
  }
  bool ex;
  const uint32_t t = kvq_f16_trunc_pos(-x, &ex);
  return 0x8000u | (ex ? t : t + 1u);
}

__device__ inline uint32_t kvq_f16_round_up(double x) {
  if (x >= 0.0) {
    bool ex;
    const uint32_t t = kvq_f16_trunc_pos(x, &ex);
    return ex ? t : t + 1u;
  }
  bool ex;
  return 0x8000u | kvq_f16_trunc_pos(-x, &ex);
}

// fp16 bit pattern -> fp64 value (exact), infinities and NaN included: a 1-bit group whose range
// exceeds the largest fp16 gets the scale +inf from the directed rounding, and its codes then
// follow from x / inf = 0.
__host__ __device__ inline double kvq_f16_bits_to_f64(uint32_t h) {
  const uint32_t s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = (double)m * 5.9604644775390625e-08;  // 2^-24
  else if (e == 31)
    v = m ? __builtin_nan("") : __builtin_inf();
  else
    v = (double)(1024 + m) * __builtin_ldexp(1.0, (int)e - 25);
  return s ? -v : v;
}

__host__ __device__ inline float kvq_bf16_bits_to_f32(uint32_t b) { return __builtin_bit_cast(float, b << 16); }

__host__ __device__ inline uint32_t kvq_f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (u >> 16) | 0x40u;  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
