// Group-wise quantizer and per-token record writer shared by the append kernels and the fused
// decode step of the attention kernel: the same IEEE fp64 operation sequence everywhere, so the
// codes and fp16 metadata of a token do not depend on which kernel quantized it.
//
// Quantizer of nalar.dev "Kuantisasi KV cache mengganggu attention melalui key dan value
// tersimpan", section "Granularitas kuantisasi menentukan nilai yang berbagi scale" (a group of
// values shares a scale and a zero point / offset).  The whole file is compiled without
// floating-point contraction (the library is built with -ffp-contract=off, and each function
// repeats the pragma).
#pragma once
#include "kvq_internal.h"

namespace kvq_quant {

// Metadata of one group from its exact minimum and maximum: zero = RD16(min),
// scale = RU16((max - zero) / (2^b - 1)), raised one fp16 step if zero + (2^b - 1) * scale
// still falls below max (fp64, no contraction, in this order).
struct GroupMeta {
  uint32_t zb, sb;  // fp16 bits
  double zf, sf, qmax;
};
__device__ inline GroupMeta group_meta(double mn, double mx, int bits) {
#pragma clang fp contract(off)
  GroupMeta g;
  mn = mn + 0.0;  // -0 -> +0
  mx = mx + 0.0;
  g.qmax = (double)((1 << bits) - 1);
  g.zb = kvq_f16_round_down(mn);
  g.zf = kvq_f16_bits_to_f64(g.zb);
  g.sb = kvq_f16_round_up((mx - g.zf) / g.qmax);
  g.sf = kvq_f16_bits_to_f64(g.sb);
  if (g.zf + g.qmax * g.sf < mx) {
    g.sb += 1u;
    g.sf = kvq_f16_bits_to_f64(g.sb);
  }
  return g;
}
// Code of x: round half to even of (x - zero) / scale, clamped to [0, 2^b - 1]; 0 when scale == 0.
__device__ inline uint32_t group_code(double x, const GroupMeta &g) {
#pragma clang fp contract(off)
  // Computed unconditionally and selected (no branch per code): with scale 0 the quotient is
  // +-inf or NaN, which the clamp keeps finite, and the select then yields 0.
  double y = __builtin_rint((x - g.zf) / g.sf);
  y = __builtin_fmin(__builtin_fmax(y, 0.0), g.qmax);
  return g.sf == 0.0 ? 0u : (uint32_t)y;
}

// group_code of x, computed in fp32 where that is provably the same integer.  With
// d = x - zero in fp64 (as in group_code) and q = d / scale, the fp32 value
// q32 = fp32(d) * r32, r32 = fp32(1 / scale), is within 3.01 * 2^-24 * q < 2^-14 of q for
// q < 256, and the fp64 quotient group_code rounds is within 2^-44 of q; so unless q32 lies
// within 2^-13 of a half-integer, both round to the same integer.  Codes in that band (exact
// ties included) take group_code's fp64 division.  For an fp32 input x (a bf16 or fp32 value)
// the fp64 difference with the fp16 zero is exact, so fp32(d) is just x - zero rounded once in
// fp32; an fp64 input (a rotated key) is subtracted in fp64 first.
__device__ inline uint32_t group_code_fast(float x, const GroupMeta &g, float r32, float qmax32) {
  const float qv = (x - (float)g.zf) * r32;
  const float fr = qv - __builtin_floorf(qv);
  const float y = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(qv), 0.f), qmax32);
  uint32_t c = g.sf == 0.0 ? 0u : (uint32_t)y;
  if (__builtin_fabsf(fr - 0.5f) <= 0x1p-13f) c = group_code((double)x, g);
  return c;
}
__device__ inline uint32_t group_code_fast(double x, const GroupMeta &g, float r32, float qmax32) {
  const double d = x - g.zf;
  const float qv = (float)d * r32;
  const float fr = qv - __builtin_floorf(qv);
  const float y = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(qv), 0.f), qmax32);
  uint32_t c = g.sf == 0.0 ? 0u : (uint32_t)y;
  if (__builtin_fabsf(fr - 0.5f) <= 0x1p-13f) c = group_code(x, g);
  return c;
}

// Quantize the 128 values held two per lane in groups of G; returns the codes of
// this lane's two channels and the {scale, zero} metadata word of its group.
__device__ inline void quantize_pair(double x0, double x1, int bits, int G, uint32_t *c0, uint32_t *c1,
                                     uint32_t *meta) {
  double mn = __builtin_fmin(x0, x1), mx = __builtin_fmax(x0, x1);
  for (int off = 1; off < G / 2; off <<= 1) {
    mn = __builtin_fmin(mn, __shfl_xor(mn, off));
    mx = __builtin_fmax(mx, __shfl_xor(mx, off));
  }
  const GroupMeta g = group_meta(mn, mx, bits);
  *c0 = group_code(x0, g);
  *c1 = group_code(x1, g);
  *meta = g.sb | (g.zb << 16);
}


// Codes and metadata of one token (codes ck[128], cv[128] and metadata words mk[128 / k_group],
// mv[128 / v_group], all in LDS) into token slot n of page record `rec` (global memory or LDS),
// by the 64 lanes of one wave, one bit plane after the other.  K codes: in each plane of width w
// the token owns w whole words in each of its four octet slots; V codes: it owns half-words (one
// byte at width 1) of its value slots; metadata: one dword per group.  Bytes of other tokens of
// the page are not touched.
__device__ inline void kvq_write_token(uint8_t *rec, const KvqLayout &lay, int n, const uint8_t *ck,
                                       const uint8_t *cv, const uint32_t *mk, const uint32_t *mv, int lane) {
  // K codes: per plane, 4 slots (octets j) x w words.
  int sh = 0;  // bit offset of the plane in the code (its area's offset / 256)
#pragma unroll 1
  for (int w = 8; w >= 1; w >>= 1) {
    if (!(lay.kb == 8 ? w == 8 : (w < 8 && (lay.kb & w) != 0))) continue;  // not a plane of kb
    const int per = 16 / w;
    const uint32_t mask = (1u << w) - 1u;
    if (lane < 4 * w) {
      const int j = lane / w, wi = lane % w;
      uint32_t word = 0;
      for (int s = 0; s < per; ++s) {
        const int u = wi * per + s, kc = u >> 2, i = u & 3;
        const int ch = 32 * kc + 8 * j + 2 * i;
        word |= (((uint32_t)ck[ch] >> sh) & mask) << (w * s);
        word |= (((uint32_t)ck[ch + 1] >> sh) & mask) << (16 + w * s);
      }
      *reinterpret_cast<uint32_t *>(rec + lay.k_codes_off + 256 * sh + (16 * j + n) * 4 * w + 4 * wi) = word;
    }
    sh += w;
  }
  // V codes: per plane, 16 slots; each token owns half-words (or one byte at width 1) of its slot.
  const int jj = n >> 2, r = n & 3, ii = r >> 1, hh = r & 1;
  sh = 0;
#pragma unroll 1
  for (int w = 8; w >= 1; w >>= 1) {
    if (!(lay.vb == 8 ? w == 8 : (w < 8 && (lay.vb & w) != 0))) continue;  // not a plane of vb
    const uint32_t mask = (1u << w) - 1u;
    uint8_t *vbase = rec + lay.v_codes_off + 256 * sh;
    if (w == 1) {
      if (lane < 16) {
        uint32_t byte = 0;
        for (int m = 0; m < 8; ++m) byte |= (((uint32_t)cv[16 * m + lane] >> sh) & 1u) << m;
        vbase[(16 * jj + lane) * 4 + 2 * hh + ii] = (uint8_t)byte;
      }
    } else {
      const int nhw = w / 2, per = 16 / w;
      if (lane < 16 * nhw) {
        const int c16 = lane & 15, hw = lane >> 4;
        uint32_t half = 0;
        for (int q = 0; q < per; ++q) {
          const int m = hw * per + q;
          half |= (((uint32_t)cv[16 * m + c16] >> sh) & mask) << ((m * w) & 15);
        }
        const int wi = ii * (w / 2) + hw;
        *reinterpret_cast<uint16_t *>(vbase + (16 * jj + c16) * 4 * w + 4 * wi + 2 * hh) = (uint16_t)half;
      }
    }
    sh += w;
  }
  // Metadata.
  if (lane < lay.nkg)
    reinterpret_cast<uint32_t *>(rec + lay.k_meta_off)[kvq_meta_dword(lay.nkg, n, lane)] = mk[lane];
  if (lane < lay.nvg)
    reinterpret_cast<uint32_t *>(rec + lay.v_meta_off)[kvq_meta_dword(lay.nvg, n, lane)] = mv[lane];
}

}  // namespace kvq_quant
