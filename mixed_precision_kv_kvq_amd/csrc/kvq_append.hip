// Fused append + quantize + pack.
//
// Quantizer of nalar.dev "Kuantisasi KV cache mengganggu attention melalui key
// dan value tersimpan", section "Granularitas kuantisasi menentukan nilai yang
// berbagi scale" (groups share a scale and a zero point / offset), with the
// K/V bit widths and group sizes of gist.science arXiv 2502.15075 "Quantize
// What Counts", sections "Belangrijkste Bijdragen" and "Resultaten"; key-only
// Walsh-Hadamard rotation from its "Resultaten" section; recent-token window
// from the nalar.dev article's section "Pertumbuhan cache mengubah trade pada
// serving".
//
// An append of n tokens to a sequence of length L with a window of R quantizes the positions
// [max(L - R, 0), max(L + n - R, 0)): the old ring tokens that leave the window and, when n > R,
// new tokens that are already older than the window on arrival.  Position t is read from ring
// slot t mod R when t < L, else from input row t - L.  Whole 16-token pages of that range go to the
// page kernel (one wave per page), the partial pages at either end (at most 15 tokens each) to the
// per-token kernel (one wave per token, lane l owning channels 2l and 2l + 1).  Whoever reads an
// old token from its ring slot also writes the slot's new content (the last appended token that
// maps to it) after the read, in the same lanes: no slot is read and written by different waves.
// Slots that held no token yet (L < R) are written by write-only items of the per-token kernel.
// All quantizer arithmetic is IEEE fp64 with no contraction, in the same operation order as its
// definition.
#include <type_traits>

#include "kvq_quant.h"

#pragma clang fp contract(off)

namespace {

using namespace kvq_quant;

__device__ inline double load_elem(const uint8_t *row, int c, int kv_f32) {
  if (kv_f32) return (double)reinterpret_cast<const float *>(row)[c];
  return (double)kvq_bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(row)[c]);
}

// Positions quantized by an append of n tokens to a length-L sequence with window R, and their
// split between the two kernels: whole pages [p_start, p_end) to the page kernel, `head` positions
// before p_start and `tail` positions from p_end * 16 to the per-token kernel.
struct QuantRange {
  int64_t q0, q1;          // quantized positions [q0, q1)
  int64_t p_start, p_end;  // whole pages
  int head, tail;
};
__device__ inline QuantRange quant_range(int64_t L, int n, int R) {
  QuantRange d;
  d.q0 = L - R > 0 ? L - R : 0;
  d.q1 = L + n - R > 0 ? L + n - R : 0;
  d.p_start = (d.q0 + KVQ_PAGE - 1) / KVQ_PAGE;
  d.p_end = d.q1 / KVQ_PAGE;
  if (d.p_end > d.p_start) {
    d.head = (int)(d.p_start * KVQ_PAGE - d.q0);
    d.tail = (int)(d.q1 - d.p_end * KVQ_PAGE);
  } else {
    d.p_start = d.p_end = 0;
    d.head = (int)(d.q1 - d.q0);
    d.tail = 0;
  }
  return d;
}
// The last appended position (< L + n) that maps to ring slot t mod R, for an old position t < L
// that leaves the window in this append (so that position is t + R or later, an appended token).
__device__ inline int64_t ring_final(int64_t t, int64_t L, int n, int R) {
  return t + (int64_t)R * ((L + n - 1 - t) / R);
}

// Tokens appended to sequence b: n_new_per_seq[b] clamped into [0, n_new] (the rows of k_new and
// v_new end there), or n_new for every sequence.
// A clamped entry is reported as KVQ_DEV_COUNT.
__device__ inline int append_count(const KvqAppendArgs &a, int b) {
  if (!a.n_new_per_seq) return a.n_new;
  const int n = a.n_new_per_seq[b];
  kvq_raise(a.cache, n < 0 || n > a.n_new, KVQ_DEV_COUNT);
  return n < 0 ? 0 : (n > a.n_new ? a.n_new : n);
}
// Length of sequence b before the append; a negative length is taken as 0 and reported as
// KVQ_DEV_LENGTH.
__device__ inline int append_base(const KvqAppendArgs &a, int b) {
  const int L = a.seq_lens_before[b];
  kvq_raise(a.cache, L < 0, KVQ_DEV_LENGTH);
  return L < 0 ? 0 : L;
}

// One position of the quantized range outside whole pages (one wave, lane l owning channels 2l
// and 2l + 1), item < head + tail; lds: at least 280 bytes.
__device__ void token_item(const KvqAppendArgs &a, int item, int h, int b, uint8_t *lds) {
  uint8_t *ck = lds, *cv = lds + KVQ_D;
  uint32_t *mk = reinterpret_cast<uint32_t *>(lds + 2 * KVQ_D), *mv = mk + KVQ_D / 32;
  const int lane = threadIdx.x;
  const int L = append_base(a, b);
  const int nb = append_count(a, b);
  const int R = a.R, Hkv = a.Hkv;
  const int esz = a.kv_f32 ? 4 : 2;
  const size_t row_bytes = (size_t)KVQ_D * esz;
  const KvqLayout &lay = a.lay;

  int64_t t_q = -1;
  const uint8_t *srcK = nullptr, *srcV = nullptr;
  uint8_t *dstK = nullptr, *dstV = nullptr;
  const uint8_t *newK = nullptr, *newV = nullptr;
  const QuantRange d = quant_range(L, nb, R);
  auto input_row = [&](int64_t pos) { return (((size_t)b * a.n_new + (size_t)(pos - L)) * Hkv + h) * row_bytes; };
  auto ring_row = [&](int64_t pos) { return (((size_t)b * Hkv + h) * R + (size_t)(pos % R)) * row_bytes; };
  if (item >= d.head + d.tail) return;
  {
    t_q = item < d.head ? d.q0 + item : d.p_end * KVQ_PAGE + (item - d.head);
    if (t_q < L) {  // an old token leaving the ring: read it, then write the slot's new content
      dstK = a.cache.k_win + ring_row(t_q);
      dstV = a.cache.v_win + ring_row(t_q);
      srcK = dstK;
      srcV = dstV;
      const int64_t f = ring_final(t_q, L, nb, R);
      newK = a.k_new + input_row(f);
      newV = a.v_new + input_row(f);
    } else {
      srcK = a.k_new + input_row(t_q);
      srcV = a.v_new + input_row(t_q);
    }
  }

  double k0 = 0, k1 = 0, v0 = 0, v1 = 0;
  if (t_q >= 0) {
    k0 = load_elem(srcK, 2 * lane, a.kv_f32);
    k1 = load_elem(srcK, 2 * lane + 1, a.kv_f32);
    v0 = load_elem(srcV, 2 * lane, a.kv_f32);
    v1 = load_elem(srcV, 2 * lane + 1, a.kv_f32);
  }
  if (newK) {  // same lane, same channels: the old values above are read first
    if (a.kv_f32) {
      reinterpret_cast<uint2 *>(dstK)[lane] = reinterpret_cast<const uint2 *>(newK)[lane];
      reinterpret_cast<uint2 *>(dstV)[lane] = reinterpret_cast<const uint2 *>(newV)[lane];
    } else {
      reinterpret_cast<uint32_t *>(dstK)[lane] = reinterpret_cast<const uint32_t *>(newK)[lane];
      reinterpret_cast<uint32_t *>(dstV)[lane] = reinterpret_cast<const uint32_t *>(newV)[lane];
    }
  }
  if (t_q < 0) return;

  if (a.rotation) kvq_wht128_fp64(k0, k1, lane);
  if (a.value_rotation) kvq_wht128_fp64(v0, v1, lane);
  uint32_t a0, a1, am, b0, b1, bm;
  quantize_pair(k0, k1, lay.kb, lay.kg, &a0, &a1, &am);
  quantize_pair(v0, v1, lay.vb, lay.vg, &b0, &b1, &bm);
  ck[2 * lane] = (uint8_t)a0;
  ck[2 * lane + 1] = (uint8_t)a1;
  cv[2 * lane] = (uint8_t)b0;
  cv[2 * lane + 1] = (uint8_t)b1;
  if (((2 * lane) % lay.kg) == 0) mk[(2 * lane) / lay.kg] = am;
  if (((2 * lane) % lay.vg) == 0) mv[(2 * lane) / lay.vg] = bm;
  __syncthreads();

  const int64_t page = t_q / KVQ_PAGE;
  const int n = (int)(t_q % KVQ_PAGE);
  if (page >= (a.cache.paged ? (int64_t)a.cache.mbps : a.cache.pages_per_seq)) {  // beyond the cache: dropped
    kvq_raise(a.cache, true, KVQ_DEV_CAPACITY);
    return;
  }
  const int64_t rec_idx = kvq_record_index_dev(a.cache, Hkv, b, h, page);
  uint8_t *rec = a.cache.pages + (size_t)rec_idx * lay.record;

  kvq_write_token(rec, lay, n, ck, cv, mk, mv, lane);
}

// Whole pages of tokens quantized on arrival: one wave per (page, kv head, sequence).  Lane
// 16 q + t holds channels [32 q, 32 q + 32) of the page's token t, so a 32-channel group's
// minimum and maximum are taken inside the lane (wider groups combine 2 or 4 lanes); the
// record is assembled in LDS (codes OR-ed into their words) and written with 16-byte stores.
// Same quantizer arithmetic as the per-token kernel (group_meta / group_code), so the codes
// and metadata are identical.
// ROT: keys and/or values (a.rotation, a.value_rotation) are rotated first; the lane's values
// are then fp64 (the transform's results).  Without rotation they are the inputs themselves,
// exact in fp32, which halves the registers.
constexpr int kMaxRecordWords = (256 * 8 + 64 * 4 + 256 * 8 + 64 * 2) / 4;

template <bool ROT>
__device__ void page_item(const KvqAppendArgs &a, int pidx, int h, int b, uint32_t *rw) {
  const int lane = threadIdx.x;
  const int L = append_base(a, b);
  const int nb = append_count(a, b);
  const int R = a.R;
  const QuantRange d = quant_range(L, nb, R);
  const int64_t page = d.p_start + pidx;
  if (page >= d.p_end) return;
  if (page >= (a.cache.paged ? (int64_t)a.cache.mbps : a.cache.pages_per_seq)) {  // beyond the cache: dropped
    kvq_raise(a.cache, true, KVQ_DEV_CAPACITY);
    return;
  }
  const KvqLayout &lay = a.lay;
  const int Hkv = a.Hkv;
  const int t = lane & 15, q = lane >> 4;
  const int esz = a.kv_f32 ? 4 : 2;
  const size_t row_bytes = (size_t)KVQ_D * esz;
  // this lane's page token: an old token in ring slot pos mod R, or input row pos - L
  const int64_t pos = page * KVQ_PAGE + t;
  const bool from_ring = pos < L;
  const size_t src_off = from_ring ? (((size_t)b * Hkv + h) * R + (size_t)(pos % (R > 0 ? R : 1))) * row_bytes
                                   : (((size_t)b * a.n_new + (size_t)(pos - L)) * Hkv + h) * row_bytes;
  const uint8_t *srcK = (from_ring ? a.cache.k_win : a.k_new) + src_off;
  const uint8_t *srcV = (from_ring ? a.cache.v_win : a.v_new) + src_off;
  for (int w = lane; w < lay.record / 4; w += 64) rw[w] = 0u;
  __syncthreads();

  typedef typename std::conditional<ROT, double, float>::type Val;
  Val x[32];
  // This lane's 32 channels of a key or value row: 16-byte loads of bf16 or fp32 values.
  auto load32 = [&](const uint8_t *row) __attribute__((always_inline)) {
    if (a.kv_f32) {
      const uint4 *p = reinterpret_cast<const uint4 *>(row + 128 * q);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint4 w = p[k];
        x[4 * k + 0] = (Val)__builtin_bit_cast(float, w.x);
        x[4 * k + 1] = (Val)__builtin_bit_cast(float, w.y);
        x[4 * k + 2] = (Val)__builtin_bit_cast(float, w.z);
        x[4 * k + 3] = (Val)__builtin_bit_cast(float, w.w);
      }
    } else {
      const uint4 *p = reinterpret_cast<const uint4 *>(row + 64 * q);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 w = p[k];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[8 * k + 2 * i] = (Val)kvq_bf16_bits_to_f32(ws[i] & 0xFFFFu);
          x[8 * k + 2 * i + 1] = (Val)kvq_bf16_bits_to_f32(ws[i] >> 16);
        }
      }
    }
  };
  // Normalized 128-point Walsh-Hadamard transform of the row: butterflies in stage order
  // 1, 2, ..., 64, stages up to 16 inside the lane, 32 and 64 across lanes q ^ 1 and q ^ 2
  // (same operands and order as the definition).
  auto rotate = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int hs = 1; hs < 32; hs <<= 1) {
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        if ((e & hs) == 0) {
          const double u = x[e], v = x[e + hs];
          x[e] = u + v;
          x[e + hs] = u - v;
        }
      }
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int lx = st == 0 ? 16 : 32;  // lane distance of channel distance 32 / 64
      const bool upper = (lane & lx) != 0;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const double p = __shfl_xor(x[e], lx);
        x[e] = upper ? p - x[e] : x[e] + p;
      }
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = x[e] * KVQ_WHT_C;
  };
  // ---- keys ----
  load32(srcK);
  if constexpr (ROT) {
    if (a.rotation) rotate();
  }
  {
    Val mnv = x[0], mxv = x[0];
#pragma unroll
    for (int e = 1; e < 32; ++e) {
      mnv = mnv < x[e] ? mnv : x[e];  // exact in either precision
      mxv = mxv > x[e] ? mxv : x[e];
    }
    double mn = (double)mnv, mx = (double)mxv;
    for (int off = 16; off < 16 * (lay.kg / 32); off <<= 1) {  // groups wider than 32 channels
      mn = __builtin_fmin(mn, __shfl_xor(mn, off));
      mx = __builtin_fmax(mx, __shfl_xor(mx, off));
    }
    const GroupMeta g = group_meta(mn, mx, lay.kb);
    const float r32 = 1.0f / (float)g.sf, qmax32 = (float)g.qmax;  // fp16 scale: exact in fp32
    if ((lay.kb & (lay.kb - 1)) == 0) {
      // a single-plane width: the octet's channel pairs u = 4q + i fill word u / per of slot
      // 16 jo + t: one word for widths up to 4, two at 8; the codes are gathered per word
      // before one OR
      const int kb = lay.kb, per = 16 / kb;
      uint32_t *kw = rw + lay.k_codes_off / 4;
#pragma unroll
      for (int jo = 0; jo < 4; ++jo) {      // channel octet within the chunk
        uint32_t acc = 0;
        int wcur = (4 * q) / per;
#pragma unroll
        for (int i = 0; i < 4; ++i) {       // channel pair within the octet
          const uint32_t c0 = group_code_fast(x[8 * jo + 2 * i], g, r32, qmax32);
          const uint32_t c1 = group_code_fast(x[8 * jo + 2 * i + 1], g, r32, qmax32);
          const int u = 4 * q + i;
          if (u / per != wcur) {
            atomicOr(kw + (16 * jo + t) * kb + wcur, acc);
            acc = 0;
            wcur = u / per;
          }
          acc |= (c0 << (kb * (u % per))) | (c1 << (16 + kb * (u % per)));
        }
        atomicOr(kw + (16 * jo + t) * kb + wcur, acc);
      }
    } else {
      // bit planes: the same per plane (width w, bits [sh, sh + w) of the codes) in its area
#pragma unroll
      for (int jo = 0; jo < 4; ++jo) {
        uint32_t c[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) c[e] = group_code_fast(x[8 * jo + e], g, r32, qmax32);
        int sh = 0;
#pragma unroll
        for (int w = 4; w >= 1; w >>= 1) {
          if ((lay.kb & w) == 0) continue;  // not a plane of kb
          const int per = 16 / w;
          const uint32_t mask = (1u << w) - 1u;
          uint32_t *kw = rw + (lay.k_codes_off + 256 * sh) / 4;
          uint32_t acc = 0;
          int wcur = (4 * q) / per;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int u = 4 * q + i;
            if (u / per != wcur) {
              atomicOr(kw + (16 * jo + t) * w + wcur, acc);
              acc = 0;
              wcur = u / per;
            }
            acc |= (((c[2 * i] >> sh) & mask) << (w * (u % per))) |
                   (((c[2 * i + 1] >> sh) & mask) << (16 + w * (u % per)));
          }
          atomicOr(kw + (16 * jo + t) * w + wcur, acc);
          sh += w;
        }
      }
    }
    const int grp = (32 * q) / lay.kg;
    if ((32 * q) % lay.kg == 0) rw[lay.k_meta_off / 4 + kvq_meta_dword(lay.nkg, t, grp)] = g.sb | (g.zb << 16);
  }
  // ---- values ----
  load32(srcV);
  if constexpr (ROT) {
    if (a.value_rotation) rotate();
  }
  {
    Val mnv = x[0], mxv = x[0];
#pragma unroll
    for (int e = 1; e < 32; ++e) {
      mnv = mnv < x[e] ? mnv : x[e];
      mxv = mxv > x[e] ? mxv : x[e];
    }
    double mn = (double)mnv, mx = (double)mxv;
    for (int off = 16; off < 16 * (lay.vg / 32); off <<= 1) {
      mn = __builtin_fmin(mn, __shfl_xor(mn, off));
      mx = __builtin_fmax(mx, __shfl_xor(mx, off));
    }
    const GroupMeta g = group_meta(mn, mx, lay.vb);
    const float r32 = 1.0f / (float)g.sf, qmax32 = (float)g.qmax;
    const int jj = t >> 2, r = t & 3, iv = r >> 1, hv = r & 1;
    // channels 32 q + e and 32 q + 16 + e (tiles 2q and 2q + 1, same column) share a word of
    // every plane area for every width: one OR per plane for both codes
    if ((lay.vb & (lay.vb - 1)) == 0) {  // a single-plane width
      const int vb = lay.vb;
      uint32_t *vw = rw + lay.v_codes_off / 4;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m0 = 2 * q, pos0 = iv * 8 * vb + m0 * vb, pos1 = pos0 + vb;
        const uint32_t bits = (group_code_fast(x[e], g, r32, qmax32) << (16 * hv + (pos0 & 15))) |
                              (group_code_fast(x[e + 16], g, r32, qmax32) << (16 * hv + (pos1 & 15)));
        atomicOr(vw + (16 * jj + e) * vb + (pos0 >> 4), bits);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t c0 = group_code_fast(x[e], g, r32, qmax32), c1 = group_code_fast(x[e + 16], g, r32, qmax32);
        int sh = 0;
#pragma unroll
        for (int w = 4; w >= 1; w >>= 1) {
          if ((lay.vb & w) == 0) continue;  // not a plane of vb
          const uint32_t mask = (1u << w) - 1u;
          const int m0 = 2 * q, pos0 = iv * 8 * w + m0 * w, pos1 = pos0 + w;
          const uint32_t bits = (((c0 >> sh) & mask) << (16 * hv + (pos0 & 15))) |
                                (((c1 >> sh) & mask) << (16 * hv + (pos1 & 15)));
          atomicOr(rw + (lay.v_codes_off + 256 * sh) / 4 + (16 * jj + e) * w + (pos0 >> 4), bits);
          sh += w;
        }
      }
    }
    const int grp = (32 * q) / lay.vg;
    if ((32 * q) % lay.vg == 0) rw[lay.v_meta_off / 4 + kvq_meta_dword(lay.nvg, t, grp)] = g.sb | (g.zb << 16);
  }
  __syncthreads();
  const int64_t rec_idx = kvq_record_index_dev(a.cache, Hkv, b, h, page);
  uint4 *rec = reinterpret_cast<uint4 *>(a.cache.pages + (size_t)rec_idx * lay.record);
  const uint4 *src = reinterpret_cast<const uint4 *>(rw);
  for (int c = lane; c < lay.record / 16; c += 64) rec[c] = src[c];
  // A token read from the ring: its slot receives the last appended token that maps to it (this
  // lane read those very bytes above, so the read precedes the write).
  if (from_ring) {
    const size_t in_off = (((size_t)b * a.n_new + (size_t)(ring_final(pos, L, nb, R) - L)) * Hkv + h) * row_bytes;
    const int cb = 32 * esz;  // this lane's 32 channels
    const uint4 *nk = reinterpret_cast<const uint4 *>(a.k_new + in_off + cb * q);
    const uint4 *nv = reinterpret_cast<const uint4 *>(a.v_new + in_off + cb * q);
    uint4 *dk = reinterpret_cast<uint4 *>(a.cache.k_win + src_off + cb * q);
    uint4 *dv = reinterpret_cast<uint4 *>(a.cache.v_win + src_off + cb * q);
    for (int k = 0; k < cb / 16; ++k) {
      dk[k] = nk[k];
      dv[k] = nv[k];
    }
  }
}

// Appended positions that stay in the ring and whose slot held no token before the append (the
// ring was not yet full): plain row copies, all of one (sequence, kv head) by one wave, 16 bytes
// per lane per instruction.
__device__ void write_only_rows(const KvqAppendArgs &a, int h, int b) {
  const int lane = threadIdx.x, R = a.R, Hkv = a.Hkv;
  if (R == 0) return;
  const int L = append_base(a, b);
  const int nb = append_count(a, b);
  const size_t row_bytes = (size_t)KVQ_D * (a.kv_f32 ? 4 : 2);
  const int chunks = (int)(row_bytes / 16);  // 16-byte chunks per row
  // the kept positions [first_kept, L + nb) (at most R) whose slot had no occupant before the
  // append: the occupant, L - R + ((pos - L) mod R), is negative
  const int64_t first_kept = L + nb - R > L ? L + nb - R : L;
  const int64_t npos = L + nb - first_kept;
  for (int64_t e = lane; e < npos * chunks; e += 64) {
    const int64_t pos = first_kept + e / chunks;
    const int c = (int)(e % chunks);
    if (L - R + (pos - L) % R >= 0) continue;
    const size_t in_off = (((size_t)b * a.n_new + (size_t)(pos - L)) * Hkv + h) * row_bytes + 16 * c;
    const size_t win_off = (((size_t)b * Hkv + h) * R + (size_t)(pos % R)) * row_bytes + 16 * c;
    *reinterpret_cast<uint4 *>(a.cache.k_win + win_off) = *reinterpret_cast<const uint4 *>(a.k_new + in_off);
    *reinterpret_cast<uint4 *>(a.cache.v_win + win_off) = *reinterpret_cast<const uint4 *>(a.v_new + in_off);
  }
}

// One launch per append: blocks [0, pages) take whole pages of the quantized range, the next
// `tokens` blocks one position each of its partial pages, the last block the write-only ring rows.
// The three kinds touch disjoint ring slots and records, so they run concurrently.
template <bool ROT>
__global__ __launch_bounds__(64) void kvq_append_kernel(KvqAppendArgs a, int pages, int tokens) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[kMaxRecordWords];
  const int bx = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  if (bx < pages)
    page_item<ROT>(a, bx, h, b, lds);
  else if (bx < pages + tokens)
    token_item(a, bx - pages, h, b, reinterpret_cast<uint8_t *>(lds));
  else
    write_only_rows(a, h, b);
}

}  // namespace

hipError_t kvq_launch_append(const KvqAppendArgs &a, hipStream_t s) {
  if (a.n_new <= 0 || a.cache.batch <= 0) return hipSuccess;
  (void)hipGetLastError();  // drop a stale error left by an earlier, unrelated call
  // The quantized range of a sequence is at most n positions long: at most ceil(n / 16) whole pages
  // (none when n < 16) and at most 15 positions before and 15 after them.
  const int n = a.n_new;
  const int pages = n >= KVQ_PAGE ? (n + KVQ_PAGE - 1) / KVQ_PAGE : 0;
  const int part = n < KVQ_PAGE - 1 ? n : KVQ_PAGE - 1;
  const dim3 grid((unsigned)(pages + 2 * part + (a.R > 0 ? 1 : 0)), (unsigned)a.Hkv, (unsigned)a.cache.batch);
  if (a.rotation || a.value_rotation)
    hipLaunchKernelGGL(kvq_append_kernel<true>, grid, dim3(64), 0, s, a, pages, 2 * part);
  else
    hipLaunchKernelGGL(kvq_append_kernel<false>, grid, dim3(64), 0, s, a, pages, 2 * part);
  return hipGetLastError();
}
