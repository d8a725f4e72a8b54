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

// The reconstruction of 8 channels [8c, 8c + 8) of token n of a page record staged in LDS (keys
// or values), as zero + code * scale in fp32.
template <bool KEYS>
__device__ __attribute__((always_inline)) inline void decode8(const KvqLayout &lay, const uint8_t *rs, int n, int c,
                                                              float *xh) {
  const uint32_t m = reinterpret_cast<const uint32_t *>(rs + (KEYS ? lay.k_meta_off : lay.v_meta_off))
      [kvq_meta_dword(KEYS ? lay.nkg : lay.nvg, n, (8 * c) / (KEYS ? lay.kg : lay.vg))];
  const float zero = f16f(m >> 16), scale = f16f(m & 0xFFFF);
  uint32_t code[8];
  if (KEYS)
    kvq_k_codes8(rs + lay.k_codes_off, lay.kb, n, c, code);
  else
    kvq_v_codes8(rs + lay.v_codes_off, lay.vb, n, c, code);
#pragma unroll
  for (int e = 0; e < 8; ++e) xh[e] = zero + (float)code[e] * scale;
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;
constexpr int EB_WAVES = 8;
constexpr int EB_REC16 = (256 * 8 + 64 * 4 + 256 * 8 + 64 * 2) / 16;  // largest record, 16-byte units
template <int HG>
__global__ __launch_bounds__(64 * EB_WAVES) void kvq_errbudget_kernel(KvqErrArgs a) {
  __shared__ float red[EB_WAVES][6 * HG];
  __shared__ float ured[EB_WAVES][6];
  __shared__ float accs[4][HG][KVQ_D];
  __shared__ uint4 recs[EB_WAVES][2][EB_REC16];  // page records (two: the next one lands meanwhile)
  __shared__ uint4 rows[EB_WAVES][2][KVQ_PAGE * 16];  // the page's original K and V rows
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane >> 4, c = lane & 15;
  const int Hkv = a.Hkv, g = a.Hq / a.Hkv, ngrp = g / HG;
  // workgroup -> (unit, head group): the groups of unit u at blocks 8 ngrp (u / 8) + 8 grp + u mod 8
  const int blk = blockIdx.x / (8 * ngrp), rem = blockIdx.x % (8 * ngrp);
  const int grp = rem / 8, unit = 8 * blk + rem % 8;
  if (unit >= a.B * Hkv) return;  // padding of the last group of 8 units
  const int b = unit / Hkv, h = unit % Hkv;
  const int hq0 = h * g + grp * HG;  // first query head of the group
  const bool unit_lead = grp == 0;
  int64_t L = a.seq_lens[b];
  kvq_raise(a.cache, hq0 == 0 && (L < 0 || L > a.max_len), KVQ_DEV_LENGTH);
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  int64_t nq = L > a.R ? L - a.R : 0;
  const int64_t cap_tokens = (a.cache.paged ? (int64_t)a.cache.mbps : a.cache.pages_per_seq) * KVQ_PAGE;
  if (nq > cap_tokens) nq = cap_tokens;
  const float ninf = -__builtin_inff();
  const KvqLayout &lay = a.lay;
  const int rec16 = lay.record / 16;

  float q[HG][8];
#pragma unroll
  for (int j = 0; j < HG; ++j) {
    const size_t qrow = ((size_t)b * a.Hq + hq0 + j) * KVQ_D + 8 * c;
    if (a.q_f32) {
      const float4 *qp = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.q) + qrow);
      const float4 x = qp[0], y = qp[1];
      q[j][0] = x.x; q[j][1] = x.y; q[j][2] = x.z; q[j][3] = x.w;
      q[j][4] = y.x; q[j][5] = y.y; q[j][6] = y.z; q[j][7] = y.w;
    } else {
      bf16x8(*reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a.q) + qrow), q[j]);
    }
  }
  // This lane's 16 bytes (8 channels) of original row t (t < L; callers pass a valid t).
  auto ref8 = [&](const uint16_t *base, int64_t t) {
    return *reinterpret_cast<const uint4 *>(base + (((size_t)b * a.max_len + (size_t)t) * Hkv + h) * KVQ_D + 8 * c);
  };
  // One page's original rows in flight: the lane's 16 bytes of the K (and V) rows of positions
  // 4 i + r, loaded for the next page before the current one is computed, then stored to the
  // wave's LDS region (positions past L re-read row L - 1).  The page record goes straight to LDS
  // (buffer loads to LDS, one lane per 16-byte chunk) into the other of the wave's two record
  // buffers; an explicit wait for all of the wave's loads precedes each page.
  struct PageRegs {
    uint4 k[4], v[4];
  };
  auto load_rows = [&](int64_t pg, PageRegs &pr, bool with_v) __attribute__((always_inline)) {
    const int64_t t0 = pg * KVQ_PAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t t = t0 + 4 * i + r < L ? t0 + 4 * i + r : L - 1;
      pr.k[i] = ref8(a.k_ref, t);
      if (with_v) pr.v[i] = ref8(a.v_ref, t);
    }
  };
  auto store_rows = [&](const PageRegs &pr, bool with_v) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rows[w][0][(4 * i + r) * 16 + c] = pr.k[i];
      if (with_v) rows[w][1][(4 * i + r) * 16 + c] = pr.v[i];
    }
  };
  auto load_rec = [&](int64_t pg, int buf) __attribute__((always_inline)) {
    if (pg * KVQ_PAGE >= nq) return;  // no quantized position on this page
    const int64_t rec_idx = kvq_record_index_dev(a.cache, Hkv, b, h, pg);
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)(a.cache.pages + (size_t)rec_idx * lay.record), 0, lay.record,
                                          0x00020000);
    const uint32_t dst = (uint32_t)(uintptr_t)&recs[w][buf][0];
#pragma unroll
    for (int i = 0; i < (EB_REC16 + 63) / 64; ++i) {
      if (64 * i < rec16 && lane + 64 * i < rec16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(size_t)(dst + 1024u * i), 16, 16 * (lane + 64 * i),
                                                 0, 0, 0);
    }
  };
  const float sl2 = a.scale * 1.4426950408889634f;  // softmax scale in log2 units
  const int64_t npages = (L + KVQ_PAGE - 1) / KVQ_PAGE;

  // ---- pass 1 ----
  float m0[HG], z0[HG], m1[HG], z1[HG], ds_max[HG], ds_sq[HG];
#pragma unroll
  for (int j = 0; j < HG; ++j) {
    m0[j] = m1[j] = ninf;
    z0[j] = z1[j] = ds_max[j] = ds_sq[j] = 0.f;
  }
  float ek_sq = 0.f, ek_max = 0.f, k_sq = 0.f;  // key reconstruction error (lead group)
  PageRegs pr;
  int buf = 0;
  if (w < npages) {
    load_rows(w, pr, false);
    load_rec(w, 0);
  }
  for (int64_t pg = w; pg < npages; pg += EB_WAVES, buf ^= 1) {
    const int64_t t0 = pg * KVQ_PAGE;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this page's rows and record have landed
    store_rows(pr, false);
    if (pg + EB_WAVES < npages) {
      load_rows(pg + EB_WAVES, pr, false);
      load_rec(pg + EB_WAVES, buf ^ 1);
    }
    const uint8_t *rs = reinterpret_cast<const uint8_t *>(recs[w][buf]);
#pragma unroll 1
    for (int it = 0; it < 4; ++it) {
      const int n = 4 * it + r;
      const int64_t t = t0 + n;
      const bool valid = t < L, quant = t < nq;
      float k[8], kh[8];
      if (valid) {
        bf16x8(rows[w][0][n * 16 + c], k);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) k[e] = 0.f;
      }
      if (quant) {
        decode8<true>(lay, rs, n, c, kh);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) kh[e] = k[e];
      }
      // Rotated keys are rotated back first (the normalized transform is its own inverse), so
      // both scores use the raw query: q.(H kh) = (H q).kh.  Window keys are stored raw.
      if (a.rotation) row_wht(kh, c, quant);
#pragma unroll
      for (int j = 0; j < HG; ++j) {
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          d0 = __builtin_fmaf(q[j][e], k[e], d0);
          d1 = __builtin_fmaf(q[j][e], kh[e], d1);
        }
        d0 = row16_sum(d0);
        d1 = row16_sum(d1);
        if (valid) {
          const float s0 = d0 * sl2, s1 = d1 * sl2;
          const float n0 = __builtin_fmaxf(m0[j], s0), n1 = __builtin_fmaxf(m1[j], s1);
          z0[j] = z0[j] * __builtin_amdgcn_exp2f(m0[j] - n0) + __builtin_amdgcn_exp2f(s0 - n0);
          z1[j] = z1[j] * __builtin_amdgcn_exp2f(m1[j] - n1) + __builtin_amdgcn_exp2f(s1 - n1);
          m0[j] = n0;
          m1[j] = n1;
          const float ds = (d1 - d0) * a.scale;
          ds_max[j] = __builtin_fmaxf(ds_max[j], __builtin_fabsf(ds));
          ds_sq[j] = __builtin_fmaf(ds, ds, ds_sq[j]);
        }
      }
      if (unit_lead && valid && quant) {
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
  // combine the four position classes (lanes of one row hold equal values), then the waves
#pragma unroll
  for (int j = 0; j < HG; ++j) {
    for (int off = 16; off <= 32; off <<= 1) {
      const float om0 = __shfl_xor(m0[j], off), oz0 = __shfl_xor(z0[j], off);
      const float om1 = __shfl_xor(m1[j], off), oz1 = __shfl_xor(z1[j], off);
      const float n0 = __builtin_fmaxf(m0[j], om0), n1 = __builtin_fmaxf(m1[j], om1);
      z0[j] = (n0 == ninf) ? 0.f : z0[j] * __builtin_amdgcn_exp2f(m0[j] - n0) + oz0 * __builtin_amdgcn_exp2f(om0 - n0);
      z1[j] = (n1 == ninf) ? 0.f : z1[j] * __builtin_amdgcn_exp2f(m1[j] - n1) + oz1 * __builtin_amdgcn_exp2f(om1 - n1);
      m0[j] = n0;
      m1[j] = n1;
      ds_max[j] = __builtin_fmaxf(ds_max[j], __shfl_xor(ds_max[j], off));
      ds_sq[j] += __shfl_xor(ds_sq[j], off);
    }
    if (lane == 0) {
      red[w][6 * j + 0] = m0[j];
      red[w][6 * j + 1] = z0[j];
      red[w][6 * j + 2] = m1[j];
      red[w][6 * j + 3] = z1[j];
      red[w][6 * j + 4] = ds_max[j];
      red[w][6 * j + 5] = ds_sq[j];
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < HG; ++j) {
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
    m0[j] = M0;
    m1[j] = M1;
    z0[j] = Z0 > 0.f ? 1.f / Z0 : 0.f;  // from here on: reciprocal sums
    z1[j] = Z1 > 0.f ? 1.f / Z1 : 0.f;
    ds_max[j] = dmx;
    ds_sq[j] = dsq;
  }
  __syncthreads();

  // ---- pass 2 ----
  float tv[HG];
  float o[HG][8], ov[HG][8], ok[HG][8], oj[HG][8];
#pragma unroll
  for (int j = 0; j < HG; ++j) {
    tv[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[j][e] = ov[j][e] = ok[j][e] = oj[j][e] = 0.f;
  }
  float ev_sq = 0.f, ev_max = 0.f, v_sq = 0.f;
  buf = 0;
  if (w < npages) {
    load_rows(w, pr, true);
    load_rec(w, 0);
  }
  for (int64_t pg = w; pg < npages; pg += EB_WAVES, buf ^= 1) {
    const int64_t t0 = pg * KVQ_PAGE;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this page's rows and record have landed
    store_rows(pr, true);
    if (pg + EB_WAVES < npages) {
      load_rows(pg + EB_WAVES, pr, true);
      load_rec(pg + EB_WAVES, buf ^ 1);
    }
    const uint8_t *rs = reinterpret_cast<const uint8_t *>(recs[w][buf]);
#pragma unroll 1
    for (int it = 0; it < 4; ++it) {
      const int n = 4 * it + r;
      const int64_t t = t0 + n;
      const bool valid = t < L, quant = t < nq;
      float k[8], kh[8], v[8], vh[8];
      if (valid) {
        bf16x8(rows[w][0][n * 16 + c], k);
        bf16x8(rows[w][1][n * 16 + c], v);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) k[e] = v[e] = 0.f;
      }
      if (quant) {
        decode8<true>(lay, rs, n, c, kh);
        decode8<false>(lay, rs, n, c, vh);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kh[e] = k[e];
          vh[e] = v[e];
        }
      }
      if (a.rotation) row_wht(kh, c, quant);
#pragma unroll
      for (int j = 0; j < HG; ++j) {
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          d0 = __builtin_fmaf(q[j][e], k[e], d0);
          d1 = __builtin_fmaf(q[j][e], kh[e], d1);
        }
        d0 = row16_sum(d0);
        d1 = row16_sum(d1);
        const float w0 = valid ? __builtin_amdgcn_exp2f(d0 * sl2 - m0[j]) * z0[j] : 0.f;
        const float w1 = valid ? __builtin_amdgcn_exp2f(d1 * sl2 - m1[j]) * z1[j] : 0.f;
        if (c == 0) tv[j] += __builtin_fabsf(w1 - w0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o[j][e] = __builtin_fmaf(w0, v[e], o[j][e]);
          ov[j][e] = __builtin_fmaf(w0, vh[e], ov[j][e]);
          ok[j][e] = __builtin_fmaf(w1, v[e], ok[j][e]);
          oj[j][e] = __builtin_fmaf(w1, vh[e], oj[j][e]);
        }
      }
      // With rotated values the sums over vh are in the rotated domain (rotated back per head at
      // the end; no recent window then); the reconstruction statistics rotate each position back.
      if (unit_lead && a.value_rotation) row_wht(vh, c, true);
      if (unit_lead && valid && quant) {
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
  // sums over the position classes, then over the waves (one wave at a time into LDS)
#pragma unroll
  for (int j = 0; j < HG; ++j) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[j][e] += __shfl_xor(o[j][e], 16);
      o[j][e] += __shfl_xor(o[j][e], 32);
      ov[j][e] += __shfl_xor(ov[j][e], 16);
      ov[j][e] += __shfl_xor(ov[j][e], 32);
      ok[j][e] += __shfl_xor(ok[j][e], 16);
      ok[j][e] += __shfl_xor(ok[j][e], 32);
      oj[j][e] += __shfl_xor(oj[j][e], 16);
      oj[j][e] += __shfl_xor(oj[j][e], 32);
    }
    for (int off = 1; off <= 32; off <<= 1) tv[j] += __shfl_xor(tv[j], off);
  }
  if (unit_lead) {
    for (int off = 1; off <= 32; off <<= 1) {
      ek_sq += __shfl_xor(ek_sq, off);
      k_sq += __shfl_xor(k_sq, off);
      ev_sq += __shfl_xor(ev_sq, off);
      v_sq += __shfl_xor(v_sq, off);
      ek_max = __builtin_fmaxf(ek_max, __shfl_xor(ek_max, off));
      ev_max = __builtin_fmaxf(ev_max, __shfl_xor(ev_max, off));
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < HG; ++j) red[w][j] = tv[j];
    ured[w][0] = ek_sq;
    ured[w][1] = ev_sq;
    ured[w][2] = ek_max;
    ured[w][3] = ev_max;
    ured[w][4] = k_sq;
    ured[w][5] = v_sq;
  }
  for (int i = 0; i < EB_WAVES; ++i) {
    if (w == i && r == 0) {
#pragma unroll
      for (int j = 0; j < HG; ++j) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int ch = 8 * c + e;
          accs[0][j][ch] = (i == 0 ? 0.f : accs[0][j][ch]) + o[j][e];
          accs[1][j][ch] = (i == 0 ? 0.f : accs[1][j][ch]) + ov[j][e];
          accs[2][j][ch] = (i == 0 ? 0.f : accs[2][j][ch]) + ok[j][e];
          accs[3][j][ch] = (i == 0 ? 0.f : accs[3][j][ch]) + oj[j][e];
        }
      }
    }
    __syncthreads();
  }
  // wave j < HG finishes head j: norms over the channels (lane l takes channels l and l + 64)
  if (w < HG) {
    const int j = w;
    float tvj = 0.f;
    for (int i = 0; i < EB_WAVES; ++i) tvj += red[i][j];
    // lane l takes channels 2l, 2l + 1; sums over rotated values are rotated back first
    float o2[2], v2[2], k2[2], j2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      o2[e] = accs[0][j][2 * lane + e];
      v2[e] = accs[1][j][2 * lane + e];
      k2[e] = accs[2][j][2 * lane + e];
      j2[e] = accs[3][j][2 * lane + e];
    }
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
    // the head's pass-1 statistics: every wave merged them identically
    float dmx = 0.f, dsq = 0.f;
#pragma unroll
    for (int jj = 0; jj < HG; ++jj) {
      if (jj == j) {
        dmx = ds_max[jj];
        dsq = ds_sq[jj];
      }
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
  }
  if (unit_lead && w == 0 && lane == 0) {
    float s[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < EB_WAVES; ++i) {
      s[0] += ured[i][0];
      s[1] += ured[i][1];
      s[2] = __builtin_fmaxf(s[2], ured[i][2]);
      s[3] = __builtin_fmaxf(s[3], ured[i][3]);
      s[4] += ured[i][4];
      s[5] += ured[i][5];
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

}  // namespace

hipError_t kvq_launch_errbudget(const KvqErrArgs &a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  (void)hipGetLastError();  // drop a stale error left by an earlier, unrelated call
  // two heads per group: four would need more than the 256 registers of two waves per SIMD
  const int g = a.Hq / a.Hkv, hg = g < 2 ? g : 2;
  const int units = a.B * a.Hkv;
  // groups of 8 units, each group's head groups 8 workgroups apart (padding after the last unit)
  const dim3 grid((unsigned)(((units + 7) / 8) * 8 * (g / hg))), block(64 * EB_WAVES);
  if (hg == 1)
    hipLaunchKernelGGL(kvq_errbudget_kernel<1>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(kvq_errbudget_kernel<2>, grid, block, 0, s, a);
  return hipGetLastError();
}
