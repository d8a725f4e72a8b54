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
// One 64-lane wave per work item; lane l owns channels 2l and 2l+1.  Work
// items of sequence b (L = current length, n = tokens appended, R = window):
//   item i < min(n, R): ring slot (L + i) mod R.  The token leaving that slot
//       (position L + i - R, when >= 0) is quantized from the ring, then the
//       last new token that lands in the slot is written to it.
//   item i >= R (only when n > R): new token L + i - R, which is already older
//       than the window when the append finishes, is quantized directly.
// Each ring slot is owned by exactly one wave, so the read of the old token and
// the write of the new one never race.  All quantizer arithmetic is IEEE fp64
// with no contraction, in the same operation order as its definition.
#include <type_traits>

#include "kvq_quant.h"

#pragma clang fp contract(off)

namespace {

using namespace kvq_quant;

__device__ inline double load_elem(const uint8_t *row, int c, int kv_f32) {
  if (kv_f32) return (double)reinterpret_cast<const float *>(row)[c];
  return (double)kvq_bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(row)[c]);
}

// Tokens quantized on arrival (an append of n > R tokens to a length-L sequence: input tokens
// j < m = n - R go to positions L + j) are split between the two kernels: whole 16-token pages
// inside [L, L + m) go to the page kernel, the partial pages at either end to the per-token
// kernel (at most 15 tokens each).
struct DirectSplit {
  int64_t p_start, p_end;  // whole pages [p_start, p_end)
  int head, tail;          // tokens before p_start and after p_end handled one by one
};
__device__ inline DirectSplit direct_split(int64_t L, int m) {
  DirectSplit d;
  d.p_start = (L + KVQ_PAGE - 1) / KVQ_PAGE;
  d.p_end = (L + m) / KVQ_PAGE;
  if (d.p_end > d.p_start) {
    d.head = (int)(d.p_start * KVQ_PAGE - L);
    d.tail = (int)(L + m - d.p_end * KVQ_PAGE);
  } else {
    d.p_end = d.p_start;
    d.head = m;
    d.tail = 0;
  }
  return d;
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

__global__ __launch_bounds__(64) void kvq_append_kernel(KvqAppendArgs a) {
  __shared__ uint8_t ck[KVQ_D];
  __shared__ uint8_t cv[KVQ_D];
  __shared__ uint32_t mk[KVQ_D / 32];
  __shared__ uint32_t mv[KVQ_D / 64];

  const int item = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int L = append_base(a, b);
  const int nb = append_count(a, b);
  if (item >= nb) return;
  const int R = a.R, Hkv = a.Hkv;
  const int esz = a.kv_f32 ? 4 : 2;
  const size_t row_bytes = (size_t)KVQ_D * esz;
  const KvqLayout &lay = a.lay;

  int64_t t_q = -1;
  const uint8_t *srcK = nullptr, *srcV = nullptr;
  uint8_t *dstK = nullptr, *dstV = nullptr;
  const uint8_t *newK = nullptr, *newV = nullptr;
  const int nring = nb < R ? nb : R;
  if (item < nring) {
    const int64_t slot = ((int64_t)L + item) % R;
    const size_t win_off = (((size_t)b * Hkv + h) * R + slot) * row_bytes;
    dstK = a.cache.k_win + win_off;
    dstV = a.cache.v_win + win_off;
    const int64_t t_old = (int64_t)L + item - R;
    if (t_old >= 0) {
      t_q = t_old;
      srcK = dstK;
      srcV = dstV;
    }
    const int64_t first = (int64_t)L + item, last = (int64_t)L + nb - 1;
    const int64_t t_final = first + (int64_t)R * ((last - first) / R);
    const size_t in_off = (((size_t)b * a.n_new + (size_t)(t_final - L)) * Hkv + h) * row_bytes;
    newK = a.k_new + in_off;
    newV = a.v_new + in_off;
  } else {
    // item nring + k: the k-th token quantized on arrival that is not in a whole page
    const DirectSplit d = direct_split(L, nb - R);
    const int k = item - nring;
    int j;
    if (k < d.head)
      j = k;
    else if (k - d.head < d.tail)
      j = (int)(d.p_end * KVQ_PAGE - L) + (k - d.head);
    else
      return;
    t_q = (int64_t)L + j;
    const size_t in_off = (((size_t)b * a.n_new + j) * Hkv + h) * row_bytes;
    srcK = a.k_new + in_off;
    srcV = a.v_new + in_off;
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
template <bool ROT>
__global__ __launch_bounds__(64) void kvq_append_pages_kernel(KvqAppendArgs a) {
  constexpr int kMaxRecordWords = (256 * 8 + 64 * 4 + 256 * 8 + 64 * 2) / 4;
  __shared__ __attribute__((aligned(16))) uint32_t rw[kMaxRecordWords];
  const int h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int L = append_base(a, b);
  const int nb = append_count(a, b);
  const int m = nb - a.R;
  if (m <= 0) return;
  const DirectSplit d = direct_split(L, m);
  const int64_t page = d.p_start + blockIdx.x;
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
  const int j = (int)(page * KVQ_PAGE + t - L);  // input token of this lane's page token
  const size_t in_off = (((size_t)b * a.n_new + j) * Hkv + h) * row_bytes;
  for (int w = lane; w < lay.record / 4; w += 64) rw[w] = 0u;
  __syncthreads();

  typedef typename std::conditional<ROT, double, float>::type Val;
  Val x[32];
  // This lane's 32 channels of a key or value row: 16-byte loads of bf16 or fp32 values.
  auto load32 = [&](const uint8_t *row) {
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
  auto rotate = [&]() {
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
  load32(a.k_new + in_off);
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
    const int kb = lay.kb, per = 16 / kb;
    uint32_t *kw = rw + lay.k_codes_off / 4;
#pragma unroll
    for (int jo = 0; jo < 4; ++jo) {      // channel octet within the chunk
      // the octet's channel pairs u = 4q + i fill word u / per of slot 16 jo + t: one word for
      // bit widths up to 4, two at 8; the codes are gathered per word before one OR
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
    const int grp = (32 * q) / lay.kg;
    if ((32 * q) % lay.kg == 0) rw[lay.k_meta_off / 4 + kvq_meta_dword(lay.nkg, t, grp)] = g.sb | (g.zb << 16);
  }
  // ---- values ----
  load32(a.v_new + in_off);
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
    const int vb = lay.vb;
    const int jj = t >> 2, r = t & 3, iv = r >> 1, hv = r & 1;
    uint32_t *vw = rw + lay.v_codes_off / 4;
    // channels 32 q + e and 32 q + 16 + e (tiles 2q and 2q + 1, same column) share a record word
    // for every value bit width: one OR for both codes
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m0 = 2 * q, pos0 = iv * 8 * vb + m0 * vb, pos1 = pos0 + vb;
      const uint32_t bits = (group_code_fast(x[e], g, r32, qmax32) << (16 * hv + (pos0 & 15))) |
                            (group_code_fast(x[e + 16], g, r32, qmax32) << (16 * hv + (pos1 & 15)));
      atomicOr(vw + (16 * jj + e) * vb + (pos0 >> 4), bits);
    }
    const int grp = (32 * q) / lay.vg;
    if ((32 * q) % lay.vg == 0) rw[lay.v_meta_off / 4 + kvq_meta_dword(lay.nvg, t, grp)] = g.sb | (g.zb << 16);
  }
  __syncthreads();
  const int64_t rec_idx = kvq_record_index_dev(a.cache, Hkv, b, h, page);
  uint4 *rec = reinterpret_cast<uint4 *>(a.cache.pages + (size_t)rec_idx * lay.record);
  const uint4 *src = reinterpret_cast<const uint4 *>(rw);
  for (int c = lane; c < lay.record / 16; c += 64) rec[c] = src[c];
}

}  // namespace

hipError_t kvq_launch_append(const KvqAppendArgs &a, hipStream_t s) {
  if (a.n_new <= 0 || a.cache.batch <= 0) return hipSuccess;
  (void)hipGetLastError();  // drop a stale error left by an earlier, unrelated call
  // per-token kernel: the ring items, then at most 2 * 15 tokens quantized on arrival outside
  // whole pages; page kernel: the whole pages (at most (n - R) / 16 per sequence)
  const int ring = a.n_new < a.R ? a.n_new : a.R;
  const int direct = a.n_new - ring;
  const int items = ring + (direct < 2 * (KVQ_PAGE - 1) ? direct : 2 * (KVQ_PAGE - 1));
  hipLaunchKernelGGL(kvq_append_kernel, dim3((unsigned)items, (unsigned)a.Hkv, (unsigned)a.cache.batch), dim3(64), 0,
                     s, a);
  if (direct >= KVQ_PAGE) {
    const unsigned pages = (unsigned)(direct / KVQ_PAGE);
    const dim3 grid(pages, (unsigned)a.Hkv, (unsigned)a.cache.batch);
    if (a.rotation || a.value_rotation)
      hipLaunchKernelGGL(kvq_append_pages_kernel<true>, grid, dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL(kvq_append_pages_kernel<false>, grid, dim3(64), 0, s, a);
  }
  return hipGetLastError();
}
