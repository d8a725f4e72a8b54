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
#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace {

__device__ inline double load_elem(const uint8_t *row, int c, int kv_f32) {
  if (kv_f32) return (double)reinterpret_cast<const float *>(row)[c];
  return (double)kvq_bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(row)[c]);
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
  mn = mn + 0.0;
  mx = mx + 0.0;
  const double qmax = (double)((1 << bits) - 1);
  const uint32_t zb = kvq_f16_round_down(mn);
  const double zf = kvq_f16_bits_to_f64(zb);
  uint32_t sb = kvq_f16_round_up((mx - zf) / qmax);
  double sf = kvq_f16_bits_to_f64(sb);
  if (zf + qmax * sf < mx) {
    sb += 1u;
    sf = kvq_f16_bits_to_f64(sb);
  }
  uint32_t r0 = 0, r1 = 0;
  if (sf != 0.0) {
    double y0 = __builtin_rint((x0 - zf) / sf);
    double y1 = __builtin_rint((x1 - zf) / sf);
    y0 = __builtin_fmin(__builtin_fmax(y0, 0.0), qmax);
    y1 = __builtin_fmin(__builtin_fmax(y1, 0.0), qmax);
    r0 = (uint32_t)y0;
    r1 = (uint32_t)y1;
  }
  *c0 = r0;
  *c1 = r1;
  *meta = sb | (zb << 16);
}

// Normalized 128-point Walsh-Hadamard transform of the values held two per lane.
__device__ inline void wht128_fp64(double &x0, double &x1, int lane) {
  {
    const double a = x0, b = x1;
    x0 = a + b;
    x1 = a - b;
  }
  for (int h = 2; h < 128; h <<= 1) {
    const int pl = h >> 1;
    const double p0 = __shfl_xor(x0, pl), p1 = __shfl_xor(x1, pl);
    if ((lane & pl) == 0) {
      x0 = x0 + p0;
      x1 = x1 + p1;
    } else {
      x0 = p0 - x0;
      x1 = p1 - x1;
    }
  }
  x0 = x0 * KVQ_WHT_C;
  x1 = x1 * KVQ_WHT_C;
}

__global__ __launch_bounds__(64) void kvq_append_kernel(KvqAppendArgs a) {
  __shared__ uint8_t ck[KVQ_D];
  __shared__ uint8_t cv[KVQ_D];
  __shared__ uint32_t mk[KVQ_D / 32];
  __shared__ uint32_t mv[KVQ_D / 64];

  const int item = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int L = a.seq_lens_before[b];
  const int nb = a.n_new_per_seq ? a.n_new_per_seq[b] : a.n_new;
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
    const int j = item - R;
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

  if (a.rotation) wht128_fp64(k0, k1, lane);
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
  if (page >= (a.cache.paged ? (int64_t)a.cache.mbps : a.cache.pages_per_seq)) return;  // beyond the cache
  const int64_t rec_idx = kvq_record_index(a.cache.paged, a.cache.block_table, a.cache.mbps,
                                           (int64_t)a.cache.batch * Hkv, a.cache.pool_pages, Hkv, b, h, page);
  uint8_t *rec = a.cache.pages + (size_t)rec_idx * lay.record;

  // K codes: 4 slots (octets j) x kb words.
  const int kb = lay.kb, per_k = 16 / kb;
  if (lane < 4 * kb) {
    const int j = lane / kb, wi = lane % kb;
    uint32_t word = 0;
    for (int s = 0; s < per_k; ++s) {
      const int u = wi * per_k + s, kc = u >> 2, i = u & 3;
      const int ch = 32 * kc + 8 * j + 2 * i;
      word |= (uint32_t)ck[ch] << (kb * s);
      word |= (uint32_t)ck[ch + 1] << (16 + kb * s);
    }
    *reinterpret_cast<uint32_t *>(rec + lay.k_codes_off + (16 * j + n) * 4 * kb + 4 * wi) = word;
  }
  // V codes: 16 slots; each token owns half-words (or one byte when vb == 1) of its slot.
  const int vb = lay.vb;
  const int jj = n >> 2, r = n & 3, ii = r >> 1, hh = r & 1;
  uint8_t *vbase = rec + lay.v_codes_off;
  if (vb == 1) {
    if (lane < 16) {
      uint32_t byte = 0;
      for (int m = 0; m < 8; ++m) byte |= (uint32_t)cv[16 * m + lane] << m;
      vbase[(16 * jj + lane) * 4 + 2 * hh + ii] = (uint8_t)byte;
    }
  } else {
    const int nhw = vb / 2, per_v = 16 / vb;
    if (lane < 16 * nhw) {
      const int c16 = lane & 15, hw = lane >> 4;
      uint32_t half = 0;
      for (int q = 0; q < per_v; ++q) {
        const int m = hw * per_v + q;
        half |= (uint32_t)cv[16 * m + c16] << ((m * vb) & 15);
      }
      const int wi = ii * (vb / 2) + hw;
      *reinterpret_cast<uint16_t *>(vbase + (16 * jj + c16) * 4 * vb + 4 * wi + 2 * hh) = (uint16_t)half;
    }
  }
  // Metadata.
  if (lane < lay.nkg)
    reinterpret_cast<uint32_t *>(rec + lay.k_meta_off)[kvq_meta_dword(lay.nkg, n, lane)] = mk[lane];
  if (lane < lay.nvg)
    reinterpret_cast<uint32_t *>(rec + lay.v_meta_off)[kvq_meta_dword(lay.nvg, n, lane)] = mv[lane];
}

}  // namespace

hipError_t kvq_launch_append(const KvqAppendArgs &a, hipStream_t s) {
  if (a.n_new <= 0 || a.cache.batch <= 0) return hipSuccess;
  dim3 grid((unsigned)a.n_new, (unsigned)a.Hkv, (unsigned)a.cache.batch);
  (void)hipGetLastError();  // drop a stale error left by an earlier, unrelated call
  hipLaunchKernelGGL(kvq_append_kernel, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}
