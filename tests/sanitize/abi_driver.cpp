// Drives every host-side path of kvq_api.cpp (argument validation, sizing, split plans, launch
// argument set-up) under AddressSanitizer and UndefinedBehaviorSanitizer, with the launches
// replaced by launch_stubs.cpp.  Prints one line per workspace size it computes (for comparison
// with the real library), and exits non-zero at the first unexpected status.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../include/kvq.h"

extern int stub_launches;

static int failures = 0;
#define EXPECT(call, want)                                                                       \
  do {                                                                                          \
    const kvq_status got_ = (call);                                                             \
    if (got_ != (want)) {                                                                       \
      fprintf(stderr, "line %d: %s -> %d, expected %d\n", __LINE__, #call, (int)got_, (int)(want)); \
      ++failures;                                                                               \
    }                                                                                           \
  } while (0)

static void *fake(uintptr_t k) { return (void *)(uintptr_t)(0x100000 + 0x1000 * k); }  // 16-byte aligned stand-ins

static kvq_params params(int hq, int hkv, int kb, int kg, int vb, int vg, int window, int block, int rot = 0,
                         int vrot = 0, int dtype = KVQ_BF16) {
  kvq_params p;
  memset(&p, 0, sizeof(p));
  p.head_dim = 128;
  p.num_q_heads = hq;
  p.num_kv_heads = hkv;
  p.k_bits = kb;
  p.k_group = kg;
  p.v_bits = vb;
  p.v_group = vg;
  p.window = window;
  p.key_rotation = rot;
  p.kv_dtype = dtype;
  p.block_size = block;
  p.value_rotation = vrot;
  return p;
}

static kvq_cache cache_of(const kvq_params &p, int batch, int64_t capacity, int mbps = 0) {
  kvq_cache c;
  memset(&c, 0, sizeof(c));
  c.pages = fake(1);
  if (p.window > 0) {
    c.k_win = fake(2);
    c.v_win = fake(3);
  }
  if (p.block_size) {
    c.block_table = (const int32_t *)fake(4);
    c.max_blocks_per_seq = mbps;
  }
  c.batch = batch;
  c.capacity = capacity;
  return c;
}

// Every entry point with valid arguments (the launch stubs check the workspaces), then each with
// one argument broken.
static void print_params(const char *what, const kvq_params &p, int batch, int64_t max_len, size_t bytes) {
  printf("%s %d %d %d %d %d %d %d %d %d %d %d %d %lld %zu\n", what, p.num_q_heads, p.num_kv_heads, p.k_bits,
         p.k_group, p.v_bits, p.v_group, p.window, p.key_rotation, p.kv_dtype, p.block_size, p.value_rotation, batch,
         (long long)max_len, bytes);
}

static void exercise(const kvq_params &p, int batch, int64_t cap, int64_t max_len, int mbps) {
  const kvq_cache c = cache_of(p, batch, cap, mbps);
  const int32_t *lens = (const int32_t *)fake(5);
  const void *q = fake(6), *knew = fake(7), *vnew = fake(8);
  void *out = fake(9);
  kvq_sizes sz;
  EXPECT(kvq_cache_sizes(&p, batch, cap, &sz), KVQ_OK);
  EXPECT(kvq_quantize_append(&p, &c, lens, nullptr, knew, vnew, 64, nullptr), KVQ_OK);
  EXPECT(kvq_quantize_append(&p, &c, lens, lens, knew, vnew, 1, nullptr), KVQ_OK);
  EXPECT(kvq_quantize_append(&p, &c, lens, nullptr, knew, vnew, 0, nullptr), KVQ_OK);

  const size_t wsb = kvq_decode_workspace_bytes(&p, batch, max_len);
  print_params("decode", p, batch, max_len, wsb);
  std::vector<uint8_t> ws(wsb ? wsb : 1);
  for (int qd = 0; qd <= 1; ++qd) {
    EXPECT(kvq_decode_attention(&p, &c, lens, max_len, q, qd, out, KVQ_F32, 0.f, ws.data(), wsb, nullptr), KVQ_OK);
    EXPECT(kvq_decode_partials(&p, &c, lens, max_len, q, qd, 0.f, ws.data(), wsb, nullptr), KVQ_OK);
    EXPECT(kvq_decode_combine(&p, batch, max_len, qd, ws.data(), out, KVQ_BF16, nullptr), KVQ_OK);
    if (max_len >= 1) {
      EXPECT(kvq_decode_step(&p, &c, lens, knew, vnew, max_len, q, qd, out, KVQ_F32, 0.f, ws.data(), wsb, nullptr),
             KVQ_OK);
      EXPECT(kvq_decode_step_partials(&p, &c, lens, knew, vnew, max_len, q, qd, 0.f, ws.data(), wsb, nullptr),
             KVQ_OK);
    }
    if (wsb > 16)
      EXPECT(kvq_decode_partials(&p, &c, lens, max_len, q, qd, 0.f, ws.data(), wsb - 16, nullptr), KVQ_ENOSPACE);
  }
  EXPECT(kvq_decode_attention(&p, &c, lens, max_len, q, KVQ_BF16, out, KVQ_F32, -1.f, ws.data(), wsb, nullptr),
         KVQ_EINVAL);
  EXPECT(kvq_decode_attention(&p, &c, nullptr, max_len, q, KVQ_BF16, out, KVQ_F32, 0.f, ws.data(), wsb, nullptr),
         KVQ_EINVAL);
  EXPECT(kvq_decode_attention(&p, &c, lens, max_len, (const char *)q + 4, KVQ_BF16, out, KVQ_F32, 0.f, ws.data(),
                              wsb, nullptr),
         KVQ_EINVAL);

  EXPECT(kvq_dequantize_debug(&p, &c, lens, 0, 0, 16, (uint8_t *)fake(10), (uint8_t *)fake(11), (uint16_t *)fake(12),
                              (uint16_t *)fake(13), (float *)fake(14), (float *)fake(15), nullptr),
         KVQ_OK);
  EXPECT(kvq_dequantize_debug(&p, &c, lens, batch, 0, 16, (uint8_t *)fake(10), (uint8_t *)fake(11),
                              (uint16_t *)fake(12), (uint16_t *)fake(13), (float *)fake(14), (float *)fake(15), nullptr),
         KVQ_EINVAL);

  EXPECT(kvq_dequantize_dense(&p, &c, lens, max_len, (uint16_t *)fake(16), (uint16_t *)fake(17), nullptr), KVQ_OK);
  const size_t dwsb = kvq_dense_workspace_bytes(&p, batch, max_len);
  print_params("dense", p, batch, max_len, dwsb);
  std::vector<uint8_t> dws(dwsb ? dwsb : 1);
  EXPECT(kvq_dense_decode_attention(&p, batch, (const uint16_t *)fake(16), (const uint16_t *)fake(17), lens, max_len, q,
                                    KVQ_BF16, out, KVQ_F32, 0.f, dws.data(), dwsb, nullptr),
         KVQ_OK);

  const size_t ewsb = kvq_error_budget_workspace_bytes(&p, batch, max_len);
  print_params("errbudget", p, batch, max_len, ewsb);
  std::vector<float> ews(ewsb / 4 + 1);
  EXPECT(kvq_error_budget(&p, &c, lens, max_len, (const uint16_t *)fake(18), (const uint16_t *)fake(19), q, KVQ_BF16,
                          0.f, (float *)fake(20), (float *)fake(21), ews.data(), ewsb, nullptr),
         KVQ_OK);
  EXPECT(kvq_error_budget(&p, &c, lens, max_len, (const uint16_t *)fake(18), (const uint16_t *)fake(19), q, KVQ_BF16,
                          0.f, (float *)fake(20), (float *)fake(21), ews.data(), ewsb - 4, nullptr),
         KVQ_ENOSPACE);
}

int main() {
  const int before = stub_launches;
  // the supported set: bit widths, groups, heads per kv head, windows, rotations, paging
  const int widths[] = {1, 2, 3, 4, 5, 6, 8};
  for (int kb : widths)
    for (int vb : widths) exercise(params(32, 8, kb, 32, vb, 128, 0, 0), 2, 1024, 1000, 0);
  exercise(params(32, 8, 4, 32, 2, 128, 128, 0), 16, 32768 + 64, 32768 + 8, 0);
  exercise(params(64, 8, 4, 32, 2, 128, 0, 0, 1), 64, 131072, 131072, 0);
  exercise(params(32, 8, 4, 64, 2, 64, 0, 16), 8, 8 * 1024, 16384, 1024);
  exercise(params(8, 8, 8, 128, 8, 64, 16, 0, 1, 0, KVQ_F32), 3, 200, 150, 0);
  exercise(params(2, 1, 1, 32, 1, 128, 0, 0, 0, 1), 70, 64, 60, 0);
  exercise(params(16, 2, 5, 32, 3, 128, 32, 16), 5, 4096, 700, 128);
  exercise(params(32, 8, 4, 32, 2, 128, 0, 0), 1, 16, 0, 0);  // empty lengths
  if (stub_launches == before) {
    fprintf(stderr, "no launch reached\n");
    return 2;
  }

  // rejected parameters
  kvq_sizes sz;
  const kvq_params ok = params(32, 8, 4, 32, 2, 128, 0, 0);
  kvq_params p = ok;
  p.num_q_heads = 0;
  EXPECT(kvq_cache_sizes(&p, 1, 16, &sz), KVQ_EINVAL);
  p = ok;
  p.num_q_heads = 24;  // 3 query heads per kv head
  EXPECT(kvq_cache_sizes(&p, 1, 16, &sz), KVQ_EUNSUPPORTED);
  p = ok;
  p.k_bits = 7;
  EXPECT(kvq_cache_sizes(&p, 1, 16, &sz), KVQ_EUNSUPPORTED);
  p = ok;
  p.v_group = 32;
  EXPECT(kvq_cache_sizes(&p, 1, 16, &sz), KVQ_EUNSUPPORTED);
  p = ok;
  p.head_dim = 64;
  EXPECT(kvq_cache_sizes(&p, 1, 16, &sz), KVQ_EUNSUPPORTED);
  p = ok;
  p.window = -1;
  EXPECT(kvq_cache_sizes(&p, 1, 16, &sz), KVQ_EINVAL);
  p = ok;
  p.value_rotation = 1;
  p.window = 16;
  EXPECT(kvq_cache_sizes(&p, 1, 16, &sz), KVQ_EUNSUPPORTED);
  EXPECT(kvq_cache_sizes(nullptr, 1, 16, &sz), KVQ_EINVAL);
  EXPECT(kvq_cache_sizes(&ok, 0, 16, &sz), KVQ_EINVAL);
  EXPECT(kvq_cache_sizes(&ok, 1, -1, &sz), KVQ_EINVAL);
  EXPECT(kvq_cache_sizes(&ok, 1, 16, nullptr), KVQ_EINVAL);
  // extreme sizes: rejected or computed without overflow
  (void)kvq_cache_sizes(&ok, INT32_MAX, INT64_MAX, &sz);
  (void)kvq_cache_sizes(&ok, INT32_MAX, (int64_t)1 << 40, &sz);
  (void)kvq_decode_workspace_bytes(&ok, INT32_MAX, INT32_MAX);
  (void)kvq_dense_workspace_bytes(&ok, INT32_MAX, INT32_MAX);
  (void)kvq_error_budget_workspace_bytes(&ok, INT32_MAX, INT32_MAX);
  (void)kvq_decode_splits(&ok, INT32_MAX, INT32_MAX, KVQ_BF16);
  (void)kvq_decode_workspace_bytes(&ok, 1, INT64_MAX);
  (void)kvq_error_budget_workspace_bytes(&ok, 1, INT64_MAX);
  (void)kvq_dense_workspace_bytes(&ok, 1, INT64_MAX);
  if (kvq_decode_workspace_bytes(&ok, 0, 10) != 0 || kvq_error_budget_workspace_bytes(&ok, 2, -1) != 0) ++failures;

  // bad caches
  kvq_cache c = cache_of(ok, 2, 64);
  c.pages = nullptr;
  EXPECT(kvq_quantize_append(&ok, &c, (const int32_t *)fake(5), nullptr, fake(7), fake(8), 4, nullptr), KVQ_EINVAL);
  c = cache_of(ok, 2, 64);
  c.pages = (char *)fake(1) + 8;
  EXPECT(kvq_quantize_append(&ok, &c, (const int32_t *)fake(5), nullptr, fake(7), fake(8), 4, nullptr), KVQ_EINVAL);
  c = cache_of(ok, 2, 64);
  c.error_flags = (uint32_t *)((char *)fake(22) + 2);
  EXPECT(kvq_quantize_append(&ok, &c, (const int32_t *)fake(5), nullptr, fake(7), fake(8), 4, nullptr), KVQ_EINVAL);
  const kvq_params paged = params(32, 8, 4, 32, 2, 128, 0, 16);
  c = cache_of(paged, 2, 64, 0);
  EXPECT(kvq_quantize_append(&paged, &c, (const int32_t *)fake(5), nullptr, fake(7), fake(8), 4, nullptr),
         KVQ_EINVAL);

  // device status and status strings
  uint32_t flags = 7;
  c = cache_of(ok, 2, 64);
  EXPECT(kvq_device_status(&c, &flags, nullptr), KVQ_EINVAL);  // no error word
  c.error_flags = (uint32_t *)fake(22);
  EXPECT(kvq_device_status(&c, &flags, nullptr), KVQ_OK);
  EXPECT(kvq_device_status(&c, nullptr, nullptr), KVQ_EINVAL);
  for (int s = -1; s < 8; ++s)
    if (!kvq_status_str((kvq_status)s)) ++failures;

  if (failures) {
    fprintf(stderr, "%d unexpected statuses\n", failures);
    return 1;
  }
  printf("ok %d launches\n", stub_launches);
  return 0;
}
