// Instantiations of the split-K attention kernel for 8-bit keys and 4-bit values.
#include "../kvq_attn_impl.h"

namespace kvq_attn {

template <int G, int P, int NVG>
static hipError_t launch(const KvqAttnArgs &a, hipStream_t s) {
  const unsigned waves = (unsigned)((int64_t)a.cache.batch * a.Hkv * a.splits);
  (void)hipGetLastError();  // drop a stale error left by an earlier, unrelated call
  hipLaunchKernelGGL((kvq_attn_split_kernel<8, 4, G, P, NVG>), dim3(waves), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <int G, int P>
static hipError_t by_nvg(const KvqAttnArgs &a, int nvg, hipStream_t s) {
  return nvg == 1 ? launch<G, P, 1>(a, s) : launch<G, P, 2>(a, s);
}

template <int G>
static hipError_t by_p(const KvqAttnArgs &a, int p, int nvg, hipStream_t s) {
  return p == 1 ? by_nvg<G, 1>(a, nvg, s) : by_nvg<G, 2>(a, nvg, s);
}

hipError_t launch_k8v4(const KvqAttnArgs &a, int g, int p, int nvg, hipStream_t s) {
  switch (g) {
    case 1: return by_p<1>(a, p, nvg, s);
    case 2: return by_p<2>(a, p, nvg, s);
    case 4: return by_p<4>(a, p, nvg, s);
    default: return by_p<8>(a, p, nvg, s);
  }
}

}  // namespace kvq_attn
