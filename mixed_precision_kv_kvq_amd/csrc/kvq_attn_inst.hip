// Instantiations of the split-K attention kernel for KVQ_KB-bit keys and KVQ_VB-bit values.
// The build compiles this file once per (key bits, value bits) pair, with -DKVQ_KB=.. -DKVQ_VB=..,
// each object defining kvq_attn::launch_k<KB>v<VB>.
#include "kvq_attn_impl.h"

#if !defined(KVQ_KB) || !defined(KVQ_VB)
#error "compile with -DKVQ_KB=<key bits> -DKVQ_VB=<value bits>"
#endif

#define KVQ_CAT4(a, b, c, d) a##b##c##d
#define KVQ_LAUNCH_NAME(kb, vb) KVQ_CAT4(launch_k, kb, v, vb)

namespace kvq_attn {

template <int G, int P, int NVG>
static hipError_t launch(const KvqAttnArgs &a, hipStream_t s) {
  (void)hipGetLastError();  // drop a stale error left by an earlier, unrelated call
  hipLaunchKernelGGL((kvq_attn_split_kernel<KVQ_KB, KVQ_VB, G, P, NVG>), dim3((unsigned)a.grid), dim3(64), 0, s, a);
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

hipError_t KVQ_LAUNCH_NAME(KVQ_KB, KVQ_VB)(const KvqAttnArgs &a, int g, int p, int nvg, hipStream_t s) {
  switch (g) {
    case 1: return by_p<1>(a, p, nvg, s);
    case 2: return by_p<2>(a, p, nvg, s);
    case 4: return by_p<4>(a, p, nvg, s);
    default: return by_p<8>(a, p, nvg, s);
  }
}

}  // namespace kvq_attn
