// Fused causal prefill indexer + exact top-B (LongCat Sparse Attention,
// abstract: the indexer's O(L^2) causal scoring). Not built yet: the entry
// point reports LSA_ERR_UNSUPPORTED for fused selection until it is.
#include "common.hpp"
#include "kernels.hpp"

namespace lsa {

bool prefill_topk_supported(int r, int B) {
  (void)r;
  (void)B;
  return false;
}

size_t prefill_topk_workspace(int L, int Hkv, int B) {
  (void)L;
  (void)Hkv;
  (void)B;
  return 0;
}

hipError_t launch_prefill_topk(const PrefillTopkArgs& a, hipStream_t s) {
  (void)a;
  (void)s;
  return hipErrorInvalidValue;
}

}  // namespace lsa
