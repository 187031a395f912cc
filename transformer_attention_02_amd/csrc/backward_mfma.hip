// bf16 matrix-core kernels of the prefill backward (filled in below).
#include "attn_internal.h"

namespace attn {

bool bwd_mfma_supported(const BwdArgs& a) {
  (void)a;
  return false;
}

hipError_t launch_bwd_mfma(const BwdArgs& a, hipStream_t s, const TimingHook& tm) {
  (void)a;
  (void)s;
  (void)tm;
  return hipErrorInvalidValue;
}

}  // namespace attn
