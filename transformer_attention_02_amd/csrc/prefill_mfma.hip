// bf16 MFMA prefill kernel (gfx950). Placeholder until the MFMA kernel lands.
#include "attn_internal.h"

namespace attn {

bool prefill_mfma_supported(const PrefillArgs&, int) { return false; }

hipError_t launch_prefill_mfma(const PrefillArgs&, hipStream_t) { return hipErrorInvalidDeviceFunction; }

}  // namespace attn
