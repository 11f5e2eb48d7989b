// Paged prefill / speculative-verify attention (MFMA). Placeholder until the
// kernel lands: the entry point reports PA_ERR_UNSUPPORTED.
#include "pa_launch.h"

namespace pa {

hipError_t launch_prefill(const PrefillArgs& a, int32_t head_dim, hipStream_t stream) {
  (void)a;
  (void)head_dim;
  (void)stream;
  return hipErrorNotSupported;
}

}  // namespace pa
