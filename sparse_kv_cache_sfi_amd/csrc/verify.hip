// Multi-query causal verification (t_q > 1).  The MFMA kernel is not built yet;
// the C-ABI layer rejects t_q > 1 before reaching these launchers.
#include "common.h"
#include "kernels.h"

namespace sfi {

hipError_t launch_verify(const AttnArgs&, int, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_mixed(const AttnArgs&, const AttnArgs&, const MixedPlan&, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_combine_mixed(const AttnArgs&, const AttnArgs&, const MixedPlan&, int, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace sfi
