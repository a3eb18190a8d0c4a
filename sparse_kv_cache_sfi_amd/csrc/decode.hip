// Launcher of the split-K decode (one query token per request): dispatch on the
// element type and head size to the kernels instantiated in decode_*.hip.
#include "kernels.h"

namespace sfi {

hipError_t launch_decode_bf16_d128(const AttnArgs& a, int G, bool sparse, int B, hipStream_t stream);
hipError_t launch_decode_bf16_d64(const AttnArgs& a, int G, bool sparse, int B, hipStream_t stream);
hipError_t launch_decode_f32_d128(const AttnArgs& a, int G, bool sparse, int B, hipStream_t stream);
hipError_t launch_decode_f32_d64(const AttnArgs& a, int G, bool sparse, int B, hipStream_t stream);

hipError_t launch_decode(const AttnArgs& a, int dtype, int d, int G, bool sparse, int B,
                         hipStream_t stream) {
  if (dtype == 1) {
    if (d == 128) return launch_decode_bf16_d128(a, G, sparse, B, stream);
    if (d == 64) return launch_decode_bf16_d64(a, G, sparse, B, stream);
  } else {
    if (d == 128) return launch_decode_f32_d128(a, G, sparse, B, stream);
    if (d == 64) return launch_decode_f32_d64(a, G, sparse, B, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace sfi
