// Split-K decode kernels for fp32 rows of head size 64.
#include "decode_kernels.h"

namespace sfi {

hipError_t launch_decode_f32_d64(const AttnArgs& a, int G, bool sparse, int B, hipStream_t stream) {
  return launch_decode_g<float, 64>(a, G, sparse, B, stream);
}

}  // namespace sfi
