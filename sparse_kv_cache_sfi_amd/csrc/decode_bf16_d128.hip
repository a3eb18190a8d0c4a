// Split-K decode kernels for bf16 rows of head size 128.
#include "decode_kernels.h"

namespace sfi {

hipError_t launch_decode_bf16_d128(const AttnArgs& a, int G, bool sparse, int B, hipStream_t stream) {
  return launch_decode_g<uint16_t, 128>(a, G, sparse, B, stream);
}

}  // namespace sfi
