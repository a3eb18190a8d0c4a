// Kernels and launchers of the MFMA multi-query verification (t_q > 1).
// The device code and its design notes are in verify_unit.h.
#include "verify_unit.h"

namespace sfi {

template <int D, bool SCORES>
__global__ __launch_bounds__(256) void verify_kernel(AttnArgs a, int G) {
  __shared__ __attribute__((aligned(16))) char smem[VerifyShape<D>::SMEM];
  verify_unit<D, SCORES>(a, blockIdx.z, blockIdx.y, blockIdx.x, blockIdx.z * a.t_q, G, smem);
}

hipError_t launch_verify(const AttnArgs& a, int d, int G, int B, hipStream_t stream) {
  const dim3 grid(a.n_split, a.Hkv, B), block(256);
  if (d == 128) {
    if (a.scores)
      hipLaunchKernelGGL((verify_kernel<128, true>), grid, block, 0, stream, a, G);
    else
      hipLaunchKernelGGL((verify_kernel<128, false>), grid, block, 0, stream, a, G);
  } else if (d == 64) {
    if (a.scores)
      hipLaunchKernelGGL((verify_kernel<64, true>), grid, block, 0, stream, a, G);
    else
      hipLaunchKernelGGL((verify_kernel<64, false>), grid, block, 0, stream, a, G);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sfi
