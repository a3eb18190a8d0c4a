// Kernels and launchers of the MFMA multi-query verification (t_q > 1).
// The device code and its design notes are in verify_unit.h.
#include "verify_unit.h"

namespace sfi {

template <int D, int G, bool SCORES>
__global__ __launch_bounds__(256) void verify_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[VerifyShape<D>::SMEM];
  verify_unit<D, SCORES>(a, blockIdx.z, blockIdx.y, blockIdx.x, blockIdx.z * a.t_q, G, smem);
}

template <int D, int G>
static hipError_t launch_g(const AttnArgs& a, int B, hipStream_t stream) {
  const dim3 grid(a.n_split, a.Hkv, B), block(256);
  if (a.scores)
    hipLaunchKernelGGL((verify_kernel<D, G, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((verify_kernel<D, G, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const AttnArgs& a, int G, int B, hipStream_t stream) {
  switch (G) {
    case 1: return launch_g<D, 1>(a, B, stream);
    case 2: return launch_g<D, 2>(a, B, stream);
    case 4: return launch_g<D, 4>(a, B, stream);
    case 8: return launch_g<D, 8>(a, B, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_verify(const AttnArgs& a, int d, int G, int B, hipStream_t stream) {
  if (d == 128) return launch_d<128>(a, G, B, stream);
  if (d == 64) return launch_d<64>(a, G, B, stream);
  return hipErrorInvalidValue;
}

}  // namespace sfi
