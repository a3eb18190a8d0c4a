// Kernels and launch templates of the split-K decode (one query token per request).
// The device code and its design notes are in decode_unit.h; each decode_*.hip file
// instantiates one (dtype, head size), so the four compile in parallel.
#pragma once

#include "decode_unit.h"

namespace sfi {

template <typename T, int D, int G, bool SPARSE, int SCORES, bool APPEND = false, bool INDEXED = false,
          bool DEFER = false>
__global__ __launch_bounds__(256) void decode_kernel(AttnArgs a) {
  using S = DecodeShape<T, D, G>;
  __shared__ __attribute__((aligned(16))) char smem[(INDEXED || SCORES == 1) ? S::SMEM_IDX : S::SMEM];
  decode_unit<T, D, G, SPARSE, SCORES, APPEND, INDEXED, DEFER>(a, blockIdx.z, blockIdx.y, blockIdx.x, blockIdx.z,
                                                               smem);
}

template <typename T, int D, int G>
static hipError_t launch_decode_t(const AttnArgs& a, bool sparse, int B, hipStream_t stream) {
  const dim3 grid(a.n_split, a.Hkv, B), block(256);
  if (sparse && a.sel_k >= 0 && a.k_new)
    hipLaunchKernelGGL((decode_kernel<T, D, G, true, 0, true, true>), grid, block, 0, stream, a);
  else if (sparse && a.sel_k >= 0)
    hipLaunchKernelGGL((decode_kernel<T, D, G, true, 0, false, true>), grid, block, 0, stream, a);
  else if (sparse && a.k_new)
    hipLaunchKernelGGL((decode_kernel<T, D, G, true, 0, true>), grid, block, 0, stream, a);
  else if (sparse)
    hipLaunchKernelGGL((decode_kernel<T, D, G, true, 0>), grid, block, 0, stream, a);
  else if (a.scores && a.head_scores)
    hipLaunchKernelGGL((decode_kernel<T, D, G, false, 2>), grid, block, 0, stream, a);
  else if (a.scores && a.defer_merge)
    hipLaunchKernelGGL((decode_kernel<T, D, G, false, 1, false, false, true>), grid, block, 0, stream, a);
  else if (a.scores)
    hipLaunchKernelGGL((decode_kernel<T, D, G, false, 1>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<T, D, G, false, 0>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_decode_g(const AttnArgs& a, int G, bool sparse, int B, hipStream_t stream) {
  switch (G) {
    case 1: return launch_decode_t<T, D, 1>(a, sparse, B, stream);
    case 2: return launch_decode_t<T, D, 2>(a, sparse, B, stream);
    case 4: return launch_decode_t<T, D, 4>(a, sparse, B, stream);
    case 8: return launch_decode_t<T, D, 8>(a, sparse, B, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sfi
