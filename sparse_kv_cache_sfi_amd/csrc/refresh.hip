// Slow step of layer i+1 with layer i's maintenance riding in the same launch.
// The rider and attention device code and their design notes are in
// refresh_unit.h and decode_unit.h.
#include "decode_unit.h"
#include "refresh_unit.h"

namespace sfi {

// Work-groups [0, rows) are riders (dispatched first, so they start before the
// attention grid fills the CUs); the rest are the slow step's split-K units.
template <typename T, int D, int G, int SCORES>
__global__ __launch_bounds__(256) void dense_refresh_kernel(AttnArgs a, RefreshArgs r) {
  constexpr int SD = SCORES == 1 ? DecodeShape<T, D, G>::SMEM_IDX : DecodeShape<T, D, G>::SMEM;
  constexpr int SR = RiderShape::SMEM;
  __shared__ __attribute__((aligned(16))) char smem[SD > SR ? SD : SR];
  int bid = blockIdx.x;
  if (bid < r.rows) {
    refresh_row<D * (int)sizeof(T)>(r, bid, smem);
    return;
  }
  bid -= r.rows;
  const int split = bid % a.n_split;
  const int g = (bid / a.n_split) % a.Hkv;
  const int b = bid / (a.n_split * a.Hkv);
  decode_unit<T, D, G, false, SCORES>(a, b, g, split, b, smem);
}

template <typename T, int D, int G>
static hipError_t launch_t(const AttnArgs& a, const RefreshArgs& r, int B, hipStream_t stream) {
  const int64_t n_wg = (int64_t)r.rows + (int64_t)a.n_split * a.Hkv * B;
  if (a.scores)
    hipLaunchKernelGGL((dense_refresh_kernel<T, D, G, true>), dim3((unsigned)n_wg), dim3(256), 0, stream, a, r);
  else
    hipLaunchKernelGGL((dense_refresh_kernel<T, D, G, false>), dim3((unsigned)n_wg), dim3(256), 0, stream, a, r);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_g(const AttnArgs& a, const RefreshArgs& r, int G, int B, hipStream_t stream) {
  switch (G) {
    case 1: return launch_t<T, D, 1>(a, r, B, stream);
    case 2: return launch_t<T, D, 2>(a, r, B, stream);
    case 4: return launch_t<T, D, 4>(a, r, B, stream);
    case 8: return launch_t<T, D, 8>(a, r, B, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dense_refresh(const AttnArgs& a, const RefreshArgs& r, int dtype, int d, int G, int B,
                                hipStream_t stream) {
  if (dtype == 1) {
    if (d == 128) return launch_g<uint16_t, 128>(a, r, G, B, stream);
    if (d == 64) return launch_g<uint16_t, 64>(a, r, G, B, stream);
  } else {
    if (d == 128) return launch_g<float, 128>(a, r, G, B, stream);
    if (d == 64) return launch_g<float, 64>(a, r, G, B, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace sfi
