// Drafting and verifying requests served by one launch.
//
// ASPIRE abstract: a unified mixed forward lets drafting and verifying requests
// share one batched pass.  SparseSpec-L abstract: drafts attend over a sparse,
// recallable KV cache (here the fast step: compact + recent), verification is
// full-context attention whose statistics are kept.  The host orders a work list
// (verifying requests first, they are the longest) that travels in the kernel
// arguments; each work-group finds its entry, takes that entry's split plan and
// runs the split-K fast-step unit (vector ALUs) or the MFMA verification unit.
// Both publish split partials into one workspace whose rows are the packed query
// rows, and both finish through the same split tail.
#include "decode_unit.h"
#include "verify_unit.h"

namespace sfi {

template <int D, int G, bool SCORES>
__global__ __launch_bounds__(256) void mixed_kernel(AttnArgs base, MixedPlan plan) {
  constexpr int SD = DecodeShape<uint16_t, D, G>::SMEM, SV = VerifyShape<D>::SMEM;
  __shared__ __attribute__((aligned(16))) char smem[SD > SV ? SD : SV];
  const int bid = blockIdx.x;
  int e = 0;
  while (e + 1 < plan.n_entries && plan.wg_begin[e + 1] <= bid) ++e;
  const int ns = plan.n_split[e];
  const int local = bid - plan.wg_begin[e];
  const int g = local / ns, split = local % ns;
  AttnArgs a = base;
  a.n_split = ns;
  a.split_tokens = plan.split_tokens[e];
  a.t_q = plan.t_q[e];
  if (plan.mode[e] == 0)
    decode_unit<uint16_t, D, G, true, false>(a, plan.req[e], g, split, plan.q_row0[e], smem);
  else
    verify_unit<D, SCORES>(a, plan.req[e], g, split, plan.q_row0[e], G, smem);
}

template <int D, int G>
static hipError_t launch_mixed_g(const AttnArgs& a, const MixedPlan& plan, hipStream_t stream) {
  const int n_wg = plan.wg_begin[plan.n_entries];
  if (a.scores)
    hipLaunchKernelGGL((mixed_kernel<D, G, true>), dim3(n_wg), dim3(256), 0, stream, a, plan);
  else
    hipLaunchKernelGGL((mixed_kernel<D, G, false>), dim3(n_wg), dim3(256), 0, stream, a, plan);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_mixed_d(const AttnArgs& a, const MixedPlan& plan, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch_mixed_g<D, 1>(a, plan, stream);
    case 2: return launch_mixed_g<D, 2>(a, plan, stream);
    case 4: return launch_mixed_g<D, 4>(a, plan, stream);
    case 8: return launch_mixed_g<D, 8>(a, plan, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_mixed(const AttnArgs& a, const MixedPlan& plan, int d, int G, hipStream_t stream) {
  if (plan.n_entries < 1 || plan.wg_begin[plan.n_entries] < 1) return hipSuccess;
  if (d == 128) return launch_mixed_d<128>(a, plan, G, stream);
  if (d == 64) return launch_mixed_d<64>(a, plan, G, stream);
  return hipErrorInvalidValue;
}

}  // namespace sfi
