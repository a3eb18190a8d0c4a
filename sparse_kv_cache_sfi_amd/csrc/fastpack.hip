// Fast step over an index set with the gather-pack, and optionally a deferred slow
// step's split-K combine, in the same launch.
//
// SFI page, Fig. 3B: the fast step attends over sink + selected + recent; the
// selected rows can be read in place through the block table (the index-set fast
// step in decode_unit.h, bit-identical to attending over the packed buffer), so
// the attention does not have to wait for the pack.  Here the pack's row blocks
// (pack_unit.h) and, when asked, the merge of a slow step that left its partials
// behind (split_tail.h) run as separate work-groups of the attention's launch:
// at small batches the attention grid leaves most CUs idle, and the pack and the
// merge fill them instead of running as launches of their own.  Work-groups
// [0, n_attn) are the attention's split-K units (dispatched first, they start at
// once), then one merge work-group per (request, KV head), then the pack's blocks.
// When the packed rows are large (the host chooses by their bytes), the launch has no
// pack blocks: the attention writes the rows it loads (a.pack_k set), so they are read
// once, and the merge rides alone.
#include <algorithm>

#include "decode_unit.h"
#include "pack_unit.h"

namespace sfi {

// Rows per pack work-group in this launch.
constexpr int kFastPackRows = 32;

template <typename T, int D, int G, bool MERGE>
__global__ __launch_bounds__(256) void fast_pack_kernel(AttnArgs a, PackArgs p, AttnArgs m, int B, int pack_x) {
  using S = DecodeShape<T, D, G>;
  constexpr int SM = SplitTail<D>::bytes(G, kMaxSplits);
  __shared__ __attribute__((aligned(16))) char smem[S::SMEM_IDX > SM ? S::SMEM_IDX : SM];
  const int n_units = B * a.Hkv;
  int bid = blockIdx.x;
  const int n_attn = a.n_split * n_units;
  if (bid < n_attn) {
    const int split = bid % a.n_split, g = (bid / a.n_split) % a.Hkv, b = bid / (a.n_split * a.Hkv);
    decode_unit<T, D, G, true, 0, false, true>(a, b, g, split, b, smem);
    return;
  }
  bid -= n_attn;
  if constexpr (MERGE) {
    if (bid < n_units) {
      SplitTail<D>::merge(m, bid % a.Hkv, bid / a.Hkv, G, G, kMaxSplits, reinterpret_cast<float*>(smem));
      return;
    }
    bid -= n_units;
  }
  if (pack_x == 0) return;   // (no pack blocks in the grid then)
  const int bx = bid % pack_x, g = (bid / pack_x) % a.Hkv, b = bid / (pack_x * a.Hkv);
  pack_block<D * (int)sizeof(T), kFastPackRows>(p, bx, g, b);
}

template <typename T, int D, int G>
static hipError_t launch_fp_t(const AttnArgs& a, const PackArgs& p, const AttnArgs* merge, bool pack_blocks, int B,
                              hipStream_t stream) {
  const int64_t units = (int64_t)B * a.Hkv;
  // at least one block per unit: block 0 of KV head 0 writes n_compact
  const int pack_x =
      pack_blocks ? (int)std::max<int64_t>(1, ((int64_t)p.n_sink + p.k + kFastPackRows - 1) / kFastPackRows) : 0;
  const int64_t n_wg = (int64_t)a.n_split * units + (merge ? units : 0) + (int64_t)pack_x * units;
  if (n_wg > INT32_MAX) return hipErrorInvalidValue;
  if (merge)
    hipLaunchKernelGGL((fast_pack_kernel<T, D, G, true>), dim3((unsigned)n_wg), dim3(256), 0, stream, a, p, *merge,
                       B, pack_x);
  else
    hipLaunchKernelGGL((fast_pack_kernel<T, D, G, false>), dim3((unsigned)n_wg), dim3(256), 0, stream, a, p,
                       AttnArgs{}, B, pack_x);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_fp_g(const AttnArgs& a, const PackArgs& p, const AttnArgs* merge, bool pack_blocks, int G,
                              int B, hipStream_t stream) {
  switch (G) {
    case 1: return launch_fp_t<T, D, 1>(a, p, merge, pack_blocks, B, stream);
    case 2: return launch_fp_t<T, D, 2>(a, p, merge, pack_blocks, B, stream);
    case 4: return launch_fp_t<T, D, 4>(a, p, merge, pack_blocks, B, stream);
    case 8: return launch_fp_t<T, D, 8>(a, p, merge, pack_blocks, B, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fast_pack(const AttnArgs& a, const PackArgs& p, const AttnArgs* merge, bool pack_blocks, int dtype,
                            int d, int G, int B, hipStream_t stream) {
  if (dtype == 1) {
    if (d == 128) return launch_fp_g<uint16_t, 128>(a, p, merge, pack_blocks, G, B, stream);
    if (d == 64) return launch_fp_g<uint16_t, 64>(a, p, merge, pack_blocks, G, B, stream);
  } else {
    if (d == 128) return launch_fp_g<float, 128>(a, p, merge, pack_blocks, G, B, stream);
    if (d == 64) return launch_fp_g<float, 64>(a, p, merge, pack_blocks, G, B, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace sfi
