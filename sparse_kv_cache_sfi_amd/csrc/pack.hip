// Cache reorganisation: gather-pack sink + selected tokens into the compact buffer.
//
// SFI page, Fig. 3B: sink and selected tokens are packed into a contiguous
// compact buffer so that the fast step streams them sequentially; Fig. 3A runs
// this reorganisation on the auxiliary stream.  Row i of (request b, KV head g)
// is the token at position i for i < ns = min(n_sink, L_b), and the token at
// sel_idx[b, g, i - ns] after that.  Each thread moves one 16-byte chunk of a
// K row and of the matching V row (bitwise copy).  Positions outside [0, L_b),
// or behind an invalid block-table entry, produce zero rows; negative entries
// of sel_idx (padding) produce no row.
//
// With MD = d > 0 the launch also finishes a slow step whose kernel left its split-K
// partials behind (SFI page, Fig. 2: the slow step feeds the Selector, which feeds this
// reorganisation; on one stream this launch is the first with spare CUs after the
// slow step): the first work-group of every (request b, KV head g) merges the partials
// of query heads g G ... g G + G - 1 of request b into out and lse with the slow step's
// own merge code, while the other work-groups copy rows.
#include "common.h"
#include "kernels.h"
#include "pack_unit.h"
#include "split_tail.h"

namespace sfi {

// Query heads per KV head, at most (the merge's LDS is sized for it).
constexpr int kPackMergeRows = 8;

template <int ROW_BYTES, int RPB, int MD>
__global__ __launch_bounds__(256) void pack_kernel(PackArgs p, AttnArgs m) {
  const int b = blockIdx.z, g = blockIdx.y;
  if constexpr (MD > 0) {
    if (blockIdx.x == 0) {
      __shared__ float tail[SplitTail<MD>::bytes(kPackMergeRows, kMaxSplits) / 4];
      const int G = m.Hq / m.Hkv;
      SplitTail<MD>::merge(m, g, b, G, G, kMaxSplits, tail);
      return;
    }
  }
  pack_block<ROW_BYTES, RPB>(p, blockIdx.x - (MD > 0 ? 1 : 0), g, b);
}

hipError_t launch_pack(int dtype, int d, int B, int Hkv, const void* k_pool, const void* v_pool,
                       const int32_t* block_table, int max_pages, int num_pages, int max_seq_len,
                       const int32_t* seq_lens, int n_sink, const int32_t* sel, int k, void* ck, void* cv,
                       int cap, int32_t* n_compact, hipStream_t stream, const AttnArgs* merge) {
  PackArgs p{k_pool, v_pool, block_table, max_pages, num_pages, max_seq_len, Hkv, seq_lens,
             n_sink, sel, k, ck, cv, cap, n_compact};
  const int64_t rows = (int64_t)n_sink + k;
  const bool small = (int64_t)B * Hkv * ((rows + 15) / 16) <= kPackSmallGrid;
  const int rpb = small ? 16 : 32;
  const int md = merge ? d : 0;
  const dim3 grid((unsigned)((rows + rpb - 1) / rpb + (md ? 1 : 0)), Hkv, B), block(256);
  const AttnArgs m = merge ? *merge : AttnArgs{};
  const int row_bytes = d * (dtype == 1 ? 2 : 4);
#define SFI_PACK(RB, RPB_)                                                                            \
  do {                                                                                                \
    if (md == 128) hipLaunchKernelGGL((pack_kernel<RB, RPB_, 128>), grid, block, 0, stream, p, m);    \
    else if (md == 64) hipLaunchKernelGGL((pack_kernel<RB, RPB_, 64>), grid, block, 0, stream, p, m); \
    else hipLaunchKernelGGL((pack_kernel<RB, RPB_, 0>), grid, block, 0, stream, p, m);                \
  } while (0)
  switch (row_bytes * (small ? 1 : -1)) {
    case 128: SFI_PACK(128, 16); break;
    case 256: SFI_PACK(256, 16); break;
    case 512: SFI_PACK(512, 16); break;
    case -128: SFI_PACK(128, 32); break;
    case -256: SFI_PACK(256, 32); break;
    case -512: SFI_PACK(512, 32); break;
    default: return hipErrorInvalidValue;
  }
#undef SFI_PACK
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- calibration copy
// Plain streaming copy of n16 16-byte words; its hardware byte counters calibrate
// the counters read on the attention kernels.
__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                          int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- streaming read
// Plain streaming read of n16 16-byte words (each read once; consecutive threads read
// consecutive words, the grid strides through the buffer one 16-byte load per thread
// and step, which measured faster than unrolled steps whose loads land in distant
// regions): the HBM read rate the decode kernels are compared against.  The words are
// folded into a per-thread xor whose only store is guarded by a condition that never
// holds for it (a sentinel that the fold of the buffer would have to hit exactly), so
// the loads stay and the kernel moves read traffic only.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t acc = 0u;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
    const u32x4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace sfi
