// Gather-pack device code shared by the pack launch and the fast step that packs in
// the same launch (the row copy is described in pack.hip).
#pragma once

#include "common.h"
#include "kernels.h"

namespace sfi {

// Rows per work-group: 16 while that keeps the grid within kPackSmallGrid work-groups
// (small batches: more, shorter work-groups cut the launch's latency), else 32.
constexpr int kPackSmallGrid = 4096;

struct PackArgs {
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  int32_t max_pages, num_pages, max_seq_len, Hkv;
  const int32_t* seq_lens;
  int32_t n_sink;
  const int32_t* sel;
  int32_t k;
  void* ck;
  void* cv;
  int32_t cap;
  int32_t* n_compact;
};

// Rows [bx RPB, bx RPB + RPB) of (request b, KV head g), one 16-byte chunk per thread
// and pass; block 0 of KV head 0 also writes n_compact[b].
template <int ROW_BYTES, int RPB>
__device__ __forceinline__ void pack_block(const PackArgs& p, const int bx, const int g, const int b) {
  constexpr int CPR = ROW_BYTES / 16;  // 16-byte chunks per row
  constexpr int RPP = 256 / CPR;       // rows per pass of the work-group
  const int L = clamp_len(p.seq_lens[b], p.max_seq_len, p.max_pages);
  const int ns = min(p.n_sink, L);
  const int32_t* srow = p.sel + ((int64_t)b * p.Hkv + g) * p.k;
  const int32_t* bt = p.block_table + (int64_t)b * p.max_pages;
  const int chunk = threadIdx.x % CPR;
  const int64_t dst_head = ((int64_t)b * p.Hkv + g) * p.cap;
  const int64_t page_bytes = (int64_t)p.Hkv * kPage * ROW_BYTES;
  const char* kp = reinterpret_cast<const char*>(p.k_pool);
  const char* vp = reinterpret_cast<const char*>(p.v_pool);
  char* ckp = reinterpret_cast<char*>(p.ck);
  char* cvp = reinterpret_cast<char*>(p.cv);

  for (int rr = threadIdx.x / CPR; rr < RPB; rr += RPP) {
    const int i = bx * RPB + rr;
    if (i >= ns + p.k || i >= p.cap) continue;
    const int pos = i < ns ? i : srow[i - ns];
    if (pos < 0) continue;
    u32x4 kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
    if (pos < L) {
      const int pg = bt[pos >> 4];
      if (pg >= 0 && pg < p.num_pages) {
        const int64_t off = (int64_t)pg * page_bytes + ((int64_t)g * kPage + (pos & 15)) * ROW_BYTES + chunk * 16;
        // each source row is read once: streaming loads keep it out of the caches
        kx = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + off));
        vx = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + off));
      }
    }
    // Streaming (non-temporal) stores: the packed rows are read by the next fast step,
    // launches later, and write-back stores left them dirty in the caches, where the
    // write-back of several MiB slowed the next launch (the 16K step: 40.9 -> 38.6 us
    // with these, the slow step that follows the pack 2.3 us faster).
    const int64_t dst = (dst_head + i) * ROW_BYTES + chunk * 16;
    __builtin_nontemporal_store(kx, reinterpret_cast<u32x4*>(ckp + dst));
    __builtin_nontemporal_store(vx, reinterpret_cast<u32x4*>(cvp + dst));
  }

  if (bx == 0 && g == 0) {
    // n_compact[b] = ns + (entries of head 0's selection before its first negative one).
    __shared__ int first_neg;
    if (threadIdx.x == 0) first_neg = p.k;
    __syncthreads();
    const int32_t* s0 = p.sel + (int64_t)b * p.Hkv * p.k;
    for (int i = threadIdx.x; i < p.k; i += 256)
      if (s0[i] < 0) atomicMin(&first_neg, i);
    __syncthreads();
    if (threadIdx.x == 0) p.n_compact[b] = ns + first_neg;
  }
}

}  // namespace sfi
