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

  // Each row waits for up to four dependent loads (the request's length, its selection
  // entry, its page, its data).  All passes of the work-group go through each stage
  // together, and the selection entries are read before the length is known, assuming
  // ns = n_sink (a request shorter than the sink re-reads them), so the chain costs three
  // memory round trips per work-group instead of four per pass.
  constexpr int NP = (RPB + RPP - 1) / RPP;   // passes
  const int r0 = threadIdx.x / CPR;
  int pos[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int rr = r0 + j * RPP, i = bx * RPB + rr;
    const bool row = rr < RPB && i < p.n_sink + p.k && i < p.cap;
    pos[j] = !row ? -1 : (i < p.n_sink ? i : srow[i - p.n_sink]);
  }
  if (ns != p.n_sink) {   // uniform: the request is shorter than the sink
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int rr = r0 + j * RPP, i = bx * RPB + rr;
      const bool row = rr < RPB && i < ns + p.k && i < p.cap;
      pos[j] = !row ? -1 : (i < ns ? i : srow[i - ns]);
    }
  }
  int pg[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int e = (pos[j] >= 0 && pos[j] < L) ? bt[pos[j] >> 4] : -1;
    pg[j] = (e >= 0 && e < p.num_pages) ? e : -1;
  }
  u32x4 kx[NP], vx[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    kx[j] = u32x4{0u, 0u, 0u, 0u};
    vx[j] = u32x4{0u, 0u, 0u, 0u};
    if (pg[j] >= 0) {
      const int64_t off = (int64_t)pg[j] * page_bytes + ((int64_t)g * kPage + (pos[j] & 15)) * ROW_BYTES + chunk * 16;
      // each source row is read once: streaming loads keep it out of the caches
      kx[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + off));
      vx[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + off));
    }
  }
  // Streaming (non-temporal) stores: the packed rows are read by the next fast step,
  // launches later, and write-back stores left them dirty in the caches, where the
  // write-back of several MiB slowed the next launch (the 16K step: 40.9 -> 38.6 us
  // with these, the slow step that follows the pack 2.3 us faster).  A padding entry
  // (negative) writes nothing; a position past the end or behind an invalid page
  // writes a zero row.
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    if (pos[j] < 0) continue;
    const int64_t dst = (dst_head + bx * RPB + r0 + j * RPP) * ROW_BYTES + chunk * 16;
    __builtin_nontemporal_store(kx[j], reinterpret_cast<u32x4*>(ckp + dst));
    __builtin_nontemporal_store(vx[j], reinterpret_cast<u32x4*>(cvp + dst));
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
