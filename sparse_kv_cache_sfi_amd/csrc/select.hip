// Selector: exact, deterministic per-KV-head top-k over the slow step's masked logits.
//
// SFI page, Abstract and Fig. 2: the slow step hands its masked attention logits
// over the candidate set to the Selector, which refreshes the selected memory;
// Fig. 3A runs it on the auxiliary stream.  The reading implemented here: the
// k_eff = min(k, |candidates|) highest scores, ties to the lower position,
// output in ascending position order.
//
// One 1024-thread work-group per (request, KV head) row.  Scores become
// order-preserving uint32 keys (-0.0 folded onto +0.0, so the key order is the
// IEEE order).  Four 8-bit radix passes, most significant digit first, narrow
// the key T of the k_eff-th largest element, each pass a per-wave LDS histogram
// of the keys that still match the digits found so far (integer counts:
// order-independent).  A final ordered pass takes every key > T and the
// lowest-positioned keys == T, writing positions through two block-wide
// exclusive scans, so the output is ascending and identical on every run.
#include "common.h"
#include "kernels.h"

namespace sfi {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelPerThread = 4;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of one value per thread over the work-group, in thread
// order; *total receives the sum.  sh needs kSelWaves + 1 ints.
__device__ __forceinline__ int block_exclusive_scan(int x, int* total, int* sh) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  int incl = x;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) sh[w] = incl;
  __syncthreads();
  if (w == 0) {
    const int v = lane < kSelWaves ? sh[lane] : 0;
    int vi = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(vi, off);
      if (lane >= off) vi += y;
    }
    if (lane < kSelWaves) sh[lane] = vi - v;
    if (lane == kSelWaves - 1) sh[kSelWaves] = vi;
  }
  __syncthreads();
  const int res = sh[w] + incl - x;
  *total = sh[kSelWaves];
  __syncthreads();
  return res;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ scores, int Hkv,
                                                             int64_t stride, const int32_t* __restrict__ seq_lens,
                                                             int t_q, int n_sink, int n_recent, int k,
                                                             int32_t* __restrict__ sel) {
  __shared__ uint32_t hist[kSelWaves][256];
  __shared__ int scan_sh[kSelWaves + 1];
  __shared__ int pick[2];
  const int row = blockIdx.x;
  const int b = row / Hkv;
  const int tid = threadIdx.x, w = tid / kWave;
  const float* srow = scores + (int64_t)row * stride;
  int32_t* out = sel + (int64_t)row * k;

  const int L = max(seq_lens[b], 0);
  int lo, hi;
  candidate_bounds(L, t_q, n_sink, n_recent, &lo, &hi);
  if ((int64_t)hi > stride) hi = (int)stride;
  if (lo > hi) lo = hi;
  const int n = hi - lo;
  const int k_eff = min(k, n);

  if (k_eff == n || k_eff == 0) {  // every candidate (or none) is selected
    for (int i = tid; i < k; i += kSelThreads) out[i] = i < n ? lo + i : -1;
    return;
  }

  // Radix select: after the passes, prefix == key of the k_eff-th largest element
  // and `remaining` == how many elements equal to it are taken.
  uint32_t prefix = 0u, mask = 0u;
  int remaining = k_eff;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kSelWaves * 256; i += kSelThreads) (&hist[0][0])[i] = 0u;
    __syncthreads();
    for (int i = lo + tid; i < hi; i += kSelThreads) {
      const uint32_t key = order_key(srow[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[w][(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    // Thread t < 256 owns digit 255 - t; an exclusive scan in that order gives the
    // number of matching keys with a larger digit.
    int cnt = 0;
    if (tid < 256) {
#pragma unroll
      for (int x = 0; x < kSelWaves; ++x) cnt += (int)hist[x][255 - tid];
    }
    int tot;
    const int above = block_exclusive_scan(cnt, &tot, scan_sh);
    if (tid < 256 && above < remaining && above + cnt >= remaining) {
      pick[0] = 255 - tid;
      pick[1] = above;
    }
    __syncthreads();
    const uint32_t digit = (uint32_t)pick[0];
    remaining -= pick[1];
    prefix |= digit << shift;
    mask |= 255u << shift;
    __syncthreads();
  }

  // Ordered collection: keys > prefix, plus the first `remaining` keys == prefix.
  const uint32_t T = prefix;
  int base = 0, eq_base = 0;
  for (int t0 = lo; t0 < hi; t0 += kSelThreads * kSelPerThread) {
    const int j0 = t0 + tid * kSelPerThread;
    uint32_t key[kSelPerThread];
    int ne = 0;
#pragma unroll
    for (int v = 0; v < kSelPerThread; ++v) {
      const int j = j0 + v;
      key[v] = j < hi ? order_key(srow[j]) : 0u;
      ne += (j < hi && key[v] == T) ? 1 : 0;
    }
    int tot_eq;
    int eqi = eq_base + block_exclusive_scan(ne, &tot_eq, scan_sh);
    bool take[kSelPerThread];
    int ns = 0;
#pragma unroll
    for (int v = 0; v < kSelPerThread; ++v) {
      const int j = j0 + v;
      bool t = false;
      if (j < hi) {
        if (key[v] > T) {
          t = true;
        } else if (key[v] == T) {
          t = eqi < remaining;
          ++eqi;
        }
      }
      take[v] = t;
      ns += t ? 1 : 0;
    }
    int tot_sel;
    int pos = base + block_exclusive_scan(ns, &tot_sel, scan_sh);
#pragma unroll
    for (int v = 0; v < kSelPerThread; ++v)
      if (take[v] && pos < k) out[pos++] = j0 + v;
    base += tot_sel;
    eq_base += tot_eq;
  }
  for (int i = k_eff + tid; i < k; i += kSelThreads) out[i] = -1;
}

hipError_t launch_select(const float* scores, int B, int Hkv, int64_t stride, const int32_t* seq_lens,
                         int t_q, int n_sink, int n_recent, int k, int32_t* sel, hipStream_t stream) {
  hipLaunchKernelGGL(select_kernel, dim3(B * Hkv), dim3(kSelThreads), 0, stream, scores, Hkv, stride,
                     seq_lens, t_q, n_sink, n_recent, k, sel);
  return hipGetLastError();
}

}  // namespace sfi
