// Split-K partial publication and the merge done by the last work-group of a
// (request, KV head) unit.  Shared by the decode and the verification kernels.
#pragma once

#include "common.h"
#include "kernels.h"

namespace sfi {

// Split partials cross XCDs, whose L2 caches are not coherent with each other.
// They are written and read with agent-scope atomic accesses (coherent at the
// device level, no cache-wide write-back or invalidate), and a writer drains its
// stores before it takes a ticket.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave-wide reductions (all 64 lanes receive the result).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

// A unit (b, g) owns R = t_q * G output rows: row r = (t, h) with t = r / G,
// h = r % G is head row (q_row0 + t) * Hq + g * G + h of out, lse and the partials
// [.., part_stride, D] / [.., part_stride, 2].
template <int D>
struct SplitTail {
  static constexpr int NT = 256;
  static constexpr int BATCH = 32;

  __host__ __device__ static constexpr int bytes(int R, int ns_max) { return (2 * R * ns_max + 2 * R) * 4; }

  __device__ static int64_t row(const AttnArgs& a, int q_row0, int g, int G, int r) {
    return (int64_t)(q_row0 + r / G) * a.Hq + g * G + r % G;
  }

  // Called by every work-group of the unit after it has stored its partials.
  // The last one to arrive merges the n_split partials of each row (M = max m_s;
  // out = sum 2^(m_s - M) o_s / sum 2^(m_s - M) l_s; lse = (M + log2 of that sum) *
  // ln 2; an empty split adds 0), in fixed split order, and returns the arrival
  // counter to zero.  Every step is parallel: all (m, l) pairs are fetched at
  // once, per-row max and sum are wave reductions, and each output element keeps
  // up to BATCH partial loads in flight.  tail: LDS of bytes(R, ns_max).
  __device__ static void run(const AttnArgs& a, int b, int g, int q_row0, int G, int R, int ns_max, int* flag,
                             float* tail) {
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    constexpr int WAVES = NT / kWave;
    __builtin_amdgcn_s_waitcnt(0);   // this thread's partial stores have completed
    __syncthreads();
    if (tid == 0) {
      const int ticket = __hip_atomic_fetch_add(&a.counters[b * a.Hkv + g], 1, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
      *flag = (ticket == a.n_split - 1) ? 1 : 0;
    }
    __syncthreads();
    if (*flag == 0) return;
    const int ns = a.n_split;
    float* w_s = tail;                // [R][ns_max]: m, then the weight 2^(m - M)
    float* l_s = tail + R * ns_max;   // [R][ns_max]
    float* M_r = tail + 2 * R * ns_max;
    float* L_r = M_r + R;
    for (int i = tid; i < R * ns; i += NT) {
      const int r = i / ns, s = i % ns;
      const float* ml = a.part_ml + (row(a, q_row0, g, G, r) * a.part_stride + s) * 2;
      w_s[r * ns_max + s] = load_coherent(ml);
      l_s[r * ns_max + s] = load_coherent(ml + 1);
    }
    __syncthreads();
    for (int r = w; r < R; r += WAVES) {
      float M = neg_inf();
      for (int s = lane; s < ns; s += kWave) M = fmaxf(M, w_s[r * ns_max + s]);
      M = wave_max(M);
      float L = 0.f;
      for (int s = lane; s < ns; s += kWave) {
        const float m = w_s[r * ns_max + s];
        const float wt = (m == neg_inf()) ? 0.f : exp2_fast(m - M);
        w_s[r * ns_max + s] = wt;
        L = fmaf(wt, l_s[r * ns_max + s], L);
      }
      L = wave_sum(L);
      if (lane == 0) {
        M_r[r] = M;
        L_r[r] = L;
      }
    }
    __syncthreads();
    for (int idx = tid; idx < R * D; idx += NT) {
      const int r = idx / D, e = idx % D;
      const int64_t orow = row(a, q_row0, g, G, r);
      const float* po = a.part_o + orow * a.part_stride * D + e;
      const float* wr = w_s + r * ns_max;
      float os = 0.f;
      for (int s0 = 0; s0 < ns; s0 += BATCH) {
        float v[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) v[j] = (s0 + j < ns) ? load_coherent(po + (int64_t)(s0 + j) * D) : 0.f;
#pragma unroll
        for (int j = 0; j < BATCH; ++j)
          if (s0 + j < ns) os = fmaf(wr[s0 + j], v[j], os);
      }
      const float ls = L_r[r];
      a.out[orow * D + e] = ls > 0.f ? os / ls : 0.f;
      if (e == 0 && a.lse) a.lse[orow] = ls > 0.f ? (M_r[r] + log2f(ls)) * kLn2 : neg_inf();
    }
    if (tid == 0) __hip_atomic_store(&a.counters[b * a.Hkv + g], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
};

}  // namespace sfi
