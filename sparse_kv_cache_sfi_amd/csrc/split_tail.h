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
// A split's (m, l) pair as one 8-byte access (p is 8-byte aligned).
__device__ __forceinline__ void store_coherent2(float* p, float x, float y) {
  const uint64_t v = (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_coherent2(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

// Arrival counter of unit c.  Consecutive units' counters sit 4 KiB apart (a
// bijection of [0, kMaxCounters)): every split of every unit takes its ticket at
// about the same time, and tickets on one cache line queue behind each other.
__device__ __forceinline__ int32_t* unit_counter(int32_t* counters, int c) {
  return counters + (c % 64) * (kMaxCounters / 64) + c / 64;
}

// Buffer-resource word 3 for raw (unswizzled, untyped) buffers on CDNA, and the
// cache-policy bit (sc1) that makes a buffer load coherent at device scope, as an
// agent-scope atomic load is.
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kCoherentLoad = 16;

// Wave-wide reduction (every lane receives the result; all 64 lanes active): the
// 16-lane rows reduce with DPP (quad_perm xor 1 and 2, row_half_mirror, row_mirror;
// VALU operations, no LDS round trip), then the four row totals are combined from
// readlanes in the order (r0 op r1) op (r2 op r3).
template <typename Op>
__device__ __forceinline__ float wave_reduce(float x, Op op) {
  x = op(x, dpp_mov<0xB1>(x));
  x = op(x, dpp_mov<0x4E>(x));
  x = op(x, dpp_mov<0x141>(x));
  x = op(x, dpp_mov<0x140>(x));
  auto row = [&](int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l)); };
  return op(op(row(0), row(16)), op(row(32), row(48)));
}
__device__ __forceinline__ float wave_max(float x) {
  return wave_reduce(x, [](float u, float v) { return fmaxf(u, v); });
}
__device__ __forceinline__ float wave_sum(float x) {
  return wave_reduce(x, [](float u, float v) { return u + v; });
}

// A unit (b, g) owns R = t_q * G output rows: row r = (t, h) with t = r / G,
// h = r % G is head row (q_row0 + t) * Hq + g * G + h of out, lse and the partials
// [.., part_stride, D] / [.., part_stride, 2].
template <int D, int NT = 256>
struct SplitTail {
  static constexpr int PRE = 16;   // float4 partial loads in flight per lane

  __host__ __device__ static constexpr int bytes(int R, int ns_max) { return (2 * R * ns_max + 2 * R) * 4; }

  __device__ static int64_t row(const AttnArgs& a, int q_row0, int g, int G, int r) {
    return (int64_t)(q_row0 + r / G) * a.Hq + g * G + r % G;
  }

  // Per-row max M and weighted sum L over the splits (one wave per row); each m_s
  // in w_s is replaced by its weight 2^(m_s - M) (0 for an empty split).
  __device__ static void row_stats(int R, int ns, int ns_max, float* w_s, const float* l_s, float* M_r, float* L_r) {
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    for (int r = w; r < R; r += NT / kWave) {
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
  }

  // x combined by op over the P lanes of its group (P a power of two, uniform over the
  // wave, whose lanes must all be active) by a fixed xor tree; every lane of the group
  // receives the same value.
  template <typename Op>
  __device__ static float fold_p(float x, int P, Op op) {
    if (1 < P) x = op(x, lane_xor<1>(x));
    if (2 < P) x = op(x, lane_xor<2>(x));
    if (4 < P) x = op(x, lane_xor<4>(x));
    if (8 < P) x = op(x, lane_xor<8>(x));
    if (16 < P) x = op(x, lane_xor<16>(x));
    if (32 < P) x = op(x, lane_xor<32>(x));
    return x;
  }

  // Sums the P lane partials of one float4 output group by a fixed xor tree (P is
  // uniform over the wave, whose lanes must all be active) and, when `store`, writes the
  // group's outputs, and the row's lse, from lane p = 0 (M: the row's max in log2 units,
  // L: its weighted sum).
  __device__ static void fold_store(const AttnArgs& a, int q_row0, int g, int G, int r, int e4, int P, int p,
                                    float4 acc, float M, float L, bool store) {
    const auto add = [](float u, float v) { return u + v; };
    acc.x = fold_p(acc.x, P, add);
    acc.y = fold_p(acc.y, P, add);
    acc.z = fold_p(acc.z, P, add);
    acc.w = fold_p(acc.w, P, add);
    if (store && p == 0) {
      const int64_t orow = row(a, q_row0, g, G, r);
      *reinterpret_cast<float4*>(a.out + orow * D + e4 * 4) =
          L > 0.f ? make_float4(acc.x / L, acc.y / L, acc.z / L, acc.w / L) : make_float4(0.f, 0.f, 0.f, 0.f);
      if (e4 == 0 && a.lse) a.lse[orow] = L > 0.f ? (M + log2f(L)) * kLn2 : neg_inf();
    }
  }

  // Called by every work-group of the unit after it has stored its partials.
  // The last one to arrive merges the n_split partials of each row (M = max m_s;
  // out = sum 2^(m_s - M) o_s / sum 2^(m_s - M) l_s; lse = (M + log2 of that sum) *
  // ln 2; an empty split adds 0) and returns the arrival counter to zero.
  //
  // The merge sits on the critical path of every call and is run by one
  // work-group, so it is built for few instructions and one memory round trip:
  // outputs are handled as float4 groups, P consecutive lanes share a group and
  // take splits p, p + P, ... (16-byte device-coherent loads), and the P lane sums
  // are combined by a fixed xor tree.  The row statistics come either from each
  // lane's own (m, l) pairs folded by the same tree (a decode unit: no LDS, no
  // barrier) or from all pairs staged in LDS and reduced by one wave per row.  Every
  // sum has a fixed order, so the result does not depend on which work-group
  // merges.  tail: LDS of bytes(R, ns_max).
  __device__ static void run(const AttnArgs& a, int b, int g, int q_row0, int G, int R, int ns_max, int* flag,
                             float* tail) {
    __builtin_amdgcn_s_waitcnt(0);   // this thread's partial stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
      const int ticket = __hip_atomic_fetch_add(unit_counter(a.counters, b * a.Hkv + g), 1, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
      *flag = (ticket == a.n_split - 1) ? 1 : 0;
    }
    __syncthreads();
    if (*flag == 0) return;
    merge(a, g, q_row0, G, R, ns_max, tail);
    if (threadIdx.x == 0)
      __hip_atomic_store(unit_counter(a.counters, b * a.Hkv + g), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // The merge itself: every thread of the work-group takes part (the LDS form has
  // barriers, and both forms exchange values across the lanes of whole waves).
  // Also run by a later launch on the partials an earlier one left (the pack or the
  // fast-step launch that finishes a deferred slow step), where the device-coherent
  // loads cost nothing extra.
  __device__ static void merge(const AttnArgs& a, int g, int q_row0, int G, int R, int ns_max, float* tail) {
    const int tid = threadIdx.x;
    constexpr int D4 = D / 4;
    const int ns = a.n_split;
    float* w_s = tail;                // [R][ns_max]: m, then the weight 2^(m - M)
    float* l_s = tail + R * ns_max;   // [R][ns_max]
    float* M_r = tail + 2 * R * ns_max;
    float* L_r = M_r + R;

    // Lanes per float4 group: a power of two, at most a wave, filling 256 threads.  P
    // fixes the summation order, so it is set by that width rather than NT: a wider
    // work-group would leave its extra threads idle and add in exactly the order of
    // the slow step's own merge.
    const int n_grp = R * D4;
    int P = 1;
    while (P < kWave && 2 * P * n_grp <= 256) P *= 2;
    const int grp0 = tid / P, p = tid % P;
    // The unit's partial rows as one buffer resource (its base is uniform over the
    // work-group); loads outside it return zero.
    const int64_t row0 = row(a, q_row0, g, G, 0);
    const int64_t row_span = row(a, q_row0, g, G, R - 1) - row0 + 1;
    const __amdgpu_buffer_rsrc_t part = __builtin_amdgcn_make_buffer_rsrc(
        a.part_o + row0 * a.part_stride * D, (short)0, (int)(row_span * a.part_stride * D * 4), kBufferRsrcWord3);
    auto offset = [&](int grp, int s) {
      const int r = grp / D4;
      return (int)(((row(a, q_row0, g, G, r) - row0) * a.part_stride + s) * (D * 4) + (grp % D4) * 16);
    };
    auto load4 = [&](int off) { return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(part, off, 0, kCoherentLoad)); };

    // One output group per thread and all its splits in one batch of loads (the decode
    // layers' units: two rows of 128 dimensions and up to 2 PRE splits): each lane also
    // loads the (m, l) pairs of its own splits, and the group's P lanes combine the row
    // max and the weighted sum by the same xor tree as the output sums, so this merge
    // takes one memory round trip and no LDS or barrier.  (At d 64 its registers would
    // cost the decode kernels a wave per SIMD; they keep the merge below.)
    if (D >= 128 && n_grp * P <= NT && ns <= P * PRE) {
      const bool act = grp0 < n_grp;
      const int r = act ? grp0 / D4 : 0;
      const float* mlp = a.part_ml + row(a, q_row0, g, G, r) * a.part_stride * 2;
      float4 ov[PRE];
      float2 ml[PRE];
#pragma unroll
      for (int j = 0; j < PRE; ++j) {
        const int sj = p + P * j;
        const bool in = act && sj < ns;
        ov[j] = in ? load4(offset(grp0, sj)) : make_float4(0.f, 0.f, 0.f, 0.f);
        ml[j] = in ? load_coherent2(mlp + sj * 2) : make_float2(neg_inf(), 0.f);
      }
      float M = neg_inf();
#pragma unroll
      for (int j = 0; j < PRE; ++j) M = fmaxf(M, ml[j].x);
      M = fold_p(M, P, [](float u, float v) { return fmaxf(u, v); });
      float L = 0.f;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int j = 0; j < PRE; ++j) {
        const float wt = (ml[j].x == neg_inf()) ? 0.f : exp2_fast(ml[j].x - M);
        L = fmaf(wt, ml[j].y, L);
        acc.x = fmaf(wt, ov[j].x, acc.x);
        acc.y = fmaf(wt, ov[j].y, acc.y);
        acc.z = fmaf(wt, ov[j].z, acc.z);
        acc.w = fmaf(wt, ov[j].w, acc.w);
      }
      L = fold_p(L, P, [](float u, float v) { return u + v; });
      fold_store(a, q_row0, g, G, r, grp0 % D4, P, p, acc, M, L, act);
      return;
    }

    float4 first[PRE];
    if (grp0 < n_grp) {
#pragma unroll
      for (int j = 0; j < PRE; ++j) {
        const int sj = p + P * j;
        first[j] = sj < ns ? load4(offset(grp0, sj)) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    for (int i = tid; i < R * ns; i += NT) {
      const int r = i / ns, s = i % ns;
      const float2 ml = load_coherent2(a.part_ml + (row(a, q_row0, g, G, r) * a.part_stride + s) * 2);
      w_s[r * ns_max + s] = ml.x;
      l_s[r * ns_max + s] = ml.y;
    }
    __syncthreads();
    row_stats(R, ns, ns_max, w_s, l_s, M_r, L_r);
    __syncthreads();
    for (int grp = grp0; grp < n_grp; grp += NT / P) {
      const int r = grp / D4;
      const float* wr = w_s + r * ns_max;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      auto add = [&](float wt, const float4& v) {
        acc.x = fmaf(wt, v.x, acc.x);
        acc.y = fmaf(wt, v.y, acc.y);
        acc.z = fmaf(wt, v.z, acc.z);
        acc.w = fmaf(wt, v.w, acc.w);
      };
      int j0 = 0;
      if (grp == grp0) {
#pragma unroll
        for (int j = 0; j < PRE; ++j)
          if (p + P * j < ns) add(wr[p + P * j], first[j]);
        j0 = PRE;
      }
      for (; p + P * j0 < ns; j0 += PRE) {
        float4 v[PRE];
#pragma unroll
        for (int j = 0; j < PRE; ++j) {
          const int sj = p + P * (j0 + j);
          v[j] = sj < ns ? load4(offset(grp, sj)) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int j = 0; j < PRE; ++j)
          if (p + P * (j0 + j) < ns) add(wr[p + P * (j0 + j)], v[j]);
      }
      fold_store(a, q_row0, g, G, r, grp % D4, P, p, acc, M_r[r], L_r[r], true);
    }
  }
};

}  // namespace sfi
