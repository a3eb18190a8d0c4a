// Slow-step Selector (and optionally the pack) of one (request, KV head) row, run
// by one 256-thread work-group that rides inside another launch.
//
// SFI page, Fig. 3A: the Selector and the cache reorganisation of layer i are
// meant to run while layer i+1's attention runs.  Here the Selector runs inside
// the same grid: the first work-groups of the launch are riders that select the
// top-k of layer i's masked logits for one row, while the remaining work-groups
// stream layer i+1's attention.  The Selector is latency-bound and the attention
// bandwidth-bound, so the riders' time can hide under the attention, with no
// second queue and no cross-queue event.  A rider can also pack its row's compact
// buffer (Fig. 3B), but the pack is bandwidth-bound itself and gains nothing from
// hiding; a single work-group per row also copies it slowly.
//
// Selection follows the same definition as the Selector kernel (k_eff = min(k, |C|)
// highest logits, ties to the lower position, ascending output, -1 padding):
// three radix passes of 12, 12 and 8 bits over a 4096-bin LDS histogram, then an
// ordered collection through block-wide scans.  Rows of up to 256 * 32 candidates
// keep their keys in registers (the row is read once); longer rows are read once
// per pass (they stay in L2).  The chosen positions are kept in LDS for the pack.
#pragma once

#include "common.h"
#include "kernels.h"

namespace sfi {

struct RiderShape {
  static constexpr int NT = 256;
  static constexpr int WAVES = NT / kWave;
  static constexpr int BINS = 4096;
  static constexpr int RV = 32;      // keys per thread of the register path
  static constexpr int CHUNK = 16;   // positions per thread per streaming collection step
  static constexpr int UNR = 8;      // 16-byte loads in flight per thread in a streaming pass
  static constexpr int SMEM = BINS * 4 + (WAVES + 1) * 8 + 16 + kMaxRiderK * 4;
};

__device__ __forceinline__ uint32_t rider_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sums of two values per thread, in thread order; *total gets the sums.
__device__ __forceinline__ int2 rider_scan2(int x, int y, int2* total, int2* sh) {
  constexpr int W = RiderShape::WAVES;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  int ix = x, iy = y;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int ux = __shfl_up(ix, off), uy = __shfl_up(iy, off);
    if (lane >= off) {
      ix += ux;
      iy += uy;
    }
  }
  if (lane == kWave - 1) sh[w] = make_int2(ix, iy);
  __syncthreads();
  if (w == 0) {
    const int2 v = lane < W ? sh[lane] : make_int2(0, 0);
    int vx = v.x, vy = v.y;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int ux = __shfl_up(vx, off), uy = __shfl_up(vy, off);
      if (lane >= off) {
        vx += ux;
        vy += uy;
      }
    }
    if (lane < W) sh[lane] = make_int2(vx - v.x, vy - v.y);
    if (lane == W - 1) sh[W] = make_int2(vx, vy);
  }
  __syncthreads();
  const int2 base = sh[w];
  *total = sh[W];
  __syncthreads();
  return make_int2(base.x + ix - x, base.y + iy - y);
}

// Digit of this pass holding the remaining-th largest matching key: pick[0] = digit,
// pick[1] = matching keys with a larger digit.  Thread t owns bins nb-1-c*t ...
// nb-c*t-c (c = nb / 256) and zeroes them once read.
__device__ __forceinline__ void rider_find_digit(uint32_t* hist, int nb, int remaining, int* pick, int2* scan_sh) {
  constexpr int NT = RiderShape::NT, MC = RiderShape::BINS / NT;
  const int tid = threadIdx.x;
  const int c = nb / NT;
  int cnt[MC];
  int tot_t = 0;
#pragma unroll
  for (int i = 0; i < MC; ++i) {
    cnt[i] = 0;
    if (i < c) {
      const int bin = nb - 1 - c * tid - i;
      cnt[i] = (int)hist[bin];
      hist[bin] = 0u;
      tot_t += cnt[i];
    }
  }
  int2 tot;
  int run = rider_scan2(tot_t, 0, &tot, scan_sh).x;
#pragma unroll
  for (int i = 0; i < MC; ++i)
    if (i < c) {
      if (run < remaining && run + cnt[i] >= remaining) {
        pick[0] = nb - 1 - c * tid - i;
        pick[1] = run;
      }
      run += cnt[i];
    }
  __syncthreads();
}

// Output of one thread's V consecutive candidates from j0 (those outside [lo, hi) do
// not count): keys > T, and keys == T while fewer than `remaining` equal keys come
// first.  gt0 / eq0 count the keys > T / == T at lower positions.
template <int V>
__device__ __forceinline__ void rider_collect(int32_t* out, int* sel_s, int k, int j0, int lo, int hi,
                                              const uint32_t (&key)[V], uint32_t T, int remaining, int gt0,
                                              int eq0) {
  int eqi = eq0;
  int pos = gt0 + min(eq0, remaining);
#pragma unroll
  for (int v = 0; v < V; ++v) {
    if (j0 + v < lo || j0 + v >= hi) continue;
    bool t = key[v] > T;
    if (key[v] == T) {
      t = eqi < remaining;
      ++eqi;
    }
    if (t && pos < k) {
      out[pos] = j0 + v;
      sel_s[pos] = j0 + v;
      ++pos;
    }
  }
}

template <int ROW_BYTES>
__device__ __forceinline__ void refresh_row(const RefreshArgs& r, const int row, char* smem) {
  using S = RiderShape;
  constexpr int NT = S::NT, BINS = S::BINS, RV = S::RV, CHUNK = S::CHUNK, UNR = S::UNR;
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem);
  int2* scan_sh = reinterpret_cast<int2*>(smem + BINS * 4);
  int* pick = reinterpret_cast<int*>(smem + BINS * 4 + (S::WAVES + 1) * 8);
  int* sel_s = reinterpret_cast<int*>(smem + BINS * 4 + (S::WAVES + 1) * 8 + 16);
  const int tid = threadIdx.x;
  const int b = row / r.Hkv, g = row % r.Hkv;
  const float* srow = r.scores + (int64_t)row * r.score_stride;
  int32_t* out = r.sel + (int64_t)row * r.k;

  for (int i = tid; i < BINS; i += NT) hist[i] = 0u;
  const int L = clamp_len(r.seq_lens[b], r.max_seq_len, r.max_pages);
  int lo, hi;
  candidate_bounds(L, 1, r.n_sink, r.n_recent, &lo, &hi);
  if ((int64_t)hi > r.score_stride) hi = (int)r.score_stride;
  if (lo > hi) lo = hi;
  const int n = hi - lo;
  const int k_eff = min(r.k, n);
  // 16-byte loads when the row allows them: groups of four start at lo4 (aligned), and
  // a group that starts below hi ends below the row stride.
  const bool vec = (r.score_stride & 3) == 0 && ((uintptr_t)r.scores & 15u) == 0;
  const int lo4 = vec ? (lo & ~3) : lo;
  auto load4 = [&](int j) {   // candidates j .. j + 3 (zero where j + e >= hi)
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (vec) {
      if (j < hi) x = *reinterpret_cast<const float4*>(srow + j);
    } else {
      if (j < hi) x.x = srow[j];
      if (j + 1 < hi) x.y = srow[j + 1];
      if (j + 2 < hi) x.z = srow[j + 2];
      if (j + 3 < hi) x.w = srow[j + 3];
    }
    return x;
  };
  __syncthreads();   // histogram cleared

  if (k_eff == n || k_eff == 0) {   // every candidate, or none
    for (int i = tid; i < r.k; i += NT) {
      const int v = i < n ? lo + i : -1;
      out[i] = v;
      sel_s[i] = v;
    }
  } else if (lo4 + NT * RV >= hi) {
    // Keys in registers: thread t holds positions [lo4 + t RV, lo4 + t RV + RV).
    const int j0 = lo4 + tid * RV;
    uint32_t key[RV];
#pragma unroll
    for (int v = 0; v < RV; v += 4) {
      const float4 x = load4(j0 + v);
      key[v] = rider_key(x.x);
      key[v + 1] = rider_key(x.y);
      key[v + 2] = rider_key(x.z);
      key[v + 3] = rider_key(x.w);
    }
    uint32_t prefix = 0u, mask = 0u;
    int remaining = k_eff;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
      const int nb = pass == 2 ? 256 : 4096;
      const uint32_t dmask = (uint32_t)nb - 1u;
#pragma unroll
      for (int v = 0; v < RV; ++v)
        if (j0 + v >= lo && j0 + v < hi && (key[v] & mask) == prefix)
          atomicAdd(&hist[(key[v] >> shift) & dmask], 1u);
      __syncthreads();
      rider_find_digit(hist, nb, remaining, pick, scan_sh);
      remaining -= pick[1];
      prefix |= (uint32_t)pick[0] << shift;
      mask |= dmask << shift;
    }
    const uint32_t T = prefix;
    int n_gt = 0, n_eq = 0;
#pragma unroll
    for (int v = 0; v < RV; ++v) {
      const bool ok = j0 + v >= lo && j0 + v < hi;
      n_gt += (ok && key[v] > T) ? 1 : 0;
      n_eq += (ok && key[v] == T) ? 1 : 0;
    }
    int2 tot;
    const int2 ex = rider_scan2(n_gt, n_eq, &tot, scan_sh);
    rider_collect<RV>(out, sel_s, r.k, j0, lo, hi, key, T, remaining, ex.x, ex.y);
    for (int i = k_eff + tid; i < r.k; i += NT) {
      out[i] = -1;
      sel_s[i] = -1;
    }
  } else {
    // Streaming: every pass reads the row again, UNR groups of four per thread in flight.
    uint32_t prefix = 0u, mask = 0u;
    int remaining = k_eff;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
      const int nb = pass == 2 ? 256 : 4096;
      const uint32_t dmask = (uint32_t)nb - 1u;
      auto count = [&](int j, float f) {
        if (j < lo || j >= hi) return;
        const uint32_t key = rider_key(f);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
      };
      for (int j0 = lo4 + 4 * tid; j0 < hi; j0 += 4 * NT * UNR) {
        float4 x[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) x[u] = load4(j0 + 4 * NT * u);
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int j = j0 + 4 * NT * u;
          count(j, x[u].x);
          count(j + 1, x[u].y);
          count(j + 2, x[u].z);
          count(j + 3, x[u].w);
        }
      }
      __syncthreads();
      rider_find_digit(hist, nb, remaining, pick, scan_sh);
      remaining -= pick[1];
      prefix |= (uint32_t)pick[0] << shift;
      mask |= dmask << shift;
    }
    const uint32_t T = prefix;
    int gt_base = 0, eq_base = 0;
    for (int c0 = lo4; c0 < hi; c0 += NT * CHUNK) {
      const int j0 = c0 + tid * CHUNK;
      uint32_t key[CHUNK];
#pragma unroll
      for (int v = 0; v < CHUNK; v += 4) {
        const float4 x = load4(j0 + v);
        key[v] = rider_key(x.x);
        key[v + 1] = rider_key(x.y);
        key[v + 2] = rider_key(x.z);
        key[v + 3] = rider_key(x.w);
      }
      int n_gt = 0, n_eq = 0;
#pragma unroll
      for (int v = 0; v < CHUNK; ++v) {
        const bool ok = j0 + v >= lo && j0 + v < hi;
        n_gt += (ok && key[v] > T) ? 1 : 0;
        n_eq += (ok && key[v] == T) ? 1 : 0;
      }
      int2 tot;
      const int2 ex = rider_scan2(n_gt, n_eq, &tot, scan_sh);
      rider_collect<CHUNK>(out, sel_s, r.k, j0, lo, hi, key, T, remaining, gt_base + ex.x, eq_base + ex.y);
      gt_base += tot.x;
      eq_base += tot.y;
    }
    for (int i = k_eff + tid; i < r.k; i += NT) {
      out[i] = -1;
      sel_s[i] = -1;
    }
  }
  if (!r.ck) return;   // selection only: the caller packs
  __syncthreads();     // the selection is complete in LDS

  // Pack: row i of the compact buffer is position i for i < ns, then sel[i - ns].
  constexpr int CPR = ROW_BYTES / 16;
  constexpr int RPP = NT / CPR;
  constexpr int PU = 8;
  const int ns = min(r.n_sink, L);
  const int rows = min(ns + r.k, r.cap);
  const int chunk = tid % CPR;
  const int32_t* bt = r.block_table + (int64_t)b * r.max_pages;
  const int64_t page_bytes = (int64_t)r.Hkv * kPage * ROW_BYTES;
  const int64_t dst_head = ((int64_t)b * r.Hkv + g) * r.cap;
  const char* kp = reinterpret_cast<const char*>(r.k_pool);
  const char* vp = reinterpret_cast<const char*>(r.v_pool);
  char* ckp = reinterpret_cast<char*>(r.ck);
  char* cvp = reinterpret_cast<char*>(r.cv);
  for (int i0 = tid / CPR; i0 < rows; i0 += RPP * PU) {
    int pos[PU];
    int pg[PU];
#pragma unroll
    for (int u = 0; u < PU; ++u) {
      const int i = i0 + RPP * u;
      pos[u] = i < rows ? (i < ns ? i : sel_s[i - ns]) : -1;
      pg[u] = (pos[u] >= 0 && pos[u] < L) ? bt[pos[u] >> 4] : -1;
    }
    u32x4 kx[PU], vx[PU];
#pragma unroll
    for (int u = 0; u < PU; ++u) {
      const bool valid = pg[u] >= 0 && pg[u] < r.num_pages;
      const int64_t off = valid ? (int64_t)pg[u] * page_bytes + ((int64_t)g * kPage + (pos[u] & 15)) * ROW_BYTES
                                : 0;
      const u32x4 z = {0u, 0u, 0u, 0u};
      kx[u] = valid ? *reinterpret_cast<const u32x4*>(kp + off + chunk * 16) : z;
      vx[u] = valid ? *reinterpret_cast<const u32x4*>(vp + off + chunk * 16) : z;
    }
#pragma unroll
    for (int u = 0; u < PU; ++u) {
      if (pos[u] < 0) continue;   // beyond the rows, or selection padding: no row
      const int i = i0 + RPP * u;
      const int64_t dst = (dst_head + i) * ROW_BYTES + chunk * 16;
      *reinterpret_cast<u32x4*>(ckp + dst) = kx[u];
      *reinterpret_cast<u32x4*>(cvp + dst) = vx[u];
    }
  }
  if (g == 0 && tid == 0) r.n_compact[b] = ns + k_eff;
}

}  // namespace sfi
