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
// IEEE order).  Radix passes, most significant digit first, narrow the key T of
// the k_eff-th largest element, each pass an LDS histogram of the keys that
// still match the digits found so far (integer counts: order-independent); the
// narrowing stops once the chosen bin holds exactly the keys still wanted.  A
// final ordered pass takes every key > T and the lowest-positioned keys == T,
// writing positions in ascending order through block-wide exclusive scans, so
// the output is identical on every run.  Rows of up to 65536 candidates keep
// their keys in registers (three passes of 12, 12 and 8 bits, one scan in the
// collection); longer rows stream from memory (four 8-bit passes).
#include <stdlib.h>

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
// order; *total receives the sum.  One barrier: each wave scans its lanes, publishes
// its total in sh (kSelWaves ints), and every thread then adds up the totals of the
// lower waves itself.  Two calls that share sh need a barrier between them (every
// caller has one).
__device__ __forceinline__ int block_exclusive_scan(int x, int* total, int* sh) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int incl = wave_inclusive_sum(x);
  if (lane == kWave - 1) sh[w] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    const int v = sh[i];
    before += i < w ? v : 0;
    tot += v;
  }
  *total = tot;
  return before + incl - x;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ scores, int Hkv,
                                                             int64_t stride, const int32_t* __restrict__ seq_lens,
                                                             int t_q, int n_sink, int n_recent, int k,
                                                             int32_t* __restrict__ sel) {
  __shared__ uint32_t hist[kSelWaves][256];
  __shared__ int scan_sh[kSelWaves + 1];
  __shared__ int scan_sh2[kSelWaves + 1];   // the collection's second scan (no barrier between the two)
  __shared__ int pick[3];
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
  // and `remaining` == how many elements equal to it are taken (or, after an early
  // exit, prefix is a lower bound of the taken keys and all keys equal to it count).
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
      pick[2] = cnt;
    }
    __syncthreads();
    const uint32_t digit = (uint32_t)pick[0];
    const int in_bin = pick[2];
    remaining -= pick[1];
    prefix |= digit << shift;
    mask |= 255u << shift;
    __syncthreads();
    // The digit's bin holds exactly the keys still wanted: the selection is every
    // key >= prefix (its low digits are zero), as the remaining passes would find,
    // and each of them costs a read of the row.
    if (pass < 3 && in_bin == remaining) {
      remaining = n;
      break;
    }
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
    int pos = base + block_exclusive_scan(ns, &tot_sel, scan_sh2);
#pragma unroll
    for (int v = 0; v < kSelPerThread; ++v)
      if (take[v] && pos < k) out[pos++] = j0 + v;
    base += tot_sel;
    eq_base += tot_eq;
  }
  for (int i = k_eff + tid; i < k; i += kSelThreads) out[i] = -1;
}

// ---------------------------------------------------------------------------- register-resident variant
// For rows of at most 1024 * V candidates: thread t keeps candidates
// [lo + t V, lo + t V + V) as keys in registers, so the row is read once.  Three
// radix passes take 12, 12 and 8 bits; the first digit (sign, exponent, three
// mantissa bits) spreads float scores over many bins of one shared 4096-bin LDS
// histogram, which keeps atomic contention low.

constexpr int kHistBins = 4096;

// Exclusive prefix sums of two values per thread over the work-group, in thread
// order, with one barrier for both (as block_exclusive_scan); *total receives the
// sums.  sh needs kSelWaves entries.
__device__ __forceinline__ int2 block_exclusive_scan2(int x, int y, int2* total, int2* sh) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int ix = wave_inclusive_sum(x), iy = wave_inclusive_sum(y);
  if (lane == kWave - 1) sh[w] = make_int2(ix, iy);
  __syncthreads();
  int bx = 0, by = 0, tx = 0, ty = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    const int2 v = sh[i];
    bx += i < w ? v.x : 0;
    by += i < w ? v.y : 0;
    tx += v.x;
    ty += v.y;
  }
  *total = make_int2(tx, ty);
  return make_int2(bx + ix - x, by + iy - y);
}

// Among the bins of this pass (histogram `hist`, nb bins), find the digit holding
// the remaining-th largest matching key: pick[0] = digit, pick[1] = number of
// matching keys with a larger digit, pick[2] = keys in the digit's bin.  Thread t
// owns bins nb-1-c*t ... nb-c*t-c; it zeroes them once read, so the histogram is
// clear for the next pass.
__device__ __forceinline__ void find_digit(uint32_t* hist, int nb, int remaining, int* pick, int* scan_sh) {
  const int tid = threadIdx.x;
  const int c = nb / kSelThreads > 0 ? nb / kSelThreads : 1;
  const bool owner = tid * c < nb;
  int cnt[4] = {0, 0, 0, 0};
  int tot_t = 0;
  if (owner) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < c) {
        cnt[i] = (int)hist[nb - 1 - c * tid - i];
        hist[nb - 1 - c * tid - i] = 0u;
        tot_t += cnt[i];
      }
  }
  int total;
  int run = block_exclusive_scan(tot_t, &total, scan_sh);
  if (owner) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < c) {
        if (run < remaining && run + cnt[i] >= remaining) {
          pick[0] = nb - 1 - c * tid - i;
          pick[1] = run;
          pick[2] = cnt[i];
        }
        run += cnt[i];
      }
  }
  __syncthreads();
}

// The radix core shared by the register-resident kernels.  Thread t holds nv <= V
// keys (the others never count).  Finds the key T of the k_eff-th largest held key
// and how many keys equal to T are taken (`remaining`; after an early exit every key
// equal to T is taken and remaining is set to INT32_MAX).  hist: kHistBins zeroed LDS
// bins (left zeroed); pick: 3 ints; scan_sh: kSelWaves + 1 ints.
template <int V>
__device__ __forceinline__ void radix_threshold(const uint32_t (&key)[V], int nv, int k_eff, uint32_t* hist,
                                                int* pick, int* scan_sh, uint32_t* T_out, int* rem_out) {
  constexpr int kShift[3] = {20, 8, 0};
  constexpr int kBits[3] = {12, 12, 8};
  uint32_t prefix = 0u, mask = 0u;
  int remaining = k_eff;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = kShift[pass], nb = 1 << kBits[pass];
    const uint32_t dmask = (uint32_t)nb - 1u;
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (v < nv && (key[v] & mask) == prefix) atomicAdd(&hist[(key[v] >> shift) & dmask], 1u);
    __syncthreads();
    find_digit(hist, nb, remaining, pick, scan_sh);
    remaining -= pick[1];
    prefix |= (uint32_t)pick[0] << shift;
    mask |= dmask << shift;
    // The digit's bin holds exactly the keys still wanted: they are all taken, so the
    // selection is every key >= prefix (the low digits of prefix are zero), and the keys
    // == prefix are all taken as well.  The set is the one the remaining passes would reach.
    if (pass < 2 && pick[2] == remaining) {
      remaining = INT32_MAX;
      break;
    }
  }
  *T_out = prefix;
  *rem_out = remaining;
}

// Ordered collection: every held key > T, and the first `remaining` keys == T in the
// order the keys are held (thread t, then key v).  One two-value scan gives each
// thread the number of keys > T and == T held by lower threads, hence its first
// output slot; emit(slot, v) is called for each taken key v, slot < limit.
template <int V, typename Emit>
__device__ __forceinline__ void ordered_collect(const uint32_t (&key)[V], int nv, uint32_t T, int remaining,
                                                int limit, int2* scan2_sh, Emit emit) {
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    n_gt += (v < nv && key[v] > T) ? 1 : 0;
    n_eq += (v < nv && key[v] == T) ? 1 : 0;
  }
  int2 tot;
  const int2 ex = block_exclusive_scan2(n_gt, n_eq, &tot, scan2_sh);
  int eqi = ex.y;
  int pos = ex.x + max(0, min(ex.y, remaining));
#pragma unroll
  for (int v = 0; v < V; ++v) {
    if (v < nv) {
      bool t = key[v] > T;
      if (key[v] == T) {
        t = eqi < remaining;
        ++eqi;
      }
      if (t && pos < limit) emit(pos++, v);
    }
  }
}

// Keys [j0, j0 + nv) of a score row into registers (16-byte loads when aligned).
template <int V>
__device__ __forceinline__ void load_keys(const float* srow, int j0, int nv, bool vec_ok, uint32_t (&key)[V]) {
  if (vec_ok) {
    // a group of four starting below the row's end ends below the stride
#pragma unroll
    for (int v = 0; v < V; v += 4) {
      const float4 x = v < nv ? *reinterpret_cast<const float4*>(srow + j0 + v) : make_float4(0.f, 0.f, 0.f, 0.f);
      key[v] = order_key(x.x);
      key[v + 1] = order_key(x.y);
      key[v + 2] = order_key(x.z);
      key[v + 3] = order_key(x.w);
    }
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) key[v] = v < nv ? order_key(srow[j0 + v]) : 0u;
  }
}

struct SelRow {
  int lo, hi, n, k_eff;
};

__device__ __forceinline__ SelRow sel_row(const int32_t* seq_lens, int b, int64_t stride, int t_q, int n_sink,
                                          int n_recent, int k) {
  const int L = max(seq_lens[b], 0);
  SelRow r;
  candidate_bounds(L, t_q, n_sink, n_recent, &r.lo, &r.hi);
  if ((int64_t)r.hi > stride) r.hi = (int)stride;
  if (r.lo > r.hi) r.lo = r.hi;
  r.n = r.hi - r.lo;
  r.k_eff = min(k, r.n);
  return r;
}

template <int V>
__global__ __launch_bounds__(kSelThreads) void select_reg_kernel(const float* __restrict__ scores, int Hkv,
                                                                 int64_t stride, const int32_t* __restrict__ seq_lens,
                                                                 int t_q, int n_sink, int n_recent, int k,
                                                                 int32_t* __restrict__ sel) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ int scan_sh[kSelWaves + 1];
  __shared__ int2 scan2_sh[kSelWaves + 1];
  __shared__ int pick[3];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const float* srow = scores + (int64_t)row * stride;
  int32_t* out = sel + (int64_t)row * k;

  for (int i = tid; i < kHistBins; i += kSelThreads) hist[i] = 0u;
  const SelRow R = sel_row(seq_lens, row / Hkv, stride, t_q, n_sink, n_recent, k);
  if (R.k_eff == R.n || R.k_eff == 0) {   // every candidate (or none) is selected
    for (int i = tid; i < k; i += kSelThreads) out[i] = i < R.n ? R.lo + i : -1;
    return;
  }
  // Thread t holds candidates [lo + t V, lo + t V + V).
  const int j0 = R.lo + tid * V;
  const int nv = clampi(R.hi - j0, 0, V);
  uint32_t key[V];
  load_keys<V>(srow, j0, nv, (R.lo & 3) == 0 && (stride & 3) == 0 && ((uintptr_t)scores & 15u) == 0, key);
  __syncthreads();   // histogram cleared
  uint32_t T;
  int remaining;
  radix_threshold<V>(key, nv, R.k_eff, hist, pick, scan_sh, &T, &remaining);
  ordered_collect<V>(key, nv, T, remaining, k, scan2_sh, [&](int pos, int v) { out[pos] = j0 + v; });
  for (int i = R.k_eff + tid; i < k; i += kSelThreads) out[i] = -1;
}

// ---------------------------------------------------------------------------- long rows over several work-groups
// A row of many candidates is cut into S segments of `seg` positions (the last ones
// shorter or empty).  The first kernel selects each segment's own top-min(k, n_s)
// (n_s: the segment's candidates) and writes them as (key, position) pairs, in position
// order, at the segment's offset in the row's candidate list: the offsets depend only on
// the row's candidate bounds, so each work-group computes them alone.  The second
// kernel selects the row's top-k among those candidates.  This is exact: a key among the
// row's best k (score descending, position ascending) is beaten by at most k - 1 keys of
// its own segment, so it is among that segment's candidates; and the candidate list is
// in ascending position order, so the second kernel's ordered collection reproduces the
// tie-break and the ascending output.

__device__ __forceinline__ int seg_keep(const SelRow& R, int s, int seg, int k) {
  const int n_s = clampi(R.hi - (R.lo + s * seg), 0, seg);
  return min(k, n_s);
}

template <int V>
__global__ __launch_bounds__(kSelThreads) void select_segment_kernel(const float* __restrict__ scores, int Hkv,
                                                                     int64_t stride,
                                                                     const int32_t* __restrict__ seq_lens, int t_q,
                                                                     int n_sink, int n_recent, int k, int S, int seg,
                                                                     int mstride, uint32_t* __restrict__ cand_key,
                                                                     int32_t* __restrict__ cand_pos) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ int scan_sh[kSelWaves + 1];
  __shared__ int2 scan2_sh[kSelWaves + 1];
  __shared__ int pick[3];
  const int row = blockIdx.y, s = blockIdx.x;
  const int tid = threadIdx.x;
  const float* srow = scores + (int64_t)row * stride;
  const SelRow R = sel_row(seq_lens, row / Hkv, stride, t_q, n_sink, n_recent, k);
  if (R.k_eff == R.n || R.k_eff == 0) return;   // the merge kernel handles it without candidates
  const int kk = seg_keep(R, s, seg, k);
  if (kk == 0) return;
  int off = 0;
  for (int x = 0; x < s; ++x) off += seg_keep(R, x, seg, k);
  uint32_t* dkey = cand_key + (int64_t)row * mstride + off;
  int32_t* dpos = cand_pos + (int64_t)row * mstride + off;
  for (int i = tid; i < kHistBins; i += kSelThreads) hist[i] = 0u;
  const int slo = R.lo + s * seg;
  const int n_s = clampi(R.hi - slo, 0, seg);
  const int j0 = slo + tid * V;
  const int nv = clampi(slo + n_s - j0, 0, V);
  uint32_t key[V];
  load_keys<V>(srow, j0, nv, (slo & 3) == 0 && (stride & 3) == 0 && ((uintptr_t)scores & 15u) == 0, key);
  __syncthreads();   // histogram cleared
  uint32_t T = 0u;
  int remaining = INT32_MAX;   // kk == n_s: every key of the segment is a candidate
  if (kk < n_s) radix_threshold<V>(key, nv, kk, hist, pick, scan_sh, &T, &remaining);
  ordered_collect<V>(key, nv, T, remaining, kk, scan2_sh, [&](int pos, int v) {
    dkey[pos] = key[v];
    dpos[pos] = j0 + v;
  });
}

template <int V>
__global__ __launch_bounds__(kSelThreads) void select_merge_kernel(const uint32_t* __restrict__ cand_key,
                                                                   const int32_t* __restrict__ cand_pos, int Hkv,
                                                                   int64_t stride,
                                                                   const int32_t* __restrict__ seq_lens, int t_q,
                                                                   int n_sink, int n_recent, int k, int S, int seg,
                                                                   int mstride, int32_t* __restrict__ sel) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ int scan_sh[kSelWaves + 1];
  __shared__ int2 scan2_sh[kSelWaves + 1];
  __shared__ int pick[3];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  int32_t* out = sel + (int64_t)row * k;
  const SelRow R = sel_row(seq_lens, row / Hkv, stride, t_q, n_sink, n_recent, k);
  if (R.k_eff == R.n || R.k_eff == 0) {
    for (int i = tid; i < k; i += kSelThreads) out[i] = i < R.n ? R.lo + i : -1;
    return;
  }
  int m = 0;
  for (int x = 0; x < S; ++x) m += seg_keep(R, x, seg, k);
  for (int i = tid; i < kHistBins; i += kSelThreads) hist[i] = 0u;
  // Thread t holds candidates [t V, t V + V) of the row's list, keys and positions, read
  // with 16-byte loads (the row stride is a multiple of four) that are all in flight
  // together, so the collection only stores.
  const uint32_t* skey = cand_key + (int64_t)row * mstride;
  const int32_t* spos = cand_pos + (int64_t)row * mstride;
  const int c0 = tid * V;
  const int nv = clampi(m - c0, 0, V);
  uint32_t key[V];
  int32_t pos[V];
#pragma unroll
  for (int v = 0; v < V; v += 4) {
    const u32x4 x = v < nv ? *reinterpret_cast<const u32x4*>(skey + c0 + v) : u32x4{0u, 0u, 0u, 0u};
    const u32x4 y = v < nv ? *reinterpret_cast<const u32x4*>(spos + c0 + v) : u32x4{0u, 0u, 0u, 0u};
    key[v] = v < nv ? x.x : 0u;
    key[v + 1] = v + 1 < nv ? x.y : 0u;
    key[v + 2] = v + 2 < nv ? x.z : 0u;
    key[v + 3] = v + 3 < nv ? x.w : 0u;
    pos[v] = (int32_t)y.x;
    pos[v + 1] = (int32_t)y.y;
    pos[v + 2] = (int32_t)y.z;
    pos[v + 3] = (int32_t)y.w;
  }
  __syncthreads();   // histogram cleared
  uint32_t T;
  int remaining;
  radix_threshold<V>(key, nv, R.k_eff, hist, pick, scan_sh, &T, &remaining);
  ordered_collect<V>(key, nv, T, remaining, k, scan2_sh, [&](int p, int v) { out[p] = pos[v]; });
  for (int i = R.k_eff + tid; i < k; i += kSelThreads) out[i] = -1;
}

// Segments of a long-row plan: S work-groups of seg positions per row, the segment
// kernel's keys per thread V1 and the merge kernel's V2; S = 0 means one work-group
// per row.  Taken when the rows are long (at least 32768 candidates) and the segments'
// candidates are at most half of the row.
struct SelPlan {
  int S, seg, V1, V2;
};

SelPlan plan_select(int64_t span, int k) {
  SelPlan p{0, 0, 0, 0};
  // SFI_TUNE_SELECT_SEGMENTS=0 (environment, read on every call) keeps every row on one
  // work-group, for comparisons of the two paths.
  const char* env = getenv("SFI_TUNE_SELECT_SEGMENTS");
  if (env && env[0] == '0') return p;
  if (span < 32768 || k < 1) return p;
  // Segments of up to 16 keys per thread (16384 positions): at 64K (32 rows x 65276, k
  // 2048) four segments and a merge over 8192 candidates take 22.5 us, eight of 8192
  // positions and a merge over 16384 take 24.0, two of 32768 take 31.9.
  // SFI_TUNE_SELECT_SEG (environment, read on every call) sets another target size.
  const char* segenv = getenv("SFI_TUNE_SELECT_SEG");
  const int64_t seg_target = segenv && atoll(segenv) >= 1024 ? atoll(segenv) : 16 * kSelThreads;
  int64_t S = (span + seg_target - 1) / seg_target;
  if (S > 16) S = 16;
  int64_t seg = (span + S - 1) / S;
  seg = (seg + 3) / 4 * 4;
  const int64_t m = S * (int64_t)k;
  // (The merge keeps a key and a position per candidate in registers: 32 of each per
  // thread at most, 64 would spill.)
  if (2 * m > span || m > 32 * kSelThreads || seg > 64 * kSelThreads) return p;
  p.S = (int)S;
  p.seg = (int)seg;
  p.V1 = seg <= 8 * kSelThreads ? 8 : seg <= 16 * kSelThreads ? 16 : seg <= 32 * kSelThreads ? 32 : 64;
  p.V2 = m <= 4 * kSelThreads ? 4 : m <= 8 * kSelThreads ? 8 : m <= 16 * kSelThreads ? 16 : 32;
  return p;
}

// Candidates per row, padded to a multiple of four (16-byte rows for the merge's loads).
int64_t cand_stride(const SelPlan& p, int k) { return ((int64_t)p.S * k + 3) / 4 * 4; }

size_t select_workspace_bytes(int B, int Hkv, int64_t stride, int n_sink, int k) {
  const SelPlan p = plan_select(stride - n_sink, k);
  // keys (uint32) then positions (int32), [rows, cand_stride] each
  return p.S ? (size_t)B * Hkv * cand_stride(p, k) * 8 : 0;
}

hipError_t launch_select(const float* scores, int B, int Hkv, int64_t stride, const int32_t* seq_lens,
                         int t_q, int n_sink, int n_recent, int k, int32_t* sel, void* ws, hipStream_t stream) {
  // The widest candidate row any request can have decides the variant.
  const int64_t span = stride - n_sink;
  const int rows = B * Hkv;
  const SelPlan p = plan_select(span, k);
  const dim3 block(kSelThreads);
  if (p.S && ws) {
    const int mstride = (int)cand_stride(p, k);
    uint32_t* cand_key = static_cast<uint32_t*>(ws);
    int32_t* cand_pos = reinterpret_cast<int32_t*>(cand_key + (int64_t)rows * mstride);
    const dim3 g1(p.S, rows);
#define SFI_SEG(V_)                                                                                            \
  hipLaunchKernelGGL((select_segment_kernel<V_>), g1, block, 0, stream, scores, Hkv, stride, seq_lens, t_q, \
                     n_sink, n_recent, k, p.S, p.seg, mstride, cand_key, cand_pos)
    switch (p.V1) {
      case 8: SFI_SEG(8); break;
      case 16: SFI_SEG(16); break;
      case 32: SFI_SEG(32); break;
      default: SFI_SEG(64); break;
    }
#undef SFI_SEG
#define SFI_MRG(V_)                                                                                                \
  hipLaunchKernelGGL((select_merge_kernel<V_>), dim3(rows), block, 0, stream, cand_key, cand_pos, Hkv, stride, \
                     seq_lens, t_q, n_sink, n_recent, k, p.S, p.seg, mstride, sel)
    switch (p.V2) {
      case 4: SFI_MRG(4); break;
      case 8: SFI_MRG(8); break;
      case 16: SFI_MRG(16); break;
      default: SFI_MRG(32); break;
    }
#undef SFI_MRG
    return hipGetLastError();
  }
  const dim3 grid(rows);
  if (span <= 16 * kSelThreads)
    hipLaunchKernelGGL((select_reg_kernel<16>), grid, block, 0, stream, scores, Hkv, stride, seq_lens, t_q, n_sink,
                       n_recent, k, sel);
  else if (span <= 32 * kSelThreads)
    hipLaunchKernelGGL((select_reg_kernel<32>), grid, block, 0, stream, scores, Hkv, stride, seq_lens, t_q, n_sink,
                       n_recent, k, sel);
  else if (span <= 64 * kSelThreads)
    hipLaunchKernelGGL((select_reg_kernel<64>), grid, block, 0, stream, scores, Hkv, stride, seq_lens, t_q, n_sink,
                       n_recent, k, sel);
  else
    hipLaunchKernelGGL(select_kernel, grid, block, 0, stream, scores, Hkv, stride, seq_lens, t_q, n_sink, n_recent,
                       k, sel);
  return hipGetLastError();
}

}  // namespace sfi
