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
  const int b = row / Hkv;
  const int tid = threadIdx.x;
  const float* srow = scores + (int64_t)row * stride;
  int32_t* out = sel + (int64_t)row * k;

  for (int i = tid; i < kHistBins; i += kSelThreads) hist[i] = 0u;

  const int L = max(seq_lens[b], 0);
  int lo, hi;
  candidate_bounds(L, t_q, n_sink, n_recent, &lo, &hi);
  if ((int64_t)hi > stride) hi = (int)stride;
  if (lo > hi) lo = hi;
  const int n = hi - lo;
  const int k_eff = min(k, n);
  if (k_eff == n || k_eff == 0) {
    for (int i = tid; i < k; i += kSelThreads) out[i] = i < n ? lo + i : -1;
    return;
  }

  // Thread t holds candidates [lo + t V, lo + t V + V) as keys; padding never counts.
  const int j0 = lo + tid * V;
  const int nv = clampi(hi - j0, 0, V);
  uint32_t key[V];
  if ((lo & 3) == 0 && (stride & 3) == 0 && ((uintptr_t)scores & 15u) == 0) {
    // 16-byte loads: a group of four starting below hi ends below stride.
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
  __syncthreads();   // histogram cleared

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
    // The digit's bin holds exactly the keys still wanted: they are all taken, so
    // the selection is every key >= prefix (the low digits of prefix are zero), and
    // the keys == prefix are all taken as well.  The set is the one the remaining
    // passes would reach.
    if (pass < 2 && pick[2] == remaining) {
      remaining = n;
      break;
    }
  }

  // Ordered collection: every key > T, and the first `remaining` keys == T in
  // position order.  One two-value scan gives each thread the number of keys > T
  // and == T held by lower threads, hence its first output slot.
  const uint32_t T = prefix;
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
      if (t && pos < k) out[pos++] = j0 + v;
    }
  }
  for (int i = k_eff + tid; i < k; i += kSelThreads) out[i] = -1;
}

hipError_t launch_select(const float* scores, int B, int Hkv, int64_t stride, const int32_t* seq_lens,
                         int t_q, int n_sink, int n_recent, int k, int32_t* sel, hipStream_t stream) {
  // The widest candidate row any request can have decides the variant.
  const int64_t span = stride - n_sink;
  const dim3 grid(B * Hkv), block(kSelThreads);
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
