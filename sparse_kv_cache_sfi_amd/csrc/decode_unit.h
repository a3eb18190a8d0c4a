// Split-K flash-decoding device code for one query token per request, on CDNA4 vector ALUs.
//
// Serves two calls:
//  * the fast step (SFI page, Fig. 2: attention over sink + selected + recent;
//    Fig. 3B: sink and selected stream from a contiguous compact buffer, recent
//    tokens are read in place from paged KV), and
//  * the slow step (Fig. 2: dense attention over the whole paged KV, which also
//    writes the masked logits the Selector consumes).
//
// Work decomposition: one work-group (4 waves) per (split, KV head g, request b).
// All G query heads of the group share every K/V row the work-group loads.
// A K or V row is read by LPR = 8 or 16 lanes with 16-byte loads, so each load
// instruction covers 64/LPR consecutive rows with full 128-byte lines; a lane
// owns the same d/LPR dimensions of every row it touches.  Each wave streams
// its own rows (no barrier in the loop) with a two-deep register pipeline:
// the loads of iteration i+1 are in flight while iteration i is computed.
// Per row: G dot products (v_dot2_f32_bf16 for bf16) reduced across the
// row's lanes with DPP, an online softmax in log2 units whose reference maximum is
// only raised when a score exceeds it by more than 8 (2^8 headroom in fp32),
// and fp32 FMA accumulation of P*V.  The split's partial (max, sum, o) per head
// goes to the split tail (split_tail.h), or straight to out/lse when there is one
// split.
//
// The fast step's rows form a layout the host knows in full: virtual rows
// [0, cap) are the compact slots (a slot at or past n_compact is masked) and rows
// [cap, cap + n_recent) are the recent window, position rs + i for row cap + i with
// rs = max(n_sink, L - n_recent) (masked at or past L).  Split boundaries therefore
// need no device value, and a split that holds only compact rows issues its first
// K/V loads at once, before the request's length, n_compact or any block-table entry
// has arrived.  The splits either cut [0, cap + n_recent) evenly or (recent_split)
// cover [0, cap) and leave the recent window to the last split alone, which is the
// only one that waits for the length and the block table.  The index-set fast step
// uses the same layout with cap = n_sink + k: rows [0, n_sink) are the sink positions
// and rows n_sink + j the j-th entry of the selection, each read in place through the
// block table.
#pragma once

#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "split_tail.h"

namespace sfi {

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kPerChunk = 4;
};
template <>
struct Elem<uint16_t> {
  static constexpr int kPerChunk = 8;
};

template <typename T, int D, int G>
struct DecodeShape {
  static constexpr int ROW_BYTES = D * (int)sizeof(T);
  // Lanes per K/V row: 16 when the group is wide (fewer dimensions per lane keep the G
  // accumulators in registers), else 8; never more lanes than 16-byte chunks.  Wide is
  // G 8, and G 4 with rows longer than 256 bytes: at G 4 and 256-byte rows (bf16, d 128)
  // 8 lanes per row halve the cross-lane reductions per row, which outweighs the wave
  // per SIMD their accumulators cost (64K x 4 dense 174 -> 166 us).
  static constexpr int LPR = ((G >= 8 && ROW_BYTES >= 256) || (G >= 4 && ROW_BYTES > 256)) ? 16 : 8;
  static constexpr int EPC = Elem<T>::kPerChunk;               // elements per 16-byte chunk
  static constexpr int C = ROW_BYTES / (16 * LPR);             // chunks per lane per row
  static constexpr int E = C * EPC;                            // elements owned per lane
  static constexpr int ROWS = kWave / LPR;                     // rows per wave per slot
  static constexpr int U = (LPR == 16 && C == 1) ? 4 : 2;      // slots per iteration
  static constexpr int WAVES = 4;
  static constexpr int TILE = WAVES * U * ROWS;                // tokens per work-group iteration
  static constexpr int TAIL = SplitTail<D>::bytes(G, kMaxSplits);
  static constexpr int SMEM = kBtSlots * 4 + WAVES * G * D * 4 + WAVES * G * 2 * 4 + 16 + TAIL;
  // The index-set fast step also stages its split's sink and selected rows as page
  // slots (page * 16 + row, or -1), one int per token; the slow step keeps its split's
  // group-summed logits there until the loop ends.
  static constexpr int IDX_OFF = (SMEM + 15) / 16 * 16;
  static constexpr int SMEM_IDX = IDX_OFF + kMaxSplitTokens * 4;
  static_assert(C >= 1, "row too short for the lane mapping");
  static_assert(2 * U * ROWS <= kWave, "a wave's logits of an iteration pair fit its lanes");
};

template <typename T>
__device__ __forceinline__ float dot_chunk(const u32x4& q, const u32x4& k, float acc);

template <>
__device__ __forceinline__ float dot_chunk<uint16_t>(const u32x4& q, const u32x4& k, float acc) {
  acc = dot2_bf16(q.x, k.x, acc);
  acc = dot2_bf16(q.y, k.y, acc);
  acc = dot2_bf16(q.z, k.z, acc);
  acc = dot2_bf16(q.w, k.w, acc);
  return acc;
}

template <>
__device__ __forceinline__ float dot_chunk<float>(const u32x4& q, const u32x4& k, float acc) {
  acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
  acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
  acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
  acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  return acc;
}

// SCORES: 0 no logits, 1 the group-summed logits [B, Hkv, stride], 2 one logit row per
// query head [B, Hq, stride].  DEFER: leave the split partials for a later launch to
// merge (the slow step whose combine runs in the pack launch).
template <typename T, int D, int G, bool SPARSE, int SCORES, bool APPEND = false, bool INDEXED = false,
          bool DEFER = false>
__device__ __forceinline__ void decode_unit(const AttnArgs& a, const int b, const int g, const int split,
                                            const int q_row0, char* smem) {
  using S = DecodeShape<T, D, G>;
  constexpr int LPR = S::LPR, EPC = S::EPC, C = S::C, E = S::E, ROWS = S::ROWS, U = S::U;
  constexpr int WAVES = S::WAVES, TILE = S::TILE, NT = WAVES * kWave;
  // The slow step visits rows in iteration pairs (a wave's logits of a pair are
  // contiguous, see compute); the fast step visits them in plain tile order.
  constexpr bool PAIRED = SCORES == 1;
  static_assert(!INDEXED || (SPARSE && !SCORES), "the index-set path is a fast step");
  const int tid = threadIdx.x;
  const int w = tid / kWave, lane = tid % kWave;
  const int r = lane / LPR, sub = lane % LPR;
  const bool multi = a.n_split > 1;

  int* bt_s = reinterpret_cast<int*>(smem);
  float* wo = reinterpret_cast<float*>(smem + kBtSlots * 4);
  float* wml = wo + WAVES * G * D;

  // This lane's slice of the G query vectors.
  const T* qb = reinterpret_cast<const T*>(a.q) + ((int64_t)q_row0 * a.Hq + g * G) * D;
  u32x4 q[G][C];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < C; ++c)
      q[h][c] = *reinterpret_cast<const u32x4*>(qb + h * D + (c * LPR + sub) * EPC);

  // Virtual rows: [0, cap_v) compact (or sink + selection), then the recent window.
  int cap_v = 0, t1 = 0;
  int t0 = split * a.split_tokens;
  if constexpr (SPARSE) {
    cap_v = INDEXED ? a.n_sink + a.sel_k : a.cap;
    const int rec = min(a.n_recent, a.max_seq_len);
    if (!a.recent_split) {
      t1 = min(cap_v + rec, t0 + a.split_tokens);
    } else if (split == a.n_split - 1) {   // the recent window alone
      t0 = cap_v;
      t1 = cap_v + rec;
    } else {
      t1 = min(cap_v, t0 + a.split_tokens);
    }
  }
  const bool has_recent = SPARSE && t1 > cap_v;
  // A split of compact-buffer rows only never needs the request's length: it is not
  // even loaded, so nothing ahead of the split's K/V loads waits for it.
  // (A fused append always loads it: the last split stores the new row at L - 1.)
  const bool compact_only = SPARSE && !INDEXED && !APPEND && !has_recent;
  const int L = compact_only ? 0 : clamp_len(a.seq_lens[b], a.max_seq_len, a.max_pages);
  if constexpr (!SPARSE) t1 = min(L, t0 + a.split_tokens);
  const int rs = min(max(a.n_sink, L - a.n_recent), L);   // first recent position

  // Stage the block-table entries of this split's paged positions in LDS.  A dense
  // split stages every page of its token range that the table holds, without
  // waiting for the request's length (entries past the end are never used); a fast
  // step's split stages the pages of its recent rows.
  int pg_lo = 0, n_pg = 0;
  const int32_t* bt_row = a.block_table + (int64_t)b * a.max_pages;
  if constexpr (SPARSE) {
    if (has_recent) {
      const int v_first = max(t0, cap_v);
      const int p_first = rs + v_first - cap_v, p_last = min(rs + t1 - 1 - cap_v, L - 1);
      pg_lo = p_first >> 4;   // (also when nothing is staged: keeps every slot index in range)
      if (p_last >= p_first) n_pg = (p_last >> 4) - pg_lo + 1;
    }
  } else {
    pg_lo = t0 >> 4;
    n_pg = max(0, min(((t0 + a.split_tokens - 1) >> 4) - pg_lo + 1, a.max_pages - pg_lo));
  }
  for (int i = tid; i < n_pg; i += NT) {
    const int e = bt_row[pg_lo + i];
    bt_s[i] = (e >= 0 && e < a.num_pages) ? e : -1;
  }
  int* slot_s = nullptr;
  if constexpr (INDEXED) {
    // Resolve the split's sink and selected rows to page slots: first every position
    // (sink rows are their own index, selected rows come from the selection), then
    // every block-table entry, so the staging costs two memory round trips.
    slot_s = reinterpret_cast<int*>(smem + S::IDX_OFF);
    const int cnt = min(t1, cap_v) - t0;
    const int32_t* sel_row = a.sel + ((int64_t)b * a.Hkv + g) * a.sel_k;
    constexpr int PER = kMaxSplitTokens / NT;
    int pos[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = tid + j * NT;
      const int vi = t0 + i;
      pos[j] = -1;
      if (i < cnt) pos[j] = vi < a.n_sink ? vi : sel_row[vi - a.n_sink];
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = tid + j * NT;
      if (i < cnt) {
        // -1: padding (no row); -2: a position past the end or behind an invalid page
        // (a masked row, packed as zeros)
        int sl = pos[j] < 0 ? -1 : -2;
        if (pos[j] >= 0 && pos[j] < L) {
          const int e = bt_row[pos[j] >> 4];
          if (e >= 0 && e < a.num_pages) sl = e * kPage + (pos[j] & 15);
        }
        // a sink slot at or past the request's end is not a row of the packed buffer
        if (t0 + i < a.n_sink && t0 + i >= L) sl = -1;
        slot_s[i] = sl;
      }
    }
    if (a.pack_n && split == 0 && g == 0 && w == 0) {
      // n_compact of the packed buffer: min(n_sink, L) + the entries of unit 0's
      // selection before its first negative one (as the gather-pack counts them).
      const int32_t* sel0 = a.sel + (int64_t)b * a.Hkv * a.sel_k;
      float first = (float)a.sel_k;
      for (int i = lane; i < a.sel_k; i += kWave)
        if (sel0[i] < 0) first = fminf(first, (float)i);
      first = xor_fold<1>(first, [](float x, float y) { return fminf(x, y); });
      if (lane == 0) a.pack_n[b] = min(a.n_sink, L) + (int)first;
    }
  }
  // Only splits that read through the block table wait here; a fast-step split of
  // compact rows goes straight to its loads.
  if (!SPARSE || INDEXED || has_recent) __syncthreads();

  const T* kpool = reinterpret_cast<const T*>(a.k_pool);
  const T* vpool = reinterpret_cast<const T*>(a.v_pool);
  const T* ckb = kpool;
  const T* cvb = vpool;
  if constexpr (SPARSE && !INDEXED) {
    const int64_t base = ((int64_t)b * a.Hkv + g) * a.cap * D;
    ckb = reinterpret_cast<const T*>(a.ck) + base;
    cvb = reinterpret_cast<const T*>(a.cv) + base;
  }
  // Units are KV heads, or with head_div > 1 (per-query-head selection) query heads,
  // head_div of them per KV head of the pool.
  const int gp = INDEXED ? g / a.head_div : g;
  const int pool_heads = INDEXED ? a.Hkv / a.head_div : a.Hkv;
  const int64_t page_elems = (int64_t)pool_heads * kPage * D;
  const int64_t head_off = (int64_t)gp * kPage * D;
  const T* knew = nullptr;
  const T* vnew = nullptr;
  if constexpr (APPEND) {
    // The new token (position L - 1) is attended from the arguments; the last split's
    // work-group also stores it into its page (no other work-group reads that row).
    knew = reinterpret_cast<const T*>(a.k_new) + ((int64_t)b * pool_heads + gp) * D;
    vnew = reinterpret_cast<const T*>(a.v_new) + ((int64_t)b * pool_heads + gp) * D;
    constexpr int CH = D * (int)sizeof(T) / 16;
    if (split == a.n_split - 1 && g == gp * (INDEXED ? a.head_div : 1) && L > 0 && tid < 2 * CH) {
      const int pg = bt_row[(L - 1) >> 4];
      if (pg >= 0 && pg < a.num_pages) {
        const int64_t off = (int64_t)pg * page_elems + head_off + (int64_t)((L - 1) & 15) * D;
        const int c = tid % CH;
        const T* src = tid < CH ? knew : vnew;
        T* dst = const_cast<T*>(tid < CH ? kpool : vpool) + off;
        *reinterpret_cast<u32x4*>(dst + c * (16 / (int)sizeof(T))) =
            *reinterpret_cast<const u32x4*>(src + c * (16 / (int)sizeof(T)));
      }
    }
  }

  int clo = 0, chi = 0;
  float* srow = nullptr;
  if constexpr (SCORES) {
    candidate_bounds(L, a.t_q, a.n_sink, a.n_recent, &clo, &chi);
    srow = SCORES == 2 ? a.scores + ((int64_t)b * a.Hq + g * G) * a.score_stride
                       : a.scores + ((int64_t)b * a.Hkv + g) * a.score_stride;
  }

  float sbuf = 0.f;   // logits of the current iteration pair (SCORES == 1)
  float* sc_s = reinterpret_cast<float*>(smem + S::IDX_OFF);
  float m[G], l[G], o[G][E];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = neg_inf();
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[h][e] = 0.f;
  }

  // n_compact: a compact slot at or past it is masked (read in compute only; loaded
  // after the first K/V loads are out, see stream).
  int n_c = 0;

  struct Buf {
    u32x4 k[U][C];
    u32x4 v[U][C];
  };

  // Virtual row of slot u in iteration `it`.  Paired order: in pair it / 2 wave w takes
  // the 2 U ROWS consecutive rows starting at w * 2 U ROWS of the pair's 2 TILE rows, so
  // a wave's logits of both iterations are contiguous.  Plain order: iteration it is
  // rows [it TILE, it TILE + TILE) of the split.
  // A compact-buffer split of 8 or more iterations without recent rows starts at
  // iteration rot of its n_rot and wraps around (set below; 0 and 0 otherwise).
  int rot = 0, n_rot = 0;
  auto vrow = [&](int it, int u) {
    if constexpr (SPARSE && !INDEXED && !PAIRED) {
      const int x = it + rot;
      it = it < n_rot ? (x >= n_rot ? x - n_rot : x) : it;
    }
    if constexpr (PAIRED)
      return t0 + (it >> 1) * (2 * TILE) + w * (2 * U * ROWS) + (it & 1) * (U * ROWS) + u * ROWS + r;
    else
      return t0 + it * TILE + w * (U * ROWS) + u * ROWS + r;
  };
  // Where virtual row vi lives in the pool: its position p, its page pg (-1: none) and
  // whether a real row backs it (ok).  A compact-buffer row is handled by the callers.
  auto paged = [&](int vi, bool in, int& p, int& pg, bool& ok) {
    if constexpr (INDEXED) {
      if (vi < cap_v) {
        // an index-set row: its page slot was staged (p & 15 is the row in the page)
        const int sl = in ? slot_s[vi - t0] : -1;
        p = sl;
        pg = sl >> 4;
        ok = in && sl >= 0;
        return;
      }
    }
    // (The slot stays inside bt_s: a split spans at most kMaxSplitTokens positions.  A
    // dense row in the split is before L; a recent row at or past L reads a stale slot and
    // is masked.)
    p = SPARSE ? rs + vi - cap_v : vi;
    pg = bt_s[in ? (p >> 4) - pg_lo : 0];
    ok = in && pg >= 0 && (!SPARSE || p < L);
  };

  // The streaming loop.  CO: every row of the split is a compact-buffer row, whose
  // address needs no device value; that loop never reads the request's length or the
  // block table, so its loads go out at once.
  auto stream = [&](auto co_tag) {
  constexpr bool CO = decltype(co_tag)::value;
  // Issue the loads of one iteration.  Every lane always loads (rows outside the
  // split or behind an invalid page read row 0 of the pool and are masked), so the
  // loop carries no conditionally-loaded registers.
  auto issue = [&](int it, Buf& B) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int vi = vrow(it, u);
      const bool in = vi < t1;
      const T* kr;
      const T* vr;
      if (CO || (SPARSE && !INDEXED && vi < cap_v)) {
        // a row past the split reads row 0 of the pool (finite data, masked)
        kr = in ? ckb + (int64_t)vi * D : kpool;
        vr = in ? cvb + (int64_t)vi * D : vpool;
      } else {
        int p, pg;
        bool ok;
        paged(vi, in, p, pg, ok);
        int64_t off = (int64_t)(pg < 0 ? 0 : pg) * page_elems + head_off + (int64_t)(p & 15) * D;
        off = ok ? off : 0;
        kr = kpool + off;
        vr = vpool + off;
        if constexpr (APPEND) {
          if (ok && (!SPARSE || vi >= cap_v) && p == L - 1) {
            kr = knew;
            vr = vnew;
          }
        }
      }
      // Streaming (non-temporal) loads: every K/V row is read once per launch, so
      // letting it pass through the caches without displacing anything keeps L2 for
      // the index set, the block table and the split-K partials.
#pragma unroll
      for (int c = 0; c < C; ++c) {
        B.k[u][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kr + (c * LPR + sub) * EPC));
        B.v[u][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vr + (c * LPR + sub) * EPC));
      }
    }
  };

  auto compute = [&](int it, Buf& B) {
    bool in_[U], ok_[U];
    int pos_[U];
    // Compact slots in [n_compact, cap) were loaded without knowing n_compact and may
    // hold anything; a split that has such slots zeroes their V (0 * NaN would poison
    // the sums).  The test is uniform, so full compact buffers skip it.
    const bool scrub = SPARSE && !INDEXED && n_c < min(t1, cap_v);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int vi = vrow(it, u);
      in_[u] = vi < t1;
      if (CO || (SPARSE && !INDEXED && vi < cap_v)) {
        pos_[u] = vi;
        ok_[u] = in_[u] && vi < n_c;
        if (scrub && !ok_[u]) {
#pragma unroll
          for (int c = 0; c < C; ++c) B.v[u][c] = u32x4{0u, 0u, 0u, 0u};
        }
      } else {
        int pg;
        paged(vi, in_[u], pos_[u], pg, ok_[u]);
      }
      if constexpr (INDEXED) {
        // Pack while attending: the row just loaded goes to its compact slot vi
        // (zeros for a masked position, nothing for padding).
        // (The gather-pack puts selection entry j at slot min(n_sink, L) + j.)
        const bool compact = vi < cap_v;
        if (a.pack_k && in_[u] && compact && pos_[u] != -1) {
          const int dslot = vi < a.n_sink ? vi : min(a.n_sink, L) + vi - a.n_sink;
          const int64_t dst = (((int64_t)b * a.Hkv + g) * a.pack_cap + dslot) * D;
          T* dk = reinterpret_cast<T*>(a.pack_k) + dst;
          T* dv = reinterpret_cast<T*>(a.pack_v) + dst;
          const bool real = pos_[u] >= 0;
#pragma unroll
          for (int c = 0; c < C; ++c) {
            // streaming stores, as in the gather-pack (pack_unit.h)
            __builtin_nontemporal_store(real ? B.k[u][c] : u32x4{0u, 0u, 0u, 0u},
                                        reinterpret_cast<u32x4*>(dk + (c * LPR + sub) * EPC));
            __builtin_nontemporal_store(real ? B.v[u][c] : u32x4{0u, 0u, 0u, 0u},
                                        reinterpret_cast<u32x4*>(dv + (c * LPR + sub) * EPC));
          }
        }
      }
    }
    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) acc = dot_chunk<T>(q[h][c], B.k[u][c], acc);
        s[u][h] = group_sum<LPR>(acc);
      }
    if constexpr (SCORES == 2) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (sub == 0 && in_[u]) {
          const int j = pos_[u];
          const bool cand = ok_[u] && j >= clo && j < chi;
#pragma unroll
          for (int h = 0; h < G; ++h) srow[h * a.score_stride + j] = cand ? s[u][h] * a.scale : neg_inf();
        }
      }
    } else if constexpr (SCORES == 1) {
      // Group-summed logits, gathered so that lane (it mod 2) WR + u ROWS + r holds row (u, r)
      // of this iteration (every lane of a row group holds its sum; lane r LPR is the
      // source); after the second iteration of a pair the wave's 2 WR consecutive positions
      // go to the split's LDS copy, which is written out in one burst after the loop
      // (writes spread through the K/V stream cost several times their bytes).
      constexpr int WR = U * ROWS;
      float val[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float sc = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h) sc += s[u][h];
        const int j = pos_[u];
        val[u] = (ok_[u] && j >= clo && j < chi) ? sc * a.scale : neg_inf();
      }
      const int jj = lane % WR, uu = jj / ROWS, rr = jj % ROWS;
      float mine = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float t = __shfl(val[u], rr * LPR);
        mine = (u == uu) ? t : mine;
      }
      if (lane / WR == (it & 1)) sbuf = mine;
      if ((it & 1) && lane < 2 * WR) {
        const int pos = t0 + (it >> 1) * (2 * TILE) + w * (2 * WR) + lane;
        if (pos < t1) sc_s[pos - t0] = sbuf;
      }
    }
    bool need = false;
    float mx[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int u = 0; u < U; ++u) s[u][h] = ok_[u] ? s[u][h] * a.scale_log2 : neg_inf();
      mx[h] = s[0][h];
#pragma unroll
      for (int u = 1; u < U; ++u) mx[h] = fmaxf(mx[h], s[u][h]);
      need |= mx[h] > m[h] + 8.f;
    }
    if (__any(need)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m[h], mx[h]);
        const float al = (m[h] == neg_inf()) ? 0.f : exp2_fast(m[h] - mn);
        l[h] *= al;
#pragma unroll
        for (int e = 0; e < E; ++e) o[h][e] *= al;
        m[h] = mn;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float p[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        p[h] = (m[h] == neg_inf()) ? 0.f : exp2_fast(s[u][h] - m[h]);
        l[h] += p[h];
      }
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const uint32_t wv[4] = {B.v[u][c].x, B.v[u][c].y, B.v[u][c].z, B.v[u][c].w};
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float lo = bf16_lo(wv[i]);
            const float hi = bf16_hi(wv[i]);
#pragma unroll
            for (int h = 0; h < G; ++h) {
              o[h][c * EPC + 2 * i] = fmaf(p[h], lo, o[h][c * EPC + 2 * i]);
              o[h][c * EPC + 2 * i + 1] = fmaf(p[h], hi, o[h][c * EPC + 2 * i + 1]);
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = __uint_as_float(wv[i]);
#pragma unroll
            for (int h = 0; h < G; ++h) o[h][c * EPC + i] = fmaf(p[h], x, o[h][c * EPC + i]);
          }
        }
      }
    }
  };

  // Two-deep software pipeline; the prefetches are unconditional (see issue()).  In
  // plain order an iteration past the split's last is empty and is not computed.
  const int n_it = (t1 > t0) ? (t1 - t0 + TILE - 1) / TILE : 0;
  // Long compact-buffer splits read long contiguous runs of rows, and split-K
  // work-groups start together: run in step, they all sit at the same offsets of their
  // runs.  Each work-group starts at its own iteration instead (the rows and their merge
  // are unchanged; the order of the online softmax is fixed by the plan).  16K x 16 at
  // 50 %: 96.3 -> 86.8 us; 16K batch 1 at 98.4 % and 100 %: 16.6 -> 16.2 and 17.0 ->
  // 16.6; splits below 8 iterations gained nothing and keep the plain order.  The
  // index-set variant reads its rows through the block table, already spread over the
  // pool, and keeps the plain order (the rotation cost its step 0.2 us).
  if constexpr (SPARSE && !INDEXED && !PAIRED) {
    if (!has_recent && n_it >= 8) {
      n_rot = n_it;
      rot = (int)((((int64_t)b * a.Hkv + g) * a.n_split + split) % n_it);
    }
  }
  Buf A, Bb;
  if (n_it > 0) {
    // Scheduling barriers keep each refill below the last use of its buffer (so
    // the buffers keep their registers across the back edge; a hoisted refill
    // forces copies that wait on the loads) and all of a refill's loads ahead of
    // the computation they overlap.
    issue(0, A);
    if constexpr (SPARSE && !INDEXED) n_c = clampi(a.n_compact[b], 0, a.cap);
    for (int it = 0; it < n_it; it += 2) {
      issue(it + 1, Bb);
      __builtin_amdgcn_sched_barrier(0);
      compute(it, A);
      __builtin_amdgcn_sched_barrier(0);
      issue(it + 2, A);
      __builtin_amdgcn_sched_barrier(0);
      if (PAIRED || it + 1 < n_it) compute(it + 1, Bb);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  };
  if constexpr (SPARSE && !INDEXED) {
    if (compact_only)
      stream(std::true_type{});
    else
      stream(std::false_type{});
  } else {
    stream(std::false_type{});
  }

  if constexpr (SCORES) {
    // Positions of this split past the request's end are not candidates.
    const int f0 = max(t1, t0);
    const int64_t f1 = (split == a.n_split - 1) ? a.score_stride
                                                : min((int64_t)t0 + a.split_tokens, a.score_stride);
    for (int h = 0; h < (SCORES == 2 ? G : 1); ++h)
      for (int64_t j = f0 + tid; j < f1; j += NT) srow[h * a.score_stride + j] = neg_inf();
  }

  // Merge the row groups of this wave (lanes that share `sub`).
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const auto fmax_op = [](float x, float y) { return fmaxf(x, y); };
    const auto add_op = [](float x, float y) { return x + y; };
    const float M = xor_fold<LPR>(m[h], fmax_op);
    const float al = (m[h] == neg_inf()) ? 0.f : exp2_fast(m[h] - M);
    const float ls = xor_fold<LPR>(l[h] * al, add_op);
#pragma unroll
    for (int e = 0; e < E; ++e) o[h][e] = xor_fold<LPR>(o[h][e] * al, add_op);
    m[h] = M;
    l[h] = ls;
  }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int i = 0; i < EPC; ++i) wo[(w * G + h) * D + (c * LPR + sub) * EPC + i] = o[h][c * EPC + i];
      if (sub == 0) {
        wml[(w * G + h) * 2] = m[h];
        wml[(w * G + h) * 2 + 1] = l[h];
      }
    }
  }
  __syncthreads();
  if constexpr (SCORES == 1)
    for (int j = tid; j < t1 - t0; j += NT) srow[t0 + j] = sc_s[j];

  // Merge the waves and write the split's result.
  for (int idx = tid; idx < G * D; idx += NT) {
    const int h = idx / D, e = idx % D;
    float M = neg_inf();
#pragma unroll
    for (int x = 0; x < WAVES; ++x) M = fmaxf(M, wml[(x * G + h) * 2]);
    float ls = 0.f, os = 0.f;
#pragma unroll
    for (int x = 0; x < WAVES; ++x) {
      const float mw = wml[(x * G + h) * 2];
      const float al = (mw == neg_inf()) ? 0.f : exp2_fast(mw - M);
      ls = fmaf(al, wml[(x * G + h) * 2 + 1], ls);
      os = fmaf(al, wo[(x * G + h) * D + e], os);
    }
    const int64_t orow = SplitTail<D>::row(a, q_row0, g, G, h);
    if (!multi) {
      a.out[orow * D + e] = ls > 0.f ? os / ls : 0.f;
      if (e == 0 && a.lse) a.lse[orow] = ls > 0.f ? (M + log2f(ls)) * kLn2 : neg_inf();
    } else {
      const int64_t prow = orow * a.part_stride + split;
      store_coherent(a.part_o + prow * D + e, os);
      if (e == 0) store_coherent2(a.part_ml + prow * 2, M, ls);
    }
  }
  if (multi && !DEFER)
    SplitTail<D>::run(a, b, g, q_row0, G, G, kMaxSplits, reinterpret_cast<int*>(wml + WAVES * G * 2),
                      wml + WAVES * G * 2 + 4);
}

}  // namespace sfi
