// Multi-query causal attention on MFMA for t_q > 1 query tokens per request.
//
// Full-context verification of t_q draft tokens (SparseSpec-L abstract: drafts
// are verified with full attention, whose per-head statistics are reused as the
// importance signal) is a real dense contraction: the R = t_q * G query rows of
// one KV head share every K/V row, so QK^T and PV run on the matrix cores.
//
// One work-group (4 waves) per (split, KV head g, request b); each wave takes
// 32-token tiles of the split in turn.  Per tile:
//   * the K and V rows (one or two 16-token pages) are loaded with coalesced
//     16-byte loads into registers one tile ahead and parked in the wave's LDS;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (tokens x rows), so every lane
//     owns one query row and 16 of the tile's tokens: the causal mask, the
//     online softmax (log2 units, reference max raised only by > 8) and the row
//     max need no cross-lane work beyond one swap between the lane halves;
//   * O^T += V^T P^T on the same instruction.  The probabilities are split into
//     bf16 hi + lo parts (two MFMAs) so the product keeps fp32-level accuracy;
//     the token order of the contraction is chosen so that P^T comes straight
//     from the S^T accumulator registers, and V^T is gathered from LDS;
//   * optionally the masked logits summed over all R rows (the verification
//     statistics) for every candidate token.
// Waves are merged through LDS; splits through the shared split tail.
#pragma once

#include "common.h"
#include "kernels.h"
#include "split_tail.h"

namespace sfi {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
#define LDS_AS __attribute__((address_space(3)))
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) float f32x2;

template <int D>
struct VerifyShape {
  static constexpr int KS = D / 16;                         // QK^T k-steps of 16 dims
  static constexpr int DB = D / 32;                         // 32-dim blocks of O^T
  static constexpr int ROW_BYTES = D * 2;                   // bf16 row
  static constexpr int LDS_ROW = ROW_BYTES + 16;            // padded LDS row stride of the query rows
  // K and V tile rows: at d 128 unpadded, their 16-byte chunks XOR-swizzled (tile_off);
  // at d 64 padded like the query rows.
  static constexpr bool SWZ = D == 128;
  static constexpr int TILE_ROW = SWZ ? ROW_BYTES : LDS_ROW;
  static constexpr int TILE = kVerifyTile;                  // 32 tokens
  static constexpr int WAVES = 4;
  static constexpr int CPR = ROW_BYTES / 16;                // 16-byte chunks per row
  static constexpr int LOADS = TILE * CPR / kWave;          // loads per lane per tile per tensor
  static constexpr int WAVE_LDS = 2 * TILE * TILE_ROW;      // K and V tiles of one wave
  // Per-wave O rows of the merge, one float longer than d: the 32 rows a write
  // instruction touches then start on different banks.
  static constexpr int MO_ROW = D + 1;
  static constexpr int MERGE = WAVES * (32 * MO_ROW + 64) * 4;   // per-wave O, m, l for the merge
  static constexpr int TILES_LDS = WAVES * WAVE_LDS > MERGE ? WAVES * WAVE_LDS : MERGE;
  static constexpr int TAIL = SplitTail<D>::bytes(32, kMaxVerifySplits);
  static constexpr int BIG = TILES_LDS > TAIL ? TILES_LDS : TAIL;
  // The tiles start on a 128-byte boundary: 16-byte LDS accesses must be 16-byte
  // aligned to run at full rate.
  static constexpr int BIG_OFF = (kVerifyBtSlots * 4 + 16 + 127) / 128 * 128;
  // The 32 query rows (the B operand of S^T) live in LDS, shared by the waves, rather
  // than in 32 registers per lane: that keeps the kernel within two waves per SIMD.
  static constexpr int Q_OFF = BIG_OFF + BIG;
  static constexpr int SMEM = Q_OFF + 32 * LDS_ROW;
  static_assert(LOADS >= 1, "tile too small");
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Byte offset of byte `byte` of tile row r.  Swizzled rows (d 128, 256 bytes) keep
// logical 16-byte chunk c at chunk c ^ (4 (r mod 4) + (r / 4) mod 4): sixteen
// consecutive rows read at one chunk (the K operand, 16 bytes per lane) and four
// consecutive rows read over four consecutive chunks (a half-wave of transposed V
// reads, 8 bytes per lane) each cover sixteen distinct chunks of a 256-byte span.
template <bool SWZ>
__device__ __forceinline__ int tile_off(int r, int byte, int row_bytes) {
  if constexpr (SWZ) return r * row_bytes + (((byte >> 4) ^ (4 * (r & 3) + ((r >> 2) & 3))) << 4) + (byte & 15);
  return r * row_bytes + byte;
}

template <int D, bool SCORES>
__device__ __forceinline__ void verify_unit(const AttnArgs& a, const int b, const int g, const int split,
                                            const int q_row0, const int G, char* smem) {
  using S = VerifyShape<D>;
  constexpr int KS = S::KS, DB = S::DB, LDS_ROW = S::LDS_ROW, TILE = S::TILE, WAVES = S::WAVES;
  constexpr int CPR = S::CPR, LOADS = S::LOADS, NT = WAVES * kWave;
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int hb = lane >> 5, n = lane & 31;
  const int R = a.t_q * G;

  int* bt_s = reinterpret_cast<int*>(smem);
  int* flag = bt_s + kVerifyBtSlots;
  char* big = smem + S::BIG_OFF;
  char* kt = big + w * S::WAVE_LDS;   // this wave's K tile, then its V tile
  char* vt = kt + TILE * S::TILE_ROW;

  const int L = clamp_len(a.seq_lens[b], a.max_seq_len, a.max_pages);
  const int t0 = split * a.split_tokens;
  const int t1 = min(L, t0 + a.split_tokens);

  int pg_lo = 0, n_pg = 0;
  if (t1 > t0) {
    pg_lo = t0 >> 4;
    n_pg = ((t1 - 1) >> 4) - pg_lo + 1;
  }
  const int32_t* bt_row = a.block_table + (int64_t)b * a.max_pages;
  for (int i = tid; i < n_pg; i += NT) {
    const int e = bt_row[pg_lo + i];
    bt_s[i] = (e >= 0 && e < a.num_pages) ? e : -1;
  }

  // Query rows r = (t, h) into LDS, zero rows past R (they contribute nothing).
  char* q_s = smem + S::Q_OFF;
  for (int i = tid; i < 32 * CPR; i += NT) {
    const int r = i / CPR, ch = i % CPR;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < R) {
      const uint16_t* qr =
          reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)(q_row0 + r / G) * a.Hq + g * G + r % G) * D;
      v = *reinterpret_cast<const u32x4*>(qr + ch * 8);
    }
    *reinterpret_cast<u32x4*>(q_s + r * LDS_ROW + ch * 16) = v;
  }
  const int qt = n / G;
  const bool row_ok = n < R;
  // Query token t sits at position L - t_q + t and sees keys up to it.
  const int lim = row_ok ? L - a.t_q + qt : -1;
  __syncthreads();

  int clo = 0, chi = 0;
  float* srow = nullptr;
  if constexpr (SCORES) {
    candidate_bounds(L, a.t_q, a.n_sink, a.n_recent, &clo, &chi);
    srow = a.scores + ((int64_t)b * a.Hkv + g) * a.score_stride;
  }

  const uint16_t* kpool = reinterpret_cast<const uint16_t*>(a.k_pool);
  const uint16_t* vpool = reinterpret_cast<const uint16_t*>(a.v_pool);
  const int64_t page_elems = (int64_t)a.Hkv * kPage * D;
  const int64_t head_off = (int64_t)g * kPage * D;

  const int n_tiles = (t1 > t0) ? (t1 - t0 + TILE - 1) / TILE : 0;
  const int iters = (n_tiles + WAVES - 1) / WAVES;   // uniform across waves (barriers inside)

  // Global loads of one tile: lane covers rows (i * kWave + lane) / CPR, chunk lane % CPR.
  auto load_tile = [&](int it, u32x4 (&kr)[LOADS], u32x4 (&vr)[LOADS]) {
    const int tb = t0 + (it * WAVES + w) * TILE;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int rr = (i * kWave + lane) / CPR, ch = (i * kWave + lane) % CPR;
      const int pos = tb + rr;
      const bool in = pos < t1;
      const int pg = bt_s[in ? (pos >> 4) - pg_lo : 0];
      const int64_t off = (in && pg >= 0) ? (int64_t)pg * page_elems + head_off + (int64_t)(pos & 15) * D : 0;
      // streaming loads: each K/V row is read once per launch
      kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kpool + off + ch * 8));
      vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vpool + off + ch * 8));
    }
  };
  auto park_tile = [&](const u32x4 (&kr)[LOADS], const u32x4 (&vr)[LOADS]) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int rr = (i * kWave + lane) / CPR, ch = (i * kWave + lane) % CPR;
      *reinterpret_cast<u32x4*>(kt + tile_off<S::SWZ>(rr, ch * 16, S::TILE_ROW)) = kr[i];
      *reinterpret_cast<u32x4*>(vt + tile_off<S::SWZ>(rr, ch * 16, S::TILE_ROW)) = vr[i];
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = neg_inf(), l_run = 0.f;

  if (iters > 0) {
    u32x4 kr[LOADS], vr[LOADS];
    load_tile(0, kr, vr);
    park_tile(kr, vr);
  }
  for (int it = 0; it < iters; ++it) {
    u32x4 kr[LOADS], vr[LOADS];
    const bool more = it + 1 < iters;
    if (more) load_tile(it + 1, kr, vr);   // consumed at the end of this iteration

    const int tb = t0 + (it * WAVES + w) * TILE;
    // Which of the tile's 32 tokens exist (inside the split, behind a valid page).
    bool tok_ok;
    {
      const int pos = tb + n;
      tok_ok = pos < t1 && bt_s[pos < t1 ? (pos >> 4) - pg_lo : 0] >= 0;
    }
    const uint64_t okmask = __ballot(tok_ok);

    // S^T = K Q^T over the tile: lane (n, hb) -> token 8 (i / 4) + 4 hb + i % 4, row n.
    f32x16 sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      // B operand: lane holds query row n, dims [16 s + 8 hb, +8).
      const u32x4 ka = *reinterpret_cast<const u32x4*>(kt + tile_off<S::SWZ>(n, (16 * s + 8 * hb) * 2, S::TILE_ROW));
      const u32x4 qb = *reinterpret_cast<const u32x4*>(q_s + n * LDS_ROW + (16 * s + 8 * hb) * 2);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka), __builtin_bit_cast(bf16x8, qb),
                                                      sacc, 0, 0, 0);
    }

    if constexpr (SCORES) {
      // Masked logits summed over all R rows (rows past R hold zero queries): a
      // transposing butterfly over the 32 lanes of each half-wave halves the values a
      // lane holds at every step, so lane n ends with the total of its register n / 2.
      float v16[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v16[i] = sacc[i];
#pragma unroll
      for (int w2 = 8; w2 >= 1; w2 >>= 1) {
        const bool up = (n & (2 * w2)) != 0;   // this lane keeps the upper half of its values
#pragma unroll
        for (int i = 0; i < w2; ++i) {
          const float keep = up ? v16[i + w2] : v16[i];
          const float send = up ? v16[i] : v16[i + w2];
          float got;
          if (w2 == 8) got = lane_xor<16>(send);
          else if (w2 == 4) got = lane_xor<8>(send);
          else if (w2 == 2) got = lane_xor<4>(send);
          else got = lane_xor<2>(send);
          v16[i] = keep + got;
        }
      }
      const float tot = v16[0] + lane_xor<1>(v16[0]);
      const int ri = n >> 1;
      const int tok = 8 * (ri / 4) + 4 * hb + (ri % 4);
      const int pos = tb + tok;
      if ((n & 1) == 0 && pos < t1) {
        const bool ok = (okmask >> tok) & 1ull;
        // Streaming stores: 4 bytes per token written into the K/V stream with write-back
        // stores cost the 128K verification 9 us (387 against 379 us with statistics).
        __builtin_nontemporal_store((ok && pos >= clo && pos < chi) ? tot * a.scale : neg_inf(), srow + pos);
      }
    }

    float sv[16];
    float mx = neg_inf();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tok = 8 * (i / 4) + 4 * hb + (i % 4);
      const bool vis = ((okmask >> tok) & 1ull) && tb + tok <= lim;
      sv[i] = vis ? sacc[i] * a.scale_log2 : neg_inf();
      mx = fmaxf(mx, sv[i]);
    }
    mx = fmaxf(mx, lane_xor<32>(mx));
    if (__any(mx > m_run + 8.f)) {
      const float mn = fmaxf(m_run, mx);
      const float al = (m_run == neg_inf()) ? 0.f : exp2_fast(m_run - mn);
      l_run *= al;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= al;
      m_run = mn;
    }
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = (m_run == neg_inf()) ? 0.f : exp2_fast(sv[i] - m_run);
      l_run += p[i];
    }
    // P^T as the B operand, hi and lo bf16 parts; k-index 8 hb + j of step s is the
    // token held in accumulator register 8 s + j.
    u32x4 phi[2], plo[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = p[8 * s + 2 * j], x1 = p[8 * s + 2 * j + 1];
        hw[j] = pack_bf16x2(x0, x1);
        const float h0 = bf16_lo(hw[j]), h1 = bf16_hi(hw[j]);
        lw[j] = pack_bf16x2(x0 - h0, x1 - h1);
      }
      phi[s] = (u32x4){hw[0], hw[1], hw[2], hw[3]};
      plo[s] = (u32x4){lw[0], lw[1], lw[2], lw[3]};
    }
    // O^T += V^T P^T.  Lane (dim 32 db + n, hb) needs V at tokens 16 s + 8 h + 4 hb + 0..3
    // for h = 0, 1: two transposing LDS reads, each filled by the 16-lane group the lane
    // sits in (lane i of a group receives element i % 4 of the row that lane
    // 4 j + i / 4 points at, for j = 0..3), so group lane s points at token
    // 16 s + 8 h + 4 hb + s / 4, dims 32 db + 16 (group & 1) + 4 (s % 4) + 0..3.
    const int tgrp = lane >> 4, tl = lane & 15;
    const int vrow = 4 * hb + (tl >> 2), vbyte = (16 * (tgrp & 1) + 4 * (tl & 3)) * 2;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const char* p0 = vt + tile_off<S::SWZ>(vrow + 16 * s, vbyte + 64 * db, S::TILE_ROW);
        const char* p1 = vt + tile_off<S::SWZ>(vrow + 16 * s + 8, vbyte + 64 * db, S::TILE_ROW);
        const bf16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p0));
        const bf16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p1));
        const bf16x8 vA = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vA, __builtin_bit_cast(bf16x8, phi[s]), oacc[db], 0, 0, 0);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vA, __builtin_bit_cast(bf16x8, plo[s]), oacc[db], 0, 0, 0);
      }
    }
    // A wave reads only its own tiles and its LDS accesses take effect in program
    // order, so the refill needs no barrier and the waves stream independently.
    if (more) park_tile(kr, vr);
  }
  __syncthreads();   // every wave is done with its tiles before the merge reuses the area

  // Merge the waves through LDS (the tile area is free now).
  constexpr int MO_ROW = S::MO_ROW;
  float* mo = reinterpret_cast<float*>(big);                // [WAVES][32][MO_ROW]
  float* mml = mo + WAVES * 32 * MO_ROW;                    // [WAVES][32][2]
  l_run += lane_xor<32>(l_run);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int dim = 32 * db + 8 * (i / 4) + 4 * hb + (i % 4);
      mo[(w * 32 + n) * MO_ROW + dim] = oacc[db][i];
    }
  if (hb == 0) {
    mml[(w * 32 + n) * 2] = m_run;
    mml[(w * 32 + n) * 2 + 1] = l_run;
  }
  __syncthreads();
  for (int idx = tid; idx < R * D; idx += NT) {
    const int r = idx / D, e = idx % D;
    float M = neg_inf();
#pragma unroll
    for (int x = 0; x < WAVES; ++x) M = fmaxf(M, mml[(x * 32 + r) * 2]);
    float ls = 0.f, os = 0.f;
#pragma unroll
    for (int x = 0; x < WAVES; ++x) {
      const float mw = mml[(x * 32 + r) * 2];
      const float al = (mw == neg_inf()) ? 0.f : exp2_fast(mw - M);
      ls = fmaf(al, mml[(x * 32 + r) * 2 + 1], ls);
      os = fmaf(al, mo[(x * 32 + r) * MO_ROW + e], os);
    }
    const int64_t orow = SplitTail<D>::row(a, q_row0, g, G, r);
    if (a.n_split == 1) {
      a.out[orow * D + e] = ls > 0.f ? os / ls : 0.f;
      if (e == 0 && a.lse) a.lse[orow] = ls > 0.f ? (M + log2f(ls)) * kLn2 : neg_inf();
    } else {
      store_coherent(a.part_o + (orow * a.part_stride + split) * D + e, os);
      if (e == 0) {
        store_coherent2(a.part_ml + (orow * a.part_stride + split) * 2, M, ls);
      }
    }
  }
  if constexpr (SCORES) {
    const int f0 = max(t1, t0);
    const int64_t f1 = (split == a.n_split - 1) ? a.score_stride : min((int64_t)t0 + a.split_tokens, a.score_stride);
    for (int64_t j = f0 + tid; j < f1; j += NT) srow[j] = neg_inf();
  }
  if (a.n_split > 1) {
    __syncthreads();   // the merge area becomes the tail's scratch
    SplitTail<D>::run(a, b, g, q_row0, G, R, kMaxVerifySplits, flag, reinterpret_cast<float*>(big));
  }
}

}  // namespace sfi
