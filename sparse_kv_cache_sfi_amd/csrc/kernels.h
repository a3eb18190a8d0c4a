// Internal interface between the C-ABI layer (sfi_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfi {

// Tokens processed by one work-group iteration of the split-K decode kernel is a
// multiple of this; split sizes are rounded to it.
constexpr int kDecodeTile = 64;
// Largest split (tokens) a work-group handles; bounds the block-table slice it
// stages in LDS.
constexpr int kMaxSplitTokens = 4096;
constexpr int kBtSlots = kMaxSplitTokens / 16 + 2;
// Most splits per (request, KV head); the split tail keeps one weight per split
// and head in LDS.
constexpr int kMaxSplits = 256;
// Most splits of a verification unit (its tail keeps t_q * G rows of weights).
constexpr int kMaxVerifySplits = 64;
// Largest verification split: twice the decode kernels' (its block-table slice, 2 KiB of
// LDS, fits beside the tiles), so that long contexts take half the splits, one wave of
// work-groups and half the partials for the unit's merge.
constexpr int kMaxVerifySplitTokens = 8192;
constexpr int kVerifyBtSlots = kMaxVerifySplitTokens / 16 + 2;
// Most query rows (t_q * G) of one KV head in a verification call.
constexpr int kMaxVerifyRows = 32;
// Split-K arrival counters live at the start of every workspace that holds
// partials: one int per (request, KV head), at most kMaxCounters of them.  They
// must be zero before the first call; every call returns them to zero.
constexpr int kMaxCounters = 65536;
constexpr size_t kCounterBytes = (size_t)kMaxCounters * 4;
// Token tile of the MFMA verification kernel.
constexpr int kVerifyTile = 32;
// Largest batch of the mixed launch (its per-request plan travels in kernel arguments).
constexpr int kMaxMixedBatch = 64;

// Arguments of the split-K attention kernels (by value).
struct AttnArgs {
  int32_t Hq, Hkv;
  int32_t max_pages, num_pages, max_seq_len;
  // Query rows: request b's query token t is row (q_row0(b) + t) of q, out and lse,
  // with q_row0(b) = b * t_q for single-kind calls (a per-request table for the
  // mixed launch); head hq of that token is element row * Hq + hq.
  const void* q;          // [rows, Hq, d]
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const void* ck;         // compact buffers [B, Hkv, cap, d] (sparse only)
  const void* cv;
  int32_t cap;
  const int32_t* n_compact;
  int32_t n_sink, n_recent;
  float scale;            // logit scale
  float scale_log2;       // scale * log2(e)
  int32_t split_tokens, n_split;
  int32_t t_q;            // query tokens of the request (dense / verify)
  float* out;             // [rows, Hq, d]
  float* lse;             // [rows, Hq] (nullable)
  float* part_o;          // split partials [rows * Hq, part_stride, d]
  float* part_ml;         // [rows * Hq, part_stride, 2] = (max in log2 units, sum)
  int32_t part_stride;    // split slots per partial row (>= n_split)
  int32_t* counters;      // kMaxCounters split arrival counters (zero between calls; unit_counter)
  float* scores;          // [B, Hkv, score_stride] (nullable)
  int64_t score_stride;
  // Fast step with append: request b's token at position L_b - 1 arrives here
  // ([B, Hkv, d], pool dtype); the launch writes it into its page and attends to it.
  const void* k_new;
  const void* v_new;
  // Fast step over an index set (sel_k >= 0; -1 otherwise): sel [B, Hkv, sel_k]
  // positions whose rows are read in place through the block table instead of from
  // compact buffers (sel may be NULL when sel_k is 0).
  const int32_t* sel;
  int32_t sel_k;
  // Units per KV head of the pool (1; the number of query heads per KV head when an
  // index-set fast step runs one unit per query head).
  int32_t head_div;
  // Slow step: write one logit row per query head ([B, Hq, score_stride]) instead of
  // the group sums.
  int32_t head_scores;
  // Index-set fast step that also packs (nullable): the sink and selected rows it
  // reads are written to pack_k / pack_v [B, units, pack_cap, d] exactly as the
  // gather-pack would, and pack_n[b] as its n_compact.
  void* pack_k;
  void* pack_v;
  int32_t* pack_n;
  int32_t pack_cap;
  // Leave the split partials for a later launch to merge (no arrival ticket, out and
  // lse are not written when there is more than one split); selects the kernel variant.
  int32_t defer_merge;
  // Fast step: the recent window is the unit's last split on its own (splits 0 ..
  // n_split - 2 cover the compact rows [0, cap) in split_tokens pieces); 0: the splits
  // cut the virtual rows [0, cap + n_recent) evenly.
  int32_t recent_split;
};

// Work list of the mixed launch (travels in kernel arguments).  Entry e serves
// request req[e] with work-groups [wg_begin[e], wg_begin[e + 1]), Hkv * n_split[e]
// of them; verifying requests come first (they are the longest).
struct MixedPlan {
  int32_t n_entries;
  int32_t wg_begin[kMaxMixedBatch + 1];
  int32_t req[kMaxMixedBatch];
  int32_t mode[kMaxMixedBatch];         // 0 draft (fast step), 1 verify (dense, causal)
  int32_t t_q[kMaxMixedBatch];
  int32_t q_row0[kMaxMixedBatch];       // first query row of the request
  int32_t n_split[kMaxMixedBatch];
  int32_t split_tokens[kMaxMixedBatch];
};

// Launchers.  Each returns hipGetLastError() after enqueueing.
hipError_t launch_decode(const AttnArgs& a, int dtype, int d, int G, bool sparse, int B,
                         hipStream_t stream);
hipError_t launch_verify(const AttnArgs& a, int d, int G, int B, hipStream_t stream);
hipError_t launch_mixed(const AttnArgs& a, const MixedPlan& plan, int d, int G, hipStream_t stream);
// ws: the candidate buffer of long rows (select_workspace_bytes bytes; may be NULL when
// that is 0, and then rows run on one work-group each).
hipError_t launch_select(const float* scores, int B, int Hkv, int64_t stride, const int32_t* seq_lens,
                         int t_q, int n_sink, int n_recent, int k, int32_t* sel, void* ws,
                         hipStream_t stream);
size_t select_workspace_bytes(int B, int Hkv, int64_t stride, int n_sink, int k);
hipError_t launch_pack(int dtype, int d, int B, int Hkv, const void* k_pool, const void* v_pool,
                       const int32_t* block_table, int max_pages, int num_pages, int max_seq_len,
                       const int32_t* seq_lens, int n_sink, const int32_t* sel, int k, void* ck,
                       void* cv, int cap, int32_t* n_compact, hipStream_t stream);
struct PackArgs;
// Index-set fast step (a.sel, a.sel_k) whose launch also packs the compact buffer
// described by p, with pack_blocks in work-groups of its own (a.pack_k NULL), else in
// the attention's work-groups (a.pack_k set), and, with merge non-NULL, merges a
// deferred slow step.
hipError_t launch_fast_pack(const AttnArgs& a, const PackArgs& p, const AttnArgs* merge, bool pack_blocks, int dtype,
                            int d, int G, int B, hipStream_t stream);
hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace sfi
