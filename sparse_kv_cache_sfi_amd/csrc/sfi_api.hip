// C-ABI entry points of libsfi: host validation, split planning, workspace
// sizing and kernel launches.  Every check runs before anything is enqueued, so
// a rejected call launches nothing and touches no output.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <mutex>
#include <string>

#include "sfi.h"
#include "common.h"
#include "kernels.h"
#include "pack_unit.h"

namespace {

thread_local std::string g_last_error;

sfi_status fail(sfi_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

sfi_status ok() {
  g_last_error.clear();
  return SFI_OK;
}

sfi_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SFI_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Longest sequence (or compact + recent span) one split-K launch can cover.
constexpr int64_t kMaxTokens = (int64_t)sfi::kMaxSplits * sfi::kMaxSplitTokens;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define SFI_TRY(expr)                 \
  do {                                \
    const sfi_status _s = (expr);     \
    if (_s != SFI_OK) return _s;      \
  } while (0)

sfi_status check_shape(const sfi_shape* s) {
  if (!s) return fail(SFI_ERR_INVALID_ARG, "shape is NULL");
  if (s->batch < 1) return fail(SFI_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", s->batch);
  if (s->num_q_heads < 1 || s->num_kv_heads < 1)
    return fail(SFI_ERR_INVALID_ARG, "head counts must be >= 1 (Hq=%d, Hkv=%d)", s->num_q_heads, s->num_kv_heads);
  if (s->num_q_heads % s->num_kv_heads)
    return fail(SFI_ERR_INVALID_ARG, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)", s->num_q_heads,
                s->num_kv_heads);
  const int G = s->num_q_heads / s->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(SFI_ERR_UNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8 (got %d)", G);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(SFI_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", s->head_dim);
  if (s->dtype != SFI_F32 && s->dtype != SFI_BF16)
    return fail(SFI_ERR_INVALID_ARG, "dtype must be SFI_F32 or SFI_BF16 (got %d)", s->dtype);
  if (!(s->scale > 0.f) || !std::isfinite(s->scale))
    return fail(SFI_ERR_INVALID_ARG, "scale must be a positive finite number");
  return SFI_OK;
}

sfi_status check_kv(const sfi_paged_kv* kv) {
  if (!kv) return fail(SFI_ERR_INVALID_ARG, "kv descriptor is NULL");
  if (!kv->k || !kv->v || !kv->block_table) return fail(SFI_ERR_INVALID_ARG, "kv.k, kv.v and kv.block_table must be non-NULL");
  if (!aligned16(kv->k) || !aligned16(kv->v)) return fail(SFI_ERR_INVALID_ARG, "kv.k and kv.v must be 16-byte aligned");
  if (kv->page_size != 16) return fail(SFI_ERR_UNSUPPORTED, "page_size must be 16 (got %d)", kv->page_size);
  if (kv->max_pages < 1 || kv->num_pages < 1)
    return fail(SFI_ERR_INVALID_ARG, "max_pages and num_pages must be >= 1");
  if (kv->max_seq_len < 1) return fail(SFI_ERR_INVALID_ARG, "max_seq_len must be >= 1");
  if (kv->max_seq_len > kMaxTokens)
    return fail(SFI_ERR_UNSUPPORTED, "max_seq_len (%d) exceeds %lld tokens", kv->max_seq_len, (long long)kMaxTokens);
  if ((int64_t)kv->max_seq_len > (int64_t)kv->max_pages * 16)
    return fail(SFI_ERR_INVALID_ARG, "max_seq_len (%d) exceeds max_pages * page_size (%lld)", kv->max_seq_len,
                (long long)kv->max_pages * 16);
  return SFI_OK;
}

sfi_status check_ptr16(const void* p, const char* name, bool nullable = false) {
  if (!p) return nullable ? SFI_OK : fail(SFI_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(SFI_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
  return SFI_OK;
}

sfi_status check_budgets(int32_t n_sink, int32_t n_recent) {
  if (n_sink < 0 || n_recent < 0) return fail(SFI_ERR_INVALID_ARG, "n_sink and n_recent must be >= 0");
  return SFI_OK;
}

// Split-K plan: about one work-group per CU (256), but splits of at least
// min_split tokens, at most kMaxSplitTokens, at most max_splits splits, rounded to
// the kernel's tile.  SFI_TUNE_MIN_SPLIT and SFI_TUNE_TARGET_WGS (environment, read
// on every call) override the two targets for tuning sweeps; results stay correct
// for any value.
struct Split {
  int tokens;
  int n;
  bool recent = false;   // fast step: the recent window is the last split on its own
};

int64_t tune_env(const char* name, int64_t fallback) {
  const char* v = getenv(name);
  if (!v || !*v) return fallback;
  const long long x = atoll(v);
  return x > 0 ? x : fallback;
}

Split plan_split(int64_t units, int64_t n_tok, int tile, int64_t min_split, int max_splits = sfi::kMaxSplits,
                 int64_t target = 0, int64_t max_tokens = sfi::kMaxSplitTokens) {
  if (target <= 0) target = tune_env("SFI_TUNE_TARGET_WGS", 256);
  min_split = tune_env("SFI_TUNE_MIN_SPLIT", min_split);
  if (n_tok <= 0) return {tile, 1};
  const int64_t by_min = (n_tok + min_split - 1) / min_split;
  const int64_t want = (target + units - 1) / units;
  int64_t ns = by_min < want ? by_min : want;
  if (ns > max_splits) ns = max_splits;
  if (ns < 1) ns = 1;
  int64_t st = (n_tok + ns - 1) / ns;
  st = (st + tile - 1) / tile * tile;
  if (st > max_tokens) {
    // Capped splits give more work-groups than the target, and cut at the cap they can
    // leave CUs with two long splits beside CUs with one: at 16 requests x 8 KV heads x
    // 12288 tokens, three splits of 4096 make 384 work-groups (a third of a second wave),
    // and at 12305 tokens three of 4096 and one of 17 do the same.  Cut evenly into as
    // many splits as fill the waves of work-groups the cap needs anyway (there, four
    // splits of 3072 or 3136 tokens: two work-groups per CU).
    const int64_t ns_cap = (n_tok + max_tokens - 1) / max_tokens;
    const int64_t waves = (units * ns_cap + target - 1) / target;
    const int64_t fill = std::max<int64_t>(ns_cap, std::min<int64_t>(waves * target / units, max_splits));
    st = (n_tok + fill - 1) / fill;
    st = (st + tile - 1) / tile * tile;
  }
  ns = (n_tok + st - 1) / st;
  return {(int)st, (int)ns};
}

// Verification work-groups: about two per CU.  A verification work-group keeps one
// 32-token K/V tile in flight per wave, so the launch needs two of them on a CU to
// keep enough bytes in flight (one per CU left the HBM idle half the time).
int64_t verify_target_wgs() { return tune_env("SFI_TUNE_VERIFY_WGS", 512); }

// Dense splits: 256 tokens, 512 once a unit has 8192 or more (the merge of many
// splits costs more than the parallelism gains).
int64_t dense_min_split(int64_t n_tok) { return n_tok >= 8192 ? 512 : 256; }
// Fast-step splits: 128 tokens, so that at small batches the step spreads over many
// CUs (a CU streams only some tens of GB/s), but a unit of at most 320 tokens stays one
// split: below that the split-K tail (partial stores drained, arrival ticket, merge)
// costs more than the shorter stream saves.
int64_t sparse_min_split(int64_t n_tok) { return n_tok <= 320 ? n_tok : 128; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace of a split-K call: the arrival counters (fixed region at offset 0, so
// calls of any shape can share one zero-filled workspace), then the partials
// [rows, n_split, d] floats and [rows, n_split, 2] floats.
size_t partial_bytes(int64_t rows, int n_split, int d) {
  if (n_split <= 1) return 0;
  return sfi::kCounterBytes + align_up((size_t)rows * n_split * d * 4, 256) +
         align_up((size_t)rows * n_split * 2 * 4, 256);
}

Split plan_dense(const sfi_shape* s, const sfi_paged_kv* kv, int t_q) {
  if (t_q > 1)
    return plan_split((int64_t)s->batch * s->num_kv_heads, kv->max_seq_len, sfi::kVerifyTile,
                      dense_min_split(kv->max_seq_len), sfi::kMaxVerifySplits, verify_target_wgs(),
                      sfi::kMaxVerifySplitTokens);
  return plan_split((int64_t)s->batch * s->num_kv_heads, kv->max_seq_len, sfi::kDecodeTile,
                    dense_min_split(kv->max_seq_len));
}

// The split that holds the recent window reads it through the block table, so its
// loads wait for two memory round trips (the request's length, then the pages'
// entries) that a split of compact rows never waits for; cut evenly with the compact
// rows, it arrives last at every unit's combine (per-work-group timestamps, 16K at 1/8
// retention: 0.7 us behind the other splits).  When the compact rows need several
// splits anyway and one more work-group per unit still fits the work-group target, the
// recent window becomes a short split of its own and the compact splits keep their
// size.  SFI_TUNE_RECENT_SPLIT=0 (environment, read on every call) keeps the even cut.
Split plan_sparse(const sfi_shape* s, int32_t cap, int32_t n_recent, const sfi_paged_kv* kv) {
  const int64_t rec = n_recent < kv->max_seq_len ? n_recent : kv->max_seq_len;
  const int64_t n_tok = (int64_t)cap + rec;
  const int64_t units = (int64_t)s->batch * s->num_kv_heads;
  const Split even = plan_split(units, n_tok, sfi::kDecodeTile, sparse_min_split(n_tok));
  const char* off = getenv("SFI_TUNE_RECENT_SPLIT");
  if (even.n > 1 && rec > 0 && rec <= sfi::kMaxSplitTokens && cap > 0 && !(off && off[0] == '0')) {
    const Split c = plan_split(units, cap, sfi::kDecodeTile, sparse_min_split(n_tok), sfi::kMaxSplits - 1);
    if (c.n > 1 && c.tokens == even.tokens && units * (c.n + 1) <= tune_env("SFI_TUNE_TARGET_WGS", 256))
      return {c.tokens, c.n + 1, true};
  }
  return even;
}

sfi::AttnArgs base_args(const sfi_shape* s, const sfi_paged_kv* kv, const int32_t* seq_lens) {
  sfi::AttnArgs a{};
  a.Hq = s->num_q_heads;
  a.Hkv = s->num_kv_heads;
  a.max_pages = kv->max_pages;
  a.num_pages = kv->num_pages;
  a.max_seq_len = kv->max_seq_len;
  a.k_pool = kv->k;
  a.v_pool = kv->v;
  a.block_table = kv->block_table;
  a.seq_lens = seq_lens;
  a.scale = s->scale;
  a.scale_log2 = s->scale * sfi::kLog2e;
  a.sel_k = -1;   // not an index-set call
  a.head_div = 1;
  return a;
}

// The merge of a unit's partials addresses them with 32-bit byte offsets from its
// first row: rows (t, h) of one unit lie (t_q - 1) * Hq + G rows apart at most.
sfi_status check_unit_span(const sfi_shape* s, int t_q_max, int n_split) {
  if (n_split <= 1) return SFI_OK;
  const int G = s->num_q_heads / s->num_kv_heads;
  const int64_t span = ((int64_t)(t_q_max - 1) * s->num_q_heads + G) * n_split * s->head_dim * 4;
  if (span > INT32_MAX)
    return fail(SFI_ERR_UNSUPPORTED, "split partials of one (request, KV head) span %lld bytes (limit %d)",
                (long long)span, INT32_MAX);
  return SFI_OK;
}

void set_partials(sfi::AttnArgs& a, void* ws, int64_t rows, int d) {
  a.part_stride = a.n_split;
  if (a.n_split <= 1) return;
  char* p = static_cast<char*>(ws);
  a.counters = reinterpret_cast<int32_t*>(p);
  a.part_o = reinterpret_cast<float*>(p + sfi::kCounterBytes);
  a.part_ml = reinterpret_cast<float*>(p + sfi::kCounterBytes + align_up((size_t)rows * a.n_split * d * 4, 256));
}

sfi_status check_workspace(const void* ws, size_t have, size_t need) {
  if (need == 0) return SFI_OK;
  if (have < need) return fail(SFI_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed", have, need);
  if (!ws) return fail(SFI_ERR_INVALID_ARG, "workspace is NULL but %zu bytes are needed", need);
  if (!aligned16(ws)) return fail(SFI_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return SFI_OK;
}

// Work list of a mixed launch: verifying requests first, then drafting ones.
struct MixedSetup {
  sfi::MixedPlan plan;
  int part_stride;   // largest split count of any entry
  int rows;          // packed query rows (sum of t_q)
};

sfi_status plan_mixed(const sfi_shape* shape, const sfi_paged_kv* kv, const int32_t* modes, const int32_t* t_q,
                      int32_t cap, int32_t n_recent, MixedSetup* ms) {
  SFI_TRY(check_shape(shape));
  SFI_TRY(check_kv(kv));
  if (!modes || !t_q) return fail(SFI_ERR_INVALID_ARG, "modes and t_q must be non-NULL host arrays");
  const int B = shape->batch, G = shape->num_q_heads / shape->num_kv_heads;
  if (B > sfi::kMaxMixedBatch) return fail(SFI_ERR_UNSUPPORTED, "mixed launch takes at most %d requests", sfi::kMaxMixedBatch);
  if (shape->dtype != SFI_BF16) return fail(SFI_ERR_UNSUPPORTED, "mixed launch needs bf16 inputs");
  if (cap < 1 || n_recent < 0) return fail(SFI_ERR_INVALID_ARG, "cap must be >= 1 and n_recent >= 0");
  if ((int64_t)cap + n_recent > kMaxTokens)
    return fail(SFI_ERR_UNSUPPORTED, "cap + n_recent exceeds %lld tokens", (long long)kMaxTokens);
  if ((int64_t)kv->max_seq_len > (int64_t)sfi::kMaxVerifySplits * sfi::kMaxVerifySplitTokens)
    return fail(SFI_ERR_UNSUPPORTED, "max_seq_len (%d) exceeds %lld tokens for verification", kv->max_seq_len,
                (long long)sfi::kMaxVerifySplits * sfi::kMaxVerifySplitTokens);
  int rows = 0;
  for (int b = 0; b < B; ++b) {
    if (modes[b] != 0 && modes[b] != 1) return fail(SFI_ERR_INVALID_ARG, "modes[%d] must be 0 or 1", b);
    if (t_q[b] < 1 || t_q[b] > 16) return fail(SFI_ERR_INVALID_ARG, "t_q[%d] must be in [1, 16]", b);
    if (modes[b] == 0 && t_q[b] != 1) return fail(SFI_ERR_INVALID_ARG, "drafting request %d must have t_q = 1", b);
    if (modes[b] == 1 && t_q[b] * G > sfi::kMaxVerifyRows)
      return fail(SFI_ERR_UNSUPPORTED, "t_q[%d] * G must be <= %d", b, sfi::kMaxVerifyRows);
    rows += t_q[b];
  }
  // Each kind is planned over its own requests: the verifying ones fill the GPU about
  // twice over, the drafting ones (a small share of the bytes) take one pass.
  int n_verify = 0;
  for (int b = 0; b < B; ++b) n_verify += modes[b] == 1 ? 1 : 0;
  const int64_t units_v = (int64_t)std::max(n_verify, 1) * shape->num_kv_heads;
  const int64_t units_d = (int64_t)std::max(B - n_verify, 1) * shape->num_kv_heads;
  const int64_t rec = n_recent < kv->max_seq_len ? n_recent : kv->max_seq_len;
  const int64_t n_tok = (int64_t)cap + rec;
  const Split sp_d = plan_split(units_d, n_tok, sfi::kDecodeTile, sparse_min_split(n_tok));
  const Split sp_v = plan_split(units_v, kv->max_seq_len, sfi::kVerifyTile, dense_min_split(kv->max_seq_len),
                                sfi::kMaxVerifySplits, verify_target_wgs(), sfi::kMaxVerifySplitTokens);
  sfi::MixedPlan& p = ms->plan;
  p = sfi::MixedPlan{};
  int q_row0[sfi::kMaxMixedBatch];
  for (int b = 0, r = 0; b < B; ++b) {
    q_row0[b] = r;
    r += t_q[b];
  }
  int e = 0, wg = 0, stride = 1;
  for (int pass = 1; pass >= 0; --pass)
    for (int b = 0; b < B; ++b) {
      if (modes[b] != pass) continue;
      const Split& sp = pass ? sp_v : sp_d;
      p.req[e] = b;
      p.mode[e] = pass;
      p.t_q[e] = t_q[b];
      p.q_row0[e] = q_row0[b];
      p.n_split[e] = sp.n;
      p.split_tokens[e] = sp.tokens;
      p.wg_begin[e] = wg;
      wg += shape->num_kv_heads * sp.n;
      stride = sp.n > stride ? sp.n : stride;
      ++e;
    }
  p.n_entries = e;
  p.wg_begin[e] = wg;
  int tq_max = 1;
  for (int b = 0; b < B; ++b) tq_max = t_q[b] > tq_max ? t_q[b] : tq_max;
  SFI_TRY(check_unit_span(shape, tq_max, stride));
  ms->part_stride = stride;
  ms->rows = rows;
  return SFI_OK;
}

size_t mixed_workspace_bytes(const MixedSetup& ms, const sfi_shape* shape) {
  return partial_bytes((int64_t)ms.rows * shape->num_q_heads, ms.part_stride, shape->head_dim);
}

}  // namespace

extern "C" {

sfi_status sfi_dense_attn_workspace_size(const sfi_shape* shape, const sfi_paged_kv* kv, int32_t t_q, size_t* bytes) {
  SFI_TRY(check_shape(shape));
  SFI_TRY(check_kv(kv));
  if (!bytes) return fail(SFI_ERR_INVALID_ARG, "bytes is NULL");
  if (t_q < 1 || t_q > 16) return fail(SFI_ERR_INVALID_ARG, "t_q must be in [1, 16] (got %d)", t_q);
  const Split sp = plan_dense(shape, kv, t_q);
  *bytes = partial_bytes((int64_t)shape->batch * t_q * shape->num_q_heads, sp.n, shape->head_dim);
  return ok();
}

}  // extern "C"

namespace {

sfi_status dense_call(const sfi_shape* shape, const sfi_paged_kv* kv, const void* q, int32_t t_q,
                      const int32_t* seq_lens, int32_t n_sink, int32_t n_recent, float* out, float* lse,
                      float* scores, int64_t score_stride, bool head_scores, void* workspace, size_t workspace_bytes,
                      void* stream, bool defer_merge = false) {
  SFI_TRY(check_shape(shape));
  SFI_TRY(check_kv(kv));
  SFI_TRY(check_ptr16(q, "q"));
  SFI_TRY(check_ptr16(out, "out"));
  if (!seq_lens) return fail(SFI_ERR_INVALID_ARG, "seq_lens is NULL");
  if (t_q < 1 || t_q > 16) return fail(SFI_ERR_INVALID_ARG, "t_q must be in [1, 16] (got %d)", t_q);
  SFI_TRY(check_budgets(n_sink, n_recent));
  if (scores && score_stride < kv->max_seq_len)
    return fail(SFI_ERR_INVALID_ARG, "score_stride (%lld) must be >= max_seq_len (%d)", (long long)score_stride,
                kv->max_seq_len);
  const int G = shape->num_q_heads / shape->num_kv_heads;
  if (t_q > 1) {
    if (shape->dtype != SFI_BF16) return fail(SFI_ERR_UNSUPPORTED, "t_q > 1 needs bf16 inputs");
    if (t_q * G > sfi::kMaxVerifyRows)
      return fail(SFI_ERR_UNSUPPORTED, "t_q * G must be <= %d (got %d)", sfi::kMaxVerifyRows, t_q * G);
    if ((int64_t)kv->max_seq_len > (int64_t)sfi::kMaxVerifySplits * sfi::kMaxVerifySplitTokens)
      return fail(SFI_ERR_UNSUPPORTED, "max_seq_len (%d) exceeds %lld tokens for t_q > 1", kv->max_seq_len,
                  (long long)sfi::kMaxVerifySplits * sfi::kMaxVerifySplitTokens);
  }
  if ((int64_t)shape->batch * shape->num_kv_heads > sfi::kMaxCounters)
    return fail(SFI_ERR_UNSUPPORTED, "batch * num_kv_heads must be <= %d", sfi::kMaxCounters);
  const Split sp = plan_dense(shape, kv, t_q);
  const int64_t rows = (int64_t)shape->batch * t_q * shape->num_q_heads;
  SFI_TRY(check_unit_span(shape, t_q, sp.n));
  SFI_TRY(check_workspace(workspace, workspace_bytes, partial_bytes(rows, sp.n, shape->head_dim)));

  sfi::AttnArgs a = base_args(shape, kv, seq_lens);
  a.q = q;
  a.n_sink = n_sink;
  a.n_recent = n_recent;
  a.split_tokens = sp.tokens;
  a.n_split = sp.n;
  a.t_q = t_q;
  a.out = out;
  a.lse = lse;
  a.scores = scores;
  a.score_stride = score_stride;
  a.head_scores = head_scores ? 1 : 0;
  a.defer_merge = defer_merge ? 1 : 0;
  set_partials(a, workspace, rows, shape->head_dim);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (t_q == 1)
    e = sfi::launch_decode(a, shape->dtype, shape->head_dim, G, false, shape->batch, st);
  else
    e = sfi::launch_verify(a, shape->head_dim, G, shape->batch, st);
  return hip_status(e, "attention launch");
}

sfi_status pack_call(const sfi_shape* shape, const sfi_paged_kv* kv, const int32_t* seq_lens, int32_t n_sink,
                     const int32_t* sel_idx, int32_t k, void* compact_k, void* compact_v, int32_t cap,
                     int32_t* n_compact, void* stream) {
  SFI_TRY(check_shape(shape));
  SFI_TRY(check_kv(kv));
  if (!seq_lens || !sel_idx || !n_compact) return fail(SFI_ERR_INVALID_ARG, "seq_lens, sel_idx and n_compact must be non-NULL");
  SFI_TRY(check_ptr16(compact_k, "compact_k"));
  SFI_TRY(check_ptr16(compact_v, "compact_v"));
  if (k < 1) return fail(SFI_ERR_INVALID_ARG, "k must be >= 1 (got %d)", k);
  if (n_sink < 0) return fail(SFI_ERR_INVALID_ARG, "n_sink must be >= 0");
  if ((int64_t)cap < (int64_t)n_sink + k)
    return fail(SFI_ERR_INVALID_ARG, "cap (%d) must be >= n_sink + k (%lld)", cap, (long long)n_sink + k);
  const hipError_t e = sfi::launch_pack(shape->dtype, shape->head_dim, shape->batch, shape->num_kv_heads, kv->k, kv->v,
                                        kv->block_table, kv->max_pages, kv->num_pages, kv->max_seq_len, seq_lens,
                                        n_sink, sel_idx, k, compact_k, compact_v, cap, n_compact,
                                        static_cast<hipStream_t>(stream));
  return hip_status(e, "pack launch");
}

}  // namespace

extern "C" {

sfi_status sfi_dense_attn_with_stats(const sfi_shape* shape, const sfi_paged_kv* kv, const void* q, int32_t t_q,
                                     const int32_t* seq_lens, int32_t n_sink, int32_t n_recent, float* out,
                                     float* lse, float* scores, int64_t score_stride, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return dense_call(shape, kv, q, t_q, seq_lens, n_sink, n_recent, out, lse, scores, score_stride, false, workspace,
                    workspace_bytes, stream);
}

sfi_status sfi_dense_attn_with_stats_deferred(const sfi_shape* shape, const sfi_paged_kv* kv, const void* q,
                                              const int32_t* seq_lens, int32_t n_sink, int32_t n_recent, float* out,
                                              float* lse, float* scores, int64_t score_stride, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  if (!scores) return fail(SFI_ERR_INVALID_ARG, "scores is NULL (the Selector that finishes the call reads them)");
  return dense_call(shape, kv, q, 1, seq_lens, n_sink, n_recent, out, lse, scores, score_stride, false, workspace,
                    workspace_bytes, stream, true);
}

sfi_status sfi_dense_attn_with_head_stats(const sfi_shape* shape, const sfi_paged_kv* kv, const void* q,
                                          const int32_t* seq_lens, int32_t n_sink, int32_t n_recent, float* out,
                                          float* lse, float* scores, int64_t score_stride, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  if (!scores) return fail(SFI_ERR_INVALID_ARG, "scores is NULL");
  return dense_call(shape, kv, q, 1, seq_lens, n_sink, n_recent, out, lse, scores, score_stride, true, workspace,
                    workspace_bytes, stream);
}

sfi_status sfi_select_topk_workspace_size(int32_t batch, int32_t num_kv_heads, int64_t score_stride, int32_t n_sink,
                                          int32_t k, size_t* bytes) {
  if (!bytes) return fail(SFI_ERR_INVALID_ARG, "bytes is NULL");
  if (batch < 1 || num_kv_heads < 1 || score_stride < 1 || k < 1 || n_sink < 0)
    return fail(SFI_ERR_INVALID_ARG, "batch, num_kv_heads, score_stride and k must be >= 1, n_sink >= 0");
  *bytes = sfi::select_workspace_bytes(batch, num_kv_heads, score_stride, n_sink, k);
  return ok();
}

sfi_status sfi_select_topk(const float* scores, int32_t batch, int32_t num_kv_heads, int64_t score_stride,
                           const int32_t* seq_lens, int32_t t_q, int32_t n_sink, int32_t n_recent, int32_t k,
                           int32_t* sel_idx, void* workspace, size_t workspace_bytes, void* stream) {
  if (!scores || !seq_lens || !sel_idx) return fail(SFI_ERR_INVALID_ARG, "scores, seq_lens and sel_idx must be non-NULL");
  if (batch < 1 || num_kv_heads < 1) return fail(SFI_ERR_INVALID_ARG, "batch and num_kv_heads must be >= 1");
  if (score_stride < 1 || score_stride > INT32_MAX)
    return fail(SFI_ERR_INVALID_ARG, "score_stride must be in [1, 2^31)");
  if (k < 1) return fail(SFI_ERR_INVALID_ARG, "k must be >= 1 (got %d)", k);
  if (t_q < 1 || t_q > 16) return fail(SFI_ERR_INVALID_ARG, "t_q must be in [1, 16] (got %d)", t_q);
  SFI_TRY(check_budgets(n_sink, n_recent));
  const size_t need = sfi::select_workspace_bytes(batch, num_kv_heads, score_stride, n_sink, k);
  SFI_TRY(check_workspace(workspace, workspace_bytes, need));
  const hipError_t e = sfi::launch_select(scores, batch, num_kv_heads, score_stride, seq_lens, t_q, n_sink, n_recent,
                                          k, sel_idx, need ? workspace : nullptr, static_cast<hipStream_t>(stream));
  return hip_status(e, "select launch");
}


sfi_status sfi_pack_compact(const sfi_shape* shape, const sfi_paged_kv* kv, const int32_t* seq_lens, int32_t n_sink,
                            const int32_t* sel_idx, int32_t k, void* compact_k, void* compact_v, int32_t cap,
                            int32_t* n_compact, void* stream) {
  return pack_call(shape, kv, seq_lens, n_sink, sel_idx, k, compact_k, compact_v, cap, n_compact, stream);
}

sfi_status sfi_sparse_decode_workspace_size(const sfi_shape* shape, const sfi_paged_kv* kv, int32_t cap,
                                            int32_t n_recent, size_t* bytes) {
  SFI_TRY(check_shape(shape));
  SFI_TRY(check_kv(kv));
  if (!bytes) return fail(SFI_ERR_INVALID_ARG, "bytes is NULL");
  if (cap < 0 || n_recent < 0) return fail(SFI_ERR_INVALID_ARG, "cap and n_recent must be >= 0");
  const Split sp = plan_sparse(shape, cap, n_recent, kv);
  *bytes = partial_bytes((int64_t)shape->batch * shape->num_q_heads, sp.n, shape->head_dim);
  return ok();
}

}  // extern "C"

namespace {

// The fast step.  Sink and selected rows come from compact buffers, or, when sel_k is
// >= 0, from paged KV at the positions sel lists (cap is then n_sink + sel_k).
sfi_status sparse_call(const sfi_shape* shape_in, const sfi_paged_kv* kv, const void* q, const void* k_new,
                       const void* v_new, const int32_t* seq_lens, int32_t n_sink, int32_t n_recent,
                       const void* compact_k, const void* compact_v, int32_t cap, const int32_t* n_compact,
                       const int32_t* sel, int32_t sel_k, bool per_head, float* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream, void* pack_k = nullptr, void* pack_v = nullptr,
                       int32_t pack_cap = 0, int32_t* pack_n = nullptr, const sfi::AttnArgs* merge = nullptr) {
  SFI_TRY(check_shape(shape_in));
  // One unit per query head when each query head has its own selection: the units see
  // a shape with as many KV heads as query heads, head_div of them per pool head.
  const int head_div = per_head ? shape_in->num_q_heads / shape_in->num_kv_heads : 1;
  sfi_shape unit_shape = *shape_in;
  if (per_head) unit_shape.num_kv_heads = shape_in->num_q_heads;
  const sfi_shape* shape = &unit_shape;
  SFI_TRY(check_kv(kv));
  SFI_TRY(check_ptr16(q, "q"));
  SFI_TRY(check_ptr16(out, "out"));
  if (!seq_lens) return fail(SFI_ERR_INVALID_ARG, "seq_lens is NULL");
  SFI_TRY(check_budgets(n_sink, n_recent));
  if (sel_k >= 0) {
    if ((int64_t)kv->num_pages * sfi::kPage > INT32_MAX)
      return fail(SFI_ERR_UNSUPPORTED, "num_pages (%d) too large for 32-bit page slots", kv->num_pages);
    cap = (int32_t)std::min<int64_t>((int64_t)n_sink + sel_k, INT32_MAX);
  } else {
    SFI_TRY(check_ptr16(compact_k, "compact_k"));
    SFI_TRY(check_ptr16(compact_v, "compact_v"));
    if (!n_compact) return fail(SFI_ERR_INVALID_ARG, "n_compact is NULL");
  }
  // An index-set step may have no sink and no selection (cap 0: the recent window alone).
  if (cap < (sel_k >= 0 ? 0 : 1)) return fail(SFI_ERR_INVALID_ARG, "cap must be >= 1");
  if ((int64_t)cap + n_recent > kMaxTokens)
    return fail(SFI_ERR_UNSUPPORTED, "cap + n_recent exceeds %lld tokens", (long long)kMaxTokens);
  if ((int64_t)shape->batch * shape->num_kv_heads > sfi::kMaxCounters)
    return fail(SFI_ERR_UNSUPPORTED, "batch * num_kv_heads must be <= %d", sfi::kMaxCounters);
  const Split sp = plan_sparse(shape, cap, n_recent, kv);
  const int64_t rows = (int64_t)shape->batch * shape->num_q_heads;
  SFI_TRY(check_unit_span(shape, 1, sp.n));
  SFI_TRY(check_workspace(workspace, workspace_bytes, partial_bytes(rows, sp.n, shape->head_dim)));

  sfi::AttnArgs a = base_args(shape, kv, seq_lens);
  a.q = q;
  a.ck = compact_k;
  a.cv = compact_v;
  a.cap = cap;
  a.n_compact = n_compact;
  a.n_sink = n_sink;
  a.n_recent = n_recent;
  a.split_tokens = sp.tokens;
  a.n_split = sp.n;
  a.recent_split = sp.recent ? 1 : 0;
  a.t_q = 1;
  a.out = out;
  a.lse = lse;
  a.k_new = k_new;
  a.v_new = v_new;
  a.sel = sel;
  a.sel_k = sel_k;
  a.head_div = head_div;
  a.pack_k = pack_k;
  a.pack_v = pack_v;
  a.pack_n = pack_n;
  a.pack_cap = pack_cap;
  set_partials(a, workspace, rows, shape->head_dim);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int G = shape->num_q_heads / shape->num_kv_heads;
  // Who writes the packed rows.  Pack blocks of their own in the same launch read the
  // selected rows a second time, on CUs the attention leaves idle; the attention's
  // work-groups can instead write the rows they have just loaded, which saves those
  // reads but lengthens the attention.  The second wins once the rows are many (16K
  // per request, 8 KV heads, d 128, bf16; pack blocks / rows written by the attention):
  // 1/8 retention at batch 1 11.7 / 18.2 us, 2: 14.6 / 20.4, 4: 19.0 / 24.3,
  // 8: 33.8 / 32.5, 16: 82.1 / 52.5; 1/64 retention, any batch up to 16: blocks by
  // ~1 us.  The switch is at 48 MiB of packed K and V (SFI_TUNE_PACK_IN_ATTN_BYTES,
  // environment, moves it for tuning; the results do not depend on it).  A deferred
  // combine rides in both forms.
  if (merge && !(pack_k && head_div == 1 && !k_new))
    return fail(SFI_ERR_INVALID_ARG, "a deferred combine rides only with packing and no appended token");
  const int64_t packed_bytes = (int64_t)shape->batch * shape->num_kv_heads * cap * 2 * shape->head_dim *
                               (shape->dtype == SFI_BF16 ? 2 : 4);
  const bool pack_blocks = pack_k && head_div == 1 && !k_new &&
                           packed_bytes < tune_env("SFI_TUNE_PACK_IN_ATTN_BYTES", 48ll << 20);
  if (pack_blocks || merge) {
    if (pack_blocks) {
      a.pack_k = a.pack_v = nullptr;
      a.pack_n = nullptr;
    }
    const sfi::PackArgs p{kv->k, kv->v, kv->block_table, kv->max_pages, kv->num_pages, kv->max_seq_len,
                          shape->num_kv_heads, seq_lens, n_sink, sel, sel_k, pack_k, pack_v, pack_cap, pack_n};
    const hipError_t e =
        sfi::launch_fast_pack(a, p, merge, pack_blocks, shape->dtype, shape->head_dim, G, shape->batch, st);
    return hip_status(e, "sparse decode + pack launch");
  }
  hipError_t e = sfi::launch_decode(a, shape->dtype, shape->head_dim, G, true, shape->batch, st);
  return hip_status(e, "sparse decode launch");
}

}  // namespace

extern "C" {

sfi_status sfi_sparse_decode_attn(const sfi_shape* shape, const sfi_paged_kv* kv, const void* q,
                                  const int32_t* seq_lens, int32_t n_sink, int32_t n_recent, const void* compact_k,
                                  const void* compact_v, int32_t cap, const int32_t* n_compact, float* out, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return sparse_call(shape, kv, q, nullptr, nullptr, seq_lens, n_sink, n_recent, compact_k, compact_v, cap,
                     n_compact, nullptr, -1, false, out, lse, workspace, workspace_bytes, stream);
}

sfi_status sfi_sparse_decode_append_attn(const sfi_shape* shape, const sfi_paged_kv* kv, const void* q,
                                         const void* k_new, const void* v_new, const int32_t* seq_lens,
                                         int32_t n_sink, int32_t n_recent, const void* compact_k,
                                         const void* compact_v, int32_t cap, const int32_t* n_compact, float* out,
                                         float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  SFI_TRY(check_ptr16(k_new, "k_new"));
  SFI_TRY(check_ptr16(v_new, "v_new"));
  return sparse_call(shape, kv, q, k_new, v_new, seq_lens, n_sink, n_recent, compact_k, compact_v, cap,
                     n_compact, nullptr, -1, false, out, lse, workspace, workspace_bytes, stream);
}

sfi_status sfi_sparse_decode_indexed_attn(const sfi_shape* shape, const sfi_paged_kv* kv, const void* q,
                                          const void* k_new, const void* v_new, const int32_t* seq_lens,
                                          int32_t n_sink, int32_t n_recent, const int32_t* sel_idx, int32_t k,
                                          int32_t per_head, void* compact_k, void* compact_v, int32_t cap,
                                          int32_t* n_compact, float* out, float* lse, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  if (per_head != 0 && per_head != 1) return fail(SFI_ERR_INVALID_ARG, "per_head must be 0 or 1");
  if (compact_k || compact_v || n_compact) {
    SFI_TRY(check_ptr16(compact_k, "compact_k"));
    SFI_TRY(check_ptr16(compact_v, "compact_v"));
    if (!n_compact) return fail(SFI_ERR_INVALID_ARG, "n_compact is NULL (compact_k, compact_v and n_compact go together)");
    if ((int64_t)cap < (int64_t)n_sink + k)
      return fail(SFI_ERR_INVALID_ARG, "cap (%d) must be >= n_sink + k (%lld)", cap, (long long)n_sink + k);
  }
  if (k < 0) return fail(SFI_ERR_INVALID_ARG, "k must be >= 0");
  if (!sel_idx && k > 0) return fail(SFI_ERR_INVALID_ARG, "sel_idx is NULL");
  if (!k_new != !v_new) return fail(SFI_ERR_INVALID_ARG, "k_new and v_new must both be NULL or both be set");
  if (k_new) {
    SFI_TRY(check_ptr16(k_new, "k_new"));
    SFI_TRY(check_ptr16(v_new, "v_new"));
  }
  return sparse_call(shape, kv, q, k_new, v_new, seq_lens, n_sink, n_recent, nullptr, nullptr, 0, nullptr, sel_idx,
                     k, per_head == 1, out, lse, workspace, workspace_bytes, stream, compact_k, compact_v, cap,
                     n_compact);
}

sfi_status sfi_sparse_decode_indexed_attn_merge(const sfi_shape* shape, const sfi_paged_kv* kv, const void* q,
                                                const int32_t* seq_lens, int32_t n_sink, int32_t n_recent,
                                                const int32_t* sel_idx, int32_t k, void* compact_k, void* compact_v,
                                                int32_t cap, int32_t* n_compact, float* out, float* lse,
                                                void* workspace, size_t workspace_bytes, float* slow_out,
                                                float* slow_lse, void* slow_workspace, size_t slow_workspace_bytes,
                                                void* stream) {
  SFI_TRY(check_shape(shape));
  SFI_TRY(check_kv(kv));
  SFI_TRY(check_ptr16(compact_k, "compact_k"));
  SFI_TRY(check_ptr16(compact_v, "compact_v"));
  SFI_TRY(check_ptr16(slow_out, "slow_out"));
  if (!n_compact) return fail(SFI_ERR_INVALID_ARG, "n_compact is NULL");
  if (k < 0) return fail(SFI_ERR_INVALID_ARG, "k must be >= 0");
  if (!sel_idx && k > 0) return fail(SFI_ERR_INVALID_ARG, "sel_idx is NULL");
  if ((int64_t)cap < (int64_t)n_sink + k)
    return fail(SFI_ERR_INVALID_ARG, "cap (%d) must be >= n_sink + k (%lld)", cap, (long long)n_sink + k);
  // The deferred slow step's partials, laid out as sfi_dense_attn_with_stats_deferred left them.
  const Split sp = plan_dense(shape, kv, 1);
  const int64_t rows = (int64_t)shape->batch * shape->num_q_heads;
  SFI_TRY(check_unit_span(shape, 1, sp.n));
  SFI_TRY(check_workspace(slow_workspace, slow_workspace_bytes, partial_bytes(rows, sp.n, shape->head_dim)));
  if (sp.n > 1 && workspace && workspace_bytes > 0) {
    const char* a0 = static_cast<const char*>(workspace);
    const char* b0 = static_cast<const char*>(slow_workspace);
    if (a0 < b0 + slow_workspace_bytes && b0 < a0 + workspace_bytes)
      return fail(SFI_ERR_INVALID_ARG, "workspace and slow_workspace must not overlap (both are in use in one launch)");
  }
  sfi::AttnArgs m = base_args(shape, kv, seq_lens);
  m.n_split = sp.n;
  m.split_tokens = sp.tokens;
  m.t_q = 1;
  m.out = slow_out;
  m.lse = slow_lse;
  set_partials(m, slow_workspace, rows, shape->head_dim);
  return sparse_call(shape, kv, q, nullptr, nullptr, seq_lens, n_sink, n_recent, nullptr, nullptr, 0, nullptr, sel_idx,
                     k, false, out, lse, workspace, workspace_bytes, stream, compact_k, compact_v, cap, n_compact,
                     sp.n > 1 ? &m : nullptr);
}

sfi_status sfi_mixed_attn_workspace_size(const sfi_shape* shape, const sfi_paged_kv* kv, const int32_t* modes,
                                         const int32_t* t_q, int32_t cap, int32_t n_recent, size_t* bytes) {
  if (!bytes) return fail(SFI_ERR_INVALID_ARG, "bytes is NULL");
  MixedSetup ms;
  SFI_TRY(plan_mixed(shape, kv, modes, t_q, cap, n_recent, &ms));
  *bytes = mixed_workspace_bytes(ms, shape);
  return ok();
}

sfi_status sfi_mixed_attn(const sfi_shape* shape, const sfi_paged_kv* kv, const void* q, const int32_t* modes,
                          const int32_t* t_q, const int32_t* seq_lens, int32_t n_sink, int32_t n_recent,
                          const void* compact_k, const void* compact_v, int32_t cap, const int32_t* n_compact,
                          float* out, float* lse, float* scores, int64_t score_stride, void* workspace,
                          size_t workspace_bytes, void* stream) {
  MixedSetup ms;
  SFI_TRY(plan_mixed(shape, kv, modes, t_q, cap, n_recent, &ms));
  SFI_TRY(check_ptr16(q, "q"));
  SFI_TRY(check_ptr16(out, "out"));
  SFI_TRY(check_ptr16(compact_k, "compact_k"));
  SFI_TRY(check_ptr16(compact_v, "compact_v"));
  if (!seq_lens || !n_compact) return fail(SFI_ERR_INVALID_ARG, "seq_lens and n_compact must be non-NULL");
  SFI_TRY(check_budgets(n_sink, n_recent));
  if (scores && score_stride < kv->max_seq_len)
    return fail(SFI_ERR_INVALID_ARG, "score_stride (%lld) must be >= max_seq_len (%d)", (long long)score_stride,
                kv->max_seq_len);
  if ((int64_t)shape->batch * shape->num_kv_heads > sfi::kMaxCounters)
    return fail(SFI_ERR_UNSUPPORTED, "batch * num_kv_heads must be <= %d", sfi::kMaxCounters);
  SFI_TRY(check_workspace(workspace, workspace_bytes, mixed_workspace_bytes(ms, shape)));

  sfi::AttnArgs a = base_args(shape, kv, seq_lens);
  a.q = q;
  a.ck = compact_k;
  a.cv = compact_v;
  a.cap = cap;
  a.n_compact = n_compact;
  a.n_sink = n_sink;
  a.n_recent = n_recent;
  a.out = out;
  a.lse = lse;
  a.scores = scores;
  a.score_stride = score_stride;
  a.n_split = ms.part_stride;   // sizes the partial layout; every entry uses its own split count
  set_partials(a, workspace, (int64_t)ms.rows * shape->num_q_heads, shape->head_dim);
  const int G = shape->num_q_heads / shape->num_kv_heads;
  const hipError_t e = sfi::launch_mixed(a, ms.plan, shape->head_dim, G, static_cast<hipStream_t>(stream));
  return hip_status(e, "mixed launch");
}

sfi_status sfi_plan_splits(int32_t op, const sfi_shape* shape, const sfi_paged_kv* kv, int32_t t_q, int32_t cap,
                           int32_t n_recent, int32_t* split_tokens, int32_t* n_split) {
  SFI_TRY(check_shape(shape));
  SFI_TRY(check_kv(kv));
  if (!split_tokens || !n_split) return fail(SFI_ERR_INVALID_ARG, "output pointers are NULL");
  Split sp;
  if (op == 0) {
    if (t_q < 1 || t_q > 16) return fail(SFI_ERR_INVALID_ARG, "t_q must be in [1, 16] (got %d)", t_q);
    sp = plan_dense(shape, kv, t_q);
  } else if (op == 1) {
    if (cap < 0 || n_recent < 0) return fail(SFI_ERR_INVALID_ARG, "cap and n_recent must be >= 0");
    sp = plan_sparse(shape, cap, n_recent, kv);
  } else {
    return fail(SFI_ERR_INVALID_ARG, "op must be 0 (dense) or 1 (sparse)");
  }
  *split_tokens = sp.tokens;
  *n_split = sp.n;
  return ok();
}

sfi_status sfi_stream_copy(const void* src, void* dst, size_t bytes, void* stream) {
  SFI_TRY(check_ptr16(src, "src"));
  SFI_TRY(check_ptr16(dst, "dst"));
  if (bytes % 16) return fail(SFI_ERR_INVALID_ARG, "bytes must be a multiple of 16");
  return hip_status(sfi::launch_stream_copy(src, dst, bytes, static_cast<hipStream_t>(stream)), "copy launch");
}

sfi_status sfi_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
  SFI_TRY(check_ptr16(src, "src"));
  if (!sink) return fail(SFI_ERR_INVALID_ARG, "sink is NULL");
  if (bytes % 16) return fail(SFI_ERR_INVALID_ARG, "bytes must be a multiple of 16");
  return hip_status(sfi::launch_stream_read(src, bytes, static_cast<uint32_t*>(sink), static_cast<hipStream_t>(stream)),
                    "read launch");
}

const char* sfi_status_string(sfi_status status) {
  switch (status) {
    case SFI_OK: return "SFI_OK";
    case SFI_ERR_INVALID_ARG: return "SFI_ERR_INVALID_ARG";
    case SFI_ERR_UNSUPPORTED: return "SFI_ERR_UNSUPPORTED";
    case SFI_ERR_WORKSPACE: return "SFI_ERR_WORKSPACE";
    case SFI_ERR_HIP: return "SFI_ERR_HIP";
  }
  return "SFI_ERR_UNKNOWN";
}

const char* sfi_last_error(void) { return g_last_error.c_str(); }

int32_t sfi_version(void) { return SFI_VERSION; }

}  // extern "C"

// ---------------------------------------------------------------------------- no-allocation fast step
// The fast step's split-K scratch (arrival counters, then partials) in a file-scope
// device array instead of a caller workspace, for callers that cannot allocate.  Each
// GPU the library runs on holds its own copy until the process ends; host code uses
// the per-device address that hipGetSymbolAddress reports, never the array's name.
constexpr size_t kStaticScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

struct StaticScratch {
  std::mutex mu;
  void* ptr[kMaxDevices] = {};
};
StaticScratch g_static;

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

// The current device's scratch.  On the first call on a device: look up its address
// (that device current) and zero its counter region with a fill kernel on `stream`
// (the counters must start at zero; every call leaves them at zero again).
sfi_status static_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SFI_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_static.mu);
  if (!g_static.ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    const int64_t words = (int64_t)(sfi::kCounterBytes / 4);
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<uint32_t*>(p), words);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e, "scratch clear launch");
    g_static.ptr[dev] = p;
  }
  *out = g_static.ptr[dev];
  return SFI_OK;
}

}  // namespace

extern "C" {

sfi_status sfi_sparse_decode_attn_static(const sfi_shape* shape, const sfi_paged_kv* kv, const void* q,
                                         const int32_t* seq_lens, int32_t n_sink, int32_t n_recent,
                                         const void* compact_k, const void* compact_v, int32_t cap,
                                         const int32_t* n_compact, float* out, float* lse, void* stream) {
  // The size check runs before any device call.
  SFI_TRY(check_shape(shape));
  SFI_TRY(check_kv(kv));
  if (cap < 1 || n_recent < 0) return fail(SFI_ERR_INVALID_ARG, "cap must be >= 1 and n_recent >= 0");
  const Split sp = plan_sparse(shape, cap, n_recent, kv);
  const size_t need = partial_bytes((int64_t)shape->batch * shape->num_q_heads, sp.n, shape->head_dim);
  if (need > kStaticScratchBytes)
    return fail(SFI_ERR_WORKSPACE, "this call needs %zu bytes of split-K scratch; the static scratch holds %zu", need,
                kStaticScratchBytes);
  void* ws = nullptr;
  if (need > 0) SFI_TRY(static_scratch(static_cast<hipStream_t>(stream), &ws));
  return sparse_call(shape, kv, q, nullptr, nullptr, seq_lens, n_sink, n_recent, compact_k, compact_v, cap,
                     n_compact, nullptr, -1, false, out, lse, ws, need > 0 ? kStaticScratchBytes : 0, stream);
}

size_t sfi_static_scratch_bytes(void) { return kStaticScratchBytes; }

}  // extern "C"
