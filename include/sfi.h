/*
 * sfi.h - C ABI of libsfi, the Slow-Fast Inference (SFI) decode-attention
 * hot path for AMD Instinct MI355X (gfx950).
 *
 * Sources: the SFI page ("Slow-Fast Inference: Training-Free Inference
 * Acceleration via Within-Sentence Support Stability",
 * thelatestinai.com/papers/2603.12038), the SparseSpec-L abstract ("A Sparse
 * Glimpse of the Whole: Train-Free Self-Speculative Decoding") and the
 * ASPIRE abstract.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor argument is DEVICE memory owned by the caller; the
 *    descriptors (sfi_shape, sfi_paged_kv) and any array documented as "host"
 *    are host memory read during the call only.  The library allocates
 *    nothing, owns no stream and keeps no state beyond a thread-local error
 *    string.
 *  - Layouts are dense row-major with the shapes given.  B = batch,
 *    Hq / Hkv = query / KV heads, G = Hq / Hkv, d = head_dim, P = page_size.
 *    Query head h reads KV head h / G.
 *  - A paged pool k or v has shape [num_pages, Hkv, P, d]; token j of request
 *    b, KV head g, is row [block_table[b * max_pages + j / P], g, j % P].
 *  - seq_lens[b] (device int32) counts every token of request b including its
 *    t_q query tokens, whose K/V must already be in the pool; query token t
 *    sits at position seq_lens[b] - t_q + t and sees keys [0, that position].
 *  - Candidate set of a slow step / verification: positions
 *    [n_sink, max(n_sink, seq_lens[b] - t_q + 1 - n_recent)).  Recent window
 *    of a fast step: [max(n_sink, seq_lens[b] - n_recent), seq_lens[b]).
 *  - Outputs out / lse are float32; lse is the natural-log sum of exp(logit)
 *    over the keys seen, logit = scale * q . k.  A row that sees no key gets
 *    out = 0 and lse = -inf.
 *  - Workspaces: a workspace must be zero-filled before its first use (it
 *    starts with split-K arrival counters); every call leaves those counters
 *    at zero again, so one workspace may serve calls of any shape.  Calls
 *    that share a workspace must be ordered on one stream (or by events).
 *  - Calls only enqueue work on `stream` (a hipStream_t, NULL = default
 *    stream) and return without synchronising.  Ordering across streams is
 *    the caller's job (events).
 *  - Errors: every argument is validated on the host before anything is
 *    enqueued; on failure nothing is launched, no output is touched, and
 *    sfi_last_error() describes the problem.  A failed launch returns
 *    SFI_ERR_HIP.  No C++ exception crosses this boundary.
 *  - Device-side safety: block-table entries outside [0, num_pages), and
 *    positions outside [0, seq_lens[b]), are never dereferenced; keys behind
 *    such entries are skipped (attention) or written as zero rows (pack).
 *    seq_lens[b] is clamped to [0, min(max_seq_len, max_pages * P)].
 *  - Supported: d in {64, 128}; G in {1, 2, 4, 8}; P = 16; dtype F32 or BF16
 *    for t_q = 1; BF16 with t_q * G <= 32 for t_q in [2, 16].  max_seq_len up
 *    to 2^20 tokens (2^18 for t_q > 1).  Pointers to q, k, v, compact buffers,
 *    out and workspace must be 16-byte aligned.
 */
#ifndef SFI_H_
#define SFI_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SFI_VERSION 10000 /* major * 10000 + minor * 100 + patch */

#if defined(__GNUC__) || defined(__clang__)
#define SFI_API __attribute__((visibility("default")))
#else
#define SFI_API
#endif

typedef enum sfi_status {
  SFI_OK = 0,
  SFI_ERR_INVALID_ARG = 1, /* null / misaligned pointer, out-of-range size */
  SFI_ERR_UNSUPPORTED = 2, /* valid request outside the supported shapes   */
  SFI_ERR_WORKSPACE = 3,   /* workspace smaller than the size query says   */
  SFI_ERR_HIP = 4          /* the HIP runtime reported an error            */
} sfi_status;

typedef enum sfi_dtype { SFI_F32 = 0, SFI_BF16 = 1 } sfi_dtype;

/* Problem shape shared by the attention and pack calls (host memory). */
typedef struct sfi_shape {
  int32_t batch;        /* B >= 1                                           */
  int32_t num_q_heads;  /* Hq                                               */
  int32_t num_kv_heads; /* Hkv, Hq % Hkv == 0                               */
  int32_t head_dim;     /* d                                                */
  int32_t dtype;        /* sfi_dtype of q, the pools and the compact buffers */
  float scale;          /* logit scale, normally 1 / sqrt(d)                */
} sfi_shape;

/* Paged KV cache (host descriptor of device memory).  The whole cache stays
 * resident: tokens left out of the sparse state remain recallable
 * (SparseSpec-L abstract: the dense KV cache is never discarded). */
typedef struct sfi_paged_kv {
  const void* k;              /* [num_pages, Hkv, P, d]                      */
  const void* v;              /* [num_pages, Hkv, P, d]                      */
  const int32_t* block_table; /* [B, max_pages] physical page ids            */
  int32_t max_pages;          /* row length of block_table                   */
  int32_t page_size;          /* P, must be 16                               */
  int32_t num_pages;          /* pool size in pages                          */
  int32_t max_seq_len;        /* host upper bound on every seq_lens[b]; sizes
                                 the launch (and the workspace)             */
} sfi_paged_kv;

/*
 * Slow step: dense attention that also emits the masked logits.
 * SFI page, Fig. 2 caption: a slow step performs dense attention and collects
 * masked attention logits over the allowed candidate set for the Selector;
 * Table 1 uses dense-attention latency as its baseline.  With t_q > 1 it is
 * full-context causal verification of t_q draft tokens that also yields the
 * per-head statistics reused as the importance signal (SparseSpec-L
 * abstract).
 *
 *  q       [B, t_q, Hq, d]  dtype            t_q in [1, 16]
 *  out     [B, t_q, Hq, d]  float32
 *  lse     [B, t_q, Hq]     float32 or NULL
 *  scores  [B, Hkv, score_stride] float32 or NULL (NULL = plain dense
 *          attention).  scores[b, g, j] = sum over query tokens t and query
 *          heads h of group g of scale * q[b,t,h] . k_j for j in the candidate
 *          set, -inf for every other j < score_stride.  Requires
 *          score_stride >= max_seq_len.
 *  workspace: device scratch of at least sfi_dense_attn_workspace_size()
 *          bytes (may be NULL when that size is 0).
 */
SFI_API sfi_status sfi_dense_attn_with_stats(const sfi_shape* shape, const sfi_paged_kv* kv,
                                     const void* q, int32_t t_q, const int32_t* seq_lens,
                                     int32_t n_sink, int32_t n_recent, float* out, float* lse,
                                     float* scores, int64_t score_stride, void* workspace,
                                     size_t workspace_bytes, void* stream);

SFI_API sfi_status sfi_dense_attn_workspace_size(const sfi_shape* shape, const sfi_paged_kv* kv,
                                         int32_t t_q, size_t* bytes);

/*
 * Selector: top-k over each KV head's masked logits.
 * SFI page, Abstract and Fig. 2 caption (the Selector refreshes the selected
 * memory from the slow step's logits); Fig. 3A (it runs on the auxiliary
 * stream).  Per (b, g), among candidate positions the k_eff = min(k, number
 * of candidates) with the largest score are chosen, equal scores going to
 * the lower position (-0.0 == +0.0, -inf is the lowest score; NaN scores are
 * not supported).  Output is exact and deterministic.
 *
 *  scores   [B, Hkv, score_stride] float32 (only candidate positions are read)
 *  sel_idx  [B, Hkv, k] int32: the chosen positions ascending, then -1.
 *  t_q, n_sink, n_recent define the candidate set as above.
 *  workspace: at least sfi_select_topk_workspace_size() bytes (no zero-fill needed;
 *           NULL when that is 0).  Rows of at least 32768 possible candidates
 *           (score_stride - n_sink) whose k is small enough are cut into up to 16
 *           segments: one launch selects each segment's own top-k into the workspace,
 *           a second selects the row's top-k among those candidates (exact: a key in
 *           the row's top-k is in its segment's).  Other rows need no workspace.
 *  Errors: SFI_ERR_WORKSPACE when the workspace is smaller than required.
 */
SFI_API sfi_status sfi_select_topk(const float* scores, int32_t batch, int32_t num_kv_heads,
                           int64_t score_stride, const int32_t* seq_lens, int32_t t_q,
                           int32_t n_sink, int32_t n_recent, int32_t k, int32_t* sel_idx,
                           void* workspace, size_t workspace_bytes, void* stream);

SFI_API sfi_status sfi_select_topk_workspace_size(int32_t batch, int32_t num_kv_heads,
                                          int64_t score_stride, int32_t n_sink, int32_t k,
                                          size_t* bytes);

/*
 * Cache reorganisation: gather-pack sink and selected tokens into the compact
 * buffer (SFI page, Fig. 3B: sink and selected tokens packed into a
 * contiguous compact buffer; Fig. 3A: reorganisation on the auxiliary
 * stream).  For request b with ns = min(n_sink, seq_lens[b]) and k_eff = the
 * number of entries of sel_idx[b, 0, :] before its first negative entry:
 * row i < ns of KV head g is the token at position i; row ns + i is the
 * token at position sel_idx[b, g, i].  Copies are bitwise.  n_compact[b] =
 * ns + k_eff.  Rows from n_compact[b] to cap are not written.
 *
 *  sel_idx   [B, Hkv, k] int32 (as produced by sfi_select_topk)
 *  compact_k [B, Hkv, cap, d] dtype, compact_v likewise; cap >= n_sink + k
 *  n_compact [B] int32
 */
SFI_API sfi_status sfi_pack_compact(const sfi_shape* shape, const sfi_paged_kv* kv,
                            const int32_t* seq_lens, int32_t n_sink, const int32_t* sel_idx,
                            int32_t k, void* compact_k, void* compact_v, int32_t cap,
                            int32_t* n_compact, void* stream);

/*
 * Slow step whose split-K combine runs in a later launch of the step.  SFI page,
 * Fig. 2 caption: the slow step's logits go to the Selector, whose selection is
 * packed into the compact buffer (Fig. 3B) for the fast steps that follow; when
 * these run in order on one stream, the launch after the Selector (the fast step
 * over the selection with the pack, sfi_sparse_decode_indexed_attn_merge) has CUs
 * to spare and finishes the slow step there.  sfi_dense_attn_with_stats_deferred
 * computes the slow step (arguments as sfi_dense_attn_with_stats with t_q = 1;
 * scores must be non-NULL; workspace of sfi_dense_attn_workspace_size(shape, kv, 1)
 * bytes) but, when the call is split over more than one work-group per (request,
 * KV head), leaves the split partials in the workspace and writes neither out nor
 * lse.  sfi_sparse_decode_indexed_attn_merge must then be enqueued after it, on
 * the same stream (or ordered by events), with the same shape, kv, seq_lens, out,
 * lse and workspace (as slow_out, slow_lse, slow_workspace), and no other call may
 * use the workspace in between (the Selector, sfi_select_topk, uses none).  out,
 * lse, scores, the selection and the compact buffer are then bit-identical to
 * sfi_dense_attn_with_stats, sfi_select_topk and sfi_pack_compact.  Until that
 * launch has run, out and lse are undefined.  Errors as sfi_dense_attn_with_stats;
 * nothing is launched on any error.
 */
SFI_API sfi_status sfi_dense_attn_with_stats_deferred(const sfi_shape* shape, const sfi_paged_kv* kv,
                                              const void* q, const int32_t* seq_lens,
                                              int32_t n_sink, int32_t n_recent, float* out,
                                              float* lse, float* scores, int64_t score_stride,
                                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fast step: sparse decode attention over the two-segment state.
 * SFI page, Fig. 2 caption (fast steps attend to sink + selected + recent)
 * and Fig. 3B (sink and selected stream from the contiguous compact buffer;
 * recent tokens are read in place from paged KV).  One query token per
 * request: out[b, h] = softmax attention of q[b, h] over compact rows
 * [0, n_compact[b]) of KV head g(h) followed by the recent window.
 *
 *  q          [B, Hq, d] dtype
 *  compact_k  [B, Hkv, cap, d] dtype, compact_v likewise
 *  n_compact  [B] int32 (clamped to [0, cap])
 *  out        [B, Hq, d] float32;  lse [B, Hq] float32 or NULL
 *  workspace: at least sfi_sparse_decode_workspace_size() bytes.
 */
SFI_API sfi_status sfi_sparse_decode_attn(const sfi_shape* shape, const sfi_paged_kv* kv, const void* q,
                                  const int32_t* seq_lens, int32_t n_sink, int32_t n_recent,
                                  const void* compact_k, const void* compact_v, int32_t cap,
                                  const int32_t* n_compact, float* out, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream);

SFI_API sfi_status sfi_sparse_decode_workspace_size(const sfi_shape* shape, const sfi_paged_kv* kv,
                                            int32_t cap, int32_t n_recent, size_t* bytes);

/*
 * The fast step for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): exactly
 * sfi_sparse_decode_attn, with the same kernels and the same results bit for bit,
 * but its split-K scratch is a library-owned static device array of
 * sfi_static_scratch_bytes() bytes (8 MiB) on each GPU instead of a workspace
 * argument.  The call allocates nothing, neither through HIP nor otherwise.
 *
 *  - The first call on a device looks up that device's copy of the array and
 *    enqueues one small kernel on `stream` that zeroes its arrival counters; every
 *    call leaves them at zero again.  The array lives until the process ends.
 *  - Every call on a GPU shares that GPU's array, which keeps the last call's
 *    contents: calls that may overlap on one GPU (other streams, other threads)
 *    race and must be ordered by the caller.
 *  - Errors: as sfi_sparse_decode_attn; SFI_ERR_WORKSPACE, before anything touches
 *    the device, when the call's split-K scratch (the size
 *    sfi_sparse_decode_workspace_size reports) exceeds the array.
 */
SFI_API sfi_status sfi_sparse_decode_attn_static(const sfi_shape* shape, const sfi_paged_kv* kv, const void* q,
                                         const int32_t* seq_lens, int32_t n_sink, int32_t n_recent,
                                         const void* compact_k, const void* compact_v, int32_t cap,
                                         const int32_t* n_compact, float* out, float* lse, void* stream);

/* Bytes of the static scratch sfi_sparse_decode_attn_static uses on each device. */
SFI_API size_t sfi_static_scratch_bytes(void);

/*
 * Fast step with KV append: the token being decoded (position seq_lens[b] - 1)
 * has its K/V in k_new / v_new [B, Hkv, d] (pool dtype, 16-byte aligned).  The
 * launch stores them into that position's page of kv.k / kv.v (which must be
 * writable device memory) and attends exactly as sfi_sparse_decode_attn would
 * after that store; the new row is read from k_new / v_new, so the result does
 * not depend on the store.  The recent tokens are read in place from paged KV
 * (SFI page, Fig. 3B); appending in the same launch saves the separate append
 * launch before every fast step.  A position whose block-table entry is invalid
 * is neither stored nor attended.  Arguments and workspace otherwise as
 * sfi_sparse_decode_attn.
 */
SFI_API sfi_status sfi_sparse_decode_append_attn(const sfi_shape* shape, const sfi_paged_kv* kv,
                                         const void* q, const void* k_new, const void* v_new,
                                         const int32_t* seq_lens, int32_t n_sink, int32_t n_recent,
                                         const void* compact_k, const void* compact_v, int32_t cap,
                                         const int32_t* n_compact, float* out, float* lse,
                                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Slow step with per-query-head logits (t_q = 1): as sfi_dense_attn_with_stats,
 * but scores [B, Hq, score_stride] holds one masked logit row per query head,
 * scale * q_h . k_j, instead of the sum over the group (the per-head attention
 * statistics of the SparseSpec-L abstract, kept per head).  Feeding its rows to
 * sfi_select_topk with num_kv_heads = Hq selects per query head.  scores must be
 * non-NULL; the workspace is sfi_dense_attn_workspace_size(shape, kv, 1).
 */
SFI_API sfi_status sfi_dense_attn_with_head_stats(const sfi_shape* shape, const sfi_paged_kv* kv, const void* q,
                                          const int32_t* seq_lens, int32_t n_sink, int32_t n_recent,
                                          float* out, float* lse, float* scores, int64_t score_stride,
                                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fast step over an index set read in place (sink + selected + recent, SFI page,
 * Fig. 2; the selected set shared by the layers of a draft step that an intra-draft
 * refresh layer refreshes, ASPIRE abstract).  Every row is read from paged KV through
 * the block table, so no compact buffer is packed.  For request b and KV head g the
 * attended positions are, in order: [0, min(n_sink, L_b)), every entry of
 * sel_idx[b, g, 0:k] that lies in [0, L_b) (negative entries are padding), then
 * [max(n_sink, L_b - n_recent), L_b).  A position behind an invalid block-table
 * entry is skipped.  With every entry of sel_idx a valid position (no padding), the
 * result equals sfi_pack_compact followed by sfi_sparse_decode_attn with cap =
 * n_sink + k bit for bit while no split of the plan holds 8 or more loop iterations
 * of compact rows only (512 rows at most shapes; sfi_sparse_decode_attn starts such
 * splits at a rotated iteration); otherwise, and with padding (the two then split
 * the work at other tokens), they agree to rounding.
 *
 *   sel_idx  int32 [B, Hkv, k], device, e.g. the output of sfi_select_topk; k >= 0
 *            (sel_idx may be NULL when k is 0; n_sink = k = 0 attends the recent
 *            window alone).
 *   per_head 0: one set per KV head, shared by its query heads.  1: one set per
 *            query head, sel_idx [B, Hq, k] (per-query-head selection, e.g.
 *            sfi_select_topk over the rows of sfi_dense_attn_with_head_stats); query
 *            head h reads KV head h / G at its own positions.  The workspace is then
 *            sized by the same query with num_kv_heads set to num_q_heads.
 *   k_new, v_new  both NULL, or the decoded token's K/V [B, Hkv, d] (16-byte aligned)
 *            stored and attended as in sfi_sparse_decode_append_attn.
 *   compact_k, compact_v, cap, n_compact  all NULL (cap ignored), or a compact buffer
 *            [B, units, cap, d] (units = Hkv, or Hq with per_head; 16-byte aligned,
 *            cap >= n_sink + k) and n_compact [B]: the launch also writes them exactly as
 *            sfi_pack_compact would for sel_idx (SFI page, Fig. 3B), so the first fast
 *            step after a refresh packs the state the following fast steps read.  With
 *            one set per KV head and no appended token, work-groups of their own in the
 *            same launch copy the rows; otherwise the attention work-groups write the
 *            rows they read.
 *   workspace  as sfi_sparse_decode_workspace_size(shape, kv, n_sink + k, n_recent).
 *   Other arguments as sfi_sparse_decode_attn.  Errors: SFI_ERR_INVALID_ARG for a
 *   NULL sel_idx with k > 0, negative k, per_head not 0 or 1, an unpaired
 *   k_new / v_new, or a partial or misaligned compact buffer or cap < n_sink + k;
 *   SFI_ERR_UNSUPPORTED when
 *   num_pages * 16 exceeds INT32_MAX.
 */
SFI_API sfi_status sfi_sparse_decode_indexed_attn(const sfi_shape* shape, const sfi_paged_kv* kv, const void* q,
                                          const void* k_new, const void* v_new, const int32_t* seq_lens,
                                          int32_t n_sink, int32_t n_recent, const int32_t* sel_idx, int32_t k,
                                          int32_t per_head, void* compact_k, void* compact_v, int32_t cap,
                                          int32_t* n_compact, float* out, float* lse, void* workspace,
                                          size_t workspace_bytes, void* stream);

/*
 * The rest of a slow step in one launch: the index-set fast step (as
 * sfi_sparse_decode_indexed_attn with no appended token and one selection per
 * KV head) that also packs compact_k / compact_v / n_compact (as
 * sfi_pack_compact) and merges the split partials that
 * sfi_dense_attn_with_stats_deferred left in slow_workspace into slow_out and
 * slow_lse (SFI page, Fig. 2 and Fig. 3B: the slow step's selection is packed
 * while the next attention runs; here all three run as work-groups of one
 * launch, the attention reading the selected rows in place).  The compact
 * buffer, n_compact, slow_out and slow_lse are bit-identical to the plain calls;
 * out and lse are as sfi_sparse_decode_indexed_attn gives them.  The shape, kv and
 * seq_lens are the slow step's; workspace (for this call's own split partials, of
 * sfi_sparse_decode_workspace_size(shape, kv, n_sink + k, n_recent) bytes) and
 * slow_workspace must not overlap.  Errors as the calls it replaces; nothing is
 * launched on any error.
 *
 *   q         [B, Hq, d] (pool dtype); out [B, Hq, d] float32, lse [B, Hq] float32 or NULL
 *   sel_idx   int32 [B, Hkv, k]; compact_k, compact_v [B, Hkv, cap, d] (16-byte aligned,
 *             cap >= n_sink + k); n_compact int32 [B]
 *   slow_out  [B, 1, Hq, d] float32 and slow_lse [B, 1, Hq] float32 or NULL, as passed to
 *             sfi_dense_attn_with_stats_deferred; slow_workspace its workspace
 */
SFI_API sfi_status sfi_sparse_decode_indexed_attn_merge(const sfi_shape* shape, const sfi_paged_kv* kv,
                                                const void* q, const int32_t* seq_lens,
                                                int32_t n_sink, int32_t n_recent,
                                                const int32_t* sel_idx, int32_t k, void* compact_k,
                                                void* compact_v, int32_t cap, int32_t* n_compact,
                                                float* out, float* lse, void* workspace,
                                                size_t workspace_bytes, float* slow_out,
                                                float* slow_lse, void* slow_workspace,
                                                size_t slow_workspace_bytes, void* stream);

/*
 * Drafting and verifying requests in one launch (ASPIRE abstract: a unified
 * mixed forward lets drafting and verifying requests share one batched
 * pass; SparseSpec-L abstract: drafts attend over a sparse, recallable KV
 * cache, verification is full-context attention that yields per-head
 * statistics).  modes[b] = 0: request b drafts one token with the fast step
 * (t_q[b] must be 1).  modes[b] = 1: request b verifies t_q[b] draft tokens
 * with dense causal attention and writes its scores row.  BF16 only; B <= 64.
 *
 *  modes, t_q  host int32 [B]
 *  q           [R, Hq, d] dtype, R = sum of t_q; request b's rows start at
 *              the sum of t_q over requests before b
 *  out         [R, Hq, d] float32;  lse [R, Hq] float32 or NULL
 *  scores      [B, Hkv, score_stride] float32 or NULL; rows of drafting
 *              requests are not written
 *  compact_k/v, cap, n_compact as for sfi_sparse_decode_attn (used by
 *              drafting requests only)
 *  workspace: at least sfi_mixed_attn_workspace_size() bytes.
 */
SFI_API sfi_status sfi_mixed_attn(const sfi_shape* shape, const sfi_paged_kv* kv, const void* q,
                          const int32_t* modes, const int32_t* t_q, const int32_t* seq_lens,
                          int32_t n_sink, int32_t n_recent, const void* compact_k,
                          const void* compact_v, int32_t cap, const int32_t* n_compact,
                          float* out, float* lse, float* scores, int64_t score_stride,
                          void* workspace, size_t workspace_bytes, void* stream);

SFI_API sfi_status sfi_mixed_attn_workspace_size(const sfi_shape* shape, const sfi_paged_kv* kv,
                                         const int32_t* modes, const int32_t* t_q, int32_t cap,
                                         int32_t n_recent, size_t* bytes);

/*
 * Launch plan of the split-K attention calls, for inspection and tests
 * (host only, no GPU needed).  op: 0 = dense / verify (t_q as given),
 * 1 = sparse decode.  Returns the tokens per split and splits per (b, g).
 * A split holds at most 4096 tokens; where that cap needs more work-groups
 * than the target, the tokens are cut evenly over as many splits as fill the
 * waves of work-groups the cap needs (so that no CU streams two long splits
 * while another streams one).
 * For op 1 the splits cut the virtual rows [0, cap + recent) evenly, except
 * when the compact rows need several splits and one more work-group per
 * (b, g) still fits the plan's target of about one work-group per CU: then
 * n_split - 1 splits of split_tokens cover the compact rows [0, cap) and the
 * recent window is the last split on its own.
 */
SFI_API sfi_status sfi_plan_splits(int32_t op, const sfi_shape* shape, const sfi_paged_kv* kv,
                           int32_t t_q, int32_t cap, int32_t n_recent,
                           int32_t* split_tokens, int32_t* n_split);

/*
 * Measurement helper, not part of the decode path: a plain streaming copy
 * of `bytes` bytes (a multiple of 16) from src to dst, used to calibrate
 * hardware byte counters against a kernel of known traffic.
 */
SFI_API sfi_status sfi_stream_copy(const void* src, void* dst, size_t bytes, void* stream);

/*
 * Measurement helper, not part of the decode path: reads `bytes` bytes (a multiple
 * of 16) of device memory at src once, in address order, and writes nothing but (in
 * practice never) one word at sink (device, 4 bytes).  Its rate is the streaming HBM
 * read rate the decode kernels are compared against.
 */
SFI_API sfi_status sfi_stream_read(const void* src, size_t bytes, void* sink, void* stream);

SFI_API const char* sfi_status_string(sfi_status status);
SFI_API const char* sfi_last_error(void);
SFI_API int32_t sfi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SFI_H_ */
