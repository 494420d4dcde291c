/*
 * kap.h -- C ABI of the selected-KV paged decode attention library (libkap.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * The path, per request and attention layer:
 *   1. kap_score_blocks  score every KV page: rotated query . block-mean K
 *      (kap_score_pool_blocks also folds the heads into the pooled key)
 *   2. kap_select_topk   pick pages under an anchor / recent / middle split
 *   3. kap_compact_view  compact block table + slot mapping over the pick
 *      (kap_select_compact does steps 2 and 3 in one launch)
 *   4. kap_decode_attn   q = 1 GQA decode over the compact view
 *   5. kap_verify_attn   short query window over the full paged KV
 * and around it: kap_append_kv writes the window's K/V through the slot
 * mapping (so the verify can attend causally to it), kap_update_summary /
 * kap_build_summary keep the block-mean K summaries current, kap_proxy_query
 * (or kap_proxy_query_packed over a weight packed once) forms an early-routing
 * query, and kap_kv_pool_layout says where to place a layer's K and V pools.
 *
 * Sources (web pages the method is described on):
 *   [KAP]  "KAP: Bridging the Knowledge Selection-Runtime Consumption Gap in
 *          LLM Systems" (arXiv 2607.24260): selected-KV view, executor,
 *          verifier, shape stabilization and fallback paragraphs.
 *   [KRI]  knlp.io "KRI" page: KRI-Q variant and the A<a>R<r>K<k> tag section.
 *   [ESKV] EarlySelectKV news item, Interpretation: proxy-query routing over a
 *          K-summary cache.
 *
 * Conventions shared by every entry point
 *   - Pointers named *device* are device memory owned by the caller; the
 *     library never frees, keeps or allocates memory (the one exception is the
 *     static per-GPU scratch of kap_decode_attn_noalloc, part of the loaded
 *     code object).  Scalars are host values.
 *   - Every call enqueues kernels on `stream` (a hipStream_t; NULL = default
 *     stream) and returns without synchronizing, so a sequence of calls can be
 *     captured in a HIP graph ([KAP] stabilizes shapes, tables and metadata so
 *     that proposal and verify replay as graphs).
 *   - All shape, dtype and size checks run on the host before any launch and
 *     return a status; kap_last_error() then holds a message for the calling
 *     thread.  Bulk-data pointers (queries, hidden states, weights, K/V pools,
 *     summaries, attention outputs, workspaces) must be 16-byte aligned, as
 *     hipMalloc and torch allocations are: the kernels move them in 16-byte
 *     vectors.  A call with one that is not returns KAP_ERR_INVALID_ARG.  Device-side data are trusted: page ids outside [0, num_pages)
 *     or lengths beyond a table's width are undefined behaviour.
 *   - Element types: KAP_F32 (float) and KAP_BF16 (bfloat16 stored as 16-bit).
 *   - Page size is 16 tokens; head_dim is 64 or 128; Hq is a multiple of Hkv,
 *     query heads map to KV heads in contiguous groups g(h) = h / (Hq/Hkv).
 *   - Paged KV layout, per attention layer (dense, element offsets):
 *       K pool [num_pages][Hkv][16][D]   (token-major inside a page)
 *       V pool [num_pages][Hkv][D][16]   (dim-major inside a page: the 16
 *                                         values of one dim are contiguous)
 *     Summary pool [num_pages][Hkv][D].  Block table [B][max_pages] int32
 *     maps logical page p of request b to its physical page (-1: none).
 *     The K and V pools may sit anywhere; kap_kv_pool_layout gives the
 *     placement in one allocation that reads fastest.
 *   - Results are bit-identical from run to run and do not depend on where
 *     pages sit in the pool.
 */
#ifndef KAP_H
#define KAP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KAP_API __attribute__((visibility("default")))

typedef enum {
  KAP_OK = 0,
  KAP_ERR_INVALID_ARG = 1, /* null pointer, negative or inconsistent size        */
  KAP_ERR_UNSUPPORTED = 2, /* valid but not implemented (dtype, head_dim, ...)    */
  KAP_ERR_CAPACITY = 3,    /* selection budget exceeds the compact capacity: the
                              caller's cue to fall back to full context ([KAP]
                              fallback when a plan exceeds the compact workspace) */
  KAP_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required          */
  KAP_ERR_HIP = 5          /* a HIP launch or runtime call failed                 */
} kap_status;

typedef enum { KAP_F32 = 0, KAP_BF16 = 1 } kap_dtype;

typedef void* kap_stream; /* hipStream_t */

/* Static text for a status code. */
KAP_API const char* kap_status_string(kap_status s);
/* Detail of the last failing call on this thread ("" if none). */
KAP_API const char* kap_last_error(void);
/* Library version string. */
KAP_API const char* kap_version(void);

/*
 * Page scores.  [KRI] KRI-Q: query-aware agreement of the query with each
 * block's mean key; the query is first rotated at its full-sequence logical
 * position ([KAP] executor).  For request b, KV head g and logical page p:
 *   u_g        = sum over query heads h of group g of RoPE(q[b][h], positions[b])
 *   scores[b][g][p] = u_g . summary[block_table[b][p]][g]   for p < ceil(seq_lens[b]/16)
 *                   = -inf                                   for the other p < max_pages
 * A raw dot product (no 1/sqrt(D), no softmax).  RoPE pairs element i with
 * i + D/2 at frequency rope_theta^(-2i/D); angles are formed in fp64.
 *   q          device [B][Hq][D], q_dtype (unrotated query)
 *   positions  device [B] int32 logical position of the query
 *   summary    device [num_pages][Hkv][D], sum_dtype (block-mean K per page)
 *   block_table device [B][max_pages] int32; seq_lens device [B] int32
 *   scores     device out [B][Hkv][max_pages] float
 */
KAP_API kap_status kap_score_blocks(const void* q, int32_t q_dtype, const int32_t* positions,
                            float rope_theta, const void* summary, int32_t sum_dtype,
                            int32_t num_pages, const int32_t* block_table, int32_t max_pages,
                            const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                            int32_t D, int32_t page_size, float* scores, kap_stream stream);

/*
 * Page scores of every KV head plus the head-pooled key in one launch, for
 * pooled selection ([KRI] the connector mean-pools scores across heads before
 * the per-request top-K).  scores as in kap_score_blocks, bit for bit the
 * same arithmetic per head, and
 *   pooled[b][p] = (((S0 + S1) + S2) + ... + S_{Hkv-1}) / Hkv   for p < N_b
 *                = -inf                                         for the other p < max_pages
 * in fp32 with round-to-nearest adds in head order and one rounded division:
 * exactly the key kap_select_topk forms for per_head = 0.  So kap_select_topk
 * on (pooled, Hkv = 1) makes the same selection as on (scores, Hkv) pooled,
 * while it reads one key row per request instead of Hkv.
 *   pooled device out [B][max_pages] float
 * Either output may be NULL (not both): it is then not written.
 * Hkv <= 16 and Hq * D * (q element bytes) <= 64 KiB (else KAP_ERR_UNSUPPORTED);
 * otherwise as kap_score_blocks.
 */
KAP_API kap_status kap_score_pool_blocks(const void* q, int32_t q_dtype, const int32_t* positions,
                                 float rope_theta, const void* summary, int32_t sum_dtype,
                                 int32_t num_pages, const int32_t* block_table,
                                 int32_t max_pages, const int32_t* seq_lens, int32_t B,
                                 int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size,
                                 float* scores, float* pooled, kap_stream stream);

/*
 * Proxy query for early routing.  [ESKV] Interpretation: the side flow builds
 * a proxy query from a preceding hidden state through the query projection,
 * then scores and selects over the K-summary cache before the target layer.
 *   q_out[b][n] = sum_c hidden[b][c] * w_q[c][n]     (bf16 inputs, fp32 accumulation on
 *                 the matrix cores, row splits of 128 added in split order: deterministic)
 *   hidden device [B][d_model] bf16; w_q device [d_model][n_out] bf16 (row-major)
 *   q_out  device out [B][n_out] float -- feed to kap_score_blocks as KAP_F32
 *          with n_out = Hq * D.
 *   workspace device, >= kap_proxy_workspace_bytes(B, d_model, n_out)
 * 1 <= B <= 16; d_model a multiple of 128; n_out a multiple of 512.
 */
KAP_API size_t kap_proxy_workspace_bytes(int32_t B, int32_t d_model, int32_t n_out);
KAP_API kap_status kap_proxy_query(const void* hidden, const void* w_q, int32_t B, int32_t d_model,
                           int32_t n_out, float* q_out, void* workspace, size_t workspace_bytes,
                           kap_stream stream);

/*
 * The same proxy query in one launch, over a query projection packed once
 * for it ([ESKV] Interpretation: the side flow's projection of the preceding
 * hidden state; W_q is a static weight, so its layout is ours to choose).
 * kap_proxy_pack_weights writes the packed copy (same size, 2 * d_model *
 * n_out bytes) of a row-major W_q: element (r, c) goes to
 *   w_packed[((((c / 16) * (d_model / 32) + r / 32) * 4 + (r % 32) / 8) * 16 + c % 16) * 8 + r % 8]
 * (each 16-column tile's whole d_model contiguous; 8 consecutive rows of one
 * column per 16 bytes).  kap_proxy_query_packed then computes
 *   q_out[b][n] = sum_c hidden[b][c] * w_q[c][n]
 * with bf16 inputs and fp32 accumulation on the matrix cores: each of eight
 * row shares of a 16-column tile is summed in row order, and the shares are
 * added in order (deterministic; it agrees with kap_proxy_query to fp32
 * rounding, not bit for bit).  No workspace.
 *   w_q      device [d_model][n_out] bf16 (row-major); w_packed device out, a
 *            separate buffer of the same size
 *   hidden   device [B][d_model] bf16; q_out device out [B][n_out] float (as
 *            kap_proxy_query writes it)
 * 1 <= B <= 16; d_model a multiple of 32; n_out a multiple of 16.
 */
KAP_API kap_status kap_proxy_pack_weights(const void* w_q, int32_t d_model, int32_t n_out,
                                          void* w_packed, kap_stream stream);
KAP_API kap_status kap_proxy_query_packed(const void* hidden, const void* w_packed, int32_t B,
                                          int32_t d_model, int32_t n_out, float* q_out,
                                          kap_stream stream);

/*
 * Top-K pages under the A<a>R<r>K<k> split ([KRI] A<a>R<r>K<k> tag section):
 * anchors = the first a logical pages, recents = the last r, plus the best
 * k_mid pages of the middle [a, N - r) by score (N = ceil(seq_lens[b]/16)).
 * When a + r >= N every page is taken.  Ranking: score descending, ties to the
 * lowest page index; -0 equals +0; NaN ranks below -inf.
 * per_head = 0 (pooled): one selection per request on the mean over KV heads,
 *   folded in fp32 as ((S0 + S1) + ... + S_{H-1}) / H ([KRI] the connector
 *   mean-pools across heads before the per-request top-K).
 * per_head = 1: an independent selection per KV head ([ESKV] per-head routing).
 * Output lists are ascending ([KAP] selected pages are compacted in access
 * order) and padded with -1.  G = per_head ? Hkv : 1.
 *   scores     device [B][Hkv][max_pages] float (from kap_score_blocks)
 *   anchor, recent, k_mid  device [B] int32
 *   max_budget host upper bound of anchor+recent+k_mid over the batch
 *   capacity   pages per output row; max_budget > capacity -> KAP_ERR_CAPACITY
 *              before any launch.  If the device values still exceed it, the
 *              row is truncated to capacity (memory stays in bounds).
 *   sel_pages  device out [B][G][capacity] int32; sel_count device out [B][G]
 * max_pages <= 65536.
 */
KAP_API kap_status kap_select_topk(const float* scores, int32_t B, int32_t Hkv, int32_t max_pages,
                           const int32_t* seq_lens, int32_t page_size, int32_t per_head,
                           const int32_t* anchor, const int32_t* recent, const int32_t* k_mid,
                           int32_t max_budget, int32_t capacity, int32_t* sel_pages,
                           int32_t* sel_count, kap_stream stream);

/*
 * Host helper: keep the selected-KV plan or fall back to full-context decoding.
 * [KAP] stability/fallback paragraph: the plan falls back to full context when
 * it exceeds the compact workspace, or when the retained ratio s is high or the
 * acceptance h low; [KAP-T] (the tutorial's phase-boundary section) makes the
 * second condition exact under the memory-bound cost model of one cycle of k
 * proposal steps and one verification:
 *   Cost_base = (1 + k h) (W_main + KV),  Cost_plan = k (W_main + s KV) + (W_main + KV)
 * (proposal weights = main weights), and Cost_plan < Cost_base  <=>
 *   (h - s) KV > (1 - h) W_main.
 *   h             acceptance rate of proposed tokens, in [0, 1]
 *   s             retained ratio: bytes a proposal step reads / bytes a
 *                 full-context step reads, in [0, 1]
 *   w_main_bytes  per-step weight (and other non-KV) bytes of the main model, >= 0
 *   kv_bytes      per-step full-context KV bytes, >= 0
 *   k             proposal steps per cycle, >= 1
 *   budget_pages  largest selection budget of the batch (a + r + k pages);
 *   capacity      compact capacity in pages
 *   choice        out: KAP_PLAN_SELECTED, or the first fallback reason in the
 *                 order capacity, margin (h <= s), boundary
 *   speedup       out (may be NULL): Cost_base / Cost_plan of the cycle (> 1
 *                 exactly when the boundary holds); computed for every choice
 * Returns KAP_ERR_INVALID_ARG for values outside these ranges (NaN included).
 */
typedef enum {
  KAP_PLAN_SELECTED = 0,       /* keep the selected-KV plan                       */
  KAP_PLAN_FULL_CAPACITY = 1,  /* budget_pages > capacity                          */
  KAP_PLAN_FULL_MARGIN = 2,    /* h <= s: the plan cannot pay off at any KV size   */
  KAP_PLAN_FULL_BOUNDARY = 3   /* (h - s) KV <= (1 - h) W_main                     */
} kap_plan_choice;
KAP_API kap_status kap_choose_plan(double h, double s, double w_main_bytes, double kv_bytes,
                                   int32_t k, int32_t budget_pages, int32_t capacity,
                                   int32_t* choice, double* speedup);

/* Host helper: page budget for retention s = s_num/s_den over n_pages pages,
 * ceil(n_pages * s) in integers, raised to anchor + recent, capped at n_pages.
 * The middle count is budget - anchor - recent.  Returns -1 on bad input. */
KAP_API int32_t kap_budget_from_ratio(int32_t n_pages, int64_t s_num, int64_t s_den, int32_t anchor,
                              int32_t recent);

/*
 * Host helper: where to place one attention layer's K pool and V pool (the
 * paged pools every block table indexes, [KAP] selected-KV view) in a single
 * device allocation.  Any placement gives the same results; this one reads
 * fastest.  The K pool starts at byte 0 and the V pool at
 *   v_offset = (K pool bytes rounded up to 16 KiB) + 4 KiB,
 * so that the K tile and the V tile of one (page, KV head), which one wave
 * requests together, never share address bits 12-13.  V pools at a multiple
 * of 16 KiB from their K pool (two separate 2 MiB-aligned allocations always
 * are) made the full-context verify at 128K 1.5-5 % slower on MI355X.
 *   num_pages, num_kv_heads, head_dim (64 or 128), page_size (16),
 *   elem_bytes (2: bf16, 4: f32)  the pools' shape, as the attention calls take it
 *   v_offset_bytes  host out: byte offset of the V pool from the allocation
 *   total_bytes     host out: bytes to allocate (K pool, gap, V pool)
 * Returns KAP_ERR_INVALID_ARG for null outputs, negative or oversized pools,
 * KAP_ERR_UNSUPPORTED for other head_dim or page_size values.
 */
KAP_API kap_status kap_kv_pool_layout(int64_t num_pages, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t page_size, int32_t elem_bytes,
                                      int64_t* v_offset_bytes, int64_t* total_bytes);

/*
 * Compact view over a selection ([KAP] selected-KV view: a compact table of
 * the chosen pages' physical ids in ascending logical order, the logical pages
 * kept beside it, and a slot for each new token).  For row (b, gr):
 *   compact_bt[j]      = block_table[b][sel_pages[j]]   (j < sel_count, else -1)
 *   compact_logical[j] = sel_pages[j]                   (j < sel_count, else -1)
 *   compact_len        = total valid tokens of the selected pages (the last
 *                        logical page holds seq_len - 16 (N - 1) tokens)
 *   slot_mapping[b][i] = block_table[b][t/16]*16 + t%16 for t = positions[b] + i,
 *                        or -1 when t/16 >= max_pages or that entry is -1.
 * The compact table is a plain paged view: its first compact_len tokens are the
 * selected tokens in ascending logical order, so kap_decode_attn reads it like
 * any other table.
 *   sel_pages device [B][G][capacity], sel_count device [B][G] (kap_select_topk)
 *   compact_bt, compact_logical device out [B][G][capacity]; compact_len device out [B][G]
 *   slot_mapping device out [B][q_new] int64 (may be NULL when q_new == 0)
 */
KAP_API kap_status kap_compact_view(const int32_t* sel_pages, const int32_t* sel_count, int32_t B,
                            int32_t G, int32_t capacity, const int32_t* block_table,
                            int32_t max_pages, const int32_t* seq_lens, int32_t page_size,
                            const int32_t* positions, int32_t q_new, int32_t* compact_bt,
                            int32_t* compact_logical, int32_t* compact_len,
                            int64_t* slot_mapping, kap_stream stream);

/*
 * Top-K and compact view in one launch: kap_select_topk followed by
 * kap_compact_view over its output, with the same results ([KAP] selected-KV
 * view: the selection is compacted in access order).  compact_logical is the
 * selection list itself (what kap_select_topk writes to sel_pages), sel_count
 * its length; compact_bt, compact_len and slot_mapping are as
 * kap_compact_view writes them.  Arguments as in those two calls; capacity
 * may be 0 (counts and lengths are still written).
 */
KAP_API kap_status kap_select_compact(const float* scores, int32_t B, int32_t Hkv,
                              int32_t max_pages, const int32_t* seq_lens, int32_t page_size,
                              int32_t per_head, const int32_t* anchor, const int32_t* recent,
                              const int32_t* k_mid, int32_t max_budget, int32_t capacity,
                              const int32_t* block_table, const int32_t* positions,
                              int32_t q_new, int32_t* sel_count, int32_t* compact_bt,
                              int32_t* compact_logical, int32_t* compact_len,
                              int64_t* slot_mapping, kap_stream stream);

/*
 * Workspace for kap_decode_attn (q_len = 1) and kap_verify_attn: the split-K
 * work plan's per-row offsets and the split partials (m and l in fp32; o in
 * bf16, normalized, for bf16 pools and unnormalized fp32 for f32 pools).
 * Caller-owned device memory of at least this many bytes; its contents need
 * no initialization and are overwritten by every call (so concurrent calls
 * need separate workspaces).
 */
KAP_API size_t kap_attn_workspace_bytes(int32_t B, int32_t q_len, int32_t Hq, int32_t Hkv, int32_t D);

/*
 * q = 1 GQA decode attention over a paged view ([KAP] executor: each proposal
 * step is a decode-like forward with one query token at its full-sequence
 * logical position, over the compact block table and compact metadata).
 * For request b and query head h (KV head g = g(h), table row gr = G == 1 ? 0 : g),
 * with j = (b*G + gr)*table_width + t/16:
 *   view   = the first lens[b][gr] tokens of table row (b, gr): token t lives at
 *            page block_table[j], slot t%16, and sits at logical position
 *            lambda(t) = logical_table[j]*16 + t%16 (lambda(t) = t when
 *            logical_table is NULL: a full block table, entry p = logical page p)
 *   keys   = the tokens t of the view with lambda(t) <= positions[b] (logical
 *            positions are kept in the compact view, [KAP] selected-KV view, so
 *            the causal rule is the full-context one)
 *   z_t    = scale * RoPE(q[b][h], positions[b]) . K(t)
 *   out    = sum_t e^{z_t - m} V(t) / sum_t e^{z_t - m};  lse = m + ln sum_t e^{z_t - m}
 * Work is split over page chunks (split-K) and merged with a log-sum-exp
 * combine in fixed order.  Use (block_table, NULL, max_pages, G = 1, seq_lens)
 * for full-context decode and (compact_bt, compact_logical, capacity, G,
 * compact_len) for the selected view.  A row with no key yields out = 0 and
 * lse = -inf.
 * The view holds the context only: tokens proposed after positions[b] are not
 * in a compact view built over seq_lens, so proposal step j > 0 does not see
 * the drafts of steps 0 .. j-1 (their KV is written by kap_append_kv before
 * the verify, which reads the full table).
 * Precision: bf16 K/V run on the matrix cores with the rotated query and the
 * probabilities rounded to bf16 and fp32 accumulation, softmax and merge;
 * fp32 K/V run in fp32 throughout.
 *   q        device [B][Hq][D], q_dtype; out device [B][Hq][D], same dtype as q
 *   lse      device out [B][Hq] float, natural log, or NULL
 *   k_pool, v_pool device, kv_dtype, layouts above; q_dtype must equal kv_dtype
 *   logical_table device [B][G][table_width] int32 or NULL (see above)
 *   lens     device [B][G] int32 (lens <= 16 * table_width)
 *   workspace device, >= kap_attn_workspace_bytes(B, 1, Hq, Hkv, D)
 */
KAP_API kap_status kap_decode_attn(const void* q, int32_t q_dtype, const int32_t* positions,
                           float rope_theta, float scale, const void* k_pool, const void* v_pool,
                           int32_t kv_dtype, int32_t num_pages, int32_t Hkv, int32_t D,
                           int32_t page_size, const int32_t* block_table,
                           const int32_t* logical_table, int32_t table_width, int32_t G,
                           const int32_t* lens, int32_t B, int32_t Hq, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, kap_stream stream);

/*
 * Allocation-free variant of kap_decode_attn, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments without the
 * workspace, the same kernels and the same results bit for bit.  The split-K
 * workspace is a static device array of KAP_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends; its address is looked up
 * once per device on the first call with that device current.  No call
 * allocates or frees memory.
 *   Returns KAP_ERR_WORKSPACE, before any HIP call, when the call needs more
 *   than KAP_NOALLOC_SCRATCH_BYTES (kap_attn_workspace_bytes(B, 1, Hq, Hkv, D)
 *   is the need); use kap_decode_attn with a workspace then.
 *   Every call on one GPU shares that GPU's array and overwrites what the last
 *   call left there (nothing in it needs to start at zero).  Calls that
 *   overlap on one GPU (other streams, other threads) race: serialize them.
 */
#define KAP_NOALLOC_SCRATCH_BYTES (16u << 20)
KAP_API kap_status kap_decode_attn_noalloc(const void* q, int32_t q_dtype,
                                           const int32_t* positions, float rope_theta,
                                           float scale, const void* k_pool, const void* v_pool,
                                           int32_t kv_dtype, int32_t num_pages, int32_t Hkv,
                                           int32_t D, int32_t page_size,
                                           const int32_t* block_table,
                                           const int32_t* logical_table, int32_t table_width,
                                           int32_t G, const int32_t* lens, int32_t B, int32_t Hq,
                                           void* out, float* lse, kap_stream stream);

/*
 * Full-context verification window ([KAP] verifier: a short contiguous query
 * window scored against the full KV cache, full block table and original
 * logical positions).  Query i of request b sits at start_positions[b] + i and
 * is rotated there; it sees key t (logical position t, read through the full
 * block table) iff t < seq_lens[b] and t <= start_positions[b] + i.
 * Otherwise as kap_decode_attn.  1 <= q_len <= 16.
 *   q   device [B][q_len][Hq][D]; out device [B][q_len][Hq][D] (q dtype)
 *   lse device out [B][q_len][Hq] float or NULL
 *   workspace >= kap_attn_workspace_bytes(B, q_len, Hq, Hkv, D)
 */
KAP_API kap_status kap_verify_attn(const void* q, int32_t q_dtype, const int32_t* start_positions,
                           int32_t q_len, float rope_theta, float scale, const void* k_pool,
                           const void* v_pool, int32_t kv_dtype, int32_t num_pages, int32_t Hkv,
                           int32_t D, int32_t page_size, const int32_t* block_table,
                           int32_t max_pages, const int32_t* seq_lens, int32_t B, int32_t Hq,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           kap_stream stream);

/*
 * Block-mean K summary maintenance ([ESKV] the K-summary cache kept beside the
 * KV; [KRI] KRI-Q's block-mean K).  For every logical page p < N_b of every
 * request, summary[block_table[b][p]][g][:] = mean of K over that page's valid
 * tokens (seq_len - 16 p on the last page), fp32 accumulation, stored in
 * sum_dtype with round-to-nearest-even.  Pages not referenced are untouched.
 */
KAP_API kap_status kap_build_summary(const void* k_pool, int32_t kv_dtype, int32_t num_pages,
                             int32_t Hkv, int32_t D, int32_t page_size,
                             const int32_t* block_table, int32_t max_pages,
                             const int32_t* seq_lens, int32_t B, void* summary,
                             int32_t sum_dtype, kap_stream stream);

/*
 * Block-mean K summary update after an append ([ESKV] the K-summary cache is
 * kept current as tokens arrive).  Recomputes, exactly as kap_build_summary
 * does, only the logical pages that hold the tokens at positions[b] + i,
 * 0 <= i < q_new (pages at or past ceil(seq_lens[b] / 16) are skipped).
 * seq_lens are the lengths after the append.  Every other summary row is
 * untouched.
 *   positions device [B] int32 (first new token's logical position)
 */
KAP_API kap_status kap_update_summary(const void* k_pool, int32_t kv_dtype, int32_t num_pages,
                                      int32_t Hkv, int32_t D, int32_t page_size,
                                      const int32_t* block_table, int32_t max_pages,
                                      const int32_t* seq_lens, const int32_t* positions,
                                      int32_t q_new, int32_t B, void* summary, int32_t sum_dtype,
                                      kap_stream stream);

/*
 * Compact KV workspace ([KAP] selected-KV view: the executor materializes a
 * compact physical view of the selected pages; [KAP] shape stabilization: a
 * reusable compact KV workspace, filled once per plan).  Workspace page
 * b*capacity + j receives, in head slot g, head g of compact page j of row
 * (b, G == 1 ? 0 : g) -- K and V tiles copied bit for bit -- and
 * ws_table[b][gr][j] = b*capacity + j where compact_bt[b][gr][j] >= 0, else -1.
 * kap_decode_attn over (k_ws, v_ws, ws_table, compact_len) then gives the same
 * bits as over (k_pool, v_pool, compact_bt, compact_len), reading contiguous
 * workspace pages instead of scattered pool pages.  Workspace slots without a
 * source page are left as they were.
 *   compact_bt device [B][G][capacity] (kap_compact_view); G is 1 or Hkv
 *   k_ws, v_ws device [ws_pages][Hkv][16][D] and [ws_pages][Hkv][D][16], kv_dtype;
 *     ws_pages >= B * capacity, else KAP_ERR_WORKSPACE
 *   ws_table device out [B][G][capacity]
 */
KAP_API kap_status kap_materialize_view(const void* k_pool, const void* v_pool, int32_t kv_dtype,
                                        int32_t num_pages, int32_t Hkv, int32_t D,
                                        int32_t page_size, const int32_t* compact_bt, int32_t B,
                                        int32_t G, int32_t capacity, void* k_ws, void* v_ws,
                                        int32_t ws_pages, int32_t* ws_table, kap_stream stream);

/*
 * KV append through a slot mapping ([KAP] verifier: a verify pass moves the
 * committed full-context KV forward; [KAP] selected-KV view: the slot mapping
 * gives each new token its physical page and offset).  Token i of request b
 * goes to slot s = slot_mapping[b][i] = page * 16 + offset: its K row for KV
 * head g becomes k_pool[page][g][offset][:] and its V values become
 * v_pool[page][g][:][offset].  Rows are copied bit for bit (K as the cache
 * holds it, already rotated).  Slots equal to -1, or at or beyond
 * num_pages * 16, are skipped.  Two tokens with the same slot race; the caller
 * keeps slots distinct (kap_compact_view's slot mapping is).
 *   k_new, v_new device [B][q_new][Hkv][D] in kv_dtype
 *   slot_mapping device [B][q_new] int64
 *   k_pool, v_pool device, updated in place (layouts as in kap_decode_attn)
 */
KAP_API kap_status kap_append_kv(const void* k_new, const void* v_new, int32_t kv_dtype,
                                 const int64_t* slot_mapping, int32_t B, int32_t q_new,
                                 int32_t Hkv, int32_t D, int32_t page_size, int32_t num_pages,
                                 void* k_pool, void* v_pool, kap_stream stream);

/*
 * CPU-offloaded early routing ([ESKV] Interpretation: once indices are
 * available early, proxy-query construction, routing and the K-summary state
 * can move to the CPU and finish before target attention; the GPU keeps the
 * KV and receives only page indices).  Same definitions as kap_proxy_query,
 * kap_score_blocks and kap_select_topk, computed on host threads over HOST
 * memory; every pointer below is host memory.  Synchronous; `threads` <= 0
 * means OMP_NUM_THREADS, else the CPUs this process may run on.  The GPU side
 * takes sel_pages / sel_count as uploaded indices (copy them to the device,
 * then kap_compact_view).
 *   kap_host_proxy_query: q_out [B][n_out] fp32 = hidden [B][d_model] (bf16)
 *     . w_q [d_model][n_out] (bf16); fp32 sums in index order; B <= 64.
 *   kap_host_score_blocks: q [B][Hq][D] fp32 (unrotated), summary
 *     [num_pages][Hkv][D] bf16, scores [B][Hkv][max_pages] (-inf past N_b);
 *     rotation and group sum in fp64, dot in fp64, one rounding to fp32.
 *   kap_host_select_topk: as kap_select_topk, bit-identical on the same scores;
 *     returns KAP_ERR_CAPACITY if some request's a + r + k exceeds capacity.
 */
KAP_API kap_status kap_host_proxy_query(const uint16_t* hidden, const uint16_t* w_q, int32_t B,
                                        int32_t d_model, int32_t n_out, float* q_out,
                                        int32_t threads);
KAP_API kap_status kap_host_score_blocks(const float* q, const int32_t* positions,
                                         float rope_theta, const uint16_t* summary,
                                         int32_t num_pages, const int32_t* block_table,
                                         int32_t max_pages, const int32_t* seq_lens, int32_t B,
                                         int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size,
                                         float* scores, int32_t threads);
KAP_API kap_status kap_host_select_topk(const float* scores, int32_t B, int32_t Hkv,
                                        int32_t max_pages, const int32_t* seq_lens,
                                        int32_t page_size, int32_t per_head,
                                        const int32_t* anchor, const int32_t* recent,
                                        const int32_t* k_mid, int32_t capacity,
                                        int32_t* sel_pages, int32_t* sel_count, int32_t threads);

/*
 * Diagnostic, not part of the path: reads `bytes` (a multiple of 16) of device
 * memory with 16-byte loads from a 2048 x 256 grid-stride kernel, the load
 * shape of the attention kernels.  Timing it gives the sustained read
 * bandwidth those kernels are compared against.  sink: device, one uint32
 * (written only with probability ~2^-32).
 */
KAP_API kap_status kap_diag_stream_read(const void* buf, size_t bytes, uint32_t* sink,
                                        kap_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* KAP_H */
