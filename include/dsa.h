/*
 * dsa.h -- C ABI of the MI355X (gfx950) query-aware block-sparse paged
 * decode attention library, libdsa.so.
 *
 * One decode step of dynamic sparse attention over a paged KV cache:
 *   page_meta_build        per-page key min/max metadata
 *   kv_append              one new token per sequence into its page, with
 *                          that page's min/max kept current
 *   page_score             page criticality against that metadata, with a
 *                          group-mean query and a logical->physical max
 *   page_select_topk       fixed top-k pages (ties to the lower index)
 *   page_select_progressive  PSA's threshold-driven progressive selection,
 *                          fused with the attention it drives
 *   sparse_decode_attn     softmax attention over the selected pages only,
 *                          emitting (O, l, m)
 *   attn_repair            folds the pages of A that the speculative set P
 *                          missed into a speculative (O, l, m)
 *   ema_predict_update     PRR's EMA page-score predictor
 *   prr_calibrate          PRR's search of the EMA hyper-parameters over a
 *                          score trace
 *   signal_host            zero-copy notification of the host (PSA)
 *   block_sparse_prefill   LServe's prefill attention with tile skipping
 *
 * Sources, cited by page title and section:
 *   [PSA]    "PSA: Progressive Sparse Attention -- Algorithm and System
 *            Co-design for Efficient Attention in LLM Serving"
 *   [LServe] "LServe: Efficient Long-sequence LLM Serving with Unified
 *            Sparse Attention"
 *   [PRR]    "Predict, Reuse, and Repair: Accelerating Dynamic Sparse
 *            Attention for Long-Context LLM Decoding"
 *
 * Common conventions
 * ------------------
 * - Every data pointer is DEVICE memory owned by the caller unless marked
 *   HOST.  The library never allocates, frees, copies to the host or
 *   synchronises; each call only enqueues kernels on `stream` (a
 *   hipStream_t; NULL = the default stream) and returns.  Buffers must stay
 *   alive until that stream work completes.  Scratch memory comes from the
 *   caller's workspace `ws` of `ws_bytes` bytes, sized by
 *   dsa_workspace_bytes(); its content needs no initialisation, and calls
 *   that share one workspace must not overlap in time.
 * - Return value: DSA_OK (0) or a negative DSA_ERR_* code.  All arguments
 *   are validated on the host before anything is enqueued, so an error means
 *   no work was queued.  Errors inside a kernel surface at the caller's next
 *   synchronisation.  Calls on distinct streams with distinct outputs may
 *   run concurrently; the library keeps no state between calls.
 * - KV pool (struct dsa_kv): one block pool cut into equal slots shared by
 *   all sequences ([PSA] section 3.4; [LServe] section 3.2.1):
 *     k, v        [num_slots][n_kv_heads][page_size][head_dim], dtype
 *     page_table  int32 [batch][max_pages]: slot of page j of a sequence,
 *                 i.e. of its tokens [j*page_size, (j+1)*page_size)
 *     seq_lens    int32 [batch]: tokens of each sequence
 *   Page j of sequence b is valid when j*page_size < seq_lens[b] and
 *   j < max_pages (longer sequences are clamped to max_pages pages).  Rows of
 *   a valid page past seq_lens[b] are never read.  A page-table entry outside
 *   [0, num_slots) makes that page hold no tokens; entries of invalid pages
 *   are never read.
 * - Supported shapes: dtype DSA_BF16 or DSA_F32; head_dim 64 or 128;
 *   page_size 16, 32 or 64; logical_page a multiple of 16 that divides
 *   page_size; n_q_heads = G * n_kv_heads with G in {1, 2, 4, 8, 16};
 *   q head h belongs to KV head h / G.  k, v, q and meta 16-byte aligned.
 * - Selected page ids are page indices j of the sequence (page-table
 *   columns), never slots.
 * - Logits are scale * q.k with the caller's scale (> 0; normally
 *   1/sqrt(head_dim) rounded to float).  Attention outputs, per q head:
 *   m = max logit, l = sum exp(logit - m), O = sum exp(logit - m) v / l; an
 *   empty page set gives O = 0, l = 0, m = -inf.  Accumulation is fp32.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DSA_OK = 0,
  DSA_ERR_NULL = -1,        /* a required pointer is NULL                    */
  DSA_ERR_SHAPE = -2,       /* a size or count is out of range / inconsistent */
  DSA_ERR_DTYPE = -3,       /* unknown dtype                                  */
  DSA_ERR_UNSUPPORTED = -4, /* valid but not built (head_dim, group, ...)     */
  DSA_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than required        */
  DSA_ERR_ALIGN = -6,       /* pointer not 16-byte aligned                    */
  DSA_ERR_LAUNCH = -7,      /* the HIP runtime rejected a launch              */
  DSA_ERR_SCRATCH = -8      /* the call needs more than the fixed scratch of
                               dsa_sparse_decode_attn_noalloc                 */
};

enum { DSA_F32 = 0, DSA_BF16 = 1 };

typedef struct dsa_kv {
  const void *k;               /* device [num_slots][n_kv_heads][page_size][head_dim] */
  const void *v;               /* device, same layout as k                     */
  int32_t dtype;               /* DSA_F32 | DSA_BF16 (also the dtype of q and meta) */
  int32_t num_slots;
  int32_t n_kv_heads;
  int32_t page_size;
  int32_t head_dim;
  int32_t batch;
  int32_t max_pages;
  const int32_t *page_table;   /* device int32 [batch][max_pages]              */
  const int32_t *seq_lens;     /* device int32 [batch]                         */
} dsa_kv;

/* Streaming heads ([LServe] section 4.1): a KV head flagged here attends
 * only to its sink tokens [0, sink) and local tokens [L - local, L). */
typedef struct dsa_stream_cfg {
  const uint8_t *kv_head_streaming; /* HOST [n_kv_heads], nonzero = streaming; at most 64 heads */
  int32_t sink;
  int32_t local;
} dsa_stream_cfg;

/* Operation ids for dsa_workspace_bytes(). */
enum { DSA_OP_SPARSE_DECODE_ATTN = 1, DSA_OP_ATTN_REPAIR = 2, DSA_OP_PRR_DECODE_STEP = 3 };

/* Human-readable name of a status code (static storage). */
const char *dsa_status_str(int status);

/* Library version, as major*10000 + minor*100 + patch. */
int dsa_version(void);

/*
 * dsa_page_meta_build -- per-page key metadata ([LServe] section 4.2 and
 * Figure 7: kmin/kmax vectors attached to each physical page, built during
 * prefill and earlier decode steps; [PSA] section 3.1: block metadata kept
 * in GPU memory).
 *
 * For pages j in [first_page, first_page + n_pages) of every sequence
 * (n_pages < 0: all valid pages), for every KV head and every logical
 * sub-page s (g = page_size / logical_page of them), writes the per-channel
 * minimum and maximum of the keys of the sub-page's valid tokens:
 *   meta[slot][h][s][0][c] = min_t k[t][c],  meta[slot][h][s][1][c] = max_t k[t][c]
 * meta: device [num_slots][n_kv_heads][g][2][head_dim] in kv->dtype (exact:
 * the min/max of stored values).  A sub-page with no valid token is written
 * as zeros (page_score never reads it).  Slots of pages outside the range
 * are left untouched.
 */
int dsa_page_meta_build(const dsa_kv *kv, int32_t logical_page, void *meta,
                        int32_t first_page, int32_t n_pages, void *stream);

/*
 * dsa_kv_append -- decode-time append of one token per sequence ([PSA]
 * section 3.1: the KV cache manager writes each newly generated token's K/V
 * into its block on the GPU and the block metadata stays in GPU memory;
 * [LServe] section 4.2 and Figure 7: a physical page's kmin/kmax vectors
 * come from the prefill and the earlier decoding steps).
 *
 * For every sequence b, with p = kv->seq_lens[b], page j = p / page_size,
 * row o = p % page_size and slot = page_table[b][j]:
 *   k[slot][h][o][:] = k_new[b][h][:] and v[slot][h][o][:] = v_new[b][h][:]
 *   for every KV head h, and in the logical sub-page s = o / logical_page:
 *     o % logical_page == 0:  meta[slot][h][s][0] = meta[slot][h][s][1] = k_new[b][h]
 *     otherwise:              meta[slot][h][s][0] = min(meta[slot][h][s][0], k_new[b][h]),
 *                             meta[slot][h][s][1] = max(meta[slot][h][s][1], k_new[b][h])
 *   (per channel); new_seq_lens[b] = p + 1; status[b] = 1.
 * The metadata before the call must describe the sub-page's earlier tokens
 * (as dsa_page_meta_build or earlier appends wrote it); afterwards it equals
 * dsa_page_meta_build of the grown page exactly.  A sequence whose page j is
 * not below max_pages, or whose page-table entry lies outside
 * [0, num_slots), is skipped: nothing is written for it, new_seq_lens[b] = p
 * and status[b] = 0.  Giving a new page its slot is the caller's job.
 * k_new, v_new: device [batch][n_kv_heads][head_dim] in kv->dtype, 16-byte
 * aligned, not overlapping the pool.  meta: layout of dsa_page_meta_build
 * with the same logical_page.  new_seq_lens: device int32 [batch]; it may be
 * kv->seq_lens itself (each length is read before it is rewritten).
 * status: device int32 [batch] or NULL.  This call writes through kv->k and
 * kv->v.  NaN keys are not supported.
 */
int dsa_kv_append(const dsa_kv *kv, int32_t logical_page, const void *k_new, const void *v_new,
                  void *meta, int32_t *new_seq_lens, int32_t *status, void *stream);

/*
 * dsa_page_score -- page criticality ([LServe] section 4.2, importance of a
 * logical page and max-reduction to the physical page; [PSA] section 3.2,
 * the CS step; [PRR] section 5, the Quest GQA extension's representative
 * query).
 *
 * Per (sequence b, KV head h): qbar = mean of the G q heads of h (fp32);
 * for each valid logical sub-page s of page j:
 *   S_s = sum_c max(qbar[c] * kmax_s[c], qbar[c] * kmin_s[c])
 * and scores[b][h][j] = max over the page's valid sub-pages of S_s.
 * Invalid pages and every page of a streaming head score -inf.
 * q: device [batch][n_q_heads][head_dim] in kv->dtype.  meta as written by
 * dsa_page_meta_build with the same logical_page.  stream_cfg may be NULL.
 * scores: device float [batch][n_kv_heads][max_pages].
 */
int dsa_page_score(const void *q, int32_t n_q_heads, const dsa_kv *kv, const void *meta,
                   int32_t logical_page, const dsa_stream_cfg *stream_cfg, float *scores,
                   void *stream);

/*
 * dsa_page_score_ema -- dsa_page_score with PRR's EMA predictor update
 * ([PRR] section 3.1) applied to the new scores in the same launch.
 *
 * Equivalent to dsa_page_score(...) followed by
 * dsa_ema_predict_update(scores, level, trend, pred,
 *                        batch * n_kv_heads * max_pages, alpha, beta, gamma, init)
 * (bit for bit: the same float operations in the same order), without the
 * second launch.  level, trend, pred: device float [batch][n_kv_heads][max_pages],
 * distinct from each other and from scores (DSA_ERR_SHAPE), none NULL
 * (DSA_ERR_NULL).  Other arguments and errors as dsa_page_score.
 */
int dsa_page_score_ema(const void *q, int32_t n_q_heads, const dsa_kv *kv, const void *meta,
                       int32_t logical_page, const dsa_stream_cfg *stream_cfg, float *scores,
                       float *level, float *trend, float *pred, float alpha, float beta,
                       float gamma, int32_t init, void *stream);

/*
 * dsa_page_select_topk -- fixed top-k page selection ([PSA] section 2.2;
 * [PRR] section 2, the selection stage of a DSA step).
 *
 * Per (b, h) row of scores[batch][n_kv_heads][max_pages] (float, device),
 * considers the valid pages j < ceil(seq_lens[b] / page_size) (clamped to
 * max_pages) and keeps the min(k, valid) highest scores; equal scores are
 * kept in favour of the lower page index; -0.0 equals +0.0.  Writes the kept
 * ids in ascending order to ids[b][h][0..count) and -1 to the rest of
 * ids[b][h][0..k); counts[b][h] = count.  For a streaming head (stream_cfg
 * non-NULL and flagged) the ids are instead the pages holding a sink token
 * or a local token, ascending; the call fails with DSA_ERR_SHAPE if that
 * list could exceed k.  NaN scores are not supported.
 * ids: device int32 [batch][n_kv_heads][k]; counts: device int32 [batch][n_kv_heads].
 * Requires 1 <= k and max_pages <= 65536.
 */
int dsa_page_select_topk(const float *scores, int32_t batch, int32_t n_kv_heads,
                         int32_t max_pages, const int32_t *seq_lens, int32_t page_size,
                         int32_t k, const dsa_stream_cfg *stream_cfg, int32_t *ids,
                         int32_t *counts, void *stream);

/*
 * dsa_page_select_progressive -- PSA progressive sparse attention ([PSA]
 * section 3.2, the PSAttention algorithm; section 3.3, the on-GPU check of
 * the accumulated weight; section 5, on-chip aggregation of block weights).
 *
 * Per (b, KV head h): ranks the valid pages by descending score (ties: lower
 * index), then visits them in rank order, computing each page's attention
 * for the G q heads and its block weight AS = sum over the page's tokens and
 * the G heads of exp(logit).  After each page: AS_acc += AS,
 * AS_min = min(AS_min, AS), and the walk stops when
 *   stop_mode 0:  AS_acc / (AS_acc + AS_min) >= threshold            (printed rule)
 *   stop_mode 1:  AS_acc / (AS_acc + N_left * AS_min) >= threshold   (N_left = pages not visited)
 * threshold >= 1 never stops early; if the test never passes, every valid
 * page is visited.  The test is evaluated on the device in the log domain
 * (no host round trip).  Outputs: ids[b][h][0..n) the visited pages in rank
 * order, -1 after; counts[b][h] = n; O/l/m for the G q heads = attention
 * over the visited pages.
 * scores as from dsa_page_score; ids: device int32 [batch][n_kv_heads][max_pages];
 * O: device float [batch][n_q_heads][head_dim]; l, m: device float [batch][n_q_heads].
 * Requires max_pages <= 65536 (else DSA_ERR_UNSUPPORTED).
 * stream_cfg (nullable): a streaming head ([LServe] section 4.1) is not
 * ranked: it visits the pages holding a sink or a local token, ascending,
 * attends only to those tokens, and never stops early (ids = that list,
 * counts = its length).
 */
int dsa_page_select_progressive(const void *q, int32_t n_q_heads, const dsa_kv *kv,
                                const float *scores, float threshold, int32_t stop_mode,
                                const dsa_stream_cfg *stream_cfg, float scale, int32_t *ids,
                                int32_t *counts, float *O, float *l, float *m, void *stream);

/*
 * dsa_psa_decode -- dsa_page_score followed by dsa_page_select_progressive
 * ([LServe] section 4.2 criticality, [PSA] section 3.2 progressive
 * selection) in one call, for meta built with logical_page = page_size; a
 * streaming head of stream_cfg (nullable) gets -inf scores and its sink and
 * local pages, as in the two calls.  When there are at least as many (b, KV head) rows as the
 * GPU has CUs and max_pages <= 8192, one workgroup per row computes its
 * row's scores into LDS and goes straight on to the selection and walk (one
 * launch); otherwise the two calls run in sequence.  Either way the results
 * are those of the two calls: scores (device float [batch][n_kv_heads]
 * [max_pages], written), ids, counts, O, l, m as dsa_page_select_progressive.
 * Requires max_pages <= 65536 and 1, 2 or 4 q heads per KV head.
 */
int dsa_psa_decode(const void *q, int32_t n_q_heads, const dsa_kv *kv, const void *meta,
                   float threshold, int32_t stop_mode, const dsa_stream_cfg *stream_cfg, float scale,
                   float *scores, int32_t *ids, int32_t *counts, float *O, float *l, float *m,
                   void *stream);

/*
 * dsa_sparse_decode_attn -- attention over the selected pages only ([LServe]
 * section 3.3: the decode kernel loops only over the needed pages through a
 * two-level index, step -> page -> cache slot; [PRR] section 3.3: the
 * speculative kernel also writes the softmax denominator l and the running
 * max m per head).
 *
 * Per (b, KV head h): the pages ids[b][h][0..counts[b][h]) (each a valid
 * page index; duplicates are attended twice), through page_table to slots.
 * For a streaming head only sink and local tokens of those pages count.
 * Writes O[b][hq][:], l[b][hq], m[b][hq] for the G q heads hq of h.
 * ids: device int32 [batch][n_kv_heads][ids_stride], counts <= ids_stride.
 * ws: device scratch of dsa_workspace_bytes(DSA_OP_SPARSE_DECODE_ATTN, ...).
 */
int dsa_sparse_decode_attn(const void *q, int32_t n_q_heads, const dsa_kv *kv,
                           const int32_t *ids, const int32_t *counts, int32_t ids_stride,
                           const dsa_stream_cfg *stream_cfg, float scale, float *O, float *l,
                           float *m, void *ws, size_t ws_bytes, void *stream);

/*
 * dsa_sparse_decode_attn_noalloc -- dsa_sparse_decode_attn for callers that
 * cannot allocate: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, semantics and results
 * as dsa_sparse_decode_attn (the same kernels run), minus the workspace:
 * the split partials go to a fixed device array inside the library, of
 * DSA_NOALLOC_SCRATCH_BYTES bytes, that each GPU the library runs on holds
 * until the process ends.  The call allocates nothing, ever.
 *
 * Limit: a call that needs more scratch than that, i.e.
 * dsa_workspace_bytes(DSA_OP_SPARSE_DECODE_ATTN, kv, n_q_heads, ids_stride)
 * > DSA_NOALLOC_SCRATCH_BYTES, returns DSA_ERR_SCRATCH and enqueues nothing.
 * Every call on one GPU shares that GPU's array (its content carries over
 * from the last call and is never read before it is written), so calls
 * that overlap in time on one GPU -- on different streams, or from several
 * host threads -- race and must be avoided; calls on one stream are
 * ordered and safe.  The first call on a device looks up the array's
 * address on that device (the stream's device, or the current device for
 * the NULL stream).
 */
#define DSA_NOALLOC_SCRATCH_BYTES (8u << 20)
int dsa_sparse_decode_attn_noalloc(const void *q, int32_t n_q_heads, const dsa_kv *kv,
                                   const int32_t *ids, const int32_t *counts, int32_t ids_stride,
                                   const dsa_stream_cfg *stream_cfg, float scale, float *O, float *l,
                                   float *m, void *stream);

/*
 * dsa_sparse_decode_attn_topk -- dsa_page_select_topk followed by
 * dsa_sparse_decode_attn over the pages it selects, in one call ([PSA]
 * section 2.2 / [PRR] section 2: the selection stage feeding the sparse
 * attention of a dynamic sparse attention step).
 *
 * Results are those of the two calls with ids_stride = k: ids[b][h][0..k)
 * (ascending, -1 padded) and counts[b][h] are written, and O, l, m are
 * attention over those pages.  For groups of at most 4 q heads and
 * max_pages <= 4096 every attention workgroup ranks its row of scores itself
 * (no separate selection launch); otherwise the two launches run in order.
 * Arguments as for the two calls; ws: device scratch of
 * dsa_workspace_bytes(DSA_OP_SPARSE_DECODE_ATTN, kv, n_q_heads, k).
 * Errors: those of either call.
 */
int dsa_sparse_decode_attn_topk(const void *q, int32_t n_q_heads, const dsa_kv *kv,
                                const float *scores, int32_t k, const dsa_stream_cfg *stream_cfg,
                                float scale, int32_t *ids, int32_t *counts, float *O, float *l,
                                float *m, void *ws, size_t ws_bytes, void *stream);

/*
 * dsa_attn_repair -- PRR incremental repair ([PRR] section 3.3, the repair
 * kernel's online-softmax recurrence; section 3.4, the missing set M = A\P).
 *
 * On entry O, l, m hold a speculative result over page set P (e.g. from
 * dsa_sparse_decode_attn over p_ids).  Per (b, KV head h) the call forms
 * M = the entries of a_ids[b][h][0..a_counts) not among
 * p_ids[b][h][0..p_counts), in a_ids order, attends over M only, and folds
 * that into (O, l, m) in place:
 *   m' = max(m, m~), l' = e^(m-m') l + e^(m~-m') l~,
 *   O' = (e^(m-m') l O + e^(m~-m') l~ O~) / l'
 * so the result is attention over P u A.  KV traffic scales with |M|; each
 * workgroup of the split over A also reads p_ids once into an LDS bitmap of
 * max_pages bits (DSA_ERR_UNSUPPORTED if that bitmap does not fit in LDS).
 * p_ids and p_counts may both be NULL: then a_ids already lists M (as
 * dsa_prr_select writes it) and is attended as it is.
 * a_ids, p_ids: device int32 [batch][n_kv_heads][ids_stride] with page ids
 * < max_pages.  stream_cfg (nullable): for a streaming head only the sink
 * and local tokens of M's pages count, as in dsa_sparse_decode_attn.
 * ws: device scratch of dsa_workspace_bytes(DSA_OP_ATTN_REPAIR, ...).
 */
int dsa_attn_repair(const void *q, int32_t n_q_heads, const dsa_kv *kv, const int32_t *a_ids,
                    const int32_t *a_counts, const int32_t *p_ids, const int32_t *p_counts,
                    int32_t ids_stride, const dsa_stream_cfg *stream_cfg, float scale, float *O,
                    float *l, float *m, void *ws, size_t ws_bytes, void *stream);

/*
 * dsa_prr_decode_step -- one speculative PRR decode step on one stream
 * ([PRR] sections 2-3: the speculative attention over the predicted set
 * runs while the page scores are computed and the exact set selected; the
 * repair then folds in the pages the prediction missed; section 3.1: the
 * EMA update and the next prediction).
 *
 * Results are those of, in order:
 *   dsa_page_score_ema(q, n_q_heads, kv, meta, logical_page, NULL, scores,
 *                      level, trend, pred, alpha, beta, gamma, 0)
 *   dsa_sparse_decode_attn(q, n_q_heads, kv, p_cur_ids, p_cur_counts, k, NULL,
 *                          scale, O, l, m)
 *   dsa_prr_select(scores, ..., k, a_ids, a_counts, NULL, NULL, pred, alpha,
 *                  beta, gamma, 0, k, p_ids, p_counts, p_cur_ids, p_cur_counts,
 *                  m_ids, m_counts, NULL, 0)
 *   dsa_attn_repair(q, n_q_heads, kv, m_ids, m_counts, NULL, NULL, k, NULL,
 *                   scale, O, l, m)
 * i.e. IS^t into scores, level/trend/pred updated with it, O/l/m = attention
 * over P^t union A^t, a_ids = A^t, m_ids = M^t = A^t \ P^t and p_ids =
 * P^{t+1} (|A| = |P| = k; every id row has stride k, ascending, -1 padded).
 * Independent parts share launches instead of streams (the scores with the
 * speculative partials, the speculative combine with the repair's
 * partials): 4 launches on the given stream, nothing for a caller to join.
 * P^t = p_cur_ids/p_cur_counts must not be p_ids/p_counts; level, trend,
 * pred and scores distinct (DSA_ERR_SHAPE); every pointer non-NULL
 * (DSA_ERR_NULL); meta 16-byte aligned.  Requires bf16 KV, logical_page =
 * page_size, no streaming heads and max_pages <= 65536, else
 * DSA_ERR_UNSUPPORTED (use the separate calls); any group size the
 * attention calls take (the matrix-core partials for 8 or 16 q heads per
 * KV head, the VALU partials below).
 * ws: device scratch of dsa_workspace_bytes(DSA_OP_PRR_DECODE_STEP, kv,
 * n_q_heads, k) bytes, 16-byte aligned.
 */
int dsa_prr_decode_step(const void *q, int32_t n_q_heads, const dsa_kv *kv, const void *meta,
                        int32_t logical_page, float *scores, float *level, float *trend,
                        float *pred, float alpha, float beta, float gamma, int32_t k,
                        const int32_t *p_cur_ids, const int32_t *p_cur_counts, int32_t *a_ids,
                        int32_t *a_counts, int32_t *m_ids, int32_t *m_counts, int32_t *p_ids,
                        int32_t *p_counts, float scale, float *O, float *l, float *m, void *ws,
                        size_t ws_bytes, void *stream);

/*
 * dsa_ema_predict_update -- PRR EMA predictor ([PRR] section 3.1).
 *
 * Elementwise over n blocks (float, device):
 *   is_true == NULL:  pred = level + gamma * trend                (predict only)
 *   init != 0:        level = IS, trend = 0, pred = IS            (first observation)
 *   otherwise:        trend' = beta*(IS - level) + (1-beta)*trend,
 *                     level' = alpha*IS + (1-alpha)*level   (both read the old level),
 *                     pred = level' + gamma * trend'        (the next step's prediction)
 * level and trend are updated in place; pred may not alias them.  Every
 * product and sum is rounded to fp32 on its own, in the order written (no
 * fused multiply-add), so a float32 reference reproduces it bit for bit.
 */
int dsa_ema_predict_update(const float *is_true, float *level, float *trend, float *pred,
                           int64_t n, float alpha, float beta, float gamma, int32_t init,
                           void *stream);

/*
 * dsa_prr_select -- PRR's selection stage ([PRR] section 2:
 * the exact selection A^t; section 3.1: the EMA update with IS^t and the
 * next speculative set P^{t+1} = top-k_spec of the prediction).
 *
 * Equivalent to, in order:
 *   dsa_page_select_topk(scores, ..., k, NULL, a_ids, a_counts)
 *   dsa_ema_predict_update(scores, level, trend, pred, batch*n_kv_heads*max_pages,
 *                          alpha, beta, gamma, init)
 *   dsa_page_select_topk(pred, ..., k_spec, NULL, p_ids, p_counts)
 * as two launches (see ws below for how they are split).  With m_ids non-NULL
 * the call also writes the repair's missing set ([PRR] section 3.4)
 * M^t = A^t \ P^t, where P^t = p_cur_ids[b][h][0..p_cur_counts) (row
 * stride k_spec) is this step's speculative set: m_ids int32
 * [batch][n_kv_heads][k] ascending, -1 padded, m_counts[b][h] = |M|.
 * p_cur_ids/p_cur_counts must not be p_ids/p_counts; all four M pointers may
 * be NULL.
 * scores: IS^t, device float [batch][n_kv_heads][max_pages]; level, trend,
 * pred: device float arrays of the same shape, distinct.  level and trend
 * may both be NULL when pred already holds the updated prediction (after
 * dsa_page_score_ema): the EMA step is then skipped; one of them NULL is
 * DSA_ERR_NULL.  a_ids: int32
 * [batch][n_kv_heads][k]; p_ids: int32 [batch][n_kv_heads][k_spec]; ids
 * ascending, -1 padded.  No streaming heads.  max_pages <= 65536.
 * ws: device scratch of dsa_prr_select_workspace_bytes(batch, n_kv_heads,
 * max_pages) bytes (16-byte aligned), or NULL.  Rows longer than 4096 pages
 * given a workspace are split into chunks of 2048 pages, one workgroup each,
 * in two launches (chunk histograms, then the cut and the writes; the EMA
 * update happens inside them); otherwise, and always without a workspace,
 * one workgroup takes a whole row after the elementwise EMA launch.  The
 * results are the same either way.  DSA_ERR_WORKSPACE if ws is given but
 * smaller than required.
 */
int dsa_prr_select(const float *scores, int32_t batch, int32_t n_kv_heads, int32_t max_pages,
                   const int32_t *seq_lens, int32_t page_size, int32_t k, int32_t *a_ids,
                   int32_t *a_counts, float *level, float *trend, float *pred, float alpha,
                   float beta, float gamma, int32_t init, int32_t k_spec, int32_t *p_ids,
                   int32_t *p_counts, const int32_t *p_cur_ids, const int32_t *p_cur_counts,
                   int32_t *m_ids, int32_t *m_counts, void *ws, size_t ws_bytes, void *stream);

/*
 * dsa_prr_select_workspace_bytes -- scratch bytes dsa_prr_select uses for
 * rows of max_pages pages (0 when its rows are short enough for one
 * workgroup each, or the shape is invalid).
 */
size_t dsa_prr_select_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t max_pages);

/*
 * dsa_prr_calibrate -- PRR online predictor calibration ([PRR] section 3.2:
 * the EMA hyper-parameters are chosen per prompt by the score-weighted hit
 * rate H(theta; IS) over a prefill score trace, maximised over the printed
 * grid alpha in {0.2, 0.4, 0.6, 0.8}, beta in {0.1, 0.2, 0.3, 0.4, 0.5},
 * gamma in {0, 0.25, 0.5, 0.75}: 80 candidates).
 *
 * trace: device float [steps][units][n], the scores IS_phi of `steps`
 * consecutive steps of each unit (for instance one (sequence, KV head) row
 * of dsa_page_score per step); the pages j < n_valid[u] of unit u are valid
 * (n_valid: device int32 [units], clamped to [0, n]).  Candidate
 * c = (ia*5 + ib)*4 + ig has alpha = {0.2, 0.4, 0.6, 0.8}[ia],
 * beta = {0.1, ..., 0.5}[ib], gamma = 0.25*ig (as float).  Per unit and
 * candidate the EMA starts at level = IS_0, trend = 0, and every step
 * phi = 1 .. steps-1 is
 *   predicted:  pred = level + gamma*trend (rounded as dsa_ema_predict_update),
 *   scored:     h_phi = sum_{b in P & A} IS_phi,b / sum_{b in A} IS_phi,b with
 *               A = top-k(IS_phi), P = top-m(pred) over the valid pages
 *               (ties to the lower index; h_phi = 1 when A is empty or
 *               weighs 0),
 *   absorbed:   trend and level updated with IS_phi as in dsa_ema_predict_update.
 * H[u][c] = mean of h_phi over the steps - 1 predicted steps (device float
 * [units][80]); best[u] = the c of the largest H[u][c], the lowest c among
 * equal values (device int32 [units]; may be NULL).
 * ws: device scratch of dsa_prr_calibrate_workspace_bytes(steps, units, n)
 * bytes.  Requires steps >= 2, 1 <= n <= 65536, k >= 0, m >= 0.  NaN scores
 * are not supported.
 */
int dsa_prr_calibrate(const float *trace, int32_t steps, int32_t units, int32_t n,
                      const int32_t *n_valid, int32_t k, int32_t m, float *H, int32_t *best,
                      void *ws, size_t ws_bytes, void *stream);

/*
 * dsa_block_sparse_prefill -- block-sparse prefill attention of one
 * sequence ([LServe] section 2.3: every T_Q x T_K tile is skipped or
 * computed like causal attention; section 3.3 and Figure 5: dense and
 * streaming heads in one kernel that visits only the needed tiles; section
 * 4.1: the Lambda mask of a streaming head).
 *
 * q: device bf16 [L][n_q_heads][head_dim]; k, v: device bf16
 * [L][n_kv_heads][head_dim] (the prompt's projections, token-major); q head
 * hq reads KV head hq / G.  Query i attends to the keys j <= i; for a KV
 * head flagged streaming in stream_cfg (may be NULL) only to j < sink or
 * j > i - local.  Outputs per (token, q head), as in the decode calls:
 * O device float [L][n_q_heads][head_dim] (normalised), l and m device float
 * [L][n_q_heads] (m in scaled-logit units; an empty key set gives O = 0,
 * l = 0, m = -inf).  Tiles of 64 queries x 64 keys without an attended pair
 * are not visited.  Requires head_dim 64 or 128 and a finite scale > 0;
 * q, k, v and O 16-byte aligned.
 */
int dsa_block_sparse_prefill(const void *q, const void *k, const void *v, int32_t L, int32_t n_q_heads,
                             int32_t n_kv_heads, int32_t head_dim, const dsa_stream_cfg *stream_cfg,
                             float scale, float *O, float *l, float *m, void *stream);

/*
 * dsa_signal_host -- zero-copy notification of the host ([PSA] section 3.3:
 * after the threshold test passes, the GPU writes a signal variable into
 * pinned host memory, so the CPU learns of it asynchronously).
 *
 * Enqueued on `stream` after the producing calls (for instance after
 * dsa_page_select_progressive with src = its counts): copies src[0..n)
 * (device int32) to host_dst[0..n) and then writes seq to *host_flag, both
 * with system-scope stores, the flag last with release ordering.  A host
 * thread that reads *host_flag == seq then reads the n values as written,
 * with no stream or device synchronisation.  host_dst and host_flag must be
 * pinned host memory the device can address (hipHostMalloc, or a pinned
 * torch tensor); host_dst may be NULL when n == 0.
 */
int dsa_signal_host(const int32_t *src, int32_t n, int32_t *host_dst, int32_t *host_flag, int32_t seq,
                    void *stream);

/* Scratch bytes dsa_prr_calibrate needs (0 for invalid sizes). */
size_t dsa_prr_calibrate_workspace_bytes(int32_t steps, int32_t units, int32_t n);

/*
 * dsa_workspace_bytes -- scratch needed by dsa_sparse_decode_attn (op
 * DSA_OP_SPARSE_DECODE_ATTN), dsa_attn_repair (DSA_OP_ATTN_REPAIR) or
 * dsa_prr_decode_step (DSA_OP_PRR_DECODE_STEP, ids_stride = k) for this
 * pool, n_q_heads and ids_stride.  Returns 0 for invalid arguments.
 */
size_t dsa_workspace_bytes(int32_t op, const dsa_kv *kv, int32_t n_q_heads, int32_t ids_stride);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
