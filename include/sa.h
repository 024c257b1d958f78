/*
 * sa.h - C ABI of the query-aware sparse decode-attention library (gfx950).
 *
 * One decode step of attention over a paged KV cache reads only the pages
 * that matter for the current query:
 *   1. score every page (Quest per-dimension min/max upper bound) or every
 *      64-token block (SALS low-rank int4 index key + block log-sum-exp);
 *   2. keep an exact top-K of the scored units, ties to the lower index, with
 *      forced leading (sink) and trailing (recent / tail) units;
 *   3. flash-decoding attention over the kept pages only: online softmax,
 *      fp32 accumulation, split-K partials and a rescaling merge; K/V may be
 *      fp32, bf16, or int8 codes with one fp16 scale per (token, kv-head).
 *
 * Pages these calls follow:
 *  [Quest]  "Quest 完全拆解：查询感知的页级稀疏注意力" (pinghaoyang.com.cn):
 *           16-token pages addressed through a page table; per-page min/max
 *           metadata; the bound sum_i max(q_i m_i, q_i M_i); the
 *           criticality-estimation, top-K filtering and approximate-attention
 *           kernels (only page numbers pass between the last two); GQA
 *           group-shared selection.
 *  [SALS]   "SALS长序列推理优化" (CANN learning hub): QSI (group-mean index
 *           query, int4 low-rank index key, block LSE, exact top-k, fixed tail
 *           blocks appended) and SFAA (attention over the QSI indices on int8
 *           K/V: QK, online softmax, P@V, rescale; split rows reduced).
 *  [RK]     "Day 10·2 sparse top-k 块选择" (xxmr.cn): lower index wins ties,
 *           the last block is always kept, no padding below k, bit-identical
 *           selection for identical inputs.
 *  [SeqO1]  "SequenceO1" explainer (mhpn.cn), FlashSA section: selection and
 *           sparse attention as two kernels joined only by integer indices.
 *
 * Conventions for every entry point:
 *  - Pointers named in the structs and arguments are DEVICE pointers on the
 *    current HIP device unless stated otherwise; the caller owns them.  Device
 *    arrays must be 16-byte aligned; workspaces 256-byte aligned.
 *  - 'stream' is a hipStream_t passed as void* (NULL = the null stream).  Work
 *    is enqueued on it and nothing synchronises; a return of SA_OK means
 *    "enqueued".  Device faults surface at the caller's next synchronisation.
 *  - All argument checks are made on the host before anything is enqueued; on
 *    any error nothing is launched.  No call allocates or frees device memory.
 *  - Errors are returned as negative sa_status codes; nothing aborts or
 *    throws across this interface.
 *  - Thread safety: calls on distinct streams (or with distinct buffers) are
 *    independent.  The only library-wide state is a per-device cache of
 *    fixed device and kernel properties (compute-unit count, the fused step
 *    kernel's resident workgroups), filled on first use with atomic stores;
 *    it never changes what a call computes.
 *  - Sequence semantics: seq_lens[b] >= 1 counts the current token, whose K/V
 *    is already in the cache; attention covers positions [0, seq_lens[b]).
 *    Sequence b has n_b = ceil(seq_lens[b] / 16) logical pages; page_table
 *    entries at or past n_b are never read.  A physical page belongs to one
 *    (b, p).  Device-side, seq_lens values are clamped to
 *    [0, max_pages * 16] and physical page ids outside [0, num_pages) are
 *    skipped (their tokens are treated as masked); neither is reported.
 *  - Query heads h*G .. h*G+G-1 share kv-head h (G = num_q_heads / num_kv_heads)
 *    and share one selection ([Quest] GQA section; [SALS] SFAA indices).
 */
#ifndef SA_H
#define SA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sa_status {
  SA_OK = 0,
  SA_ERR_INVALID_ARG = -1,        /* null pointer, bad shape or inconsistent sizes */
  SA_ERR_UNSUPPORTED = -2,        /* valid request this build does not implement */
  SA_ERR_WORKSPACE_TOO_SMALL = -3,
  SA_ERR_HIP = -4                 /* a HIP runtime call failed (launch error) */
} sa_status;

enum { SA_F32 = 0, SA_BF16 = 1, SA_I8 = 2 };      /* element types */
enum { SA_MODE_QUEST = 0, SA_MODE_SALS = 1, SA_MODE_PROBE = 2 };  /* scoring modes */

/* Paged KV cache of one layer. */
typedef struct sa_kv_cache {
  const void *k;            /* [num_pages, page_size, num_kv_heads, head_dim] of dtype */
  const void *v;            /* same layout as k */
  const uint16_t *k_scale;  /* SA_I8 only: fp16 bits [num_pages, page_size, num_kv_heads]; else NULL */
  const uint16_t *v_scale;  /* SA_I8 only: as k_scale */
  int32_t dtype;            /* SA_F32 | SA_BF16 | SA_I8 (value = code * scale) */
  int32_t num_pages;        /* physical pages in k / v */
  int32_t page_size;        /* tokens per page; must be 16 [Quest page-level management] */
  int32_t num_kv_heads;
  int32_t head_dim;         /* must be 128 */
} sa_kv_cache;

/* The batch of sequences being decoded. */
typedef struct sa_seqs {
  const int32_t *page_table; /* [batch, max_pages]: physical page of logical page p of sequence b */
  const int32_t *seq_lens;   /* [batch] tokens per sequence */
  int32_t batch;
  int32_t max_pages;         /* row length of page_table; bounds every n_b */
} sa_seqs;

/* How units are scored and selected. */
typedef struct sa_select_cfg {
  int32_t mode;          /* SA_MODE_QUEST, SA_MODE_SALS or SA_MODE_PROBE */
  int32_t unit_tokens;   /* tokens per selection unit: 16 for QUEST (one page); multiple of 16 for SALS (64) and PROBE (32) */
  int32_t k_compete;     /* units chosen by score among the non-forced units (>= 0) */
  int32_t n_head_forced; /* leading units always kept (QUEST: 1, the sink page) */
  int32_t n_tail_forced; /* trailing units always kept (QUEST: 1, the recent page; SALS: 2 tail blocks) */
  int32_t rank;          /* SALS: width r of the low-rank index key; must be 16. QUEST: ignored */
  const float *proj;     /* SALS: device [head_dim, rank] fp32 projection P. QUEST: NULL */
  float lse_scale;       /* SALS: temperature tau of the block LSE (typically 1/sqrt(head_dim)) */
  int32_t n_probe;       /* PROBE: keys probed per block (>= 1; 8 in [RK]). Others: ignored */
  int32_t per_head;      /* QUEST: 1 = every query head selects its own pages (scores and page
                            lists per query head; the attention reads the group's union once,
                            [Quest] GQA section); 0 = one selection per group. Others: 0 */
} sa_select_cfg;

/* Library version (monotonic integer). */
int sa_version(void);

/* Human-readable text of a status code (static string, never NULL). */
const char *sa_status_string(int status);

/*
 * Selection metadata buffers, sized for the whole cache.
 *  QUEST [Quest, min/max metadata]: meta = [num_kv_heads, num_pages, 2, head_dim]
 *        in the KV dtype (head-major, so one kv-head's records of consecutive
 *        physical pages are contiguous); slot 0 = per-dimension max M, slot 1 =
 *        min m over the page's valid tokens.  Stored in the KV dtype (not fp16)
 *        so the values are exact and the bound stays valid.  meta_scale unused.
 *  SALS  [SALS low-rank preprocessing; SeqO1 sketch K*P]: meta = int4 codes
 *        [num_pages, page_size, num_kv_heads, rank/2] bytes (two codes per
 *        byte, low nibble = even index, two's complement in [-7, 7]);
 *        meta_scale = fp16 bits [num_pages, page_size, num_kv_heads].
 * sa_meta_bytes / sa_meta_scale_bytes return the byte sizes (0 on bad input).
 */
size_t sa_meta_bytes(const sa_kv_cache *kv, const sa_select_cfg *cfg);
size_t sa_meta_scale_bytes(const sa_kv_cache *kv, const sa_select_cfg *cfg);

/*
 * sa_build_page_meta - build the metadata of every page referenced by the
 * batch (pages (b, p < n_b)); other pages of meta are left untouched.
 *  QUEST: M_i = max and m_i = min over the page's valid tokens, i.e. the
 *         insert-time update M <- max(M, k), m <- min(m, k) folded over the page
 *         [Quest, incremental metadata update].  Not available for SA_I8 caches
 *         (SA_ERR_UNSUPPORTED).
 *  SALS:  per (token, kv-head) in fp32: khat = key (int8: code * scale);
 *         kp_j = fmaf chain over i = 0..d-1 of khat_i * P[i][j];
 *         scale = fp16_rne(max_j |kp_j| / 7); c_j = clamp(rint(kp_j / scale), -7, 7)
 *         (0 when scale == 0).  Slots past the sequence end are written as zeros.
 *         The codes are an encoding: identical inputs give identical bytes.
 * Amortised work (done once per token on insert in a serving loop), not part
 * of sa_decode_step.
 */
int sa_build_page_meta(const sa_kv_cache *kv, const sa_seqs *seqs, const sa_select_cfg *cfg,
                       void *meta, uint16_t *meta_scale, void *stream);

/*
 * sa_append_kv - decode-time insert of one new token per sequence with the
 * incremental metadata update [Quest, insert-time update M <- max(M, k),
 * m <- min(m, k) when a token joins a page; SALS, per-token low-rank
 * preprocessing of the index key].  For every b the new token is position
 * t = seq_lens[b] - 1 (seq_lens already counts it): slot s = t mod 16 of
 * physical page pp = page_table[b, t / 16].
 *  - k_new, v_new: [batch, num_kv_heads, head_dim] in the cache dtype (SA_I8:
 *    codes, with k_scale_new, v_scale_new = [batch, num_kv_heads] fp16 bits;
 *    both NULL for other dtypes).  They are copied into slot s of page pp of
 *    kv->k, kv->v (and kv->k_scale, kv->v_scale): this call WRITES the cache
 *    buffers that sa_kv_cache names (declared const for the read-only calls).
 *  - QUEST: s == 0 starts the page, M = m = k; otherwise M <- max(M, k) and
 *    m <- min(m, k) per (kv-head, dim), with the ordered comparisons that
 *    sa_build_page_meta folds a page with.  After any run of appends, meta
 *    equals a rebuild over the updated cache, bit for bit.
 *  - SALS: the token's codes and scale, exactly as sa_build_page_meta
 *    computes them (meta_scale required).
 * A sequence whose seq_lens[b] is outside [1, max_pages * 16], or whose page
 * id is outside [0, num_pages), is skipped (not reported).  The tokens of one
 * call belong to distinct pages (a page belongs to one sequence), so a call
 * has no write conflicts.  Not available for QUEST with SA_I8 caches
 * (SA_ERR_UNSUPPORTED).
 */
int sa_append_kv(const void *k_new, const void *v_new, const uint16_t *k_scale_new,
                 const uint16_t *v_scale_new, const sa_kv_cache *kv, const sa_seqs *seqs,
                 const sa_select_cfg *cfg, void *meta, uint16_t *meta_scale, void *stream);

/* Units per scores row: QUEST max_pages; SALS ceil(max_pages * 16 / unit_tokens). 0 on bad input. */
int32_t sa_max_units(const sa_seqs *seqs, const sa_select_cfg *cfg);

/*
 * sa_score_pages - one fp32 score per (b, kv-head, unit), written to
 * scores [batch, num_kv_heads, sa_max_units] (entries past each sequence's
 * unit count are not written).  QUEST with per_head: one score per (b, query
 * head, unit), scores [batch, num_q_heads, sa_max_units], each head's own bound.
 *  QUEST [Quest, criticality estimation + GQA]: score = max over the G query
 *        heads g of the group of sum_i max(q_gi * m_i, q_gi * M_i).
 *  PROBE [RK probe signal]: block u covers [u*U, min((u+1)*U, L)) with len
 *        tokens; step = max(1, len / n_probe); score = max over the probed
 *        positions u*U, u*U + step, ... (< block end) and over the group's G
 *        query heads of q_g . k_t (unscaled).  Reads K itself (no metadata:
 *        meta and meta_scale may be NULL, sa_meta_bytes is 0 and
 *        sa_build_page_meta does nothing).
 *  SALS  [SALS QSI steps 1-3]: qbar = mean of the group's G query heads;
 *        qt = qbar * P; s_t = scale_t * sum_j qt_j * c_tj per token;
 *        score_u = ln sum over the valid tokens t of block u of exp(lse_scale * s_t).
 * q: [batch, num_q_heads, head_dim] of q_dtype (SA_F32 or SA_BF16).
 */
int sa_score_pages(const void *q, int32_t q_dtype, int32_t num_q_heads, const sa_kv_cache *kv,
                   const sa_seqs *seqs, const sa_select_cfg *cfg, const void *meta,
                   const uint16_t *meta_scale, float *scores, void *stream);

/* Length of each selection list: min((k_compete + n_head + n_tail) * unit_tokens/16, max_pages). 0 on bad input. */
int32_t sa_max_selected(const sa_seqs *seqs, const sa_select_cfg *cfg);

/*
 * sa_topk_pages - exact selection per (b, kv-head) [Quest top-K filtering;
 * SALS QSI exact top-k and tail append; RK greedy fill, tie rule, recency].
 * With n = ceil(seq_lens[b] / unit_tokens) units: the first n_head_forced and
 * last n_tail_forced units are always kept; if n <= n_head + n_tail + k_compete
 * all n units are kept (no padding); otherwise the k_compete best of the
 * middle units are kept, ordered by (score descending, unit index ascending),
 * with -0.0 equal to +0.0.  The kept units are written as an ascending list of
 * LOGICAL page indices (each unit expands to its pages, clipped to n_b) into
 * sel [batch, num_kv_heads, sa_max_selected]; unused entries are -1; the
 * count goes to num_sel [batch, num_kv_heads].  Scores must be finite for the
 * units read (NaN is invalid input).  Identical inputs give identical output.
 */
int sa_topk_pages(const float *scores, int32_t num_kv_heads, const sa_seqs *seqs,
                  const sa_select_cfg *cfg, int32_t *sel, int32_t *num_sel, void *stream);

/*
 * sa_sparse_decode_attn_heads - attention with per-head selection [Quest, GQA
 * section: each query head's own pages, and the union the group then reads].
 * sel: [batch, num_q_heads, max_sel] logical pages, one list per query head
 * (sa_topk_pages on per-head scores, with num_q_heads lists per sequence),
 * num_sel [batch, num_q_heads].  Each head attends over its own pages only;
 * the pages of a (b, kv-head) group are read once, as the union of the
 * group's lists, which this call builds in the workspace (the union has at
 * most min(G * max_sel, max_pages) pages).  max_pages <= 16384.  Output and
 * the other arguments as sa_sparse_decode_attn; workspace:
 * >= sa_attn_heads_workspace_size(...) bytes.
 */
int sa_sparse_decode_attn_heads(const void *q, int32_t q_dtype, int32_t num_q_heads,
                                const sa_kv_cache *kv, const sa_seqs *seqs, const int32_t *sel,
                                const int32_t *num_sel, int32_t max_sel, float softmax_scale,
                                float *out, void *workspace, size_t workspace_bytes, void *stream);

/* Workspace of sa_sparse_decode_attn_heads.  0 on bad input. */
size_t sa_attn_heads_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t max_pages, int32_t max_sel);

/*
 * Workspace bytes of sa_sparse_decode_attn for a batch of `batch` sequences
 * with num_q_heads / num_kv_heads heads, page-table rows of max_pages entries
 * and selection lists of up to max_sel pages (max_sel <= 0: a dense pass over
 * up to max_pages pages per sequence).  The workspace holds the split-K
 * partial records (max, sum and accumulator per split and query head); it
 * needs no initial contents.  0 on bad input (unsupported group size,
 * batch < 1, max_pages < 1).
 */
size_t sa_attn_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t max_pages, int32_t max_sel);

/*
 * sa_sparse_decode_attn - out[b, hq, :] = softmax over the valid tokens of
 * the selected pages of (softmax_scale * q . k_t), applied to v_t
 * [Quest approximate attention; SALS SFAA; RK exact attention on the
 * selected set].  fp32 accumulation with an online softmax; the selected
 * pages of each (b, kv-head) are cut into splits whose partial (max, sum,
 * acc) triples are merged with the usual rescaling [SALS split-row reduce].
 * int8 caches use k = code * k_scale and v = code * v_scale.
 * sel: [batch, num_kv_heads, max_sel] logical pages (from sa_topk_pages), with
 * num_sel [batch, num_kv_heads] valid entries; sel == NULL and num_sel == NULL
 * selects every page of every sequence (dense decode attention).  A dense
 * pass over 2 .. 1024 sequences sizes its splits on the device from the
 * actual lengths, so short sequences get few splits [SALS tiling for
 * variable-length input]; the result does not depend on the split plan
 * beyond fp32 rounding order.
 * out: [batch, num_q_heads, head_dim] fp32.  A sequence with no valid token
 * gets zeros.  workspace: >= sa_attn_workspace_size(...) bytes.
 */
int sa_sparse_decode_attn(const void *q, int32_t q_dtype, int32_t num_q_heads,
                          const sa_kv_cache *kv, const sa_seqs *seqs, const int32_t *sel,
                          const int32_t *num_sel, int32_t max_sel, float softmax_scale, float *out,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * sa_sparse_decode_attn_noalloc - sa_sparse_decode_attn for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same computation, kernels and
 * results (bit for bit), with the split-K partial records in a scratch array
 * the library holds itself instead of a caller workspace.  The scratch is
 * 32 MiB of device memory per GPU the library runs on, held until the process
 * ends; its address is looked up on the first call on each device (make that
 * first call outside stream capture).  A call whose partial records would
 * exceed it (sa_attn_workspace_size(...) > 32 MiB, e.g. thousands of lists
 * with 16-head groups) returns SA_ERR_WORKSPACE_TOO_SMALL before anything is
 * enqueued.  No call allocates or frees.  Every call on one GPU shares that
 * GPU's scratch: calls that overlap in time on one GPU (on different streams,
 * or from different host threads without ordering) race and give undefined
 * output; calls ordered on one stream are safe.  Arguments, output and errors
 * otherwise as sa_sparse_decode_attn (SA_ERR_HIP if the scratch cannot be
 * located).
 */
int sa_sparse_decode_attn_noalloc(const void *q, int32_t q_dtype, int32_t num_q_heads,
                                  const sa_kv_cache *kv, const sa_seqs *seqs, const int32_t *sel,
                                  const int32_t *num_sel, int32_t max_sel, float softmax_scale,
                                  float *out, void *stream);

/* Workspace of sa_decode_step.  0 on bad input. */
size_t sa_decode_step_workspace_size(int32_t num_q_heads, const sa_kv_cache *kv,
                                     const sa_seqs *seqs, const sa_select_cfg *cfg);

/*
 * sa_decode_step - sa_score_pages -> sa_topk_pages -> sa_sparse_decode_attn
 * on one stream, with every intermediate in the caller's workspace; only the
 * integer page lists pass from selection to attention [SeqO1, FlashSA].
 * Metadata must already be built (sa_build_page_meta).  When every list keeps
 * all of its units (k_compete + forced units >= sa_max_units) scoring is
 * skipped and dense attention runs.  sel / num_sel (optional, may be NULL)
 * receive the selection as sa_topk_pages writes it.  With per_head (QUEST),
 * the step runs sa_score_pages -> sa_topk_pages over the query heads ->
 * sa_sparse_decode_attn_heads, and sel / num_sel are per query head:
 * [batch, num_q_heads, sa_max_selected] and [batch, num_q_heads].
 * Quest mode with one query head per kv-head and lists of up to 4096 pages
 * runs as a single persistent kernel (one workgroup per compute unit) whose
 * workgroups hand score keys and partial records to each other through the
 * workspace; no workgroup ever waits for another, so the result does not
 * depend on how many of them are resident at a time (a build that uses
 * scratch memory runs the separate kernels instead; same results).  Other
 * steps with a bf16 query, bf16 or int8 K/V and lists short enough for the
 * selection's register keys (sa_max_units up to 4 per selection thread) run
 * the scorer and then one persistent kernel for the top-K, the attention and
 * the merge, whose chunk workgroups hand partial records to the last-arriving
 * one the same way; the rest run the separate kernels.
 * Workspace protocol of every sa_decode_step call:
 *  - the workspace must be zero-filled before its first use;
 *  - every call leaves its hand-off words (per-list arrival counters and score
 *    keys) zero again when it completes; a call that does not complete (the
 *    process or the device is stopped mid-kernel) leaves them undefined, and
 *    the workspace must then be zero-filled before it is used again;
 *  - one workspace serves one call at a time: calls that share it must be
 *    ordered on one stream.
 * The environment variable SA_STEP_MAX_WORKGROUPS (a positive integer, read
 * at every call) caps the persistent kernels' workgroups, e.g. to leave
 * compute units to other work; the result is the same bit for bit.
 */
int sa_decode_step(const void *q, int32_t q_dtype, int32_t num_q_heads, const sa_kv_cache *kv,
                   const sa_seqs *seqs, const sa_select_cfg *cfg, const void *meta,
                   const uint16_t *meta_scale, float softmax_scale, float *out, int32_t *sel,
                   int32_t *num_sel, void *workspace, size_t workspace_bytes, void *stream);

/*
 * sa_stream_read - measurement helper, not a step of the path: reads `bytes`
 * (a nonzero multiple of 16) of device memory at src (16-byte aligned) once,
 * with 16-byte loads spread over about eight workgroups per compute unit, so
 * that its time gives the bandwidth a plain streaming read reaches on this
 * device.  The decode step is bound by the bytes it reads ([SeqO1] bottleneck
 * analysis; [Quest] read-volume formula), so this is the second denominator
 * its effective bandwidth is quoted against, beside the HBM peak.  sink:
 * device words, one per workgroup (min(sink_words, 8 * compute units)
 * workgroups); they are written only when a workgroup's XOR of its words
 * equals one fixed value.  SA_ERR_INVALID_ARG on a null or misaligned src,
 * a bad size, or a null sink.
 */
int sa_stream_read(const void *src, size_t bytes, uint32_t *sink, size_t sink_words, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SA_H */
