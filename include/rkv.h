/*
 * rkv.h -- C ABI of librkv, the MI355X (gfx950) library for RocketKV's decode
 * path: SnapKV++ stage-1 eviction once per prefill, then Hybrid Sparse
 * Attention (HSA) over the pruned, paged KV cache at every decode step.
 *
 * Sources (web pages on RocketKV, cited by title and section):
 *   [P1] "RocketKV: Accelerating Long-Context LLM Inference via Two-Stage KV
 *        Cache Compression" (atlas.scime.ai summary): "Approach".
 *   [P2] The paper's abstract (papers.pytorch.kr/papers/2502.14051).
 *   [P3] "RocketKV-adapted -- Two-Stage Compression" (veloxquant-mlx docs):
 *        "Where it sits -- the mechanism gap", "The one setting worth
 *        tuning", "Adaptation notes", "Evidence".
 *
 * Conventions shared by every entry point
 *  - Device pointers are HIP device addresses (for example torch CUDA tensor
 *    data pointers); host pointers are marked "host".  The caller owns every
 *    buffer; the library allocates nothing and keeps no mutable global state.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls only enqueue work on it; nothing synchronises the host.  Calls on
 *    different streams are independent as long as their buffers are.
 *  - Every call returns an rkv status (0 = RKV_OK).  Arguments are checked on
 *    the host before anything is enqueued; a failed check enqueues nothing.
 *    Lengths known on the host that do not fit the cache give RKV_ECAPACITY.
 *    Values that live in device memory (sequence lengths, page tables, page
 *    lists) cannot be checked on the host: kernels keep every access inside
 *    the buffers described here (a length is clamped to the cache capacity,
 *    a page whose physical block is outside [0, num_blocks) contributes no
 *    rows) and report each such input in the optional device status word of
 *    rkv_opts (RKV_DEV_* flags below), so a caller that overruns the cache
 *    can find out; results for such inputs are defined but meaningless.
 *  - A HIP error left pending on the calling host thread by earlier runtime
 *    calls is cleared when an entry point starts, so RKV_EHIP reports only
 *    the launches of that call.
 *  - Element type `dtype` (RKV_F32 or RKV_BF16) applies to queries, keys,
 *    values and page summaries alike.  Attention outputs are always fp32.
 *  - GQA: query head h*G + j (j < G) reads KV head h.
 *  - Index outputs are ascending and padded with -1.
 */
#ifndef RKV_H
#define RKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define RKV_OK 0
#define RKV_EINVAL (-1)       /* bad argument (null pointer, out-of-range size) */
#define RKV_EWORKSPACE (-2)   /* workspace missing or smaller than required */
#define RKV_ECAPACITY (-3)    /* rows do not fit the cache / page table */
#define RKV_EUNSUPPORTED (-4) /* shape or dtype the library has no kernel for */
#define RKV_EHIP (-5)         /* a HIP launch reported an error */
#define RKV_ESCRATCH (-6)     /* rkv_decode_step_static: the shapes need more than the
                                 library's static scratch (RKV_STATIC_SCRATCH_BYTES) */

/* ---- element types ----------------------------------------------------- */
#define RKV_F32 0
#define RKV_BF16 1

/* Supported shapes: head_dim in {64, 128}; group in {1, 2, 4, 8};
 * page_size in [1, 256]; 1 <= k1 <= head_dim; 1 <= k2 <= RKV_MAX_K2. */
#define RKV_MAX_K2 4096
#define RKV_MAX_EVICT_BATCH 128

/* GQA layout: Hq = n_kv_heads * group query heads. */
typedef struct rkv_gqa {
    int32_t n_kv_heads; /* Hkv */
    int32_t group;      /* G */
    int32_t head_dim;   /* d */
} rkv_gqa;

/* Paged KV cache.  A physical block holds one page of every KV head:
 *   k_pool, v_pool : [num_blocks][Hkv][page_size][d]  (dtype)
 *   page_table     : [B][max_pages] int32, physical block of logical page p
 *                    of sequence b.
 * Logical row r of sequence b, KV head h lives at
 *   pool[page_table[b][r / page_size]][h][r % page_size][:].
 * The page size is also HSA's page: summaries and page selection are per
 * logical page.  Pools must be 16-byte aligned, and num_blocks * Hkv *
 * page_size must be below 2^32 - 1 (the kernels name a pool row with 32
 * bits; larger pools give RKV_EUNSUPPORTED). */
typedef struct rkv_paged_cache {
    void *k_pool;
    void *v_pool;
    const int32_t *page_table;
    int64_t num_blocks;
    int32_t page_size; /* P */
    int32_t max_pages; /* capacity per sequence = max_pages * P rows */
} rkv_paged_cache;

/* Page summaries ("summaries" below): [B][Hkv][2][d][max_pages] in dtype.
 * [..][0][c][p] is the element-wise maximum and [..][1][c][p] the minimum of
 * channel c over the valid rows of logical page p ([P3] "Where it sits":
 * Quest-style paged max/min along the sequence).  Channel-major so that each
 * selected channel is one contiguous run over the pages.  Among equal values
 * the earliest row's bits are kept, so an incremental append gives the same
 * bits as a rebuild ([P3] "Evidence"). */

/* ---- execution options ---------------------------------------------------
 * The last argument of every call that enqueues device work.  NULL, or a
 * zero-initialised struct, means: the library picks every kernel form and
 * size by its documented rule, and no status word is written.  The fields
 * other than `status` fix how the decode calls run (tests and tuning); they
 * never change results beyond the documented tolerances, and
 * rkv_hsa_workspace_bytes must be given the same options as the calls whose
 * workspace it sizes. */
#define RKV_FORM_AUTO 0       /* the rule given at rkv_decode_step */
#define RKV_FORM_STANDALONE 1 /* separate select and attention kernels */
#define RKV_FORM_FUSED 2      /* one fused kernel, one block per (sequence, KV head) */
#define RKV_FORM_SPLITK 3     /* the fused kernel split K-wise, plus a merge kernel */

/* Device status flags, ORed into *rkv_opts.status by the kernels. */
#define RKV_DEV_LENGTH 1 /* a row count was negative or beyond max_pages * P: clamped */
#define RKV_DEV_BLOCK 2  /* a page-table entry in use was outside [0, num_blocks): skipped */
#define RKV_DEV_PAGE 4   /* a page index given to rkv_hsa_attend was outside [0, NP): skipped */

typedef struct rkv_opts {
    int32_t form;           /* RKV_FORM_*; a form the shapes do not allow falls back to
                               RKV_FORM_STANDALONE */
    int32_t splitk_blocks;  /* RKV_FORM_SPLITK: blocks to aim for in all (0 = 128, or 256
                               when more than 65,536 rows are selected in all) */
    int32_t select_chunk;   /* standalone selection: pages per block (0 = automatic) */
    int32_t select_radix;   /* standalone selection over several chunks: 1 = radix top-k
                               and radix merge instead of rank-ordered lists (0 = auto) */
    int32_t attend_variant; /* standalone attention block shape, 1..4 (0 = automatic):
                               1 = 4 waves, 8 rows of K and V per lane in flight;
                               2 = 8 waves, pipelined; 3 = 16 waves; 4 = 16 waves,
                               pipelined */
    int32_t attend_pages;   /* standalone attention: selected pages per block
                               (0 = automatic) */
    int32_t *status;        /* device int32, optional: RKV_DEV_* flags are ORed in; the
                               library never clears it */
    uint64_t *trace;        /* device buffer, optional, read only by a library built with
                               RKV_PHASE_TIMING: the fused decode kernel writes
                               RKV_TRACE_SLOTS clock stamps per block (block x + gridDim.x *
                               (y + gridDim.y * z)); ignored by the normal build */
} rkv_opts;

/* Phase stamps of the fused decode kernel in a RKV_PHASE_TIMING build, in
 * units of the device's constant wall clock (hipDeviceAttributeWallClockRate):
 * slot 0 block start, 1 queries loaded, 2 channels ranked, 3 summaries
 * staged, 24 page bounds done, 4 pages chosen and visible to the block, 5
 * stream starts, 6..21 the end of each wave's stream (6 + wave; the stream
 * runs on the first 8 waves, the others stamp at once), 22 block end, 23 the
 * XCC the block ran on; slots 25..31 are unused. */
#define RKV_TRACE_SLOTS 32

/* Human-readable text for a status code (static storage). */
const char *rkv_status_string(int status);

/* Content hash of the sources this library was built from (static storage). */
const char *rkv_build_id(void);

/* ---- adaptive split (host only) ---------------------------------------- */
/* [P3] "The one setting worth tuning"; [P1] "Approach".
 * r = clip(0.2 + 0.06 * log2(c), 0.2, 0.8); stage 1 keeps a 1/c^r share,
 * stage 2 attends a 1/c^(1-r) share of what stage 1 kept.
 *   c  : overall target compression ratio, finite and >= 1.
 *   L  : prompt length (rows), >= 0;  w : observation window, >= 0.
 *   keep = min(L, max(w, floor(L / c^r))).
 * Any output pointer may be NULL.  Errors: RKV_EINVAL for c < 1, non-finite
 * c, L < 0 or w < 0.  Pure host arithmetic in double precision. */
int rkv_split_ratio(double c, int64_t L, int64_t w, double *r, double *c_evict,
                    double *c_hsa, int64_t *keep);

/* ---- SnapKV++ stage-1 eviction ------------------------------------------ */
/* [P2] abstract: SnapKV++ = SnapKV with adaptive pooling size and full GQA
 * compatibility.  [P1] "Approach": large pooling kernel, GQA-group-level
 * selection.  Per sequence b and KV head h, with L = prompt_lens[b]:
 *   - the last w prompt queries of the G heads of the group score every key
 *     they can see (causal): p = softmax(scale * q . k) per query;
 *   - the probabilities are summed over the window queries and then over
 *     the G heads, for the prefix keys t < L - w;
 *   - the sums are max-pooled with an odd window `pool_kernel` (centred,
 *     stride 1, clipped at the ends of the prefix);
 *   - the keep[b] - w best prefix keys (ties to the lower position) are
 *     kept in ascending order, followed by the w window rows;
 *   - K and V rows of the kept positions are written, in that order, to
 *     logical rows [0, keep[b]) of sequence b in the paged cache.
 * If keep[b] >= L every row is kept in place (no scoring).
 * The softmax denominator is accumulated in fp64 and rounded once to fp32;
 * everything else is fp32 with bf16 inputs widened exactly.
 *
 * Arguments
 *   g, dtype      : GQA layout and element type.
 *   B             : sequences, 1..RKV_MAX_EVICT_BATCH.
 *   prompt_lens   : host [B], 0 <= L <= L_max.
 *   keep          : host [B], rows to keep; w <= keep unless keep >= L.
 *   L_max, w      : prompt row stride of q/k/v and observation window (>= 1).
 *   pool_kernel   : odd, >= 1.
 *   scale         : logit scale (normally 1/sqrt(d)), finite and > 0.
 *   q_win         : device [B][Hq][w][d], query i of a head sits at L-w+i.
 *   k, v          : device [B][Hkv][L_max][d], prompt keys/values (keys
 *                   already position-encoded), 16-byte aligned.
 *   cache         : destination; needs min(keep, L) <= max_pages * P.
 *   summaries     : device, optional (NULL = skip); rebuilt for the kept
 *                   rows [0, min(keep, L)) of every sequence.
 *   kept_idx      : device [B][Hkv][keep_stride], optional; kept prompt
 *                   positions, ascending, -1 padded.
 *   keep_stride   : row stride of kept_idx; >= max_b min(keep[b], L_b).
 *   pooled_scores : device [B][Hkv][L_max] fp32, optional; pooled score of
 *                   every prefix key (entries >= L-w are left untouched).
 *   seq_lens_out  : device [B] int32, optional; receives min(keep, L).
 *   ws, ws_bytes  : device workspace of at least
 *                   rkv_prefill_evict_workspace_bytes(g, B, L_max, w).
 * Errors: RKV_EINVAL, RKV_EUNSUPPORTED, RKV_ECAPACITY, RKV_EWORKSPACE,
 * RKV_EHIP. */
size_t rkv_prefill_evict_workspace_bytes(const rkv_gqa *g, int32_t B, int64_t L_max,
                                         int32_t w);
int rkv_prefill_evict(const rkv_gqa *g, int32_t dtype, int32_t B,
                      const int32_t *prompt_lens, const int32_t *keep, int64_t L_max,
                      int32_t w, int32_t pool_kernel, float scale, const void *q_win,
                      const void *k, const void *v, const rkv_paged_cache *cache,
                      void *summaries, int32_t *kept_idx, int32_t keep_stride,
                      float *pooled_scores, int32_t *seq_lens_out, void *ws,
                      size_t ws_bytes, void *stream,
                   const rkv_opts *opts);

/* ---- chunked-prefill eviction -------------------------------------------- */
/* [P3] "Evidence": stage-1 eviction re-enforces its budget across the calls
 * of a chunked prefill.  Each call evicts over the sequence formed by the
 * n_cached[b] rows already in the cache (logical rows 0 .. n_cached-1, in
 * order) followed by the chunk_lens[b] rows of the new chunk, exactly as
 * rkv_prefill_evict does for a prompt of L = n_cached + chunk_len rows whose
 * observation window is the chunk's last w queries; the kept rows end up in
 * logical rows [0, min(keep, L)) of the cache and the summaries are rebuilt
 * for them.  kept_idx and pooled_scores index that concatenated sequence.
 *
 * Arguments (as rkv_prefill_evict unless noted)
 *   n_cached      : host [B], rows now in the cache (>= 0).
 *   chunk_lens    : host [B], rows in this chunk; chunk_len >= w unless
 *                   n_cached + chunk_len <= keep (nothing to evict).
 *   C_max         : row stride of k_chunk/v_chunk, >= every chunk_len.
 *   q_win         : device [B][Hq][w][d], the chunk's last w queries.
 *   k_chunk, v_chunk : device [B][Hkv][C_max][d], 16-byte aligned.
 *   cache         : holds the n_cached rows (n_cached <= max_pages * P);
 *                   needs min(keep, L) <= max_pages * P; its rows are read,
 *                   then rewritten.
 *   pooled_scores : device [B][Hkv][L_max] fp32, optional, with
 *                   L_max = max_b (n_cached + chunk_len).
 *   ws, ws_bytes  : device workspace of at least
 *                   rkv_prefill_evict_chunk_workspace_bytes(g, B, L_max, w)
 *                   for that L_max.
 * Errors: RKV_EINVAL, RKV_EUNSUPPORTED, RKV_ECAPACITY, RKV_EWORKSPACE,
 * RKV_EHIP. */
size_t rkv_prefill_evict_chunk_workspace_bytes(const rkv_gqa *g, int32_t B, int64_t L_max,
                                               int32_t w);
int rkv_prefill_evict_chunk(const rkv_gqa *g, int32_t dtype, int32_t B,
                            const int32_t *n_cached, const int32_t *chunk_lens,
                            const int32_t *keep, int64_t C_max, int32_t w,
                            int32_t pool_kernel, float scale, const void *q_win,
                            const void *k_chunk, const void *v_chunk,
                            const rkv_paged_cache *cache, void *summaries, int32_t *kept_idx,
                            int32_t keep_stride, float *pooled_scores, int32_t *seq_lens_out,
                            void *ws, size_t ws_bytes, void *stream,
                   const rkv_opts *opts);

/* ---- multi-turn view (RocketKV-MT) ----------------------------------------- */
/* [P1] "Approach" and "Limitations": RocketKV-MT retains the tokens stage 1
 * would evict for later turns (memory-traffic savings only); [P3] "Should you
 * use this?": it skips permanent eviction so that earlier-turn tokens
 * survive.  Reading: at the start of a turn, with the turn's rows already
 * appended to the full cache, SnapKV++ (as rkv_prefill_evict) scores the
 * first n_rows[b] rows of `full` with the turn's last w queries and keeps
 * keep[b] of them; the kept rows, in ascending position, are written to
 * logical rows [0, min(keep, n)) of `view` and the view's summaries are
 * rebuilt.  HSA then decodes over the view for the turn.  `full` is only
 * read: nothing is deleted, so a row left out of one turn's view can be in
 * the next one's.
 *   n_rows, keep  : host [B]; keep >= w and n_rows >= w unless keep >= n_rows
 *                   (the view is then the whole history).
 *   q_win         : device [B][Hq][w][d], the turn's last w queries (query i
 *                   at position n - w + i).
 *   full          : the retained history, n_rows <= capacity.
 *   view          : destination, needs min(keep, n) <= capacity; its blocks
 *                   must not overlap those of full's first n rows.
 *   view_summaries: device [B][Hkv][2][d][view max_pages], optional.
 *   kept_idx, keep_stride, pooled_scores, view_lens_out : as rkv_prefill_evict
 *                   (positions in the full history; pooled_scores
 *                   [B][Hkv][max n]).
 *   ws, ws_bytes  : rkv_turn_filter_workspace_bytes(g, B, max n, w).
 * Errors: RKV_EINVAL, RKV_EUNSUPPORTED, RKV_ECAPACITY, RKV_EWORKSPACE,
 * RKV_EHIP. */
size_t rkv_turn_filter_workspace_bytes(const rkv_gqa *g, int32_t B, int64_t L_max, int32_t w);
int rkv_turn_filter(const rkv_gqa *g, int32_t dtype, int32_t B, const int32_t *n_rows,
                    const int32_t *keep, int32_t w, int32_t pool_kernel, float scale,
                    const void *q_win, const rkv_paged_cache *full, const rkv_paged_cache *view,
                    void *view_summaries, int32_t *kept_idx, int32_t keep_stride,
                    float *pooled_scores, int32_t *view_lens_out, void *ws, size_t ws_bytes,
                    void *stream, const rkv_opts *opts);

/* ---- incremental page-summary append ------------------------------------ */
/* [P3] "Where it sits" (paged max/min) and "Evidence" (incremental update
 * == rebuild).  For every sequence b, rows [n_old[b], n_new[b]) are folded
 * into the summaries of the pages they fall in.  A page that begins at or
 * after n_old[b] is initialised from its first new row.  If k_src/v_src are
 * given, the new rows are first copied into the paged cache from
 *   k_src, v_src : device [B][Hkv][max_new_rows][d] (row r at index r-n_old).
 * n_old, n_new  : device [B] int32; rows beyond n_old + max_new_rows and
 *                 beyond the cache capacity are ignored; n_new <= n_old is a
 *                 no-op for that sequence.
 * max_new_rows  : >= 1, host-side bound on n_new - n_old (sizes the grid).
 * summaries     : device [B][Hkv][2][d][max_pages].
 * Errors: RKV_EINVAL, RKV_EUNSUPPORTED, RKV_EHIP. */
int rkv_append_summaries(const rkv_gqa *g, int32_t dtype, int32_t B,
                         const rkv_paged_cache *cache, const int32_t *n_old,
                         const int32_t *n_new, int32_t max_new_rows, const void *k_src,
                         const void *v_src, void *summaries, void *stream,
                   const rkv_opts *opts);

/* ---- Hybrid Sparse Attention decode ------------------------------------- */
/* [P3] "Where it sits": scores are approximated by a two-dimensional
 * reduction, SparQ-style top-magnitude channels along the head dimension and
 * Quest-style page summaries along the sequence.  [P3] "Adaptation notes":
 * whole pages (k2 of them) are selected.  [P3] "Evidence": the page score
 * bounds every in-page dot product.  Per sequence b and KV head h with
 * n = seq_lens[b] rows (NP = ceil(n/P) pages):
 *   a[c]   = sum_j |q_j[c]|                         (fp32, j ascending)
 *   I1     = k1 channels with the largest a (ties: lower c), ascending
 *   s_j(p) = sum_{c in I1 asc} max(q_j[c]*Kmax[p][c], q_j[c]*Kmin[p][c])
 *   S(p)   = sum_{j asc} s_j(p)                      (fp32, no fused mul-add)
 *   I2     = min(k2, NP) pages with the largest S (ties: lower p), ascending
 *   out_j  = softmax(scale * q_j . k_t) v_t over the valid rows t of the
 *            pages in I2, fp32 accumulation.
 * n = 0 selects nothing and writes zeros.
 *
 * Arguments
 *   q            : device [B][Hq][d] decode queries, 16-byte aligned.
 *   seq_lens     : device [B] int32 rows per sequence (current token
 *                  included); clamped to [0, max_pages * P] (RKV_DEV_LENGTH).
 *   page_idx, for rkv_hsa_attend: its first min(k2, NP) entries must be
 *                  pages in [0, NP); others are skipped (RKV_DEV_PAGE).
 *   summaries    : device [B][Hkv][2][d][max_pages], current for seq_lens.
 *   k1, k2       : channels and pages kept.
 *   chan_idx     : device [B][Hkv][k1] int32, optional.
 *   page_idx     : device [B][Hkv][k2] int32 (required by rkv_hsa_select and
 *                  rkv_hsa_attend, optional for rkv_hsa_decode).
 *   page_scores  : device [B][Hkv][max_pages] fp32, optional; S(p) for
 *                  p < NP (entries beyond are untouched).
 *   scale        : logit scale (normally 1/sqrt(d)), finite and > 0.
 *   out          : device [B][Hq][d] fp32.
 *   ws, ws_bytes : device workspace of at least rkv_hsa_workspace_bytes(...)
 *                  for the same shapes and options; calls sharing one
 *                  workspace must be ordered on one stream.
 *   opts         : execution options (NULL = automatic); see rkv_opts.
 * rkv_hsa_decode gives the results of rkv_hsa_select followed by
 * rkv_hsa_attend on `stream`; it runs as rkv_decode_step without an append
 * (one of the fused forms where the shapes allow).
 * Errors: RKV_EINVAL, RKV_EUNSUPPORTED, RKV_EWORKSPACE, RKV_EHIP. */
size_t rkv_hsa_workspace_bytes(const rkv_gqa *g, int32_t B, int32_t page_size,
                               int32_t max_pages, int32_t k1, int32_t k2,
                               const rkv_opts *opts);
int rkv_hsa_select(const rkv_gqa *g, int32_t dtype, int32_t B, const void *q,
                   const int32_t *seq_lens, int32_t page_size, int32_t max_pages,
                   const void *summaries, int32_t k1, int32_t k2, int32_t *chan_idx,
                   int32_t *page_idx, float *page_scores, void *ws, size_t ws_bytes,
                   void *stream,
                   const rkv_opts *opts);
int rkv_hsa_attend(const rkv_gqa *g, int32_t dtype, int32_t B, const void *q,
                   const rkv_paged_cache *cache, const int32_t *seq_lens,
                   const int32_t *page_idx, int32_t k2, float scale, float *out, void *ws,
                   size_t ws_bytes, void *stream,
                   const rkv_opts *opts);
int rkv_hsa_decode(const rkv_gqa *g, int32_t dtype, int32_t B, const void *q,
                   const rkv_paged_cache *cache, const int32_t *seq_lens,
                   const void *summaries, int32_t k1, int32_t k2, float scale, float *out,
                   int32_t *chan_idx, int32_t *page_idx, float *page_scores, void *ws,
                   size_t ws_bytes, void *stream,
                   const rkv_opts *opts);

/* ---- one decode step of one layer ---------------------------------------- */
/* The per-layer hot path: append the new token, then HSA decode.  With
 * n = seq_lens[b] (the new token included), row n-1 of every (sequence, KV
 * head) is written from k_new/v_new and folded into the summary of its page
 * ([P3] "Evidence": incremental update == rebuild), then selection and
 * attention run exactly as rkv_hsa_decode.  Equivalent to
 * rkv_append_summaries(n-1 -> n, copying k_new/v_new) followed by
 * rkv_hsa_decode, with identical results.
 *   k_new, v_new : device [B][Hkv][d], or both NULL (no append: this is then
 *                  rkv_hsa_decode).
 *   summaries    : current for rows [0, n-1) on entry, for [0, n) on return.
 * How it runs (same results every way; max_pages <= 2048 is needed for
 * either fused form; groups of 8 run 8-wave blocks, whose split-K stage
 * holds at most 512 pages):
 *   - B * Hkv >= 192 (the batch fills the chip) and k2 * P <= 2048: a single
 *     kernel, one 16-wave block per (sequence, KV head);
 *   - otherwise, when the summaries fit the kernel's LDS stage (max_pages <=
 *     1024, 512 for G = 8, and 2 * k1 * max_pages * sizeof(element) <= 64 KiB,
 *     max_pages rounded up to 16 bytes of elements): the same kernel split
 *     K-wise,
 *     about 128 blocks in all (256 when more than 65,536 rows are selected
 *     in all, more when a share would exceed 2048 rows),
 *     each making the unit's selection and attending to a share of its
 *     pages, then a merge kernel (two launches);
 *   - otherwise the standalone append, select and attention kernels.
 * rkv_opts.form picks a form explicitly: RKV_FORM_FUSED wherever its limits
 * hold, RKV_FORM_SPLITK where the stage fits, else the standalone kernels.
 * Other arguments and errors as for rkv_hsa_decode. */
/* Which form rkv_decode_step (and rkv_hsa_decode) takes for these shapes and
 * options, by the rule above: RKV_FORM_STANDALONE, RKV_FORM_FUSED or
 * RKV_FORM_SPLITK (never RKV_FORM_AUTO).  Host only, no device work.
 * Errors: RKV_EINVAL (bad layout or sizes), RKV_EUNSUPPORTED (dtype). */
int rkv_decode_mode(const rkv_gqa *g, int32_t dtype, int32_t B, int32_t page_size,
                    int32_t max_pages, int32_t k1, int32_t k2, const rkv_opts *opts);

int rkv_decode_step(const rkv_gqa *g, int32_t dtype, int32_t B, const void *q,
                    const void *k_new, const void *v_new, const rkv_paged_cache *cache,
                    const int32_t *seq_lens, void *summaries, int32_t k1, int32_t k2,
                    float scale, float *out, int32_t *chan_idx, int32_t *page_idx,
                    float *page_scores, void *ws, size_t ws_bytes, void *stream,
                   const rkv_opts *opts);

/* ---- the same step without a caller workspace ------------------------------ */
/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): exactly
 * rkv_decode_step, but the workspace is a static device array of
 * RKV_STATIC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  Nothing is allocated or freed by this call.
 * The array's address on the current device is looked up on the first call
 * on that device.  Every call on one GPU shares that GPU's array, so calls
 * that may overlap on one GPU (different streams, or host threads without
 * ordering) race and must not be issued; calls ordered on one stream are
 * fine.  The array's contents are whatever the last call left; the decode
 * kernels write every part they read, so nothing needs clearing.
 * Errors: as rkv_decode_step, plus RKV_ESCRATCH when
 * rkv_hsa_workspace_bytes(g, B, P, max_pages, k1, k2, opts) exceeds
 * RKV_STATIC_SCRATCH_BYTES, and RKV_EHIP when the array's address cannot be
 * obtained. */
#define RKV_STATIC_SCRATCH_BYTES (16u << 20)
int rkv_decode_step_static(const rkv_gqa *g, int32_t dtype, int32_t B, const void *q,
                           const void *k_new, const void *v_new, const rkv_paged_cache *cache,
                           const int32_t *seq_lens, void *summaries, int32_t k1, int32_t k2,
                           float scale, float *out, int32_t *chan_idx, int32_t *page_idx,
                           float *page_scores, void *stream, const rkv_opts *opts);

#ifdef __cplusplus
/* ---- measurement helper (not part of the method) ---------------------- */
/* Reads n_chunks chunks of RKV_READ_PROBE_CHUNK bytes from the device buffer
 * buf (16-byte aligned) with 16-byte non-temporal loads, over at most
 * RKV_READ_PROBE_BLOCKS blocks of 256 threads, and stores per wave the XOR
 * of the 32-bit words it read into sink (device uint32; the first
 * min(n_chunks, RKV_READ_PROBE_BLOCKS) * 4 words are written, at most
 * RKV_READ_PROBE_SINK_WORDS), so no load can be dropped and the stored words
 * XOR to the XOR of every word read.  Chunk i starts at byte offsets[i]
 * (device int64; each a multiple of 16 with the chunk inside buf: device
 * data, not checked) or, with offsets NULL, at i * RKV_READ_PROBE_CHUNK (buf
 * then holds n_chunks chunks).  Asynchronous on stream.  It times the
 * device's plain streaming read and its 4 KB page-slice gather (the decode
 * kernel's K/V access pattern) beside the decode kernel.
 * RKV_EINVAL: buf or sink NULL, buf not 16-byte aligned, or n_chunks < 1. */
#define RKV_READ_PROBE_CHUNK 4096
#define RKV_READ_PROBE_BLOCKS 2048
#define RKV_READ_PROBE_SINK_WORDS (RKV_READ_PROBE_BLOCKS * 4)
int rkv_read_probe(const void *buf, const int64_t *offsets, int64_t n_chunks, uint32_t *sink,
                   void *stream);

} /* extern "C" */
#endif

#endif /* RKV_H */
