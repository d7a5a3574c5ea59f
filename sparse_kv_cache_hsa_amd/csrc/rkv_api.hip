// rkv_api.hip -- the extern "C" entry points of librkv: argument checks on
// the host, workspace sizing and dispatch to the kernel launchers.
#include <math.h>
#include <string.h>

#include <mutex>

#include "rkv_internal.h"

#ifndef RKV_BUILD_ID
#define RKV_BUILD_ID "unknown"
#endif

using namespace rkv;

// The workspace of rkv_decode_step_static.  In host code `scratch` names a
// host-side stand-in, never the device array: its device address is looked
// up per device with hipGetSymbolAddress and only that address is used.
static __device__ __align__(256) unsigned char scratch[RKV_STATIC_SCRATCH_BYTES];

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0u; }

int check_gqa(const rkv_gqa *g) {
    if (!g) return RKV_EINVAL;
    if (g->n_kv_heads < 1 || g->n_kv_heads > 65535 || g->group < 1 || g->head_dim < 1)
        return RKV_EINVAL;
    if (g->group != 1 && g->group != 2 && g->group != 4 && g->group != 8) return RKV_EUNSUPPORTED;
    if (g->head_dim != 64 && g->head_dim != 128) return RKV_EUNSUPPORTED;
    return RKV_OK;
}

int check_dtype(int dtype) {
    return (dtype == RKV_F32 || dtype == RKV_BF16) ? RKV_OK : RKV_EUNSUPPORTED;
}

// g has passed check_gqa.
int check_cache(const rkv_gqa *g, const rkv_paged_cache *c) {
    if (!c || !c->k_pool || !c->v_pool || !c->page_table) return RKV_EINVAL;
    if (c->num_blocks < 1 || c->page_size < 1 || c->max_pages < 1) return RKV_EINVAL;
    if (c->page_size > 256) return RKV_EUNSUPPORTED;
    // the kernels name a pool row by a 32-bit unit (block * Hkv + head) * P
    // + slot, with 0xffffffff reserved for "no row"
    if (c->num_blocks > ((int64_t)0xffffffff - 1) / ((int64_t)g->n_kv_heads * c->page_size))
        return RKV_EUNSUPPORTED;
    if ((int64_t)c->max_pages * c->page_size > (int64_t)1 << 30) return RKV_EINVAL;
    if (!aligned16(c->k_pool) || !aligned16(c->v_pool)) return RKV_EINVAL;
    return RKV_OK;
}

int check_select_args(const rkv_gqa *g, int32_t dtype, int32_t B, const void *q,
                      const int32_t *seq_lens, int32_t P, int32_t max_pages, int32_t k1,
                      int32_t k2) {
    int st = check_gqa(g);
    if (st != RKV_OK) return st;
    if ((st = check_dtype(dtype)) != RKV_OK) return st;
    if (B < 1 || B > 65535 || !q || !seq_lens || !aligned16(q)) return RKV_EINVAL;
    if (P < 1 || max_pages < 1) return RKV_EINVAL;
    if (P > 256) return RKV_EUNSUPPORTED;
    if ((int64_t)max_pages * P > (int64_t)1 << 30) return RKV_EINVAL;
    if (k1 < 1 || k1 > g->head_dim || k2 < 1 || k2 > RKV_MAX_K2) return RKV_EINVAL;
    return RKV_OK;
}

// Workspace of the decode family: [select candidates][attention partials]
// [page_idx when the caller passes none][split-K partials], each part sized
// for the plan the options give.
struct HsaWs {
    size_t select, attend, pages, split, total;
};
HsaWs hsa_ws(const rkv_gqa &g, int B, int P, int max_pages, int k2, const Knobs &kn) {
    HsaWs w;
    w.select = align_up(select_ws_bytes(g, B, max_pages, k2, kn));
    w.attend = align_up(attend_ws_bytes(g, B, P, k2, kn));
    w.pages = align_up((size_t)B * g.n_kv_heads * k2 * sizeof(int32_t));
    w.split = fused_split_ws_bytes(g, B, P, k2, kn);
    // +256 so that the size is never 0
    w.total = w.select + w.attend + w.pages + w.split + 256;
    return w;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per
// device), or nullptr with *st set on failure.
void *static_scratch(int *st) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *st = RKV_EHIP;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            *st = RKV_EHIP;
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char *rkv_status_string(int status) {
    switch (status) {
        case RKV_OK: return "ok";
        case RKV_EINVAL: return "invalid argument";
        case RKV_EWORKSPACE: return "workspace missing or too small";
        case RKV_ECAPACITY: return "rows do not fit the paged cache";
        case RKV_EUNSUPPORTED: return "unsupported shape or dtype";
        case RKV_EHIP: return "HIP launch error";
        case RKV_ESCRATCH: return "shapes need more than the static scratch holds";
    }
    return "unknown status";
}

const char *rkv_build_id(void) { return RKV_BUILD_ID; }

int rkv_split_ratio(double c, int64_t L, int64_t w, double *r, double *c_evict, double *c_hsa,
                    int64_t *keep) {
    if (!isfinite(c) || c < 1.0 || L < 0 || w < 0) return RKV_EINVAL;
    double rr = 0.2 + 0.06 * log2(c);
    rr = rr < 0.2 ? 0.2 : (rr > 0.8 ? 0.8 : rr);
    const double ce = pow(c, rr);
    if (r) *r = rr;
    if (c_evict) *c_evict = ce;
    if (c_hsa) *c_hsa = pow(c, 1.0 - rr);
    if (keep) {
        int64_t kk = (int64_t)floor((double)L / ce);
        if (kk < w) kk = w;
        if (kk > L) kk = L;
        *keep = kk;
    }
    return RKV_OK;
}

size_t rkv_prefill_evict_workspace_bytes(const rkv_gqa *g, int32_t B, int64_t L_max, int32_t w) {
    if (check_gqa(g) != RKV_OK || B < 1 || L_max < 1 || w < 1) return 0;
    return evict_ws_bytes(*g, B, L_max, w);
}

int rkv_prefill_evict(const rkv_gqa *g, int32_t dtype, int32_t B, const int32_t *prompt_lens,
                      const int32_t *keep, int64_t L_max, int32_t w, int32_t pool_kernel,
                      float scale, const void *q_win, const void *k, const void *v,
                      const rkv_paged_cache *cache, void *summaries, int32_t *kept_idx,
                      int32_t keep_stride, float *pooled_scores, int32_t *seq_lens_out,
                      void *ws, size_t ws_bytes, void *stream, const rkv_opts *opts) {
    clear_pending_error();
    int st = check_gqa(g);
    if (st != RKV_OK) return st;
    if ((st = check_dtype(dtype)) != RKV_OK) return st;
    if (B < 1 || !prompt_lens || !keep || !q_win || !k || !v) return RKV_EINVAL;
    if (B > RKV_MAX_EVICT_BATCH) return RKV_EUNSUPPORTED;
    if (L_max < 1 || L_max > ((int64_t)1 << 30) || w < 1 || pool_kernel < 1 ||
        (pool_kernel % 2) == 0)
        return RKV_EINVAL;
    if (!(scale > 0.0f) || !isfinite(scale)) return RKV_EINVAL;
    if (!aligned16(k) || !aligned16(v)) return RKV_EINVAL;
    if ((st = check_cache(g, cache)) != RKV_OK) return st;
    EvictSeq seq;
    memset(&seq, 0, sizeof seq);
    int64_t keep_rows = 0;
    for (int b = 0; b < B; ++b) {
        const int32_t L = prompt_lens[b], kp = keep[b];
        if (L < 0 || L > L_max || kp < 0) return RKV_EINVAL;
        if (kp < L && kp < w) return RKV_EINVAL;
        const int64_t ke = kp < L ? kp : L;
        if (ke > (int64_t)cache->max_pages * cache->page_size) return RKV_ECAPACITY;
        if (ke > keep_rows) keep_rows = ke;
        seq.L[b] = L;
        seq.keep[b] = kp;
    }
    if (kept_idx && keep_stride < keep_rows) return RKV_EINVAL;
    const size_t need = evict_ws_bytes(*g, B, L_max, w);
    if (!ws || ws_bytes < need) return RKV_EWORKSPACE;
    return launch_evict(*g, dtype, B, seq, L_max, w, pool_kernel, scale, q_win, k, v, *cache,
                        summaries, kept_idx, keep_stride, pooled_scores, seq_lens_out, ws,
                        knobs_of(opts).status, (hipStream_t)stream);
}

size_t rkv_prefill_evict_chunk_workspace_bytes(const rkv_gqa *g, int32_t B, int64_t L_max,
                                               int32_t w) {
    if (check_gqa(g) != RKV_OK || B < 1 || L_max < 1 || w < 1) return 0;
    return evict_chunk_ws_bytes(*g, B, L_max, w);
}

int rkv_prefill_evict_chunk(const rkv_gqa *g, int32_t dtype, int32_t B,
                            const int32_t *n_cached, const int32_t *chunk_lens,
                            const int32_t *keep, int64_t C_max, int32_t w,
                            int32_t pool_kernel, float scale, const void *q_win,
                            const void *k_chunk, const void *v_chunk,
                            const rkv_paged_cache *cache, void *summaries, int32_t *kept_idx,
                            int32_t keep_stride, float *pooled_scores, int32_t *seq_lens_out,
                            void *ws, size_t ws_bytes, void *stream, const rkv_opts *opts) {
    clear_pending_error();
    int st = check_gqa(g);
    if (st != RKV_OK) return st;
    if ((st = check_dtype(dtype)) != RKV_OK) return st;
    if (B < 1 || !n_cached || !chunk_lens || !keep || !q_win || !k_chunk || !v_chunk)
        return RKV_EINVAL;
    if (B > RKV_MAX_EVICT_BATCH) return RKV_EUNSUPPORTED;
    if (C_max < 1 || C_max > ((int64_t)1 << 30) || w < 1 || pool_kernel < 1 ||
        (pool_kernel % 2) == 0)
        return RKV_EINVAL;
    if (!(scale > 0.0f) || !isfinite(scale)) return RKV_EINVAL;
    if (!aligned16(k_chunk) || !aligned16(v_chunk)) return RKV_EINVAL;
    if ((st = check_cache(g, cache)) != RKV_OK) return st;
    const int64_t cap = (int64_t)cache->max_pages * cache->page_size;
    ChunkSeq cs;
    EvictSeq seq;
    memset(&cs, 0, sizeof cs);
    memset(&seq, 0, sizeof seq);
    int64_t L_max = 1, keep_rows = 0;
    for (int b = 0; b < B; ++b) {
        const int32_t nc = n_cached[b], cl = chunk_lens[b], kp = keep[b];
        if (nc < 0 || cl < 0 || cl > C_max || kp < 0) return RKV_EINVAL;
        if (nc > cap) return RKV_ECAPACITY;
        const int64_t L = (int64_t)nc + cl;
        if (L > 0x7fffffff) return RKV_EINVAL;
        if (kp < L && (kp < w || cl < w)) return RKV_EINVAL;
        const int64_t ke = kp < L ? kp : L;
        if (ke > cap) return RKV_ECAPACITY;
        if (ke > keep_rows) keep_rows = ke;
        if (L > L_max) L_max = L;
        cs.n_cached[b] = nc;
        cs.L[b] = (int32_t)L;
        seq.L[b] = (int32_t)L;
        seq.keep[b] = kp;
    }
    if (kept_idx && keep_stride < keep_rows) return RKV_EINVAL;
    const size_t need = evict_chunk_ws_bytes(*g, B, L_max, w);
    if (!ws || ws_bytes < need) return RKV_EWORKSPACE;
    return launch_evict_chunk(*g, dtype, B, cs, seq, L_max, C_max, w, pool_kernel, scale, q_win,
                              k_chunk, v_chunk, *cache, *cache, summaries, kept_idx, keep_stride,
                              pooled_scores, seq_lens_out, ws, knobs_of(opts).status,
                              (hipStream_t)stream);
}

size_t rkv_turn_filter_workspace_bytes(const rkv_gqa *g, int32_t B, int64_t L_max, int32_t w) {
    if (check_gqa(g) != RKV_OK || B < 1 || L_max < 1 || w < 1) return 0;
    return evict_chunk_ws_bytes(*g, B, L_max, w);
}

int rkv_turn_filter(const rkv_gqa *g, int32_t dtype, int32_t B, const int32_t *n_rows,
                    const int32_t *keep, int32_t w, int32_t pool_kernel, float scale,
                    const void *q_win, const rkv_paged_cache *full, const rkv_paged_cache *view,
                    void *view_summaries, int32_t *kept_idx, int32_t keep_stride,
                    float *pooled_scores, int32_t *view_lens_out, void *ws, size_t ws_bytes,
                    void *stream, const rkv_opts *opts) {
    clear_pending_error();
    int st = check_gqa(g);
    if (st != RKV_OK) return st;
    if ((st = check_dtype(dtype)) != RKV_OK) return st;
    if (B < 1 || !n_rows || !keep || !q_win) return RKV_EINVAL;
    if (B > RKV_MAX_EVICT_BATCH) return RKV_EUNSUPPORTED;
    if (w < 1 || pool_kernel < 1 || (pool_kernel % 2) == 0) return RKV_EINVAL;
    if (!(scale > 0.0f) || !isfinite(scale)) return RKV_EINVAL;
    if ((st = check_cache(g, full)) != RKV_OK) return st;
    if ((st = check_cache(g, view)) != RKV_OK) return st;
    const int64_t cap_full = (int64_t)full->max_pages * full->page_size;
    const int64_t cap_view = (int64_t)view->max_pages * view->page_size;
    ChunkSeq cs;
    EvictSeq seq;
    memset(&cs, 0, sizeof cs);
    memset(&seq, 0, sizeof seq);
    int64_t L_max = 1, keep_rows = 0;
    for (int b = 0; b < B; ++b) {
        const int32_t n = n_rows[b], kp = keep[b];
        if (n < 0 || kp < 0) return RKV_EINVAL;
        if (n > cap_full) return RKV_ECAPACITY;
        if (kp < n && (kp < w || n < w)) return RKV_EINVAL;
        const int64_t ke = kp < n ? kp : n;
        if (ke > cap_view) return RKV_ECAPACITY;
        if (ke > keep_rows) keep_rows = ke;
        if (n > L_max) L_max = n;
        cs.n_cached[b] = n;
        cs.L[b] = n;
        seq.L[b] = n;
        seq.keep[b] = kp;
    }
    if (kept_idx && keep_stride < keep_rows) return RKV_EINVAL;
    if (!ws || ws_bytes < evict_chunk_ws_bytes(*g, B, L_max, w)) return RKV_EWORKSPACE;
    return launch_evict_chunk(*g, dtype, B, cs, seq, L_max, 1, w, pool_kernel, scale, q_win,
                              nullptr, nullptr, *full, *view, view_summaries, kept_idx,
                              keep_stride, pooled_scores, view_lens_out, ws,
                              knobs_of(opts).status, (hipStream_t)stream);
}

int rkv_append_summaries(const rkv_gqa *g, int32_t dtype, int32_t B,
                         const rkv_paged_cache *cache, const int32_t *n_old,
                         const int32_t *n_new, int32_t max_new_rows, const void *k_src,
                         const void *v_src, void *summaries, void *stream,
                         const rkv_opts *opts) {
    clear_pending_error();
    int st = check_gqa(g);
    if (st != RKV_OK) return st;
    if ((st = check_dtype(dtype)) != RKV_OK) return st;
    if (B < 1 || B > 65535 || !n_old || !n_new || !summaries || max_new_rows < 1)
        return RKV_EINVAL;
    if ((st = check_cache(g, cache)) != RKV_OK) return st;
    if ((k_src == nullptr) != (v_src == nullptr)) return RKV_EINVAL;
    const int64_t pages = (int64_t)(max_new_rows + cache->page_size - 1) / cache->page_size + 1;
    if (pages > 0x7fffffff) return RKV_EINVAL;
    return launch_append(*g, dtype, B, *cache, n_old, n_new, max_new_rows, k_src, v_src,
                         summaries, knobs_of(opts).status, (hipStream_t)stream);
}

size_t rkv_hsa_workspace_bytes(const rkv_gqa *g, int32_t B, int32_t page_size,
                               int32_t max_pages, int32_t k1, int32_t k2,
                               const rkv_opts *opts) {
    (void)k1;
    if (check_gqa(g) != RKV_OK || B < 1 || page_size < 1 || max_pages < 1 || k2 < 1) return 0;
    return hsa_ws(*g, B, page_size, max_pages, k2, knobs_of(opts)).total;
}

int rkv_hsa_select(const rkv_gqa *g, int32_t dtype, int32_t B, const void *q,
                   const int32_t *seq_lens, int32_t page_size, int32_t max_pages,
                   const void *summaries, int32_t k1, int32_t k2, int32_t *chan_idx,
                   int32_t *page_idx, float *page_scores, void *ws, size_t ws_bytes,
                   void *stream, const rkv_opts *opts) {
    clear_pending_error();
    int st = check_select_args(g, dtype, B, q, seq_lens, page_size, max_pages, k1, k2);
    if (st != RKV_OK) return st;
    if (!summaries || !page_idx) return RKV_EINVAL;
    const Knobs kn = knobs_of(opts);
    if (!ws || ws_bytes < hsa_ws(*g, B, page_size, max_pages, k2, kn).total)
        return RKV_EWORKSPACE;
    return launch_select(*g, dtype, B, q, seq_lens, page_size, max_pages, (void *)summaries, k1,
                         k2, chan_idx, page_idx, page_scores, ws, nullptr, nullptr, nullptr, kn,
                         (hipStream_t)stream);
}

int rkv_hsa_attend(const rkv_gqa *g, int32_t dtype, int32_t B, const void *q,
                   const rkv_paged_cache *cache, const int32_t *seq_lens,
                   const int32_t *page_idx, int32_t k2, float scale, float *out, void *ws,
                   size_t ws_bytes, void *stream, const rkv_opts *opts) {
    clear_pending_error();
    int st = check_gqa(g);
    if (st != RKV_OK) return st;
    if ((st = check_cache(g, cache)) != RKV_OK) return st;
    st = check_select_args(g, dtype, B, q, seq_lens, cache->page_size, cache->max_pages, 1, k2);
    if (st != RKV_OK) return st;
    if (!page_idx || !out || !(scale > 0.0f) || !isfinite(scale)) return RKV_EINVAL;
    const Knobs kn = knobs_of(opts);
    const HsaWs w = hsa_ws(*g, B, cache->page_size, cache->max_pages, k2, kn);
    if (!ws || ws_bytes < w.total) return RKV_EWORKSPACE;
    return launch_attend(*g, dtype, B, q, *cache, seq_lens, page_idx, k2, scale, out,
                         (char *)ws + w.select, kn, (hipStream_t)stream);
}

int rkv_decode_mode(const rkv_gqa *g, int32_t dtype, int32_t B, int32_t page_size,
                    int32_t max_pages, int32_t k1, int32_t k2, const rkv_opts *opts) {
    int st = check_gqa(g);
    if (st != RKV_OK) return st;
    if (dtype != RKV_F32 && dtype != RKV_BF16) return RKV_EUNSUPPORTED;
    if (B < 1 || page_size < 1 || max_pages < 1 || k1 < 1 || k1 > g->head_dim || k2 < 1 ||
        k2 > RKV_MAX_K2)
        return RKV_EINVAL;
    return plan_fused(*g, dtype, B, page_size, max_pages, k1, k2, knobs_of(opts)).form;
}

int rkv_decode_step(const rkv_gqa *g, int32_t dtype, int32_t B, const void *q,
                    const void *k_new, const void *v_new, const rkv_paged_cache *cache,
                    const int32_t *seq_lens, void *summaries, int32_t k1, int32_t k2,
                    float scale, float *out, int32_t *chan_idx, int32_t *page_idx,
                    float *page_scores, void *ws, size_t ws_bytes, void *stream,
                    const rkv_opts *opts) {
    clear_pending_error();
    int st = check_gqa(g);
    if (st != RKV_OK) return st;
    if ((st = check_cache(g, cache)) != RKV_OK) return st;
    st = check_select_args(g, dtype, B, q, seq_lens, cache->page_size, cache->max_pages, k1, k2);
    if (st != RKV_OK) return st;
    if (!summaries || !out || !(scale > 0.0f) || !isfinite(scale)) return RKV_EINVAL;
    if ((k_new == nullptr) != (v_new == nullptr)) return RKV_EINVAL;
    const Knobs kn = knobs_of(opts);
    const HsaWs w = hsa_ws(*g, B, cache->page_size, cache->max_pages, k2, kn);
    if (!ws || ws_bytes < w.total) return RKV_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    char *base = (char *)ws;
    const FusedPlan fp = plan_fused(*g, dtype, B, cache->page_size, cache->max_pages, k1, k2, kn);
    if (fp.form != RKV_FORM_STANDALONE) {
        const size_t off = w.select + w.attend + w.pages;
        return launch_decode_fused(fp, *g, dtype, B, q, k_new, v_new, *cache, seq_lens, summaries,
                                   k1, k2, scale, out, chan_idx, page_idx, page_scores,
                                   (float *)(base + off), ws_bytes - off, kn, s);
    }
    if (!page_idx) page_idx = (int32_t *)(base + w.select + w.attend);
    // the select kernel appends the new token itself
    st = launch_select(*g, dtype, B, q, seq_lens, cache->page_size, cache->max_pages, summaries,
                       k1, k2, chan_idx, page_idx, page_scores, ws, k_new, v_new, cache, kn, s);
    if (st != RKV_OK) return st;
    return launch_attend(*g, dtype, B, q, *cache, seq_lens, page_idx, k2, scale, out,
                         base + w.select, kn, s);
}

int rkv_decode_step_static(const rkv_gqa *g, int32_t dtype, int32_t B, const void *q,
                           const void *k_new, const void *v_new, const rkv_paged_cache *cache,
                           const int32_t *seq_lens, void *summaries, int32_t k1, int32_t k2,
                           float scale, float *out, int32_t *chan_idx, int32_t *page_idx,
                           float *page_scores, void *stream, const rkv_opts *opts) {
    clear_pending_error();
    int st = check_gqa(g);
    if (st != RKV_OK) return st;
    if ((st = check_cache(g, cache)) != RKV_OK) return st;
    st = check_select_args(g, dtype, B, q, seq_lens, cache->page_size, cache->max_pages, k1, k2);
    if (st != RKV_OK) return st;
    const size_t need = hsa_ws(*g, B, cache->page_size, cache->max_pages, k2, knobs_of(opts)).total;
    if (need > (size_t)RKV_STATIC_SCRATCH_BYTES) return RKV_ESCRATCH;
    void *ws = static_scratch(&st);
    if (!ws) return st;
    return rkv_decode_step(g, dtype, B, q, k_new, v_new, cache, seq_lens, summaries, k1, k2, scale,
                           out, chan_idx, page_idx, page_scores, ws, need, stream, opts);
}

int rkv_hsa_decode(const rkv_gqa *g, int32_t dtype, int32_t B, const void *q,
                   const rkv_paged_cache *cache, const int32_t *seq_lens, const void *summaries,
                   int32_t k1, int32_t k2, float scale, float *out, int32_t *chan_idx,
                   int32_t *page_idx, float *page_scores, void *ws, size_t ws_bytes,
                   void *stream, const rkv_opts *opts) {
    return rkv_decode_step(g, dtype, B, q, nullptr, nullptr, cache, seq_lens, (void *)summaries,
                           k1, k2, scale, out, chan_idx, page_idx, page_scores, ws, ws_bytes,
                           stream, opts);
}

}  // extern "C"
