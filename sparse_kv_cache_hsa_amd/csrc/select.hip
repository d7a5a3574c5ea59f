// select.hip -- HSA selection: head-dimension channel choice, per-page bound
// scores and page top-k2.
//
// "RocketKV-adapted -- Two-Stage Compression", section "Where it sits": the
// attention score is approximated by SparQ-style top-magnitude channels along
// the head dimension combined with Quest-style page max/min summaries along
// the sequence, giving a per-page score bound ("Evidence": the bound holds
// for every in-page dot product); "Adaptation notes": whole pages, k2 of
// them, are selected.  The channel ranking sums |q| over the G query heads of
// the group, and the page score sums the per-head bounds in head order.
//
// Exactness: channel sums, products, max and sums are plain fp32 operations
// in a fixed order (channels ascending, then heads ascending, from +0), and
// this file is compiled without multiply-add contraction, so the scores are
// reproducible bit for bit.  Ranking uses a 32-bit order-preserving key with
// ties resolved to the lower index.
//
// Kernels
//   select_kernel : grid (chunks, Hkv, B), 256 threads.  Each block ranks the
//                   channels (cheap, repeated per chunk), scores one chunk of
//                   pages (one thread per page, k1 summary pairs each,
//                   coalesced along the page axis) and keeps the chunk's top
//                   k2.  With one chunk it writes page_idx directly.
//   merge_kernel  : grid (Hkv, B).  Top-k2 over the chunks' candidates, which
//                   are stored chunk-major in ascending page order, so the
//                   position order equals the page order for tie-breaking.
#include <stdlib.h>

#include "rkv_internal.h"

namespace rkv {
namespace {

constexpr int kSelBlock = 256;
constexpr int kMaxChunk = 2048;
constexpr int kChanBatch = 16;

template <typename T, int D, int G>
__global__ void __launch_bounds__(kSelBlock)
select_kernel(int Hkv, int P, int max_pages, int chunk, int n_chunks, const T *q,
              const int32_t *seq_lens, const T *summ, int k1, int k2, int32_t *chan_out,
              int32_t *page_out, float *score_out, uint32_t *cand_key, int32_t *cand_page) {
    constexpr int NW = kSelBlock / kWave;
    __shared__ float qs[G][D];
    __shared__ float a_s[D];
    __shared__ int ch_s[D];
    __shared__ uint32_t key_s[kMaxChunk];
    __shared__ uint32_t hist[256];
    __shared__ int wave_tot[NW];
    __shared__ int sh[2];

    const int b = blockIdx.z, h = blockIdx.y, ck = blockIdx.x, tid = threadIdx.x;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t cap = (int64_t)max_pages * P;
    const int64_t n = min<int64_t>(max<int64_t>(seq_lens[b], 0), cap);
    const int NP = (int)((n + P - 1) / P);

    for (int i = tid; i < G * D; i += kSelBlock)
        qs[i / D][i % D] = Elem<T>::ld(q, bh * G * D + i);
    __syncthreads();

    // channel ranking: a[c] = sum_j |q_j[c]|, j ascending, from +0
    if (tid < D) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < G; ++j) acc = acc + fabsf(qs[j][tid]);
        a_s[tid] = acc;
    }
    __syncthreads();
    bool pick = false;
    if (tid < D) {
        const float mine = a_s[tid];
        int rank = 0;
        for (int c2 = 0; c2 < D; ++c2) {
            const float o = a_s[c2];
            rank += (o > mine) || (o == mine && c2 < tid);
        }
        pick = rank < k1;
    }
    int n_pick;
    const int pos = block_excl_count<NW>(pick, wave_tot, n_pick);
    if (pick) ch_s[pos] = tid;
    __syncthreads();
    if (chan_out && ck == 0 && tid < k1) chan_out[bh * k1 + tid] = ch_s[tid];

    // page bound scores for this chunk
    const int p0 = ck * chunk;
    const int cnt = max(0, min(NP, p0 + chunk) - p0);
    const T *smax = summ + bh * 2 * D * max_pages;
    const T *smin = smax + (int64_t)D * max_pages;
    for (int pi = tid; pi < cnt; pi += kSelBlock) {
        const int p = p0 + pi;
        float s[G];
#pragma unroll
        for (int j = 0; j < G; ++j) s[j] = 0.0f;
        for (int i0 = 0; i0 < k1; i0 += kChanBatch) {
            float hi_v[kChanBatch], lo_v[kChanBatch];
            int cc[kChanBatch];
#pragma unroll
            for (int u = 0; u < kChanBatch; ++u) {
                const int i = i0 + u;
                cc[u] = ch_s[i < k1 ? i : 0];
                hi_v[u] = Elem<T>::ld(smax, (int64_t)cc[u] * max_pages + p);
                lo_v[u] = Elem<T>::ld(smin, (int64_t)cc[u] * max_pages + p);
            }
#pragma unroll
            for (int u = 0; u < kChanBatch; ++u) {
                if (i0 + u < k1) {
#pragma unroll
                    for (int j = 0; j < G; ++j) {
                        const float qc = qs[j][cc[u]];
                        const float hi = qc * hi_v[u];
                        const float lo = qc * lo_v[u];
                        s[j] = s[j] + (hi > lo ? hi : lo);
                    }
                }
            }
        }
        float tot = 0.0f;
#pragma unroll
        for (int j = 0; j < G; ++j) tot = tot + s[j];
        key_s[pi] = ordered_key(tot);
        if (score_out) score_out[bh * max_pages + p] = tot;
    }
    __syncthreads();

    const int K = min(k2, cnt);
    if (K > 0) {
        uint32_t thr;
        int take_eq;
        auto load = [&](int i) { return key_s[i]; };
        block_topk_threshold<kSelBlock>(load, cnt, K, hist, sh, thr, take_eq);
        if (n_chunks == 1) {
            int32_t *dst = page_out + bh * k2;
            block_topk_emit<kSelBlock>(load, cnt, thr, take_eq, wave_tot,
                                       [&](int o, int i) { dst[o] = p0 + i; });
        } else {
            const int64_t base = (bh * n_chunks + ck) * k2;
            block_topk_emit<kSelBlock>(load, cnt, thr, take_eq, wave_tot, [&](int o, int i) {
                cand_key[base + o] = key_s[i];
                cand_page[base + o] = p0 + i;
            });
        }
    }
    if (n_chunks == 1) {
        for (int o = K + tid; o < k2; o += kSelBlock) page_out[bh * k2 + o] = -1;
    } else {
        const int64_t base = (bh * n_chunks + ck) * k2;
        for (int o = K + tid; o < k2; o += kSelBlock) {
            cand_key[base + o] = 0u;  // below every finite score's key
            cand_page[base + o] = -1;
        }
    }
}

__global__ void __launch_bounds__(kSelBlock)
merge_kernel(int Hkv, int P, int max_pages, int n_chunks, const int32_t *seq_lens, int k2,
             const uint32_t *cand_key, const int32_t *cand_page, int32_t *page_out) {
    constexpr int NW = kSelBlock / kWave;
    __shared__ uint32_t hist[256];
    __shared__ int wave_tot[NW];
    __shared__ int sh[2];
    const int b = blockIdx.y, h = blockIdx.x;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t cap = (int64_t)max_pages * P;
    const int64_t n = min<int64_t>(max<int64_t>(seq_lens[b], 0), cap);
    const int NP = (int)((n + P - 1) / P);
    const int K = min(k2, NP);
    const int m = n_chunks * k2;
    const uint32_t *keys = cand_key + bh * m;
    const int32_t *pages = cand_page + bh * m;
    int32_t *dst = page_out + bh * k2;
    if (K > 0) {
        uint32_t thr;
        int take_eq;
        auto load = [&](int i) { return keys[i]; };
        block_topk_threshold<kSelBlock>(load, m, K, hist, sh, thr, take_eq);
        block_topk_emit<kSelBlock>(load, m, thr, take_eq, wave_tot,
                                   [&](int o, int i) { dst[o] = pages[i]; });
    }
    for (int o = K + threadIdx.x; o < k2; o += kSelBlock) dst[o] = -1;
}

template <typename T, int D, int G>
void launch_t(dim3 grid, hipStream_t s, int Hkv, int P, int max_pages, const SelectPlan &pl,
              const void *q, const int32_t *seq_lens, const void *summ, int k1, int k2,
              int32_t *chan_out, int32_t *page_out, float *score_out, uint32_t *ck,
              int32_t *cp) {
    select_kernel<T, D, G><<<grid, kSelBlock, 0, s>>>(
        Hkv, P, max_pages, pl.chunk_pages, pl.n_chunks, (const T *)q, seq_lens,
        (const T *)summ, k1, k2, chan_out, page_out, score_out, ck, cp);
}

template <typename T, int D>
bool dispatch_g(int G, dim3 grid, hipStream_t s, int Hkv, int P, int max_pages,
                const SelectPlan &pl, const void *q, const int32_t *seq_lens, const void *summ,
                int k1, int k2, int32_t *chan_out, int32_t *page_out, float *score_out,
                uint32_t *ck, int32_t *cp) {
    switch (G) {
        case 1: launch_t<T, D, 1>(grid, s, Hkv, P, max_pages, pl, q, seq_lens, summ, k1, k2, chan_out, page_out, score_out, ck, cp); return true;
        case 2: launch_t<T, D, 2>(grid, s, Hkv, P, max_pages, pl, q, seq_lens, summ, k1, k2, chan_out, page_out, score_out, ck, cp); return true;
        case 4: launch_t<T, D, 4>(grid, s, Hkv, P, max_pages, pl, q, seq_lens, summ, k1, k2, chan_out, page_out, score_out, ck, cp); return true;
        case 8: launch_t<T, D, 8>(grid, s, Hkv, P, max_pages, pl, q, seq_lens, summ, k1, k2, chan_out, page_out, score_out, ck, cp); return true;
    }
    return false;
}

int env_int(const char *name, int dflt) {
    const char *v = getenv(name);
    return (v && *v) ? atoi(v) : dflt;
}

}  // namespace

SelectPlan plan_select(const rkv_gqa &g, int B, int max_pages, int k2) {
    (void)k2;
    const int units = B * g.n_kv_heads;
    int chunk = env_int("RKV_SELECT_CHUNK", 0);
    if (chunk <= 0) {
        // Aim for >= 512 blocks (two per CU) while keeping >= 128 pages each.
        int want = (512 + units - 1) / units;
        int most = (max_pages + 127) / 128;
        int nch = want < most ? want : most;
        if (nch < 1) nch = 1;
        chunk = (max_pages + nch - 1) / nch;
    }
    chunk = (chunk + 63) / 64 * 64;
    if (chunk > kMaxChunk) chunk = kMaxChunk;
    if (chunk < 64) chunk = 64;
    SelectPlan p;
    p.chunk_pages = chunk;
    p.n_chunks = (max_pages + chunk - 1) / chunk;
    if (p.n_chunks < 1) p.n_chunks = 1;
    return p;
}

size_t select_ws_bytes(const rkv_gqa &g, int B, int max_pages, int k2) {
    const SelectPlan p = plan_select(g, B, max_pages, k2);
    if (p.n_chunks == 1) return 0;
    const size_t m = (size_t)B * g.n_kv_heads * p.n_chunks * k2;
    return align_up(m * sizeof(uint32_t)) + align_up(m * sizeof(int32_t));
}

int launch_select(const rkv_gqa &g, int dtype, int B, const void *q, const int32_t *seq_lens,
                  int P, int max_pages, const void *summaries, int k1, int k2,
                  int32_t *chan_idx, int32_t *page_idx, float *page_scores, void *ws,
                  hipStream_t s) {
    const SelectPlan pl = plan_select(g, B, max_pages, k2);
    uint32_t *ck = nullptr;
    int32_t *cp = nullptr;
    if (pl.n_chunks > 1) {
        const size_t m = (size_t)B * g.n_kv_heads * pl.n_chunks * k2;
        ck = (uint32_t *)ws;
        cp = (int32_t *)((char *)ws + align_up(m * sizeof(uint32_t)));
    }
    dim3 grid(pl.n_chunks, g.n_kv_heads, B);
    bool ok = false;
    const int d = g.head_dim;
    if (dtype == RKV_F32) {
        if (d == 64) ok = dispatch_g<float, 64>(g.group, grid, s, g.n_kv_heads, P, max_pages, pl, q, seq_lens, summaries, k1, k2, chan_idx, page_idx, page_scores, ck, cp);
        else if (d == 128) ok = dispatch_g<float, 128>(g.group, grid, s, g.n_kv_heads, P, max_pages, pl, q, seq_lens, summaries, k1, k2, chan_idx, page_idx, page_scores, ck, cp);
    } else {
        if (d == 64) ok = dispatch_g<uint16_t, 64>(g.group, grid, s, g.n_kv_heads, P, max_pages, pl, q, seq_lens, summaries, k1, k2, chan_idx, page_idx, page_scores, ck, cp);
        else if (d == 128) ok = dispatch_g<uint16_t, 128>(g.group, grid, s, g.n_kv_heads, P, max_pages, pl, q, seq_lens, summaries, k1, k2, chan_idx, page_idx, page_scores, ck, cp);
    }
    if (!ok) return RKV_EUNSUPPORTED;
    int st = launch_status();
    if (st != RKV_OK || pl.n_chunks == 1) return st;
    merge_kernel<<<dim3(g.n_kv_heads, B), kSelBlock, 0, s>>>(
        g.n_kv_heads, P, max_pages, pl.n_chunks, seq_lens, k2, ck, cp, page_idx);
    return launch_status();
}

}  // namespace rkv
