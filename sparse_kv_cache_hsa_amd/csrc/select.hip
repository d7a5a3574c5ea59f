// select.hip -- standalone HSA selection (channel ranking, page bound
// scores, page top-k2); the fused decode kernel covers the common case in one
// launch with the same device code (select_core.h), hence the same bits.
//
// Kernels
//   select_kernel : grid (chunks, Hkv, B), 256 threads.  Each block ranks the
//                   channels (cheap, repeated per chunk), scores one chunk of
//                   pages (one thread per page, coalesced along the page axis)
//                   and keeps the chunk's top k2.  With one chunk it writes
//                   page_idx directly.  For a decode step it also appends the
//                   new token: the block whose chunk holds row n-1 writes the
//                   K/V row, folds it into that page's summary and scores the
//                   page from the new summary (no other block reads it).
//   merge_sorted_kernel : grid (Hkv, B).  With several chunks of at most
//                   256 pages (and k2 <= 256), every block sorts its chunk's
//                   keys and writes its candidates in rank order; the merge
//                   folds the sorted lists pairwise (the bitonic top k2 of
//                   two lists per wave) and sorts the winners by page.
//   merge_kernel  : grid (Hkv, B).  Otherwise: a radix top-k2 over the
//                   chunks' candidates, which are stored chunk-major in
//                   ascending page order, so the position order equals the
//                   page order for tie-breaking.
#include <type_traits>

#include "select_core.h"

namespace rkv {
namespace {

constexpr int kSelBlock = 256;
constexpr int kMaxChunk = 2048;
constexpr int kStageBytes = 48 * 1024;  // staged summaries
// Sorted multi-chunk mode: a chunk holds at most one page per thread (256),
// a sorting network over the block gives the chunk's candidates in rank
// order, and the merge folds those sorted lists.  The select block's LDS
// (about 45 KB) lets three blocks share a CU.
constexpr int kSortedChunk = kSelBlock;
constexpr int kSortedStageBytes = 32 * 1024;
constexpr int kSortedMaxLists = 32;
constexpr int kSortedMaxCand = 4096;

struct SelArgs {
    int Hkv, P, max_pages, chunk, n_chunks, k1, k2;
    const int32_t *seq_lens;
    // decode-step append (k_new == nullptr: none)
    const void *k_new, *v_new;
    void *k_pool, *v_pool;
    const int32_t *page_table;
    int64_t num_blocks;
    int32_t *chan_out, *page_out;
    float *score_out;
    uint32_t *cand_key;
    int32_t *cand_page;
    int32_t *status;
};

// ---- bitonic lists held by one wave ----------------------------------------
// A list of L = E * 64 keys is held by one wave, key i = e * 64 + lane in
// v[e].  cx_stage is one compare-exchange stage at distance J: of each pair
// (i, i + J) the lower index keeps the larger key when up(i) holds, else the
// smaller one.
template <int E, int J, typename K, typename Up>
__device__ __forceinline__ void cx_stage(K (&v)[E], int lane, Up up) {
    if constexpr (J >= kWave) {
        constexpr int R = J / kWave;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if ((e & R) == 0) {
                const K a = v[e], b = v[e + R];
                const bool hi_first = up(e * kWave + lane);
                const K big = a > b ? a : b, small = a > b ? b : a;
                v[e] = hi_first ? big : small;
                v[e + R] = hi_first ? small : big;
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = bitonic_stage<J>(v[e], up(e * kWave + lane));
    }
}

// Half-cleaner cascade: sorts a bitonic list of L keys descending.
template <int E, int J, typename K>
__device__ __forceinline__ void list_clean(K (&v)[E], int lane) {
    cx_stage<E, J>(v, lane, [](int i) { return (i & J) == 0; });
    if constexpr (J > 1) list_clean<E, J / 2>(v, lane);
}

template <int E, int M, int J, typename K>
__device__ __forceinline__ void list_merge(K (&v)[E], int lane) {
    cx_stage<E, J>(v, lane, [](int i) { return ((i & M) == 0) == ((i & J) == 0); });
    if constexpr (J > 1) list_merge<E, M, J / 2>(v, lane);
}

// Full bitonic sort of L keys, descending.
template <int E, int M, typename K>
__device__ __forceinline__ void list_sort(K (&v)[E], int lane) {
    list_merge<E, M, M / 2>(v, lane);
    if constexpr (M < E * kWave) list_sort<E, M * 2>(v, lane);
}

// The K <= 256 largest of a chunk's 256 keys (key i held by thread i of
// the 4-wave block, 0 for pages past the chunk) in descending order:
// emit(r, key) for r < K.  Every wave sorts its 64 keys; waves 0 and 2 merge
// their neighbour's list into a sorted 128 (own list, then the other list
// reversed, is bitonic); wave 0 merges the two 128-lists the same way into
// all 256 keys, sorted.  buf: LDS of 256 keys.  All threads must call it;
// the caller synchronises the block before reusing buf.
template <typename Emit>
__device__ __forceinline__ void chunk_sorted_topk(uint64_t key, int K, uint64_t *buf, Emit emit) {
    static_assert(kSelBlock == 4 * kWave, "four waves");
    const int tid = threadIdx.x, w = tid / kWave, lane = tid & (kWave - 1);
    key = wave_sort_desc(key);
    buf[tid] = key;
    lds_barrier();
    if (w == 0 || w == 2) {
        uint64_t v[2];
        v[0] = key;
        v[1] = buf[(w + 1) * kWave + (kWave - 1 - lane)];
        list_clean<2, kWave>(v, lane);
        buf[w * kWave + lane] = v[0];
        buf[w * kWave + kWave + lane] = v[1];
    }
    lds_barrier();
    if (w == 0) {
        uint64_t v[4];
        v[0] = buf[lane];
        v[1] = buf[kWave + lane];
        v[2] = buf[4 * kWave - 1 - lane];
        v[3] = buf[3 * kWave - 1 - lane];
        list_clean<4, 2 * kWave>(v, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e * kWave + lane < K) emit(e * kWave + lane, v[e]);
    }
}

template <typename T, int D, int G, bool SORTED>
__global__ void __launch_bounds__(kSelBlock) select_kernel(SelArgs a, const T *q, T *summ) {
    constexpr int kChunkCap = SORTED ? kSortedChunk : kMaxChunk;
    constexpr int kStageCap = SORTED ? kSortedStageBytes : kStageBytes;
    constexpr int NW = kSelBlock / kWave;
    __shared__ float qs[G][D];
    __shared__ float qsel[G][D];
    __shared__ __align__(16) float qpm_s[D * 2 * G];
    constexpr bool kPacked = std::is_same<T, uint16_t>::value;
    __shared__ int ch_s[D];
    __shared__ T ovr_hi[D], ovr_lo[D];
    __shared__ uint64_t comp_s[kChunkCap];
    constexpr int kStageElems = kStageCap / (int)sizeof(T);
    __shared__ __align__(16) T stage[kStageElems];
    __shared__ int cnt_s[kSelBlock];
    __shared__ uint32_t hist[256];
    __shared__ int wave_tot[NW];
    __shared__ int sh[2];

    const int b = blockIdx.z, h = blockIdx.y, ck = blockIdx.x, tid = threadIdx.x;
    const int P = a.P, k1 = a.k1, k2 = a.k2;
    const int64_t bh = (int64_t)b * a.Hkv + h;
    const int64_t cap = (int64_t)a.max_pages * P;
    const int64_t n = clamp_rows(a.seq_lens[b], cap, (ck == 0 && h == 0 && tid == 0) ? a.status : nullptr);
    const int NP = (int)((n + P - 1) / P);

    const int p0 = ck * a.chunk;
    const int cnt = max(0, min(NP, p0 + a.chunk) - p0);
    T *smax = summ + bh * 2 * D * a.max_pages;
    T *smin = smax + (int64_t)D * a.max_pages;
    load_group_q<T, D, G, kSelBlock>(q, bh, qs);
    // the append, when this chunk holds row n-1 (first of equal values kept:
    // strict comparisons, as in a rebuild); after the query loads, which its
    // stores would otherwise hold back
    const int p_new = (a.k_new && n > 0) ? (int)((n - 1) / P) : -1;
    const bool app = p_new >= p0 && p_new < p0 + cnt;
    if (app && tid < D) {
        const int slot = (int)(n - 1 - (int64_t)p_new * P);
        const int64_t im = (int64_t)tid * a.max_pages + p_new;
        const T x = ((const T *)a.k_new)[bh * D + tid];
        T nmax = x, nmin = x;
        if (slot != 0) {
            const T omax = smax[im], omin = smin[im];
            const float fx = Elem<T>::ld(&x, 0);
            nmax = fx > Elem<T>::ld(&omax, 0) ? x : omax;
            nmin = fx < Elem<T>::ld(&omin, 0) ? x : omin;
        }
        ovr_hi[tid] = nmax;
        ovr_lo[tid] = nmin;
        const int32_t blk = a.page_table[(int64_t)b * a.max_pages + p_new];
        if (blk >= 0 && blk < a.num_blocks) {
            const int64_t dst = (((int64_t)blk * a.Hkv + h) * P + slot) * D + tid;
            ((T *)a.k_pool)[dst] = x;
            ((T *)a.v_pool)[dst] = ((const T *)a.v_new)[bh * D + tid];
            smax[im] = nmax;
            smin[im] = nmin;
        } else if (tid == 0) {
            report(a.status, RKV_DEV_BLOCK);
        }
    }
    lds_barrier();
    rank_channels_wave<D, G>(qs, k1, ch_s, qsel, kPacked ? qpm_s : nullptr);
    if (a.chan_out && ck == 0 && tid < k1) a.chan_out[bh * k1 + tid] = ch_s[tid];
    constexpr int V = 16 / (int)sizeof(T);
    if (2 * k1 * ((cnt + V - 1) / V * V) <= kStageElems) {
        const int npad = stage_summaries<T, kSelBlock>(smax, smin, a.max_pages, p0, cnt, ch_s, k1,
                                                       stage);
        lds_barrier();
        if (app && tid < k1) {
            const int c = ch_s[tid];
            const int pi = p_new - p0;
            stage[(int64_t)tid * npad + pi] = ovr_hi[c];
            stage[(int64_t)(k1 + tid) * npad + pi] = ovr_lo[c];
        }
        lds_barrier();
        // a full chunk of 256 pages with 32 channels: the row stride is the
        // constant 256, so the unrolled bound reads LDS at constant offsets
        const bool fixed = npad == kSortedChunk && k1 == 32 &&
                           (size_t)2 * 32 * kSortedChunk * sizeof(T) <= (size_t)kStageCap;
        for (int pi = tid; pi < cnt; pi += kSelBlock) {
            float s;
            if constexpr (kPacked)
                s = fixed ? staged_bound_fixed<G, 32, kSortedChunk>((const uint16_t *)stage, pi, qpm_s)
                          : staged_bound_exact<G>((const uint16_t *)stage, npad, pi, k1, qpm_s);
            else
                s = staged_bound<T, D, G>(stage, npad, pi, k1, qsel);
            comp_s[pi] = composite_key(ordered_key(s), pi);
            if (a.score_out) a.score_out[bh * a.max_pages + p0 + pi] = s;
        }
    } else {
        for (int pi = tid; pi < cnt; pi += kSelBlock) {
            const float s = app && p0 + pi == p_new
                                ? page_bound_ovr<T, D, G>(ch_s, k1, qsel, ovr_hi, ovr_lo)
                                : page_bound<T, D, G>(smax, smin, a.max_pages, p0 + pi, ch_s, k1, qsel);
            comp_s[pi] = composite_key(ordered_key(s), pi);
            if (a.score_out) a.score_out[bh * a.max_pages + p0 + pi] = s;
        }
    }
    lds_barrier();

    const int K = min(k2, cnt);
    if (a.n_chunks == 1) {
        int32_t *dst = a.page_out + bh * k2;
        topk_ascending<kSelBlock>(comp_s, cnt, K, cnt_s, hist, sh, wave_tot,
                                  [&](int o, int i) { dst[o] = p0 + i; });
        for (int o = K + tid; o < k2; o += kSelBlock) dst[o] = -1;
    } else if constexpr (SORTED) {
        // cnt <= kSelBlock: exact ranks, candidates stored in rank order
        // (score descending, then page ascending)
        const int64_t base = (bh * a.n_chunks + ck) * k2;
        const uint64_t key = tid < cnt ? comp_s[tid] : 0ull;
        lds_barrier();  // comp_s is reused as the merge buffer
        chunk_sorted_topk(key, K, comp_s, [&](int r, uint64_t kk) {
            a.cand_key[base + r] = (uint32_t)(kk >> 32);
            a.cand_page[base + r] = p0 + (int)~(uint32_t)kk;
        });
        for (int o = K + tid; o < k2; o += kSelBlock) {
            a.cand_key[base + o] = 0u;  // below every finite score's key
            a.cand_page[base + o] = -1;
        }
    } else {
        const int64_t base = (bh * a.n_chunks + ck) * k2;
        topk_ascending<kSelBlock>(comp_s, cnt, K, cnt_s, hist, sh, wave_tot, [&](int o, int i) {
            a.cand_key[base + o] = (uint32_t)(comp_s[i] >> 32);
            a.cand_page[base + o] = p0 + i;
        });
        for (int o = K + tid; o < k2; o += kSelBlock) {
            a.cand_key[base + o] = 0u;  // below every finite score's key
            a.cand_page[base + o] = -1;
        }
    }
}

// Top-k2 over the chunks' candidates of one (sequence, KV head): one block
// of 1,024 threads.  The candidate keys are copied to LDS once when they fit,
// so the four radix rounds and the ordered emit read LDS only.
constexpr int kMergeBlock = 1024;
constexpr int kMergeStage = 8192;  // candidate keys held in LDS

__global__ void __launch_bounds__(kMergeBlock)
merge_kernel(int Hkv, int P, int max_pages, int n_chunks, const int32_t *seq_lens, int k2,
             const uint32_t *cand_key, const int32_t *cand_page, int32_t *page_out) {
    constexpr int NW = kMergeBlock / kWave;
    __shared__ uint32_t hist[256];
    __shared__ int wave_tot[NW];
    __shared__ int sh[2];
    __shared__ uint32_t key_s[kMergeStage];
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
        auto emit = [&](int o, int i) { dst[o] = pages[i]; };
        if (m <= kMergeStage) {
            for (int i = threadIdx.x; i < m; i += kMergeBlock) key_s[i] = keys[i];
            lds_barrier();
            auto load = [&](int i) { return key_s[i]; };
            block_topk_threshold<kMergeBlock>(load, m, K, hist, sh, thr, take_eq);
            block_topk_emit<kMergeBlock>(load, m, thr, take_eq, wave_tot, emit);
        } else {
            auto load = [&](int i) { return keys[i]; };
            block_topk_threshold<kMergeBlock>(load, m, K, hist, sh, thr, take_eq);
            block_topk_emit<kMergeBlock>(load, m, thr, take_eq, wave_tot, emit);
        }
    }
    for (int o = K + threadIdx.x; o < k2; o += kMergeBlock) dst[o] = -1;
}

// Top-k2 over the chunks' rank-ordered candidates of one (sequence, KV
// head): one block of 1,024 threads.  As 64-bit keys (score key, then the
// complemented page) every list is descending and every real key is unique
// and nonzero (padding is 0).  Waves fold pairs of lists in rounds: the
// element-wise maximum of a descending list and a reversed one is bitonic and
// holds the L largest keys of both, which a half-cleaner cascade sorts.  The
// last list holds the top L; wave 0 sorts its first K by page and writes
// them in ascending order.
template <int E>
__global__ void __launch_bounds__(kMergeBlock)
merge_sorted_kernel(int Hkv, int P, int max_pages, int n_chunks, const int32_t *seq_lens, int k2,
                    const uint32_t *cand_key, const int32_t *cand_page, int32_t *page_out) {
    constexpr int L = E * kWave;
    __shared__ uint64_t buf[2][kSortedMaxCand];
    const int b = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
    const int w = tid / kWave, lane = tid & (kWave - 1);
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t cap = (int64_t)max_pages * P;
    const int64_t n = min<int64_t>(max<int64_t>(seq_lens[b], 0), cap);
    const int NP = (int)((n + P - 1) / P);
    const int K = min(k2, NP);
    const int m = n_chunks * k2;
    const uint32_t *keys = cand_key + bh * m;
    const int32_t *pages = cand_page + bh * m;
    int32_t *dst = page_out + bh * k2;
    for (int i = tid; i < n_chunks * L; i += kMergeBlock) {
        const int l = i / L, r = i - l * L;
        uint64_t ck = 0ull;
        if (r < k2) {
            const int j = l * k2 + r;
            ck = ((uint64_t)keys[j] << 32) | (uint64_t)(~(uint32_t)pages[j]);
        }
        buf[0][i] = ck;
    }
    int src = 0, nl = n_chunks;
    while (nl > 1) {
        lds_barrier();
        const int half = (nl + 1) / 2;
        if (w < half) {
            uint64_t v[E];
#pragma unroll
            for (int e = 0; e < E; ++e) v[e] = buf[src][(2 * w) * L + e * kWave + lane];
            if (2 * w + 1 < nl) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const uint64_t o = buf[src][(2 * w + 1) * L + (L - 1) - (e * kWave + lane)];
                    v[e] = o > v[e] ? o : v[e];
                }
                list_clean<E, L / 2>(v, lane);
            }
#pragma unroll
            for (int e = 0; e < E; ++e) buf[1 - src][w * L + e * kWave + lane] = v[e];
        }
        src = 1 - src;
        nl = half;
    }
    lds_barrier();
    if (w == 0) {
        // ~page of the K winners, sorted descending = page ascending; the
        // other slots carry 0 and sort last
        uint32_t inv[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = e * kWave + lane;
            inv[e] = i < K ? (uint32_t)buf[src][i] : 0u;
        }
        list_sort<E, 2>(inv, lane);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = e * kWave + lane;
            if (i < K) dst[i] = (int)~inv[e];
        }
    }
    for (int o = K + tid; o < k2; o += kMergeBlock) dst[o] = -1;
}

template <typename T, int D, int G>
void launch_t(dim3 grid, bool sorted, hipStream_t s, const SelArgs &a, const void *q, void *summ) {
    if (sorted)
        select_kernel<T, D, G, true><<<grid, kSelBlock, 0, s>>>(a, (const T *)q, (T *)summ);
    else
        select_kernel<T, D, G, false><<<grid, kSelBlock, 0, s>>>(a, (const T *)q, (T *)summ);
}

template <typename T, int D>
bool dispatch_g(int G, dim3 grid, bool sorted, hipStream_t s, const SelArgs &a, const void *q,
                void *summ) {
    switch (G) {
        case 1: launch_t<T, D, 1>(grid, sorted, s, a, q, summ); return true;
        case 2: launch_t<T, D, 2>(grid, sorted, s, a, q, summ); return true;
        case 4: launch_t<T, D, 4>(grid, sorted, s, a, q, summ); return true;
        case 8: launch_t<T, D, 8>(grid, sorted, s, a, q, summ); return true;
    }
    return false;
}

}  // namespace

SelectPlan plan_select(const rkv_gqa &g, int B, int max_pages, int k2, const Knobs &kn) {
    const int units = B * g.n_kv_heads;
    int chunk = kn.select_chunk;
    if (chunk <= 0) {
        // One block per (sequence, head) when the batch fills the chip;
        // otherwise aim for >= 512 blocks of >= 128 pages each.
        int want = units >= 192 ? 1 : (512 + units - 1) / units;
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
    p.sorted = 0;
    if (p.n_chunks > 1 && k2 <= 4 * kWave && kn.select_radix == 0) {
        // elements per lane of a merge list: k2 rounded up to 64, 128 or 256
        const int E = k2 <= kWave ? 1 : (k2 <= 2 * kWave ? 2 : 4);
        const int sc = chunk < kSortedChunk ? chunk : kSortedChunk;
        const int nch = (max_pages + sc - 1) / sc;
        if (nch > 1 && nch <= kSortedMaxLists && nch * E * kWave <= kSortedMaxCand) {
            p.chunk_pages = sc;
            p.n_chunks = nch;
            p.sorted = E;
        }
    }
    return p;
}

size_t select_ws_bytes(const rkv_gqa &g, int B, int max_pages, int k2, const Knobs &kn) {
    const SelectPlan p = plan_select(g, B, max_pages, k2, kn);
    if (p.n_chunks == 1) return 0;
    const size_t m = (size_t)B * g.n_kv_heads * p.n_chunks * k2;
    return align_up(m * sizeof(uint32_t)) + align_up(m * sizeof(int32_t));
}

int launch_select(const rkv_gqa &g, int dtype, int B, const void *q, const int32_t *seq_lens,
                  int P, int max_pages, void *summaries, int k1, int k2,
                  int32_t *chan_idx, int32_t *page_idx, float *page_scores, void *ws,
                  const void *k_new, const void *v_new, const rkv_paged_cache *cache,
                  const Knobs &kn, hipStream_t s) {
    const SelectPlan pl = plan_select(g, B, max_pages, k2, kn);
    SelArgs a;
    a.Hkv = g.n_kv_heads;
    a.P = P;
    a.max_pages = max_pages;
    a.chunk = pl.chunk_pages;
    a.n_chunks = pl.n_chunks;
    a.k1 = k1;
    a.k2 = k2;
    a.seq_lens = seq_lens;
    a.chan_out = chan_idx;
    a.page_out = page_idx;
    a.score_out = page_scores;
    a.cand_key = nullptr;
    a.cand_page = nullptr;
    a.k_new = cache ? k_new : nullptr;
    a.v_new = v_new;
    a.k_pool = cache ? cache->k_pool : nullptr;
    a.v_pool = cache ? cache->v_pool : nullptr;
    a.page_table = cache ? cache->page_table : nullptr;
    a.num_blocks = cache ? cache->num_blocks : 0;
    a.status = kn.status;
    if (pl.n_chunks > 1) {
        const size_t m = (size_t)B * g.n_kv_heads * pl.n_chunks * k2;
        a.cand_key = (uint32_t *)ws;
        a.cand_page = (int32_t *)((char *)ws + align_up(m * sizeof(uint32_t)));
    }
    dim3 grid(pl.n_chunks, g.n_kv_heads, B);
    bool ok = false;
    const int d = g.head_dim;
    if (dtype == RKV_F32) {
        if (d == 64) ok = dispatch_g<float, 64>(g.group, grid, pl.sorted != 0, s, a, q, summaries);
        else if (d == 128) ok = dispatch_g<float, 128>(g.group, grid, pl.sorted != 0, s, a, q, summaries);
    } else {
        if (d == 64) ok = dispatch_g<uint16_t, 64>(g.group, grid, pl.sorted != 0, s, a, q, summaries);
        else if (d == 128) ok = dispatch_g<uint16_t, 128>(g.group, grid, pl.sorted != 0, s, a, q, summaries);
    }
    if (!ok) return RKV_EUNSUPPORTED;
    int st = launch_status();
    if (st != RKV_OK || pl.n_chunks == 1) return st;
    const dim3 mgrid(g.n_kv_heads, B);
    if (pl.sorted == 1)
        merge_sorted_kernel<1><<<mgrid, kMergeBlock, 0, s>>>(
            g.n_kv_heads, P, max_pages, pl.n_chunks, seq_lens, k2, a.cand_key, a.cand_page, page_idx);
    else if (pl.sorted == 2)
        merge_sorted_kernel<2><<<mgrid, kMergeBlock, 0, s>>>(
            g.n_kv_heads, P, max_pages, pl.n_chunks, seq_lens, k2, a.cand_key, a.cand_page, page_idx);
    else if (pl.sorted == 4)
        merge_sorted_kernel<4><<<mgrid, kMergeBlock, 0, s>>>(
            g.n_kv_heads, P, max_pages, pl.n_chunks, seq_lens, k2, a.cand_key, a.cand_page, page_idx);
    else
        merge_kernel<<<dim3(g.n_kv_heads, B), kMergeBlock, 0, s>>>(
            g.n_kv_heads, P, max_pages, pl.n_chunks, seq_lens, k2, a.cand_key, a.cand_page, page_idx);
    return launch_status();
}

}  // namespace rkv
