// decode.hip -- one decode step of one layer in a single launch: append the
// new token (K/V row and its page summary), rank channels, score pages, pick
// the top-k2 pages and attend over them.
//
// The steps are those of RocketKV's decode path ("RocketKV-adapted --
// Two-Stage Compression": "Where it sits" for the two-dimensional score bound,
// "Adaptation notes" for whole-page selection, "Evidence" for the incremental
// summary update).  One block of 16 waves (8 for groups of 8 query heads)
// owns one (sequence, KV head): the
// chosen channels, page scores and page list never leave LDS, and the block's
// attention phase starts as soon as its own selection is done, so a layer
// costs one launch and one dependent chain of memory round trips instead of
// a chain of kernels.  Selection uses the same device code as the standalone
// kernels (select_core.h), so its bits are identical; attention uses the
// streaming core (attend_core.h).
//
// Used when the batch fills the chip (enough (sequence, head) units for
// every CU) and the shapes fit LDS.  For smaller batches the split-K variant
// runs S blocks per unit: every block makes the same selection (the unit's
// summaries are small and stay in L2), streams 1/S of the selected pages and
// writes a partial (max, sum, acc) that the attention merge kernel combines
// in split order; block 0 of a unit writes the appended row, the summary and
// the index outputs.  Two launches per step instead of four.  Otherwise the
// standalone select (which appends the token) and attention kernels run in
// sequence.
#include <type_traits>

#include "attend_core.h"
#include "select_core.h"

namespace rkv {
namespace {

constexpr int kNW = 16;
constexpr int fused_waves(int G) { return G > 4 ? 8 : kNW; }
constexpr int kFusedMaxPages = 2048;
constexpr int kFusedMaxRows = 2048;
constexpr size_t kStageBytes = 64 * 1024;
constexpr int kSplitBlocks = 128;
constexpr int kSplitBlocksWide = 256;

constexpr size_t cmax(size_t x, size_t y) { return x > y ? x : y; }

struct DecArgs {
    int Hkv, P, max_pages, k1, k2;
    int64_t num_blocks;
    const int32_t *page_table, *seq_lens;
    float qscale;
    float *out;
    int32_t *chan_out, *page_out;
    float *score_out;
    float *part;  // split-K: [B][Hkv][n_splits][G][D + 2] partials
    int pps;      // split-K: selected pages per split
    int32_t *status;
    uint64_t *trace;  // RKV_PHASE_TIMING builds: RKV_TRACE_SLOTS stamps per block
};

// Phase stamps (RKV_PHASE_TIMING builds only): thread 0 of the block, or lane
// 0 of a wave, writes the constant-rate wall clock into its slot.
#ifdef RKV_PHASE_TIMING
#define RKV_STAMP(cond, slot)                                                          \
    do {                                                                               \
        if (a.trace && (cond))                                                         \
            a.trace[(((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x +     \
                     blockIdx.x) * RKV_TRACE_SLOTS + (slot)] = wall_clock64();         \
    } while (0)
#else
#define RKV_STAMP(cond, slot) \
    do {                      \
    } while (0)
#endif

// NW waves per block: 16, or 8 for groups of 8 query heads (their attention
// state needs twice the registers and LDS per wave).
template <typename T, int D, int G, bool SPLIT, int NW>
__global__ void __launch_bounds__(NW *kWave)
decode_kernel(DecArgs a, const T *q, const T *k_new, const T *v_new, T *k_pool, T *v_pool,
              T *summ) {
    constexpr int kBlock = NW * kWave;
    // The stream runs on the first half of the waves (the two oldest of
    // each SIMD) with four rows per lane per iteration: as many bytes in
    // flight as sixteen waves with two rows, with two age tiers to balance
    // instead of four (measurably faster).
    constexpr int NWS = NW == 16 ? 8 : NW;
    using Core = AttendCore<T, D, G, NWS, NW == 16 ? 4 : 2, false>;
    constexpr size_t kKeyBytes = sizeof(uint64_t) * kFusedMaxPages;
    constexpr size_t kUnion = cmax(kStageBytes, kKeyBytes);
    __shared__ float qs[G][D];
    __shared__ float qsel[G][D];
    __shared__ __align__(16) float qpm_s[D * 2 * G];
    constexpr bool kPacked = std::is_same<T, uint16_t>::value;
    __shared__ int ch_s[D];
    __shared__ T ovr_hi[D], ovr_lo[D];
    // the selected pages: K = min(k2, NP) <= max_pages <= kFusedMaxPages
    __shared__ int32_t sel_s[kFusedMaxPages];
    __shared__ int32_t blk_s[kFusedMaxPages];
    __shared__ int cnt_s[kBlock];
    __shared__ uint32_t pkey_s[kBlock];  // page score keys of the staged path's top-k
    __shared__ uint32_t hist[256];
    __shared__ int wave_tot[NW];
    __shared__ int sh[2];
    // staged summaries or page keys (selection): never live at the same
    // time
    __shared__ __align__(16) unsigned char u_s[kUnion];
    T *stage = (T *)u_s;
    uint64_t *comp_s = (uint64_t *)u_s;
    // the waves' partial attention states have LDS of their own, so a wave
    // stores its state as soon as its own rows are done while other waves
    // still stream
    __shared__ typename Core::Shared csh;

    const int sp = SPLIT ? blockIdx.x : 0, nsp = SPLIT ? gridDim.x : 1;
    const int h = SPLIT ? blockIdx.y : blockIdx.x, b = SPLIT ? blockIdx.z : blockIdx.y;
    const int tid = threadIdx.x;
    const bool lead = sp == 0;  // writes the append and the index outputs
    const int P = a.P, k1 = a.k1, k2 = a.k2, max_pages = a.max_pages;
    const int64_t bh = (int64_t)b * a.Hkv + h;
    const int64_t cap = (int64_t)max_pages * P;
    const int64_t n = clamp_rows(a.seq_lens[b], cap, (lead && h == 0 && tid == 0) ? a.status : nullptr);
    const int NP = (int)((n + P - 1) / P);
    T *sm_max = summ + bh * 2 * D * max_pages;
    T *sm_min = sm_max + (int64_t)D * max_pages;

    const bool append = k_new != nullptr && n > 0;
    const int p_new = append ? (int)((n - 1) / P) : -1;
    const int slot = append ? (int)(n - 1 - (int64_t)p_new * P) : 0;
    const int64_t im = (int64_t)tid * max_pages + p_new;
    const int K = min(k2, NP);
    constexpr int V = 16 / (int)sizeof(T);
    const bool staged = (size_t)2 * k1 * ((NP + V - 1) / V * V) * sizeof(T) <= kStageBytes &&
                        NP <= kBlock;

    // 1. the loads that do not depend on the row count: the new K/V row and
    //    the queries (they share a memory round trip with the row count).
    T x{}, vx{};
    if (k_new != nullptr && tid < D) {
        x = k_new[bh * D + tid];
        vx = v_new[bh * D + tid];
    }
    RKV_STAMP(tid == 0, 0);
    load_group_q<T, D, G, kBlock>(q, bh, qs);
    lds_barrier();
    RKV_STAMP(tid == 0, 1);

    // 2. channels.  The page-table row and the appended page's old summary
    //    (which depend on the row count) are loaded into registers
    //    meanwhile.
    int32_t pt = 0;
    T omax{}, omin{};
    if (staged) {
        if (tid < NP) pt = a.page_table[(int64_t)b * max_pages + tid];
        if (append && tid < D && slot != 0) {
            omax = sm_max[im];
            omin = sm_min[im];
        }
    }
    rank_channels_wave<D, G>(qs, k1, ch_s, qsel, kPacked ? qpm_s : nullptr);
    RKV_STAMP(tid == 0, 2);
    if (a.chan_out && lead && tid < k1) a.chan_out[bh * k1 + tid] = ch_s[tid];

    // 3. the appended row is folded into its page's summary (first of equal
    //    values kept: strict comparisons, as in a rebuild) and stored; when
    //    they fit, the summaries of the chosen channels are copied to LDS
    //    (the second memory round trip) and the appended page's column is
    //    replaced there by its new summary.
    // 4. page bounds and page top-k2.
    auto emit = [&](int o, int i) { sel_s[o] = i; };
    auto fold = [&](T xv, T omax, T omin, T &nmax, T &nmin) {
        nmax = xv;
        nmin = xv;
        if (slot != 0) {
            const float fx = Elem<T>::ld(&xv, 0);
            nmax = fx > Elem<T>::ld(&omax, 0) ? xv : omax;
            nmin = fx < Elem<T>::ld(&omin, 0) ? xv : omin;
        }
    };
    // The kernel's own results (the appended row and summary, the output, the
    // page list) are written through to memory: the summary append alone
    // touches one cache line per channel, and dirty lines left in L2 are
    // written back at the end of the launch, before the next layer's kernel
    // can start (measured: about 3.6 us per launch).
    auto store_append = [&](T nmax, T nmin) {
        const int32_t blk = blk_s[p_new];
        if (lead && blk >= 0 && blk < a.num_blocks) {
            const int64_t dst = (((int64_t)blk * a.Hkv + h) * P + slot) * D + tid;
            store_through(&k_pool[dst], x);
            store_through(&v_pool[dst], vx);
            store_through(&sm_max[im], nmax);
            store_through(&sm_min[im], nmin);
        } else if (lead && tid == 0) {
            report(a.status, RKV_DEV_BLOCK);
        }
    };
    // bf16 with 32 channels and up to 512 pages: the staged rows sit at a
    // fixed stride of 512 pages, so the bound loop (unrolled over the 32
    // channels) reads LDS at constant offsets with no address arithmetic
    constexpr int kSR = kWave * V;
    const bool fixed = kPacked && staged && k1 == 32 && NP <= kSR && max_pages % V == 0 &&
                       (((uintptr_t)sm_max) & 15u) == 0 && (((uintptr_t)sm_min) & 15u) == 0;
    if (staged) {
        int npad;
        if (fixed) {
            // one wave per summary row: row r (the max rows of the k1
            // channels, then the min rows) lands at stage + r * kSR, lane l's
            // 16-byte chunk at l * V within it
            const int lane = tid & (kWave - 1), nv = (NP + V - 1) / V;
            for (int row = tid / kWave; row < 2 * k1; row += NW) {
                const int kind = row >= k1, i = row - kind * k1;
                if (lane < nv) {
                    const T *src = (kind ? sm_min : sm_max) + (int64_t)ch_s[i] * max_pages + lane * V;
                    lds_load16_nt(src, stage + row * kSR);
                }
            }
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            npad = kSR;
        } else {
            npad = stage_summaries<T, kBlock>(sm_max, sm_min, max_pages, 0, NP, ch_s, k1, stage);
        }
        if (tid < NP) blk_s[tid] = pt;
        if (append && tid < D) {
            T nmax, nmin;
            fold(x, omax, omin, nmax, nmin);
            ovr_hi[tid] = nmax;
            ovr_lo[tid] = nmin;
        }
        lds_barrier();
        if (append && tid < D) store_append(ovr_hi[tid], ovr_lo[tid]);
        if (append && tid < k1) {
            const int c = ch_s[tid];
            stage[(int64_t)tid * npad + p_new] = ovr_hi[c];
            stage[(int64_t)(k1 + tid) * npad + p_new] = ovr_lo[c];
        }
        lds_barrier();
        RKV_STAMP(tid == 0, 3);
        // every page's score key to LDS (0 past the last page: below every
        // real key), then the first wave picks the top K in page order
        uint32_t skey = 0u;
        if (tid < NP) {
            float sc;
            if constexpr (kPacked)
                sc = fixed ? staged_bound_fixed<G, 32, kSR>((const uint16_t *)stage, tid, qpm_s)
                           : staged_bound_exact<G>((const uint16_t *)stage, npad, tid, k1, qpm_s);
            else
                sc = staged_bound<T, D, G>(stage, npad, tid, k1, qsel);
            skey = ordered_key(sc);
            if (a.score_out && lead) a.score_out[bh * max_pages + tid] = sc;
        }
        pkey_s[tid] = skey;
        lds_barrier();
        RKV_STAMP(tid == 0, 24);
        if (K > 0 && tid < kWave) wave_topk_lds(pkey_s, NP, K, emit);
    } else {
        for (int p = tid; p < NP; p += kBlock) blk_s[p] = a.page_table[(int64_t)b * max_pages + p];
        if (append && tid < D && slot != 0) {
            omax = sm_max[im];
            omin = sm_min[im];
        }
        lds_barrier();
        if (append && tid < D) {
            T nmax, nmin;
            fold(x, omax, omin, nmax, nmin);
            ovr_hi[tid] = nmax;
            ovr_lo[tid] = nmin;
            store_append(nmax, nmin);
        }
        lds_barrier();
        for (int p = tid; p < NP; p += kBlock) {
            float sc = page_bound<T, D, G>(sm_max, sm_min, max_pages, p, ch_s, k1, qsel);
            if (p == p_new) sc = page_bound_ovr<T, D, G>(ch_s, k1, qsel, ovr_hi, ovr_lo);
            comp_s[p] = composite_key(ordered_key(sc), p);
            if (a.score_out && lead) a.score_out[bh * max_pages + p] = sc;
        }
        lds_barrier();
        topk_ascending<kBlock>(comp_s, NP, K, cnt_s, hist, sh, wave_tot, emit);
    }
    Core core;
    core.init_lds(qs, a.qscale);
    // The full barrier makes the page list visible and the appended K/V row
    // (a global store of this block) visible to every wave before any of
    // them reads it.
    __syncthreads();
    RKV_STAMP(tid == 0, 4);

    // 5. stream the rows of the selected pages; each wave resolves its own
    //    rows from the page list as it goes.
    // (split-K: this block's share of the page list, pages [i0, i1))
    const int i0 = SPLIT ? min(K, sp * a.pps) : 0, i1 = SPLIT ? min(K, i0 + a.pps) : K;
    const int nrows = (i1 - i0) * P;
    // (checked by the waves that do not stream, when there are such)
    constexpr int kChk0 = NWS < NW ? NWS * kWave : 0;
    if (tid >= kChk0)
        for (int o = tid - kChk0; o < i1 - i0; o += kBlock - kChk0) {
            const int32_t blk = blk_s[sel_s[i0 + o]];
            if (blk < 0 || blk >= a.num_blocks) report(a.status, RKV_DEV_BLOCK);
        }
    // page size a power of two: shifts instead of divisions; row units in
    // 32 bits (the pool holds fewer than 2^32 rows)
    const int pshift = (P & (P - 1)) == 0 ? __builtin_ctz(P) : -1;
    const uint32_t rows_per_blk = (uint32_t)(a.Hkv * P), row_h = (uint32_t)(h * P);
    auto rowfn = [&](int f) -> uint32_t {
        int pi, sl;
        if (pshift >= 0) {
            pi = f >> pshift;
            sl = f & (P - 1);
        } else {
            pi = f / P;
            sl = f - pi * P;
        }
        const int32_t pg = sel_s[i0 + pi];
        const int32_t blk = blk_s[pg];
        if ((int64_t)pg * P + sl >= n || blk < 0 || blk >= a.num_blocks) return kBadRow;
        return (uint32_t)blk * rows_per_blk + row_h + (uint32_t)sl;
    };
    if constexpr (SPLIT) {
        // the lead block's store of the appended row may land after this
        // block reads it, so a block whose share holds that row writes the
        // same bytes itself
        if (!lead && append && tid < D) {
            bool mine = false;
            for (int pi = i0; pi < i1; ++pi) mine |= sel_s[pi] == p_new;
            const int32_t blk = blk_s[p_new];
            if (mine && blk >= 0 && blk < a.num_blocks) {
                const int64_t dst = (((int64_t)blk * a.Hkv + h) * P + slot) * D + tid;
                store_through(&k_pool[dst], x);
                store_through(&v_pool[dst], vx);
            }
        }
    }
    if constexpr (SPLIT) __syncthreads();  // the row written just above
    RKV_STAMP(tid == 0, 5);
    // (the older wave of each SIMD pair takes 56 % of their rows: the split
    // at which both finish together, measured)
    if (tid < NWS * kWave) core.template stream_fn<56>(nrows, k_pool, v_pool, rowfn);
    RKV_STAMP((tid & (kWave - 1)) == 0, 6 + tid / kWave);
    if (tid < NWS * kWave) core.to_shared(csh);
    lds_barrier();
    if constexpr (SPLIT) {
        float *base = a.part + (bh * nsp + sp) * G * (D + 2);
        Core::combine(csh, [&](int j, int c, float M, float Ls, float A0, float A1) {
            float *pp = base + j * (D + 2);
            pp[c] = A0;
            pp[c + 1] = A1;
            if (c == 0) {
                pp[D] = M;
                pp[D + 1] = Ls;
            }
        });
    } else {
        Core::combine(csh, [&](int j, int c, float M, float Ls, float A0, float A1) {
            float *o = a.out + (bh * G + j) * D + c;
            store_through(&o[0], Ls > 0.0f ? A0 / Ls : 0.0f);
            store_through(&o[1], Ls > 0.0f ? A1 / Ls : 0.0f);
        });
    }
    // the page list goes out last: stored earlier, it would hold up the full
    // barrier before the stream (which waits for this wave's stores)
    if (a.page_out && lead)
        for (int o = tid; o < k2; o += kBlock)
            store_through(&a.page_out[bh * k2 + o], o < K ? sel_s[o] : -1);
#ifdef RKV_PHASE_TIMING
    lds_barrier();
    RKV_STAMP(tid == 0, 22);
    // XCC_ID hardware register (id 20), bits [3:0]
    if (a.trace && tid == 0)
        a.trace[(((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) *
                    RKV_TRACE_SLOTS + 23] =
            (uint64_t)(__builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & 15);
#endif
}

template <typename T, int D, int G>
void launch_t(int B, int nsp, const rkv_gqa &g, const DecArgs &a, const void *q,
              const void *k_new, const void *v_new, const rkv_paged_cache &c, void *summ,
              hipStream_t s) {
    constexpr int NW = fused_waves(G);
    if (nsp > 0)
        decode_kernel<T, D, G, true, NW><<<dim3(nsp, g.n_kv_heads, B), NW * kWave, 0, s>>>(
            a, (const T *)q, (const T *)k_new, (const T *)v_new, (T *)c.k_pool, (T *)c.v_pool,
            (T *)summ);
    else
        decode_kernel<T, D, G, false, NW><<<dim3(g.n_kv_heads, B), NW * kWave, 0, s>>>(
            a, (const T *)q, (const T *)k_new, (const T *)v_new, (T *)c.k_pool, (T *)c.v_pool,
            (T *)summ);
}

template <typename T, int D>
bool dispatch_g(int B, int nsp, const rkv_gqa &g, const DecArgs &a, const void *q,
                const void *k_new, const void *v_new, const rkv_paged_cache &c, void *summ,
                hipStream_t s) {
    switch (g.group) {
        case 1: launch_t<T, D, 1>(B, nsp, g, a, q, k_new, v_new, c, summ, s); return true;
        case 2: launch_t<T, D, 2>(B, nsp, g, a, q, k_new, v_new, c, summ, s); return true;
        case 4: launch_t<T, D, 4>(B, nsp, g, a, q, k_new, v_new, c, summ, s); return true;
        case 8: launch_t<T, D, 8>(B, nsp, g, a, q, k_new, v_new, c, summ, s); return true;
    }
    return false;
}

// Split-K shape: about `target` blocks in all, whole pages per split, and at
// most kFusedMaxRows rows per split (the stream share one block takes on).
// The default target is kSplitBlocks; selections of more than
// kSplitBlocks * 512 rows in all (a stream that is bandwidth work, not
// latency) take one block per CU instead.
void split_counts(int units, int k2, int P, int target, int &n_splits, int &pages_per_split) {
    if (target <= 0)
        target = (int64_t)units * k2 * P > (int64_t)kSplitBlocks * 512 ? kSplitBlocksWide
                                                                       : kSplitBlocks;
    int want = (target + units - 1) / units;
    if (want > k2) want = k2;
    if (want < 1) want = 1;
    pages_per_split = (k2 + want - 1) / want;
    const int most = kFusedMaxRows / P > 0 ? kFusedMaxRows / P : 1;
    if (pages_per_split > most) pages_per_split = most;
    n_splits = (k2 + pages_per_split - 1) / pages_per_split;
}

}  // namespace

FusedPlan plan_fused(const rkv_gqa &g, int dtype, int B, int P, int max_pages, int k1, int k2,
                     const Knobs &kn) {
    FusedPlan p{RKV_FORM_STANDALONE, 0, 0};
    if (g.group > 8) return p;
    const int block = fused_waves(g.group) * kWave;
    if (max_pages > kFusedMaxPages || P > kFusedMaxRows) return p;
    const int units = B * g.n_kv_heads;
    // one block per unit streams every selected row, at most kFusedMaxRows
    // (the range this form is tested on); split-K blocks stream only their
    // share, so larger selections split further
    const bool rows_fit = (int64_t)k2 * P <= kFusedMaxRows;
    // split-K needs the staged selection (every page's summaries in LDS),
    // else each of its blocks would read the summaries from memory
    const int esz = dtype == RKV_F32 ? 4 : 2, V = 16 / esz;
    const bool stage_fits = max_pages <= block &&
        (int64_t)2 * k1 * ((max_pages + V - 1) / V * V) * esz <= (int64_t)kStageBytes;
    int form = units >= 192 && rows_fit ? RKV_FORM_FUSED
                                        : (stage_fits ? RKV_FORM_SPLITK : RKV_FORM_STANDALONE);
    if (kn.form == RKV_FORM_STANDALONE) form = RKV_FORM_STANDALONE;
    else if (kn.form == RKV_FORM_FUSED) form = rows_fit ? RKV_FORM_FUSED : RKV_FORM_STANDALONE;
    else if (kn.form == RKV_FORM_SPLITK) form = stage_fits ? RKV_FORM_SPLITK : RKV_FORM_STANDALONE;
    p.form = form;
    if (form == RKV_FORM_SPLITK)
        split_counts(units, k2, P, kn.splitk_blocks, p.n_splits, p.pages_per_split);
    return p;
}

size_t fused_split_ws_bytes(const rkv_gqa &g, int B, int P, int k2, const Knobs &kn) {
    // the split-K plan's partials for any dtype, k1 and form: the same split
    // count as plan_fused, whatever the batch
    const int units = B * g.n_kv_heads;
    int nsp, pps;
    split_counts(units, k2, P, kn.splitk_blocks, nsp, pps);
    return align_up((size_t)units * nsp * g.group * (g.head_dim + 2) * sizeof(float));
}

int launch_decode_fused(const FusedPlan &pl, const rkv_gqa &g, int dtype, int B, const void *q,
                        const void *k_new, const void *v_new, const rkv_paged_cache &c,
                        const int32_t *seq_lens, void *summaries, int k1, int k2, float scale,
                        float *out, int32_t *chan_idx, int32_t *page_idx, float *page_scores,
                        float *part, size_t part_bytes, const Knobs &kn, hipStream_t s) {
    DecArgs a;
    a.Hkv = g.n_kv_heads;
    a.P = c.page_size;
    a.max_pages = c.max_pages;
    a.k1 = k1;
    a.k2 = k2;
    a.num_blocks = c.num_blocks;
    a.page_table = c.page_table;
    a.seq_lens = seq_lens;
    a.qscale = scale * kLog2e;
    a.out = out;
    a.chan_out = chan_idx;
    a.page_out = page_idx;
    a.score_out = page_scores;
    a.part = part;
    a.pps = pl.pages_per_split;
    a.status = kn.status;
    a.trace = kn.trace;
    const int nsp = pl.form == RKV_FORM_SPLITK ? pl.n_splits : 0;
    if (nsp > 0 && (!part || (size_t)B * g.n_kv_heads * nsp * g.group * (g.head_dim + 2) *
                                     sizeof(float) > part_bytes))
        return RKV_EWORKSPACE;
    bool ok = false;
    const int d = g.head_dim;
    if (dtype == RKV_F32) {
        if (d == 64) ok = dispatch_g<float, 64>(B, nsp, g, a, q, k_new, v_new, c, summaries, s);
        else if (d == 128) ok = dispatch_g<float, 128>(B, nsp, g, a, q, k_new, v_new, c, summaries, s);
    } else {
        if (d == 64) ok = dispatch_g<uint16_t, 64>(B, nsp, g, a, q, k_new, v_new, c, summaries, s);
        else if (d == 128) ok = dispatch_g<uint16_t, 128>(B, nsp, g, a, q, k_new, v_new, c, summaries, s);
    }
    if (!ok) return RKV_EUNSUPPORTED;
    const int st = launch_status();
    if (st != RKV_OK || nsp == 0) return st;
    return launch_attend_merge(g, B, nsp, part, out, s);
}

}  // namespace rkv
