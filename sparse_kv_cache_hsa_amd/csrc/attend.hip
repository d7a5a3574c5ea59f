// attend.hip -- exact attention over the rows of the selected pages (the
// standalone second half of HSA decode; the fused decode kernel covers the
// common case in one launch).
//
// A block handles one (sequence, KV head, split); a split is a range of the
// selected-page list.  At block start every row of the block's pages is
// resolved once (page table, validity) into an LDS row table, then the
// streaming core (attend_core.h) reads whole K/V rows with 16-byte loads and
// keeps an online softmax per query head.  With more than one split, each
// block writes (max, sum, acc) to the workspace and a small merge kernel
// combines the splits in split order.  (Merging inside the kernel through an
// arrival counter needs a device-scope release per block, which on this chip
// writes back the whole L2 and costs far more than the extra launch.)
#include "attend_core.h"

namespace rkv {
namespace {

constexpr int kMaxRows = 2048;  // rows resolved per block (LDS table)

struct AttArgs {
    int Hkv, P, max_pages, k2, ppb, n_splits;
    int64_t num_blocks;
    const int32_t *page_table, *seq_lens, *page_idx;
    float qscale;
    float *out, *part;
    int32_t *status;
};

template <typename T, int D, int G, int NW, int U, bool PIPE>
__global__ void __launch_bounds__(NW *kWave)
attend_kernel(AttArgs a, const T *k_pool, const T *v_pool, const T *q) {
    using Core = AttendCore<T, D, G, NW, U, PIPE>;
    constexpr int BLOCK = NW * kWave;
    __shared__ uint32_t row_s[kMaxRows];
    __shared__ typename Core::Shared sh;

    const int b = blockIdx.z, h = blockIdx.y, sp = blockIdx.x, tid = threadIdx.x;
    const int P = a.P;
    const int64_t bh = (int64_t)b * a.Hkv + h;
    const int64_t cap = (int64_t)a.max_pages * P;
    const int64_t n = clamp_rows(a.seq_lens[b], cap, (sp == 0 && h == 0 && tid == 0) ? a.status : nullptr);
    const int NP = (int)((n + P - 1) / P);
    const int nsel = min(a.k2, NP);
    const int i0 = sp * a.ppb;
    const int npg = max(0, min(i0 + a.ppb, nsel) - i0);
    const int nrows = npg * P;

    for (int f = tid; f < nrows; f += BLOCK) {
        const int pi = f / P, slot = f - pi * P;
        const int32_t pg = a.page_idx[bh * a.k2 + i0 + pi];
        uint32_t r = kBadRow;
        if (pg >= 0 && pg < NP) {
            if ((int64_t)pg * P + slot < n) {
                const int32_t blk = a.page_table[(int64_t)b * a.max_pages + pg];
                if (blk >= 0 && blk < a.num_blocks)
                    r = (uint32_t)(((int64_t)blk * a.Hkv + h) * P + slot);
                else if (slot == 0)
                    report(a.status, RKV_DEV_BLOCK);
            }
        } else if (slot == 0) {
            report(a.status, RKV_DEV_PAGE);
        }
        row_s[f] = r;
    }
    Core core;
    core.init(q, bh, a.qscale);
    __syncthreads();
    if constexpr (PIPE)
        core.stream(row_s, nrows, k_pool, v_pool);
    else
        core.stream_fn(nrows, k_pool, v_pool, [&](int f) { return row_s[f]; });
    core.to_shared(sh);
    __syncthreads();
    if (a.n_splits == 1) {
        Core::combine(sh, [&](int j, int c, float M, float Ls, float A0, float A1) {
            float *o = a.out + (bh * G + j) * D + c;
            o[0] = Ls > 0.0f ? A0 / Ls : 0.0f;
            o[1] = Ls > 0.0f ? A1 / Ls : 0.0f;
        });
    } else {
        float *base = a.part + (bh * a.n_splits + sp) * G * (D + 2);
        Core::combine(sh, [&](int j, int c, float M, float Ls, float A0, float A1) {
            float *pp = base + j * (D + 2);
            pp[c] = A0;
            pp[c + 1] = A1;
            if (c == 0) {
                pp[D] = M;
                pp[D + 1] = Ls;
            }
        });
    }
}

// Combines the splits of one (sequence, KV head, query head of the group):
// block (h, b, j), one thread per channel.  M = max of the splits' m and
// Ls = sum of l_s 2^(m_s - M) come from wave reductions in a fixed order; the
// split weights 2^(m_s - M) go to LDS, and each channel then sums its split
// partials in split order.  The partials of the first 16 splits and the
// splits' (m, l) are loaded up front, so the usual case costs one memory
// round trip.
constexpr int kMergeMaxSplits = 1024;

template <int D, int G>
__global__ void __launch_bounds__(D)
attend_merge_kernel(int Hkv, int n_splits, const float *part, float *out) {
    constexpr int NW = D / kWave;
    __shared__ float cw_s[kMergeMaxSplits];
    __shared__ float red_s[2][NW];
    const int h = blockIdx.x, b = blockIdx.y, j = blockIdx.z, c = threadIdx.x;
    const int lane = c & (kWave - 1), w = c / kWave;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t stride = (int64_t)G * (D + 2);
    const float *base_p = part + (bh * n_splits * G + j) * (D + 2);
    // One memory round trip for the common case: the channel's partials of
    // the first kPre splits and (thread sp) split sp's max and sum are all
    // loaded before any of them is used.
    constexpr int kPre = 16;
    float pre[kPre];
#pragma unroll
    for (int u = 0; u < kPre; ++u)
        pre[u] = u < n_splits ? base_p[(int64_t)u * stride + c] : 0.0f;
    const bool own = c < n_splits;
    const float m_own = own ? base_p[(int64_t)c * stride + D] : -INFINITY;
    const float l_own = own ? base_p[(int64_t)c * stride + D + 1] : 0.0f;
    float m = m_own;
    for (int sp = c + D; sp < n_splits; sp += D) m = fmaxf(m, base_p[sp * stride + D]);
    m = pair_max<1>(m);
    m = pair_max<2>(m);
    m = pair_max<4>(m);
    m = pair_max<8>(m);
    m = pair_max<16>(m);
    m = pair_max<32>(m);
    if (lane == 0) red_s[0][w] = m;
    __syncthreads();
    float M = red_s[0][0];
#pragma unroll
    for (int i = 1; i < NW; ++i) M = fmaxf(M, red_s[0][i]);
    float ls = 0.0f;
    if (own) {
        const float wt = exp2_diff(m_own, M);
        cw_s[c] = wt;
        ls = l_own * wt;
    }
    for (int sp = c + D; sp < n_splits; sp += D) {
        const float wt = exp2_diff(base_p[sp * stride + D], M);
        cw_s[sp] = wt;
        ls += base_p[sp * stride + D + 1] * wt;
    }
    ls = pair_sum<1>(ls);
    ls = pair_sum<2>(ls);
    ls = pair_sum<4>(ls);
    ls = pair_sum<8>(ls);
    ls = pair_sum<16>(ls);
    ls = pair_sum<32>(ls);
    if (lane == 0) red_s[1][w] = ls;
    __syncthreads();
    float Ls = red_s[1][0];
#pragma unroll
    for (int i = 1; i < NW; ++i) Ls += red_s[1][i];
    // the channel's sum over the splits, in split order
    float A = 0.0f;
#pragma unroll
    for (int u = 0; u < kPre; ++u)
        if (u < n_splits) A += pre[u] * cw_s[u];
    constexpr int kBatch = 8;
    for (int s0 = kPre; s0 < n_splits; s0 += kBatch) {
        float v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            v[u] = s0 + u < n_splits ? base_p[(int64_t)(s0 + u) * stride + c] : 0.0f;
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (s0 + u < n_splits) A += v[u] * cw_s[s0 + u];
    }
    out[(bh * G + j) * D + c] = Ls > 0.0f ? A / Ls : 0.0f;
}

// Kernel variants: (waves per block, row loads per iteration, pipelined).
constexpr int kVariantWaves[4] = {4, 8, 16, 16};

template <typename T, int D, int G>
int launch_t(const rkv_gqa &g, int B, const void *q, const rkv_paged_cache &c,
             const int32_t *seq_lens, const int32_t *page_idx, int k2, float scale, float *out,
             void *ws, const Knobs &kn, hipStream_t s) {
    const AttendPlan pl = plan_attend(g, B, c.page_size, k2, kn);
    AttArgs a;
    a.Hkv = g.n_kv_heads;
    a.P = c.page_size;
    a.max_pages = c.max_pages;
    a.k2 = k2;
    a.ppb = pl.pages_per_block;
    a.n_splits = pl.n_splits;
    a.num_blocks = c.num_blocks;
    a.page_table = c.page_table;
    a.seq_lens = seq_lens;
    a.page_idx = page_idx;
    a.qscale = scale * kLog2e;
    a.out = out;
    a.part = (float *)ws;
    a.status = kn.status;
    dim3 grid(pl.n_splits, g.n_kv_heads, B);
    const T *kp = (const T *)c.k_pool, *vp = (const T *)c.v_pool, *qp = (const T *)q;
    switch (pl.variant) {
        case 1: attend_kernel<T, D, G, 8, 2, true><<<grid, 8 * kWave, 0, s>>>(a, kp, vp, qp); break;
        case 2: attend_kernel<T, D, G, 16, 4, false><<<grid, 16 * kWave, 0, s>>>(a, kp, vp, qp); break;
        case 3: attend_kernel<T, D, G, 16, 2, true><<<grid, 16 * kWave, 0, s>>>(a, kp, vp, qp); break;
        default: attend_kernel<T, D, G, 4, 8, false><<<grid, 4 * kWave, 0, s>>>(a, kp, vp, qp); break;
    }
    int st = launch_status();
    if (st != RKV_OK || pl.n_splits == 1) return st;
    attend_merge_kernel<D, G><<<dim3(g.n_kv_heads, B, G), D, 0, s>>>(g.n_kv_heads, pl.n_splits,
                                                                     a.part, out);
    return launch_status();
}

template <typename T, int D>
int dispatch_g(const rkv_gqa &g, int B, const void *q, const rkv_paged_cache &c,
               const int32_t *seq_lens, const int32_t *page_idx, int k2, float scale, float *out,
               void *ws, const Knobs &kn, hipStream_t s) {
    switch (g.group) {
        case 1: return launch_t<T, D, 1>(g, B, q, c, seq_lens, page_idx, k2, scale, out, ws, kn, s);
        case 2: return launch_t<T, D, 2>(g, B, q, c, seq_lens, page_idx, k2, scale, out, ws, kn, s);
        case 4: return launch_t<T, D, 4>(g, B, q, c, seq_lens, page_idx, k2, scale, out, ws, kn, s);
        case 8: return launch_t<T, D, 8>(g, B, q, c, seq_lens, page_idx, k2, scale, out, ws, kn, s);
    }
    return RKV_EUNSUPPORTED;
}

}  // namespace

AttendPlan plan_attend(const rkv_gqa &g, int B, int P, int k2, const Knobs &kn) {
    const int units = B * g.n_kv_heads;
    const int max_ppb = kMaxRows / P > 0 ? kMaxRows / P : 1;
    AttendPlan p;
    int variant = kn.attend_variant - 1;  // option 1..4 -> kernel variant 0..3
    const bool wide_ok = g.group * g.head_dim <= 512;  // wide blocks keep G*D per wave in LDS
    if (variant < 0 || variant > 3) {
        // One wide block per (sequence, head) once the batch fills the chip;
        // otherwise 4-wave blocks over splits of the page list.
        variant = (units >= 192 && wide_ok && (int64_t)k2 * P <= kMaxRows) ? 2 : 0;
    }
    if (kVariantWaves[variant] > 4 && !wide_ok) variant = 0;
    const int waves = kVariantWaves[variant];
    int ppb = kn.attend_pages;
    if (ppb <= 0) {
        if (waves == 16) {
            ppb = k2;
        } else {
            // about 1024 blocks, with at least one full pass of the block's
            // waves (64 rows each) per split
            const int min_rows = (64 * waves + P - 1) / P;
            const int spread = (int)(((int64_t)k2 * units * waves / 4 + 1023) / 1024);
            ppb = min_rows > spread ? min_rows : spread;
        }
    }
    if (ppb > k2) ppb = k2;
    if (ppb > max_ppb) ppb = max_ppb;
    if (ppb < 1) ppb = 1;
    p.pages_per_block = ppb;
    p.n_splits = (k2 + ppb - 1) / ppb;
    p.waves = waves;
    p.variant = variant;
    return p;
}

size_t attend_ws_bytes(const rkv_gqa &g, int B, int P, int k2, const Knobs &kn) {
    const AttendPlan p = plan_attend(g, B, P, k2, kn);
    if (p.n_splits == 1) return 0;
    return align_up((size_t)B * g.n_kv_heads * p.n_splits * g.group * (g.head_dim + 2) *
                    sizeof(float));
}

int launch_attend_merge(const rkv_gqa &g, int B, int n_splits, const float *part, float *out,
                        hipStream_t s) {
    if (n_splits > kMergeMaxSplits) return RKV_EUNSUPPORTED;
    const dim3 grid(g.n_kv_heads, B, g.group);
    const int d = g.head_dim;
    switch (g.group * 1000 + d) {
        case 1064: attend_merge_kernel<64, 1><<<grid, 64, 0, s>>>(g.n_kv_heads, n_splits, part, out); break;
        case 2064: attend_merge_kernel<64, 2><<<grid, 64, 0, s>>>(g.n_kv_heads, n_splits, part, out); break;
        case 4064: attend_merge_kernel<64, 4><<<grid, 64, 0, s>>>(g.n_kv_heads, n_splits, part, out); break;
        case 8064: attend_merge_kernel<64, 8><<<grid, 64, 0, s>>>(g.n_kv_heads, n_splits, part, out); break;
        case 1128: attend_merge_kernel<128, 1><<<grid, 128, 0, s>>>(g.n_kv_heads, n_splits, part, out); break;
        case 2128: attend_merge_kernel<128, 2><<<grid, 128, 0, s>>>(g.n_kv_heads, n_splits, part, out); break;
        case 4128: attend_merge_kernel<128, 4><<<grid, 128, 0, s>>>(g.n_kv_heads, n_splits, part, out); break;
        case 8128: attend_merge_kernel<128, 8><<<grid, 128, 0, s>>>(g.n_kv_heads, n_splits, part, out); break;
        default: return RKV_EUNSUPPORTED;
    }
    return launch_status();
}

int launch_attend(const rkv_gqa &g, int dtype, int B, const void *q, const rkv_paged_cache &c,
                  const int32_t *seq_lens, const int32_t *page_idx, int k2, float scale,
                  float *out, void *ws, const Knobs &kn, hipStream_t s) {
    const int d = g.head_dim;
    if (dtype == RKV_F32) {
        if (d == 64) return dispatch_g<float, 64>(g, B, q, c, seq_lens, page_idx, k2, scale, out, ws, kn, s);
        if (d == 128) return dispatch_g<float, 128>(g, B, q, c, seq_lens, page_idx, k2, scale, out, ws, kn, s);
    } else {
        if (d == 64) return dispatch_g<uint16_t, 64>(g, B, q, c, seq_lens, page_idx, k2, scale, out, ws, kn, s);
        if (d == 128) return dispatch_g<uint16_t, 128>(g, B, q, c, seq_lens, page_idx, k2, scale, out, ws, kn, s);
    }
    return RKV_EUNSUPPORTED;
}

}  // namespace rkv
