// attend.hip -- exact attention over the rows of the selected pages.
//
// RocketKV's second stage attends exactly over the tokens it selected
// ("RocketKV-adapted -- Two-Stage Compression", "Adaptation notes": every row
// of a selected page takes part).  The work is an HBM stream of whole K/V
// page slices (P rows x d contiguous per KV head) at about 4 flop per byte,
// far below the vector-ALU ridge, so it runs on the vector ALU in fp32
// (bf16 widened exactly), not on MFMA.
//
// Mapping (gfx950, 64-lane waves)
//   - A block (4 waves) handles one (sequence, KV head, split); a split is a
//     contiguous range of the selected-page list.  The G query heads of the
//     group share every K/V load (GQA reuse in registers).
//   - A row of d elements is read by LPR lanes with one 16-byte load each;
//     a wave reads RPW = 64/LPR rows per load and keeps U such loads of K and
//     V in flight.
//   - Dot products are finished with xor-shuffles inside the LPR lanes of a
//     row; each row group keeps an online-softmax state (max, sum, acc) in
//     the log2 domain (the query is pre-scaled by scale*log2(e)).
//   - States are merged across row groups (shuffles), waves (LDS) and, when
//     there is more than one split, across splits by merge_kernel in a fixed
//     order, so results do not depend on scheduling.
#include <stdlib.h>

#include "rkv_internal.h"

namespace rkv {
namespace {

constexpr int kAttBlock = 256;
constexpr int kAttNW = kAttBlock / kWave;
constexpr int kMaxPPB = 1024;
constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int D, int G>
__global__ void __launch_bounds__(kAttBlock)
attend_kernel(int Hkv, int P, int max_pages, int64_t num_blocks, const int32_t *page_table,
              const T *k_pool, const T *v_pool, const T *q, const int32_t *seq_lens,
              const int32_t *page_idx, int k2, int ppb, int n_splits, float qscale, float *out,
              float *part) {
    constexpr int EPL = Vec16<T>::N;
    constexpr int LPR = D / EPL;
    constexpr int RPW = kWave / LPR;
    constexpr int U = 4;
    constexpr int NW = kAttNW;
    __shared__ int32_t blk_s[kMaxPPB];
    __shared__ int32_t row0_s[kMaxPPB];
    __shared__ float wm[NW][G], wl[NW][G];
    __shared__ float wacc[NW][G][D];

    const int b = blockIdx.z, h = blockIdx.y, sp = blockIdx.x, tid = threadIdx.x;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t cap = (int64_t)max_pages * P;
    const int64_t n = min<int64_t>(max<int64_t>(seq_lens[b], 0), cap);
    const int NP = (int)((n + P - 1) / P);
    const int nsel = min(k2, NP);
    const int i0 = sp * ppb;
    const int npg = max(0, min(i0 + ppb, nsel) - i0);

    for (int i = tid; i < npg; i += kAttBlock) {
        const int32_t pg = page_idx[bh * k2 + i0 + i];
        int32_t blk = -1;
        if (pg >= 0 && pg < NP) blk = page_table[(int64_t)b * max_pages + pg];
        if (blk < 0 || blk >= num_blocks) blk = -1;
        blk_s[i] = blk;
        row0_s[i] = pg * P;
    }
    __syncthreads();

    const int lane = tid & (kWave - 1), w = tid / kWave;
    const int sub = lane % LPR, rsub = lane / LPR;

    float qv[G][EPL];
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            qv[j][e] = Elem<T>::ld(q, (bh * G + j) * D + sub * EPL + e) * qscale;

    float m[G], l[G], acc[G][EPL];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] = 0.0f;
    }

    const int nrows = npg * P;
    for (int base = w * U * RPW; base < nrows; base += NW * U * RPW) {
        uint4 kr[U], vr[U];
        bool valid[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int f = base + u * RPW + rsub;
            valid[u] = false;
            kr[u] = make_uint4(0u, 0u, 0u, 0u);
            vr[u] = make_uint4(0u, 0u, 0u, 0u);
            if (f < nrows) {
                const int pi = f / P;
                const int slot = f - pi * P;
                const int32_t blk = blk_s[pi];
                if (blk >= 0 && (int64_t)row0_s[pi] + slot < n) {
                    valid[u] = true;
                    const int64_t off = (((int64_t)blk * Hkv + h) * P + slot) * D + sub * EPL;
                    kr[u] = *(const uint4 *)(k_pool + off);
                    vr[u] = *(const uint4 *)(v_pool + off);
                }
            }
        }
        float sc[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[EPL];
            Vec16<T>::unpack(kr[u], kf);
#pragma unroll
            for (int j = 0; j < G; ++j) {
                float p = 0.0f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) p = __builtin_fmaf(qv[j][e], kf[e], p);
                sc[u][j] = p;
            }
        }
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1)
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int j = 0; j < G; ++j) sc[u][j] += __shfl_xor(sc[u][j], off, kWave);

        float vf[U][EPL];
#pragma unroll
        for (int u = 0; u < U; ++u) Vec16<T>::unpack(vr[u], vf[u]);
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float mn = m[j];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (valid[u]) mn = fmaxf(mn, sc[u][j]);
            const float corr = exp2_diff(m[j], mn);
            m[j] = mn;
            l[j] *= corr;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[j][e] *= corr;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (valid[u]) {
                    const float p = exp2f(sc[u][j] - mn);
                    l[j] += p;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[j][e] = __builtin_fmaf(p, vf[u][e], acc[j][e]);
                }
            }
        }
    }

    // merge the RPW row groups of the wave
#pragma unroll
    for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float mo = __shfl_xor(m[j], off, kWave);
            const float lo = __shfl_xor(l[j], off, kWave);
            const float mn = fmaxf(m[j], mo);
            const float c1 = exp2_diff(m[j], mn), c2 = exp2_diff(mo, mn);
            l[j] = l[j] * c1 + lo * c2;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float ao = __shfl_xor(acc[j][e], off, kWave);
                acc[j][e] = acc[j][e] * c1 + ao * c2;
            }
            m[j] = mn;
        }
    }
    if (rsub == 0) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
            if (sub == 0) {
                wm[w][j] = m[j];
                wl[w][j] = l[j];
            }
#pragma unroll
            for (int e = 0; e < EPL; ++e) wacc[w][j][sub * EPL + e] = acc[j][e];
        }
    }
    __syncthreads();

    // merge the waves; one thread per (head, channel)
    for (int t = tid; t < G * D; t += kAttBlock) {
        const int j = t / D, c = t % D;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, wm[ww][j]);
        float Lsum = 0.0f, A = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float cw = exp2_diff(wm[ww][j], M);
            Lsum += wl[ww][j] * cw;
            A += wacc[ww][j][c] * cw;
        }
        if (n_splits == 1) {
            out[(bh * G + j) * D + c] = Lsum > 0.0f ? A / Lsum : 0.0f;
        } else {
            float *pp = part + ((bh * n_splits + sp) * G + j) * (D + 2);
            pp[c] = A;
            if (c == 0) {
                pp[D] = M;
                pp[D + 1] = Lsum;
            }
        }
    }
}

template <int D, int G>
__global__ void __launch_bounds__(kAttBlock)
attend_merge_kernel(int Hkv, int n_splits, const float *part, float *out) {
    const int b = blockIdx.y, h = blockIdx.x;
    const int64_t bh = (int64_t)b * Hkv + h;
    for (int t = threadIdx.x; t < G * D; t += kAttBlock) {
        const int j = t / D, c = t % D;
        float M = -INFINITY;
        for (int s = 0; s < n_splits; ++s)
            M = fmaxf(M, part[((bh * n_splits + s) * G + j) * (D + 2) + D]);
        float Lsum = 0.0f, A = 0.0f;
        for (int s = 0; s < n_splits; ++s) {
            const float *pp = part + ((bh * n_splits + s) * G + j) * (D + 2);
            const float cw = exp2_diff(pp[D], M);
            Lsum += pp[D + 1] * cw;
            A += pp[c] * cw;
        }
        out[(bh * G + j) * D + c] = Lsum > 0.0f ? A / Lsum : 0.0f;
    }
}

int env_int(const char *name, int dflt) {
    const char *v = getenv(name);
    return (v && *v) ? atoi(v) : dflt;
}

template <typename T, int D, int G>
int launch_t(const rkv_gqa &g, int B, const void *q, const rkv_paged_cache &c,
             const int32_t *seq_lens, const int32_t *page_idx, int k2, float scale, float *out,
             void *ws, hipStream_t s) {
    const AttendPlan pl = plan_attend(g, B, c.page_size, k2);
    dim3 grid(pl.n_splits, g.n_kv_heads, B);
    float *part = (float *)ws;
    attend_kernel<T, D, G><<<grid, kAttBlock, 0, s>>>(
        g.n_kv_heads, c.page_size, c.max_pages, c.num_blocks, c.page_table, (const T *)c.k_pool,
        (const T *)c.v_pool, (const T *)q, seq_lens, page_idx, k2, pl.pages_per_block,
        pl.n_splits, scale * kLog2e, out, part);
    int st = launch_status();
    if (st != RKV_OK || pl.n_splits == 1) return st;
    attend_merge_kernel<D, G><<<dim3(g.n_kv_heads, B), kAttBlock, 0, s>>>(g.n_kv_heads,
                                                                         pl.n_splits, part, out);
    return launch_status();
}

template <typename T, int D>
int dispatch_g(const rkv_gqa &g, int B, const void *q, const rkv_paged_cache &c,
               const int32_t *seq_lens, const int32_t *page_idx, int k2, float scale, float *out,
               void *ws, hipStream_t s) {
    switch (g.group) {
        case 1: return launch_t<T, D, 1>(g, B, q, c, seq_lens, page_idx, k2, scale, out, ws, s);
        case 2: return launch_t<T, D, 2>(g, B, q, c, seq_lens, page_idx, k2, scale, out, ws, s);
        case 4: return launch_t<T, D, 4>(g, B, q, c, seq_lens, page_idx, k2, scale, out, ws, s);
        case 8: return launch_t<T, D, 8>(g, B, q, c, seq_lens, page_idx, k2, scale, out, ws, s);
    }
    return RKV_EUNSUPPORTED;
}

}  // namespace

AttendPlan plan_attend(const rkv_gqa &g, int B, int P, int k2) {
    const int units = B * g.n_kv_heads;
    int ppb = env_int("RKV_ATTEND_PPB", 0);
    if (ppb <= 0) {
        // >= 64 rows per block (one full pass of the 4 waves), and about
        // 1024 blocks in total when the batch allows it.
        const int min_rows = (64 + P - 1) / P;
        const int spread = (int)(((int64_t)k2 * units + 1023) / 1024);
        ppb = min_rows > spread ? min_rows : spread;
    }
    if (ppb > k2) ppb = k2;
    if (ppb > kMaxPPB) ppb = kMaxPPB;
    if (ppb < 1) ppb = 1;
    AttendPlan p;
    p.pages_per_block = ppb;
    p.n_splits = (k2 + ppb - 1) / ppb;
    return p;
}

size_t attend_ws_bytes(const rkv_gqa &g, int B, int P, int k2) {
    const AttendPlan p = plan_attend(g, B, P, k2);
    if (p.n_splits == 1) return 0;
    return align_up((size_t)B * g.n_kv_heads * p.n_splits * g.group * (g.head_dim + 2) *
                    sizeof(float));
}

int launch_attend(const rkv_gqa &g, int dtype, int B, const void *q, const rkv_paged_cache &c,
                  const int32_t *seq_lens, const int32_t *page_idx, int k2, float scale,
                  float *out, void *ws, hipStream_t s) {
    const int d = g.head_dim;
    if (dtype == RKV_F32) {
        if (d == 64) return dispatch_g<float, 64>(g, B, q, c, seq_lens, page_idx, k2, scale, out, ws, s);
        if (d == 128) return dispatch_g<float, 128>(g, B, q, c, seq_lens, page_idx, k2, scale, out, ws, s);
    } else {
        if (d == 64) return dispatch_g<uint16_t, 64>(g, B, q, c, seq_lens, page_idx, k2, scale, out, ws, s);
        if (d == 128) return dispatch_g<uint16_t, 128>(g, B, q, c, seq_lens, page_idx, k2, scale, out, ws, s);
    }
    return RKV_EUNSUPPORTED;
}

}  // namespace rkv
