// summaries.hip -- incremental page max/min summaries (optionally copying the
// appended rows into the paged cache first).
//
// Page summaries follow the Quest-style paged element-wise max/min of
// "RocketKV-adapted -- Two-Stage Compression" (section "Where it sits"), and
// the incremental update must reproduce a rebuild bit for bit (section
// "Evidence").  Max and min select an existing element, so they are exact in
// any precision; scanning rows in ascending order with a strict comparison
// keeps the earliest of equal values, which makes append == rebuild hold for
// signed zeros as well.
//
// Grid: (pages touched per sequence, Hkv, B); one thread per channel.
#include "rkv_internal.h"

namespace rkv {
namespace {

template <typename T, int D>
__global__ void __launch_bounds__(D)
append_kernel(int Hkv, int P, int max_pages, int64_t num_blocks, const int32_t *page_table,
              T *k_pool, T *v_pool, const int32_t *n_old, const int32_t *n_new, int max_new,
              const T *k_src, const T *v_src, T *summ, int32_t *status) {
    const int b = blockIdx.z, h = blockIdx.y, c = threadIdx.x;
    const int64_t cap = (int64_t)max_pages * P;
    // one thread per sequence reports out-of-range row counts
    int32_t *st = (blockIdx.x == 0 && h == 0 && c == 0) ? status : nullptr;
    const int64_t e_raw = n_new[b];
    int64_t e = clamp_rows(n_new[b], cap, st);
    const int64_t o = n_old ? clamp_rows(n_old[b], cap, st)
                            : min<int64_t>(max<int64_t>(e_raw - 1, 0), cap);
    e = min<int64_t>(e, o + max_new);
    if (e <= o) return;
    const int64_t pg = o / P + blockIdx.x;
    const int64_t r0 = pg * P;
    if (r0 >= e) return;
    const int32_t blk = page_table[(int64_t)b * max_pages + pg];
    if (blk < 0 || blk >= num_blocks) {
        if (c == 0) report(status, RKV_DEV_BLOCK);
        return;
    }
    const int64_t rs = max<int64_t>(r0, o), re = min<int64_t>(r0 + P, e);

    T *kp = k_pool + ((int64_t)blk * Hkv + h) * P * D;
    T *sm = summ + (int64_t)(b * Hkv + h) * 2 * D * max_pages;
    const int64_t imax = (int64_t)c * max_pages + pg;
    const int64_t imin = (int64_t)(D + c) * max_pages + pg;

    T bmax, bmin;
    int64_t r = rs;
    auto fetch = [&](int64_t row) -> T {
        const int64_t dst = (row - r0) * D + c;
        if (k_src) {
            const int64_t src = (((int64_t)b * Hkv + h) * max_new + (row - o)) * D + c;
            const T kv = k_src[src];
            kp[dst] = kv;
            v_pool[((int64_t)blk * Hkv + h) * P * D + dst] = v_src[src];
            return kv;
        }
        return kp[dst];
    };
    if (r0 < o) {
        bmax = sm[imax];
        bmin = sm[imin];
    } else {
        bmax = bmin = fetch(r);
        ++r;
    }
    float fmax_ = Elem<T>::ld(&bmax, 0), fmin_ = Elem<T>::ld(&bmin, 0);
    for (; r < re; ++r) {
        const T x = fetch(r);
        const float fx = Elem<T>::ld(&x, 0);
        if (fx > fmax_) { fmax_ = fx; bmax = x; }
        if (fx < fmin_) { fmin_ = fx; bmin = x; }
    }
    sm[imax] = bmax;
    sm[imin] = bmin;
}

template <typename T, int D>
int launch_t(const rkv_gqa &g, int B, const rkv_paged_cache &c, const int32_t *n_old,
             const int32_t *n_new, int max_new, const void *k_src, const void *v_src,
             void *summ, int32_t *status, hipStream_t s) {
    const int pages = (max_new + c.page_size - 1) / c.page_size + 1;
    dim3 grid(pages, g.n_kv_heads, B);
    append_kernel<T, D><<<grid, D, 0, s>>>(
        g.n_kv_heads, c.page_size, c.max_pages, c.num_blocks, c.page_table, (T *)c.k_pool,
        (T *)c.v_pool, n_old, n_new, max_new, (const T *)k_src, (const T *)v_src, (T *)summ,
        status);
    return launch_status();
}

}  // namespace

int launch_append(const rkv_gqa &g, int dtype, int B, const rkv_paged_cache &c,
                  const int32_t *n_old, const int32_t *n_new, int max_new_rows,
                  const void *k_src, const void *v_src, void *summaries, int32_t *status,
                  hipStream_t s) {
    const int d = g.head_dim;
    if (dtype == RKV_F32) {
        if (d == 64) return launch_t<float, 64>(g, B, c, n_old, n_new, max_new_rows, k_src, v_src, summaries, status, s);
        if (d == 128) return launch_t<float, 128>(g, B, c, n_old, n_new, max_new_rows, k_src, v_src, summaries, status, s);
    } else {
        if (d == 64) return launch_t<uint16_t, 64>(g, B, c, n_old, n_new, max_new_rows, k_src, v_src, summaries, status, s);
        if (d == 128) return launch_t<uint16_t, 128>(g, B, c, n_old, n_new, max_new_rows, k_src, v_src, summaries, status, s);
    }
    return RKV_EUNSUPPORTED;
}

}  // namespace rkv
