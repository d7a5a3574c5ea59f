// attend_core.h -- the streaming attention core shared by the split-K
// attention kernel and the fused decode kernel.
//
// RocketKV's second stage attends exactly over the tokens of the selected
// pages ("RocketKV-adapted -- Two-Stage Compression", "Adaptation notes").
// The work is an HBM stream of K/V page slices at about 4 flop per byte, far
// below the vector-ALU ridge, so it runs on the vector ALU in fp32 (bf16
// widened exactly).
//
// Layout of the work inside a block of NW waves:
//   - the block's rows are given as row units (block * Hkv + h) * P + slot,
//     or kBadRow for rows that do not exist: listed in an LDS table (row_s),
//     or resolved by the caller's function one iteration ahead of the
//     loads that use them;
//   - a row of d elements is read by LPR lanes with one 16-byte non-temporal
//     load each (the rows are streamed once per step), a
//     wave reads RPW = 64/LPR rows per load and U loads of K and of V per
//     iteration; waves take iterations round-robin, or (the fused decode
//     kernel) in contiguous ranges sized by the waves' age on their SIMD;
//   - each lane holds its EPL channels of the G query heads (the G heads share
//     every K/V load) and an online-softmax state per head in the log2 domain
//     (hardware exp2); the running maximum is kept uniform across the row
//     groups of a wave, so their sums merge without rescaling;
//   - bf16 dot products use the packed bf16 dot instruction (exact products,
//     fp32 accumulation) with the query kept as exact bf16 pairs and the
//     scale*log2(e) factor applied to the finished dot product; fp32 inputs
//     use fp32 multiply-adds with a pre-scaled query;
//   - dot products are finished inside the LPR lanes of a row with DPP
//     butterflies; at the end the row groups of a wave are summed with lane
//     swaps and the waves are merged through LDS in a fixed order, so the
//     result does not depend on timing.
#pragma once

#include <type_traits>

#include "rkv_internal.h"

namespace rkv {

constexpr uint32_t kBadRow = 0xffffffffu;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr float kLog2e = 1.4426950408889634f;

// DPP lane permutes (gfx9 encodings).
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within 16

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}

template <int OFF>
__device__ __forceinline__ float xor_lanes(float v) {
    return __uint_as_float(lane_xor<OFF>(__float_as_uint(v)));
}

// Sum over the LPR consecutive lanes that share a row; every lane of the row
// gets the same bits (each step adds a commutative pair).
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
    static_assert(LPR == 4 || LPR == 8 || LPR == 16 || LPR == 32, "lanes per row");
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    if constexpr (LPR >= 8) v += dpp<kDppHalfMirror>(v);
    if constexpr (LPR >= 16) v += dpp<kDppMirror>(v);
    if constexpr (LPR >= 32) v = pair_sum<16>(v);
    return v;
}


// Maximum over the row groups of a wave (every lane of a row group holds
// the same value); every lane gets the result.
template <int LPR>
__device__ __forceinline__ float rows_max(float v) {
    if constexpr (LPR < kWave) {
        v = pair_max<LPR>(v);
        return rows_max<LPR * 2>(v);
    } else {
        return v;
    }
}

template <typename T, int D, int G, int NW, int U, bool PIPE>
struct AttendCore {
    static constexpr bool kPacked = std::is_same<T, uint16_t>::value;
    static constexpr int EPL = Vec16<T>::N;  // channels per lane
    static constexpr int LPR = D / EPL;      // lanes per row
    static constexpr int RPW = kWave / LPR;  // rows per wave load
    static constexpr int ROWS_IT = U * RPW;  // rows per wave iteration

    struct alignas(16) Shared {
        float wm[NW][G], wl[NW][G];
        float wacc[NW][G][D];
    };

    float qv[G][EPL];       // fp32 inputs: pre-scaled query
    uint32_t qp[G][4];      // bf16 inputs: query channel pairs, exact
    float qs_;              // bf16 inputs: scale*log2(e)
    float m[G], l[G], acc[G][EPL];
    int lane, w, sub, rsub;

    // q of the G heads sharing KV head bh, this lane's channels.
    __device__ __forceinline__ void init(const T *q, int64_t bh, float qscale) {
        lane = threadIdx.x & (kWave - 1);
        w = threadIdx.x / kWave;
        sub = lane % LPR;
        rsub = lane / LPR;
        qs_ = qscale;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const uint4 raw = *(const uint4 *)(q + (bh * G + j) * D + sub * EPL);
            if constexpr (kPacked) {
                qp[j][0] = raw.x;
                qp[j][1] = raw.y;
                qp[j][2] = raw.z;
                qp[j][3] = raw.w;
            } else {
                Vec16<T>::unpack(raw, qv[j]);
#pragma unroll
                for (int e = 0; e < EPL; ++e) qv[j][e] *= qscale;
            }
            m[j] = -INFINITY;
            l[j] = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[j][e] = 0.0f;
        }
    }

    // Same state as init(), from the queries already in LDS as fp32 (qs[j][c],
    // exact widenings of the inputs).
    __device__ __forceinline__ void init_lds(const float (*qs)[D], float qscale) {
        lane = threadIdx.x & (kWave - 1);
        w = threadIdx.x / kWave;
        sub = lane % LPR;
        rsub = lane / LPR;
        qs_ = qscale;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float x[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) x[e] = qs[j][sub * EPL + e];
            if constexpr (kPacked) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    qp[j][e] = (__float_as_uint(x[2 * e]) >> 16) |
                               (__float_as_uint(x[2 * e + 1]) & 0xffff0000u);
            } else {
#pragma unroll
                for (int e = 0; e < EPL; ++e) qv[j][e] = x[e] * qscale;
            }
            m[j] = -INFINITY;
            l[j] = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[j][e] = 0.0f;
        }
    }

    __device__ __forceinline__ void issue(const uint32_t *row_s, int nrows, const T *k_pool,
                                          const T *v_pool, int base, uint4 *kr, uint4 *vr,
                                          bool *ok) const {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int f = base + u * RPW + rsub;
            const uint32_t r = f < nrows ? row_s[f] : kBadRow;
            ok[u] = r != kBadRow;
            const int64_t off = (int64_t)(ok[u] ? r : 0u) * D + sub * EPL;
            // every K/V row is read once per step: non-temporal loads keep
            // the stream from displacing cached data (measurably faster)
            const u32x4 kz = ok[u] ? __builtin_nontemporal_load((const u32x4 *)(k_pool + off)) : u32x4{0u, 0u, 0u, 0u};
            const u32x4 vz = ok[u] ? __builtin_nontemporal_load((const u32x4 *)(v_pool + off)) : u32x4{0u, 0u, 0u, 0u};
            kr[u] = make_uint4(kz.x, kz.y, kz.z, kz.w);
            vr[u] = make_uint4(vz.x, vz.y, vz.z, vz.w);
        }
    }

    // ALL: every row of the iteration exists (ok[] is then not read).
    template <bool ALL = false>
    __device__ __forceinline__ void consume(const uint4 *kr, const uint4 *vr, const bool *ok) {
        float sc[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (kPacked) {
                const uint32_t kw[4] = {kr[u].x, kr[u].y, kr[u].z, kr[u].w};
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    float p = 0.0f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) p = dot2_bf16(qp[j][e], kw[e], p);
                    sc[u][j] = row_sum<LPR>(p) * qs_;
                }
            } else {
                float kf[EPL];
                Vec16<T>::unpack(kr[u], kf);
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    float p = 0.0f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) p = __builtin_fmaf(qv[j][e], kf[e], p);
                    sc[u][j] = row_sum<LPR>(p);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            // the running maximum is kept uniform across the wave's row
            // groups, so merging them at the end needs no rescaling
            float mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (ALL || ok[u]) mx = fmaxf(mx, sc[u][j]);
            mx = rows_max<LPR>(mx);
            // Rescale only when the running maximum rises (it is uniform
            // across the wave, so this is a uniform branch): otherwise the
            // factor would be exp2(0) = 1 exactly, and the state unchanged.
            if (mx > m[j]) {
                const float corr = exp2_diff(m[j], mx);
                m[j] = mx;
                l[j] *= corr;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[j][e] *= corr;
            }
            const float mn = m[j];
            float lj = l[j];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                sc[u][j] = (ALL || ok[u]) ? fast_exp2(sc[u][j] - mn) : 0.0f;
                lj += sc[u][j];
            }
            l[j] = lj;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[EPL];
            Vec16<T>::unpack(vr[u], vf);
#pragma unroll
            for (int j = 0; j < G; ++j)
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[j][e] = __builtin_fmaf(sc[u][j], vf[e], acc[j][e]);
        }
    }

    // Loads this lane's rows of one iteration given their row units.
    __device__ __forceinline__ void load_rows(const uint32_t *rid, const T *k_pool,
                                              const T *v_pool, uint4 *kr, uint4 *vr,
                                              bool *ok) const {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            ok[u] = rid[u] != kBadRow;
            const int64_t off = (int64_t)(ok[u] ? rid[u] : 0u) * D + sub * EPL;
            const u32x4 kz = ok[u] ? __builtin_nontemporal_load((const u32x4 *)(k_pool + off)) : u32x4{0u, 0u, 0u, 0u};
            const u32x4 vz = ok[u] ? __builtin_nontemporal_load((const u32x4 *)(v_pool + off)) : u32x4{0u, 0u, 0u, 0u};
            kr[u] = make_uint4(kz.x, kz.y, kz.z, kz.w);
            vr[u] = make_uint4(vz.x, vz.y, vz.z, vz.w);
        }
    }

    // load_rows when every row unit is valid: no masks.
    __device__ __forceinline__ void load_rows_all(const uint32_t *rid, const T *k_pool,
                                                  const T *v_pool, uint4 *kr, uint4 *vr) const {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t off = (int64_t)rid[u] * D + sub * EPL;
            const u32x4 kz = __builtin_nontemporal_load((const u32x4 *)(k_pool + off));
            const u32x4 vz = __builtin_nontemporal_load((const u32x4 *)(v_pool + off));
            kr[u] = make_uint4(kz.x, kz.y, kz.z, kz.w);
            vr[u] = make_uint4(vz.x, vz.y, vz.z, vz.w);
        }
    }

    // Streams rows [0, nrows) whose row units rowfn(f) gives (kBadRow for a
    // row that does not exist).  The row units of the next iteration are
    // resolved while this iteration's loads are in flight, so no row table
    // (and no block barrier after building one) is needed.
    //
    // Iterations of ROWS_IT rows go to the waves round-robin (OLDER_PCT = 0)
    // or, for a block whose waves w and w + NW/2 share a SIMD, in contiguous
    // ranges: each such pair of waves takes an equal range, of which the
    // older wave (w < NW/2, which the SIMD serves first) takes the first
    // OLDER_PCT percent.  Either way the split depends only on nrows, so the
    // rows of a wave and their order, hence the bits, do not depend on timing.
    template <int OLDER_PCT = 0, typename RowFn>
    __device__ __forceinline__ void stream_fn(int nrows, const T *k_pool, const T *v_pool,
                                              RowFn rowfn) {
        static_assert(OLDER_PCT == 0 || (NW % 2 == 0 && OLDER_PCT > 0 && OLDER_PCT < 100),
                      "wave pairs");
        int it0, n_it, stride;
        if constexpr (OLDER_PCT == 0) {
            const int T_it = (nrows + ROWS_IT - 1) / ROWS_IT;
            it0 = w;
            n_it = w < T_it ? (T_it - w + NW - 1) / NW : 0;
            stride = NW;
        } else {
            const int T_it = (nrows + ROWS_IT - 1) / ROWS_IT;
            const int half = NW / 2, pr = w % half;
            const int p0 = (int)((int64_t)T_it * pr / half);
            const int p1 = (int)((int64_t)T_it * (pr + 1) / half);
            const int cut = p0 + ((p1 - p0) * OLDER_PCT + 50) / 100;
            it0 = w < half ? p0 : cut;
            n_it = w < half ? cut - p0 : p1 - cut;
            stride = 1;
        }
        const int step = stride * ROWS_IT;
        uint32_t rid[U];
        int base = it0 * ROWS_IT;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int f = base + u * RPW + rsub;
            rid[u] = n_it > 0 && f < nrows ? rowfn(f) : kBadRow;
        }
        // The SIMDs serve their waves oldest first, so of equal shares the
        // youngest wave of each SIMD finishes last.  A wave's issue priority
        // steps down 3 -> 0 as it gets through the quarters of its share, so
        // a wave that is behind outranks one that is ahead (measurably
        // faster; scheduling only, the bits are unchanged).
        int lvl = 0;
        __builtin_amdgcn_s_setprio(3);
        for (int it = 0; it < n_it; base += step, ++it) {
            const int nl = (4 * it >= n_it) + (4 * it >= 2 * n_it) + (4 * it >= 3 * n_it);
            if (nl != lvl) {
                lvl = nl;
                if (lvl == 1) __builtin_amdgcn_s_setprio(2);
                else if (lvl == 2) __builtin_amdgcn_s_setprio(1);
                else __builtin_amdgcn_s_setprio(0);
            }
            uint4 kr[U], vr[U];
            bool ok[U];
            bool mine = true;
#pragma unroll
            for (int u = 0; u < U; ++u) mine &= rid[u] != kBadRow;
            // the usual iteration: every row of the wave exists (a uniform
            // branch), so loads and softmax need no per-row masks
            if (__ballot(!mine) == 0ull) {
                load_rows_all(rid, k_pool, v_pool, kr, vr);
#pragma unroll
                for (int u = 0; u < U; ++u) ok[u] = true;
            } else {
                load_rows(rid, k_pool, v_pool, kr, vr, ok);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int f = base + step + u * RPW + rsub;
                rid[u] = it + 1 < n_it && f < nrows ? rowfn(f) : kBadRow;
            }
            consume(kr, vr, ok);
        }
        __builtin_amdgcn_s_setprio(0);
    }

    // Streams rows [0, nrows) of row_s (visible to the block), double
    // buffered: each wave issues its next iteration's loads before it
    // consumes the current rows (the pipelined attention variants; the
    // others use stream_fn).
    __device__ __forceinline__ void stream(const uint32_t *row_s, int nrows, const T *k_pool,
                                           const T *v_pool) {
        static_assert(PIPE, "the unpipelined form streams through stream_fn");
        const int step = NW * ROWS_IT;
        uint4 kn[U], vn[U];
        bool okn[U];
        int base = w * ROWS_IT;
        issue(row_s, nrows, k_pool, v_pool, base, kn, vn, okn);
        for (; base < nrows; base += step) {
            uint4 kr[U], vr[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                kr[u] = kn[u];
                vr[u] = vn[u];
                ok[u] = okn[u];
            }
            if (base + step < nrows) issue(row_s, nrows, k_pool, v_pool, base + step, kn, vn, okn);
            consume(kr, vr, ok);
        }
    }

    // Merges the row groups of each wave (they share the running maximum, so
    // their sums simply add) and stores the waves' states in LDS.  The caller
    // synchronises the block before combine().
    template <int OFF>
    __device__ __forceinline__ void merge_groups() {
        if constexpr (OFF < kWave) {
#pragma unroll
            for (int j = 0; j < G; ++j) {
                l[j] = pair_sum<OFF>(l[j]);
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[j][e] = pair_sum<OFF>(acc[j][e]);
            }
            merge_groups<OFF * 2>();
        }
    }

    // With four row groups of 16 lanes, four values are summed over the row
    // groups with three lane swaps: a 16-lane swap of (a, b) and of (c, d)
    // gives rows {a01, b01, a23, b23} and {c01, d01, c23, d23} (xy = the sum
    // of rows x and y, lower row first), and a 32-lane swap of those two
    // gives the totals of a, b, c and d in rows 0..3, added in the same
    // order as pair sums over 16 and then 32 lanes.
    static __device__ __forceinline__ float sum4_rows(float a, float b, float c, float d) {
        const auto ab = __builtin_amdgcn_permlane16_swap((int)__float_as_uint(a),
                                                         (int)__float_as_uint(b), false, false);
        const auto cd = __builtin_amdgcn_permlane16_swap((int)__float_as_uint(c),
                                                         (int)__float_as_uint(d), false, false);
        const float t = __uint_as_float((uint32_t)ab[0]) + __uint_as_float((uint32_t)ab[1]);
        const float u = __uint_as_float((uint32_t)cd[0]) + __uint_as_float((uint32_t)cd[1]);
        const auto tu = __builtin_amdgcn_permlane32_swap((int)__float_as_uint(t),
                                                         (int)__float_as_uint(u), false, false);
        return __uint_as_float((uint32_t)tu[0]) + __uint_as_float((uint32_t)tu[1]);
    }

    __device__ __forceinline__ void to_shared(Shared &sh) {
        if constexpr (LPR == 16 && G % 4 == 0) {
            // row group r of lane ends with head 4*hg + r's totals: its EPL
            // channels, then its softmax sum
#pragma unroll
            for (int hg = 0; hg < G / 4; ++hg) {
                float tot[EPL];
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    tot[e] = sum4_rows(acc[4 * hg][e], acc[4 * hg + 1][e], acc[4 * hg + 2][e],
                                       acc[4 * hg + 3][e]);
                const float lt = sum4_rows(l[4 * hg], l[4 * hg + 1], l[4 * hg + 2], l[4 * hg + 3]);
                const int j = 4 * hg + rsub;
                float4 *dst = (float4 *)&sh.wacc[w][j][sub * EPL];
#pragma unroll
                for (int e = 0; e < EPL; e += 4)
                    dst[e / 4] = make_float4(tot[e], tot[e + 1], tot[e + 2], tot[e + 3]);
                if (sub == 0) sh.wl[w][j] = lt;
            }
            if (lane == 0) {
#pragma unroll
                for (int j = 0; j < G; ++j) sh.wm[w][j] = m[j];
            }
        } else {
            merge_groups<LPR>();
            if (rsub == 0) {
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    if (sub == 0) {
                        sh.wm[w][j] = m[j];
                        sh.wl[w][j] = l[j];
                    }
#pragma unroll
                    for (int e = 0; e < EPL; ++e) sh.wacc[w][j][sub * EPL + e] = acc[j][e];
                }
            }
        }
    }

    // Combines the waves in wave order: fn(j, c, max, sum, acc_c, acc_c+1)
    // once per (head, channel pair) across the block.
    template <typename Fn>
    static __device__ __forceinline__ void combine(const Shared &sh, Fn fn) {
        static_assert(D % 2 == 0, "channel pairs");
        for (int t = threadIdx.x; t < G * D / 2; t += NW * kWave) {
            const int j = t / (D / 2), c = 2 * (t % (D / 2));
            float M = -INFINITY;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sh.wm[ww][j]);
            float Ls = 0.0f, A0 = 0.0f, A1 = 0.0f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                const float cw = exp2_diff(sh.wm[ww][j], M);
                const float2 x = *(const float2 *)&sh.wacc[ww][j][c];
                Ls += sh.wl[ww][j] * cw;
                A0 += x.x * cw;
                A1 += x.y * cw;
            }
            fn(j, c, M, Ls, A0, A1);
        }
    }
};

}  // namespace rkv
