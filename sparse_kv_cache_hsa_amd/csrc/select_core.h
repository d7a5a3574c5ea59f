// select_core.h -- device building blocks of HSA selection, shared by the
// selection kernel and the fused decode kernel so both compute identical bits.
//
// "RocketKV-adapted -- Two-Stage Compression", section "Where it sits": the
// score is approximated with SparQ-style top-magnitude channels (head
// dimension) and Quest-style page max/min summaries (sequence dimension),
// giving a per-page bound; "Adaptation notes": k2 whole pages are kept.
//   channel rank : a[c] = sum_j |q_j[c]| (fp32, heads ascending, from +0),
//                  the k1 largest (ties to the lower channel), ascending;
//   page bound   : s_j(p) = sum_{c in I1 asc} max(q_j[c]*Kmax[p][c],
//                  q_j[c]*Kmin[p][c]); S(p) = sum_{j asc} s_j(p), all plain
//                  fp32 operations (this library is built without
//                  multiply-add contraction);
//   page top-k   : the min(k2, NP) largest S (ties to the lower page),
//                  reported in ascending page order.
// Rankings use 64-bit composite keys (order-preserving 32-bit score key in
// the high word, complemented index in the low word), so "larger key" is
// exactly "higher score, then lower index" and every comparison is one
// unsigned 64-bit compare.
#pragma once

#include <type_traits>

#include "rkv_internal.h"

namespace rkv {

__device__ __forceinline__ uint64_t composite_key(uint32_t key, int index) {
    return ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)index);
}

// q rows of the G query heads of KV head (b, h) into LDS as fp32.
template <typename T, int D, int G, int BLOCK>
__device__ __forceinline__ void load_group_q(const T *q, int64_t bh, float (*qs)[D]) {
    for (int i = threadIdx.x; i < G * D; i += BLOCK) qs[i / D][i % D] = Elem<T>::ld(q, bh * G * D + i);
}

// ---- top-k by per-wave sorting ----------------------------------------------
template <int J>
__device__ __forceinline__ uint64_t key_xor(uint64_t v) {
    const uint32_t lo = lane_xor<J>((uint32_t)v);
    const uint32_t hi = lane_xor<J>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

template <int J>
__device__ __forceinline__ uint32_t key_xor(uint32_t v) {
    return lane_xor<J>(v);
}

// One compare-exchange stage of a descending bitonic network at distance J:
// the lane keeps the larger key when `up`, the smaller one otherwise.
template <int J, typename K>
__device__ __forceinline__ K bitonic_stage(K key, bool up) {
    const K other = key_xor<J>(key);
    return (up == (other > key)) ? other : key;
}

// Merge of size M (stages J = M/2 .. 1) of the full sort network.
template <int M, int J, typename K>
__device__ __forceinline__ K bitonic_merge(K key, int lane) {
    key = bitonic_stage<J>(key, ((lane & M) == 0) == ((lane & J) == 0));
    if constexpr (J > 1) key = bitonic_merge<M, J / 2>(key, lane);
    return key;
}

// Half-cleaner cascade that sorts a bitonic wave sequence descending.
template <int J, typename K>
__device__ __forceinline__ K bitonic_clean(K key, int lane) {
    key = bitonic_stage<J>(key, (lane & J) == 0);
    if constexpr (J > 1) key = bitonic_clean<J / 2>(key, lane);
    return key;
}

// Sorts the 64 keys of a wave in descending order (lane i gets the i-th
// largest).  Distances 1 to 8 move through DPP (one or two lane moves),
// 16 and 32 through the lane swaps.
template <typename K>
__device__ __forceinline__ K wave_sort_desc(K key) {
    const int lane = threadIdx.x & (kWave - 1);
    key = bitonic_merge<2, 1>(key, lane);
    key = bitonic_merge<4, 2>(key, lane);
    key = bitonic_merge<8, 4>(key, lane);
    key = bitonic_merge<16, 8>(key, lane);
    key = bitonic_merge<32, 16>(key, lane);
    key = bitonic_merge<64, 32>(key, lane);
    return key;
}

// ---- top-k inside one wave by a ballot threshold search ---------------------
// The keys are unsigned words held by the 64 lanes of one wave, E slots per
// lane: slot e of lane l holds the key of index e*64 + l, for indices below n;
// every other slot must hold 0.  A threshold T with at least K keys >= T
// (1 <= K <= n) is raised bit by bit from the top, a bit kept whenever at
// least K keys stay >= T (counted with ballots), until exactly K keys are
// >= T or every bit is decided (T is then the K-th largest key).  The top K
// by (key desc, index asc) are the keys > T and the lowest-indexed keys equal
// to T; emit(pos, index) writes them in ascending index order, so no sort is
// needed.  Only the calling wave takes part; no barrier.
template <int E, typename Emit>
__device__ __forceinline__ void wave_topk(const uint32_t (&key)[E], int n, int K, Emit emit) {
    const int lane = threadIdx.x & (kWave - 1);
    // lanes below this one among the set bits of a wave mask
    auto below_cnt = [](uint64_t m) {
        return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    };
    // The bits above the highest one in which two keys differ are common to
    // all of them, so T starts with them (wave-wide OR and AND of the keys;
    // the slots past n hold 0 and are left out of the AND).
    uint32_t k_or = 0u, k_and = ~0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        k_or |= key[e];
        if (e * kWave + lane < n) k_and &= key[e];
    }
    k_or |= lane_xor<1>(k_or);
    k_and &= lane_xor<1>(k_and);
    k_or |= lane_xor<2>(k_or);
    k_and &= lane_xor<2>(k_and);
    k_or |= lane_xor<4>(k_or);
    k_and &= lane_xor<4>(k_and);
    k_or |= lane_xor<8>(k_or);
    k_and &= lane_xor<8>(k_and);
    k_or |= lane_xor<16>(k_or);
    k_and &= lane_xor<16>(k_and);
    k_or |= lane_xor<32>(k_or);
    k_and &= lane_xor<32>(k_and);
    k_or = (uint32_t)__builtin_amdgcn_readfirstlane((int)k_or);
    k_and = (uint32_t)__builtin_amdgcn_readfirstlane((int)k_and);
    const uint32_t diff = k_or ^ k_and;
    const int top = diff ? 31 - __builtin_clz(diff) : -1;
    // all keys equal above bit `top` (all equal: top = -1, T is that key)
    uint32_t T = top < 0 ? k_and : (top == 31 ? 0u : (k_and & ~((2u << top) - 1u)));
    // Then bit by bit below that.  The slots past n hold 0 and never reach a
    // candidate (every candidate is above 0), so the counting needs no
    // guards.  All compares of a candidate are issued before any count reads
    // them, so the scalar counts wait for the vector compares once.
    // (in groups of four slots, which bounds the scalar registers held).
    // The search stops early once exactly K keys are >= T: they are then the
    // top K whatever the lower bits of T, and the selection below takes them
    // all (count(key > T) + count(key == T) = K).
    constexpr int GS = E < 4 ? E : 4;
    int cnt_T = n;  // count(key >= T)
    int bit = top;
    if constexpr (E <= 2) {
        // few keys per lane: two bits per round, the three candidates of
        // bits (bit, bit-1) counted together and the largest that keeps K
        // keys taken (the same T as two one-bit rounds), which halves the
        // chain of dependent rounds
        for (; bit >= 1 && cnt_T != K; bit -= 2) {
            const uint32_t c1 = T | (1u << (bit - 1)), c2 = T | (2u << (bit - 1)),
                           c3 = T | (3u << (bit - 1));
            uint64_t m1[E], m2[E], m3[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                m1[e] = __ballot(key[e] >= c1);
                m2[e] = __ballot(key[e] >= c2);
                m3[e] = __ballot(key[e] >= c3);
            }
            __builtin_amdgcn_sched_barrier(0);
            int n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                n1 += __popcll(m1[e]);
                n2 += __popcll(m2[e]);
                n3 += __popcll(m3[e]);
            }
            if (n3 >= K) {
                T = c3;
                cnt_T = n3;
            } else if (n2 >= K) {
                T = c2;
                cnt_T = n2;
            } else if (n1 >= K) {
                T = c1;
                cnt_T = n1;
            }
        }
    }
    for (; bit >= 0 && cnt_T != K; --bit) {
        const uint32_t cand = T | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int e0 = 0; e0 < E; e0 += GS) {
            uint64_t m[GS];
#pragma unroll
            for (int e = 0; e < GS; ++e) m[e] = __ballot(key[e0 + e] >= cand);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < GS; ++e) cnt += __popcll(m[e]);
        }
        if (cnt >= K) {
            T = cand;
            cnt_T = cnt;
        }
    }
    if (cnt_T == K) {
        // exactly K keys are >= T (T > 0 whenever the search moved it, and
        // every key when K = n), so they are the top K: no tie handling
        int base = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (e * kWave >= n) break;
            const bool sel = e * kWave + lane < n && key[e] >= T;
            const uint64_t sm = __ballot(sel);
            if (sel) emit(base + below_cnt(sm), e * kWave + lane);
            base += __popcll(sm);
        }
        return;
    }
    int gt_tot = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) gt_tot += __popcll(__ballot(key[e] > T));
    const int take_eq = K - gt_tot;
    int base = 0, eq_seen = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (e * kWave >= n) break;
        const bool valid = e * kWave + lane < n;
        const bool eq = valid && key[e] == T;
        const uint64_t em = __ballot(eq);
        const bool sel = (valid && key[e] > T) || (eq && eq_seen + below_cnt(em) < take_eq);
        const uint64_t sm = __ballot(sel);
        if (sel) emit(base + below_cnt(sm), e * kWave + lane);
        base += __popcll(sm);
        eq_seen += __popcll(em);
    }
}

// wave_topk over n <= 16 * 64 keys in LDS (keys_s[i] for i < n; entries
// from n up to the next multiple of 64 must be 0), run by the calling wave
// with the smallest slot count that holds them.
template <typename Emit>
__device__ __forceinline__ void wave_topk_lds(const uint32_t *keys_s, int n, int K, Emit emit) {
    const int lane = threadIdx.x & (kWave - 1);
    const int ne = (n + kWave - 1) / kWave;
    auto run = [&](auto tag) {
        constexpr int E = decltype(tag)::value;
        uint32_t key[E];
#pragma unroll
        for (int e = 0; e < E; ++e) key[e] = e < ne ? keys_s[e * kWave + lane] : 0u;
        wave_topk<E>(key, n, K, emit);
    };
    if (ne <= 1) run(std::integral_constant<int, 1>{});
    else if (ne <= 2) run(std::integral_constant<int, 2>{});
    else if (ne <= 4) run(std::integral_constant<int, 4>{});
    else if (ne <= 8) run(std::integral_constant<int, 8>{});
    else run(std::integral_constant<int, 16>{});
}

// Channel ranking by the block's first wave (the work is 2*D small ballot
// steps, cheaper than spreading it over the block and synchronising).  qs
// must be visible to the block.  On return ch_s[0..k1) holds the chosen
// channels in ascending order and qsel[j][i] = qs[j][ch_s[i]]; if qpm is
// given (bf16 queries), also the sign-split queries of staged_bound_exact,
// qpm[i * 2G + j] = max(q, 0) and qpm[i * 2G + G + j] = min(q, 0) for
// q = qsel[j][i].  All threads must call it; ends with a block barrier.
template <int D, int G>
__device__ __forceinline__ void rank_channels_wave(const float (*qs)[D], int k1, int *ch_s,
                                                   float (*qsel)[D], float *qpm = nullptr) {
    static_assert(D % kWave == 0, "head_dim");
    constexpr int E = D / kWave;
    static_assert(E == 1 || E == 2, "head_dim 64 or 128");
    if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        // this lane's channels (lane, kWave + lane) of every head, kept for
        // the emission: a lane emits only its own channels
        float q0[G], q1[G];
        uint32_t key[E];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            q0[j] = qs[j][lane];
            q1[j] = E == 2 ? qs[j][(E - 1) * kWave + lane] : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < G; ++j) acc = acc + fabsf(e == 0 ? q0[j] : q1[j]);
            // acc >= +0, so its bits order like its value
            key[e] = __float_as_uint(acc);
        }
        wave_topk<E>(key, D, k1, [&](int o, int c) {
            ch_s[o] = c;
            const bool second = c >= kWave;
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const float qv = second ? q1[j] : q0[j];
                qsel[j][o] = qv;
                if (qpm) {
                    // by sign bit, so -0 goes to the Kmin side (both sides
                    // give a zero product there)
                    const bool neg = __float_as_uint(qv) >> 31;
                    qpm[o * 2 * G + j] = neg ? 0.0f : qv;
                    qpm[o * 2 * G + G + j] = neg ? qv : 0.0f;
                }
            }
        });
    }
    lds_barrier();
}

// Rank count for n <= BLOCK composite keys comp_s[0..n) (LDS): cnt_s[i] =
// the number of keys larger than key i.  Every key is compared with every
// other, the comparisons of one key spread over BLOCK/n threads.  cnt_s is
// LDS scratch of n ints.  All threads must call it; comp_s must be visible
// to the block; cnt_s is visible to the block on return.
template <int BLOCK>
__device__ void rank_count(const uint64_t *comp_s, int n, int *cnt_s) {
    const int tid = threadIdx.x;
    const int npad = (n + kWave - 1) / kWave * kWave;
    int parts = npad > 0 ? BLOCK / npad : 1;
    parts = parts < 1 ? 1 : (parts > 8 ? 8 : parts);
    if (parts > 1) {
        for (int i = tid; i < n; i += BLOCK) cnt_s[i] = 0;
        lds_barrier();
    }
    const int i = tid % npad, part = tid / npad;
    if (part < parts && i < n) {
        const uint64_t key = comp_s[i];
        const int chunk = (n + parts - 1) / parts;
        const int j0 = part * chunk, j1 = min(n, j0 + chunk);
        int c = 0;
#pragma unroll 8
        for (int j = j0; j < j1; ++j) c += comp_s[j] > key;
        if (parts > 1) atomicAdd(&cnt_s[i], c);
        else cnt_s[i] = c;
    }
    lds_barrier();
}

// Top-K by rank count: emit(pos, i) for the K largest of comp_s[0..n),
// i ascending.  Same contract as rank_count.
template <int BLOCK, typename Emit>
__device__ void rank_topk(const uint64_t *comp_s, int n, int K, int *cnt_s, int *wave_tot,
                          Emit emit) {
    constexpr int NW = BLOCK / kWave;
    const int tid = threadIdx.x;
    rank_count<BLOCK>(comp_s, n, cnt_s);
    const bool sel = tid < n && cnt_s[tid] < K;
    int tot;
    const int pos = block_excl_count<NW>(sel, wave_tot, tot);
    if (sel) emit(pos, tid);
}

// Page bound S(p).  smax/smin point at channel 0 of the (b, h) summaries;
// channel c of page p sits at c * max_pages + p.  The summary pairs of a
// batch of up to 32 channels are loaded before use, so one memory round trip
// serves the batch.
template <typename T, int D, int G>
__device__ __forceinline__ float page_bound(const T *smax, const T *smin, int max_pages, int p,
                                            const int *ch_s, int k1, const float (*qsel)[D]) {
    constexpr int CB = 32;
    float s[G];
#pragma unroll
    for (int j = 0; j < G; ++j) s[j] = 0.0f;
    for (int i0 = 0; i0 < k1; i0 += CB) {
        float hi_v[CB], lo_v[CB];
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            const int i = i0 + u;
            const int c = __builtin_amdgcn_readfirstlane(ch_s[i < k1 ? i : 0]);
            hi_v[u] = Elem<T>::ld(smax, (int64_t)c * max_pages + p);
            lo_v[u] = Elem<T>::ld(smin, (int64_t)c * max_pages + p);
        }
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            if (i0 + u < k1) {
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    const float qc = qsel[j][i0 + u];
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
    return tot;
}

// Page bound of a page whose summary is held in LDS (ovr_hi/ovr_lo indexed
// by channel), same arithmetic and order as page_bound.
template <typename T, int D, int G>
__device__ __forceinline__ float page_bound_ovr(const int *ch_s, int k1, const float (*qsel)[D],
                                                const T *ovr_hi, const T *ovr_lo) {
    float s[G];
#pragma unroll
    for (int j = 0; j < G; ++j) s[j] = 0.0f;
    for (int i = 0; i < k1; ++i) {
        const float hv = Elem<T>::ld(ovr_hi, ch_s[i]);
        const float lv = Elem<T>::ld(ovr_lo, ch_s[i]);
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float qc = qsel[j][i];
            const float hi = qc * hv;
            const float lo = qc * lv;
            s[j] = s[j] + (hi > lo ? hi : lo);
        }
    }
    float tot = 0.0f;
#pragma unroll
    for (int j = 0; j < G; ++j) tot = tot + s[j];
    return tot;
}

// Top-K of comp_s[0..n) (composite keys, LDS) with emit(pos, i), i
// ascending.  Up to BLOCK keys use the rank count, more a 4-pass radix
// select on the score word (ties then resolve to the lower index).  All
// threads must call it; comp_s must be visible to the block.
template <int BLOCK, typename Emit>
__device__ void topk_ascending(const uint64_t *comp_s, int n, int K, int *cnt_s, uint32_t *hist,
                               int *sh, int *wave_tot, Emit emit) {
    if (K <= 0) return;
    if (n <= BLOCK) {
        rank_topk<BLOCK>(comp_s, n, K, cnt_s, wave_tot, emit);
        return;
    }
    uint32_t thr;
    int take_eq;
    auto load = [&](int i) { return (uint32_t)(comp_s[i] >> 32); };
    block_topk_threshold<BLOCK>(load, n, K, hist, sh, thr, take_eq);
    block_topk_emit<BLOCK>(load, n, thr, take_eq, wave_tot, emit);
}


// ---- staged page bounds ------------------------------------------------------
// Copies the summaries of the k1 chosen channels for pages [p0, p0 + n) into
// LDS as stage[kind][i][p - p0] (kind 0 = max, 1 = min) with row stride npad,
// using the direct global-to-LDS loads of gfx950: no register round trip, so
// every load of the block is in flight at once and one wait ends the copy.
// The stage is a contiguous run of E-element chunks (E = 8 bf16 / 4 fp32 when
// every row is 16-byte aligned, else 1), chunk t at element t * E, which is
// the per-lane destination pattern of these loads: a wave's 64 consecutive
// chunks land in 64 consecutive slots.  Returns npad (n rounded up to E).
// The caller synchronises the block afterwards (lds_barrier).
template <typename T, int E, int BLOCK>
__device__ __forceinline__ void stage_rows(const T *smax, const T *smin, int max_pages, int p0,
                                           int nv, const int *ch_s, int k1, T *stage) {
    typedef __attribute__((address_space(3))) void lds_void;
    const int total = 2 * k1 * nv;
    const int lane = threadIdx.x & (kWave - 1);
    for (int base = threadIdx.x - lane; base < total; base += BLOCK) {
        const int t = base + lane;
        if (t < total) {
            const int row = t / nv, vi = t - row * nv;
            const int kind = row / k1, i = row - kind * k1;
            const T *src = (kind ? smin : smax) + (int64_t)ch_s[i] * max_pages + p0 + vi * E;
            // The byte count must be an int constant: a size_t expression
            // crashes this compiler's instruction selection.  Cache policy
            // 2 is the non-temporal hint: the summaries are read once per
            // step.
            __builtin_amdgcn_global_load_lds(src, (lds_void *)(stage + (int64_t)base * E),
                                             (int)(E * sizeof(T)), 0, 2);
        }
    }
}

// dst[i] = src[i] for i < n (int32, dst in LDS) with direct global-to-LDS
// loads; the caller waits for them (vmcnt) and synchronises the block.
template <int BLOCK>
__device__ __forceinline__ void dma_copy_i32(const int32_t *src, int n, int32_t *dst) {
    typedef __attribute__((address_space(3))) void lds_void;
    const int lane = threadIdx.x & (kWave - 1);
    for (int base = threadIdx.x - lane; base < n; base += BLOCK)
        if (base + lane < n)
            __builtin_amdgcn_global_load_lds(src + base + lane, (lds_void *)(dst + base), 4, 0, 0);
}

// One 16-byte direct global-to-LDS load per lane: the calling wave's
// lanes land at consecutive 16-byte slots from dst (wave-uniform).
// Non-temporal (cache policy 2).
__device__ __forceinline__ void lds_load16_nt(const void *src, void *dst) {
    typedef __attribute__((address_space(3))) void lds_void;
    __builtin_amdgcn_global_load_lds(src, (lds_void *)dst, 16, 0, 2);
}

template <typename T, int BLOCK>
__device__ __forceinline__ int stage_summaries(const T *smax, const T *smin, int max_pages, int p0,
                                               int n, const int *ch_s, int k1, T *stage) {
    constexpr int V = 16 / (int)sizeof(T);
    const bool vec = (max_pages % V) == 0 && (p0 % V) == 0 &&
                     (((uintptr_t)smax) & 15u) == 0 && (((uintptr_t)smin) & 15u) == 0;
    int npad;
    if (vec) {
        const int nv = (n + V - 1) / V;
        stage_rows<T, V, BLOCK>(smax, smin, max_pages, p0, nv, ch_s, k1, stage);
        npad = nv * V;
    } else if constexpr (sizeof(T) == 4) {
        stage_rows<T, 1, BLOCK>(smax, smin, max_pages, p0, n, ch_s, k1, stage);
        npad = n;
    } else {
        // Sub-dword direct loads fill a dword per lane, which does not match
        // this packing; copy through registers instead.
        for (int t = threadIdx.x; t < 2 * k1 * n; t += BLOCK) {
            const int row = t / n, pi = t - row * n;
            const int kind = row / k1, i = row - kind * k1;
            stage[t] = (kind ? smin : smax)[(int64_t)ch_s[i] * max_pages + p0 + pi];
        }
        npad = n;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
    return npad;
}

// Page bound S(p) from staged summaries (same arithmetic and order as
// page_bound).
template <typename T, int D, int G>
__device__ __forceinline__ float staged_bound(const T *stage, int npad, int p, int k1,
                                              const float (*qsel)[D]) {
    float s[G];
#pragma unroll
    for (int j = 0; j < G; ++j) s[j] = 0.0f;
    const T *hi_row = stage + p;
    const T *lo_row = stage + (int64_t)k1 * npad + p;
    for (int i = 0; i < k1; ++i) {
        const float hv = Elem<T>::ld(hi_row, (int64_t)i * npad);
        const float lv = Elem<T>::ld(lo_row, (int64_t)i * npad);
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float qc = qsel[j][i];
            const float hi = qc * hv;
            const float lo = qc * lv;
            s[j] = s[j] + (hi > lo ? hi : lo);
        }
    }
    float tot = 0.0f;
#pragma unroll
    for (int j = 0; j < G; ++j) tot = tot + s[j];
    return tot;
}

// bf16 page bound from staged summaries with fused multiply-adds.  For bf16
// q and K every product q*K is exact in fp32, so fma(q, K, s) is s + q*K
// rounded once, exactly the plain s + fl(q*K).  max(q*Kmax, q*Kmin) is q*Kmax
// when q >= 0 and q*Kmin when q < 0; with q+ = max(q, 0) and q- = min(q, 0)
// the two updates s = fma(q+, Kmax, s), s = fma(q-, Kmin, s) add that term
// and a zero product (which leaves a sum that starts at +0 unchanged), so
// S(p) has the same bits as staged_bound.
template <int G>
__device__ __forceinline__ float staged_bound_exact(const uint16_t *stage, int npad, int p, int k1,
                                                    const float *qpm) {
    float s[G];
#pragma unroll
    for (int j = 0; j < G; ++j) s[j] = 0.0f;
    const uint16_t *hi_row = stage + p;
    const uint16_t *lo_row = stage + (int64_t)k1 * npad + p;
    for (int i = 0; i < k1; ++i) {
        const float hv = __uint_as_float((uint32_t)hi_row[(int64_t)i * npad] << 16);
        const float lv = __uint_as_float((uint32_t)lo_row[(int64_t)i * npad] << 16);
        const float *qi = qpm + i * 2 * G;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            s[j] = __builtin_fmaf(qi[j], hv, s[j]);
            s[j] = __builtin_fmaf(qi[G + j], lv, s[j]);
        }
    }
    float tot = 0.0f;
#pragma unroll
    for (int j = 0; j < G; ++j) tot = tot + s[j];
    return tot;
}

// staged_bound_exact (same arithmetic and order) for K1 channels staged
// with the fixed row stride SR: every LDS offset is a constant, so the
// unrolled loop spends no instructions on addresses.
template <int G, int K1, int SR>
__device__ __forceinline__ float staged_bound_fixed(const uint16_t *stage, int p, const float *qpm) {
    float s[G];
#pragma unroll
    for (int j = 0; j < G; ++j) s[j] = 0.0f;
    const uint16_t *hi_row = stage + p;
    const uint16_t *lo_row = stage + K1 * SR + p;
    // the query table's address in a vector register (an opaque zero), so
    // its reads take constant offsets from one base
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    const float *qb = (const float *)__builtin_assume_aligned((const char *)qpm + z, 16);
#pragma unroll
    for (int i = 0; i < K1; ++i) {
        const float hv = __uint_as_float((uint32_t)hi_row[i * SR] << 16);
        const float lv = __uint_as_float((uint32_t)lo_row[i * SR] << 16);
        float qi[2 * G];
        if constexpr ((2 * G) % 4 == 0) {
#pragma unroll
            for (int u = 0; u < 2 * G / 4; ++u) {
                const float4 v4 = ((const float4 *)qb)[i * (2 * G / 4) + u];
                qi[4 * u] = v4.x;
                qi[4 * u + 1] = v4.y;
                qi[4 * u + 2] = v4.z;
                qi[4 * u + 3] = v4.w;
            }
        } else {
#pragma unroll
            for (int u = 0; u < 2 * G; ++u) qi[u] = qb[i * 2 * G + u];
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            s[j] = __builtin_fmaf(qi[j], hv, s[j]);
            s[j] = __builtin_fmaf(qi[G + j], lv, s[j]);
        }
    }
    float tot = 0.0f;
#pragma unroll
    for (int j = 0; j < G; ++j) tot = tot + s[j];
    return tot;
}

}  // namespace rkv
