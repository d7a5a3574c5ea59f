// rkv_internal.h -- device helpers and internal launcher declarations shared
// by the librkv translation units.  gfx950 only: 64-lane wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rkv.h"

namespace rkv {

constexpr int kWave = 64;

// ---- element types ------------------------------------------------------
// bf16 is carried as raw uint16_t bits; widening to fp32 is exact.
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

template <typename T>
struct Elem;
template <>
struct Elem<float> {
    static __device__ __forceinline__ float ld(const float *p, int64_t i) { return p[i]; }
};
template <>
struct Elem<uint16_t> {
    static __device__ __forceinline__ float ld(const uint16_t *p, int64_t i) {
        return bf16_to_f32(p[i]);
    }
};

// Unpack one 16-byte vector into fp32 lanes: 4 fp32 or 8 bf16 values.
template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void unpack(const uint4 &u, float *f) {
        f[0] = __uint_as_float(u.x);
        f[1] = __uint_as_float(u.y);
        f[2] = __uint_as_float(u.z);
        f[3] = __uint_as_float(u.w);
    }
};
template <>
struct Vec16<uint16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void unpack(const uint4 &u, float *f) {
        f[0] = __uint_as_float(u.x << 16);
        f[1] = __uint_as_float(u.x & 0xffff0000u);
        f[2] = __uint_as_float(u.y << 16);
        f[3] = __uint_as_float(u.y & 0xffff0000u);
        f[4] = __uint_as_float(u.z << 16);
        f[5] = __uint_as_float(u.z & 0xffff0000u);
        f[6] = __uint_as_float(u.w << 16);
        f[7] = __uint_as_float(u.w & 0xffff0000u);
    }
};

// ---- ordering keys --------------------------------------------------------
// Maps fp32 to uint32 so that unsigned order equals numeric order; -0 and +0
// map to the same key.  Non-finite inputs are outside the contract.
__device__ __forceinline__ uint32_t ordered_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---- block-wide helpers ---------------------------------------------------
// Barrier that orders LDS only: unlike __syncthreads() it does not wait for
// the block's outstanding global stores, so a block that has written optional
// outputs or cache rows can keep going.  Use __syncthreads() whenever threads
// exchange data through global memory.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Exclusive prefix count of `flag` over the threads of the block, in thread
// order.  `wave_tot` is LDS scratch of NW ints.  All threads must call it.
template <int NW>
__device__ __forceinline__ int block_excl_count(bool flag, int *wave_tot, int &total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const uint64_t b = __ballot(flag);
    const uint64_t below = lane ? (b & (~0ull >> (64 - lane))) : 0ull;
    const int in_wave = __popcll(below);
    if (lane == 0) wave_tot[w] = __popcll(b);
    lds_barrier();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int t = wave_tot[i];
        off += (i < w) ? t : 0;
        tot += t;
    }
    lds_barrier();
    total = tot;
    return off + in_wave;
}

// hist[bin] += 1 for the lanes with `on`.  Keys that share their leading
// bytes put most of a wave into one bin, and 64 LDS atomics on one address
// serialise; so the wave first adds the lanes of the most common bins with
// one atomic each (a ballot per distinct bin, a few rounds at most), and
// only the lanes left over add themselves.  The counts are the same.
__device__ __forceinline__ void wave_hist_add(uint32_t *hist, uint32_t bin, bool on) {
    const int lane = threadIdx.x & (kWave - 1);
    uint64_t todo = __ballot(on);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if (todo == 0ull) break;
        const int leader = __ffsll((unsigned long long)todo) - 1;
        const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, leader);
        const uint64_t same = __ballot(on && bin == lb) & todo;
        if (lane == leader) atomicAdd(&hist[lb], (uint32_t)__popcll(same));
        todo &= ~same;
    }
    if ((todo >> lane) & 1ull) atomicAdd(&hist[bin], 1u);
}

// Radix select over the keys u[0..n): finds the K-th largest key `thr`
// (1 <= K <= n) and how many keys equal to `thr` belong to the top K
// (`take_eq`, the lowest-indexed ones).  `hist` is LDS of 256 uint32,
// `sh` LDS of 2 ints.  All threads must call it.  `Load` maps i -> key.
template <int BLOCK, typename Load>
__device__ void block_topk_threshold(Load load, int n, int K, uint32_t *hist, int *sh,
                                     uint32_t &thr, int &take_eq) {
    uint32_t prefix = 0u, mask = 0u;
    int remaining = K;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += BLOCK) hist[i] = 0u;
        lds_barrier();
        for (int i = threadIdx.x; i < n; i += BLOCK) {
            const uint32_t u = load(i);
            wave_hist_add(hist, (u >> shift) & 255u, (u & mask) == prefix);
        }
        lds_barrier();
        if (threadIdx.x < kWave) {
            const int lane = threadIdx.x;
            // lane owns bins 255-4*lane .. 252-4*lane (descending order)
            uint32_t c[4];
            uint32_t mine = 0u;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                c[q] = hist[255 - 4 * lane - q];
                mine += c[q];
            }
            uint32_t incl = mine;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const uint32_t o = __shfl_up(incl, off, kWave);
                if (lane >= off) incl += o;
            }
            const uint32_t excl = incl - mine;
            if (excl < (uint32_t)remaining && (uint32_t)remaining <= incl) {
                uint32_t cum = excl;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (cum + c[q] >= (uint32_t)remaining) {
                        sh[0] = 255 - 4 * lane - q;
                        sh[1] = (int)cum;
                        break;
                    }
                    cum += c[q];
                }
            }
        }
        lds_barrier();
        const uint32_t digit = (uint32_t)sh[0];
        remaining -= sh[1];
        prefix |= digit << shift;
        mask |= 255u << shift;
        lds_barrier();
    }
    thr = prefix;
    take_eq = remaining;
}

// Writes, in ascending index order, the indices of the top-K keys found by
// block_topk_threshold: emit(pos, i) for pos = 0..K-1.
template <int BLOCK, typename Load, typename Emit>
__device__ void block_topk_emit(Load load, int n, uint32_t thr, int take_eq, int *wave_tot,
                                Emit emit) {
    int eq_base = 0, sel_base = 0;
    for (int i0 = 0; i0 < n; i0 += BLOCK) {
        const int i = i0 + threadIdx.x;
        const uint32_t u = i < n ? load(i) : 0u;
        const bool eq = (i < n) && (u == thr);
        int eq_tot;
        const int eq_rank = eq_base + block_excl_count<BLOCK / kWave>(eq, wave_tot, eq_tot);
        const bool sel = (i < n) && (u > thr || (eq && eq_rank < take_eq));
        int sel_tot;
        const int pos = sel_base + block_excl_count<BLOCK / kWave>(sel, wave_tot, sel_tot);
        if (sel) emit(pos, i);
        eq_base += eq_tot;
        sel_base += sel_tot;
    }
}

// 2^x with the hardware exponential (about 1 ulp; results below the
// smallest normal may flush to zero, which only drops softmax weights under
// 2^-126).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A store written through the caches to memory (a relaxed system-scope
// atomic store: sc0 sc1 on gfx950).  Scattered small results of a kernel
// stored this way leave no dirty L2 lines behind, which the end of the
// launch would otherwise have to write back before the next kernel starts.
template <typename T>
__device__ __forceinline__ void store_through(T *p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// The two values of lanes (lane & ~OFF, lane | OFF) of a 64-lane wave, for
// OFF = 16 or 32, in every lane: `lo` from the lower lane, `hi` from the
// upper one (the gfx950 lane-swap instructions, vector ALU only).
template <int OFF>
__device__ __forceinline__ void lane_pair(uint32_t v, uint32_t &lo, uint32_t &hi) {
    static_assert(OFF == 16 || OFF == 32, "offset");
    if constexpr (OFF == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap((int)v, (int)v, false, false);
        lo = (uint32_t)r[0];
        hi = (uint32_t)r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap((int)v, (int)v, false, false);
        lo = (uint32_t)r[0];
        hi = (uint32_t)r[1];
    }
}

// Value of lane (lane ^ OFF) of a 64-lane wave, all in the vector ALU:
//   1, 2 : one DPP quad permute ([1,0,3,2], [2,3,0,1]);
//   4    : row half-mirror (lane i of each 8 takes lane 7-i), then the
//          reversing quad permute [3,2,1,0]: lane l ends with lane
//          hm(l ^ 3 within its quad) = l ^ 4;
//   8    : row mirror (lane i of each 16 takes lane 15-i), then the half-
//          mirror: lane l ends with lane 15 - hm(l) = l ^ 8;
//   16, 32: the gfx950 lane swaps.
// (DPP controls: quad_perm = the 8-bit source map, row_mirror 0x140,
// row_half_mirror 0x141.)
template <int OFF>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
    static_assert(OFF == 1 || OFF == 2 || OFF == 4 || OFF == 8 || OFF == 16 || OFF == 32, "offset");
    if constexpr (OFF == 1) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, true);
    } else if constexpr (OFF == 2) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, true);
    } else if constexpr (OFF == 4) {
        const int h = __builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, true);
        return (uint32_t)__builtin_amdgcn_update_dpp(0, h, 0x1B, 0xf, 0xf, true);
    } else if constexpr (OFF == 8) {
        const int m = __builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, true);
        return (uint32_t)__builtin_amdgcn_update_dpp(0, m, 0x141, 0xf, 0xf, true);
    } else {
        uint32_t lo, hi;
        lane_pair<OFF>(v, lo, hi);
        return (threadIdx.x & OFF) ? lo : hi;
    }
}

// v(lane) + v(lane ^ OFF), the same bits in both lanes (lower lane's value
// first).
template <int OFF>
__device__ __forceinline__ float pair_sum(float v) {
    if constexpr (OFF >= 16) {
        uint32_t lo, hi;
        lane_pair<OFF>(__float_as_uint(v), lo, hi);
        return __uint_as_float(lo) + __uint_as_float(hi);
    } else {
        const float o = __uint_as_float(lane_xor<OFF>(__float_as_uint(v)));
        return (threadIdx.x & OFF) ? o + v : v + o;
    }
}

template <int OFF>
__device__ __forceinline__ float pair_max(float v) {
    if constexpr (OFF >= 16) {
        uint32_t lo, hi;
        lane_pair<OFF>(__float_as_uint(v), lo, hi);
        return fmaxf(__uint_as_float(lo), __uint_as_float(hi));
    } else {
        return fmaxf(v, __uint_as_float(lane_xor<OFF>(__float_as_uint(v))));
    }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// a.lo*b.lo + a.hi*b.hi + c for bf16 pairs a, b (products of bf16 values are
// exact in fp32; fp32 accumulation).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float exp2_diff(float a, float b) {
    // exp2(a - b) with exp2(-inf - x) = 0, also when both are -inf.
    return (a == -INFINITY) ? 0.0f : fast_exp2(a - b);
}

// ---- launch helpers ------------------------------------------------------
// Entry points call clear_pending_error() before enqueuing anything, so the
// error launch_status() reads after their launches is their own.
inline void clear_pending_error() { (void)hipGetLastError(); }
inline int launch_status() {
    return hipGetLastError() == hipSuccess ? RKV_OK : RKV_EHIP;
}

// Reports a device-side input the kernels had to clamp or skip (RKV_DEV_*
// flags) in the caller's optional status word.
__device__ __forceinline__ void report(int32_t *status, int32_t flag) {
    if (status) atomicOr(status, flag);
}

// Row count of a sequence from device memory, clamped to [0, cap]; a value
// outside that range is reported.
__device__ __forceinline__ int64_t clamp_rows(int32_t raw, int64_t cap, int32_t *status) {
    if (raw < 0 || (int64_t)raw > cap) {
        report(status, RKV_DEV_LENGTH);
        return raw < 0 ? 0 : cap;
    }
    return raw;
}

// The execution options with every automatic choice still open (0 = auto).
struct Knobs {
    int form = RKV_FORM_AUTO;
    int splitk_blocks = 0;
    int select_chunk = 0;
    int select_radix = 0;
    int attend_variant = 0;
    int attend_pages = 0;
    int32_t *status = nullptr;
    uint64_t *trace = nullptr;
};
inline Knobs knobs_of(const rkv_opts *o) {
    Knobs k;
    if (o) {
        k.form = o->form;
        k.splitk_blocks = o->splitk_blocks;
        k.select_chunk = o->select_chunk;
        k.select_radix = o->select_radix;
        k.attend_variant = o->attend_variant;
        k.attend_pages = o->attend_pages;
        k.status = o->status;
        k.trace = o->trace;
    }
    return k;
}

inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

// ---- internal launchers (one translation unit each) -----------------------
// n_old == nullptr appends exactly one row per sequence, ending at n_new.
int launch_append(const rkv_gqa &g, int dtype, int B, const rkv_paged_cache &c,
                  const int32_t *n_old, const int32_t *n_new, int max_new_rows,
                  const void *k_src, const void *v_src, void *summaries, int32_t *status,
                  hipStream_t s);

struct SelectPlan {
    int chunk_pages;  // pages scored per block
    int n_chunks;     // blocks per (sequence, KV head)
    int sorted;       // 0, or the keys per lane (1, 2, 4) of the rank-ordered list merge
};
SelectPlan plan_select(const rkv_gqa &g, int B, int max_pages, int k2, const Knobs &kn);
size_t select_ws_bytes(const rkv_gqa &g, int B, int max_pages, int k2, const Knobs &kn);
// With k_new/v_new and cache given (a decode step), the block whose chunk
// holds row n-1 also appends it: K/V row into the cache, page summary folded.
int launch_select(const rkv_gqa &g, int dtype, int B, const void *q, const int32_t *seq_lens,
                  int P, int max_pages, void *summaries, int k1, int k2,
                  int32_t *chan_idx, int32_t *page_idx, float *page_scores, void *ws,
                  const void *k_new, const void *v_new, const rkv_paged_cache *cache,
                  const Knobs &kn, hipStream_t s);

struct AttendPlan {
    int pages_per_block;
    int n_splits;
    int waves;    // waves per block
    int variant;  // kernel variant (waves, loads per iteration, pipelining)
};
AttendPlan plan_attend(const rkv_gqa &g, int B, int P, int k2, const Knobs &kn);
size_t attend_ws_bytes(const rkv_gqa &g, int B, int P, int k2, const Knobs &kn);
int launch_attend(const rkv_gqa &g, int dtype, int B, const void *q,
                  const rkv_paged_cache &c, const int32_t *seq_lens, const int32_t *page_idx,
                  int k2, float scale, float *out, void *ws, const Knobs &kn, hipStream_t s);

// Combines split-K attention partials [B][Hkv][n_splits][G][d + 2] in split
// order into out [B][Hq][d].
int launch_attend_merge(const rkv_gqa &g, int B, int n_splits, const float *part, float *out,
                        hipStream_t s);

// How rkv_decode_step runs: form RKV_FORM_STANDALONE (the standalone
// kernels), RKV_FORM_FUSED (the fused kernel with one block per (sequence,
// KV head)) or RKV_FORM_SPLITK (the fused kernel split K-wise over n_splits
// blocks per unit, pages_per_split selected pages each, plus the attention
// merge).
struct FusedPlan {
    int form, n_splits, pages_per_split;
};
FusedPlan plan_fused(const rkv_gqa &g, int dtype, int B, int P, int max_pages, int k1, int k2,
                     const Knobs &kn);
size_t fused_split_ws_bytes(const rkv_gqa &g, int B, int P, int k2, const Knobs &kn);
int launch_decode_fused(const FusedPlan &pl, const rkv_gqa &g, int dtype, int B, const void *q,
                        const void *k_new, const void *v_new, const rkv_paged_cache &c,
                        const int32_t *seq_lens, void *summaries, int k1, int k2, float scale,
                        float *out, int32_t *chan_idx, int32_t *page_idx, float *page_scores,
                        float *part, size_t part_bytes, const Knobs &kn, hipStream_t s);

struct EvictSeq {
    int32_t L[RKV_MAX_EVICT_BATCH];
    int32_t keep[RKV_MAX_EVICT_BATCH];
};
size_t evict_ws_bytes(const rkv_gqa &g, int B, int64_t L_max, int w);
struct ChunkSeq {
    int32_t n_cached[RKV_MAX_EVICT_BATCH];
    int32_t L[RKV_MAX_EVICT_BATCH];  // n_cached + chunk_len
};
size_t evict_chunk_ws_bytes(const rkv_gqa &g, int B, int64_t L_max, int w);
// The rows [0, n_cached) of `src` followed by the chunk's rows are copied
// into the workspace as one sequence, which is evicted into `c` (the kept
// rows and their summaries).  src may be c (chunked prefill) or another cache
// that is only read (the multi-turn view); k_chunk/v_chunk may be null when
// every chunk is empty.
int launch_evict_chunk(const rkv_gqa &g, int dtype, int B, const ChunkSeq &cs, const EvictSeq &seq,
                       int64_t L_max, int64_t C_max, int w, int pool_kernel, float scale,
                       const void *q_win, const void *k_chunk, const void *v_chunk,
                       const rkv_paged_cache &src, const rkv_paged_cache &c, void *summaries,
                       int32_t *kept_idx, int keep_stride, float *pooled, int32_t *seq_lens_out,
                       void *ws, int32_t *status, hipStream_t s);
int launch_evict(const rkv_gqa &g, int dtype, int B, const EvictSeq &seq, int64_t L_max,
                 int w, int pool_kernel, float scale, const void *q_win, const void *k,
                 const void *v, const rkv_paged_cache &c, void *summaries,
                 int32_t *kept_idx, int keep_stride, float *pooled, int32_t *seq_lens_out,
                 void *ws, int32_t *status, hipStream_t s);

}  // namespace rkv
