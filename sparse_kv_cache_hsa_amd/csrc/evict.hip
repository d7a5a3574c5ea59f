// evict.hip -- SnapKV++ stage-1 eviction, once per prefill.
//
// The paper's abstract describes SnapKV++ as SnapKV with adaptive pooling
// size and full grouped-query-attention compatibility; the atlas.scime.ai
// summary ("Approach") adds that it uses a large pooling kernel and selects
// at the GQA-group level.  Per (sequence, KV head):
//   1. logits  : z = fl(sum_c fl(q[c] k[c])) * scale for the R = G*w window
//                query rows against every prompt key (causal per row);
//   2. softmax : row max m (exact), denominator ell accumulated in fp64 and
//                rounded once to fp32, p = expf(z - m) / ell;
//   3. scores  : A[t] = sum_j (sum_i p_{j,i}[t]) for the prefix t < L-w, in
//                the same order and precision as the definition;
//   4. pooling : max over a centred odd window, clipped at the prefix ends;
//   5. keep    : top (keep - w) by (pooled desc, t asc), ascending, plus the
//                w window rows;
//   6. compact : gather K/V rows into the paged cache; rebuild summaries.
// The logits are computed with one thread per query row walking an LDS tile
// of keys in channel order, so they match a sequential fp32 evaluation bit for
// bit (fp32 inputs: separate multiply and add; bf16 inputs: fused
// multiply-add, which is the same because the products are exact); only expf
// may differ from another library's in the last place.
//
// Workspace (per call): logits Z[B][Hkv][L_max][R] fp32 (row-fastest so that
// every pass reads it coalesced), per-tile row maxima, fp64 partial sums,
// scores A, pooled scores and kept positions.
#include "rkv_internal.h"

namespace rkv {
namespace {

constexpr int kTK = 64;      // keys per logits tile
constexpr int kCH = 256;     // keys per denominator chunk
constexpr int kLogitsBlock = 128;

struct EvictWs {
    size_t z, tm, m, ell, pl, a, pooled, kept, nold, nnew, total;
    int R, ntiles, nch;
};

EvictWs evict_layout(const rkv_gqa &g, int B, int64_t L_max, int w) {
    EvictWs l;
    l.R = g.group * w;
    l.ntiles = (int)((L_max + kTK - 1) / kTK);
    l.nch = (int)((L_max + kCH - 1) / kCH);
    const size_t u = (size_t)B * g.n_kv_heads;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off += align_up(bytes);
        return at;
    };
    l.z = take(u * L_max * l.R * sizeof(float));
    l.tm = take(u * l.ntiles * l.R * sizeof(float));
    l.m = take(u * l.R * sizeof(float));
    l.ell = take(u * l.R * sizeof(float));
    l.pl = take(u * l.nch * l.R * sizeof(double));
    l.a = take(u * L_max * sizeof(float));
    l.pooled = take(u * L_max * sizeof(float));
    l.kept = take(u * L_max * sizeof(int32_t));
    l.nold = take((size_t)B * sizeof(int32_t));
    l.nnew = take((size_t)B * sizeof(int32_t));
    l.total = off;
    return l;
}

template <typename T, int D>
__global__ void __launch_bounds__(kLogitsBlock)
logits_kernel(int Hkv, int R, int w, int64_t L_max, EvictSeq seq, const T *q_win, const T *k,
              float scale, int ntiles, float *Z, float *TM) {
    __shared__ float ks[kTK][D];
    const int b = blockIdx.z, h = blockIdx.y, tile = blockIdx.x, tid = threadIdx.x;
    const int64_t L = seq.L[b];
    if (seq.keep[b] >= L) return;
    const int64_t t0 = (int64_t)tile * kTK;
    if (t0 >= L) return;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int nk = (int)min<int64_t>(kTK, L - t0);
    const T *kb = k + (bh * L_max + t0) * D;
    for (int i = tid; i < kTK * D; i += kLogitsBlock) {
        const int tt = i / D;
        ks[tt][i % D] = tt < nk ? Elem<T>::ld(kb, i) : 0.0f;
    }
    __syncthreads();
    for (int r = tid; r < R; r += kLogitsBlock) {
        float qr[D];
        const T *qp = q_win + (bh * R + r) * D;
#pragma unroll
        for (int c = 0; c < D; ++c) qr[c] = Elem<T>::ld(qp, c);
        const int64_t last = L - w + (r % w);
        float tmax = -INFINITY;
        for (int tt = 0; tt < nk; ++tt) {
            float dot = 0.0f;
            if constexpr (sizeof(T) == 2) {
                // bf16 q * bf16 k is exact in fp32, so the fused form rounds
                // once per step exactly like dot + fl(q * k)
#pragma unroll
                for (int c = 0; c < D; ++c) dot = __builtin_fmaf(qr[c], ks[tt][c], dot);
            } else {
#pragma unroll
                for (int c = 0; c < D; ++c) dot = dot + qr[c] * ks[tt][c];
            }
            const float z = dot * scale;
            Z[(bh * L_max + t0 + tt) * R + r] = z;
            if (t0 + tt <= last) tmax = fmaxf(tmax, z);
        }
        TM[(bh * ntiles + tile) * R + r] = tmax;
    }
}

// Register-tiled logits for 16-byte aligned inputs, 8 rows x 8 keys per
// thread: a block covers 128 window rows against 128 keys (two of the 64-key tiles whose maxima TM
// holds).  Every dot product still runs over the channels in ascending
// order, one rounding per step, as in logits_kernel; each channel step reads
// four 16-byte LDS vectors for 64 multiply-adds.
constexpr int kLtRows = 128, kLtKeys = 64, kLtChunk = 32;
constexpr int kL2Keys = 128;

template <typename T, int D>
__global__ void __launch_bounds__(256)
logits_tiled_kernel(int Hkv, int R, int w, int64_t L_max, EvictSeq seq, const T *q_win,
                     const T *k, float scale, int ntiles, int ntiles2, float *Z, float *TM) {
    constexpr int V = Vec16<T>::N;
    constexpr int VPR = kLtChunk / V;
    __shared__ __align__(16) float qs[kLtChunk][kLtRows];
    __shared__ __align__(16) float ks[kLtChunk][kL2Keys];
    __shared__ float tm_s[kL2Keys / 8][kLtRows];
    const int b = blockIdx.z, h = blockIdx.y, tid = threadIdx.x;
    const int tile2 = blockIdx.x % ntiles2, r0 = (blockIdx.x / ntiles2) * kLtRows;
    const int64_t L = seq.L[b];
    if (seq.keep[b] >= L) return;
    const int64_t t0 = (int64_t)tile2 * kL2Keys;
    if (t0 >= L) return;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int nk = (int)min<int64_t>(kL2Keys, L - t0);
    const int rt = tid & 15, kt = tid >> 4;   // rows rt*8.., keys kt*8..
    const T *qb = q_win + (bh * R) * D;
    const T *kb = k + (bh * L_max + t0) * D;
    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
    for (int c0 = 0; c0 < D; c0 += kLtChunk) {
        for (int i = tid; i < kLtRows * VPR; i += 256) {
            const int r = i / VPR, vv = i % VPR;
            float x[V];
            if (r0 + r < R) {
                Vec16<T>::unpack(*(const uint4 *)(qb + (int64_t)(r0 + r) * D + c0 + vv * V), x);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e) x[e] = 0.0f;
            }
#pragma unroll
            for (int e = 0; e < V; ++e) qs[vv * V + e][r] = x[e];
        }
        for (int i = tid; i < kL2Keys * VPR; i += 256) {
            const int t = i / VPR, vv = i % VPR;
            float x[V];
            if (t < nk) {
                Vec16<T>::unpack(*(const uint4 *)(kb + (int64_t)t * D + c0 + vv * V), x);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e) x[e] = 0.0f;
            }
#pragma unroll
            for (int e = 0; e < V; ++e) ks[vv * V + e][t] = x[e];
        }
        __syncthreads();
#pragma unroll 2
        for (int c = 0; c < kLtChunk; ++c) {
            const float4 qa = *(const float4 *)&qs[c][rt * 8];
            const float4 qc = *(const float4 *)&qs[c][rt * 8 + 4];
            const float4 ka = *(const float4 *)&ks[c][kt * 8];
            const float4 kc = *(const float4 *)&ks[c][kt * 8 + 4];
            const float qq[8] = {qa.x, qa.y, qa.z, qa.w, qc.x, qc.y, qc.z, qc.w};
            const float kk[8] = {ka.x, ka.y, ka.z, ka.w, kc.x, kc.y, kc.z, kc.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if constexpr (sizeof(T) == 2)
                        acc[i][j] = __builtin_fmaf(qq[i], kk[j], acc[i][j]);
                    else
                        acc[i][j] = acc[i][j] + qq[i] * kk[j];
                }
        }
        __syncthreads();
    }
    float tmax[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) tmax[i] = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int tt = kt * 8 + j;
        if (tt >= nk) break;
        float z[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            z[i] = acc[i][j] * scale;
            const int r = r0 + rt * 8 + i;
            const int64_t last = L - w + (r % w);
            if (r < R && t0 + tt <= last) tmax[i] = fmaxf(tmax[i], z[i]);
        }
        float *zr = Z + (bh * L_max + t0 + tt) * R + r0 + rt * 8;
        if (r0 + rt * 8 + 7 < R && ((R & 3) == 0)) {
            typedef float f32x4 __attribute__((ext_vector_type(4)));
            __builtin_nontemporal_store(f32x4{z[0], z[1], z[2], z[3]}, (f32x4 *)zr);
            __builtin_nontemporal_store(f32x4{z[4], z[5], z[6], z[7]}, (f32x4 *)(zr + 4));
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (r0 + rt * 8 + i < R) zr[i] = z[i];
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) tm_s[kt][rt * 8 + i] = tmax[i];
    __syncthreads();
    // the maxima of the two 64-key tiles this block covers
    const int half = tid / kLtRows, row = tid % kLtRows;
    const int tile = tile2 * 2 + half;
    if (r0 + row < R && tile < ntiles && t0 + (int64_t)half * kLtKeys < L) {
        float m = tm_s[half * 8][row];
#pragma unroll
        for (int q = 1; q < 8; ++q) m = fmaxf(m, tm_s[half * 8 + q][row]);
        TM[(bh * ntiles + tile) * R + r0 + row] = m;
    }
}

// Row maxima from the logits kernels' per-tile maxima: one block of 1,024
// threads per (sequence, KV head); with R <= 512 several threads share a row,
// each over every parts-th tile with batches of loads in flight, and the
// partial maxima meet in LDS (a maximum is exact in any order).
constexpr int kRowMaxBlock = 1024;

__global__ void __launch_bounds__(kRowMaxBlock)
rowmax_kernel(int Hkv, int R, EvictSeq seq, int ntiles, const float *TM, float *M) {
    __shared__ float part_s[kRowMaxBlock];
    const int b = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
    const int64_t L = seq.L[b];
    if (seq.keep[b] >= L) return;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int nt = (int)((L + kTK - 1) / kTK);
    const float *tm = TM + bh * ntiles * (int64_t)R;
    if (R > kRowMaxBlock / 2) {
        for (int r = tid; r < R; r += kRowMaxBlock) {
            float m = -INFINITY;
            for (int t = 0; t < nt; ++t) m = fmaxf(m, tm[(int64_t)t * R + r]);
            M[bh * R + r] = m;
        }
        return;
    }
    const int parts = kRowMaxBlock / R;
    const int r = tid % R, part = tid / R;
    float m = -INFINITY;
    if (part < parts) {
        constexpr int kBatch = 8;
        for (int t0 = part; t0 < nt; t0 += parts * kBatch) {
            float v[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int t = t0 + u * parts;
                v[u] = t < nt ? tm[(int64_t)t * R + r] : -INFINITY;
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) m = fmaxf(m, v[u]);
        }
    }
    part_s[tid] = m;
    __syncthreads();
    if (tid < R) {
        float mm = part_s[tid];
        for (int p = 1; p < parts; ++p) mm = fmaxf(mm, part_s[p * R + tid]);
        M[bh * R + tid] = mm;
    }
}

__global__ void __launch_bounds__(256)
rowsum_kernel(int Hkv, int R, int w, int64_t L_max, EvictSeq seq, int nch, const float *Z,
              const float *M, double *PL) {
    __shared__ double part_s[256];
    const int b = blockIdx.z, h = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
    const int64_t L = seq.L[b];
    if (seq.keep[b] >= L) return;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t t0 = (int64_t)ch * kCH;
    const int64_t t1 = min<int64_t>(L, t0 + kCH);
    if (R <= 128) {
        // several threads per row, each over a contiguous part of the chunk;
        // the parts are added in part order
        const int parts = 256 / R;
        const int r = tid % R, part = tid / R;
        double acc = 0.0;
        if (part < parts) {
            const int64_t last = L - w + (r % w);
            const int64_t te = min<int64_t>(t1, last + 1);
            const int64_t span = (kCH + parts - 1) / parts;
            const int64_t a0 = t0 + part * span, a1 = min<int64_t>(te, a0 + span);
            const float mr = M[bh * R + r];
            // batches of loads in flight; the sum stays in key order
            constexpr int kBatch = 8;
            for (int64_t tb = a0; tb < a1; tb += kBatch) {
                float z[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u)
                    z[u] = tb + u < a1 ? __builtin_nontemporal_load(&Z[(bh * L_max + tb + u) * R + r]) : 0.0f;
#pragma unroll
                for (int u = 0; u < kBatch; ++u)
                    if (tb + u < a1) acc += (double)expf(z[u] - mr);
            }
        }
        part_s[tid] = acc;
        __syncthreads();
        if (tid < R) {
            double sum = 0.0;
            for (int q = 0; q < parts; ++q) sum += part_s[q * R + tid];
            PL[(bh * nch + ch) * R + tid] = sum;
        }
        return;
    }
    for (int r = tid; r < R; r += 256) {
        const int64_t last = L - w + (r % w);
        const int64_t te = min<int64_t>(t1, last + 1);
        const float mr = M[bh * R + r];
        double acc = 0.0;
        for (int64_t t = t0; t < te; ++t) acc += (double)expf(Z[(bh * L_max + t) * R + r] - mr);
        PL[(bh * nch + ch) * R + r] = acc;
    }
}

__global__ void __launch_bounds__(256)
rowsum_final_kernel(int Hkv, int R, EvictSeq seq, int nch, const double *PL, float *ell) {
    const int b = blockIdx.y, h = blockIdx.x;
    const int64_t L = seq.L[b];
    if (seq.keep[b] >= L) return;
    const int64_t bh = (int64_t)b * Hkv + h;
    for (int r = threadIdx.x; r < R; r += 256) {
        double acc = 0.0;
        for (int c = 0; c < nch; ++c) acc += PL[(bh * nch + c) * R + r];
        ell[bh * R + r] = (float)acc;
    }
}

__global__ void __launch_bounds__(256)
colsum_kernel(int Hkv, int G, int w, int64_t L_max, EvictSeq seq, const float *Z,
              const float *M, const float *ell, float *A) {
    extern __shared__ float sm[];
    const int R = G * w;
    float *Ms = sm, *Es = sm + R;
    const int b = blockIdx.z, h = blockIdx.y;
    const int64_t L = seq.L[b];
    if (seq.keep[b] >= L) return;
    const int64_t bh = (int64_t)b * Hkv + h;
    for (int r = threadIdx.x; r < R; r += 256) {
        Ms[r] = M[bh * R + r];
        Es[r] = ell[bh * R + r];
    }
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= L - w) return;
    const float *zr = Z + (bh * L_max + t) * R;
    float a = 0.0f;
    for (int j = 0; j < G; ++j) {
        float aj = 0.0f;
        for (int i = 0; i < w; ++i) {
            const int r = j * w + i;
            const float p = expf(zr[r] - Ms[r]) / Es[r];
            aj = aj + p;
        }
        a = a + aj;
    }
    A[bh * L_max + t] = a;
}

// Column sums for R <= 128: a block takes 32 prefix keys (at most 17 KB of
// LDS, so eight blocks share a CU and hide each other's load round trips);
// its threads compute p = expf(z - m) / ell for whole Z rows (coalesced over
// r) into LDS, then one thread per key adds them over i, then j, in the
// definition's order.
constexpr int kCsKeys = 32;

__global__ void __launch_bounds__(256)
colsum_tiled_kernel(int Hkv, int G, int w, int64_t L_max, EvictSeq seq, const float *Z,
                    const float *M, const float *ell, float *A) {
    extern __shared__ float sm[];
    const int R = G * w, RS = R + 1;  // padded row stride: conflict-free column reads
    float *Ms = sm, *Es = sm + R, *ps = sm + 2 * R;
    const int b = blockIdx.z, h = blockIdx.y, tid = threadIdx.x;
    const int64_t L = seq.L[b];
    if (seq.keep[b] >= L) return;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t t0 = (int64_t)blockIdx.x * kCsKeys;
    const int64_t npre = L - w;
    if (t0 >= npre) return;
    const int nk = (int)min<int64_t>(kCsKeys, npre - t0);
    for (int r = tid; r < R; r += 256) {
        Ms[r] = M[bh * R + r];
        Es[r] = ell[bh * R + r];
    }
    __syncthreads();
    const int per = 256 / R;  // keys per pass
    if (tid < per * R) {
        // the loads of a batch are issued together, then used
        constexpr int kBatch = 8;
        const int r = tid % R;
        const float mr = Ms[r], er = Es[r];
        // x / er as x * (1/er) plus one residual correction: with 1/er
        // correctly rounded (an IEEE division, once per row), the corrected
        // quotient is the correctly rounded x / er for results in the normal
        // range (Markstein's theorem on division by reciprocal and FMA)
        const float inv = 1.0f / er;
        for (int tb = tid / R; tb < nk; tb += per * kBatch) {
            float z[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int tt = tb + u * per;
                z[u] = tt < nk ? __builtin_nontemporal_load(&Z[(bh * L_max + t0 + tt) * R + r]) : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int tt = tb + u * per;
                if (tt < nk) {
                    const float x = expf(z[u] - mr);
                    const float q0 = x * inv;
                    const float rr = __builtin_fmaf(-q0, er, x);
                    ps[tt * RS + r] = __builtin_fmaf(rr, inv, q0);
                }
            }
        }
    }
    __syncthreads();
    if (tid < nk) {
        const float *pr = ps + tid * RS;
        float a = 0.0f;
        for (int j = 0; j < G; ++j) {
            float aj = 0.0f;
            for (int i = 0; i < w; ++i) aj = aj + pr[j * w + i];
            a = a + aj;
        }
        A[bh * L_max + t0 + tid] = a;
    }
}

__global__ void __launch_bounds__(256)
maxpool_kernel(int Hkv, int w, int64_t L_max, EvictSeq seq, int half, const float *A,
            float *pooled) {
    const int b = blockIdx.z, h = blockIdx.y;
    const int64_t L = seq.L[b];
    if (seq.keep[b] >= L) return;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t npre = L - w;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= npre) return;
    const int64_t u0 = max<int64_t>(0, t - half), u1 = min<int64_t>(npre - 1, t + half);
    const float *a = A + bh * L_max;
    float best = a[u0];
    for (int64_t u = u0 + 1; u <= u1; ++u) best = fmaxf(best, a[u]);
    pooled[bh * L_max + t] = best;
}

constexpr int kKeepBlock = 1024;

__global__ void __launch_bounds__(kKeepBlock)
keep_kernel(int Hkv, int w, int64_t L_max, EvictSeq seq, const float *pooled, int32_t *kept,
            int64_t kept_stride, int32_t *nold, int32_t *nnew, int32_t *seq_lens_out) {
    __shared__ uint32_t hist[256];
    __shared__ int wave_tot[kKeepBlock / kWave];
    __shared__ int sh[2];
    const int b = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
    const int64_t L = seq.L[b];
    const int64_t keep_eff = min<int64_t>(seq.keep[b], L);
    const int64_t bh = (int64_t)b * Hkv + h;
    int32_t *kp = kept + bh * kept_stride;
    if (h == 0 && tid == 0) {
        nold[b] = 0;
        nnew[b] = (int32_t)keep_eff;
        if (seq_lens_out) seq_lens_out[b] = (int32_t)keep_eff;
    }
    if (seq.keep[b] >= L) {
        for (int64_t i = tid; i < kept_stride; i += kKeepBlock) kp[i] = i < L ? (int32_t)i : -1;
        return;
    }
    const int npre = (int)(L - w);
    const int K = (int)(keep_eff - w);
    const float *pl = pooled + bh * L_max;
    if (K > 0) {
        uint32_t thr;
        int take_eq;
        auto load = [&](int i) { return ordered_key(pl[i]); };
        block_topk_threshold<kKeepBlock>(load, npre, K, hist, sh, thr, take_eq);
        block_topk_emit<kKeepBlock>(load, npre, thr, take_eq, wave_tot,
                                    [&](int o, int i) { kp[o] = i; });
    }
    for (int i = tid; i < w; i += kKeepBlock) kp[K + i] = npre + i;
    for (int64_t i = keep_eff + tid; i < kept_stride; i += kKeepBlock) kp[i] = -1;
}

template <typename T, int D>
__global__ void __launch_bounds__(256)
gather_kernel(int Hkv, int64_t L_max, EvictSeq seq, const int32_t *kept, int64_t kept_stride,
              const T *k, const T *v, T *k_pool, T *v_pool, const int32_t *page_table, int P,
              int max_pages, int64_t num_blocks, int32_t *status) {
    constexpr int CPR = D * (int)sizeof(T) / 16;  // 16-byte chunks per row
    constexpr int RPB = 256 / CPR;
    const int b = blockIdx.z, h = blockIdx.y;
    const int64_t L = seq.L[b];
    const int64_t keep_eff = min<int64_t>(seq.keep[b], L);
    const int64_t qrow = (int64_t)blockIdx.x * RPB + threadIdx.x / CPR;
    const int chunk = threadIdx.x % CPR;
    if (qrow >= keep_eff) return;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int32_t t = kept[bh * kept_stride + qrow];
    if (t < 0 || t >= L) return;
    const int32_t blk = page_table[(int64_t)b * max_pages + qrow / P];
    if (blk < 0 || blk >= num_blocks) {
        if (chunk == 0 && qrow % P == 0) report(status, RKV_DEV_BLOCK);
        return;
    }
    const int64_t src = (bh * L_max + t) * D;
    const int64_t dst = (((int64_t)blk * Hkv + h) * P + qrow % P) * D;
    ((uint4 *)(k_pool + dst))[chunk] = ((const uint4 *)(k + src))[chunk];
    ((uint4 *)(v_pool + dst))[chunk] = ((const uint4 *)(v + src))[chunk];
}

// The gather and the summary rebuild in one pass, one block per destination
// page: the page's kept rows are copied into the cache with 16-byte chunks,
// their K rows staged in LDS ([row][D], dynamic), then one thread per
// channel scans them in ascending row order with strict comparisons (the
// first of equal values kept) -- the same scan as the rebuild of
// append_kernel, without reading the rows back from the pool.  A kept index
// outside the prompt leaves that cache row as it was and stages its current
// contents.  Used when a page's rows fit kGatherSummBytes of LDS.
constexpr size_t kGatherSummBytes = 32 * 1024;

template <typename T, int D>
__global__ void __launch_bounds__(256)
gather_summ_kernel(int Hkv, int64_t L_max, EvictSeq seq, const int32_t *kept,
                   int64_t kept_stride, const T *k, const T *v, T *k_pool, T *v_pool,
                   const int32_t *page_table, int P, int max_pages, int64_t num_blocks, T *summ,
                   int32_t *status) {
    extern __shared__ __align__(16) unsigned char gs_raw[];
    T *rows_s = (T *)gs_raw;                       // [P][D]
    constexpr int V = 16 / (int)sizeof(T);         // elements per 16-byte chunk
    constexpr int CPR = D / V;                      // chunks per row
    const int b = blockIdx.z, h = blockIdx.y, tid = threadIdx.x;
    const int64_t L = seq.L[b];
    const int64_t keep_eff = min<int64_t>(seq.keep[b], L);
    const int64_t pg = blockIdx.x;
    const int64_t r0 = pg * P;
    if (r0 >= keep_eff) return;
    const int nrows = (int)min<int64_t>(P, keep_eff - r0);
    const int32_t blk = page_table[(int64_t)b * max_pages + pg];
    if (blk < 0 || blk >= num_blocks) {
        if (tid == 0) report(status, RKV_DEV_BLOCK);
        return;
    }
    const int64_t bh = (int64_t)b * Hkv + h;
    T *kp = k_pool + ((int64_t)blk * Hkv + h) * P * D;
    T *vp = v_pool + ((int64_t)blk * Hkv + h) * P * D;
    for (int i = tid; i < nrows * CPR; i += 256) {
        const int row = i / CPR, chunk = i - row * CPR;
        const int32_t t = kept[bh * kept_stride + r0 + row];
        uint4 kx;
        if (t >= 0 && t < L) {
            const int64_t src = (bh * L_max + t) * D;
            kx = ((const uint4 *)(k + src))[chunk];
            ((uint4 *)(kp + (int64_t)row * D))[chunk] = kx;
            ((uint4 *)(vp + (int64_t)row * D))[chunk] = ((const uint4 *)(v + src))[chunk];
        } else {
            kx = ((const uint4 *)(kp + (int64_t)row * D))[chunk];
        }
        ((uint4 *)(rows_s + (int64_t)row * D))[chunk] = kx;
    }
    __syncthreads();
    for (int c = tid; c < D; c += 256) {
        T bmax = rows_s[c], bmin = rows_s[c];
        float fmax_ = Elem<T>::ld(&bmax, 0), fmin_ = fmax_;
        for (int r = 1; r < nrows; ++r) {
            const T x = rows_s[(int64_t)r * D + c];
            const float fx = Elem<T>::ld(&x, 0);
            if (fx > fmax_) { fmax_ = fx; bmax = x; }
            if (fx < fmin_) { fmin_ = fx; bmin = x; }
        }
        T *sm = summ + bh * 2 * D * max_pages;
        sm[(int64_t)c * max_pages + pg] = bmax;
        sm[(int64_t)(D + c) * max_pages + pg] = bmin;
    }
}

template <typename T, int D>
int launch_t(const rkv_gqa &g, int B, const EvictSeq &seq, int64_t L_max, int w, int pool_kernel,
             float scale, const void *q_win, const void *k, const void *v,
             const rkv_paged_cache &c, void *summaries, int32_t *kept_idx, int keep_stride,
             float *pooled, int32_t *seq_lens_out, void *ws, int32_t *status, hipStream_t s) {
    const EvictWs l = evict_layout(g, B, L_max, w);
    char *base = (char *)ws;
    float *Z = (float *)(base + l.z), *TM = (float *)(base + l.tm);
    float *M = (float *)(base + l.m), *ell = (float *)(base + l.ell);
    double *PL = (double *)(base + l.pl);
    float *A = (float *)(base + l.a);
    float *pl = pooled ? pooled : (float *)(base + l.pooled);
    int32_t *kept = kept_idx ? kept_idx : (int32_t *)(base + l.kept);
    const int64_t kstride = kept_idx ? keep_stride : L_max;
    int32_t *nold = (int32_t *)(base + l.nold), *nnew = (int32_t *)(base + l.nnew);
    const int Hkv = g.n_kv_heads, G = g.group, R = l.R;
    int64_t keep_rows = 0;
    for (int b = 0; b < B; ++b) {
        const int64_t ke = seq.keep[b] < seq.L[b] ? seq.keep[b] : seq.L[b];
        if (ke > keep_rows) keep_rows = ke;
    }
    const int blocks_t = (int)((L_max + 255) / 256);

    if (((uintptr_t)q_win & 15u) == 0 && ((uintptr_t)Z & 15u) == 0) {
        const int rgroups = (R + kLtRows - 1) / kLtRows;
        const int ntiles2 = (int)((L_max + kL2Keys - 1) / kL2Keys);
        logits_tiled_kernel<T, D><<<dim3(ntiles2 * rgroups, Hkv, B), 256, 0, s>>>(
            Hkv, R, w, L_max, seq, (const T *)q_win, (const T *)k, scale, l.ntiles, ntiles2, Z, TM);
    } else {
        logits_kernel<T, D><<<dim3(l.ntiles, Hkv, B), kLogitsBlock, 0, s>>>(
            Hkv, R, w, L_max, seq, (const T *)q_win, (const T *)k, scale, l.ntiles, Z, TM);
    }
    rowmax_kernel<<<dim3(Hkv, B), kRowMaxBlock, 0, s>>>(Hkv, R, seq, l.ntiles, TM, M);
    rowsum_kernel<<<dim3(l.nch, Hkv, B), 256, 0, s>>>(Hkv, R, w, L_max, seq, l.nch, Z, M, PL);
    rowsum_final_kernel<<<dim3(Hkv, B), 256, 0, s>>>(Hkv, R, seq, l.nch, PL, ell);
    if (R <= 128) {
        const int tiles = (int)((L_max + kCsKeys - 1) / kCsKeys);
        const size_t lds = (2 * R + (size_t)kCsKeys * (R + 1)) * sizeof(float);
        colsum_tiled_kernel<<<dim3(tiles, Hkv, B), 256, lds, s>>>(Hkv, G, w, L_max, seq, Z, M,
                                                                 ell, A);
    } else {
        colsum_kernel<<<dim3(blocks_t, Hkv, B), 256, 2 * R * sizeof(float), s>>>(
            Hkv, G, w, L_max, seq, Z, M, ell, A);
    }
    maxpool_kernel<<<dim3(blocks_t, Hkv, B), 256, 0, s>>>(Hkv, w, L_max, seq, pool_kernel / 2, A, pl);
    keep_kernel<<<dim3(Hkv, B), kKeepBlock, 0, s>>>(Hkv, w, L_max, seq, pl, kept, kstride, nold,
                                                    nnew, seq_lens_out);
    const size_t page_bytes = (size_t)c.page_size * D * sizeof(T);
    const bool fused_summ = summaries && page_bytes <= kGatherSummBytes;
    if (keep_rows > 0 && fused_summ) {
        const int pages = (int)((keep_rows + c.page_size - 1) / c.page_size);
        gather_summ_kernel<T, D><<<dim3(pages, Hkv, B), 256, page_bytes, s>>>(
            Hkv, L_max, seq, kept, kstride, (const T *)k, (const T *)v, (T *)c.k_pool,
            (T *)c.v_pool, c.page_table, c.page_size, c.max_pages, c.num_blocks,
            (T *)summaries, status);
        return launch_status();
    }
    if (keep_rows > 0) {
        constexpr int RPB = 256 / (D * (int)sizeof(T) / 16);
        gather_kernel<T, D><<<dim3((int)((keep_rows + RPB - 1) / RPB), Hkv, B), 256, 0, s>>>(
            Hkv, L_max, seq, kept, kstride, (const T *)k, (const T *)v, (T *)c.k_pool,
            (T *)c.v_pool, c.page_table, c.page_size, c.max_pages, c.num_blocks, status);
    }
    int st = launch_status();
    if (st != RKV_OK) return st;
    if (summaries && keep_rows > 0)
        return launch_append(g, sizeof(T) == 4 ? RKV_F32 : RKV_BF16, B, c, nold, nnew,
                             (int)keep_rows, nullptr, nullptr, summaries, status, s);
    return RKV_OK;
}

// Chunked prefill: logical rows [0, n_cached) from the paged cache followed
// by the chunk's rows, copied into one contiguous [B][Hkv][L_max][d] buffer
// that the eviction pipeline then reads like a prompt.
template <typename T, int D>
__global__ void __launch_bounds__(256)
concat_kernel(int Hkv, int64_t L_max, ChunkSeq cs, const T *k_chunk, const T *v_chunk,
              int64_t C_max, const T *k_pool, const T *v_pool, const int32_t *page_table,
              int P, int max_pages, int64_t num_blocks, T *k_cat, T *v_cat, int32_t *status) {
    constexpr int CPR = D * (int)sizeof(T) / 16;  // 16-byte chunks per row
    constexpr int RPB = 256 / CPR;
    const int b = blockIdx.z, h = blockIdx.y;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / CPR;
    const int chunk = threadIdx.x % CPR;
    if (row >= cs.L[b]) return;
    const int64_t bh = (int64_t)b * Hkv + h;
    uint4 kx = make_uint4(0u, 0u, 0u, 0u), vx = kx;
    if (row < cs.n_cached[b]) {
        const int32_t blk = page_table[(int64_t)b * max_pages + row / P];
        if (blk >= 0 && blk < num_blocks) {
            const int64_t src = (((int64_t)blk * Hkv + h) * P + row % P) * D;
            kx = ((const uint4 *)(k_pool + src))[chunk];
            vx = ((const uint4 *)(v_pool + src))[chunk];
        } else if (chunk == 0 && row % P == 0) {
            report(status, RKV_DEV_BLOCK);
        }
    } else {
        const int64_t src = (bh * C_max + (row - cs.n_cached[b])) * D;
        kx = ((const uint4 *)(k_chunk + src))[chunk];
        vx = ((const uint4 *)(v_chunk + src))[chunk];
    }
    const int64_t dst = (bh * L_max + row) * D;
    ((uint4 *)(k_cat + dst))[chunk] = kx;
    ((uint4 *)(v_cat + dst))[chunk] = vx;
}

template <typename T, int D>
void launch_concat(const rkv_gqa &g, int B, const ChunkSeq &cs, int64_t L_max,
                   const void *k_chunk, const void *v_chunk, int64_t C_max,
                   const rkv_paged_cache &c, void *k_cat, void *v_cat, int32_t *status,
                   hipStream_t s) {
    constexpr int RPB = 256 / (D * (int)sizeof(T) / 16);
    concat_kernel<T, D><<<dim3((int)((L_max + RPB - 1) / RPB), g.n_kv_heads, B), 256, 0, s>>>(
        g.n_kv_heads, L_max, cs, (const T *)k_chunk, (const T *)v_chunk, C_max,
        (const T *)c.k_pool, (const T *)c.v_pool, c.page_table, c.page_size, c.max_pages,
        c.num_blocks, (T *)k_cat, (T *)v_cat, status);
}

size_t cat_bytes(const rkv_gqa &g, int B, int64_t L_max) {
    // sized for 4-byte elements, so it serves either element type
    return align_up((size_t)B * g.n_kv_heads * L_max * g.head_dim * 4);
}

}  // namespace

size_t evict_chunk_ws_bytes(const rkv_gqa &g, int B, int64_t L_max, int w) {
    return 2 * cat_bytes(g, B, L_max) + evict_ws_bytes(g, B, L_max, w);
}

int launch_evict_chunk(const rkv_gqa &g, int dtype, int B, const ChunkSeq &cs, const EvictSeq &seq,
                       int64_t L_max, int64_t C_max, int w, int pool_kernel, float scale,
                       const void *q_win, const void *k_chunk, const void *v_chunk,
                       const rkv_paged_cache &src, const rkv_paged_cache &c, void *summaries,
                       int32_t *kept_idx, int keep_stride, float *pooled, int32_t *seq_lens_out,
                       void *ws, int32_t *status, hipStream_t s) {
    char *base = (char *)ws;
    void *k_cat = base, *v_cat = base + cat_bytes(g, B, L_max);
    void *ews = base + 2 * cat_bytes(g, B, L_max);
    const int d = g.head_dim;
    if (dtype == RKV_F32) {
        if (d == 64) launch_concat<float, 64>(g, B, cs, L_max, k_chunk, v_chunk, C_max, src, k_cat, v_cat, status, s);
        else if (d == 128) launch_concat<float, 128>(g, B, cs, L_max, k_chunk, v_chunk, C_max, src, k_cat, v_cat, status, s);
        else return RKV_EUNSUPPORTED;
    } else {
        if (d == 64) launch_concat<uint16_t, 64>(g, B, cs, L_max, k_chunk, v_chunk, C_max, src, k_cat, v_cat, status, s);
        else if (d == 128) launch_concat<uint16_t, 128>(g, B, cs, L_max, k_chunk, v_chunk, C_max, src, k_cat, v_cat, status, s);
        else return RKV_EUNSUPPORTED;
    }
    const int st = launch_status();
    if (st != RKV_OK) return st;
    return launch_evict(g, dtype, B, seq, L_max, w, pool_kernel, scale, q_win, k_cat, v_cat, c,
                        summaries, kept_idx, keep_stride, pooled, seq_lens_out, ews, status, s);
}

size_t evict_ws_bytes(const rkv_gqa &g, int B, int64_t L_max, int w) {
    return evict_layout(g, B, L_max, w).total;
}

int launch_evict(const rkv_gqa &g, int dtype, int B, const EvictSeq &seq, int64_t L_max, int w,
                 int pool_kernel, float scale, const void *q_win, const void *k, const void *v,
                 const rkv_paged_cache &c, void *summaries, int32_t *kept_idx, int keep_stride,
                 float *pooled, int32_t *seq_lens_out, void *ws, int32_t *status, hipStream_t s) {
    const int d = g.head_dim;
    if (dtype == RKV_F32) {
        if (d == 64) return launch_t<float, 64>(g, B, seq, L_max, w, pool_kernel, scale, q_win, k, v, c, summaries, kept_idx, keep_stride, pooled, seq_lens_out, ws, status, s);
        if (d == 128) return launch_t<float, 128>(g, B, seq, L_max, w, pool_kernel, scale, q_win, k, v, c, summaries, kept_idx, keep_stride, pooled, seq_lens_out, ws, status, s);
    } else {
        if (d == 64) return launch_t<uint16_t, 64>(g, B, seq, L_max, w, pool_kernel, scale, q_win, k, v, c, summaries, kept_idx, keep_stride, pooled, seq_lens_out, ws, status, s);
        if (d == 128) return launch_t<uint16_t, 128>(g, B, seq, L_max, w, pool_kernel, scale, q_win, k, v, c, summaries, kept_idx, keep_stride, pooled, seq_lens_out, ws, status, s);
    }
    return RKV_EUNSUPPORTED;
}

}  // namespace rkv
