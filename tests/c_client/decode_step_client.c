/* A plain C client of librkv: fills a paged fp32 cache through
 * rkv_append_summaries, runs one rkv_decode_step (append the new token, then
 * HSA) on the GPU, and checks every (sequence, KV head) against the CPU
 * oracle's rkvo_hsa_group: channel and page sets bit for bit, outputs within
 * 1e-3.  Test infrastructure only (it links the oracle); the point is that
 * the boundary is usable from C with nothing but rkv.h, the HIP runtime's C
 * API and plain pointers.  Exit status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "rkv.h"

/* the oracle's entry points (oracle/rkv_oracle.c) */
void rkvo_summaries_rebuild(const void *k, int dt, int64_t n, int d, int P, void *smax,
                            void *smin);
int rkvo_hsa_group(const void *q, const void *k, const void *v, int dt, const void *smax,
                   const void *smin, int64_t n, int d, int G, int P, int k1, int k2,
                   double scale, int32_t *chan, int32_t *pages, float *S_out, double *out);

#define B 2
#define HKV 2
#define G 4
#define D 128
#define P 16
#define K1 32
#define K2 8
#define MAX_PAGES 48

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

/* splitmix64, then Box-Muller: N(0, 1) floats */
static uint64_t next_u64(void) {
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static float normal(void) {
    double u1 = ((next_u64() >> 11) + 0.5) / 9007199254740992.0;
    double u2 = ((next_u64() >> 11) + 0.5) / 9007199254740992.0;
    return (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}

#define HIP_OK(x)                                                                  \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__);      \
            return 2;                                                              \
        }                                                                          \
    } while (0)

#define RKV_OK_(x)                                                                 \
    do {                                                                           \
        int s_ = (x);                                                              \
        if (s_ != RKV_OK) {                                                        \
            fprintf(stderr, "rkv error %s at line %d\n", rkv_status_string(s_),   \
                    __LINE__);                                                     \
            return 3;                                                              \
        }                                                                          \
    } while (0)

int main(void) {
    const int n[B] = {700, 333};  /* rows after the step's token */
    const int max_rows = MAX_PAGES * P;
    const int64_t num_blocks = (int64_t)B * MAX_PAGES;
    const float scale = 1.0f / sqrtf((float)D);
    rkv_gqa g = {HKV, G, D};

    /* logical rows per (sequence, head) on the host: K, V [B][HKV][max_rows][D] */
    size_t rows_elems = (size_t)B * HKV * max_rows * D;
    float *K = calloc(rows_elems, sizeof(float)), *V = calloc(rows_elems, sizeof(float));
    float *q = malloc((size_t)B * HKV * G * D * sizeof(float));
    if (!K || !V || !q) return 4;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < HKV; ++h)
            for (int t = 0; t < n[b]; ++t)
                for (int c = 0; c < D; ++c) {
                    size_t i = (((size_t)b * HKV + h) * max_rows + t) * D + c;
                    K[i] = normal();
                    V[i] = normal();
                }
    for (size_t i = 0; i < (size_t)B * HKV * G * D; ++i) q[i] = normal();

    /* page table: logical page p of sequence b in block b*MAX_PAGES + (MAX_PAGES-1-p) */
    int32_t table[B * MAX_PAGES];
    for (int b = 0; b < B; ++b)
        for (int p = 0; p < MAX_PAGES; ++p) table[b * MAX_PAGES + p] = b * MAX_PAGES + (MAX_PAGES - 1 - p);

    /* device buffers */
    size_t pool_bytes = (size_t)num_blocks * HKV * P * D * sizeof(float);
    size_t summ_bytes = (size_t)B * HKV * 2 * D * MAX_PAGES * sizeof(float);
    void *k_pool, *v_pool, *summ, *d_table, *d_src_k, *d_src_v, *d_q, *d_knew, *d_vnew;
    void *d_nold, *d_nnew, *d_seq, *d_out, *d_chan, *d_pages, *d_ws;
    HIP_OK(hipMalloc(&k_pool, pool_bytes));
    HIP_OK(hipMalloc(&v_pool, pool_bytes));
    HIP_OK(hipMemset(k_pool, 0, pool_bytes));
    HIP_OK(hipMemset(v_pool, 0, pool_bytes));
    HIP_OK(hipMalloc(&summ, summ_bytes));
    HIP_OK(hipMalloc(&d_table, sizeof(table)));
    HIP_OK(hipMemcpy(d_table, table, sizeof(table), hipMemcpyHostToDevice));
    rkv_paged_cache cache = {k_pool, v_pool, (const int32_t *)d_table, num_blocks, P, MAX_PAGES};

    /* 1. the first n-1 rows through rkv_append_summaries, from [B][HKV][max_new][D] */
    int max_new = 0;
    for (int b = 0; b < B; ++b) max_new = n[b] - 1 > max_new ? n[b] - 1 : max_new;
    size_t src_elems = (size_t)B * HKV * max_new * D;
    float *src_k = calloc(src_elems, sizeof(float)), *src_v = calloc(src_elems, sizeof(float));
    if (!src_k || !src_v) return 4;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < HKV; ++h)
            for (int t = 0; t < n[b] - 1; ++t) {
                size_t dst = (((size_t)b * HKV + h) * max_new + t) * D;
                size_t src = (((size_t)b * HKV + h) * max_rows + t) * D;
                memcpy(src_k + dst, K + src, D * sizeof(float));
                memcpy(src_v + dst, V + src, D * sizeof(float));
            }
    HIP_OK(hipMalloc(&d_src_k, src_elems * sizeof(float)));
    HIP_OK(hipMalloc(&d_src_v, src_elems * sizeof(float)));
    HIP_OK(hipMemcpy(d_src_k, src_k, src_elems * sizeof(float), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_src_v, src_v, src_elems * sizeof(float), hipMemcpyHostToDevice));
    int32_t n_old[B], n_new[B], seq[B];
    for (int b = 0; b < B; ++b) {
        n_old[b] = 0;
        n_new[b] = n[b] - 1;
        seq[b] = n[b];
    }
    HIP_OK(hipMalloc(&d_nold, sizeof(n_old)));
    HIP_OK(hipMalloc(&d_nnew, sizeof(n_new)));
    HIP_OK(hipMalloc(&d_seq, sizeof(seq)));
    HIP_OK(hipMemcpy(d_nold, n_old, sizeof(n_old), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_nnew, n_new, sizeof(n_new), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_seq, seq, sizeof(seq), hipMemcpyHostToDevice));
    RKV_OK_(rkv_append_summaries(&g, RKV_F32, B, &cache, (const int32_t *)d_nold,
                                 (const int32_t *)d_nnew, max_new, d_src_k, d_src_v, summ, NULL,
                                 NULL));

    /* 2. one decode step: the token at row n-1, then HSA */
    float knew[B * HKV * D], vnew[B * HKV * D];
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < HKV; ++h) {
            size_t src = (((size_t)b * HKV + h) * max_rows + (n[b] - 1)) * D;
            memcpy(knew + ((size_t)b * HKV + h) * D, K + src, D * sizeof(float));
            memcpy(vnew + ((size_t)b * HKV + h) * D, V + src, D * sizeof(float));
        }
    HIP_OK(hipMalloc(&d_knew, sizeof(knew)));
    HIP_OK(hipMalloc(&d_vnew, sizeof(vnew)));
    HIP_OK(hipMalloc(&d_q, (size_t)B * HKV * G * D * sizeof(float)));
    HIP_OK(hipMemcpy(d_knew, knew, sizeof(knew), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_vnew, vnew, sizeof(vnew), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_q, q, (size_t)B * HKV * G * D * sizeof(float), hipMemcpyHostToDevice));
    size_t out_elems = (size_t)B * HKV * G * D;
    HIP_OK(hipMalloc(&d_out, out_elems * sizeof(float)));
    HIP_OK(hipMalloc(&d_chan, (size_t)B * HKV * K1 * sizeof(int32_t)));
    HIP_OK(hipMalloc(&d_pages, (size_t)B * HKV * K2 * sizeof(int32_t)));
    size_t ws_bytes = rkv_hsa_workspace_bytes(&g, B, P, MAX_PAGES, K1, K2, NULL);
    if (ws_bytes == 0) return 5;
    HIP_OK(hipMalloc(&d_ws, ws_bytes));
    RKV_OK_(rkv_decode_step(&g, RKV_F32, B, d_q, d_knew, d_vnew, &cache, (const int32_t *)d_seq,
                            summ, K1, K2, scale, (float *)d_out, (int32_t *)d_chan,
                            (int32_t *)d_pages, NULL, d_ws, ws_bytes, NULL, NULL));
    HIP_OK(hipDeviceSynchronize());

    float *out = malloc(out_elems * sizeof(float));
    int32_t chan[B * HKV * K1], pages[B * HKV * K2];
    if (!out) return 4;
    HIP_OK(hipMemcpy(out, d_out, out_elems * sizeof(float), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(chan, d_chan, sizeof(chan), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(pages, d_pages, sizeof(pages), hipMemcpyDeviceToHost));

    /* 3. the oracle, unit by unit */
    int bad = 0;
    double worst = 0.0;
    float *smax = malloc((size_t)MAX_PAGES * D * sizeof(float));
    float *smin = malloc((size_t)MAX_PAGES * D * sizeof(float));
    double *ref = malloc((size_t)G * D * sizeof(double));
    if (!smax || !smin || !ref) return 4;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < HKV; ++h) {
            const float *kb = K + ((size_t)b * HKV + h) * max_rows * D;
            const float *vb = V + ((size_t)b * HKV + h) * max_rows * D;
            int32_t c_o[K1], p_o[K2];
            rkvo_summaries_rebuild(kb, 0, n[b], D, P, smax, smin);
            if (rkvo_hsa_group(q + ((size_t)b * HKV + h) * G * D, kb, vb, 0, smax, smin, n[b], D,
                               G, P, K1, K2, scale, c_o, p_o, NULL, ref) != 0)
                return 6;
            if (memcmp(c_o, chan + ((size_t)b * HKV + h) * K1, sizeof(c_o)) != 0) {
                fprintf(stderr, "unit (%d, %d): channels differ\n", b, h);
                bad = 1;
            }
            if (memcmp(p_o, pages + ((size_t)b * HKV + h) * K2, sizeof(p_o)) != 0) {
                fprintf(stderr, "unit (%d, %d): pages differ\n", b, h);
                bad = 1;
            }
            for (int i = 0; i < G * D; ++i) {
                double e = fabs((double)out[((size_t)b * HKV + h) * G * D + i] - ref[i]);
                if (e > worst) worst = e;
            }
        }
    if (worst > 1e-3) {
        fprintf(stderr, "max abs error %g above 1e-3\n", worst);
        bad = 1;
    }
    printf("c client: %s (build %s, max abs error %.3g)\n", bad ? "MISMATCH" : "ok",
           rkv_build_id(), worst);
    hipFree(k_pool); hipFree(v_pool); hipFree(summ); hipFree(d_table); hipFree(d_src_k);
    hipFree(d_src_v); hipFree(d_q); hipFree(d_knew); hipFree(d_vnew); hipFree(d_nold);
    hipFree(d_nnew); hipFree(d_seq); hipFree(d_out); hipFree(d_chan); hipFree(d_pages);
    hipFree(d_ws);
    free(K); free(V); free(q); free(src_k); free(src_v); free(out); free(smax); free(smin);
    free(ref);
    return bad;
}
