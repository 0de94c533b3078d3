/*
 * ep_example.c -- the C ABI of include/ep.h driven from plain C11 (no C++, no
 * Python, no torch): one dispatch + combine step on the default stream with
 * device memory from hipMalloc.
 *
 * Two sources of 257 tokens, hidden 512 bf16, top-6 of 48 experts on 8 ranks,
 * some lanes masked.  The expert is the identity (its output rows are the
 * received rows), so the combine must return x[s][t] * (sum of the token's
 * valid weights).  x holds multiples of 1/8 in [-1, 1] and every weight is
 * 1/8, so that product is exact in bf16 and is checked for equality.  The
 * program also checks the receive-row count (one row per distinct
 * (token, destination rank)) and that the receive rows of each destination
 * come in ascending source-token order.  Prints "ep_example: ok ..." and
 * returns 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ep.h"

#define CHECK_HIP(x)                                                                  \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "ep_example: %s failed: %s\n", #x, hipGetErrorString(e_)); \
            return 1;                                                                 \
        }                                                                             \
    } while (0)
#define CHECK_EP(x)                                                                   \
    do {                                                                              \
        int r_ = (x);                                                                 \
        if (r_ != EP_OK) {                                                            \
            fprintf(stderr, "ep_example: %s returned %s\n", #x, ep_status_string(r_)); \
            return 1;                                                                 \
        }                                                                             \
    } while (0)

enum { S = 2, T = 257, H = 512, K = 6, E = 48, R = 8, NMAX = 260 };

static uint32_t next_rand(uint32_t *state) {
    *state = *state * 1664525u + 1013904223u;
    return *state >> 8;
}

static uint16_t bf16_bits(float f) { /* exact for the values used here */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static float bf16_value(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static void *dev_alloc(uint64_t bytes) {
    void *p = NULL;
    if (bytes && hipMalloc(&p, bytes) != hipSuccess) {
        fprintf(stderr, "ep_example: hipMalloc(%llu) failed\n", (unsigned long long)bytes);
        exit(1);
    }
    return p;
}

int main(void) {
    static int64_t topk[S][T][K];
    static float w[S][T][K];
    static uint16_t x[S][T][H];
    uint32_t rng = 12345u;
    int64_t expected_rows = 0;
    for (int s = 0; s < S; ++s)
        for (int t = 0; t < T; ++t) {
            int used_rank[R] = {0};
            for (int k = 0; k < K; ++k) {
                int64_t e;
                int dup;
                do { /* distinct experts per token */
                    e = (int64_t)(next_rand(&rng) % E);
                    dup = 0;
                    for (int q = 0; q < k; ++q) dup |= topk[s][t][q] == e;
                } while (dup);
                topk[s][t][k] = (next_rand(&rng) % 7 == 0) ? -1 : e; /* about 1 lane in 7 masked */
                w[s][t][k] = 0.125f;
                if (topk[s][t][k] >= 0 && !used_rank[e / (E / R)]) {
                    used_rank[e / (E / R)] = 1;
                    ++expected_rows;
                }
            }
            for (int h = 0; h < H; ++h) x[s][t][h] = bf16_bits((float)((int)(next_rand(&rng) % 17) - 8) / 8.0f);
        }

    ep_config_t cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.num_src_ranks = S;
    cfg.num_tokens = T;
    cfg.hidden = H;
    cfg.num_topk = K;
    cfg.num_experts = E;
    cfg.num_ranks = R;
    cfg.num_max_tokens_per_rank = NMAX;
    cfg.x_dtype = EP_DTYPE_BF16;
    cfg.expert_alignment = 1;
    ep_sizes_t sz;
    CHECK_EP(ep_query_sizes(&cfg, &sz));

    ep_layout_t L;
    L.dst_slot_dev = dev_alloc(sz.dst_slot);
    L.tokens_per_rank_dev = dev_alloc(sz.tokens_per_rank);
    L.tokens_per_expert_dev = dev_alloc(sz.tokens_per_expert);
    L.recv_psum_dev = dev_alloc(sz.recv_psum);
    L.recv_base_dev = dev_alloc(sz.recv_base);
    L.expert_base_dev = dev_alloc(sz.expert_base);
    L.expand_pos_dev = dev_alloc(sz.expand_pos);
    L.error_flags_dev = dev_alloc(sz.error_flags);
    L.scratch_dev = dev_alloc(sz.layout_scratch);
    L.recv_psum_scaleup_dev = dev_alloc(sz.recv_psum_scaleup);
    ep_recv_t rv;
    rv.staging_x_dev = dev_alloc(sz.staging_x);
    rv.staging_sf_dev = dev_alloc(sz.staging_sf);
    rv.staging_meta_dev = dev_alloc(sz.staging_meta);
    rv.recv_x_dev = dev_alloc(sz.recv_x);
    rv.recv_sf_dev = dev_alloc(sz.recv_sf);
    rv.recv_src_idx_dev = dev_alloc(sz.recv_src_idx);
    rv.recv_topk_idx_dev = dev_alloc(sz.recv_topk_idx);
    rv.recv_topk_weights_dev = dev_alloc(sz.recv_topk_weights);
    rv.recv_capacity_rows = (int64_t)sz.recv_rows;
    void *d_topk = dev_alloc(sizeof topk), *d_w = dev_alloc(sizeof w), *d_x = dev_alloc(sizeof x);
    void *d_out = dev_alloc(sz.out);
    CHECK_HIP(hipMemcpy(d_topk, topk, sizeof topk, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_w, w, sizeof w, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_x, x, sizeof x, hipMemcpyHostToDevice));

    CHECK_EP(ep_layout(&cfg, (const int64_t *)d_topk, &L, NULL));
    CHECK_EP(ep_dispatch(&cfg, d_x, NULL, (const int64_t *)d_topk, (const float *)d_w, &L, &rv, EP_PHASE_ALL, NULL));
    /* identity expert: the expert-output rows are the received rows */
    CHECK_EP(ep_combine(&cfg, &L, (const int64_t *)d_topk, (const float *)d_w, rv.recv_x_dev, d_out, NULL));
    CHECK_HIP(hipDeviceSynchronize());

    int32_t recv_base[R + 1], flags = 0;
    CHECK_HIP(hipMemcpy(recv_base, L.recv_base_dev, sizeof recv_base, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&flags, L.error_flags_dev, sizeof flags, hipMemcpyDeviceToHost));
    const int n = recv_base[R];
    int32_t *src = malloc((size_t)(n > 0 ? n : 1) * sizeof *src);
    uint16_t *out = malloc(sz.out);
    if (!src || !out) return 1;
    CHECK_HIP(hipMemcpy(src, rv.recv_src_idx_dev, (size_t)n * sizeof *src, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(out, d_out, sz.out, hipMemcpyDeviceToHost));

    int bad = 0;
    if (flags != 0) fprintf(stderr, "ep_example: error flag set\n"), ++bad;
    if (n != expected_rows) fprintf(stderr, "ep_example: %d receive rows, expected %lld\n", n, (long long)expected_rows), ++bad;
    for (int d = 0; d < R; ++d)
        for (int i = recv_base[d] + 1; i < recv_base[d + 1]; ++i)
            if (src[i] <= src[i - 1]) {
                fprintf(stderr, "ep_example: destination %d rows out of order at %d\n", d, i);
                ++bad;
                break;
            }
    for (int s = 0; s < S && !bad; ++s)
        for (int t = 0; t < T && !bad; ++t) {
            float wsum = 0.0f;
            for (int k = 0; k < K; ++k) wsum += topk[s][t][k] >= 0 ? w[s][t][k] : 0.0f;
            for (int h = 0; h < H; ++h) {
                const float want = bf16_value(x[s][t][h]) * wsum;
                const float got = bf16_value(out[((size_t)s * T + t) * H + h]);
                if (got != want) {
                    fprintf(stderr, "ep_example: out[%d][%d][%d] = %g, expected %g\n", s, t, h, got, want);
                    ++bad;
                    break;
                }
            }
        }
    free(src);
    free(out);
    if (bad) return 1;
    printf("ep_example: ok (%d receive rows, libep %d)\n", n, ep_version());
    return 0;
}
