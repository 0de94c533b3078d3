/*
 * ep_oracle.c -- plain, slow, single-threaded CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY (see ep_oracle.h).  It is the definition of every
 * output written out as loops, in the order the definitions are stated; it is
 * never tuned and shares nothing with the HIP library.
 *
 * Readings of points the pages leave open (each also listed in the design
 * notes of the repository):
 *   - expert e lives on rank e / El (contiguous blocks of El experts);
 *   - a lane with a negative id is masked; an id >= E is invalid, raises bit 0
 *     of the error flags and is then treated as masked;
 *   - deduplication keeps the lowest valid lane per destination rank: that lane
 *     is the "owner" and carries the slot, the other lanes of the same rank
 *     get -1;
 *   - the running count is exclusive, over tokens in ascending order;
 *   - the row base of source partition s is s on the direct path (one
 *     receive row per source rank) and its scale-out index on the hybrid path,
 *     whose receive buffer is segmented by the scale-up index (row form);
 *   - the compact receive order is destination-major, then source, then slot,
 *     which is the order a sort by global source token index (s*T + t) gives
 *     inside each destination;
 *   - the expand layout places, inside each expert's segment, the lanes in
 *     ascending (s, t, k) order, segments padded to a multiple of A.
 */
#include "ep_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* Expert id of a lane if it routes to a real expert, else -1. */
static int64_t lane_expert(int64_t e, int E) { return (e >= 0 && e < E) ? e : -1; }

/* A lane owns its destination rank when it is valid and no lower valid lane
 * of the same token goes to the same rank.  The deterministic-dispatch page
 * ([DET] Motivation) has senders deduplicate a token's top-k lanes by
 * destination rank so that one lane per destination sends. */
static int lane_is_owner(const int64_t *tok, int k, int E, int El) {
    int64_t e = lane_expert(tok[k], E);
    if (e < 0) return 0;
    for (int k2 = 0; k2 < k; ++k2) {
        int64_t e2 = lane_expert(tok[k2], E);
        if (e2 >= 0 && e2 / El == e / El) return 0;
    }
    return 1;
}

/* Index of the owner lane of rank d in a token, or -1. */
static int owner_lane(const int64_t *tok, int K, int E, int El, int d) {
    for (int k = 0; k < K; ++k) {
        int64_t e = lane_expert(tok[k], E);
        if (e >= 0 && e / El == d) return k;
    }
    return -1;
}

static int sizes_ok(int S, int T, int K, int E, int R, int Nmax) {
    if (S < 1 || T < 0 || K < 1 || E < 1 || R < 1 || E % R != 0) return 0;
    if (Nmax < T) return 0; /* a source sends at most T rows to one destination */
    return 1;
}

/* Topology of the S source ranks: n_out <= 1 is the direct path; n_out > 1
 * is the hybrid path with S = n_out * n_up ranks, rank s having scale-out
 * index s / n_up and scale-up index s % n_up. */
static int topology_ok(int S, int n_out) { return n_out <= 1 || (S % n_out == 0); }

/* Row base of source s ([DET] Direct vs hybrid dispatch): the source rank on
 * the direct path, its scale-out index on the hybrid path. */
static int64_t row_base(int s, int S, int n_out) { return n_out > 1 ? s / (S / n_out) : s; }

/* Region (of Nmax rows) that source s fills in destination d's staging
 * buffer: one region per source on the direct path (d*S + s); in the hybrid
 * row form the buffer has one segment per scale-up index, and inside it one
 * region per scale-out index ([DET] Direct vs hybrid dispatch). */
static size_t staging_region(int d, int s, int S, int n_out) {
    if (n_out > 1) {
        const int n_up = S / n_out;
        return ((size_t)d * n_up + (size_t)(s % n_up)) * (size_t)n_out + (size_t)(s / n_up);
    }
    return (size_t)d * S + (size_t)s;
}

int epo_layout(int S, int T, int K, int E, int R, int Nmax, int expand, int A, int n_out,
               const int64_t *topk_idx, int32_t *dst_slot, int32_t *tokens_per_rank,
               int32_t *tokens_per_expert, int32_t *recv_psum, int32_t *recv_base,
               int32_t *expert_base, int32_t *expand_pos, int32_t *recv_psum_scaleup,
               int32_t *error_flags) {
    if (!sizes_ok(S, T, K, E, R, Nmax) || (expand && A < 1) || !topology_ok(S, n_out)) return -1;
    const int El = E / R;
    int32_t flags = 0;
    memset(tokens_per_rank, 0, sizeof(int32_t) * (size_t)S * R);
    memset(tokens_per_expert, 0, sizeof(int32_t) * (size_t)S * E);

    /* Counts and slots ([DET] Approach): the slot of an owner lane is
     * row_base * Nmax + the number of earlier tokens of the same source that
     * also go to that destination. */
    int32_t *run = (int32_t *)calloc((size_t)R, sizeof(int32_t));
    for (int s = 0; s < S; ++s) {
        for (int d = 0; d < R; ++d) run[d] = 0;
        for (int t = 0; t < T; ++t) {
            const int64_t *tok = topk_idx + ((size_t)s * T + t) * K;
            int32_t *slot = dst_slot + ((size_t)s * T + t) * K;
            for (int k = 0; k < K; ++k) {
                if (tok[k] >= E) flags |= 1;
                int64_t e = lane_expert(tok[k], E);
                if (e >= 0) tokens_per_expert[(size_t)s * E + e] += 1;
                if (lane_is_owner(tok, k, E, El))
                    slot[k] = (int32_t)(row_base(s, S, n_out) * Nmax + run[e / El]);
                else
                    slot[k] = -1;
            }
            /* This token now counts once for each destination it reaches. */
            for (int k = 0; k < K; ++k) {
                if (lane_is_owner(tok, k, E, El)) {
                    int d = (int)(lane_expert(tok[k], E) / El);
                    run[d] += 1;
                    tokens_per_rank[(size_t)s * R + d] += 1;
                }
            }
        }
    }
    free(run);

    /* Receiver tables: per destination, the exclusive prefix over sources of
     * what each source sends there ([DRX] Direct Recv X design: each source
     * gets an exclusive base in the compact receive layout), and the
     * exclusive prefix over destinations of the totals. */
    for (int d = 0; d < R; ++d) {
        int32_t *ps = recv_psum + (size_t)d * (S + 1);
        ps[0] = 0;
        for (int s = 0; s < S; ++s) ps[s + 1] = ps[s] + tokens_per_rank[(size_t)s * R + d];
    }
    recv_base[0] = 0;
    for (int d = 0; d < R; ++d) recv_base[d + 1] = recv_base[d] + recv_psum[(size_t)d * (S + 1) + S];

    /* Hybrid row form: per destination, also the exclusive prefix over
     * scale-up segments of the rows each segment holds (the per-segment part
     * of the extended psum, [DET] Direct vs hybrid dispatch). */
    if (n_out > 1) {
        const int n_up = S / n_out;
        for (int d = 0; d < R; ++d) {
            int32_t *ps = recv_psum_scaleup + (size_t)d * (n_up + 1);
            ps[0] = 0;
            for (int u = 0; u < n_up; ++u) {
                int32_t seg = 0;
                for (int s = 0; s < S; ++s)
                    if (s % n_up == u) seg += tokens_per_rank[(size_t)s * R + d];
                ps[u + 1] = ps[u] + seg;
            }
        }
    }

    if (expand) {
        /* Expand layout: one receive row per valid lane, grouped by expert,
         * each expert's segment rounded up to a multiple of A; inside a
         * segment lanes keep ascending (s, t, k) order, the order a sort by
         * global source token index gives ([DET] Motivation, Compatibility). */
        expert_base[0] = 0;
        for (int e = 0; e < E; ++e) {
            int64_t cnt = 0;
            for (int s = 0; s < S; ++s) cnt += tokens_per_expert[(size_t)s * E + e];
            int64_t padded = (cnt + A - 1) / A * A;
            expert_base[e + 1] = (int32_t)(expert_base[e] + padded);
        }
        int32_t *next = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
        for (int e = 0; e < E; ++e) next[e] = expert_base[e];
        for (int s = 0; s < S; ++s)
            for (int t = 0; t < T; ++t)
                for (int k = 0; k < K; ++k) {
                    size_t i = ((size_t)s * T + t) * K + k;
                    int64_t e = lane_expert(topk_idx[i], E);
                    expand_pos[i] = e >= 0 ? next[e]++ : -1;
                }
        free(next);
    }
    *error_flags = flags;
    return 0;
}

int epo_dispatch(int S, int T, int H, int K, int E, int R, int Nmax, int is_fp8,
                 int expand, int A, int n_out, const uint8_t *x, const float *x_sf,
                 const int64_t *topk_idx, const float *topk_weights,
                 const int32_t *dst_slot, const int32_t *tokens_per_rank,
                 const int32_t *tokens_per_expert, const int32_t *recv_psum,
                 const int32_t *recv_base, const int32_t *expert_base,
                 const int32_t *expand_pos, uint8_t *staging_x, float *staging_sf,
                 int32_t *staging_meta, uint8_t *recv_x, float *recv_sf,
                 int32_t *recv_src_idx, int32_t *recv_topk_idx, float *recv_topk_weights) {
    if (!sizes_ok(S, T, K, E, R, Nmax) || H < 1 || !topology_ok(S, n_out)) return -1;
    if (is_fp8 && H % 128 != 0) return -1;
    const int El = E / R;
    const size_t Rw = is_fp8 ? (size_t)H : (size_t)H * 2; /* row bytes */
    const size_t F = is_fp8 ? (size_t)H / 128 : 0;        /* scales per row */
    const size_t M = 1 + 2 * (size_t)K;                     /* metadata words */

    /* Scatter: each owner lane copies the token's row, scales and metadata to
     * row j = slot - row_base*Nmax of source s's region in destination d's
     * receive buffer, R buffers of S regions of Nmax rows ([DET] Direct vs
     * hybrid dispatch). */
    for (int s = 0; s < S; ++s)
        for (int t = 0; t < T; ++t) {
            const int64_t *tok = topk_idx + ((size_t)s * T + t) * K;
            const float *w = topk_weights + ((size_t)s * T + t) * K;
            for (int k = 0; k < K; ++k) {
                if (!lane_is_owner(tok, k, E, El)) continue;
                int d = (int)(tok[k] / El);
                int64_t j = (int64_t)dst_slot[((size_t)s * T + t) * K + k] - row_base(s, S, n_out) * Nmax;
                size_t row = staging_region(d, s, S, n_out) * Nmax + (size_t)j;
                memcpy(staging_x + row * Rw, x + ((size_t)s * T + t) * Rw, Rw);
                if (F) memcpy(staging_sf + row * F, x_sf + ((size_t)s * T + t) * F, F * sizeof(float));
                int32_t *meta = staging_meta + row * M;
                meta[0] = t;
                for (int k2 = 0; k2 < K; ++k2) {
                    int64_t e2 = lane_expert(tok[k2], E);
                    meta[1 + k2] = e2 >= 0 ? (int32_t)e2 : -1;
                    memcpy(&meta[1 + K + k2], &w[k2], sizeof(float));
                }
            }
        }

    if (!expand) {
        /* Copy epilogue ([DRX] Background): receive row
         * i = recv_base[d] + recv_psum[d][s] + j takes staging row (d, s, j)
         * for j below that source's count; top-k ids become local expert ids
         * of d (others -1, weight +0). */
        for (int d = 0; d < R; ++d)
            for (int s = 0; s < S; ++s)
                for (int j = 0; j < tokens_per_rank[(size_t)s * R + d]; ++j) {
                    size_t i = (size_t)recv_base[d] + (size_t)recv_psum[(size_t)d * (S + 1) + s] + (size_t)j;
                    size_t row = staging_region(d, s, S, n_out) * Nmax + (size_t)j;
                    memcpy(recv_x + i * Rw, staging_x + row * Rw, Rw);
                    if (F) memcpy(recv_sf + i * F, staging_sf + row * F, F * sizeof(float));
                    const int32_t *meta = staging_meta + row * M;
                    recv_src_idx[i] = (int32_t)((int64_t)s * T + meta[0]);
                    for (int k = 0; k < K; ++k) {
                        int32_t e = meta[1 + k];
                        if (e >= 0 && e / El == d) {
                            recv_topk_idx[i * K + k] = e - d * El;
                            memcpy(&recv_topk_weights[i * K + k], &meta[1 + K + k], sizeof(float));
                        } else {
                            recv_topk_idx[i * K + k] = -1;
                            recv_topk_weights[i * K + k] = 0.0f;
                        }
                    }
                }
    } else {
        /* Expand epilogue: every valid lane gets its own row at expand_pos,
         * filled from its token's staging row for that lane's rank. */
        for (int s = 0; s < S; ++s)
            for (int t = 0; t < T; ++t) {
                const int64_t *tok = topk_idx + ((size_t)s * T + t) * K;
                for (int k = 0; k < K; ++k) {
                    int64_t e = lane_expert(tok[k], E);
                    if (e < 0) continue;
                    int d = (int)(e / El);
                    int k0 = owner_lane(tok, K, E, El, d);
                    int64_t j = (int64_t)dst_slot[((size_t)s * T + t) * K + k0] - row_base(s, S, n_out) * Nmax;
                    size_t row = staging_region(d, s, S, n_out) * Nmax + (size_t)j;
                    size_t r = (size_t)expand_pos[((size_t)s * T + t) * K + k];
                    memcpy(recv_x + r * Rw, staging_x + row * Rw, Rw);
                    if (F) memcpy(recv_sf + r * F, staging_sf + row * F, F * sizeof(float));
                    recv_src_idx[r] = (int32_t)((int64_t)s * T + t);
                    recv_topk_weights[r] = topk_weights[((size_t)s * T + t) * K + k];
                }
            }
        /* Padding rows of each expert segment: zero row and scales, source
         * index -1, weight +0. */
        for (int e = 0; e < E; ++e) {
            int64_t cnt = 0;
            for (int s = 0; s < S; ++s) cnt += tokens_per_expert[(size_t)s * E + e];
            for (int64_t r = expert_base[e] + cnt; r < expert_base[e + 1]; ++r) {
                memset(recv_x + (size_t)r * Rw, 0, Rw);
                if (F) memset(recv_sf + (size_t)r * F, 0, F * sizeof(float));
                recv_src_idx[r] = -1;
                recv_topk_weights[r] = 0.0f;
            }
        }
        (void)A;
    }
    return 0;
}

static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16; /* bf16 is the upper half of an fp32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

uint16_t epo_bf16_from_double(double v) {
    /* Nearest bf16 (8 significant bits, fp32 exponent range) with ties to
     * even, computed from the value: scale to the bf16 quantum of its binade,
     * round to an integer, scale back. */
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);        /* a = m * 2^ex with m in [0.5, 1) */
    int e = ex - 1;       /* floor(log2(a)) */
    if (e < -126) e = -126; /* subnormal bf16 share the quantum 2^-133 */
    double q = ldexp(1.0, e - 7);
    double n = nearbyint(a / q); /* default mode: nearest, ties to even */
    double r = n * q;
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
    float f = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)(u >> 16));
}

/* One token's combine row: acc = sum over valid lanes k (ascending) of
 * w[k] * Y(k) in double, then one rounding to bf16 per element. */
static void combine_token(int S, int T, int H, int K, int E, int R, int Nmax, int expand, int n_out,
                          const int64_t *topk_idx, const float *topk_weights,
                          const int32_t *dst_slot, const int32_t *recv_psum,
                          const int32_t *recv_base, const int32_t *expand_pos,
                          const uint16_t *y, const uint16_t *bias0, const uint16_t *bias1,
                          int s, int t, double *acc, uint16_t *o) {
    const int El = E / R;
    const int64_t *tok = topk_idx + ((size_t)s * T + t) * K;
    const float *w = topk_weights + ((size_t)s * T + t) * K;
    for (int h = 0; h < H; ++h) acc[h] = 0.0;
    for (int k = 0; k < K; ++k) {
        int64_t e = lane_expert(tok[k], E);
        if (e < 0) continue;
        size_t row;
        if (expand) {
            row = (size_t)expand_pos[((size_t)s * T + t) * K + k];
        } else {
            /* Non-expand: the one returned row per (token, rank), at the
             * receive position of the owner lane's slot; every lane on that
             * rank weights the same row. */
            int d = (int)(e / El);
            int k0 = owner_lane(tok, K, E, El, d);
            int64_t j = (int64_t)dst_slot[((size_t)s * T + t) * K + k0] - row_base(s, S, n_out) * Nmax;
            row = (size_t)recv_base[d] + (size_t)recv_psum[(size_t)d * (S + 1) + s] + (size_t)j;
        }
        const uint16_t *yr = y + row * (size_t)H;
        for (int h = 0; h < H; ++h) acc[h] += (double)w[k] * bf16_to_double(yr[h]);
    }
    /* Bias rows of the token (the benchmark of [DET] Performance runs the
     * combine with num_bias = 2): added to the reduced sum before the one
     * rounding. */
    const uint16_t *biases[2] = {bias0, bias1};
    for (int b = 0; b < 2; ++b) {
        if (!biases[b]) continue;
        const uint16_t *br = biases[b] + ((size_t)s * T + t) * H;
        for (int h = 0; h < H; ++h) acc[h] += bf16_to_double(br[h]);
    }
    for (int h = 0; h < H; ++h) o[h] = epo_bf16_from_double(acc[h]);
}

int epo_combine(int S, int T, int H, int K, int E, int R, int Nmax, int expand, int n_out,
                const int64_t *topk_idx, const float *topk_weights,
                const int32_t *dst_slot, const int32_t *recv_psum,
                const int32_t *recv_base, const int32_t *expand_pos,
                const uint16_t *y, uint16_t *out) {
    if (!sizes_ok(S, T, K, E, R, Nmax) || H < 1 || !topology_ok(S, n_out)) return -1;
    double *acc = (double *)malloc(sizeof(double) * (size_t)H);
    for (int s = 0; s < S; ++s)
        for (int t = 0; t < T; ++t)
            combine_token(S, T, H, K, E, R, Nmax, expand, n_out, topk_idx, topk_weights, dst_slot, recv_psum,
                          recv_base, expand_pos, y, NULL, NULL, s, t, acc, out + ((size_t)s * T + t) * H);
    free(acc);
    return 0;
}

int epo_combine_bias(int S, int T, int H, int K, int E, int R, int Nmax, int expand, int n_out,
                     const int64_t *topk_idx, const float *topk_weights,
                     const int32_t *dst_slot, const int32_t *recv_psum,
                     const int32_t *recv_base, const int32_t *expand_pos,
                     const uint16_t *y, const uint16_t *bias0, const uint16_t *bias1, uint16_t *out) {
    if (!sizes_ok(S, T, K, E, R, Nmax) || H < 1 || !topology_ok(S, n_out)) return -1;
    double *acc = (double *)malloc(sizeof(double) * (size_t)H);
    for (int s = 0; s < S; ++s)
        for (int t = 0; t < T; ++t)
            combine_token(S, T, H, K, E, R, Nmax, expand, n_out, topk_idx, topk_weights, dst_slot, recv_psum,
                          recv_base, expand_pos, y, bias0, bias1, s, t, acc, out + ((size_t)s * T + t) * H);
    free(acc);
    return 0;
}

int epo_combine_tokens(int S, int T, int H, int K, int E, int R, int Nmax, int expand, int n_out,
                       const int64_t *topk_idx, const float *topk_weights,
                       const int32_t *dst_slot, const int32_t *recv_psum,
                       const int32_t *recv_base, const int32_t *expand_pos,
                       const uint16_t *y, int n_sel, const int64_t *sel, uint16_t *out) {
    if (!sizes_ok(S, T, K, E, R, Nmax) || H < 1 || n_sel < 0 || !topology_ok(S, n_out)) return -1;
    double *acc = (double *)malloc(sizeof(double) * (size_t)H);
    for (int i = 0; i < n_sel; ++i) {
        if (sel[i] < 0 || sel[i] >= (int64_t)S * T) { free(acc); return -1; }
        int s = (int)(sel[i] / T), t = (int)(sel[i] % T);
        combine_token(S, T, H, K, E, R, Nmax, expand, n_out, topk_idx, topk_weights, dst_slot, recv_psum,
                      recv_base, expand_pos, y, NULL, NULL, s, t, acc, out + (size_t)i * H);
    }
    free(acc);
    return 0;
}
