/*
 * oracle_sanitize_driver.c -- runs the CPU oracle (oracle/ep_oracle.c) over
 * random small configurations with every array allocated at exactly the size
 * its layout states (ep_oracle.h), so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer reports any access outside an array and any
 * undefined arithmetic (signed overflow, bad shifts, misaligned loads).
 *
 * Test infrastructure: built and run by tests/test_oracle_sanitized.py.
 * Usage: oracle_sanitize_driver [configurations] [seed]
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ep_oracle.h"

static uint64_t rng_state;

/* splitmix64 (Steele, Lea, Flood: "Fast splittable pseudorandom number
 * generators", 2014). */
static uint64_t next_u64(void) {
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static int rnd(int lo, int hi) { return lo + (int)(next_u64() % (uint64_t)(hi - lo + 1)); } /* inclusive */

/* Exactly n bytes (one for an empty array, which must then never be touched),
 * filled with random bytes so that no result depends on zeroed memory. */
static void *alloc_bytes(size_t n) {
    unsigned char *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    for (size_t i = 0; i < n; ++i) p[i] = (unsigned char)next_u64();
    return p;
}

#define ALLOC(type, count) ((type *)alloc_bytes(sizeof(type) * (size_t)(count)))

static int fail(const char *what, int cfg) {
    fprintf(stderr, "configuration %d: %s\n", cfg, what);
    return 1;
}

static int run_one(int cfg) {
    const int S = rnd(1, 3);
    int n_out = 1;
    const int pick = rnd(0, 2);
    if (pick == 1 && S > 1) n_out = S;
    if (pick == 2 && S % 2 == 0) n_out = 2;
    const int n_up = S / n_out;
    const int T = rnd(0, 40), K = rnd(1, 6);
    static const int ranks[] = {1, 2, 3, 4, 8};
    const int R = ranks[rnd(0, 4)], El = rnd(1, 4), E = R * El;
    const int Nmax = T + rnd(0, 3);
    const int expand = rnd(0, 1), A = expand ? rnd(1, 4) : 1;
    const int fp8 = rnd(0, 1);
    const int H = fp8 ? 128 * rnd(1, 2) : 8 * rnd(1, 5);
    const int Rw = fp8 ? H : 2 * H, F = fp8 ? H / 128 : 0, M = 1 + 2 * K;
    const int64_t lanes = (int64_t)S * T * K, toks = (int64_t)S * T;

    int64_t *topk = ALLOC(int64_t, lanes);
    float *w = ALLOC(float, lanes);
    for (int64_t g = 0; g < toks; ++g) {
        for (int k = 0; k < K; ++k) {
            const int r = rnd(0, 9);
            int64_t e = rnd(0, E - 1);
            if (r == 0) e = -1 - rnd(0, 2);                    /* masked */
            if (r == 1) e = E + rnd(0, 2);                     /* invalid: error flag, then masked */
            if (r == 2 && k > 0) e = topk[g * K + rnd(0, k - 1)]; /* duplicate of an earlier lane */
            topk[g * K + k] = e;
            w[g * K + k] = (float)(next_u64() >> 40) / (float)(1 << 24);
        }
    }
    int32_t *dst_slot = ALLOC(int32_t, lanes), *tpr = ALLOC(int32_t, (int64_t)S * R);
    int32_t *tpe = ALLOC(int32_t, (int64_t)S * E), *psum = ALLOC(int32_t, (int64_t)R * (S + 1));
    int32_t *base = ALLOC(int32_t, R + 1), *flags = ALLOC(int32_t, 1);
    int32_t *ebase = expand ? ALLOC(int32_t, E + 1) : NULL;
    int32_t *epos = expand ? ALLOC(int32_t, lanes) : NULL;
    int32_t *psum_up = n_out > 1 ? ALLOC(int32_t, (int64_t)R * (n_up + 1)) : NULL;
    if (epo_layout(S, T, K, E, R, Nmax, expand, A, n_out, topk, dst_slot, tpr, tpe, psum, base, ebase, epos,
                   psum_up, flags) != 0)
        return fail("epo_layout rejected valid sizes", cfg);
    /* the rows the layout fills, bounded by the receive capacity */
    const int64_t rows = expand ? ebase[E] : base[R];
    const int64_t cap = expand ? lanes + (int64_t)E * (A - 1) : toks * (K < R ? K : R);
    if (rows < 0 || rows > cap) return fail("filled rows outside the receive capacity", cfg);

    uint8_t *x = ALLOC(uint8_t, toks * Rw);
    float *x_sf = fp8 ? ALLOC(float, toks * F) : NULL;
    const int64_t srows = (int64_t)R * S * Nmax;
    uint8_t *stg = ALLOC(uint8_t, srows * Rw);
    float *stg_sf = ALLOC(float, srows * F);
    int32_t *stg_meta = ALLOC(int32_t, srows * M);
    uint8_t *rx = ALLOC(uint8_t, rows * Rw);
    float *rsf = ALLOC(float, rows * F);
    int32_t *rsrc = ALLOC(int32_t, rows);
    int32_t *rtk = expand ? NULL : ALLOC(int32_t, rows * K);
    float *rtw = ALLOC(float, expand ? rows : rows * K);
    if (epo_dispatch(S, T, H, K, E, R, Nmax, fp8, expand, A, n_out, x, x_sf, topk, w, dst_slot, tpr, tpe, psum,
                     base, ebase, epos, stg, stg_sf, stg_meta, rx, rsf, rsrc, rtk, rtw) != 0)
        return fail("epo_dispatch rejected valid sizes", cfg);

    uint16_t *y = ALLOC(uint16_t, rows * H), *out = ALLOC(uint16_t, toks * H);
    uint16_t *b0 = ALLOC(uint16_t, toks * H), *b1 = ALLOC(uint16_t, toks * H);
    if (epo_combine(S, T, H, K, E, R, Nmax, expand, n_out, topk, w, dst_slot, psum, base, epos, y, out) != 0)
        return fail("epo_combine rejected valid sizes", cfg);
    if (epo_combine_bias(S, T, H, K, E, R, Nmax, expand, n_out, topk, w, dst_slot, psum, base, epos, y, b0, b1,
                         out) != 0)
        return fail("epo_combine_bias rejected valid sizes", cfg);
    const int n_sel = toks > 0 ? rnd(1, (int)(toks < 5 ? toks : 5)) : 0;
    int64_t *sel = ALLOC(int64_t, n_sel);
    for (int i = 0; i < n_sel; ++i) sel[i] = rnd(0, (int)toks - 1);
    uint16_t *out_sel = ALLOC(uint16_t, (int64_t)n_sel * H);
    if (epo_combine_tokens(S, T, H, K, E, R, Nmax, expand, n_out, topk, w, dst_slot, psum, base, epos, y, n_sel,
                           sel, out_sel) != 0)
        return fail("epo_combine_tokens rejected valid arguments", cfg);
    /* sizes the oracle must refuse rather than read out of bounds */
    if (T > 0 && epo_layout(S, T, K, E, R, T - 1, expand, A, n_out, topk, dst_slot, tpr, tpe, psum, base, ebase,
                            epos, psum_up, flags) == 0)
        return fail("epo_layout accepted Nmax < T", cfg);

    void *all[] = {topk, w, dst_slot, tpr, tpe, psum, base, flags, ebase, epos, psum_up, x, x_sf, stg, stg_sf,
                   stg_meta, rx, rsf, rsrc, rtk, rtw, y, out, b0, b1, sel, out_sel};
    for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i) free(all[i]);
    return 0;
}

int main(int argc, char **argv) {
    const int n = argc > 1 ? atoi(argv[1]) : 200;
    rng_state = argc > 2 ? strtoull(argv[2], NULL, 10) : 12345u;
    for (int c = 0; c < n; ++c)
        if (run_one(c)) return 1;
    /* rounding at the special values: zero, ties, the largest finite bf16, overflow, NaN */
    static const double specials[] = {0.0, -0.0, 1.0, 1.00390625, 1.01171875, -1.00390625, 3.3895313892515355e38,
                                      3.3961775292304766e38, 1e39, -1e39, 1e-45, -1e-45};
    unsigned acc = 0;
    for (size_t i = 0; i < sizeof(specials) / sizeof(specials[0]); ++i) acc += epo_bf16_from_double(specials[i]);
    acc += epo_bf16_from_double(__builtin_nan(""));
    printf("%d configurations ok (%u)\n", n, acc);
    return 0;
}
