// ep_rows.h -- row-copy helpers shared by the dispatch kernels (scatter, copy
// epilogue) and the layout-and-dispatch kernel of small problems: 16-byte
// loads and stores with cache hints, the staging record of a token, the copy
// of one staging row to its compact receive row, and a small-problem token's
// staging and receive rows written from registers.
#pragma once

#include "ep_device.h"
#include "ep_kernels.h"

namespace ep {

// Cache hints of the streamed rows (1 = non-temporal: the row is touched once
// by this kernel and not again soon).  Measured on MI355X at T=4096, H=7168:
// non-temporal loads and stores in the copy epilogue keep its 770 MB stream
// from leaving dirty or useless lines in L2 and the Infinity Cache, which
// speeds up both the epilogue and the combine that follows; non-temporal
// staging stores in the scatter slow the scatter down more than they help.
#ifndef EP_SCATTER_NT_LOAD
#define EP_SCATTER_NT_LOAD 0
#endif
#ifndef EP_SCATTER_NT_STORE
#define EP_SCATTER_NT_STORE 0
#endif
#ifndef EP_EPILOGUE_NT_LOAD
#define EP_EPILOGUE_NT_LOAD 1
#endif
#ifndef EP_EPILOGUE_NT_STORE
#define EP_EPILOGUE_NT_STORE 1
#endif

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const uint8_t *p) {
    const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
    if constexpr (NT) return __builtin_nontemporal_load(q);
    else return *q;
}
template <bool NT>
__device__ __forceinline__ void st16(uint8_t *p, u32x4 v) {
    u32x4 *q = reinterpret_cast<u32x4 *>(p);
    if constexpr (NT) __builtin_nontemporal_store(v, q);
    else *q = v;
}

// The metadata record {t, expert ids, weight bits} of token t that this lane
// stores: words i = lane (word0) and i = lane + 64 (wv_hi; K = 32 needs 65
// words), where word 0 = t, words 1..K = expert ids, words K+1..2K = weight
// bits.  Shuffled, so every lane must be active.
__device__ __forceinline__ void record_words(const Shape &sh, int t, int e, int wbits, int lane, int &word0,
                                             int &wv_hi) {
    const int ev = shfl(e, lane >= 1 ? lane - 1 : 0);
    const int wv = shfl(wbits, lane - 1 - sh.K >= 0 ? lane - 1 - sh.K : 0);
    const int hi_src = lane + kWave - 1 - sh.K;
    wv_hi = shfl(wbits, hi_src >= 0 && hi_src < kWave ? hi_src : 0);
    word0 = lane == 0 ? t : (lane <= sh.K ? ev : wv);
}

// Scales and metadata record of token g for the staging row of every owner
// lane, with every lane active before any divergent store.
__device__ __forceinline__ void store_records(const DispatchArgs &a, int64_t g, int s, int t, int e, int slot,
                                              int wbits, uint64_t owners, int lane) {
    const Shape &sh = a.sh;
    int word0, wv_hi;
    record_words(sh, t, e, wbits, lane, word0, wv_hi);
    for (uint64_t m = owners; m; m &= m - 1) {
        const int k = __builtin_ctzll(m);
        const int d = rank_of(sh, read_lane(e, k));
        const int j = read_lane(slot, k) - row_base(sh, s) * sh.Nmax;
        if ((unsigned)j >= (unsigned)sh.Nmax) continue;
        const int64_t row = staging_region(sh, d, s) * sh.Nmax + j;
        for (int i = lane; i < sh.sf_per_row; i += kWave)
            a.staging_sf[row * sh.sf_per_row + i] = a.x_sf[g * sh.sf_per_row + i];
        if (lane < sh.meta_words) a.staging_meta[row * sh.meta_words + lane] = word0;
        if (lane + kWave < sh.meta_words) a.staging_meta[row * sh.meta_words + lane + kWave] = wv_hi;
    }
}

// Receive-row index of the compact staging path, recorded by an owner lane
// (lane < K holding a slot) of token (s, t): at its compact receive row
// i = recv_base[d] + recv_psum[d][s] + j (recv_row0 = the first two terms),
// the staging row that will hold that receive row's data, so that the copy
// epilogue finds its source with one load instead of a search of the tables.
__device__ __forceinline__ void record_recv_row(const DispatchArgs &a, int s, int e, int slot, int recv_row0) {
    const Shape &sh = a.sh;
    const int d = rank_of(sh, e);
    const int j = slot - row_base(sh, s) * sh.Nmax;
    const int64_t i = (int64_t)recv_row0 + j;
    if ((unsigned)j < (unsigned)sh.Nmax && i < a.recv_capacity_rows && i < compact_rows_bound(sh))
        a.recv_row_src[i] = staging_region(sh, d, s) * sh.Nmax + j;
}

// Staging row (d, s, j) to compact receive row i = recv_base[d] +
// recv_psum[d][s] + j: the hidden row, its scales, and the per-row metadata
// derived from the record.
template <int CPL>
__device__ __forceinline__ void epilogue_row(const DispatchArgs &a, int d, int s, int j, int i, int lane, int c_lo,
                                             int c_hi) {
    const Shape &sh = a.sh;
    const int64_t row = staging_region(sh, d, s) * sh.Nmax + j;
    const uint8_t *src = a.staging_x + row * sh.row_bytes;
    uint8_t *dst = a.recv_x + (int64_t)i * sh.row_bytes;
    for (int c0 = c_lo; c0 < c_hi; c0 += CPL * kWave) {
        u32x4 v[CPL];
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
            const int c = c0 + q * kWave + lane;
            if (c < c_hi) v[q] = ld16<EP_EPILOGUE_NT_LOAD>(src + (int64_t)c * 16);
        }
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
            const int c = c0 + q * kWave + lane;
            if (c < c_hi) st16<EP_EPILOGUE_NT_STORE>(dst + (int64_t)c * 16, v[q]);
        }
    }
    if (c_lo != 0) return;  // slice 0 also moves the scales and the metadata
    for (int q = lane; q < sh.sf_per_row; q += kWave)
        a.recv_sf[(int64_t)i * sh.sf_per_row + q] = a.staging_sf[row * sh.sf_per_row + q];
    const int32_t *meta = a.staging_meta + row * sh.meta_words;
    const int t = meta[0];
    if (lane == 0) a.recv_src_idx[i] = s * sh.T + t;
    for (int k = lane; k < sh.K; k += kWave) {
        const int e = meta[1 + k];
        const bool on_d = (unsigned)e < (unsigned)sh.E && rank_of(sh, e) == d;
        a.recv_topk_idx[(int64_t)i * sh.K + k] = on_d ? e - d * sh.El : -1;
        a.recv_topk_weights[(int64_t)i * sh.K + k] = on_d ? __int_as_float(meta[1 + sh.K + k]) : 0.0f;
    }
}

// Token (s, t)'s copy on destination d in the small-problem kernels, written
// from the wave's registers: its staging row `row` and its compact receive
// row i get the hidden row v (one pass), the scales sf (lane q < sf_per_row <=
// 64 holds scale q) and their records (record_words, and the receive row's
// local ids and weights as the copy epilogue derives them).  Stores only:
// the receive row is the staging row's copy without a load between them.
template <int CPL>
__device__ __forceinline__ void token_rows(const DispatchArgs &a, int d, int s, int t, int64_t row, int64_t i,
                                           int lane, const u32x4 (&v)[CPL], float sf, int word0, int wv_hi, int e,
                                           int wbits) {
    const Shape &sh = a.sh;
    const int nchunks = sh.row_bytes / 16;
    uint8_t *stg = a.staging_x + row * sh.row_bytes;
    uint8_t *dst = a.recv_x + i * sh.row_bytes;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
        const int c = q * kWave + lane;
        if (c < nchunks) st16<EP_SCATTER_NT_STORE>(stg + (int64_t)c * 16, v[q]);
    }
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
        const int c = q * kWave + lane;
        if (c < nchunks) st16<EP_EPILOGUE_NT_STORE>(dst + (int64_t)c * 16, v[q]);
    }
    if (lane < sh.sf_per_row) {
        a.staging_sf[row * sh.sf_per_row + lane] = sf;
        a.recv_sf[i * sh.sf_per_row + lane] = sf;
    }
    if (lane < sh.meta_words) a.staging_meta[row * sh.meta_words + lane] = word0;
    if (lane + kWave < sh.meta_words) a.staging_meta[row * sh.meta_words + lane + kWave] = wv_hi;
    if (lane == 0) a.recv_src_idx[i] = s * sh.T + t;
    if (lane < sh.K) {
        const bool on_d = (unsigned)e < (unsigned)sh.E && rank_of(sh, e) == d;
        a.recv_topk_idx[i * sh.K + lane] = on_d ? e - d * sh.El : -1;
        a.recv_topk_weights[i * sh.K + lane] = on_d ? __int_as_float(wbits) : 0.0f;
    }
}

}  // namespace ep
