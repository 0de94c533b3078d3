// ep_layout.hip -- deterministic dispatch layout prologue on gfx950.
//
// DeepEP v2 "Kernel-side deterministic dispatch for the non-expand layout"
// (PR #753), section Approach: the slot of every deduplicated (token,
// destination) entry is row_base * Nmax + the sender's running count of such
// entries to that destination, computed by a two-pass scan so that placement
// is a pure function of topk_idx.  Section Motivation: the top-k lanes of a
// token are deduplicated by destination rank (one lane per destination sends)
// instead of racing on an atomic counter.
//
// Design on CDNA4.  Work is cut into "units" of consecutive tokens of one
// source: one workgroup of 4 wavefronts per unit, each wave owning a quarter.
// A wave walks its tokens in steps of floor(64/K) tokens, one (token, lane)
// item per SIMD lane, items in (t, k) order; the items of up to kBatch steps
// are loaded with one batch of independent loads, so a wave pays about one
// memory latency per pass.  Equal destinations (or experts) inside a step are
// found with one ballot per key bit; the exclusive rank of an item among equal
// keys is a masked popcount (mbcnt), and the highest lane of each key group
// advances a per-wave running counter in LDS.  Nothing is decided by atomics
// on memory, so the result never depends on scheduling.
//
//   k_layout_count: per-unit counts of owner lanes per destination and of
//     valid lanes per expert, plus an invalid-id flag, into scratch;
//   k_layout_expert_scan (expand only): for every expert, the valid lanes of
//     all earlier units (a column prefix over units) and the total;
//   k_layout_slot: each unit reduces the counts of the earlier units of its
//     source (its base per destination), recounts per wave for the wave
//     bases, then ranks every item and writes dst_slot (and expand_pos); the
//     units also share out the per-source counts; expand adds the expert
//     segment bases (padded totals, scanned over experts) to each unit's
//     column prefix; one extra workgroup writes the receiver tables
//     (recv_psum, recv_base, expert_base, error_flags);
//   k_layout_single: for one source whose items fit one workgroup, all of the
//     above in one launch (the unit's counts are the source's totals);
//   k_layout_fused: the compact layout in one launch, the page's cooperative
//     two-pass form: every unit counts and publishes its counts, one
//     coordinating workgroup waits for all of them and releases the units,
//     which then rank their items from the counts they kept in LDS; the
//     coordinator builds the receiver tables meanwhile.  Used when the whole
//     grid fits on the device at once (checked on the host); otherwise, and
//     for the expand layout, the separate launches above run.
#include <map>
#include <mutex>
#include <utility>

#include "ep.h"
#include "ep_device.h"
#include "ep_kernels.h"
#include "ep_rows.h"

namespace ep {

// Layout workgroups of 4 waves: measured on MI355X against 8 and 16 waves
// with 32-128 units, which were 10-60% slower at T=4096 and 16 x 2048.
constexpr int kLayoutThreads = 256;
constexpr int kLayoutWaves = kLayoutThreads / kWave;
constexpr int kBatch = 8;  // steps whose items a wave loads together
#ifndef EP_LAYOUT_SINGLE_MAX_ITEMS
#define EP_LAYOUT_SINGLE_MAX_ITEMS 2048  // largest T*K laid out by one workgroup (S == 1)
#endif
constexpr int kScanThreads = 1024;

// LDS of the one-workgroup layout with nw waves: counts [nw][R+E], bases
// [R+E], scan scratch [64 nw], flags [nw].
__host__ __device__ inline size_t single_lds_bytes(const Shape &sh, int nw) {
    return sizeof(int) * ((size_t)nw * (sh.R + sh.E) + sh.R + sh.E + (size_t)nw * kWave + nw);
}
constexpr int kScanCols = 64;                        // experts per scan workgroup
constexpr int kScanSegs = kScanThreads / kScanCols;  // unit segments per expert
constexpr int kScanRegs = 16;                        // counts a scan thread keeps in registers

LayoutGeom layout_geometry(const Shape &sh, int num_layout_cus) {
    LayoutGeom g;
    const int64_t T = sh.T;  // the arithmetic below is 64-bit; every result fits an int for T <= 2^30
    // Measured on MI355X (T=4096 and 16 x 2048 tokens, K=8): about 256 units
    // of at least one step per wave are fastest; fewer, longer units leave CUs
    // idle, more units lengthen the gathers of the unit counts.
    const int tps = kWave / sh.K;              // tokens per step
    const int min_chunk = kLayoutWaves * tps;  // one step per wave
    const int64_t max_b = T > kLayoutWaves ? (T + kLayoutWaves - 1) / kLayoutWaves : 1;  // >= one token per wave
    g.single = 0;
    // One source with at most 2048 (token, lane) items: the whole layout in one
    // workgroup, 8 waves up to 1024 items, 16 above.  Measured on MI355X at
    // K=8: 4.4 / 5.7 / 7.4 us at T = 64 / 128 / 256 against 8.0-8.5 us for the
    // two launches (expand: 6.2 / 7.9 / 10.5 against 13.7-13.9 us); at 4096
    // items the two launches are faster (8.5 against 10.7 us).
    const int64_t lanes = (int64_t)T * sh.K;
    if (num_layout_cus == 0 && sh.S == 1 && lanes <= EP_LAYOUT_SINGLE_MAX_ITEMS) {
        const int nw = lanes <= 1024 ? 8 : 16;
        if (single_lds_bytes(sh, nw) <= 65536) {
            g.blocks_per_src = 1;
            g.chunk = T > 0 ? (int)((T + 3) / 4 * 4) : 4;
            g.single = nw;
            return g;
        }
    }
    int64_t B;
    if (num_layout_cus > 0) {
        B = ((int64_t)num_layout_cus + sh.S - 1) / sh.S;
    } else {
        const int64_t target_units = 256;
        const int64_t by_size = (T + min_chunk - 1) / min_chunk;
        const int64_t by_units = (target_units + sh.S - 1) / sh.S;
        B = by_size < by_units ? by_size : by_units;
    }
    if (B > max_b) B = max_b;
    if (B < 1) B = 1;
    int64_t chunk = T > 0 ? (T + B - 1) / B : kLayoutWaves;
    chunk = (chunk + kLayoutWaves - 1) / kLayoutWaves * kLayoutWaves;  // equal wave ranges
    B = T > 0 ? (T + chunk - 1) / chunk : 1;
    g.blocks_per_src = (int)B;
    g.chunk = (int)chunk;
    return g;
}

uint64_t layout_scratch_bytes(const Shape &sh, const LayoutGeom &g) {
    const uint64_t units = (uint64_t)sh.S * g.blocks_per_src;
    const uint64_t counts =
        (units * (uint64_t)(sh.R + sh.E + 1 + (sh.expand ? sh.E : 0)) + (sh.expand ? sh.E : 0)) * sizeof(int32_t);
    // the compact layout's one-launch exchange: 8-byte words after the counts
    // (plus up to 4 bytes to align them)
    return sh.expand ? counts : counts + 4 + layout_sync_words(units) * sizeof(uint64_t);
}

namespace {

// Per-lane view of one step: which (token, lane) item this lane holds and how
// it ranks among the step's items with the same destination / expert.
struct Item {
    bool in, valid, invalid, owner;
    int t, k, d, e;
    int owner_lane;     // valid only: the lowest lane of the token with the same destination
    int rank_d, cnt_d;  // owners only: exclusive rank / group size among owners of d
    bool last_d;        // highest owner lane of its destination group
    int rank_e, cnt_e;  // valid only: same among valid lanes of expert e
    bool last_e;
};

struct StepCtx {
    int lane, l_tok, l_k;
    bool used;     // lane holds an item slot in every step (l < tps*K)
    uint64_t seg;  // lanes of the same token
    int tps;       // tokens per step
};

__device__ __forceinline__ StepCtx make_ctx(int K) {
    StepCtx c;
    c.lane = lane_id();
    c.tps = kWave / K;
    c.l_tok = c.lane / K;
    c.l_k = c.lane - c.l_tok * K;
    c.used = c.l_tok < c.tps;
    const uint64_t tok_bits = (K == 64) ? ~0ull : ((1ull << K) - 1ull);
    c.seg = c.used ? (tok_bits << (c.l_tok * K)) : 0ull;
    return c;
}

// Expert ids of kBatch consecutive steps from token ts (-1 for lanes without
// an item).  They stay raw until make_item, so that nothing waits on the
// loads before the wave has issued the rest of its loads.
__device__ __forceinline__ void load_batch(const Shape &sh, const int64_t *topk_src, int ts, int t_end,
                                           const StepCtx &c, int64_t (&ids)[kBatch]) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
        const int t = ts + i * c.tps + c.l_tok;
        ids[i] = (c.used && t < t_end) ? topk_src[(int64_t)t * sh.K + c.l_k] : (int64_t)-1;
    }
}

__device__ __forceinline__ Item make_item(const Shape &sh, int64_t e64, int t_step, int t_end, const StepCtx &c,
                                          bool need_e) {
    Item it;
    it.t = t_step + c.l_tok;
    it.k = c.l_k;
    it.in = c.used && it.t < t_end;
    it.invalid = it.in && e64 >= sh.E;
    it.valid = it.in && e64 >= 0 && e64 < sh.E;
    it.e = it.valid ? (int)e64 : 0;
    it.d = rank_of(sh, it.e);
    const uint64_t vmask = ballot(it.valid);
    const uint64_t peers_d = match_key((uint32_t)it.d, sh.bits_R, vmask);
    it.owner = it.valid && ((peers_d & c.seg & mask_lt(c.lane)) == 0);
    const uint64_t same = peers_d & c.seg;
    it.owner_lane = it.valid && same ? __builtin_ctzll(same) : c.lane;
    const uint64_t po = peers_d & ballot(it.owner);
    it.rank_d = prefix_count(po);
    it.cnt_d = popc(po);
    it.last_d = it.owner && ((po & mask_gt(c.lane)) == 0);
    if (need_e) {
        const uint64_t pe = match_key((uint32_t)it.e, sh.bits_E, vmask);
        it.rank_e = prefix_count(pe);
        it.cnt_e = popc(pe);
        it.last_e = it.valid && ((pe & mask_gt(c.lane)) == 0);
    } else {
        it.rank_e = it.cnt_e = 0;
        it.last_e = false;
    }
    return it;
}

// f(item) for every step of tokens [t0, t1) of one source, in token order.
// The ids come in batches of kBatch steps (one memory latency per batch);
// when `have_first` the first batch is already in `first`.  The step loop
// stays rolled: each layout workgroup runs once on its CU, cold in the
// instruction cache, so every inlined copy of the step costs fetch latency.
template <typename F>
__device__ __forceinline__ void walk_steps(const Shape &sh, const int64_t *topk_src, int t0, int t1,
                                           const StepCtx &c, const int64_t (&first)[kBatch], bool have_first,
                                           bool need_e, F &&f) {
    for (int tb = t0; tb < t1; tb += kBatch * c.tps) {
        int64_t ids[kBatch];
        if (have_first && tb == t0) {
#pragma unroll
            for (int i = 0; i < kBatch; ++i) ids[i] = first[i];
        } else {
            load_batch(sh, topk_src, tb, t1, c, ids);
        }
#pragma unroll 1
        for (int i = 0, ts = tb; i < kBatch && ts < t1; ++i, ts += c.tps) {
            f(make_item(sh, ids[0], ts, t1, c, need_e));
#pragma unroll
            for (int j = 0; j + 1 < kBatch; ++j) ids[j] = ids[j + 1];
        }
    }
}

__device__ __forceinline__ void count_item(const Item &it, int *cnt_d, int *cnt_e, bool need_e, bool &bad) {
    if (it.last_d) cnt_d[it.d] += it.cnt_d;
    if (need_e && it.last_e) cnt_e[it.e] += it.cnt_e;
    bad |= it.invalid;
}

// Count owner lanes per destination (and valid lanes per expert) over tokens
// [t0, t1) of one source into this wave's LDS rows; returns the invalid flag.
__device__ __forceinline__ bool wave_count(const Shape &sh, const int64_t *topk_src, int t0, int t1, int *cnt_d,
                                           int *cnt_e, bool need_e, const StepCtx &c, const int64_t (&first)[kBatch],
                                           bool have_first) {
    bool bad = false;
    walk_steps(sh, topk_src, t0, t1, c, first, have_first, need_e,
               [&](const Item &it) { count_item(it, cnt_d, cnt_e, need_e, bad); });
    return ballot(bad) != 0;
}

// Exclusive scan of a[0..n) in LDS by the whole workgroup; returns the total.
template <int NT>
__device__ int block_exclusive_scan(int *a, int n, int *part) {
    const int tid = threadIdx.x;
    const int per = (n + NT - 1) / NT;
    const int lo = min(tid * per, n), hi = min(lo + per, n);
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += a[i];
    part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
        const int v = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int run = part[tid] - sum;
    const int total = part[NT - 1];
    for (int i = lo; i < hi; ++i) {
        const int v = a[i];
        a[i] = run;
        run += v;
    }
    __syncthreads();
    return total;
}

// lds[j] += the sum over rows r in [0, nrows) of p_j[r * stride_j] for every
// column j in [0, ncols), where col(j, stride_j) returns p_j.  Each thread
// owns one column of a group of up to 256 and every (256 / group)-th row,
// sums in a register with up to 8 loads in flight, and adds once to LDS.
template <typename Col>
__device__ __forceinline__ void column_sums(int nrows, int ncols, int *lds, Col col) {
    for (int jg = 0; jg < ncols; jg += kLayoutThreads) {
        const int nc = min(ncols - jg, kLayoutThreads);
        const int rstep = kLayoutThreads / nc;
        const int r0 = threadIdx.x / nc, j = jg + (threadIdx.x - r0 * nc);
        if (r0 >= rstep) continue;
        int64_t stride;
        const int32_t *p = col(j, stride);
        int sum = 0;
        for (int r = r0; r < nrows; r += 8 * rstep) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int rr = r + u * rstep;
                v[u] = rr < nrows ? p[(int64_t)rr * stride] : 0;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) sum += v[u];
        }
        if (sum != 0) atomicAdd(&lds[j], sum);
    }
}

// The same column sums for at most 256 columns, split so that the loads can
// be issued long before their sums are needed: column_issue() starts each
// thread's first 8 rows, column_finish() adds them (and any further rows,
// loaded then) into LDS.  Between the two the wave does other work while the
// loads are in flight.
struct ColumnLoads {
    int v[8];
    const int32_t *p;
    int64_t stride;
    int j, r0, rstep, nrows;
    bool on;
};

template <typename Col>
__device__ __forceinline__ void column_issue(ColumnLoads &cl, int nrows, int ncols, Col col) {
    const int nc = ncols > 0 ? ncols : 1;  // ncols <= kLayoutThreads
    cl.nrows = nrows;
    cl.rstep = kLayoutThreads / nc;
    cl.r0 = threadIdx.x / nc;
    cl.j = threadIdx.x - cl.r0 * nc;
    cl.on = ncols > 0 && cl.r0 < cl.rstep;
    cl.stride = 0;
    cl.p = cl.on ? col(cl.j, cl.stride) : nullptr;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int rr = cl.r0 + u * cl.rstep;
        cl.v[u] = (cl.on && rr < nrows) ? cl.p[(int64_t)rr * cl.stride] : 0;
    }
}

__device__ __forceinline__ void column_finish(const ColumnLoads &cl, int *lds) {
    if (!cl.on) return;
    int sum = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += cl.v[u];
    for (int r = cl.r0 + 8 * cl.rstep; r < cl.nrows; r += cl.rstep) sum += cl.p[(int64_t)r * cl.stride];
    if (sum != 0) atomicAdd(&lds[cl.j], sum);
}

__device__ __forceinline__ void wave_range(const LayoutArgs &a, int b, int w, int &t0, int &t1) {
    const int cw = a.g.chunk / kLayoutWaves;
    t0 = min(b * a.g.chunk + w * cw, a.sh.T);
    t1 = min(t0 + cw, a.sh.T);
}

// Per-wave counts [NW][n] in LDS become each wave's running base: base[i]
// plus the counts of the earlier waves.  Every thread of the workgroup calls it.
template <int NW = kLayoutWaves>
__device__ __forceinline__ void wave_bases(int *cnt, int n, const int *base) {
    for (int i = threadIdx.x; i < n; i += NW * kWave) {
        int run = base[i];
        for (int q = 0; q < NW; ++q) {
            const int v = cnt[q * n + i];
            cnt[q * n + i] = run;
            run += v;
        }
    }
}

// The expand index entry of a valid lane (alignment 1): at its expand row
// re + rank_e, the staging row of (d, s) that holds its token -- row j, its
// owner's slot relative to the source's row base -- and the lane.
__device__ __forceinline__ void record_expand_row(const LayoutArgs &a, int s, const Item &it, int j, int re) {
    const Shape &sh = a.sh;
    const int64_t pos = (int64_t)re + it.rank_e;
    if (!it.valid || (unsigned)j >= (unsigned)sh.Nmax || pos >= expand_rows_bound(sh)) return;
    a.expand_row_src[pos] = (staging_region(sh, it.d, s) * sh.Nmax + j) | ((int64_t)it.k << 56);
}

// Ranking: every item of the wave's tokens [t0, t1) of source s gets its slot
// (row_base * Nmax + running count, [DET] Approach) and, in the expand layout,
// its row (and, with an expand index, that row's entry); run_d / run_e are the
// wave's running counters in LDS.
__device__ __forceinline__ void rank_items(const LayoutArgs &a, bool expand, int s, int t0, int t1,
                                           const StepCtx &c, const int64_t (&first)[kBatch], bool have_first,
                                           int *run_d, int *run_e) {
    const Shape &sh = a.sh;
    const int32_t slot_base = row_base(sh, s) * sh.Nmax;
    const int64_t *topk_src = a.topk_idx + (int64_t)s * sh.T * sh.K;
    walk_steps(sh, topk_src, t0, t1, c, first, have_first, expand, [&](const Item &it) {
        const int rd = it.owner ? run_d[it.d] : 0;
        const int re = (expand && it.valid) ? run_e[it.e] : 0;
        const int slot = it.owner ? slot_base + rd + it.rank_d : -1;
        if (it.in) {
            const int64_t idx = ((int64_t)s * sh.T + it.t) * sh.K + it.k;
            a.dst_slot[idx] = slot;
            if (expand) a.expand_pos[idx] = it.valid ? re + it.rank_e : -1;
        }
        if (expand && a.expand_row_src) record_expand_row(a, s, it, shfl(slot, it.owner_lane) - slot_base, re);
        if (it.last_d) run_d[it.d] = rd + it.rank_d + 1;
        if (expand && it.last_e) run_e[it.e] = re + it.rank_e + 1;
    });
}

__global__ void __launch_bounds__(kLayoutThreads) k_layout_count(LayoutArgs a) {
    const Shape &sh = a.sh;
    const int b = blockIdx.x, s = blockIdx.y, B = a.g.blocks_per_src;
    const int w = threadIdx.x / kWave, tid = threadIdx.x;
    extern __shared__ int lds[];
    int *cnt_d = lds;                          // [waves][R]
    int *cnt_e = cnt_d + kLayoutWaves * sh.R;  // [waves][E]
    int *flag = cnt_e + kLayoutWaves * sh.E;   // [waves]

    int t0, t1;
    wave_range(a, b, w, t0, t1);
    const StepCtx c = make_ctx(sh.K);
    const bool single = t1 - t0 <= kBatch * c.tps;
    const int64_t *topk_src = a.topk_idx + (int64_t)s * sh.T * sh.K;
    int64_t first[kBatch] = {};
    if (single) load_batch(sh, topk_src, t0, t1, c, first);  // in flight while LDS is cleared
    for (int i = tid; i < kLayoutWaves * (sh.R + sh.E); i += kLayoutThreads) lds[i] = 0;
    __syncthreads();

    const bool bad = wave_count(sh, topk_src, t0, t1, cnt_d + w * sh.R, cnt_e + w * sh.E, true, c, first, single);
    if (lane_id() == 0) flag[w] = bad ? 1 : 0;
    __syncthreads();

    const int64_t u = (int64_t)s * B + b;
    for (int d = tid; d < sh.R; d += kLayoutThreads) {
        int v = 0;
        for (int q = 0; q < kLayoutWaves; ++q) v += cnt_d[q * sh.R + d];
        a.blk_cnt_rank[u * sh.R + d] = v;
    }
    for (int e = tid; e < sh.E; e += kLayoutThreads) {
        int v = 0;
        for (int q = 0; q < kLayoutWaves; ++q) v += cnt_e[q * sh.E + e];
        a.blk_cnt_expert[u * sh.E + e] = v;
    }
    if (tid == 0) {
        int any = 0;
        for (int q = 0; q < kLayoutWaves; ++q) any |= flag[q];
        a.blk_flags[u] = any;
    }
}

// Expand layout only.  Workgroup x covers experts [64x, 64x + 64); thread
// (seg, c) owns expert e = 64x + c over one of 16 contiguous segments of the
// units (units in (s, t) order), loads its counts in batches of independent
// loads (keeping up to 16 in registers for the second pass), and the 16
// segment sums of each expert are prefixed in LDS.  Writes blk_pre_expert[u][e]
// (valid lanes of units before u on expert e) and cnt_expert[e].
__global__ void __launch_bounds__(kScanThreads) k_layout_expert_scan(LayoutArgs a) {
    const Shape &sh = a.sh;
    const int E = sh.E, tid = threadIdx.x;
    const int64_t U = (int64_t)sh.S * a.g.blocks_per_src;
    const int c = tid % kScanCols, seg = tid / kScanCols;
    const int e = blockIdx.x * kScanCols + c;
    const bool active = e < E;
    const int64_t u0 = U * seg / kScanSegs, u1 = U * (seg + 1) / kScanSegs;
    const bool in_regs = u1 - u0 <= kScanRegs;
    __shared__ int part[kScanSegs][kScanCols];
    int v[kScanRegs];
    int sum = 0;
    if (active && in_regs) {
#pragma unroll
        for (int q = 0; q < kScanRegs; ++q) v[q] = u0 + q < u1 ? a.blk_cnt_expert[(u0 + q) * E + e] : 0;
#pragma unroll
        for (int q = 0; q < kScanRegs; ++q) sum += v[q];
    } else if (active) {
        for (int64_t u = u0; u < u1; ++u) sum += a.blk_cnt_expert[u * E + e];
    }
    part[seg][c] = sum;
    __syncthreads();
    int run = 0;
    for (int q = 0; q < seg; ++q) run += part[q][c];
    if (active && seg == kScanSegs - 1) a.cnt_expert[e] = run + sum;
    if (!active) return;
    if (in_regs) {
#pragma unroll
        for (int q = 0; q < kScanRegs; ++q) {
            if (u0 + q < u1) a.blk_pre_expert[(u0 + q) * E + e] = run;
            run += v[q];
        }
    } else {
        for (int64_t u = u0; u < u1; ++u) {
            a.blk_pre_expert[u * E + e] = run;
            run += a.blk_cnt_expert[u * E + e];
        }
    }
}

// Expert segment bases (expand): seg[e] <- sum over e' < e of the valid lanes
// of expert e' padded up to a multiple of A; returns the total.  Every thread
// of the workgroup calls it; seg has E entries in LDS, part 256.
__device__ int expert_segment_bases(const LayoutArgs &a, int *seg, int *part) {
    const Shape &sh = a.sh;
    for (int e = threadIdx.x; e < sh.E; e += kLayoutThreads) {
        const int cnt = a.cnt_expert[e];
        seg[e] = (cnt + sh.A - 1) / sh.A * sh.A;
    }
    __syncthreads();
    return block_exclusive_scan<kLayoutThreads>(seg, sh.E, part);
}

// Receiver tables, built by one extra workgroup of the slot pass while the
// units rank their items: the per-(source, destination) totals are reduced
// from the unit counts (LDS integer adds), then prefixed over sources into
// recv_psum (and, on the hybrid path, over scale-up segments into
// recv_psum_scaleup) and over destinations into recv_base; the units' invalid
// flags are OR-ed into error_flags; expand also writes expert_base.
__device__ __forceinline__ void build_receiver_tables(const LayoutArgs &a, bool expand, int *lds) {
    const Shape &sh = a.sh;
    const int tid = threadIdx.x, w = tid / kWave;
    const int R = sh.R, E = sh.E, S = sh.S, B = a.g.blocks_per_src;
    const int64_t U = (int64_t)S * B;
    int *part = lds + kLayoutWaves * (R + E) + R + E + (R + E);  // [256], as in the unit layout
    int *tot = lds;                                               // [S][R] if it fits
    const bool fits = (int64_t)S * R <= (int64_t)kLayoutWaves * (R + E);
    int bad = 0;
    for (int64_t q = tid; q < U; q += kLayoutThreads) bad |= a.blk_flags[q];  // in flight with the gather
    if (expand) {
        int *eb = lds + kLayoutWaves * (R + E) + R;  // [E], unused by the rest of this workgroup
        const int total = expert_segment_bases(a, eb, part);
        for (int e = tid; e < E; e += kLayoutThreads) a.expert_base[e] = eb[e];
        if (tid == 0) a.expert_base[E] = total;
        __syncthreads();
    }
    if (fits) {
        for (int i = tid; i < S * R; i += kLayoutThreads) tot[i] = 0;
        __syncthreads();
        column_sums(B, S * R, tot, [&](int p, int64_t &stride) {  // column p = (source, destination)
            stride = R;
            return a.blk_cnt_rank + (int64_t)(p / R) * B * R + p % R;
        });
        __syncthreads();
    }
    // recv_psum: per destination, the exclusive prefix over sources of the
    // per-(source, destination) totals.  Few sources (per-thread walk no
    // longer than the scans' barriers): one thread per destination walks
    // them.  Many: the totals go to recv_psum[d][s] in parallel, then the
    // workgroup scans each destination's row in place.
    int *tot_d = part;  // [R] totals per destination (R <= 64)
    const bool walk = (int64_t)S * (fits ? 1 : B) <= 64 * (int64_t)R;
    if (!walk) {
        for (int64_t p = tid; p < (int64_t)S * R; p += kLayoutThreads) {
            const int q = (int)(p / R), d = (int)(p - (int64_t)q * R);
            int c = 0;
            if (fits) {
                c = tot[p];
            } else {
                for (int bb = 0; bb < B; ++bb) c += a.blk_cnt_rank[((int64_t)q * B + bb) * R + d];
            }
            a.recv_psum[(int64_t)d * (S + 1) + q] = c;
        }
        __syncthreads();
        tot_d = lds;  // the per-(source, destination) totals in LDS are no longer needed
        for (int d = 0; d < R; ++d) {
            int32_t *ps = a.recv_psum + (int64_t)d * (S + 1);
            const int total = block_exclusive_scan<kLayoutThreads>(ps, S, part);
            if (tid == 0) {
                ps[S] = total;
                tot_d[d] = total;
            }
        }
        __syncthreads();
    }
    for (int d = tid; d < R; d += kLayoutThreads) {
        if (walk) {
            int run = 0;
            for (int q = 0; q < S; ++q) {
                a.recv_psum[(int64_t)d * (S + 1) + q] = run;
                if (fits) {
                    run += tot[q * R + d];
                } else {
                    for (int bb = 0; bb < B; ++bb) run += a.blk_cnt_rank[((int64_t)q * B + bb) * R + d];
                }
            }
            a.recv_psum[(int64_t)d * (S + 1) + S] = run;
            tot_d[d] = run;
        }
        if (sh.n_out > 1) {
            // Hybrid row form: prefix over scale-up segments; segment u
            // holds the sources s with s % n_up == u.
            int32_t *ps = a.recv_psum_scaleup + (int64_t)d * (sh.n_up + 1);
            int seg_run = 0;
            for (int u = 0; u < sh.n_up; ++u) {
                ps[u] = seg_run;
                for (int o = 0; o < sh.n_out; ++o) {
                    const int q = o * sh.n_up + u;
                    seg_run += a.recv_psum[(int64_t)d * (S + 1) + q + 1] - a.recv_psum[(int64_t)d * (S + 1) + q];
                }
            }
            ps[sh.n_up] = seg_run;
        }
    }
    bad = ballot(bad != 0) != 0;
    if (lane_id() == 0) part[64 + w] = bad;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int d = 0; d < R; ++d) {
            a.recv_base[d] = run;
            run += tot_d[d];
        }
        a.recv_base[R] = run;
        int any = 0;
        for (int q = 0; q < kLayoutWaves; ++q) any |= part[64 + q];
        __hip_atomic_store(a.error_flags, any ? 1 : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// One instance per layout kind, so that the compact layout's kernel carries
// none of the expand code (each workgroup runs once, cold in the instruction
// cache).
template <bool EXPAND>
__global__ void __launch_bounds__(kLayoutThreads) k_layout_slot(LayoutArgs a) {
    const Shape &sh = a.sh;
    const int b = blockIdx.x, s = blockIdx.y, B = a.g.blocks_per_src;
    const int w = threadIdx.x / kWave, tid = threadIdx.x;
    const int R = sh.R, E = sh.E;
    constexpr bool expand = EXPAND;
    const int64_t me = (int64_t)s * B + b;

    extern __shared__ int lds[];
    if (b == B) {  // the extra column: workgroup (B, 0) builds the receiver tables
        if (s == 0) build_receiver_tables(a, expand, lds);
        return;
    }
    int *cnt_d = lds;                       // [waves][R] per-wave counts, then running bases
    int *cnt_e = cnt_d + kLayoutWaves * R;  // [waves][E]
    int *base_d = cnt_e + kLayoutWaves * E; // [R]   this unit's base per destination
    int *base_e = base_d + R;               // [E]   expand: this unit's first row per expert
    int *col = base_e + E;                  // [R+E] per-source totals of this unit's share of columns

    int t0, t1;
    wave_range(a, b, w, t0, t1);
    const StepCtx c = make_ctx(sh.K);
    const bool single = t1 - t0 <= kBatch * c.tps;
    const int64_t *topk_src = a.topk_idx + (int64_t)s * sh.T * sh.K;
    int64_t first[kBatch] = {};
    if (single) load_batch(sh, topk_src, t0, t1, c, first);

    // Every global load of the unit is issued here, before the first barrier,
    // so that the ids, the unit base and the per-source totals cost one
    // memory latency together.  Unit base per destination: what the earlier
    // units of this source send there.
    const int32_t *src_rank = a.blk_cnt_rank + (int64_t)s * B * R;
    ColumnLoads lb, lc;
    column_issue(lb, b, R, [&](int d, int64_t &stride) {
        stride = R;
        return src_rank + d;
    });
    // This unit's share of the per-source totals: columns b, b+B, ...
    // (destinations first, then experts), each summed over the source's units;
    // with more than 256 such columns (few units per source) they are summed
    // at the end instead.
    const int ncol = b < R + E ? (R + E - b + B - 1) / B : 0;
    auto col_src = [&](int j, int64_t &stride) -> const int32_t * {
        const int cidx = b + j * B;
        if (cidx < R) {
            stride = R;
            return a.blk_cnt_rank + (int64_t)s * B * R + cidx;
        }
        stride = E;
        return a.blk_cnt_expert + (int64_t)s * B * E + (cidx - R);
    };
    const bool col_early = ncol <= kLayoutThreads;
    column_issue(lc, B, col_early ? ncol : 0, col_src);

    for (int i = tid; i < kLayoutWaves * (R + E) + R + E + (R + E); i += kLayoutThreads) lds[i] = 0;
    __syncthreads();
    if (expand) {
        // First row of this unit in expert e's segment: the segment base plus
        // what the earlier units put there.
        int *part = col + R + E;
        int pre[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = tid + q * kLayoutThreads;
            pre[q] = e < E ? a.blk_pre_expert[me * E + e] : 0;
        }
        expert_segment_bases(a, base_e, part);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = tid + q * kLayoutThreads;
            if (e < E) base_e[e] += pre[q];
        }
    }

    // Per-wave counts of this unit, then each wave's running base.
    wave_count(sh, topk_src, t0, t1, cnt_d + w * R, cnt_e + w * E, expand, c, first, single);
    column_finish(lb, base_d);
    __syncthreads();
    wave_bases(cnt_d, R, base_d);
    if (expand) wave_bases(cnt_e, E, base_e);
    __syncthreads();
    rank_items(a, expand, s, t0, t1, c, first, single, cnt_d + w * R, cnt_e + w * E);

    if (col_early) column_finish(lc, col);
    else column_sums(B, ncol, col, col_src);
    __syncthreads();
    for (int j = tid; j < ncol; j += kLayoutThreads) {
        const int cidx = b + j * B;
        if (cidx < R) a.tokens_per_rank[(int64_t)s * R + cidx] = col[j];
        else a.tokens_per_expert[(int64_t)s * E + cidx - R] = col[j];
    }
}

// ------------------------------------------------ one-launch layout
// Grid-wide exchange.  Each launch derives fresh 64-bit tokens from an epoch
// word that the coordinator advances at the end of every launch, so nothing
// needs resetting between launches (nor initialising: a stale or arbitrary
// word equals a token of this launch with probability 2^-64), HIP-graph
// replays get new tokens, and no memset is involved.  A unit publishes its
// counts, then stores its arrival token; every unit waits for the arrivals of
// all units of its source (it needs their counts for its base and its share of
// the source's totals), and the coordinator waits for all arrivals before it
// builds the receiver tables.  Every wait is bounded: a unit that times out
// stores a give-up token in its arrival word, skips the slot pass and sets
// bit 1 of error_flags; a coordinator that times out (or sees a give-up)
// skips the tables and sets bit 1.  The tables of such a call are not valid.
enum : uint64_t { kTokArrive = 1, kTokGiveUp = 2 };

// A 64-bit mix of (epoch, unit, kind): the SplitMix64 finaliser applied to a
// combination of the three.
__device__ __forceinline__ uint64_t sync_token(uint64_t epoch, uint64_t unit, uint64_t kind) {
    uint64_t z = epoch * 0x9E3779B97F4A7C15ull + (unit + 1) * 0xD1B54A32D192ED03ull + kind * 0xA0761D6478BD642Full;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t sync_load(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sync_store(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded wait of the whole workgroup for the arrivals of units [u0, u1):
// thread i polls units u0 + i, u0 + i + 256, ...  `flip` (tests only) makes
// the awaited word one that nobody writes.  Returns nonzero (in every thread)
// if some unit gave up or a poll ran out of its `limit`.
__device__ __forceinline__ int wait_arrivals(const LayoutArgs &a, uint64_t e1, int64_t u0, int64_t u1, uint32_t limit,
                                             uint64_t flip) {
    int late = 0;
    for (int64_t u = u0 + threadIdx.x; u < u1 && !late; u += kLayoutThreads) {
        const uint64_t want = sync_token(e1, (uint64_t)u, kTokArrive) ^ flip;
        const uint64_t gave = sync_token(e1, (uint64_t)u, kTokGiveUp);
        for (uint32_t n = 0;; ++n) {
            const uint64_t v = sync_load(a.sync + 1 + u);
            if (v == want) break;
            if (v == gave || n >= limit) {
                late = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    // Each thread that saw arrivals acquires them (pairs with the arriving
    // workgroup's release); the barrier inside __syncthreads_or then orders
    // every later read of the workgroup after those acquires.
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return __syncthreads_or(late);
}

// The coordinating workgroup: waits for every unit's arrival, builds the
// receiver tables and writes error_flags (bit 0 from the units' invalid-id
// flags, bit 1 on a time-out); finally advances the epoch for the next launch.
__device__ void fused_coordinator(const LayoutArgs &a, int *lds, uint64_t *epoch_sh) {
    const int tid = threadIdx.x;
    const int64_t U = (int64_t)a.sh.S * a.g.blocks_per_src;
    if (tid == 0) *epoch_sh = sync_load(a.sync);
    __syncthreads();
    const uint64_t e1 = *epoch_sh + 1;
    const int late = wait_arrivals(a, e1, 0, U, a.spin_master, a.sync_test == 1 ? 1ull : 0ull);
    // Every unit published its counts before it arrived, so the tables are
    // exact whenever all arrivals were seen; a time-out leaves them untouched.
    if (!late) build_receiver_tables(a, false, lds);
    if (tid == 0) {
        if (late) __hip_atomic_store(a.error_flags, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // A unit that gives up stores its give-up token and then sets bit 1;
        // with a full fence on both sides, either that token is seen by the
        // re-check below or its bit lands after the store of error_flags.
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
    }
    __syncthreads();
    int gave = 0;
    for (int64_t u = tid; u < U; u += kLayoutThreads)
        gave |= sync_load(a.sync + 1 + u) == sync_token(e1, (uint64_t)u, kTokGiveUp);
    if (__syncthreads_or(gave) && tid == 0)
        __hip_atomic_fetch_or(a.error_flags, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) sync_store(a.sync, e1);  // every unit read the epoch before it arrived
}

// The compact layout in one launch ([DET] Approach: a cooperative two-pass
// scan with a grid-wide exchange).  Grid (B + 1) x S: unit (b, s) counts its
// tokens per wave into LDS (kept for the slot pass), publishes the unit
// totals, arrives, waits for the other units of its source, then turns the
// earlier units' totals and its own per-wave counts into running bases and
// ranks its items; workgroup (B, 0) coordinates and builds the receiver
// tables, the rest of that column exits at once.  The host launches it only
// when the whole grid fits on the device at once.
__global__ void __launch_bounds__(kLayoutThreads) k_layout_fused(LayoutArgs a) {
    const Shape &sh = a.sh;
    const int b = blockIdx.x, s = blockIdx.y, B = a.g.blocks_per_src;
    const int w = threadIdx.x / kWave, tid = threadIdx.x;
    const int R = sh.R, E = sh.E;
    extern __shared__ int lds[];
    __shared__ uint64_t epoch_sh;
    __shared__ int wave_bad[kLayoutWaves];
    if (b == B) {
        if (s == 0) fused_coordinator(a, lds, &epoch_sh);
        return;
    }
    const int64_t me = (int64_t)s * B + b;
    int *cnt_d = lds;                        // [waves][R] per-wave counts, then running bases
    int *cnt_e = cnt_d + kLayoutWaves * R;   // [waves][E]
    int *base_d = cnt_e + kLayoutWaves * E;  // [R]   this unit's base per destination
    int *col = base_d + R + E;               // [R+E] per-source totals of this unit's share of columns

    int t0, t1;
    wave_range(a, b, w, t0, t1);
    const StepCtx c = make_ctx(sh.K);
    const bool single = t1 - t0 <= kBatch * c.tps;
    const int64_t *topk_src = a.topk_idx + (int64_t)s * sh.T * sh.K;
    int64_t first[kBatch] = {};
    if (single) load_batch(sh, topk_src, t0, t1, c, first);  // kept in registers for the slot pass
    if (tid == 0) epoch_sh = sync_load(a.sync);
    for (int i = tid; i < kLayoutWaves * (R + E) + R + E + (R + E); i += kLayoutThreads) lds[i] = 0;
    __syncthreads();

    // Pass 1: per-wave counts, then the unit totals for the other units.
    const bool bad = wave_count(sh, topk_src, t0, t1, cnt_d + w * R, cnt_e + w * E, true, c, first, single);
    if (lane_id() == 0) wave_bad[w] = bad ? 1 : 0;
    __syncthreads();
    for (int d = tid; d < R; d += kLayoutThreads) {
        int v = 0;
        for (int q = 0; q < kLayoutWaves; ++q) v += cnt_d[q * R + d];
        a.blk_cnt_rank[me * R + d] = v;
    }
    for (int e = tid; e < E; e += kLayoutThreads) {
        int v = 0;
        for (int q = 0; q < kLayoutWaves; ++q) v += cnt_e[q * E + e];
        a.blk_cnt_expert[me * E + e] = v;
    }
    if (tid == 0) {
        int any = 0;
        for (int q = 0; q < kLayoutWaves; ++q) any |= wave_bad[q];
        a.blk_flags[me] = any;
    }
    // Publish: after the barrier every wave's stores have reached this CU's
    // L2; one device-scope release makes them visible before the arrival.
    __syncthreads();
    const uint64_t e1 = epoch_sh + 1;
    if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        sync_store(a.sync + 1 + me, sync_token(e1, (uint64_t)me, kTokArrive));
    }
    const int64_t u0 = (int64_t)s * B;
    if (wait_arrivals(a, e1, u0, u0 + B, a.spin_unit, a.sync_test == 2 ? 1ull : 0ull)) {
        if (tid == 0) {
            sync_store(a.sync + 1 + me, sync_token(e1, (uint64_t)me, kTokGiveUp));
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
            __hip_atomic_fetch_or(a.error_flags, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }

    // Pass 2: this unit's base per destination (what the earlier units of the
    // source send there) and its share of the per-source totals.
    const int32_t *src_rank = a.blk_cnt_rank + (int64_t)s * B * R;
    ColumnLoads lb, lc;
    column_issue(lb, b, R, [&](int d, int64_t &stride) {
        stride = R;
        return src_rank + d;
    });
    const int ncol = b < R + E ? (R + E - b + B - 1) / B : 0;
    auto col_src = [&](int j, int64_t &stride) -> const int32_t * {
        const int cidx = b + j * B;
        if (cidx < R) {
            stride = R;
            return a.blk_cnt_rank + (int64_t)s * B * R + cidx;
        }
        stride = E;
        return a.blk_cnt_expert + (int64_t)s * B * E + (cidx - R);
    };
    const bool col_early = ncol <= kLayoutThreads;
    column_issue(lc, B, col_early ? ncol : 0, col_src);
    column_finish(lb, base_d);
    __syncthreads();
    wave_bases(cnt_d, R, base_d);
    __syncthreads();
    rank_items(a, false, s, t0, t1, c, first, single, cnt_d + w * R, cnt_e + w * E);
    if (col_early) column_finish(lc, col);
    else column_sums(B, ncol, col, col_src);
    __syncthreads();
    for (int j = tid; j < ncol; j += kLayoutThreads) {
        const int cidx = b + j * B;
        if (cidx < R) a.tokens_per_rank[(int64_t)s * R + cidx] = col[j];
        else a.tokens_per_expert[(int64_t)s * E + cidx - R] = col[j];
    }
}

// The layout of one small source by one workgroup of NW waves (wave w owns
// tokens [w*cw, (w+1)*cw), cw = ceil(T/NW)): the workgroup's own counts are
// the source's totals, so the receiver tables and the expert segment bases
// need no other workgroup.  Writes the tables to memory when `writer`, keeps
// the receive base of every destination in rbase[R] (LDS) when rbase is not
// null, and hands every item's slot (row base 0: one source) and expand row
// to on_item(item, slot, pos, own) -- own: the slot of the lane's owner (its
// own slot for an owner) -- in each wave's token order.  on_issued() runs
// right after the wave has issued its loads of the routing, so that loads it
// issues queue behind them.  LDS as single_lds_bytes.
template <int NW, bool EXPAND, typename OnIssued, typename OnItem>
__device__ __forceinline__ void layout_one_workgroup(const LayoutArgs &a, int *lds, bool writer, int *rbase,
                                                     OnIssued &&on_issued, OnItem &&on_item) {
    constexpr int NT = NW * kWave;
    const Shape &sh = a.sh;
    const int w = threadIdx.x / kWave, tid = threadIdx.x;
    const int R = sh.R, E = sh.E;
    int *cnt_d = lds;               // [NW][R] per-wave counts, then running bases
    int *cnt_e = cnt_d + NW * R;    // [NW][E]
    int *zero_d = cnt_e + NW * E;   // [R]    the base per destination: 0
    int *seg = zero_d + R;          // [E]    expand: expert segment bases
    int *part = seg + E;            // [NT]   totals per destination, then scan scratch
    int *flag = part + NT;          // [NW]

    const int cw = (sh.T + NW - 1) / NW;
    const int t0 = min(w * cw, sh.T), t1 = min(t0 + cw, sh.T);
    const StepCtx c = make_ctx(sh.K);
    const bool one_batch = t1 - t0 <= kBatch * c.tps;
    int64_t first[kBatch] = {};
    if (one_batch) load_batch(sh, a.topk_idx, t0, t1, c, first);
    on_issued();
    for (int i = tid; i < NW * (R + E) + R + E; i += NT) lds[i] = 0;
    __syncthreads();
    const bool bad = wave_count(sh, a.topk_idx, t0, t1, cnt_d + w * R, cnt_e + w * E, true, c, first, one_batch);
    if (lane_id() == 0) flag[w] = bad ? 1 : 0;
    __syncthreads();
    for (int d = tid; d < R; d += NT) {
        int tot = 0;
        for (int q = 0; q < NW; ++q) tot += cnt_d[q * R + d];
        if (writer) {
            a.tokens_per_rank[d] = tot;
            a.recv_psum[2 * d] = 0;
            a.recv_psum[2 * d + 1] = tot;
        }
        part[d] = tot;
    }
    for (int e = tid; e < E; e += NT) {
        int tot = 0;
        for (int q = 0; q < NW; ++q) tot += cnt_e[q * E + e];
        if (writer) a.tokens_per_expert[e] = tot;
        seg[e] = (tot + sh.A - 1) / sh.A * sh.A;
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int d = 0; d < R; ++d) {
            if (writer) a.recv_base[d] = run;
            if (rbase) rbase[d] = run;
            run += part[d];
        }
        if (writer) {
            a.recv_base[R] = run;
            int any = 0;
            for (int q = 0; q < NW; ++q) any |= flag[q];
            a.error_flags[0] = any ? 1 : 0;
        }
    }
    __syncthreads();
    if (EXPAND) {
        const int total = block_exclusive_scan<NT>(seg, E, part);
        if (writer) {
            for (int e = tid; e < E; e += NT) a.expert_base[e] = seg[e];
            if (tid == 0) a.expert_base[E] = total;
        }
    }
    wave_bases<NW>(cnt_d, R, zero_d);
    if (EXPAND) wave_bases<NW>(cnt_e, E, seg);
    __syncthreads();
    int *run_d = cnt_d + w * R, *run_e = cnt_e + w * E;
    walk_steps(sh, a.topk_idx, t0, t1, c, first, one_batch, EXPAND, [&](const Item &it) {
        const int rd = it.owner ? run_d[it.d] : 0;
        const int re = (EXPAND && it.valid) ? run_e[it.e] : 0;
        const int slot = it.owner ? rd + it.rank_d : -1;
        const int own = shfl(slot, it.owner_lane);
        if (it.in) on_item(it, slot, (EXPAND && it.valid) ? re + it.rank_e : -1, own);
        if (it.last_d) run_d[it.d] = rd + it.rank_d + 1;
        if (EXPAND && it.last_e) run_e[it.e] = re + it.rank_e + 1;
    });
}

// The whole layout in one workgroup of NW waves, for one small source, in one
// launch instead of two.
template <int NW, bool EXPAND>
__global__ void __launch_bounds__(NW * kWave) k_layout_single(LayoutArgs a) {
    extern __shared__ int lds[];
    const int K = a.sh.K;
    layout_one_workgroup<NW, EXPAND>(a, lds, true, nullptr, [] {}, [&](const Item &it, int slot, int pos, int own) {
        a.dst_slot[(int64_t)it.t * K + it.k] = slot;
        if (EXPAND) a.expand_pos[(int64_t)it.t * K + it.k] = pos;
        if (EXPAND && a.expand_row_src && pos >= 0) record_expand_row(a, 0, it, own, pos - it.rank_e);
    });
}

// ------------------------------------------ layout and dispatch, one launch
// The pages' dispatch replays the slots its prologue computed ([DET]
// Approach); for one small source (compact layout) both run in one launch.
// Every workgroup computes the whole layout of the source in LDS, as
// k_layout_single does (a few hundred items: cheaper than a second launch);
// workgroup 0 alone writes the tables to memory.  Then each workgroup
// dispatches its own NW tokens, one wave per token, as k_dispatch_fused does:
// the token's row and scales (loaded before the layout work, so their latency
// overlaps it) and its record go to the staging rows of its destinations and,
// from the same registers, to the compact receive rows the copy epilogue
// would fill from them.  The slots of the workgroup's tokens and the first
// receive row of each destination come from LDS.
template <int NW, int CPL>
__global__ void __launch_bounds__(NW * kWave) k_layout_dispatch_small(LayoutArgs a, DispatchArgs da) {
    constexpr int NT = NW * kWave;
    const Shape &sh = a.sh;
    const int w = threadIdx.x / kWave, tid = threadIdx.x, lane = lane_id();
    const int K = sh.K;
    const bool writer = blockIdx.x == 0;
    extern __shared__ int lds[];
    int *rbase = lds + single_lds_bytes(sh, NW) / sizeof(int);  // [R]     first receive row per destination
    int *slots = rbase + sh.R;                                    // [NW][K] slots of this workgroup's tokens

    // This workgroup's tokens, one per wave: the token's loads are issued
    // right behind the layout's own loads of the routing, so that the layout
    // does not wait for them.
    const int g0 = blockIdx.x * NW;
    const int g = g0 + w;
    const bool has_tok = g < sh.T;
    const int nchunks = sh.row_bytes / 16;
    u32x4 v[CPL];
    int e = -1, wbits = 0;
    float sf = 0.0f;
    auto load_token = [&] {
        if (!has_tok) return;
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
            const int c = q * kWave + lane;
            if (c < nchunks) v[q] = ld16<EP_SCATTER_NT_LOAD>(da.x + (int64_t)g * sh.row_bytes + (int64_t)c * 16);
        }
        if (lane < sh.sf_per_row) sf = da.x_sf[(int64_t)g * sh.sf_per_row + lane];
        if (lane < K) {
            const int64_t e64 = a.topk_idx[(int64_t)g * K + lane];
            e = (e64 >= 0 && e64 < sh.E) ? (int)e64 : -1;
            wbits = __float_as_int(da.topk_weights[(int64_t)g * K + lane]);
        }
    };
    for (int i = tid; i < NW * K; i += NT) slots[i] = -1;  // ordered by the layout's first barrier
    layout_one_workgroup<NW, false>(a, lds, writer, rbase, load_token, [&](const Item &it, int slot, int, int) {
        const int t = it.t, k = it.k;
        if (writer) a.dst_slot[(int64_t)t * K + k] = slot;
        if (t >= g0 && t < g0 + NW) slots[(t - g0) * K + k] = slot;
    });
    __syncthreads();
    if (!has_tok) return;

    // Dispatch of token g: its staging rows and receive rows, with records.
    const int slot = lane < K ? slots[w * K + lane] : -1;
    const uint64_t owners = ballot(lane < K && slot >= 0);
    int word0, wv_hi;
    record_words(sh, g, e, wbits, lane, word0, wv_hi);
    for (uint64_t m = owners; m; m &= m - 1) {
        const int k = __builtin_ctzll(m);
        const int d = rank_of(sh, read_lane(e, k));
        const int j = read_lane(slot, k);
        if ((unsigned)j >= (unsigned)sh.Nmax) continue;  // never true: j < T <= Nmax
        const int64_t i = (int64_t)rbase[d] + j;
        if (i >= da.recv_capacity_rows) continue;  // never true: the call checked the capacity
        token_rows<CPL>(da, d, 0, g, (int64_t)d * sh.Nmax + j, i, lane, v, sf, word0, wv_hi, e, wbits);
    }
}

#ifndef EP_SMALL_WAVES
#define EP_SMALL_WAVES 8
#endif
constexpr int kSmallWaves = EP_SMALL_WAVES;  // waves (tokens) per workgroup of k_layout_dispatch_small

size_t small_dispatch_lds_bytes(const Shape &sh) {
    return single_lds_bytes(sh, kSmallWaves) + sizeof(int) * ((size_t)sh.R + (size_t)kSmallWaves * sh.K);
}

size_t count_lds_bytes(const Shape &sh) {
    return sizeof(int) * ((size_t)kLayoutWaves * (sh.R + sh.E) + kLayoutWaves);
}
size_t slot_lds_bytes(const Shape &sh) {
    return sizeof(int) * ((size_t)kLayoutWaves * (sh.R + sh.E) + sh.R + sh.E + (sh.R + sh.E) + kLayoutThreads);
}

constexpr int kMaxDevices = 64;

// Workgroups of k_layout_fused with `lds` bytes of dynamic LDS that the
// current device holds at once (0 if unknown): resident workgroups per CU
// times the CUs, looked up once per (device, LDS size).
int64_t fused_capacity(size_t lds) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    static std::mutex mu;
    static int cus[kMaxDevices];
    static std::map<std::pair<int, size_t>, int64_t> cache;
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_pair(dev, lds);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    if (!cus[dev] && hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_layout_fused, kLayoutThreads, lds) != hipSuccess)
        return 0;
    return cache[key] = (int64_t)per_cu * cus[dev];
}

}  // namespace

bool layout_is_one_launch(const LayoutArgs &a) {
    if (a.sh.expand || a.g.single || !a.one_launch) return false;
    const int64_t grid = ((int64_t)a.g.blocks_per_src + 1) * a.sh.S;
    return grid <= fused_capacity(slot_lds_bytes(a.sh));
}

bool layout_dispatch_is_one_launch(const LayoutArgs &a, const DispatchArgs &da) {
    const Shape &sh = a.sh;
    return sh.S == 1 && !sh.expand && !sh.direct && sh.T > 0 &&
           (int64_t)sh.T * sh.K <= EP_LAYOUT_SINGLE_MAX_ITEMS && sh.row_bytes <= kWave * 16 &&
           sh.sf_per_row <= kWave &&
           small_dispatch_lds_bytes(sh) <= 65536 && da.recv_capacity_rows >= compact_rows_bound(sh);
}

hipError_t launch_layout_dispatch(const LayoutArgs &a, const DispatchArgs &da, hipStream_t stream) {
    const int blocks = (a.sh.T + kSmallWaves - 1) / kSmallWaves;
    hipLaunchKernelGGL((k_layout_dispatch_small<kSmallWaves, 1>), dim3(blocks), dim3(kSmallWaves * kWave),
                       small_dispatch_lds_bytes(a.sh), stream, a, da);
    return hipGetLastError();
}

hipError_t launch_layout(const LayoutArgs &a, hipStream_t stream) {
    if (layout_is_one_launch(a)) {
        hipLaunchKernelGGL(k_layout_fused, dim3(a.g.blocks_per_src + 1, a.sh.S), dim3(kLayoutThreads),
                           slot_lds_bytes(a.sh), stream, a);
        return hipGetLastError();
    }
    if (a.g.single) {
        const int nw = a.g.single;
        const size_t lds = single_lds_bytes(a.sh, nw);
        if (nw == 8 && a.sh.expand)
            hipLaunchKernelGGL((k_layout_single<8, true>), dim3(1), dim3(8 * kWave), lds, stream, a);
        else if (nw == 8)
            hipLaunchKernelGGL((k_layout_single<8, false>), dim3(1), dim3(8 * kWave), lds, stream, a);
        else if (a.sh.expand)
            hipLaunchKernelGGL((k_layout_single<16, true>), dim3(1), dim3(16 * kWave), lds, stream, a);
        else
            hipLaunchKernelGGL((k_layout_single<16, false>), dim3(1), dim3(16 * kWave), lds, stream, a);
        return hipGetLastError();
    }
    const dim3 grid(a.g.blocks_per_src, a.sh.S);
    hipLaunchKernelGGL(k_layout_count, grid, dim3(kLayoutThreads), count_lds_bytes(a.sh), stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (a.sh.expand) {
        hipLaunchKernelGGL(k_layout_expert_scan, dim3((a.sh.E + kScanCols - 1) / kScanCols), dim3(kScanThreads), 0,
                           stream, a);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    // One more column of workgroups: (B, 0) builds the receiver tables, the
    // rest of that column exits at once.
    const dim3 slot_grid(a.g.blocks_per_src + 1, a.sh.S);
    if (a.sh.expand)
        hipLaunchKernelGGL(k_layout_slot<true>, slot_grid, dim3(kLayoutThreads), slot_lds_bytes(a.sh), stream, a);
    else
        hipLaunchKernelGGL(k_layout_slot<false>, slot_grid, dim3(kLayoutThreads), slot_lds_bytes(a.sh), stream, a);
    return hipGetLastError();
}

// Layout scratch owned by the library, for ep_layout_no_alloc (callers that
// cannot allocate device memory).  Each GPU the library runs on holds its own
// copy until the process ends; host code never uses the array's name as an
// address (in host code it is only a stand-in for the symbol), only the device
// address hipGetSymbolAddress returns for the current device, looked up once
// per device and kept.  No word needs clearing: every count a layout reads
// was written earlier in the same layout, and the one-launch layout's
// exchange words are valid whatever they hold.
static __device__ __align__(256) uint8_t scratch[EP_NO_ALLOC_SCRATCH_BYTES];

hipError_t no_alloc_scratch(void **ptr) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    static std::mutex mu;
    static void *addr[kMaxDevices];
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace ep
