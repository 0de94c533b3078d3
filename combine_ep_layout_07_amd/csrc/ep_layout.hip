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
// item per SIMD lane, items in (t, k) order.  Equal destinations (or experts)
// inside a step are found with one ballot per key bit; the exclusive rank of
// an item among equal keys is a masked popcount (mbcnt), and the highest lane
// of each key group advances a per-wave running counter in LDS.  Nothing is
// decided by atomics, so the result never depends on scheduling.
//
//   pass 1 (k_layout_count): per-unit counts of owner lanes per destination
//     and of valid lanes per expert, plus an invalid-id flag, into scratch;
//   pass 2 (k_layout_slot): each unit reduces the counts of the units before
//     it (its exclusive base), recounts per wave for the wave bases, then
//     ranks every item and writes dst_slot (and expand_pos); the first unit
//     of each source writes that source's counts, unit (0,0) the receiver
//     tables (recv_psum, recv_base, expert_base, error_flags).
#include "ep_device.h"
#include "ep_kernels.h"

namespace ep {

constexpr int kLayoutThreads = 256;
constexpr int kLayoutWaves = kLayoutThreads / kWave;

LayoutGeom layout_geometry(const Shape &sh, int num_layout_cus) {
    LayoutGeom g;
    const int T = sh.T;
    int B = num_layout_cus > 0 ? (num_layout_cus + sh.S - 1) / sh.S : (T + 255) / 256;
    const int max_b = T > 4 ? (T + 3) / 4 : 1;  // at least 4 tokens (one per wave) per unit
    if (B < 1) B = 1;
    if (B > max_b) B = max_b;
    int chunk = T > 0 ? (T + B - 1) / B : 4;
    chunk = (chunk + 3) / 4 * 4;
    B = T > 0 ? (T + chunk - 1) / chunk : 1;
    g.blocks_per_src = B;
    g.chunk = chunk;
    return g;
}

uint64_t layout_scratch_bytes(const Shape &sh, const LayoutGeom &g) {
    const uint64_t units = (uint64_t)sh.S * g.blocks_per_src;
    return units * (uint64_t)(sh.R + sh.E + 1) * sizeof(int32_t);
}

namespace {

// Per-lane view of one step: which (token, lane) item this lane holds and how
// it ranks among the step's items with the same destination / expert.
struct Item {
    bool in, valid, invalid, owner;
    int t, k, d, e;
    int rank_d, cnt_d;  // owners only: exclusive rank / group size among owners of d
    bool last_d;        // highest owner lane of its destination group
    int rank_e, cnt_e;  // valid only: same among valid lanes of expert e
    bool last_e;
};

struct StepCtx {
    int lane, l_tok, l_k;
    bool used;          // lane holds an item slot in every step (l < tps*K)
    uint64_t seg;       // lanes of the same token
    int tps;            // tokens per step
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

__device__ __forceinline__ Item load_item(const Shape &sh, const int64_t *topk_src, int t_step, int t_end,
                                          const StepCtx &c, bool need_e) {
    Item it;
    it.t = t_step + c.l_tok;
    it.k = c.l_k;
    it.in = c.used && it.t < t_end;
    const int64_t e64 = it.in ? __builtin_nontemporal_load(topk_src + (int64_t)it.t * sh.K + c.l_k) : -1;
    it.invalid = it.in && e64 >= sh.E;
    it.valid = it.in && e64 >= 0 && e64 < sh.E;
    it.e = it.valid ? (int)e64 : 0;
    it.d = it.valid ? it.e / sh.El : 0;
    const uint64_t vmask = ballot(it.valid);
    const uint64_t peers_d = match_key((uint32_t)it.d, sh.bits_R, vmask);
    it.owner = it.valid && ((peers_d & c.seg & mask_lt(c.lane)) == 0);
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

// Count owner lanes per destination (and valid lanes per expert) over tokens
// [t0, t1) of one source into this wave's LDS rows; returns the invalid flag.
__device__ bool wave_count(const Shape &sh, const int64_t *topk_src, int t0, int t1, int *cnt_d, int *cnt_e,
                           bool need_e) {
    const StepCtx c = make_ctx(sh.K);
    bool bad = false;
    for (int ts = t0; ts < t1; ts += c.tps) {
        const Item it = load_item(sh, topk_src, ts, t1, c, need_e);
        if (it.last_d) cnt_d[it.d] += it.cnt_d;
        if (need_e && it.last_e) cnt_e[it.e] += it.cnt_e;
        bad |= it.invalid;
    }
    return ballot(bad) != 0;
}

// Exclusive scan of a[0..n) in LDS by the whole workgroup; returns the total.
__device__ int block_exclusive_scan(int *a, int n, int *part) {
    const int tid = threadIdx.x;
    const int per = (n + kLayoutThreads - 1) / kLayoutThreads;
    const int lo = min(tid * per, n), hi = min(lo + per, n);
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += a[i];
    part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < kLayoutThreads; off <<= 1) {
        const int v = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int run = part[tid] - sum;
    const int total = part[kLayoutThreads - 1];
    for (int i = lo; i < hi; ++i) {
        const int v = a[i];
        a[i] = run;
        run += v;
    }
    __syncthreads();
    return total;
}

__global__ void __launch_bounds__(kLayoutThreads) k_layout_count(LayoutArgs a) {
    const Shape &sh = a.sh;
    const int b = blockIdx.x, s = blockIdx.y, B = a.g.blocks_per_src;
    const int w = threadIdx.x / kWave, tid = threadIdx.x;
    extern __shared__ int lds[];
    int *cnt_d = lds;                               // [4][R]
    int *cnt_e = cnt_d + kLayoutWaves * sh.R;       // [4][E]
    int *flag = cnt_e + kLayoutWaves * sh.E;        // [4]
    for (int i = tid; i < kLayoutWaves * (sh.R + sh.E); i += kLayoutThreads) lds[i] = 0;
    __syncthreads();

    const int cw = a.g.chunk / kLayoutWaves;
    const int t0 = min(b * a.g.chunk + w * cw, sh.T), t1 = min(t0 + cw, sh.T);
    const int64_t *topk_src = a.topk_idx + (int64_t)s * sh.T * sh.K;
    const bool bad = wave_count(sh, topk_src, t0, t1, cnt_d + w * sh.R, cnt_e + w * sh.E, true);
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
    if (tid == 0) a.blk_flags[u] = flag[0] | flag[1] | flag[2] | flag[3];
}

__global__ void __launch_bounds__(kLayoutThreads) k_layout_slot(LayoutArgs a) {
    const Shape &sh = a.sh;
    const int b = blockIdx.x, s = blockIdx.y, B = a.g.blocks_per_src;
    const int w = threadIdx.x / kWave, tid = threadIdx.x;
    const int R = sh.R, E = sh.E, S = sh.S;
    const bool expand = sh.expand != 0;
    const int64_t U = (int64_t)S * B, me = (int64_t)s * B + b;

    extern __shared__ int lds[];
    int *cnt_d = lds;                          // [4][R] per-wave counts, then running bases
    int *cnt_e = cnt_d + kLayoutWaves * R;     // [4][E]
    int *base_d = cnt_e + kLayoutWaves * E;    // [R]   this unit's base per destination
    int *base_e = base_d + R;                  // [E+1] expert_base, then this unit's base per expert
    int *part = base_e + E + 1;                // [256] scan workspace
    for (int i = tid; i < kLayoutWaves * (R + E); i += kLayoutThreads) lds[i] = 0;

    // Unit base per destination: what the earlier units of this source send there.
    for (int d = tid; d < R; d += kLayoutThreads) {
        int v = 0;
        for (int q = 0; q < b; ++q) v += a.blk_cnt_rank[((int64_t)s * B + q) * R + d];
        base_d[d] = v;
    }
    if (expand) {
        // Expert segments ([E+1] bases, padded to A) and this unit's offset in
        // each: the valid lanes of every unit before it in (s, t) order.
        for (int e = tid; e < E; e += kLayoutThreads) {
            int tot = 0;
            for (int64_t q = 0; q < U; ++q) tot += a.blk_cnt_expert[q * E + e];
            base_e[e] = (tot + sh.A - 1) / sh.A * sh.A;
        }
        __syncthreads();
        const int total = block_exclusive_scan(base_e, E, part);
        if (tid == 0) base_e[E] = total;
        __syncthreads();
        if (me == 0)
            for (int e = tid; e <= E; e += kLayoutThreads) a.expert_base[e] = base_e[e];
        for (int e = tid; e < E; e += kLayoutThreads) {
            int pre = 0;
            for (int64_t q = 0; q < me; ++q) pre += a.blk_cnt_expert[q * E + e];
            base_e[e] += pre;
        }
    }
    __syncthreads();

    // Per-wave counts of this unit, then each wave's running base.
    const int cw = a.g.chunk / kLayoutWaves;
    const int t0 = min(b * a.g.chunk + w * cw, sh.T), t1 = min(t0 + cw, sh.T);
    const int64_t *topk_src = a.topk_idx + (int64_t)s * sh.T * sh.K;
    wave_count(sh, topk_src, t0, t1, cnt_d + w * R, cnt_e + w * E, expand);
    __syncthreads();
    for (int d = tid; d < R; d += kLayoutThreads) {
        int run = base_d[d];
        for (int q = 0; q < kLayoutWaves; ++q) {
            const int v = cnt_d[q * R + d];
            cnt_d[q * R + d] = run;
            run += v;
        }
    }
    if (expand) {
        for (int e = tid; e < E; e += kLayoutThreads) {
            int run = base_e[e];
            for (int q = 0; q < kLayoutWaves; ++q) {
                const int v = cnt_e[q * E + e];
                cnt_e[q * E + e] = run;
                run += v;
            }
        }
    }
    __syncthreads();

    // Ranking: every item of the wave's range gets its slot / expand row.
    {
        const StepCtx c = make_ctx(sh.K);
        int *run_d = cnt_d + w * R;
        int *run_e = cnt_e + w * E;
        const int32_t row_base = s * sh.Nmax;  // direct path: one Nmax-row region per source
        for (int ts = t0; ts < t1; ts += c.tps) {
            const Item it = load_item(sh, topk_src, ts, t1, c, expand);
            const int rd = it.owner ? run_d[it.d] : 0;
            const int re = (expand && it.valid) ? run_e[it.e] : 0;
            if (it.in) {
                const int64_t idx = ((int64_t)s * sh.T + it.t) * sh.K + it.k;
                a.dst_slot[idx] = it.owner ? row_base + rd + it.rank_d : -1;
                if (expand) a.expand_pos[idx] = it.valid ? re + it.rank_e : -1;
            }
            if (it.last_d) run_d[it.d] = rd + it.rank_d + 1;
            if (expand && it.last_e) run_e[it.e] = re + it.rank_e + 1;
        }
    }

    // Per-source counts (first unit of each source).
    if (b == 0) {
        for (int d = tid; d < R; d += kLayoutThreads) {
            int v = 0;
            for (int q = 0; q < B; ++q) v += a.blk_cnt_rank[((int64_t)s * B + q) * R + d];
            a.tokens_per_rank[(int64_t)s * R + d] = v;
        }
        for (int e = tid; e < E; e += kLayoutThreads) {
            int v = 0;
            for (int q = 0; q < B; ++q) v += a.blk_cnt_expert[((int64_t)s * B + q) * E + e];
            a.tokens_per_expert[(int64_t)s * E + e] = v;
        }
    }
    // Receiver tables (unit 0 only): recv_psum, recv_base, error flags.
    if (me == 0) {
        __syncthreads();
        int *tot_d = part;  // reuse: [R] totals per destination (R <= 64 < 256)
        for (int d = tid; d < R; d += kLayoutThreads) {
            int run = 0;
            for (int q = 0; q < S; ++q) {
                a.recv_psum[(int64_t)d * (S + 1) + q] = run;
                for (int bb = 0; bb < B; ++bb) run += a.blk_cnt_rank[((int64_t)q * B + bb) * R + d];
            }
            a.recv_psum[(int64_t)d * (S + 1) + S] = run;
            tot_d[d] = run;
        }
        int bad = 0;
        for (int64_t q = tid; q < U; q += kLayoutThreads) bad |= a.blk_flags[q];
        bad = ballot(bad != 0) != 0;
        __syncthreads();
        if (tid == 0) {
            int run = 0;
            for (int d = 0; d < R; ++d) {
                a.recv_base[d] = run;
                run += tot_d[d];
            }
            a.recv_base[R] = run;
        }
        __syncthreads();
        if (lane_id() == 0) part[w] = bad;
        __syncthreads();
        if (tid == 0) a.error_flags[0] = (part[0] | part[1] | part[2] | part[3]) ? 1 : 0;
    }
}

size_t count_lds_bytes(const Shape &sh) {
    return sizeof(int) * ((size_t)kLayoutWaves * (sh.R + sh.E) + kLayoutWaves);
}
size_t slot_lds_bytes(const Shape &sh) {
    return sizeof(int) * ((size_t)kLayoutWaves * (sh.R + sh.E) + sh.R + sh.E + 1 + kLayoutThreads);
}

}  // namespace

hipError_t launch_layout(const LayoutArgs &a, hipStream_t stream) {
    const dim3 grid(a.g.blocks_per_src, a.sh.S);
    hipLaunchKernelGGL(k_layout_count, grid, dim3(kLayoutThreads), count_lds_bytes(a.sh), stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_layout_slot, grid, dim3(kLayoutThreads), slot_lds_bytes(a.sh), stream, a);
    return hipGetLastError();
}

}  // namespace ep
