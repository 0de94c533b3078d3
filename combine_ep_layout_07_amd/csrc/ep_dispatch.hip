// ep_dispatch.hip -- scatter and copy epilogue of the deterministic dispatch.
//
// DeepEP v2 "Kernel-side deterministic dispatch for the non-expand layout"
// (PR #753), section Direct vs hybrid dispatch: on the direct path the
// receive buffer of a destination holds one Nmax-row region per source rank,
// and senders replay the slots the layout computed.  "Add experimental direct
// recv_x dispatch path" (PR #690), section Background: dispatch first writes
// rows into that staging area and a copy epilogue then materialises the
// compact recv_x plus the metadata and top-k tensors.
//
// Here all source and destination ranks are partitions of one GPU's HBM, so a
// send is a local store.  The kernels are HBM streams of 16-byte chunks: a
// wavefront moves one row at a time, lane l taking chunks c = l + 64*i, the
// whole row (or a CPL-chunk slice of it) loaded into VGPRs before any store, so
// every lane has CPL independent 16-byte loads in flight.
//   k_scatter        one wave per token (or per piece of its row: 1 KiB for
//                    staging rows of more than 1 GiB, 2 KiB for Direct Recv X
//                    from 512 MiB of rows), its row stored to every owner's
//                    staging row or, with Direct Recv X, receive row (plus
//                    scales and the record);
//   k_scatter_pf     the same with each wave pipelining several tokens (next
//                    row loaded before the current stores): Direct Recv X
//                    below 512 MiB of rows and staging scatters of at most
//                    1 GiB of rows;
//   k_epilogue_indexed  compact epilogue, one wave per 2 KiB piece of a
//                    receive row, its source found through the receive-row
//                    index the scatter records in the layout's scratch;
//   k_epilogue_pf    the compact epilogue without that index, pipelined the
//                    same way as k_scatter_pf over receive rows (k_epilogue
//                    for rows wider than one pass);
//   k_epilogue_meta  Direct Recv X: scales and metadata only, one thread per
//                    (row, item);
//   k_epilogue_expand_indexed  the per-expert layout with alignment 1, in
//                    expand-row order through the index the layout records;
//   k_epilogue_expand_pieces, k_expand_padding   the per-expert layout
//                    otherwise (in 2 KiB pieces of staging rows, then the
//                    padding rows).
// On the hybrid path the same kernels address a destination's staging rows in
// row form (segment = the source's scale-up index, then its scale-out index),
// through staging_region.
#include <algorithm>

#include "ep_device.h"
#include "ep_kernels.h"
#include "ep_rows.h"

namespace ep {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

#ifndef EP_DIRECT_NT_STORE
#define EP_DIRECT_NT_STORE 1  // Direct Recv X rows: written once, read by the next stage at the earliest
#endif
#ifndef EP_SCATTER_SLICES
#define EP_SCATTER_SLICES 1  // column slices of a token's row, each a separate work unit
#endif
// Column slices of a compact receive row, each a separate work unit, and the
// epilogue's grid cap.  Measured on MI355X at T=4096, H=7168: one whole row
// per wave in one pass is fastest (2, 4 and 7 slices cost 2%, 9% and 19% more
// time, two passes of half a row 3%, two rows per wave 1%).  The grid is not
// capped, so each wave takes one receive row: in back-to-back steps at
// T=4096, H=7168 bf16, 2048 / 4096 / 6144 workgroups (3.3 / 1.6 / 1.1 rows
// per wave, pipelined) gave 296 / 291.5 / 286 us per step and one row per
// wave 283 us; at T=8192, H=4096 239.5 -> 232.8 us; fp8 rows 1% slower.
#ifndef EP_EPILOGUE_SLICES
#define EP_EPILOGUE_SLICES 1
#endif
#ifndef EP_EPILOGUE_BLOCKS
#define EP_EPILOGUE_BLOCKS (1 << 20)
#endif
#ifndef EP_EXPAND_PULL_NT_LOAD
#define EP_EXPAND_PULL_NT_LOAD 0  // the expand epilogue re-reads staging rows: through the caches
#endif
#ifndef EP_INDEXED_CPW
#define EP_INDEXED_CPW 2  // chunks per lane of a k_epilogue_indexed piece
#endif
constexpr int kIndexedCpw = EP_INDEXED_CPW;
// The indexed copy epilogue's grid covers this many sixths of the pieces of
// the receive capacity (and the expand epilogue's without the index of its
// staging-row bound); waves past the end take further pieces (grid-stride).
// The host cannot know how many rows are filled, and each wave launched past
// them still costs a launch.  Measured on MI355X, whole steps (filled /
// capacity rows): 8192 tokens H = 4096 Zipf (35731 / 65536) 231-233 ->
// 225-226 us, the same as a grid sized to the filled rows exactly; 4096
// tokens H = 7168 (26758 / 32768) 278.5-279.7 -> 276.3-276.6 us; fp8 188-189
// -> 187-188 us; with half the capacity (3 sixths) 225 / 278-280 / 186 us.
#ifndef EP_INDEXED_GRID_SIXTHS
#define EP_INDEXED_GRID_SIXTHS 4
#endif
// Waves per workgroup of k_epilogue_indexed.  Measured on MI355X, whole
// steps against 4 waves: 2 waves 1 us faster at 4096 tokens H = 7168 bf16,
// 2-6 us slower at 8192 tokens H = 4096 and 3-5 us slower in fp8; 1 wave up
// to 15 us slower; 8 / 16 waves 5 / 20 us slower at 4096 tokens.
#ifndef EP_INDEXED_WAVES
#define EP_INDEXED_WAVES 4
#endif
// The staging scatter, with no grid-stride cap (measured at 16 x 2048 tokens:
// 708 us capped at 2048 workgroups, 674 us uncapped), takes one of two forms.
// When its staging rows come to at most EP_SCATTER_PIPELINE_MAX_BYTES: the
// pipelined kernel with two tokens per wave (2 waves per SIMD instead of 4).
// Measured on MI355X, steps with consecutive steps on alternating buffers,
// against one token per wave: 4096 tokens H = 7168 bf16 283 -> 277.5-278.5
// us per step (scatter 73 -> 70 us), the same in fp8 187 -> 185 us, 8192
// tokens H = 4096 Zipf 235 -> 234 us, but 16 x 2048 tokens (3 GB of staging
// rows) 2626 -> 2644 us (scatter 676 -> 706 us).  Above that bound: one wave
// per 1 KiB piece of a token's row (column slices of 64 chunks), which loads
// its piece and the token's ids at once and stores the piece to each owner:
// short-lived waves keep the write stream closer to a fill's rate (a plain
// fill of 3.3 GB in 1 KiB per wave ran at 6.9 TB/s, in 14 KiB per wave at
// 5.5).  16 x 2048 tokens: scatter 678 -> 606 us (2 KiB pieces 668 us); at
// 4096 tokens the pieces lose to the pipelined kernel (70.5 -> 73.3 us).  The
// pieces' staging stores are non-temporal: rows that large leave the
// Infinity Cache full of dirty lines that the copy epilogue then pays to
// write back (16 x 2048 tokens: scatter 600 -> 607 us, epilogue 1193 -> 1132
// us, step 2515 -> 2461 us), while below 1 GiB the cache absorbs the staging
// writes and the epilogue reads them from it (non-temporal: 14% slower).
#ifndef EP_SCATTER_BLOCKS
#define EP_SCATTER_BLOCKS (1 << 20)
#endif
// Tokens per wave of the pipelined staging scatter.  Measured on MI355X
// (scatter inside the step): 4096 tokens H = 7168 bf16 2 / 3 / 4 per wave
// 70 / 84-85 / 71 us, fp8 41 / 50 / 49 us, 8192 tokens H = 4096 60 / 67 / 63 us
// (3 per wave leaves the device's wave slots part empty).
#ifndef EP_SCATTER_TOKENS_PER_WAVE
#define EP_SCATTER_TOKENS_PER_WAVE 2
#endif
#ifndef EP_SCATTER_PIPELINE_MAX_BYTES
#define EP_SCATTER_PIPELINE_MAX_BYTES (1ll << 30)
#endif
// Direct Recv X writes its rows straight to the receive rows (non-temporal),
// pipelined (k_scatter_pf) below EP_DIRECT_PIECES_MIN_BYTES of rows (bound
// S*T*min(K,R) rows) and in 2 KiB pieces per wave from there (k_scatter<2>, column
// slices of 128 chunks).  Measured on MI355X, whole steps at H = 7168 bf16,
// top-8 of 256 on 16 ranks: 8192 tokens 349 -> 311 us, 16384 675 -> 658 us,
// 32768 1329 -> 1307 us, 4096 (470 MB) 164.2 -> 164.8 us; 8192 tokens of
// H = 4096 rows (537 MB) 141.7 -> 136.4 us; 1 KiB pieces lost at every size.
#ifndef EP_DIRECT_PIECES_MIN_BYTES
#define EP_DIRECT_PIECES_MIN_BYTES (1ll << 29)
#endif
// Compact-layout problems of at most this many tokens (all sources) with
// rows of at most EP_FUSED_DISPATCH_MAX_ROW bytes dispatch in one launch
// (k_dispatch_fused) when both phases are asked for.  Measured on MI355X:
// 128 tokens of 512-byte rows (top-4 of 32 on 8 ranks) 20.1 -> 17.7 us per
// step; with 14 KiB rows the token-serial copy loses (128 tokens: 31.9 ->
// 46.8 us per step, 2048 tokens: 142.8 -> 152.1 us).
#ifndef EP_FUSED_DISPATCH_MAX_TOKENS
#define EP_FUSED_DISPATCH_MAX_TOKENS 512
#endif
#ifndef EP_FUSED_DISPATCH_MAX_ROW
#define EP_FUSED_DISPATCH_MAX_ROW 1024
#endif
#ifndef EP_DIRECT_INFLIGHT_BYTES
#define EP_DIRECT_INFLIGHT_BYTES 7340032
#endif
#ifndef EP_COPY_BLOCKS
#define EP_COPY_BLOCKS 2048
#endif
// Chunks per lane of a k_epilogue_expand_pieces piece.  Measured on MI355X
// at 4096 tokens, H = 7168 bf16, expert alignment 128, whole steps: 1 / 2 / 4
// KiB pieces 409 / 380 / 389 us; one wave per staging row 384 us.
#ifndef EP_EXPAND_PIECE_CPW
#define EP_EXPAND_PIECE_CPW 2
#endif

// ----------------------------------------------------------------- scatter
// One wave per token (s, t): load the row once, store it to row
// j = slot - row_base(s)*Nmax of source s's region in the staging rows of
// every owner lane's destination d (with Direct Recv X, used here only for
// rows wider than one pass, to the compact receive row recv_base[d] +
// recv_psum[d][s] + j), with the fp8 scales and the metadata record.
template <int CPL, bool NT_STAGING = EP_SCATTER_NT_STORE != 0>
__global__ void __launch_bounds__(kThreads) k_scatter(DispatchArgs a) {
    const Shape &sh = a.sh;
    const int lane = lane_id();
    const int64_t n_tok = (int64_t)sh.S * sh.T;
    const int nchunks = sh.row_bytes / 16;
    // Work unit = (token, column slice of its row); slice 0 also writes the
    // scales and the metadata.
    const int slices = a.slices;
    const int cps = ((nchunks + slices - 1) / slices + kWave - 1) / kWave * kWave;  // chunks per slice
    const int64_t n_units = n_tok * slices;
    const int64_t wave0 = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t unit = wave0; unit < n_units; unit += nwaves) {
        const int64_t g = unit / slices;
        const int slice = (int)(unit - g * slices);
        const int c_lo = slice * cps, c_hi = min(c_lo + cps, nchunks);
        const int s = (int)(g / sh.T), t = (int)(g - (int64_t)s * sh.T);
        int e = -1, slot = -1, wbits = 0;
        if (lane < sh.K) {
            const int64_t e64 = a.topk_idx[g * sh.K + lane];
            e = (e64 >= 0 && e64 < sh.E) ? (int)e64 : -1;
            slot = a.dst_slot[g * sh.K + lane];
            wbits = __float_as_int(a.topk_weights[g * sh.K + lane]);
        }
        const uint64_t owners = ballot(lane < sh.K && slot >= 0);
        // Direct Recv X (and the receive-row index, slice 0): every owner
        // lane fetches its destination's compact base recv_base[d] +
        // recv_psum[d][s] at once (one gather, not a dependent scalar load
        // per owner row).
        int recv_row0 = 0;
        if ((sh.direct || (a.recv_row_src && slice == 0)) && lane < sh.K && slot >= 0) {
            const int d = rank_of(sh, e);
            recv_row0 = a.recv_base[d] + a.recv_psum[(int64_t)d * (sh.S + 1) + s];
            if (!sh.direct) record_recv_row(a, s, e, slot, recv_row0);
        }
        const uint8_t *src = a.x + g * sh.row_bytes;
        for (int c0 = c_lo; c0 < c_hi; c0 += CPL * kWave) {
            u32x4 v[CPL];
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = c0 + i * kWave + lane;
                if (c < c_hi) v[i] = ld16<EP_SCATTER_NT_LOAD>(src + (int64_t)c * 16);
            }
            for (uint64_t m = owners; m; m &= m - 1) {
                const int k = __builtin_ctzll(m);
                const int d = rank_of(sh, read_lane(e, k));
                const int j = read_lane(slot, k) - row_base(sh, s) * sh.Nmax;
                if ((unsigned)j >= (unsigned)sh.Nmax) continue;  // never true for a layout of this topk_idx
                if (sh.direct) {
                    // Direct Recv X: the compact receive row of (d, s, j).
                    const int64_t i = (int64_t)read_lane(recv_row0, k) + j;
                    if (i >= a.recv_capacity_rows) continue;
                    uint8_t *dst = a.recv_x + i * sh.row_bytes;
#pragma unroll
                    for (int q = 0; q < CPL; ++q) {
                        const int c = c0 + q * kWave + lane;
                        if (c < c_hi) st16<EP_DIRECT_NT_STORE>(dst + (int64_t)c * 16, v[q]);
                    }
                } else {
                    uint8_t *dst = a.staging_x + (staging_region(sh, d, s) * sh.Nmax + j) * sh.row_bytes;
#pragma unroll
                    for (int q = 0; q < CPL; ++q) {
                        const int c = c0 + q * kWave + lane;
                        if (c < c_hi) st16<NT_STAGING>(dst + (int64_t)c * 16, v[q]);
                    }
                }
            }
        }
        if (slice == 0) store_records(a, g, s, t, e, slot, wbits, owners, lane);
    }
}

// ------------------------------------------- Direct Recv X scatter, pipelined
// The stores of one token (whole row in one pass): rows, scales and metadata.
template <int CPL>
__device__ __forceinline__ void scatter_token(const DispatchArgs &a, int64_t g, int e, int slot, int wbits,
                                              const u32x4 (&v)[CPL], int lane) {
    const Shape &sh = a.sh;
    const int nchunks = sh.row_bytes / 16;
    const int s = (int)(g / sh.T), t = (int)(g - (int64_t)s * sh.T);
    const uint64_t owners = ballot(lane < sh.K && slot >= 0);
    int recv_row0 = 0;
    if ((sh.direct || a.recv_row_src) && lane < sh.K && slot >= 0) {
        const int d = rank_of(sh, e);
        recv_row0 = a.recv_base[d] + a.recv_psum[(int64_t)d * (sh.S + 1) + s];
        if (!sh.direct) record_recv_row(a, s, e, slot, recv_row0);
    }
    for (uint64_t m = owners; m; m &= m - 1) {
        const int k = __builtin_ctzll(m);
        const int d = rank_of(sh, read_lane(e, k));
        const int j = read_lane(slot, k) - row_base(sh, s) * sh.Nmax;
        if ((unsigned)j >= (unsigned)sh.Nmax) continue;
        if (sh.direct) {
            const int64_t i = (int64_t)read_lane(recv_row0, k) + j;
            if (i >= a.recv_capacity_rows) continue;
            uint8_t *dst = a.recv_x + i * sh.row_bytes;
#pragma unroll
            for (int q = 0; q < CPL; ++q) {
                const int c = q * kWave + lane;
                if (c < nchunks) st16<EP_DIRECT_NT_STORE>(dst + (int64_t)c * 16, v[q]);
            }
        } else {
            uint8_t *dst = a.staging_x + (staging_region(sh, d, s) * sh.Nmax + j) * sh.row_bytes;
#pragma unroll
            for (int q = 0; q < CPL; ++q) {
                const int c = q * kWave + lane;
                if (c < nchunks) st16<EP_SCATTER_NT_STORE>(dst + (int64_t)c * 16, v[q]);
            }
        }
    }
    store_records(a, g, s, t, e, slot, wbits, owners, lane);
}

// Software-pipelined scatter: each wave takes tokens g, g + nwaves, ... and
// loads the next token's ids, slots, weights and row before storing the
// current one, so its reads overlap its writes.  For Direct Recv X the grid is
// sized so that the resident waves hold about EP_DIRECT_INFLIGHT_BYTES of rows
// (measured on MI355X, Direct Recv X steps at T=4096, H=7168: 175 -> 166 us;
// fp8 and H=4096 rows 1-2% faster: with the receive rows written
// non-temporally straight to HBM, fewer waves that overlap their own reads
// and writes beat one wave per token); the staging scatter uses it with two
// tokens per wave when its rows come to at most EP_SCATTER_PIPELINE_MAX_BYTES
// (see there).  Needs the whole row in one pass (64 * CPL chunks).
template <int CPL>
__global__ void __launch_bounds__(kThreads) k_scatter_pf(DispatchArgs a) {
    const Shape &sh = a.sh;
    const int lane = lane_id();
    const int64_t n_tok = (int64_t)sh.S * sh.T;
    const int nchunks = sh.row_bytes / 16;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    int64_t g = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    if (g >= n_tok) return;
    auto fetch = [&](int64_t gg, int &e_, int &slot_, int &w_, u32x4 (&vv)[CPL]) {
        e_ = -1;
        slot_ = -1;
        w_ = 0;
        if (lane < sh.K) {
            const int64_t e64 = a.topk_idx[gg * sh.K + lane];
            e_ = (e64 >= 0 && e64 < sh.E) ? (int)e64 : -1;
            slot_ = a.dst_slot[gg * sh.K + lane];
            w_ = __float_as_int(a.topk_weights[gg * sh.K + lane]);
        }
        const uint8_t *src = a.x + gg * sh.row_bytes;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = i * kWave + lane;
            if (c < nchunks) vv[i] = ld16<EP_SCATTER_NT_LOAD>(src + (int64_t)c * 16);
        }
    };
    int e, slot, wbits;
    u32x4 v[CPL];
    fetch(g, e, slot, wbits, v);
    while (true) {
        const int64_t gn = g + nwaves;
        const bool more = gn < n_tok;
        int en = -1, sn = -1, wn = 0;
        u32x4 vn[CPL];
        if (more) fetch(gn, en, sn, wn, vn);
        scatter_token<CPL>(a, g, e, slot, wbits, v, lane);
        if (!more) break;
        g = gn;
        e = en;
        slot = sn;
        wbits = wn;
        for (int i = 0; i < CPL; ++i) v[i] = vn[i];
    }
}

// Which (destination, source, row) a compact receive row i comes from:
// d = last d with recv_base[d] <= i, s = last s with recv_psum[d][s] <= i -
// recv_base[d], j the rest.  Both tables are non-decreasing, so each index is
// the count of entries <= the key minus one: one ballot per 64 entries.
__device__ __forceinline__ void locate_row(const int32_t *recv_base, const int32_t *recv_psum, int R, int S,
                                           int i, int lane, int &d, int &s, int &j) {
    int cnt = 0;
    for (int l0 = 0; l0 < R; l0 += kWave) {
        const int l = l0 + lane;
        cnt += popc(ballot(l < R && recv_base[l] <= i));
    }
    d = cnt - 1;
    s = 0;
    j = -1;         // callers skip rows with j outside [0, Nmax)
    if (d < 0) return;  // only for tables that no layout wrote (recv_base[0] is 0)
    const int off = i - recv_base[d];
    const int32_t *ps = recv_psum + (int64_t)d * (S + 1);
    cnt = 0;
    for (int l0 = 0; l0 < S; l0 += kWave) {
        const int l = l0 + lane;
        cnt += popc(ballot(l < S && ps[l] <= off));
    }
    s = cnt - 1;
    if (s < 0) return;  // likewise (recv_psum[d][0] is 0)
    j = off - ps[s];
}

// Receiver tables in LDS: recv_base [R+1] then recv_psum [R][S+1].
__device__ __forceinline__ const int32_t *stage_tables(const DispatchArgs &a, int32_t *lds, bool fits) {
    if (!fits) return nullptr;
    const int nb = a.sh.R + 1, np = a.sh.R * (a.sh.S + 1);
    for (int i = threadIdx.x; i < nb + np; i += kThreads) lds[i] = i < nb ? a.recv_base[i] : a.recv_psum[i - nb];
    __syncthreads();
    return lds;
}

// ------------------------------------------------- compact copy epilogue

// ------------------------------------------ small dispatch, one launch
// Scatter and copy epilogue of a small compact-layout problem in one launch:
// below a few hundred tokens the fixed cost of a second launch exceeds the
// copy itself, and what remains is a chain of memory latencies.  Each wave
// takes one token and writes, for each destination d, its staging row and
// record (as k_scatter) and the compact receive row recv_base[d] +
// recv_psum[d][s] + j that the copy epilogue would fill from that staging row
// -- the same bytes, here from the registers that hold the token, so no
// staging row is read back.  Whole rows in one pass, scales <= 64 per row.
template <int CPL>
__global__ void __launch_bounds__(kThreads) k_dispatch_fused(DispatchArgs a) {
    const Shape &sh = a.sh;
    const int lane = lane_id();
    const int64_t n_tok = (int64_t)sh.S * sh.T;
    const int nchunks = sh.row_bytes / 16;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t g = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; g < n_tok; g += nwaves) {
        const int s = (int)(g / sh.T), t = (int)(g - (int64_t)s * sh.T);
        int e = -1, slot = -1, wbits = 0;
        if (lane < sh.K) {
            const int64_t e64 = a.topk_idx[g * sh.K + lane];
            e = (e64 >= 0 && e64 < sh.E) ? (int)e64 : -1;
            slot = a.dst_slot[g * sh.K + lane];
            wbits = __float_as_int(a.topk_weights[g * sh.K + lane]);
        }
        // Lane l < R fetches source s's first compact receive row in
        // destination l with the ids, so that no load waits for a rank.
        int base_l = 0;
        if (lane < sh.R) base_l = a.recv_base[lane] + a.recv_psum[(int64_t)lane * (sh.S + 1) + s];
        const uint8_t *src = a.x + g * sh.row_bytes;
        u32x4 v[CPL];
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
            const int c = q * kWave + lane;
            if (c < nchunks) v[q] = ld16<EP_SCATTER_NT_LOAD>(src + (int64_t)c * 16);
        }
        const uint64_t owners = ballot(lane < sh.K && slot >= 0);
        const float sf = lane < sh.sf_per_row ? a.x_sf[g * sh.sf_per_row + lane] : 0.0f;
        const int recv_row0 = shfl(base_l, e >= 0 ? rank_of(sh, e) : 0);
        int word0, wv_hi;
        record_words(sh, t, e, wbits, lane, word0, wv_hi);
        for (uint64_t m = owners; m; m &= m - 1) {
            const int k = __builtin_ctzll(m);
            const int d = rank_of(sh, read_lane(e, k));
            const int j = read_lane(slot, k) - row_base(sh, s) * sh.Nmax;
            if ((unsigned)j >= (unsigned)sh.Nmax) continue;  // never true for a layout of this topk_idx
            const int64_t i = (int64_t)read_lane(recv_row0, k) + j;
            if (i >= a.recv_capacity_rows) continue;  // never true: the call checked the capacity
            token_rows<CPL>(a, d, s, t, staging_region(sh, d, s) * sh.Nmax + j, i, lane, v, sf, word0, wv_hi, e,
                            wbits);
        }
    }
}

// One wave per filled receive row i < recv_base[R], in order (consecutive
// waves write consecutive recv_x rows); each finds its (d, s, j) from the
// tables.  Walking the staging rows instead, latest written first so as to
// meet them in the Infinity Cache, measured slower on MI355X.
template <int CPL>
__global__ void __launch_bounds__(kThreads) k_epilogue(DispatchArgs a, int tables_in_lds) {
    const Shape &sh = a.sh;
    extern __shared__ int32_t lds_tab[];
    const int32_t *tab = stage_tables(a, lds_tab, tables_in_lds != 0);
    const int lane = lane_id();
    const int n_rows = (int)min((int64_t)a.recv_base[sh.R], a.recv_capacity_rows);
    const int wave0 = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    const int nwaves = gridDim.x * kWavesPerBlock;
    const int32_t *rbase = tab ? tab : a.recv_base;
    const int32_t *rpsum = tab ? tab + sh.R + 1 : a.recv_psum;
    const int nchunks = sh.row_bytes / 16;
    const int slices = a.slices;
    const int cps = ((nchunks + slices - 1) / slices + kWave - 1) / kWave * kWave;  // chunks per slice
    const int64_t n_units = (int64_t)n_rows * slices;
    for (int64_t u = wave0; u < n_units; u += nwaves) {
        const int i = (int)(u / slices), slice = (int)(u - (int64_t)i * slices);
        int d, s, j;
        locate_row(rbase, rpsum, sh.R, sh.S, i, lane, d, s, j);
        if ((unsigned)j >= (unsigned)sh.Nmax) continue;  // never true for tables of one layout
        epilogue_row<CPL>(a, d, s, j, i, lane, slice * cps, min(slice * cps + cps, nchunks));
    }
}

// Compact epilogue when a row fits one pass (64 * CPL chunks): each wave
// takes receive rows i, i + nwaves, ... and loads the next row before storing
// the current one, so its reads overlap its writes.  With the default grid
// (one wave per receive row) the loop does not iterate; capped at 2048
// workgroups it took the epilogue from 143 to 139 us at T=4096, H=7168.
template <int CPL>
__global__ void __launch_bounds__(kThreads) k_epilogue_pf(DispatchArgs a, int tables_in_lds) {
    const Shape &sh = a.sh;
    extern __shared__ int32_t lds_tab[];
    const int32_t *tab = stage_tables(a, lds_tab, tables_in_lds != 0);
    const int32_t *rbase = tab ? tab : a.recv_base;
    const int32_t *rpsum = tab ? tab + sh.R + 1 : a.recv_psum;
    const int lane = lane_id();
    const int n_rows = (int)min((int64_t)a.recv_base[sh.R], a.recv_capacity_rows);
    const int nchunks = sh.row_bytes / 16;
    const int nwaves = gridDim.x * kWavesPerBlock;
    int i = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    if (i >= n_rows) return;
    auto fetch = [&](int ii, int &d_, int &s_, int &j_, u32x4 (&vv)[CPL]) {
        locate_row(rbase, rpsum, sh.R, sh.S, ii, lane, d_, s_, j_);
        if ((unsigned)j_ >= (unsigned)sh.Nmax) return;  // never true for tables of one layout
        const uint8_t *src = a.staging_x + (staging_region(sh, d_, s_) * sh.Nmax + j_) * sh.row_bytes;
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
            const int c = q * kWave + lane;
            if (c < nchunks) vv[q] = ld16<EP_EPILOGUE_NT_LOAD>(src + (int64_t)c * 16);
        }
    };
    int d, s, j;
    u32x4 v[CPL];
    fetch(i, d, s, j, v);
    while (true) {
        const bool more = nwaves < n_rows - i;  // i + nwaves < n_rows, without forming a sum past 2^31
        const int in = more ? i + nwaves : i;
        int dn = 0, sn = 0, jn = -1;
        u32x4 vn[CPL];
        if (more) fetch(in, dn, sn, jn, vn);
        if ((unsigned)j < (unsigned)sh.Nmax) {
            uint8_t *dst = a.recv_x + (int64_t)i * sh.row_bytes;
#pragma unroll
            for (int q = 0; q < CPL; ++q) {
                const int c = q * kWave + lane;
                if (c < nchunks) st16<EP_EPILOGUE_NT_STORE>(dst + (int64_t)c * 16, v[q]);
            }
            epilogue_row<CPL>(a, d, s, j, i, lane, 0, 0);  // scales and metadata only
        }
        if (!more) break;
        i = in;
        d = dn;
        s = sn;
        j = jn;
        for (int q = 0; q < CPL; ++q) v[q] = vn[q];
    }
}

// Last index q in [0, n) with tab[q] <= key, for a non-decreasing table whose
// first entry is <= key.
__device__ __forceinline__ int last_le(const int32_t *tab, int n, int key) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tab[mid] <= key) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Compact copy epilogue with the receive-row index (the staging path when the
// layout's scratch holds the index the scatter recorded): a wave per piece
// of CPW chunks per lane (2 KiB at CPW = 2) of receive row i, which loads the
// row's staging index, then its piece, and stores it; piece 0 also moves the
// scales and the metadata.  Short-lived waves with one dependent load ahead of
// the copy; the grid covers two thirds of the capacity's pieces
// (EP_INDEXED_GRID_SIXTHS), and a wave takes a further piece when the filled
// rows reach past it.  Measured on MI355X: 4096 tokens H = 7168 bf16, epilogue 129 ->
// 125 us inside the step (134 -> 123 us back to back); 8192 tokens H = 4096
// 106 -> 101 us; fp8 63 -> 62 us.  1 / 4 KiB pieces: 140 / 138 us at 4096
// tokens.  Without the index, pieces that first search the tables were far
// slower (1 KiB: 199 us; 2 KiB with the tables in LDS 128 us, 4 KiB 137 us).
template <int CPW, int NW = kWavesPerBlock>
__global__ void __launch_bounds__(NW * kWave) k_epilogue_indexed(DispatchArgs a) {
    const Shape &sh = a.sh;
    const int lane = lane_id();
    const int nchunks = sh.row_bytes / 16;
    const int P = (nchunks + CPW * kWave - 1) / (CPW * kWave);
    const int64_t n_units = min(min((int64_t)a.recv_base[sh.R], a.recv_capacity_rows), compact_rows_bound(sh)) * P;
    const int64_t n_staging = (int64_t)sh.R * sh.S * sh.Nmax;
    const int64_t nwaves = (int64_t)gridDim.x * NW;
    for (int64_t u = (int64_t)blockIdx.x * NW + threadIdx.x / kWave; u < n_units; u += nwaves) {
        const int64_t i = u / P;
        const int p = (int)(u - i * P);
        const int64_t row = a.recv_row_src[i];
        if (row < 0 || row >= n_staging) continue;  // never true after the scatter of this layout
        u32x4 v[CPW];
#pragma unroll
        for (int q = 0; q < CPW; ++q) {
            const int c = (p * CPW + q) * kWave + lane;
            if (c < nchunks) v[q] = ld16<EP_EPILOGUE_NT_LOAD>(a.staging_x + row * sh.row_bytes + (int64_t)c * 16);
        }
#pragma unroll
        for (int q = 0; q < CPW; ++q) {
            const int c = (p * CPW + q) * kWave + lane;
            if (c < nchunks) st16<EP_EPILOGUE_NT_STORE>(a.recv_x + i * sh.row_bytes + (int64_t)c * 16, v[q]);
        }
        if (p == 0) {
            const int64_t region = row / sh.Nmax;
            int d, s;
            staging_region_inverse(sh, region, d, s);
            epilogue_row<1>(a, d, s, (int)(row - region * sh.Nmax), (int)i, lane, 0, 0);  // scales and metadata
        }
    }
}

// Expand epilogue with the expand index (the staging path with expert
// alignment 1 when the layout's scratch holds it: every expand row is a lane
// row; the layout's slot pass writes the index): expand rows in order, one
// wave per piece of CPW chunks per lane (2 KiB at CPW = 2) of expand row r,
// which loads r's index entry (its staging row and top-k lane), then its piece
// of that staging row, and stores it; piece 0 also writes the row's scales,
// source index and the lane's weight.  The
// writes become one sequential stream; a staging row that feeds several
// expand rows (1.23 on average at K = 8 of 256 experts on 16 ranks) is read
// once per row, through the caches (cached loads: the repeat reads find
// some of it there).  Measured on MI355X at 16 x 2048 tokens, H = 7168 bf16,
// against the one-wave-per-staging-row kernel: epilogue 1235 -> 1198 us in
// the step, 1235 -> 1135 us back to back; non-temporal loads 1209 / 1147 us;
// pieces of 1 / 4 / 7 / 14 KiB: 1285 / 1305 / 1341 / 1430 us in the step.
// At 4096 tokens: 150 -> 142 us back to back.  A trial with alignment 128
// (half the rows padding, marked in the index by the padding kernel run
// first) measured 206 -> 210 us and the step 0.388 -> 0.419 ms, so padded
// layouts keep the other kernel and have no index.
template <int CPW>
__global__ void __launch_bounds__(kThreads) k_epilogue_expand_indexed(DispatchArgs a) {
    const Shape &sh = a.sh;
    const int lane = lane_id();
    const int nchunks = sh.row_bytes / 16;
    const int P = (nchunks + CPW * kWave - 1) / (CPW * kWave);
    const int64_t n_units = min(min((int64_t)a.expert_base[sh.E], a.recv_capacity_rows), expand_rows_bound(sh)) * P;
    const int64_t n_staging = (int64_t)sh.R * sh.S * sh.Nmax;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t u = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; u < n_units; u += nwaves) {
        const int64_t r = u / P;
        const int p = (int)(u - r * P);
        const int64_t code = a.expand_row_src[r];
        const int64_t row = code & ((1ll << 56) - 1);
        const int k = (int)(code >> 56);
        if (code < 0 || row >= n_staging || k >= sh.K) continue;  // never true after the scatter of this layout
        u32x4 v[CPW];
#pragma unroll
        for (int q = 0; q < CPW; ++q) {
            const int c = (p * CPW + q) * kWave + lane;
            if (c < nchunks) v[q] = ld16<EP_EXPAND_PULL_NT_LOAD>(a.staging_x + row * sh.row_bytes + (int64_t)c * 16);
        }
#pragma unroll
        for (int q = 0; q < CPW; ++q) {
            const int c = (p * CPW + q) * kWave + lane;
            if (c < nchunks) st16<EP_EPILOGUE_NT_STORE>(a.recv_x + r * sh.row_bytes + (int64_t)c * 16, v[q]);
        }
        if (p != 0) continue;
        int d, s;
        staging_region_inverse(sh, row / sh.Nmax, d, s);
        const int32_t *meta = a.staging_meta + row * sh.meta_words;
        for (int q = lane; q < sh.sf_per_row; q += kWave)
            a.recv_sf[r * sh.sf_per_row + q] = a.staging_sf[row * sh.sf_per_row + q];
        if (lane == 0) {
            a.recv_src_idx[r] = s * sh.T + meta[0];
            a.recv_topk_weights[r] = __int_as_float(meta[1 + sh.K + k]);
        }
    }
}

// Metadata-only epilogue (Direct Recv X: the hidden rows are already in
// place).  One thread per item (i, c) of a filled receive row i: c < K is
// top-k lane c (c = 0 also writes the source index); each further item copies
// sf_vec scales (4 = one 16-byte chunk when rows and buffers allow, else 1).
__global__ void __launch_bounds__(kThreads) k_epilogue_meta(DispatchArgs a, int tables_in_lds, int sf_vec) {
    const Shape &sh = a.sh;
    extern __shared__ int32_t lds_tab[];
    const int32_t *tab = stage_tables(a, lds_tab, tables_in_lds != 0);
    const int32_t *rbase = tab ? tab : a.recv_base;
    const int32_t *rpsum = tab ? tab + sh.R + 1 : a.recv_psum;
    const int n_rows = (int)min((int64_t)a.recv_base[sh.R], a.recv_capacity_rows);
    const int W = sh.K + sh.sf_per_row / sf_vec;
    const int64_t n_items = (int64_t)n_rows * W;
    for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < n_items; g += (int64_t)gridDim.x * kThreads) {
        const int i = (int)(g / W), c = (int)(g - (int64_t)i * W);
        const int d = last_le(rbase, sh.R + 1, i);
        const int32_t *ps = rpsum + (int64_t)d * (sh.S + 1);
        const int s = last_le(ps, sh.S + 1, i - rbase[d]);
        const int j = i - rbase[d] - ps[s];
        if ((unsigned)j >= (unsigned)sh.Nmax) continue;  // never true for tables of one layout
        const int64_t row = staging_region(sh, d, s) * sh.Nmax + j;
        const int32_t *meta = a.staging_meta + row * sh.meta_words;
        if (c < sh.K) {
            if (c == 0) a.recv_src_idx[i] = s * sh.T + meta[0];
            const int e = meta[1 + c];
            const bool on_d = (unsigned)e < (unsigned)sh.E && rank_of(sh, e) == d;
            a.recv_topk_idx[(int64_t)i * sh.K + c] = on_d ? e - d * sh.El : -1;
            a.recv_topk_weights[(int64_t)i * sh.K + c] = on_d ? __int_as_float(meta[1 + sh.K + c]) : 0.0f;
        } else if (sf_vec == 4) {
            const int q = (c - sh.K) * 4;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(a.staging_sf + row * sh.sf_per_row + q);
            *reinterpret_cast<u32x4 *>(a.recv_sf + (int64_t)i * sh.sf_per_row + q) = v;
        } else {
            a.recv_sf[(int64_t)i * sh.sf_per_row + c - sh.K] = a.staging_sf[row * sh.sf_per_row + c - sh.K];
        }
    }
}

// -------------------------------------------------- expand copy epilogue
// Without the expand index: one wave per piece of CPW chunks per lane (2 KiB
// at CPW = 2) of filled staging row i (compact receive-row order), which finds
// (d, s, j) in the receiver tables (staged in LDS), loads its piece of the
// staging row together with the row's record, then the expand rows of the
// token's lanes on d, and stores the piece to each (one per lane, duplicates
// included); piece 0 also writes the rows' scales, source index and the
// lanes' weights.  Used for expert alignment > 1, or without a layout scratch.
template <int CPW>
__global__ void __launch_bounds__(kThreads) k_epilogue_expand_pieces(DispatchArgs a, int tables_in_lds) {
    const Shape &sh = a.sh;
    extern __shared__ int32_t lds_tab[];
    const int32_t *tab = stage_tables(a, lds_tab, tables_in_lds != 0);
    const int32_t *rbase = tab ? tab : a.recv_base;
    const int32_t *rpsum = tab ? tab + sh.R + 1 : a.recv_psum;
    const int lane = lane_id();
    const int nchunks = sh.row_bytes / 16;
    const int P = (nchunks + CPW * kWave - 1) / (CPW * kWave);
    const int64_t n_units = min((int64_t)rbase[sh.R], compact_rows_bound(sh)) * P;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t u = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; u < n_units; u += nwaves) {
        const int i = (int)(u / P);  // < S*T*min(K,R) <= 2^31 - 1
        const int p = (int)(u - (int64_t)i * P);
        int d, s, j;
        locate_row(rbase, rpsum, sh.R, sh.S, i, lane, d, s, j);
        if ((unsigned)j >= (unsigned)sh.Nmax) continue;  // never true for tables of one layout
        const int64_t row = staging_region(sh, d, s) * sh.Nmax + j;
        u32x4 v[CPW];
#pragma unroll
        for (int q = 0; q < CPW; ++q) {
            const int c = (p * CPW + q) * kWave + lane;
            if (c < nchunks) v[q] = ld16<EP_EPILOGUE_NT_LOAD>(a.staging_x + row * sh.row_bytes + (int64_t)c * 16);
        }
        const int32_t *meta = a.staging_meta + row * sh.meta_words;
        const int t = meta[0];
        const int e = lane < sh.K ? meta[1 + lane] : -1;
        if ((unsigned)t >= (unsigned)sh.T) continue;  // never true for staging rows the scatter wrote
        int pos = -1, wbits = 0;
        if (lane < sh.K && (unsigned)e < (unsigned)sh.E && rank_of(sh, e) == d) {
            pos = a.expand_pos[((int64_t)s * sh.T + t) * sh.K + lane];
            wbits = meta[1 + sh.K + lane];
        }
        const uint64_t lanes_on_d = ballot(pos >= 0);
        for (uint64_t m = lanes_on_d; m; m &= m - 1) {
            const int r = read_lane(pos, __builtin_ctzll(m));
            if ((uint64_t)r >= (uint64_t)a.recv_capacity_rows) continue;
            uint8_t *dst = a.recv_x + (int64_t)r * sh.row_bytes;
#pragma unroll
            for (int q = 0; q < CPW; ++q) {
                const int c = (p * CPW + q) * kWave + lane;
                if (c < nchunks) st16<EP_EPILOGUE_NT_STORE>(dst + (int64_t)c * 16, v[q]);
            }
        }
        if (p != 0) continue;
        for (uint64_t m = lanes_on_d; m; m &= m - 1) {
            const int k = __builtin_ctzll(m);
            const int r = read_lane(pos, k);
            if ((uint64_t)r >= (uint64_t)a.recv_capacity_rows) continue;
            for (int q = lane; q < sh.sf_per_row; q += kWave)
                a.recv_sf[(int64_t)r * sh.sf_per_row + q] = a.staging_sf[row * sh.sf_per_row + q];
            if (lane == k) {
                a.recv_src_idx[r] = s * sh.T + t;
                a.recv_topk_weights[r] = __int_as_float(wbits);
            }
        }
    }
}

// Padding rows of each expert segment (alignment A > 1): zero row and
// scales, source index -1, weight +0.  Workgroup (e, y) takes rows r0 + y,
// r0 + y + gridDim.y, ... of expert e's padding (at most A - 1 rows).
__global__ void __launch_bounds__(kThreads) k_expand_padding(DispatchArgs a) {
    const Shape &sh = a.sh;
    const int e = blockIdx.x;
    int cnt = 0;
    for (int s = 0; s < sh.S; ++s) cnt += a.tokens_per_expert[(int64_t)s * sh.E + e];
    const int r0 = a.expert_base[e] + cnt;
    const int r1 = (int)min((int64_t)a.expert_base[e + 1], a.recv_capacity_rows);
    const int nchunks = sh.row_bytes / 16;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int64_t r = (int64_t)r0 + blockIdx.y; r < r1; r += gridDim.y) {  // 64-bit: r1 may approach 2^31
        uint8_t *dst = a.recv_x + (int64_t)r * sh.row_bytes;
        for (int c = threadIdx.x; c < nchunks; c += kThreads) st16<false>(dst + (int64_t)c * 16, zero);
        for (int q = threadIdx.x; q < sh.sf_per_row; q += kThreads) a.recv_sf[(int64_t)r * sh.sf_per_row + q] = 0.0f;
        if (threadIdx.x == 0) {
            a.recv_src_idx[r] = -1;
            a.recv_topk_weights[r] = 0.0f;
        }
    }
}

int chunks_per_lane(const Shape &sh) {
    const int nchunks = sh.row_bytes / 16;
    int slices = EP_SCATTER_SLICES < 1 ? 1 : EP_SCATTER_SLICES;
    if (slices > (nchunks + kWave - 1) / kWave) slices = (nchunks + kWave - 1) / kWave;
    const int cps = ((nchunks + slices - 1) / slices + kWave - 1) / kWave * kWave;
    return cps / kWave;
}
int epilogue_slices(const Shape &sh) {
    const int nchunks = sh.row_bytes / 16;
    int slices = sh.expand ? 1 : (EP_EPILOGUE_SLICES < 1 ? 1 : EP_EPILOGUE_SLICES);
    if (slices > (nchunks + kWave - 1) / kWave) slices = (nchunks + kWave - 1) / kWave;
    return slices;
}
int epilogue_chunks_per_lane(const Shape &sh) {
    const int nchunks = sh.row_bytes / 16, slices = epilogue_slices(sh);
    return (((nchunks + slices - 1) / slices + kWave - 1) / kWave * kWave) / kWave;
}

constexpr int kMaxCpl = 16;  // 16-byte chunks per lane of the widest instantiation

template <template <int> class Launcher, typename... Args>
hipError_t dispatch_cpl(int need, Args &&...args) {
    if (need <= 1) return Launcher<1>::run(args...);
    if (need <= 2) return Launcher<2>::run(args...);
    if (need <= 4) return Launcher<4>::run(args...);
    if (need <= 7) return Launcher<7>::run(args...);
    if (need <= 8) return Launcher<8>::run(args...);
    if (need <= 14) return Launcher<14>::run(args...);
    return Launcher<kMaxCpl>::run(args...);
}

int grid_for(int64_t work_waves, int max_blocks = EP_COPY_BLOCKS) {
    // Enough waves to fill 256 CUs several times over; extra work is strided.
    int64_t blocks = (work_waves + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks > max_blocks) blocks = max_blocks;
    if (blocks < 1) blocks = 1;
    return (int)blocks;
}

template <int CPL>
struct ScatterL {
    static hipError_t run(const DispatchArgs &args, hipStream_t st) {
        DispatchArgs a = args;
        const int nchunks = a.sh.row_bytes / 16;
        a.slices = EP_SCATTER_SLICES < 1 ? 1 : EP_SCATTER_SLICES;
        if (a.slices > (nchunks + kWave - 1) / kWave) a.slices = (nchunks + kWave - 1) / kWave;
        const int64_t units = (int64_t)a.sh.S * a.sh.T * a.slices;
        if (a.sh.direct && a.slices == 1 && nchunks <= CPL * kWave) {
            // about EP_DIRECT_INFLIGHT_BYTES of rows held by the resident waves
            int64_t blocks = ((int64_t)EP_DIRECT_INFLIGHT_BYTES + (int64_t)a.sh.row_bytes * kWavesPerBlock - 1) /
                             ((int64_t)a.sh.row_bytes * kWavesPerBlock);
            blocks = blocks < 1 ? 1 : (blocks > EP_COPY_BLOCKS ? EP_COPY_BLOCKS : blocks);
            hipLaunchKernelGGL(k_scatter_pf<CPL>, dim3(grid_for(units, (int)blocks)), dim3(kThreads), 0, st, a);
            return hipGetLastError();
        }
        // Staging rows of at most EP_SCATTER_PIPELINE_MAX_BYTES in all (an
        // upper bound, S*T*min(K,R) rows): the pipelined kernel, two tokens
        // per wave.
        const int64_t bound = (int64_t)a.sh.S * a.sh.T * (a.sh.K < a.sh.R ? a.sh.K : a.sh.R) * a.sh.row_bytes;
        if (a.slices == 1 && nchunks <= CPL * kWave && bound <= (int64_t)EP_SCATTER_PIPELINE_MAX_BYTES) {
            hipLaunchKernelGGL(k_scatter_pf<CPL>,
                               dim3(grid_for((units + EP_SCATTER_TOKENS_PER_WAVE - 1) / EP_SCATTER_TOKENS_PER_WAVE,
                                             EP_SCATTER_BLOCKS)),
                               dim3(kThreads), 0, st, a);
            return hipGetLastError();
        }
        hipLaunchKernelGGL(k_scatter<CPL>, dim3(grid_for(units, EP_SCATTER_BLOCKS)), dim3(kThreads), 0, st, a);
        return hipGetLastError();
    }
};

template <int CPL>
struct EpilogueL {
    static hipError_t run(const DispatchArgs &args, hipStream_t st) {
        DispatchArgs a = args;
        a.slices = epilogue_slices(a.sh);
        const size_t tab = sizeof(int32_t) * ((size_t)a.sh.R + 1 + (size_t)a.sh.R * (a.sh.S + 1));
        const bool fits = tab <= 32768;
        const int64_t rows = a.sh.expand ? (int64_t)a.sh.S * a.sh.T * (a.sh.K < a.sh.R ? a.sh.K : a.sh.R)
                                         : a.recv_capacity_rows;
        const int64_t pieces = (a.sh.row_bytes / 16 + kIndexedCpw * kWave - 1) / (kIndexedCpw * kWave);
        if (a.sh.expand && a.expand_row_src)
            hipLaunchKernelGGL(k_epilogue_expand_indexed<kIndexedCpw>,
                               dim3(grid_for(a.recv_capacity_rows * pieces, EP_EPILOGUE_BLOCKS)), dim3(kThreads), 0,
                               st, a);
        else if (a.sh.expand) {
            constexpr int cpw = EP_EXPAND_PIECE_CPW;
            const int64_t xp = (a.sh.row_bytes / 16 + cpw * kWave - 1) / (cpw * kWave);
            hipLaunchKernelGGL(k_epilogue_expand_pieces<cpw>,
                               dim3(grid_for((rows * xp * EP_INDEXED_GRID_SIXTHS + 5) / 6, EP_EPILOGUE_BLOCKS)),
                               dim3(kThreads), fits ? tab : 0, st, a, (int)fits);
        }
        else if (a.recv_row_src) {
            const int64_t units = (rows * pieces * EP_INDEXED_GRID_SIXTHS + 5) / 6;
            constexpr int nw = EP_INDEXED_WAVES;
            const int64_t blocks = std::min<int64_t>(std::max<int64_t>((units + nw - 1) / nw, 1), EP_EPILOGUE_BLOCKS);
            hipLaunchKernelGGL((k_epilogue_indexed<kIndexedCpw, nw>), dim3((int)blocks), dim3(nw * kWave), 0, st, a);
        } else if (a.slices == 1 && a.sh.row_bytes / 16 <= CPL * kWave)
            hipLaunchKernelGGL(k_epilogue_pf<CPL>, dim3(grid_for(rows, EP_EPILOGUE_BLOCKS)), dim3(kThreads),
                               fits ? tab : 0, st, a, (int)fits);
        else
            hipLaunchKernelGGL(k_epilogue<CPL>, dim3(grid_for(rows * a.slices, EP_EPILOGUE_BLOCKS)), dim3(kThreads),
                               fits ? tab : 0, st, a,
                               (int)fits);
        return hipGetLastError();
    }
};

template <int CPL>
struct FusedL {
    static hipError_t run(const DispatchArgs &a, hipStream_t st) {
        const int64_t tokens = (int64_t)a.sh.S * a.sh.T;
        hipLaunchKernelGGL(k_dispatch_fused<CPL>, dim3(grid_for(tokens, EP_SCATTER_BLOCKS)), dim3(kThreads), 0, st, a);
        return hipGetLastError();
    }
};

}  // namespace

bool dispatch_is_one_launch(const DispatchArgs &a) {
    const int64_t tokens = (int64_t)a.sh.S * a.sh.T;
    return !a.sh.expand && !a.sh.direct && tokens > 0 && tokens <= EP_FUSED_DISPATCH_MAX_TOKENS &&
           a.sh.row_bytes <= EP_FUSED_DISPATCH_MAX_ROW && a.sh.row_bytes <= kWave * 16 * kMaxCpl &&
           a.sh.sf_per_row <= kWave;
}

hipError_t launch_dispatch_fused(const DispatchArgs &a, hipStream_t stream) {
    return dispatch_cpl<FusedL>((a.sh.row_bytes / 16 + kWave - 1) / kWave, a, stream);  // whole rows
}

hipError_t launch_scatter(const DispatchArgs &a, hipStream_t stream) {
    if ((int64_t)a.sh.S * a.sh.T == 0) return hipSuccess;
    const int nchunks = a.sh.row_bytes / 16;
    const int64_t bound = (int64_t)a.sh.S * a.sh.T * (a.sh.K < a.sh.R ? a.sh.K : a.sh.R) * a.sh.row_bytes;
    if (a.sh.direct && EP_SCATTER_SLICES == 1 && bound >= (int64_t)EP_DIRECT_PIECES_MIN_BYTES) {
        DispatchArgs b = a;
        b.slices = (nchunks + 2 * kWave - 1) / (2 * kWave);  // 2 KiB pieces
        hipLaunchKernelGGL(k_scatter<2>, dim3(grid_for((int64_t)a.sh.S * a.sh.T * b.slices, EP_SCATTER_BLOCKS)),
                           dim3(kThreads), 0, stream, b);
        return hipGetLastError();
    }
    if (!a.sh.direct && EP_SCATTER_SLICES == 1 && bound > (int64_t)EP_SCATTER_PIPELINE_MAX_BYTES) {
        DispatchArgs b = a;
        b.slices = (nchunks + kWave - 1) / kWave;  // 1 KiB pieces
        hipLaunchKernelGGL((k_scatter<1, true>), dim3(grid_for((int64_t)a.sh.S * a.sh.T * b.slices, EP_SCATTER_BLOCKS)),
                           dim3(kThreads), 0, stream, b);
        return hipGetLastError();
    }
    return dispatch_cpl<ScatterL>(chunks_per_lane(a.sh), a, stream);
}

hipError_t launch_epilogue(const DispatchArgs &a, hipStream_t stream) {
    hipError_t err = hipSuccess;
    if ((int64_t)a.sh.S * a.sh.T > 0) {
        if (a.sh.direct) {
            const size_t tab = sizeof(int32_t) * ((size_t)a.sh.R + 1 + (size_t)a.sh.R * (a.sh.S + 1));
            const bool fits = tab <= 32768;
            // Scales move as 16-byte chunks when every row and both buffers are 16-byte aligned.
            const bool vec = a.sh.sf_per_row % 4 == 0 && ((uintptr_t)a.staging_sf % 16) == 0 &&
                             ((uintptr_t)a.recv_sf % 16) == 0;
            const int sf_vec = vec ? 4 : 1;
            const int64_t items = a.recv_capacity_rows * (a.sh.K + a.sh.sf_per_row / sf_vec);
            int64_t blocks = (items + kThreads - 1) / kThreads;
            blocks = blocks < 1 ? 1 : (blocks > 4 * EP_COPY_BLOCKS ? 4 * EP_COPY_BLOCKS : blocks);
            hipLaunchKernelGGL(k_epilogue_meta, dim3((int)blocks), dim3(kThreads), fits ? tab : 0, stream, a,
                               (int)fits, sf_vec);
            err = hipGetLastError();
        } else {
            err = dispatch_cpl<EpilogueL>(epilogue_chunks_per_lane(a.sh), a, stream);
        }
    }
    if (err != hipSuccess) return err;
    if (a.sh.expand && a.sh.A > 1) {
        const int split = a.sh.A - 1 < 16 ? a.sh.A - 1 : 16;  // workgroups per expert
        hipLaunchKernelGGL(k_expand_padding, dim3(a.sh.E, split), dim3(kThreads), 0, stream, a);
        err = hipGetLastError();
    }
    return err;
}

}  // namespace ep
