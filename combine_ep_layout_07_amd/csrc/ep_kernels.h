// ep_kernels.h -- launch arguments and launchers of the libep kernels.  Host
// code (ep_api.cpp) validates a configuration, fills these structs and calls
// the launchers; each launcher only enqueues on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

// Shape shared by all kernels (validated on the host).
struct Shape {
    int S, T, H, K, E, R, El, Nmax;
    int expand, A;
    int is_fp8;
    int row_bytes;   // bytes of one dispatched hidden row
    int sf_per_row;  // fp32 scales per row (fp8), else 0
    int meta_words;  // 1 + 2K
    int bits_R, bits_E;  // key widths for ballot matching of ranks / experts
    int direct;          // Direct Recv X: hidden rows go straight to recv_x
    int n_out, n_up;     // hybrid row form when n_out > 1: rank s = (s / n_up, s % n_up)
    uint32_t el_mul;     // floor(2^22 / El) + 1: e / El == (e * el_mul) >> 22 for 0 <= e < 1024
};

// Row base of source s: the source itself on the direct path, its scale-out
// index on the hybrid path.
__host__ __device__ inline int row_base(const Shape &sh, int s) { return sh.n_out > 1 ? s / sh.n_up : s; }

// Destination rank of a valid expert id e (0 <= e < E <= 1024), e / El, as a
// multiply and a shift: with m = floor(2^22 / El) + 1, e * m / 2^22 exceeds
// e / El by less than e / 2^22 < 2^-12, while the fraction of e / El is at most
// 1 - 1/El <= 1 - 2^-10, so the floor is exact for all 0 <= e < 1024 and
// El <= 1024, and e * m < 2^32.
__host__ __device__ inline int rank_of(const Shape &sh, int e) { return (int)(((uint32_t)e * sh.el_mul) >> 22); }

// Region (of Nmax rows) that source s fills in destination d's staging rows:
// d*S + s on the direct path; in the hybrid row form, segment = scale-up
// index, then the scale-out index inside the segment.
__host__ __device__ inline int64_t staging_region(const Shape &sh, int d, int s) {
    if (sh.n_out > 1) return ((int64_t)d * sh.n_up + s % sh.n_up) * sh.n_out + s / sh.n_up;
    return (int64_t)d * sh.S + s;
}

// (d, s) of a staging region: the inverse of staging_region (a destination's
// regions are the S consecutive ones from d*S; in the row form the remainder
// is (s % n_up) * n_out + s / n_up).
__host__ __device__ inline void staging_region_inverse(const Shape &sh, int64_t region, int &d, int &s) {
    d = (int)(region / sh.S);
    const int rem = (int)(region - (int64_t)d * sh.S);
    s = sh.n_out > 1 ? (rem % sh.n_out) * sh.n_up + rem / sh.n_out : rem;
}

// Layout pass geometry: B workgroups per source, each owning `chunk` tokens
// (split into equal wave ranges, one per wave of the workgroup).
struct LayoutGeom {
    int blocks_per_src;
    int chunk;
    int single;  // 0, or the waves (8 or 16) of the one-workgroup layout of a small single source
};

LayoutGeom layout_geometry(const Shape &sh, int num_layout_cus);
uint64_t layout_scratch_bytes(const Shape &sh, const LayoutGeom &g);

struct LayoutArgs {
    Shape sh;
    LayoutGeom g;
    const int64_t *topk_idx;
    int32_t *dst_slot, *tokens_per_rank, *tokens_per_expert, *recv_psum, *recv_base;
    int32_t *expert_base, *expand_pos, *error_flags;
    int32_t *recv_psum_scaleup;  // hybrid only
    int32_t *blk_cnt_rank;    // scratch [S*B][R]
    int32_t *blk_cnt_expert;  // scratch [S*B][E]
    int32_t *blk_flags;       // scratch [S*B]
    int32_t *blk_pre_expert;  // scratch [S*B][E], expand only: valid lanes of the earlier units per expert
    int32_t *cnt_expert;      // scratch [E], expand only: valid lanes per expert over all sources
    // One-launch layout (compact layout): the grid-wide exchange's words in
    // scratch, 8-byte aligned: [0] epoch, [1 + u] arrival word of unit u.
    // None of them needs initialising (see ep_layout.hip).
    uint64_t *sync;
    uint32_t spin_master, spin_unit;  // polls before the coordinator / a unit gives up
    int sync_test;                    // 0; 1 or 2 force a time-out (tests of the error path)
    int one_launch;                   // compact layout: one launch with a grid-wide exchange, where it fits
    // Expand layout with alignment 1 and a layout scratch: the expand index
    // (DispatchArgs::expand_row_src) at the scratch's head, written by the
    // slot pass; null otherwise.
    int64_t *expand_row_src;
};

// Words of the one-launch layout's exchange for `units` units.
constexpr uint64_t layout_sync_words(uint64_t units) { return 1 + units; }

struct DispatchArgs {
    Shape sh;
    const uint8_t *x;
    const float *x_sf;
    const int64_t *topk_idx;
    const float *topk_weights;
    const int32_t *dst_slot, *recv_psum, *recv_base, *tokens_per_expert, *expert_base, *expand_pos;
    uint8_t *staging_x;
    float *staging_sf;
    int32_t *staging_meta;
    uint8_t *recv_x;
    float *recv_sf;
    int32_t *recv_src_idx, *recv_topk_idx;
    float *recv_topk_weights;
    int64_t recv_capacity_rows;
    int slices;  // scatter: column slices per token (set by the launcher)
    // Compact staging path with a layout scratch: the staging row of every
    // filled receive row, written by the scatter, read by the copy epilogue;
    // null otherwise (the epilogue then locates rows in the receiver tables).
    int64_t *recv_row_src;
    // Expand layout with alignment 1 and a layout scratch: per expand row r <
    // expert_base[E], the staging row it copies with its top-k lane in the top
    // byte (row | lane << 56), written by the layout's slot pass (which knows
    // each lane's expand row and its owner's slot), read by the expand
    // epilogue.  Null otherwise.
    int64_t *expand_row_src;
};

// Compact rows of a layout at most (the compact receive-row index's length).
__host__ __device__ inline int64_t compact_rows_bound(const Shape &sh) {
    return (int64_t)sh.S * sh.T * (sh.K < sh.R ? sh.K : sh.R);
}
// Expand rows of a layout at most, padding included.
__host__ __device__ inline int64_t expand_rows_bound(const Shape &sh) {
    return (int64_t)sh.S * sh.T * sh.K + (int64_t)sh.E * (sh.A - 1);
}

struct CombineArgs {
    Shape sh;
    const int64_t *topk_idx;
    const float *topk_weights;
    const int32_t *dst_slot, *recv_psum, *recv_base, *expand_pos;
    const uint16_t *y;
    const uint16_t *bias0, *bias1;  // optional [S][T][H] rows added before rounding
    uint16_t *out;
    int64_t y_rows;  // rows of y (the receive capacity)
    int slices;      // column slices per token (set by the launcher)
};

hipError_t launch_layout(const LayoutArgs &a, hipStream_t stream);
// Whether launch_layout takes the one-launch form for these arguments on the
// current device.
bool layout_is_one_launch(const LayoutArgs &a);
// Device address of the library's own layout scratch (EP_NO_ALLOC_SCRATCH_BYTES
// bytes) on the current device; looked up once per device, thread-safe.
hipError_t no_alloc_scratch(void **ptr);
hipError_t launch_scatter(const DispatchArgs &a, hipStream_t stream);
// Both dispatch phases of a small compact-layout problem in one launch.
bool dispatch_is_one_launch(const DispatchArgs &a);
hipError_t launch_dispatch_fused(const DispatchArgs &a, hipStream_t stream);
// Layout and both dispatch phases of one small source in one launch.
bool layout_dispatch_is_one_launch(const LayoutArgs &a, const DispatchArgs &da);
hipError_t launch_layout_dispatch(const LayoutArgs &a, const DispatchArgs &da, hipStream_t stream);
hipError_t launch_epilogue(const DispatchArgs &a, hipStream_t stream);
hipError_t launch_combine(const CombineArgs &a, hipStream_t stream);

}  // namespace ep
