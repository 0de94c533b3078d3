/*
 * ep.h -- C ABI of libep: deterministic MoE expert-parallel dispatch layout,
 * dispatch (scatter + copy epilogue) and combine on one GPU's share of the
 * work, as HIP kernels for CDNA4 (gfx950).
 *
 * Sources (DeepEP v2 pages):
 *   [DET] "DeepEP v2: Kernel-side deterministic dispatch for the non-expand
 *         layout" (PR #753): sections Motivation, Approach, Direct vs hybrid
 *         dispatch, Compatibility, New API.
 *   [DRX] "DeepEP v2: Add experimental direct recv_x dispatch path" (PR #690):
 *         sections Background, Direct Recv X design, Implementation, and the
 *         review's buffer-size and guardrail comments.
 *   [UNO] "Add unordered hybrid kernels for transports without ordered
 *         delivery" (PR #732): section Changes (combine reduce epilogue).
 *
 * Model.  S source partitions ("source ranks") each hold T tokens; every token
 * routes to K experts out of E, and expert e lives on logical rank e / El,
 * El = E / R.  All S sources and all R destinations are partitions of the one
 * GPU's HBM: a "send" is a local store, and stream order replaces the pages'
 * signals and release atomics.
 *
 * Conventions for every call:
 *   - pointers named *_dev are device pointers the caller allocated (for
 *     example with torch.empty(..., device="cuda")); the library never
 *     allocates or frees, and keeps nothing between calls but the per-GPU
 *     array of ep_layout_no_alloc and cached device properties;
 *   - all arrays are dense row-major; rows of x, staging and recv are 16-byte
 *     aligned (the base pointers must be 16-byte aligned, and the row size in
 *     bytes is a multiple of 16);
 *   - `stream` is a hipStream_t (NULL = the default stream); calls only
 *     enqueue work on it and never synchronise;
 *   - argument errors are detected on the host before anything is enqueued
 *     and return a negative ep_status; a failed launch returns EP_ERR_HIP;
 *   - data errors found on the device (a top-k id >= E) set bit 0 of
 *     *error_flags and the lane is then treated as masked (id < 0); bit 1
 *     reports a timed-out one-launch layout (EP_FLAG_LAYOUT_ONE_LAUNCH);
 *   - calls on different streams with disjoint buffers may run concurrently.
 */
#ifndef EP_H
#define EP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum ep_status {
    EP_OK = 0,
    EP_ERR_INVALID_ARG = -1, /* a size, dtype or pointer is not acceptable    */
    EP_ERR_CAPACITY = -2,    /* Nmax < T, or a buffer is smaller than needed  */
    EP_ERR_UNSUPPORTED = -3, /* outside the limits below                      */
    EP_ERR_HIP = -4          /* the HIP runtime refused a launch              */
};

enum ep_dtype {
    EP_DTYPE_BF16 = 0,        /* rows of H bf16                                */
    EP_DTYPE_FP8_E4M3FN = 1   /* rows of H OCP e4m3fn bytes + H/128 fp32 scales */
};

/* Phases of ep_dispatch.  The pages time the sender's dispatch kernel and the
 * receiver's copy epilogue separately ([DET] Performance, [DRX] Background);
 * a caller may enqueue them in two calls (for example with its own event
 * between them).  EP_PHASE_ALL runs both. */
enum ep_phase {
    EP_PHASE_SCATTER = 1,
    EP_PHASE_EPILOGUE = 2,
    EP_PHASE_ALL = 3
};

/* Option bits of ep_config_t.flags. */
enum ep_flags {
    /* Direct Recv X ([DRX] Direct Recv X design): the scatter writes each hidden
     * row straight into its compact receive row recv_base[d] + recv_psum[d][s]
     * + j instead of the staging row; staging keeps the scales and metadata,
     * and the epilogue produces recv_sf and the metadata tensors but copies no
     * hidden bytes.  staging_x is not used (may be NULL).  Compact layout only
     * (EP_ERR_UNSUPPORTED with expand), as on the page. */
    EP_FLAG_DIRECT_RECV_X = 1,
    /* ep_layout of the compact layout as one launch, the form [DET] Approach
     * describes (a cooperative two-pass scan whose passes exchange their
     * counts grid-wide), used when its whole grid fits on the device at once
     * (checked on the host before the launch; otherwise the separate count
     * and slot launches run).  Same tables as the default two launches, which
     * measured faster on MI355X (8.3 against 9-11 us back to back at 4096
     * tokens, top-8 of 256 on 16 ranks): the device's kernel boundary is
     * cheaper than the exchange.  Its waits are bounded (far above any normal
     * duration); a layout whose exchange times out sets bit 1 of
     * *error_flags, and its tables are then not valid. */
    EP_FLAG_LAYOUT_ONE_LAUNCH = 2
};

/* Limits (checked on the host): 1 <= R <= 64, 1 <= K <= 32, E % R == 0,
 * E <= 1024, S <= 65535, T <= 2^30, H <= 262144, S * Nmax < 2^31,
 * S * T * K < 2^31, H * element size a multiple of 16 bytes, fp8 needs
 * H % 128 == 0.  Outside them a call returns EP_ERR_UNSUPPORTED. */
#define EP_MAX_RANKS 64
#define EP_MAX_TOKENS (1 << 30)
#define EP_MAX_TOPK 32
#define EP_MAX_EXPERTS 1024
#define EP_MAX_HIDDEN 262144

typedef struct ep_config {
    int32_t num_src_ranks;            /* S >= 1                                  */
    int32_t num_tokens;               /* T >= 0, tokens per source               */
    int32_t hidden;                   /* H                                       */
    int32_t num_topk;                 /* K                                       */
    int32_t num_experts;              /* E                                       */
    int32_t num_ranks;                /* R, destination ranks                    */
    int32_t num_max_tokens_per_rank;  /* Nmax >= T, else EP_ERR_CAPACITY: the
                                         rows a source may fill at one
                                         destination ([DET] Approach)            */
    int32_t x_dtype;                  /* enum ep_dtype                           */
    int32_t expand;                   /* 0: compact receive layout; 1: one row
                                         per valid (token, top-k) lane, grouped
                                         by expert                               */
    int32_t expert_alignment;         /* A >= 1; expand segments are padded to a
                                         multiple of A (ignored if !expand)      */
    int32_t num_layout_cus;           /* workgroups of the layout pass; 0 = auto
                                         (the pages' num_prologue_sms, [DET] New
                                         API); never changes any result          */
    int32_t flags;                    /* enum ep_flags bits; others must be 0    */
    int32_t num_scaleout_ranks;       /* 0 or 1: direct path.  > 1: hybrid path
                                         ([DET] Direct vs hybrid dispatch): the
                                         S source ranks are num_scaleout_ranks x
                                         num_scaleup_ranks, rank s = (s / n_up,
                                         s % n_up); S must be a multiple.  The
                                         row base of a slot is the sender's
                                         scale-out index, and a destination's
                                         staging buffer is read in row form:
                                         segment = scale-up index, offset =
                                         scale-out index * Nmax + row slot.
                                         Receive rows are the same as on the
                                         direct path.                            */
} ep_config_t;

/* Byte sizes of every caller-allocated buffer for a configuration (0 = not
 * used).  recv_rows is the receive capacity in rows: S*T*min(K,R) for the
 * compact layout, the largest count a destination-sum of deduplicated rows can
 * reach; S*T*K + E*(A-1) for expand. */
typedef struct ep_sizes {
    uint64_t dst_slot, tokens_per_rank, tokens_per_expert, recv_psum, recv_base;
    uint64_t expert_base, expand_pos, error_flags, layout_scratch, recv_psum_scaleup;
    uint64_t staging_x, staging_sf, staging_meta;
    uint64_t recv_rows;
    uint64_t recv_x, recv_sf, recv_src_idx, recv_topk_idx, recv_topk_weights;
    uint64_t y, out;
} ep_sizes_t;

/* Layout tables ("handle"): written by ep_layout, read by ep_dispatch and
 * ep_combine.  All device pointers, int32:
 *   dst_slot          [S][T][K]  row_base*Nmax + the number of earlier tokens
 *                                of source s that reach the same destination,
 *                                on the lowest valid lane of each destination
 *                                of a token; -1 on every other lane
 *                                ([DET] Motivation and Approach); row_base is
 *                                s (direct) or s / n_up (hybrid)
 *   tokens_per_rank   [S][R]     deduplicated tokens source s sends to rank d
 *   tokens_per_expert [S][E]     valid lanes of source s routed to expert e
 *   recv_psum         [R][S+1]   exclusive prefix over sources of
 *                                tokens_per_rank[.][d]: the base of source s
 *                                in destination d's compact receive rows
 *                                ([DRX] Direct Recv X design)
 *   recv_base         [R+1]      exclusive prefix over destinations of the
 *                                deduplicated row totals recv_psum[d][S];
 *                                recv_base[R] = rows in the compact layout
 *   expert_base       [E+1]      expand only: first row of expert e, segments
 *                                padded to a multiple of A
 *   expand_pos        [S][T][K]  expand only: receive row of a valid lane
 *                                (ascending (s,t,k) inside the expert), else -1
 *   recv_psum_scaleup [R][n_up+1] hybrid only: per destination, exclusive
 *                                prefix over scale-up segments of the rows
 *                                each segment holds (the per-segment part of
 *                                the pages' extended psum)
 *   error_flags       [1]        bit 0: some top-k id was >= E
 *   scratch           bytes      ep_sizes_t.layout_scratch, private to the
 *                                library; contents need no initialisation.
 *                                Compact layouts and expand layouts with
 *                                alignment 1: its head holds the receive-row
 *                                index (8 bytes per receive row, rounded up
 *                                to 256 bytes) that the copy epilogue reads,
 *                                written by a dispatch's scatter (compact) or
 *                                by the layout (expand, ep_layout_no_alloc
 *                                included when a scratch is given); the
 *                                layout's own words follow.  Required by
 *                                ep_layout; may be NULL for ep_dispatch (the
 *                                epilogue then searches the receiver tables
 *                                for each row's source: slower) and for
 *                                ep_combine, which do not allocate it.  */
typedef struct ep_layout {
    int32_t *dst_slot_dev;
    int32_t *tokens_per_rank_dev;
    int32_t *tokens_per_expert_dev;
    int32_t *recv_psum_dev;
    int32_t *recv_base_dev;
    int32_t *expert_base_dev;   /* NULL unless expand */
    int32_t *expand_pos_dev;    /* NULL unless expand */
    int32_t *error_flags_dev;
    void *scratch_dev;
    int32_t *recv_psum_scaleup_dev; /* NULL unless hybrid */
} ep_layout_t;

/* Staging ([R][S][Nmax] rows: destination d's receive buffer holds one Nmax-row
 * region per source, [DET] Direct vs hybrid dispatch) and receive buffers.
 *   staging_x     [R][S][Nmax][row bytes]; on the hybrid path the S regions
 *                 of a destination are ordered [n_up segments][n_out]
 *   staging_sf    [R][S][Nmax][H/128] fp32 (fp8 only, else NULL)
 *   staging_meta  [R][S][Nmax][1+2K] int32: token index t, the token's K
 *                 expert ids (masked/invalid as -1), the K weights' fp32 bits
 *   compact layout (expand == 0), row i of destination d's source s slot j is
 *   i = recv_base[d] + recv_psum[d][s] + j:
 *     recv_x [recv_rows][row bytes], recv_sf [recv_rows][H/128],
 *     recv_src_idx [recv_rows] (= s*T + t), recv_topk_idx [recv_rows][K]
 *     (local expert id on d, else -1), recv_topk_weights [recv_rows][K]
 *     (weight, else +0)
 *   expand layout: recv_x, recv_sf, recv_src_idx as above at expand_pos rows,
 *     recv_topk_weights [recv_rows] (the lane's weight); recv_topk_idx unused;
 *     padding rows get zero bytes, src -1 and weight +0.
 * Rows beyond the filled ones are left untouched. */
typedef struct ep_recv {
    void *staging_x_dev;
    float *staging_sf_dev;
    int32_t *staging_meta_dev;
    void *recv_x_dev;
    float *recv_sf_dev;
    int32_t *recv_src_idx_dev;
    int32_t *recv_topk_idx_dev;
    float *recv_topk_weights_dev;
    int64_t recv_capacity_rows;       /* rows allocated; must be >= recv_rows */
} ep_recv_t;

/* Host only (no HIP call): validate cfg and fill *sizes.  Returns EP_OK or the
 * validation error ([DRX] review: the buffer sizes are derived in one place). */
int ep_query_sizes(const ep_config_t *cfg, ep_sizes_t *sizes);

/* Deterministic layout prologue ([DET] Approach): a two-pass scan over
 * topk_idx_dev (int64 [S][T][K]) producing every table of *layout.  The result
 * is a pure function of topk_idx; num_layout_cus changes only the speed. */
int ep_layout(const ep_config_t *cfg, const int64_t *topk_idx_dev, const ep_layout_t *layout,
              void *stream);

/* Size of the layout scratch the library keeps on each GPU for
 * ep_layout_no_alloc. */
#define EP_NO_ALLOC_SCRATCH_BYTES (4u << 20)

/* ep_layout for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same launches and the same tables as ep_layout, but the scratch is an
 * EP_NO_ALLOC_SCRATCH_BYTES array the library holds on each GPU it runs on
 * until the process ends, so layout->scratch_dev is not required (may be
 * NULL; when given, only the receive-row index at its head is written).
 * The call allocates and frees nothing.  A configuration whose layout words
 * (ep_sizes_t.layout_scratch less the receive-row index at its head, which
 * the array does not hold) exceed EP_NO_ALLOC_SCRATCH_BYTES returns
 * EP_ERR_CAPACITY before anything is enqueued; EP_ERR_HIP if the array's
 * device address cannot be obtained.  Every call on one GPU uses that GPU's
 * one array: calls that overlap on one GPU (on different streams, or from
 * different host threads without ordering) race and may produce wrong tables,
 * so order them (for example, one stream).  The array needs no clearing
 * between calls. */
int ep_layout_no_alloc(const ep_config_t *cfg, const int64_t *topk_idx_dev, const ep_layout_t *layout,
                       void *stream);

/* Dispatch: scatter ([DET] Direct vs hybrid dispatch: senders replay the
 * layout's slots) of every token's row, scales and metadata into the staging
 * rows, then the copy epilogue ([DRX] Background) into the receive buffers.
 *   x_dev            [S][T][row bytes] (bf16, or e4m3fn bytes)
 *   x_sf_dev         [S][T][H/128] fp32 (fp8 only, else NULL)
 *   topk_idx_dev     int64 [S][T][K];  topk_weights_dev fp32 [S][T][K]
 *   phases           enum ep_phase mask; the epilogue reads the staging rows
 *                    the scatter of the same layout wrote (and, when the
 *                    layout's scratch is given, the receive-row index that
 *                    scatter wrote at its head: give both phases the same
 *                    layout). */
int ep_dispatch(const ep_config_t *cfg, const void *x_dev, const float *x_sf_dev,
                const int64_t *topk_idx_dev, const float *topk_weights_dev,
                const ep_layout_t *layout, const ep_recv_t *recv, int32_t phases, void *stream);

/* Layout and dispatch in one call: ep_layout followed by ep_dispatch with
 * EP_PHASE_ALL, with the same arguments, checks and results (the pages'
 * dispatch runs its deterministic prologue itself when no cached handle is
 * given, [DET] Approach and New API).  For one small source in the compact
 * layout (T*K <= 2048, rows of at most 1 KiB, no Direct Recv X) everything
 * runs as one kernel: each workgroup lays out the whole source in LDS and
 * dispatches its share of the tokens; otherwise the layout's and the
 * dispatch's launches are enqueued as the two calls would. */
int ep_layout_dispatch(const ep_config_t *cfg, const void *x_dev, const float *x_sf_dev,
                       const int64_t *topk_idx_dev, const float *topk_weights_dev, const ep_layout_t *layout,
                       const ep_recv_t *recv, void *stream);

/* Combine ([UNO] Changes: the reduce epilogue brings expert outputs back to
 * token order): out[s][t] = bf16(sum over valid lanes k of w[s][t][k] *
 * Y(s,t,k)), accumulated in fp32 and rounded to nearest-even once.  Y is, in
 * the compact layout, row recv_base[d] + recv_psum[d][s] + run of y_dev for
 * the lane's rank d (lanes sharing a rank weight the same row); in the expand
 * layout, row expand_pos[s][t][k].  A token with no valid lane gives +0.
 * Arithmetic order (fixed, so results are bitwise reproducible): in the
 * compact layout the weights of the lanes that share a rank are first summed
 * in fp32 in ascending lane order, then each distinct row is applied with one
 * fp32 fused multiply-add, rows in the order of their owner (lowest) lanes; in
 * the expand layout each valid lane's row is applied with one fused
 * multiply-add in ascending lane order.  The result is therefore within one
 * bf16 rounding of the exact sum, not bitwise that of a per-lane fp32 loop.
 *   y_dev   bf16 [rows][H] in the receive row order (at least recv_rows rows)
 *   out_dev bf16 [S][T][H] */
int ep_combine(const ep_config_t *cfg, const ep_layout_t *layout, const int64_t *topk_idx_dev,
               const float *topk_weights_dev, const void *y_dev, void *out_dev, void *stream);

/* Combine plus bias ([DET] Performance runs the combine with num_bias = 2):
 * out[s][t] = bf16(sum over valid lanes of w * Y + bias0[s][t] + bias1[s][t]),
 * the bias rows added in fp32 before the one rounding.  bias0_dev / bias1_dev
 * are bf16 [S][T][H] (16-byte aligned), either may be NULL; with both NULL
 * this is ep_combine. */
int ep_combine_bias(const ep_config_t *cfg, const ep_layout_t *layout, const int64_t *topk_idx_dev,
                    const float *topk_weights_dev, const void *y_dev, const void *bias0_dev,
                    const void *bias1_dev, void *out_dev, void *stream);

/* Static description of a status code. */
const char *ep_status_string(int status);

/* Library version, MAJOR*10000 + MINOR*100 + PATCH. */
int ep_version(void);

#ifdef __cplusplus
}
#endif
#endif /* EP_H */
