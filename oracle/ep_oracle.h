/*
 * ep_oracle.h -- plain CPU oracle for deterministic MoE expert-parallel
 * dispatch (layout prologue, scatter, copy epilogue) and combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no source,
 * header, table or helper with the HIP library; both sides only consume the
 * same seeded inputs.  All pointers are host pointers; all arrays are dense
 * row-major.
 *
 * Notation (S source partitions, T tokens per source, H hidden, K top-k,
 * E experts on R ranks, El = E / R experts per rank, Nmax =
 * num_max_tokens_per_rank, A = expert alignment of the expand layout,
 * n_out = num_scaleout_ranks: <= 1 is the direct path, > 1 the hybrid path
 * with S = n_out * n_up source ranks, rank s = (s / n_up, s % n_up)).
 *
 * Sources (DeepEP v2 pages):
 *   [DET]  "DeepEP v2: Kernel-side deterministic dispatch for the non-expand
 *          layout" (PR #753), sections Motivation, Approach, Direct vs hybrid
 *          dispatch, Compatibility.
 *   [DRX]  "DeepEP v2: Add experimental direct recv_x dispatch path" (PR #690),
 *          sections Background and Direct Recv X design.
 *   [UNO]  "Add unordered hybrid kernels for transports without ordered
 *          delivery" (PR #732), section Changes (combine reduce epilogue).
 *
 * Every function returns 0 on success and -1 when the sizes are inconsistent
 * (E % R != 0, K < 1, Nmax < T, ...).  Nothing here is tuned: loops follow
 * the definitions in the order they are stated.
 */
#ifndef EP_ORACLE_H
#define EP_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Layout prologue: per-destination counts, exclusive prefix sums and one slot
 * per (token, top-k) entry; plus the expand-layout positions when expand != 0.
 *   topk_idx          [S][T][K]  int64, expert id; < 0 masked; >= E invalid
 *   dst_slot          [S][T][K]  out: row_base(s)*Nmax + running count, or -1
 *                                (row_base = s direct, s / n_up hybrid)
 *   tokens_per_rank   [S][R]     out
 *   tokens_per_expert [S][E]     out
 *   recv_psum         [R][S+1]   out: exclusive prefix over sources
 *   recv_base         [R+1]      out: exclusive prefix over destinations of the
 *                                     deduplicated row counts
 *   expert_base       [E+1]      out (expand only, else may be NULL)
 *   expand_pos        [S][T][K]  out (expand only, else may be NULL)
 *   recv_psum_scaleup [R][n_up+1] out (hybrid only, else may be NULL):
 *                                exclusive prefix over scale-up segments
 *   error_flags       [1]        out: bit 0 = some lane had id >= E          */
int epo_layout(int S, int T, int K, int E, int R, int Nmax, int expand, int A, int n_out,
               const int64_t *topk_idx, int32_t *dst_slot, int32_t *tokens_per_rank,
               int32_t *tokens_per_expert, int32_t *recv_psum, int32_t *recv_base,
               int32_t *expert_base, int32_t *expand_pos, int32_t *recv_psum_scaleup,
               int32_t *error_flags);

/* Dispatch: scatter of each token's row (and fp8 scales, and metadata) into
 * the staging rows [R][S][Nmax], then the copy epilogue into recv_*.
 *   is_fp8: rows are H bytes of e4m3fn plus H/128 fp32 scales; else 2H bytes.
 *   x [S][T][row bytes], x_sf [S][T][H/128] (fp8 only, else NULL)
 *   staging_x [R][S][Nmax][row bytes], staging_sf [R][S][Nmax][H/128],
 *   staging_meta [R][S][Nmax][1+2K] int32; hybrid: the S regions of a
 *   destination are ordered [n_up segments][n_out regions]
 *   non-expand: recv_x [rows][row bytes], recv_sf [rows][H/128],
 *               recv_src_idx [rows], recv_topk_idx [rows][K],
 *               recv_topk_weights [rows][K]
 *   expand:     recv_x, recv_sf, recv_src_idx as above, recv_topk_weights
 *               [rows], recv_topk_idx unused (may be NULL)              */
int epo_dispatch(int S, int T, int H, int K, int E, int R, int Nmax, int is_fp8,
                 int expand, int A, int n_out, const uint8_t *x, const float *x_sf,
                 const int64_t *topk_idx, const float *topk_weights,
                 const int32_t *dst_slot, const int32_t *tokens_per_rank,
                 const int32_t *tokens_per_expert, const int32_t *recv_psum,
                 const int32_t *recv_base, const int32_t *expert_base,
                 const int32_t *expand_pos, uint8_t *staging_x, float *staging_sf,
                 int32_t *staging_meta, uint8_t *recv_x, float *recv_sf,
                 int32_t *recv_src_idx, int32_t *recv_topk_idx, float *recv_topk_weights);

/* Combine: out[s][t] = bf16(sum over valid k of w[s][t][k] * Y(s,t,k)),
 * accumulated in double and rounded to bf16 once (nearest, ties to even).
 *   y   [rows][H] bf16 bits, in the recv row order (non-expand) or the
 *       expand row order (expand)
 *   out [S][T][H] bf16 bits                                               */
int epo_combine(int S, int T, int H, int K, int E, int R, int Nmax, int expand, int n_out,
                const int64_t *topk_idx, const float *topk_weights,
                const int32_t *dst_slot, const int32_t *recv_psum,
                const int32_t *recv_base, const int32_t *expand_pos,
                const uint16_t *y, uint16_t *out);

/* Combine plus up to two bias tensors bias0/bias1 (bf16 bits [S][T][H], NULL
 * when absent): out = bf16(sum_k w*Y + bias0 + bias1), summed in double and
 * rounded once. */
int epo_combine_bias(int S, int T, int H, int K, int E, int R, int Nmax, int expand, int n_out,
                     const int64_t *topk_idx, const float *topk_weights,
                     const int32_t *dst_slot, const int32_t *recv_psum,
                     const int32_t *recv_base, const int32_t *expand_pos,
                     const uint16_t *y, const uint16_t *bias0, const uint16_t *bias1, uint16_t *out);

/* Combine restricted to the n_sel global token indices sel[i] = s*T + t;
 * out is [n_sel][H].  Same definition as epo_combine. */
int epo_combine_tokens(int S, int T, int H, int K, int E, int R, int Nmax, int expand, int n_out,
                       const int64_t *topk_idx, const float *topk_weights,
                       const int32_t *dst_slot, const int32_t *recv_psum,
                       const int32_t *recv_base, const int32_t *expand_pos,
                       const uint16_t *y, int n_sel, const int64_t *sel, uint16_t *out);

/* Round a double to bf16 bits, nearest with ties to even (exposed for pins). */
uint16_t epo_bf16_from_double(double v);

#ifdef __cplusplus
}
#endif
#endif
