// ep_api.cpp -- the C ABI declared in include/ep.h: argument validation,
// buffer sizes and kernel launches.  Everything here runs on the host; the
// only HIP calls are the launches (and hipGetLastError) inside the launchers.
//
// Guardrails follow DeepEP v2 "Add experimental direct recv_x dispatch path"
// (PR #690), section Implementation and review: unsupported combinations and
// buffers that are too small are rejected before anything runs -- here with a
// status code instead of an abort.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "ep.h"
#include "ep_kernels.h"

namespace {

constexpr int64_t kInt32Max = 2147483647;

int bits_for(int n) {
    int b = 0;
    while ((1 << b) < n) ++b;
    return b;
}

// Validate a configuration and derive the kernel shape.
int make_shape(const ep_config_t *c, ep::Shape *sh) {
    if (!c || !sh) return EP_ERR_INVALID_ARG;
    if ((c->flags & ~(EP_FLAG_DIRECT_RECV_X | EP_FLAG_LAYOUT_ONE_LAUNCH)) != 0) return EP_ERR_INVALID_ARG;
    if ((c->flags & EP_FLAG_DIRECT_RECV_X) && c->expand) return EP_ERR_UNSUPPORTED;
    if (c->num_src_ranks < 1 || c->num_tokens < 0 || c->hidden < 1 || c->num_topk < 1 || c->num_experts < 1 ||
        c->num_ranks < 1 || c->num_max_tokens_per_rank < 0 || c->num_layout_cus < 0 || c->expert_alignment < 1 ||
        c->num_scaleout_ranks < 0)
        return EP_ERR_INVALID_ARG;
    if (c->num_scaleout_ranks > 1 && c->num_src_ranks % c->num_scaleout_ranks != 0) return EP_ERR_INVALID_ARG;
    if (c->x_dtype != EP_DTYPE_BF16 && c->x_dtype != EP_DTYPE_FP8_E4M3FN) return EP_ERR_INVALID_ARG;
    if (c->expand != 0 && c->expand != 1) return EP_ERR_INVALID_ARG;
    if (c->num_experts % c->num_ranks != 0) return EP_ERR_INVALID_ARG;
    if (c->num_ranks > EP_MAX_RANKS || c->num_topk > EP_MAX_TOPK || c->num_experts > EP_MAX_EXPERTS ||
        c->hidden > EP_MAX_HIDDEN)
        return EP_ERR_UNSUPPORTED;
    const bool fp8 = c->x_dtype == EP_DTYPE_FP8_E4M3FN;
    if (fp8 && c->hidden % 128 != 0) return EP_ERR_INVALID_ARG;
    if (!fp8 && c->hidden % 8 != 0) return EP_ERR_INVALID_ARG;  // 16-byte rows
    if (c->num_max_tokens_per_rank < c->num_tokens) return EP_ERR_CAPACITY;
    const int64_t S = c->num_src_ranks, T = c->num_tokens, K = c->num_topk;
    if (S > 65535) return EP_ERR_UNSUPPORTED;  // sources index the layout grid's y dimension
    if (T > EP_MAX_TOKENS) return EP_ERR_UNSUPPORTED;  // token loops step past T in 32-bit arithmetic
    if (S * c->num_max_tokens_per_rank > kInt32Max) return EP_ERR_UNSUPPORTED;
    if (S * T * K > kInt32Max) return EP_ERR_UNSUPPORTED;
    if (S * T * K + (int64_t)c->num_experts * (c->expert_alignment - 1) > kInt32Max) return EP_ERR_UNSUPPORTED;
    sh->S = c->num_src_ranks;
    sh->T = c->num_tokens;
    sh->H = c->hidden;
    sh->K = c->num_topk;
    sh->E = c->num_experts;
    sh->R = c->num_ranks;
    sh->El = c->num_experts / c->num_ranks;
    sh->el_mul = (1u << 22) / (uint32_t)sh->El + 1u;
    sh->Nmax = c->num_max_tokens_per_rank;
    sh->expand = c->expand;
    sh->A = c->expert_alignment;
    sh->is_fp8 = fp8 ? 1 : 0;
    sh->row_bytes = fp8 ? c->hidden : 2 * c->hidden;
    sh->sf_per_row = fp8 ? c->hidden / 128 : 0;
    sh->meta_words = 1 + 2 * c->num_topk;
    sh->bits_R = bits_for(c->num_ranks);
    sh->bits_E = bits_for(c->num_experts);
    sh->direct = (c->flags & EP_FLAG_DIRECT_RECV_X) ? 1 : 0;
    sh->n_out = c->num_scaleout_ranks > 1 ? c->num_scaleout_ranks : 1;
    sh->n_up = c->num_src_ranks / sh->n_out;
    return EP_OK;
}

int64_t recv_rows(const ep::Shape &sh) {
    const int64_t S = sh.S, T = sh.T, K = sh.K;
    if (sh.expand) return S * T * K + (int64_t)sh.E * (sh.A - 1);
    return S * T * (K < sh.R ? K : sh.R);
}

// The head of a layout's scratch: the receive-row index of the staging path,
// one int64 per receive row (compact: the staging row, written by the scatter;
// expand with alignment 1: the staging row and top-k lane, written by the
// layout's slot pass), read by the copy epilogue; the layout's own words
// follow it.  Its size depends on the
// shape only (not on num_layout_cus or the flags), so one layout serves both
// dispatch paths and any workgroup count.  Padded expand layouts have none.
bool has_recv_index(const ep::Shape &sh) { return !sh.expand || sh.A == 1; }
uint64_t recv_index_bytes(const ep::Shape &sh) {
    if (!has_recv_index(sh)) return 0;
    const uint64_t rows = sh.expand ? (uint64_t)recv_rows(sh) : (uint64_t)ep::compact_rows_bound(sh);
    return (rows * sizeof(int64_t) + 255) & ~(uint64_t)255;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// need_scratch: the caller's scratch_dev is required (ep_layout; the no-alloc
// layout takes the library's own, and the dispatch and the combine do not need
// one).
int check_layout_ptrs(const ep::Shape &sh, const ep_layout_t *L, bool need_scratch = true) {
    if (!L) return EP_ERR_INVALID_ARG;
    const bool need_tok = (int64_t)sh.S * sh.T * sh.K > 0;
    if ((need_tok && !L->dst_slot_dev) || !L->tokens_per_rank_dev || !L->tokens_per_expert_dev ||
        !L->recv_psum_dev || !L->recv_base_dev || !L->error_flags_dev || (need_scratch && !L->scratch_dev))
        return EP_ERR_INVALID_ARG;
    if (sh.expand && (!L->expert_base_dev || (need_tok && !L->expand_pos_dev))) return EP_ERR_INVALID_ARG;
    if (sh.n_out > 1 && !L->recv_psum_scaleup_dev) return EP_ERR_INVALID_ARG;
    const void *ps[] = {L->dst_slot_dev, L->tokens_per_rank_dev, L->tokens_per_expert_dev, L->recv_psum_dev,
                        L->recv_base_dev, L->expert_base_dev, L->expand_pos_dev, L->error_flags_dev,
                        need_scratch ? L->scratch_dev : nullptr, L->recv_psum_scaleup_dev};
    for (const void *p : ps)
        if (!aligned(p, 4)) return EP_ERR_INVALID_ARG;
    return EP_OK;
}

}  // namespace

extern "C" {

int ep_version(void) { return 100; }

const char *ep_status_string(int status) {
    switch (status) {
        case EP_OK: return "ok";
        case EP_ERR_INVALID_ARG: return "invalid argument";
        case EP_ERR_CAPACITY: return "capacity exceeded (Nmax < T or a buffer is too small)";
        case EP_ERR_UNSUPPORTED: return "unsupported configuration";
        case EP_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

int ep_query_sizes(const ep_config_t *cfg, ep_sizes_t *sz) {
    ep::Shape sh;
    const int rc = make_shape(cfg, &sh);
    if (rc != EP_OK) return rc;
    if (!sz) return EP_ERR_INVALID_ARG;
    memset(sz, 0, sizeof(*sz));
    const uint64_t S = sh.S, T = sh.T, K = sh.K, E = sh.E, R = sh.R, Nmax = sh.Nmax;
    const uint64_t i4 = sizeof(int32_t);
    sz->dst_slot = S * T * K * i4;
    sz->tokens_per_rank = S * R * i4;
    sz->tokens_per_expert = S * E * i4;
    sz->recv_psum = R * (S + 1) * i4;
    sz->recv_base = (R + 1) * i4;
    sz->expert_base = sh.expand ? (E + 1) * i4 : 0;
    sz->expand_pos = sh.expand ? S * T * K * i4 : 0;
    sz->error_flags = i4;
    sz->layout_scratch =
        recv_index_bytes(sh) + ep::layout_scratch_bytes(sh, ep::layout_geometry(sh, cfg->num_layout_cus));
    sz->recv_psum_scaleup = sh.n_out > 1 ? R * ((uint64_t)sh.n_up + 1) * i4 : 0;
    const uint64_t staging_rows = R * S * Nmax;
    sz->staging_x = sh.direct ? 0 : staging_rows * (uint64_t)sh.row_bytes;
    sz->staging_sf = staging_rows * (uint64_t)sh.sf_per_row * sizeof(float);
    sz->staging_meta = staging_rows * (uint64_t)sh.meta_words * i4;
    const uint64_t rows = (uint64_t)recv_rows(sh);
    sz->recv_rows = rows;
    sz->recv_x = rows * (uint64_t)sh.row_bytes;
    sz->recv_sf = rows * (uint64_t)sh.sf_per_row * sizeof(float);
    sz->recv_src_idx = rows * i4;
    sz->recv_topk_idx = sh.expand ? 0 : rows * K * i4;
    sz->recv_topk_weights = sh.expand ? rows * sizeof(float) : rows * K * sizeof(float);
    sz->y = rows * (uint64_t)sh.H * 2;
    sz->out = S * T * (uint64_t)sh.H * 2;
    return EP_OK;
}

}  // extern "C"

namespace {

// Validated launch arguments of a layout on the caller's scratch or on the
// library's own (own_scratch).
int make_layout_args(const ep_config_t *cfg, const int64_t *topk_idx_dev, const ep_layout_t *layout,
                     bool own_scratch, ep::LayoutArgs *out) {
    ep::Shape sh;
    int rc = make_shape(cfg, &sh);
    if (rc != EP_OK) return rc;
    if ((rc = check_layout_ptrs(sh, layout, !own_scratch)) != EP_OK) return rc;
    if ((int64_t)sh.S * sh.T * sh.K > 0 && (!topk_idx_dev || !aligned(topk_idx_dev, 8))) return EP_ERR_INVALID_ARG;
    ep::LayoutArgs &a = *out;
    a.sh = sh;
    a.g = ep::layout_geometry(sh, cfg->num_layout_cus);
    void *scratch = layout->scratch_dev ? static_cast<char *>(layout->scratch_dev) + recv_index_bytes(sh) : nullptr;
    if (own_scratch) {  // the library's array holds the layout's own words only
        if (ep::layout_scratch_bytes(sh, a.g) > EP_NO_ALLOC_SCRATCH_BYTES) return EP_ERR_CAPACITY;
        if (ep::no_alloc_scratch(&scratch) != hipSuccess) return EP_ERR_HIP;
    }
    a.topk_idx = topk_idx_dev;
    a.dst_slot = layout->dst_slot_dev;
    a.tokens_per_rank = layout->tokens_per_rank_dev;
    a.tokens_per_expert = layout->tokens_per_expert_dev;
    a.recv_psum = layout->recv_psum_dev;
    a.recv_base = layout->recv_base_dev;
    a.expert_base = layout->expert_base_dev;
    a.expand_pos = layout->expand_pos_dev;
    a.error_flags = layout->error_flags_dev;
    a.recv_psum_scaleup = layout->recv_psum_scaleup_dev;
    const int64_t units = (int64_t)sh.S * a.g.blocks_per_src;
    a.blk_cnt_rank = static_cast<int32_t *>(scratch);
    a.blk_cnt_expert = a.blk_cnt_rank + units * sh.R;
    a.blk_flags = a.blk_cnt_expert + units * sh.E;
    a.blk_pre_expert = sh.expand ? a.blk_flags + units : nullptr;
    a.cnt_expert = sh.expand ? a.blk_pre_expert + units * sh.E : nullptr;
    // The one-launch layout's exchange words follow the counts, 8-byte aligned.
    a.sync = nullptr;
    if (!sh.expand) {
        const uintptr_t end = reinterpret_cast<uintptr_t>(a.blk_flags + units);
        a.sync = reinterpret_cast<uint64_t *>((end + 7) & ~static_cast<uintptr_t>(7));
    }
    a.one_launch = (cfg->flags & EP_FLAG_LAYOUT_ONE_LAUNCH) ? 1 : 0;
    // The expand index at the head of the caller's scratch (alignment 1), when
    // one is given -- also to ep_layout_no_alloc, whose own words live in the
    // library's array.
    a.expand_row_src = (sh.expand && has_recv_index(sh) && layout->scratch_dev && aligned(layout->scratch_dev, 8))
                           ? static_cast<int64_t *>(layout->scratch_dev)
                           : nullptr;
    // Bounds of the exchange's waits (each poll is one device-scope load and
    // a short sleep, about a microsecond): 2^21 polls for the coordinator and
    // for each unit.  EP_LAYOUT_SYNC_TEST forces a time-out, for tests of the
    // error path only: 1 = the coordinator waits for words no unit writes;
    // 2 = every unit does.
    a.spin_master = 1u << 21;
    a.spin_unit = 1u << 21;
    a.sync_test = 0;
    if (const char *t = getenv("EP_LAYOUT_SYNC_TEST")) {
        if (t[0] == '1') {
            a.sync_test = 1;
            a.spin_master = 64;
        } else if (t[0] == '2') {
            a.sync_test = 2;
            a.spin_unit = 64;
        }
    }
    return EP_OK;
}

int layout_call(const ep_config_t *cfg, const int64_t *topk_idx_dev, const ep_layout_t *layout, void *stream,
                bool own_scratch) {
    ep::LayoutArgs a;
    const int rc = make_layout_args(cfg, topk_idx_dev, layout, own_scratch, &a);
    if (rc != EP_OK) return rc;
    return ep::launch_layout(a, (hipStream_t)stream) == hipSuccess ? EP_OK : EP_ERR_HIP;
}

// Validated launch arguments of a dispatch.
int make_dispatch_args(const ep_config_t *cfg, const void *x_dev, const float *x_sf_dev, const int64_t *topk_idx_dev,
                       const float *topk_weights_dev, const ep_layout_t *layout, const ep_recv_t *recv,
                       ep::DispatchArgs *out) {
    ep::Shape sh;
    int rc = make_shape(cfg, &sh);
    if (rc != EP_OK) return rc;
    if ((rc = check_layout_ptrs(sh, layout, false)) != EP_OK) return rc;
    if (!recv) return EP_ERR_INVALID_ARG;
    const bool tok = (int64_t)sh.S * sh.T > 0;
    if (tok) {
        if (!x_dev || !aligned(x_dev, 16) || !topk_idx_dev || !aligned(topk_idx_dev, 8) || !topk_weights_dev ||
            !aligned(topk_weights_dev, 4))
            return EP_ERR_INVALID_ARG;
        if ((!sh.direct && (!recv->staging_x_dev || !aligned(recv->staging_x_dev, 16))) || !recv->staging_meta_dev ||
            !aligned(recv->staging_meta_dev, 4) || !recv->recv_x_dev || !aligned(recv->recv_x_dev, 16) ||
            !recv->recv_src_idx_dev || !aligned(recv->recv_src_idx_dev, 4) || !recv->recv_topk_weights_dev ||
            !aligned(recv->recv_topk_weights_dev, 4))
            return EP_ERR_INVALID_ARG;
        if (!sh.expand && (!recv->recv_topk_idx_dev || !aligned(recv->recv_topk_idx_dev, 4)))
            return EP_ERR_INVALID_ARG;
        if (sh.is_fp8 && (!x_sf_dev || !aligned(x_sf_dev, 4) || !recv->staging_sf_dev ||
                          !aligned(recv->staging_sf_dev, 4) || !recv->recv_sf_dev || !aligned(recv->recv_sf_dev, 4)))
            return EP_ERR_INVALID_ARG;
    }
    if (recv->recv_capacity_rows < recv_rows(sh)) return EP_ERR_CAPACITY;
    ep::DispatchArgs &a = *out;
    a.sh = sh;
    a.x = static_cast<const uint8_t *>(x_dev);
    a.x_sf = x_sf_dev;
    a.topk_idx = topk_idx_dev;
    a.topk_weights = topk_weights_dev;
    a.dst_slot = layout->dst_slot_dev;
    a.recv_psum = layout->recv_psum_dev;
    a.recv_base = layout->recv_base_dev;
    a.tokens_per_expert = layout->tokens_per_expert_dev;
    a.expert_base = layout->expert_base_dev;
    a.expand_pos = layout->expand_pos_dev;
    a.staging_x = static_cast<uint8_t *>(recv->staging_x_dev);
    a.staging_sf = recv->staging_sf_dev;
    a.staging_meta = recv->staging_meta_dev;
    a.recv_x = static_cast<uint8_t *>(recv->recv_x_dev);
    a.recv_sf = recv->recv_sf_dev;
    a.recv_src_idx = recv->recv_src_idx_dev;
    a.recv_topk_idx = recv->recv_topk_idx_dev;
    a.recv_topk_weights = recv->recv_topk_weights_dev;
    a.recv_capacity_rows = recv->recv_capacity_rows;
    a.slices = 1;
    // The receive-row index at the head of the layout's scratch (staging
    // path), when the caller passes one; else the epilogues search the
    // receiver tables.
    const bool index = has_recv_index(sh) && !sh.direct && layout->scratch_dev && aligned(layout->scratch_dev, 8);
    a.recv_row_src = index && !sh.expand ? static_cast<int64_t *>(layout->scratch_dev) : nullptr;
    a.expand_row_src = index && sh.expand ? static_cast<int64_t *>(layout->scratch_dev) : nullptr;
    return EP_OK;
}

int dispatch_launches(const ep::DispatchArgs &a, int32_t phases, hipStream_t st) {
    if (phases == EP_PHASE_ALL && ep::dispatch_is_one_launch(a))
        return ep::launch_dispatch_fused(a, st) == hipSuccess ? EP_OK : EP_ERR_HIP;
    if ((phases & EP_PHASE_SCATTER) && ep::launch_scatter(a, st) != hipSuccess) return EP_ERR_HIP;
    if ((phases & EP_PHASE_EPILOGUE) && ep::launch_epilogue(a, st) != hipSuccess) return EP_ERR_HIP;
    return EP_OK;
}

}  // namespace

extern "C" {

int ep_layout(const ep_config_t *cfg, const int64_t *topk_idx_dev, const ep_layout_t *layout, void *stream) {
    return layout_call(cfg, topk_idx_dev, layout, stream, false);
}

int ep_layout_no_alloc(const ep_config_t *cfg, const int64_t *topk_idx_dev, const ep_layout_t *layout,
                       void *stream) {
    return layout_call(cfg, topk_idx_dev, layout, stream, true);
}

int ep_dispatch(const ep_config_t *cfg, const void *x_dev, const float *x_sf_dev, const int64_t *topk_idx_dev,
                const float *topk_weights_dev, const ep_layout_t *layout, const ep_recv_t *recv, int32_t phases,
                void *stream) {
    if (phases < 1 || phases > EP_PHASE_ALL) return EP_ERR_INVALID_ARG;
    ep::DispatchArgs a;
    const int rc = make_dispatch_args(cfg, x_dev, x_sf_dev, topk_idx_dev, topk_weights_dev, layout, recv, &a);
    if (rc != EP_OK) return rc;
    return dispatch_launches(a, phases, (hipStream_t)stream);
}

int ep_layout_dispatch(const ep_config_t *cfg, const void *x_dev, const float *x_sf_dev,
                       const int64_t *topk_idx_dev, const float *topk_weights_dev, const ep_layout_t *layout,
                       const ep_recv_t *recv, void *stream) {
    ep::LayoutArgs la;
    int rc = make_layout_args(cfg, topk_idx_dev, layout, false, &la);
    if (rc != EP_OK) return rc;
    ep::DispatchArgs da;
    if ((rc = make_dispatch_args(cfg, x_dev, x_sf_dev, topk_idx_dev, topk_weights_dev, layout, recv, &da)) != EP_OK)
        return rc;
    hipStream_t st = (hipStream_t)stream;
    if (ep::layout_dispatch_is_one_launch(la, da))
        return ep::launch_layout_dispatch(la, da, st) == hipSuccess ? EP_OK : EP_ERR_HIP;
    if (ep::launch_layout(la, st) != hipSuccess) return EP_ERR_HIP;
    return dispatch_launches(da, EP_PHASE_ALL, st);
}

int ep_combine(const ep_config_t *cfg, const ep_layout_t *layout, const int64_t *topk_idx_dev,
               const float *topk_weights_dev, const void *y_dev, void *out_dev, void *stream) {
    return ep_combine_bias(cfg, layout, topk_idx_dev, topk_weights_dev, y_dev, nullptr, nullptr, out_dev, stream);
}

int ep_combine_bias(const ep_config_t *cfg, const ep_layout_t *layout, const int64_t *topk_idx_dev,
                    const float *topk_weights_dev, const void *y_dev, const void *bias0_dev,
                    const void *bias1_dev, void *out_dev, void *stream) {
    ep::Shape sh;
    int rc = make_shape(cfg, &sh);
    if (rc != EP_OK) return rc;
    if ((rc = check_layout_ptrs(sh, layout, false)) != EP_OK) return rc;
    if ((int64_t)sh.S * sh.T > 0) {
        if (!topk_idx_dev || !aligned(topk_idx_dev, 8) || !topk_weights_dev || !aligned(topk_weights_dev, 4) ||
            !y_dev || !aligned(y_dev, 16) || !out_dev || !aligned(out_dev, 16))
            return EP_ERR_INVALID_ARG;
        if ((bias0_dev && !aligned(bias0_dev, 16)) || (bias1_dev && !aligned(bias1_dev, 16)))
            return EP_ERR_INVALID_ARG;
    }
    ep::CombineArgs a;
    a.sh = sh;
    a.topk_idx = topk_idx_dev;
    a.topk_weights = topk_weights_dev;
    a.dst_slot = layout->dst_slot_dev;
    a.recv_psum = layout->recv_psum_dev;
    a.recv_base = layout->recv_base_dev;
    a.expand_pos = layout->expand_pos_dev;
    a.y = static_cast<const uint16_t *>(y_dev);
    a.bias0 = static_cast<const uint16_t *>(bias0_dev);
    a.bias1 = static_cast<const uint16_t *>(bias1_dev);
    a.out = static_cast<uint16_t *>(out_dev);
    a.y_rows = recv_rows(sh);
    return ep::launch_combine(a, (hipStream_t)stream) == hipSuccess ? EP_OK : EP_ERR_HIP;
}

}  // extern "C"
