// ep_combine.hip -- weighted top-k reduction of expert outputs back to token
// order (the combine reduce epilogue of DeepEP v2, "Add unordered hybrid
// kernels for transports without ordered delivery" (PR #732), section
// Changes).
//
// out[s][t] = bf16(sum over valid lanes k of w[s][t][k] * Y [+ bias rows]),
// accumulated in fp32 and rounded to nearest-even once.  In the compact layout
// Y is the receive row that the owner lane of the lane's rank was given
// (recv_base[d] + recv_psum[d][s] + slot - row_base(s)*Nmax), so lanes sharing
// a rank weight the same row: the kernel reads that row once and applies the
// fp32 sum of those lanes' weights (taken in lane order).  In the expand layout
// Y is the lane's own row expand_pos[s][t][k].
//
// The work is an HBM stream with about one FMA per 2 bytes read, far below
// the MFMA ridge, so it runs on the vector ALUs.  A work unit is one column
// slice of one token (by default one pass: 64 lanes x CPL 16-byte chunks);
// every lane loads its chunks of each of up to G distinct rows before any
// FMA, so G*CPL loads per lane are in flight.  Many small units balance the
// uneven number of rows per token across the resident waves.
#include "ep_device.h"
#include "ep_kernels.h"

namespace ep {
namespace {

// Waves per workgroup.  Measured on MI355X (4096 tokens H = 7168 bf16 and
// fp8, 8192 tokens H = 4096): 1 or 2 waves 0.3-1 us and 8 waves 2 us slower
// in the combine than 4.
#ifndef EP_COMBINE_WAVES
#define EP_COMBINE_WAVES 4
#endif
constexpr int kWavesPerBlock = EP_COMBINE_WAVES;
constexpr int kThreads = kWavesPerBlock * kWave;
#ifndef EP_COMBINE_ROWS
#define EP_COMBINE_ROWS 8  // G: distinct rows loaded together
#endif
#ifndef EP_COMBINE_CPL
#define EP_COMBINE_CPL 2  // 16-byte chunks per lane per row per pass
#endif
#ifndef EP_COMBINE_NT_LOAD
#define EP_COMBINE_NT_LOAD 1  // each expert-output row is read once
#endif
#ifndef EP_COMBINE_NT_STORE
#define EP_COMBINE_NT_STORE 1  // each output row is written once
#endif
#ifndef EP_COMBINE_SLICES
// Column slices of a token's row, each a separate work unit; 0 = one pass
// (64 lanes x CPL chunks) per unit, measured best on MI355X at H = 7168.
#define EP_COMBINE_SLICES 0
#endif
constexpr int kRowsPerGroup = EP_COMBINE_ROWS;
// One wave per work unit, no grid-stride cap (measured at 16 x 2048 tokens:
// 771 us capped at 16384 workgroups, 756 us uncapped).
// In the expand layout (one row per lane, 8 rows per token at top-8) the
// launch asks for enough LDS that at most three workgroups are resident per CU
// (3 waves per SIMD instead of the 4 the registers allow): measured on MI355X
// at 16 x 2048 tokens, H = 7168, 754 -> 705 us (2 per SIMD: 737 us).  The
// compact layout's combine keeps all 4: capped the same way it measured 3-7%
// slower.
#ifndef EP_COMBINE_EXPAND_LDS
#define EP_COMBINE_EXPAND_LDS lds_to_cap_residency(3)
#endif
#ifndef EP_COMBINE_MAX_BLOCKS
#define EP_COMBINE_MAX_BLOCKS (1 << 20)
#endif


__device__ __forceinline__ u32x4 ld16(const uint16_t *p) {
    const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
#if EP_COMBINE_NT_LOAD
    return __builtin_nontemporal_load(q);
#else
    return *q;
#endif
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;  // quiet NaN
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int CPL>
__device__ __forceinline__ void fma_row(float (&acc)[CPL][8], const u32x4 (&v)[CPL], float w) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t u = v[i][q];
            acc[i][2 * q] = fmaf(w, __uint_as_float(u << 16), acc[i][2 * q]);
            acc[i][2 * q + 1] = fmaf(w, __uint_as_float(u & 0xffff0000u), acc[i][2 * q + 1]);
        }
    }
}

// The distinct rows of token g, one per "row lane": every valid lane in the
// expand layout; the owner (lowest valid lane) of each rank otherwise, whose
// weight becomes the lane-ordered fp32 sum over the lanes of its rank.
// Returns the mask of row lanes; row / wrow hold each row lane's row and weight.
// With EARLY_BASES, lane l < R fetches the base of source s in destination l's
// receive rows together with the ids, so that no load waits for a decoded
// rank: one dependent load fewer, which matters for short rows only (for
// 14 KiB rows the four extra registers cost a wave per SIMD: measured 2-3%
// slower at 4096 tokens, H = 7168).
template <bool EARLY_BASES>
__device__ __forceinline__ uint64_t token_rows(const CombineArgs &a, int64_t g, int lane, int &row, float &wrow) {
    const Shape &sh = a.sh;
    const int s = (int)(g / sh.T);
    bool valid = false;
    float w = 0.0f;
    int e = 0, slot = -1, pos = -1;
    if (lane < sh.K) {
        const int64_t e64 = a.topk_idx[g * sh.K + lane];
        valid = e64 >= 0 && e64 < sh.E;
        e = valid ? (int)e64 : 0;
        w = a.topk_weights[g * sh.K + lane];
        if (sh.expand) pos = a.expand_pos[g * sh.K + lane];
        else slot = a.dst_slot[g * sh.K + lane];
    }
    int base_l = 0;
    if (EARLY_BASES && !sh.expand && lane < sh.R)
        base_l = a.recv_base[lane] + a.recv_psum[(int64_t)lane * (sh.S + 1) + s];
    const uint64_t vmask = ballot(valid);
    row = -1;
    wrow = 0.0f;
    if (sh.expand) {
        row = valid ? pos : -1;
        wrow = w;
    } else {
        const int d = valid ? rank_of(sh, e) : 0;
        const uint64_t peers = match_key((uint32_t)d, sh.bits_R, vmask);
        const int owner = peers ? __builtin_ctzll(peers) : 0;
        const bool is_owner = valid && owner == lane;
        if (EARLY_BASES) {
            const int base_d = shfl(base_l, d);
            if (is_owner) row = base_d + (slot - row_base(sh, s) * sh.Nmax);
        } else if (is_owner) {
            row = a.recv_base[d] + a.recv_psum[(int64_t)d * (sh.S + 1) + s] + (slot - row_base(sh, s) * sh.Nmax);
        }
        for (uint64_t m = vmask; m; m &= m - 1) {
            const int k = __builtin_ctzll(m);
            const float wk = __int_as_float(read_lane(__float_as_int(w), k));
            const int ok = read_lane(owner, k);
            if (lane == ok) wrow += wk;
        }
    }
    // Rows outside y never occur for a layout of this topk_idx; drop them.
    return ballot(row >= 0 && (int64_t)row < a.y_rows);
}

template <int CPL>
__global__ void __launch_bounds__(kThreads) k_combine(CombineArgs a) {
    constexpr int G = kRowsPerGroup;
    const Shape &sh = a.sh;
    const int lane = lane_id();
    const int64_t n_tok = (int64_t)sh.S * sh.T;
    const int nchunks = sh.H / 8;  // 16-byte chunks of a bf16 row
    // Work unit = (token, column slice); slices of one token are adjacent so
    // neighbouring waves read neighbouring pieces of the same rows.  More
    // units than resident waves lets early finishers pick up new work instead
    // of idling behind tokens with many rows.
    const int slices = a.slices;
    const int cps = ((nchunks + slices - 1) / slices + kWave - 1) / kWave * kWave;  // chunks per slice
    const int64_t n_units = n_tok * slices;
    const int64_t wave0 = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t unit = wave0; unit < n_units; unit += nwaves) {
        const int64_t g = unit / slices;
        const int c_lo = (int)(unit - g * slices) * cps;
        const int c_hi = min(c_lo + cps, nchunks);
        if (c_lo >= c_hi) continue;
        int row;
        float wrow;
        const uint64_t rows_mask = token_rows<CPL == 1>(a, g, lane, row, wrow);
        const int wbits = __float_as_int(wrow);
        uint16_t *out = a.out + g * sh.H;
        for (int c0 = c_lo; c0 < c_hi; c0 += CPL * kWave) {
            float acc[CPL][8];
#pragma unroll
            for (int i = 0; i < CPL; ++i)
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[i][q] = 0.0f;
            for (uint64_t m = rows_mask; m;) {
                // Up to G rows: issue every load, then the FMAs in row order.
                int rr[G];
                float ww[G];
                int n = 0;
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    rr[j] = -1;
                    ww[j] = 0.0f;
                    if (m) {
                        const int k = __builtin_ctzll(m);
                        m &= m - 1;
                        rr[j] = read_lane(row, k);
                        ww[j] = __int_as_float(read_lane(wbits, k));
                        n = j + 1;
                    }
                }
                u32x4 v[G][CPL];
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    if (j < n) {
                        const uint16_t *yr = a.y + (int64_t)rr[j] * sh.H;
#pragma unroll
                        for (int i = 0; i < CPL; ++i) {
                            const int c = c0 + i * kWave + lane;
                            v[j][i] = c < c_hi ? ld16(yr + (int64_t)c * 8) : u32x4{0u, 0u, 0u, 0u};
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < G; ++j)
                    if (j < n) fma_row<CPL>(acc, v[j], ww[j]);
            }
            // Bias rows of this token, added in fp32 before the rounding.
            for (int bi = 0; bi < 2; ++bi) {
                const uint16_t *bias = bi == 0 ? a.bias0 : a.bias1;
                if (!bias) continue;
                u32x4 bv[CPL];
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    const int c = c0 + i * kWave + lane;
                    bv[i] = c < c_hi ? ld16(bias + g * sh.H + (int64_t)c * 8) : u32x4{0u, 0u, 0u, 0u};
                }
                fma_row<CPL>(acc, bv, 1.0f);
            }
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = c0 + i * kWave + lane;
                if (c < c_hi) {
                    u32x4 o;
#pragma unroll
                    for (int q = 0; q < 4; ++q) o[q] = bf16_rne(acc[i][2 * q]) | (bf16_rne(acc[i][2 * q + 1]) << 16);
                    u32x4 *dst = reinterpret_cast<u32x4 *>(out + (int64_t)c * 8);
#if EP_COMBINE_NT_STORE
                    __builtin_nontemporal_store(o, dst);
#else
                    *dst = o;
#endif
                }
            }
        }
    }
}

template <int CPL>
hipError_t run(const CombineArgs &a, hipStream_t st) {
    const int64_t units = (int64_t)a.sh.S * a.sh.T * a.slices;
    int64_t blocks = (units + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks > EP_COMBINE_MAX_BLOCKS) blocks = EP_COMBINE_MAX_BLOCKS;
    hipLaunchKernelGGL(k_combine<CPL>, dim3((int)blocks), dim3(kThreads), a.sh.expand ? EP_COMBINE_EXPAND_LDS : 0, st,
                       a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const CombineArgs &args, hipStream_t stream) {
    if ((int64_t)args.sh.S * args.sh.T == 0) return hipSuccess;
    CombineArgs a = args;
    const int nchunks = a.sh.H / 8;
    const int cpl = (nchunks + kWave - 1) / kWave <= 1 ? 1 : EP_COMBINE_CPL;
    a.slices = EP_COMBINE_SLICES > 0 ? EP_COMBINE_SLICES : (nchunks + cpl * kWave - 1) / (cpl * kWave);
    if (a.slices > (nchunks + kWave - 1) / kWave) a.slices = (nchunks + kWave - 1) / kWave;
    if (a.slices < 1) a.slices = 1;
    const int need = (a.sh.H / 8 + kWave - 1) / kWave;  // chunks per lane for the whole row
    // Two chunks per lane per pass keeps G*CPL*4 = 64 VGPRs of loads in flight.
    if (need <= 1) return run<1>(a, stream);
    return run<EP_COMBINE_CPL>(a, stream);
}

}  // namespace ep
