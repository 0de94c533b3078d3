// ep_combine.hip -- weighted top-k reduction of expert outputs back to token
// order (the combine reduce epilogue of DeepEP v2, "Add unordered hybrid
// kernels for transports without ordered delivery" (PR #732), section
// Changes).
//
// out[s][t] = bf16(sum over valid lanes k, ascending, of w[s][t][k] * Y),
// accumulated in fp32 with fused multiply-adds and rounded to nearest-even
// once.  In the compact layout Y is the receive row that the owner lane of the
// lane's rank was given (recv_base[d] + recv_psum[d][s] + slot - s*Nmax), so
// lanes sharing a rank weight the same row; in the expand layout Y is the
// lane's own row expand_pos[s][t][k].
//
// The work is an HBM stream with about one FMA per 2 bytes read, far below
// the MFMA ridge, so it runs on the vector ALUs: one wavefront per token,
// 16-byte loads of 8 bf16 per lane, two expert rows in flight per step.
#include "ep_device.h"
#include "ep_kernels.h"

namespace ep {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;  // quiet NaN
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int CPL>
__device__ __forceinline__ void fma_rows(float (&acc)[CPL][8], const u32x4 (&v)[CPL], float w) {
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

template <int CPL>
__global__ void __launch_bounds__(kThreads) k_combine(CombineArgs a) {
    const Shape &sh = a.sh;
    const int lane = lane_id();
    const int64_t n_tok = (int64_t)sh.S * sh.T;
    const int nchunks = sh.H / 8;  // 16-byte chunks of a bf16 row
    const int64_t wave0 = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t g = wave0; g < n_tok; g += nwaves) {
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
        const uint64_t vmask = ballot(valid);
        int row = -1;
        if (sh.expand) {
            row = valid ? pos : -1;
        } else {
            // The owner of a rank is its lowest valid lane; its slot names the row.
            const int d = valid ? e / sh.El : 0;
            const uint64_t peers = match_key((uint32_t)d, sh.bits_R, vmask);
            const int owner = peers ? __builtin_ctzll(peers) : 0;
            const int owner_slot = shfl(slot, owner);
            if (valid) row = a.recv_base[d] + a.recv_psum[(int64_t)d * (sh.S + 1) + s] + (owner_slot - s * sh.Nmax);
        }
        // Rows outside y never occur for a layout of this topk_idx; drop them.
        const uint64_t use = vmask & ballot(row >= 0 && (int64_t)row < a.y_rows);
        const int wbits = __float_as_int(w);
        uint16_t *out = a.out + g * sh.H;
        for (int c0 = 0; c0 < nchunks; c0 += CPL * kWave) {
            float acc[CPL][8];
#pragma unroll
            for (int i = 0; i < CPL; ++i)
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[i][q] = 0.0f;
            uint64_t m = use;
            while (m) {
                const int k0 = __builtin_ctzll(m);
                m &= m - 1;
                const int r0 = read_lane(row, k0);
                const float w0 = __int_as_float(read_lane(wbits, k0));
                const uint16_t *y0 = a.y + (int64_t)r0 * sh.H;
                u32x4 v0[CPL], v1[CPL];
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    const int c = c0 + i * kWave + lane;
                    if (c < nchunks) v0[i] = ld16(y0 + (int64_t)c * 8);
                    else v0[i] = u32x4{0u, 0u, 0u, 0u};
                }
                if (m) {
                    const int k1 = __builtin_ctzll(m);
                    m &= m - 1;
                    const int r1 = read_lane(row, k1);
                    const float w1 = __int_as_float(read_lane(wbits, k1));
                    const uint16_t *y1 = a.y + (int64_t)r1 * sh.H;
#pragma unroll
                    for (int i = 0; i < CPL; ++i) {
                        const int c = c0 + i * kWave + lane;
                        if (c < nchunks) v1[i] = ld16(y1 + (int64_t)c * 8);
                        else v1[i] = u32x4{0u, 0u, 0u, 0u};
                    }
                    fma_rows<CPL>(acc, v0, w0);
                    fma_rows<CPL>(acc, v1, w1);
                } else {
                    fma_rows<CPL>(acc, v0, w0);
                }
            }
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = c0 + i * kWave + lane;
                if (c < nchunks) {
                    u32x4 o;
#pragma unroll
                    for (int q = 0; q < 4; ++q) o[q] = bf16_rne(acc[i][2 * q]) | (bf16_rne(acc[i][2 * q + 1]) << 16);
                    *reinterpret_cast<u32x4 *>(out + (int64_t)c * 8) = o;
                }
            }
        }
    }
}

template <int CPL>
hipError_t run(const CombineArgs &a, hipStream_t st) {
    const int64_t n_tok = (int64_t)a.sh.S * a.sh.T;
    int64_t blocks = (n_tok + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(k_combine<CPL>, dim3((int)blocks), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t stream) {
    if ((int64_t)a.sh.S * a.sh.T == 0) return hipSuccess;
    const int need = (a.sh.H / 8 + kWave - 1) / kWave;  // chunks per lane for the whole row
    // At most 8 chunks (64 fp32 accumulators) per lane per pass.
    if (need <= 1) return run<1>(a, stream);
    if (need <= 2) return run<2>(a, stream);
    if (need <= 4) return run<4>(a, stream);
    if (need <= 7 || need == 14) return run<7>(a, stream);
    return run<8>(a, stream);
}

}  // namespace ep
