// ep_device.h -- wavefront primitives and small helpers shared by the libep
// kernels (CDNA4 / gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Lanes strictly below / strictly above this one.
__device__ __forceinline__ uint64_t mask_lt(int lane) { return (lane == 0) ? 0ull : (~0ull >> (64 - lane)); }
__device__ __forceinline__ uint64_t mask_gt(int lane) { return (lane == 63) ? 0ull : (~0ull << (lane + 1)); }

// popcount(m & lanes below me), the per-lane exclusive prefix of a ballot.
__device__ __forceinline__ int prefix_count(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ int popc(uint64_t m) { return __popcll(m); }

// Wave-uniform value of `v` held by lane `src` (src must be wave-uniform).
__device__ __forceinline__ int read_lane(int v, int src) { return __builtin_amdgcn_readlane(v, src); }
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Value of `v` held by lane `src` (src may differ per lane): ds_bpermute.
__device__ __forceinline__ int shfl(int v, int src) { return __builtin_amdgcn_ds_bpermute(src << 2, v); }

// Mask of the lanes in `active` whose `nbits`-wide key equals this lane's key:
// one ballot per key bit, keeping the lanes that agree on every bit.
__device__ __forceinline__ uint64_t match_key(uint32_t key, int nbits, uint64_t active) {
    uint64_t m = active;
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1u;
        const uint64_t bal = ballot(bit);
        m &= bit ? bal : ~bal;
    }
    return m;
}

__device__ __forceinline__ int bits_for(int n) {  // smallest b with (1 << b) >= n
    int b = 0;
    while ((1 << b) < n) ++b;
    return b;
}

// 16-byte vector used for all row copies.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// LDS of one CDNA4 compute unit, and the dynamic LDS a workgroup requests so
// that at most `groups` such workgroups are resident on a CU at once (the
// kernel never touches the extra bytes): caps the waves in flight for streams
// that measured faster with fewer of them.  Below the 64 KiB per-workgroup
// limit for groups >= 2.
constexpr int kLdsPerCU = 160 * 1024;
constexpr int lds_to_cap_residency(int groups) { return kLdsPerCU / (groups + 1) + 1024; }
static_assert(lds_to_cap_residency(2) <= 65536 && 2 * lds_to_cap_residency(2) <= kLdsPerCU &&
                  3 * lds_to_cap_residency(2) > kLdsPerCU, "two workgroups per CU");
static_assert(3 * lds_to_cap_residency(3) <= kLdsPerCU && 4 * lds_to_cap_residency(3) > kLdsPerCU,
              "three workgroups per CU");

}  // namespace ep
