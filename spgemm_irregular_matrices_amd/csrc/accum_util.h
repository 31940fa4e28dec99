// Device helpers shared by the LDS accumulators: team-wide scans and sums
// (a team is one wavefront or one work group), and packing of byte flags
// into a bitmap word.
#pragma once

#include "common.h"

namespace sg {

template <int TW>
__device__ __forceinline__ int team_exclusive_scan(int v, int* sh, int* total) {
    if constexpr (TW == kWave) {
        int inc = wave_inclusive_scan(v);
        *total = __shfl(inc, kWave - 1, kWave);
        return inc - v;
    } else {
        return block_exclusive_scan<TW>(v, sh, total);
    }
}

template <int TW>
__device__ __forceinline__ int team_sum(int v, int* sh) {
    if constexpr (TW == kWave) return wave_reduce_sum(v);
    else return block_reduce_sum<TW>(v, sh);
}

// Pack 32 one-byte presence flags (each 0 or 1) into a 32-bit mask.
__device__ __forceinline__ uint32_t pack_flags32(const uint32_t* f) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t x = f[i];
        uint32_t b = (x & 1u) | ((x >> 7) & 2u) | ((x >> 14) & 4u) | ((x >> 21) & 8u);
        m |= b << (4 * i);
    }
    return m;
}

}  // namespace sg
