// Shared definitions of the HIP library (device helpers, launch helpers).
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

#include <stdexcept>
#include <string>

namespace sg {

constexpr int kWave = 64;  // CDNA wavefront width

// A HIP call failed; carried to the C ABI as SPGEMM_ERR_HIP.
struct HipError : std::runtime_error {
    hipError_t code;
    HipError(hipError_t c, const char* what) : std::runtime_error(what), code(c) {}
};
// Workspace could not be allocated; carried as SPGEMM_ERR_OUT_OF_MEMORY.
struct OomError : std::runtime_error {
    using std::runtime_error::runtime_error;
};
// A size limit of the library was exceeded; carried as SPGEMM_ERR_OVERFLOW.
struct OverflowError : std::runtime_error {
    using std::runtime_error::runtime_error;
};
// A call without allocation needs more workspace than its fixed scratch
// buffer holds; carried as SPGEMM_ERR_SCRATCH_LIMIT.
struct ScratchError : std::runtime_error {
    using std::runtime_error::runtime_error;
};
// A debug self-check found a broken internal invariant; carried as
// SPGEMM_ERR_INTERNAL.
struct InternalError : std::runtime_error {
    using std::runtime_error::runtime_error;
};

#define SG_HIP(call)                                                              \
    do {                                                                          \
        hipError_t _e = (call);                                                   \
        if (_e != hipSuccess) throw ::sg::HipError(_e, #call);                    \
    } while (0)

#define SG_LAUNCH_CHECK() SG_HIP(hipGetLastError())

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int64_t floor_pow2(int64_t x) {
    int64_t p = 1;
    while (p * 2 <= x) p *= 2;
    return p;
}
inline int64_t ceil_pow2(int64_t x) {
    int64_t p = 1;
    while (p < x) p *= 2;
    return p;
}
inline int ilog2(int64_t x) {
    int l = 0;
    while ((int64_t(1) << (l + 1)) <= x) ++l;
    return l;
}

// Grid size guard: every launch in the library goes through this.
inline unsigned grid_1d(int64_t blocks) {
    if (blocks < 1) blocks = 1;
    if (blocks > 0x7fffffffLL) throw OverflowError("grid size exceeds the HIP limit");
    return (unsigned)blocks;
}

// ----------------------------------------------------------------------------
// device helpers
// ----------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Exclusive prefix count of set bits below this lane in a 64-bit ballot.
__device__ __forceinline__ int lane_prefix(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Inclusive scan of 32-bit integers across the 64 lanes with DPP moves:
// shifts by 1, 2, 4 and 8 lanes inside each row of 16 (lanes shifted in
// from outside the row add 0), then row 0's total into row 1 and row 2's
// into row 3 (row_bcast:15), then lane 31's total into rows 2 and 3
// (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_scan_i32(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// Sum over each row of 16 lanes (DPP shifts by 1, 2, 4 and 8 inside the
// row); the row's last lane (lane % 16 == 15) receives the row's total.
__device__ __forceinline__ int row16_sum_i32(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    return x;
}

// Inclusive scan across the 64 lanes of a wavefront.
template <class T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
    if constexpr (sizeof(T) == 4 && std::is_integral<T>::value) {
        return (T)wave_inclusive_scan_i32((int)v);
    } else {
        const int l = lane_id();
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            T o = __shfl_up(v, d, kWave);
            if (l >= d) v += o;
        }
        return v;
    }
}

// Orders this wave's LDS accesses around it (a wave's LDS operations run in
// issue order; this keeps the compiler from moving them across).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <class T>
__device__ __forceinline__ T wave_reduce_sum(T v) {
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

// Exclusive scan over a whole block of NT threads; `sh` holds NT/64 values.
// Returns this thread's exclusive prefix; *total receives the block total.
template <int NT, class T>
__device__ __forceinline__ T block_exclusive_scan(T v, T* sh, T* total) {
    constexpr int NW = NT / kWave;
    const int w = threadIdx.x / kWave;
    T inc = wave_inclusive_scan(v);
    if (lane_id() == kWave - 1) sh[w] = inc;
    __syncthreads();
    if (w == 0) {
        T s = lane_id() < NW ? sh[lane_id()] : T(0);
        T si = wave_inclusive_scan(s);
        if (lane_id() < NW) sh[lane_id()] = si - s;
        if (lane_id() == NW - 1) sh[NW] = si;
    }
    __syncthreads();
    T res = sh[w] + inc - v;
    *total = sh[NW];
    __syncthreads();
    return res;
}

template <int NT, class T>
__device__ __forceinline__ T block_reduce_sum(T v, T* sh) {
    constexpr int NW = NT / kWave;
    const int w = threadIdx.x / kWave;
    T s = wave_reduce_sum(v);
    if (lane_id() == 0) sh[w] = s;
    __syncthreads();
    T r = 0;
    if (threadIdx.x == 0) {
        for (int i = 0; i < NW; ++i) r += sh[i];
        sh[NW] = r;
    }
    __syncthreads();
    r = sh[NW];
    __syncthreads();
    return r;
}

// Largest index j in [lo, hi) with a[j] <= x, given a sorted and a[lo] <= x.
template <class T>
__device__ __forceinline__ int64_t upper_index(const T* a, int64_t lo, int64_t hi, T x) {
    while (hi - lo > 1) {
        int64_t mid = lo + ((hi - lo) >> 1);
        if (a[mid] <= x) lo = mid; else hi = mid;
    }
    return lo;
}

}  // namespace sg
