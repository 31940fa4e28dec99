// Device-wide primitives: fill, exclusive prefix sum (int64) and a stable
// multi-bin partition. The gMAGNUS page (Algorithm 3 and Section III-A)
// uses a device-wide prefix sum for InterOffsets, Histogram and C.rowPtr,
// and a flagged partition (ThreshPartition) to split rows and chunks into
// heavy and light groups; these are hand-written wave64 versions.
#pragma once

#include "arena.h"
#include "common.h"

namespace sg {

// ---------------------------------------------------------------- fill
template <class T>
__global__ void k_fill(T* p, int64_t n, T v) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) p[i] = v;
}

template <class T>
inline void fill(T* p, int64_t n, T v, hipStream_t st) {
    if (n <= 0) return;
    int64_t blocks = ceil_div(n, 256);
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(k_fill<T>, dim3(grid_1d(blocks)), dim3(256), 0, st, p, n, v);
    SG_LAUNCH_CHECK();
}

template <class T>
__global__ void k_copy(T* dst, const T* src, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) dst[i] = src[i];
}

template <class T>
inline void copy(T* dst, const T* src, int64_t n, hipStream_t st) {
    if (n <= 0) return;
    int64_t blocks = ceil_div(n, 256);
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(k_copy<T>, dim3(grid_1d(blocks)), dim3(256), 0, st, dst, src, n);
    SG_LAUNCH_CHECK();
}

// ---------------------------------------------------------------- scan
constexpr int kScanNT = 256;
constexpr int kScanIPT = 16;
constexpr int kScanTile = kScanNT * kScanIPT;

struct LoadI64 {
    const int64_t* p;
    __device__ int64_t operator()(int64_t i) const { return p[i]; }
};

template <class F>
__global__ __launch_bounds__(kScanNT) void k_scan_reduce(F f, int64_t n, int64_t* tile_sums) {
    __shared__ int64_t sh[kScanNT / kWave + 1];
    int64_t base = (int64_t)blockIdx.x * kScanTile;
    int64_t s = 0;
#pragma unroll 4
    for (int j = 0; j < kScanIPT; ++j) {
        int64_t i = base + (int64_t)j * kScanNT + threadIdx.x;
        if (i < n) s += f(i);
    }
    s = block_reduce_sum<kScanNT>(s, sh);
    if (threadIdx.x == 0) tile_sums[blockIdx.x] = s;
}

// out[i] = sum_{i' < i} f(i') for i in [0, n], so out[n] is the total.
// `tile_off` holds the exclusive prefix of the tile sums. T: the output
// type (the caller guarantees that the total fits it). The tile passes
// through LDS, so that global loads and stores are coalesced (consecutive
// lanes, consecutive elements) while each thread scans 16 consecutive
// elements; one padding word every 32 keeps the per-thread reads apart in
// the banks. The tile holds values of the output type (every element and
// prefix fits it), so a 32-bit scan takes half the LDS and twice the
// resident groups.
template <class F, class T = int64_t>
__global__ __launch_bounds__(kScanNT) void k_scan_apply(F f, int64_t n, const int64_t* tile_off,
                                                        T* out) {
    __shared__ int64_t sh[kScanNT / kWave + 1];
    __shared__ T tile[kScanTile + kScanTile / 32];
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
#pragma unroll 4
    for (int j = 0; j < kScanIPT; ++j) {
        const int idx = j * kScanNT + threadIdx.x;
        const int64_t i = base + idx;
        tile[idx + (idx >> 5)] = (T)(i < n ? f(i) : 0);
    }
    __syncthreads();
    int64_t v[kScanIPT];
    int64_t s = 0;
#pragma unroll
    for (int j = 0; j < kScanIPT; ++j) {
        const int idx = threadIdx.x * kScanIPT + j;
        v[j] = tile[idx + (idx >> 5)];
        s += v[j];
    }
    int64_t tot;
    // (the scan's barriers also order the reads above before the writes below)
    int64_t pre = block_exclusive_scan<kScanNT>(s, sh, &tot) + tile_off[blockIdx.x];
#pragma unroll
    for (int j = 0; j < kScanIPT; ++j) {
        const int idx = threadIdx.x * kScanIPT + j;
        tile[idx + (idx >> 5)] = (T)pre;
        pre += v[j];
        if (base + idx == n - 1) out[n] = (T)pre;
    }
    __syncthreads();
#pragma unroll 4
    for (int j = 0; j < kScanIPT; ++j) {
        const int idx = j * kScanNT + threadIdx.x;
        const int64_t i = base + idx;
        if (i < n) out[i] = tile[idx + (idx >> 5)];
    }
}

// Exclusive scan of f over [0, n) into out[0..n]. `out` may alias the array
// that f reads only when each element is read by the same tile that writes it
// (true for an identity load of `out` itself).
template <class F, class T = int64_t>
void scan_exclusive(F f, int64_t n, T* out, Arena& ar, hipStream_t st, int depth = 0) {
    if (n <= 0) {
        fill<T>(out, 1, 0, st);
        return;
    }
    int64_t tiles = ceil_div(n, kScanTile);
    int64_t* ts = ar.get<int64_t>("scan_tiles_" + std::to_string(depth), (size_t)tiles + 1);
    if (tiles == 1) {
        fill<int64_t>(ts, 1, 0, st);
    } else {
        hipLaunchKernelGGL(k_scan_reduce<F>, dim3(grid_1d(tiles)), dim3(kScanNT), 0, st, f, n, ts);
        SG_LAUNCH_CHECK();
        scan_exclusive(LoadI64{ts}, tiles, ts, ar, st, depth + 1);
    }
    auto apply = k_scan_apply<F, T>;  // (a template-id with a comma cannot be a macro argument)
    hipLaunchKernelGGL(apply, dim3(grid_1d(tiles)), dim3(kScanNT), 0, st, f, n, ts, out);
    SG_LAUNCH_CHECK();
}

// ---------------------------------------------------------------- tile starts
// out[g] = largest j in [0, n) with a[j] <= g*step, for g in [0, ntiles): the
// first row (or entry) of every static tile of a flattened range. One
// independent search per thread, so the search latency is paid in parallel
// instead of at the start of every tile.
__global__ void k_tile_starts(const int64_t* a, int64_t n, int64_t step, int64_t ntiles,
                              int64_t* out);

inline void tile_starts(const int64_t* a, int64_t n, int64_t step, int64_t ntiles, int64_t* out,
                        hipStream_t st) {
    if (ntiles <= 0) return;
    hipLaunchKernelGGL(k_tile_starts, dim3(grid_1d(ceil_div(ntiles, 256))), dim3(256), 0, st, a, n,
                       step, ntiles, out);
    SG_LAUNCH_CHECK();
}

// ---------------------------------------------------------------- partition
// Stable partition of items [0, n) into bins 0..nb-1 (bin order, then item
// order); an item whose bin is -1 is left out. perm[pos] = item,
// pos_of[item] = pos (pos_of may be null), bin_start[0..nb] = first
// position of each bin (bin_start[nb] = the items placed, n if none is
// left out).
constexpr int kPartNT = 256;
constexpr int kPartIPT = 8;
constexpr int kPartTile = kPartNT * kPartIPT;
constexpr int kMaxBins = 16;

template <class BinF>
__global__ __launch_bounds__(kPartNT) void k_part_count(BinF bf, int64_t n, int nb,
                                                         int64_t nblocks, int64_t* counts) {
    __shared__ int h[kMaxBins];
    if (threadIdx.x < kMaxBins) h[threadIdx.x] = 0;
    __syncthreads();
    int64_t base = (int64_t)blockIdx.x * kPartTile;
    for (int j = 0; j < kPartIPT; ++j) {
        int64_t i = base + (int64_t)j * kPartNT + threadIdx.x;
        if (i < n) {
            const int b = bf(i);  // bin -1: the element is left out
            if (b >= 0) atomicAdd(&h[b], 1);
        }
    }
    __syncthreads();
    if (threadIdx.x < nb) counts[(int64_t)threadIdx.x * nblocks + blockIdx.x] = h[threadIdx.x];
}

template <class BinF>
__global__ __launch_bounds__(kPartNT) void k_part_scatter(BinF bf, int64_t n, int nb,
                                                           int64_t nblocks, const int64_t* offs,
                                                           int32_t* perm, int32_t* pos_of) {
    constexpr int NW = kPartNT / kWave;
    __shared__ int64_t run[kMaxBins];
    __shared__ int wcnt[kMaxBins][NW];
    const int w = threadIdx.x / kWave;
    if (threadIdx.x < nb) run[threadIdx.x] = offs[(int64_t)threadIdx.x * nblocks + blockIdx.x];
    __syncthreads();
    int64_t base = (int64_t)blockIdx.x * kPartTile;
    for (int j = 0; j < kPartIPT; ++j) {
        int64_t i = base + (int64_t)j * kPartNT + threadIdx.x;
        int b = i < n ? bf(i) : -1;
        int myrank = 0;
        for (int bb = 0; bb < nb; ++bb) {
            uint64_t m = __ballot(b == bb);
            if (lane_id() == 0) wcnt[bb][w] = __popcll(m);
            if (b == bb) myrank = lane_prefix(m);
        }
        __syncthreads();
        if (b >= 0) {
            int64_t dest = run[b] + myrank;
            for (int ww = 0; ww < w; ++ww) dest += wcnt[b][ww];
            perm[dest] = (int32_t)i;
            if (pos_of) pos_of[i] = (int32_t)dest;
        }
        __syncthreads();
        if (threadIdx.x < nb) {
            int64_t s = 0;
            for (int ww = 0; ww < NW; ++ww) s += wcnt[threadIdx.x][ww];
            run[threadIdx.x] += s;
        }
        __syncthreads();
    }
}

__global__ void k_part_bin_starts(const int64_t* offs, int nb, int64_t nblocks, int64_t n,
                                  int64_t* bin_start);

template <class BinF>
void partition(BinF bf, int64_t n, int nb, int32_t* perm, int32_t* pos_of, int64_t* bin_start,
               Arena& ar, hipStream_t st) {
    if (nb > kMaxBins) throw std::logic_error("too many bins");
    if (n >= (int64_t(1) << 31)) throw OverflowError("partition of more than 2^31 items");
    int64_t nblocks = n > 0 ? ceil_div(n, kPartTile) : 1;
    int64_t* counts = ar.get<int64_t>("part_counts", (size_t)(nb * nblocks + 1));
    if (n > 0) {
        hipLaunchKernelGGL(k_part_count<BinF>, dim3(grid_1d(nblocks)), dim3(kPartNT), 0, st, bf, n,
                           nb, nblocks, counts);
        SG_LAUNCH_CHECK();
    } else {
        fill<int64_t>(counts, nb * nblocks, 0, st);
    }
    scan_exclusive(LoadI64{counts}, nb * nblocks, counts, ar, st);
    if (n > 0) {
        hipLaunchKernelGGL(k_part_scatter<BinF>, dim3(grid_1d(nblocks)), dim3(kPartNT), 0, st, bf,
                           n, nb, nblocks, counts, perm, pos_of);
        SG_LAUNCH_CHECK();
    }
    hipLaunchKernelGGL(k_part_bin_starts, dim3(1), dim3(64), 0, st, counts, nb, nblocks, n,
                       bin_start);
    SG_LAUNCH_CHECK();
}

}  // namespace sg
