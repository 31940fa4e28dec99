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

// Exclusive scan of a block whose values sit in its first NA threads (NA a
// multiple of 64; the other threads hold 0) with one barrier: wave scans,
// each wave's total in sh[w], then every thread adds the totals of the
// waves before its own. *total receives the sum. sh holds NA/64 values and
// must not be rewritten before every thread has returned (the next barrier).
template <int NA>
__device__ __forceinline__ int block_scan_first(int v, int* sh, int* total) {
    constexpr int NW = NA / kWave;
    static_assert(NA % kWave == 0, "whole waves");
    const int w = threadIdx.x / kWave;
    int inc = 0;
    if (w < NW) {
        inc = wave_inclusive_scan_i32(v);
        if (lane_id() == kWave - 1) sh[w] = inc;
    }
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int t = sh[i];
        before += i < w ? t : 0;
        tot += t;
    }
    *total = tot;
    return w < NW ? before + inc - v : tot;
}

// Exclusive scan over a team of TW threads: a wave scan for one wavefront,
// else block_scan_first (one barrier).
template <int TW>
__device__ __forceinline__ int team_scan_fast(int v, int* sh, int* total) {
    if constexpr (TW == kWave) return team_exclusive_scan<TW>(v, sh, total);
    else return block_scan_first<TW>(v, sh, total);
}

template <int TW>
__device__ __forceinline__ int team_sum(int v, int* sh) {
    if constexpr (TW == kWave) return wave_reduce_sum(v);
    else return block_reduce_sum<TW>(v, sh);
}

// Bytes of LDS wave_rank_emit<KPT> needs for a chunk of W columns.
__host__ __device__ constexpr int wave_rank_lds(int kpt, int64_t W) {
    return 12 * kWave * kpt + 8 * (W >= 4096 ? (int)(W >> 11) : 1);
}

// One wave's item of at most 64*KPT products in a chunk of W columns (W a
// power of two, 32 <= W <= 65536; idx = column inside the chunk, ~0 for no
// product). The distinct columns are ranked through a two-level bitmap, so
// that the work follows the products rather than W: a top bitmap with one
// bit per 64-column bucket (max(1, W/2048) words), a prefix over its words
// that numbers the nonempty buckets in column order, a 64-bit mask of the
// columns of every nonempty bucket and a prefix over the masks' popcounts.
// A column's rank is its bucket's prefix plus the columns below it in its
// mask. With `numeric`, the values are summed at their rank and the chunk is
// written sorted: oc[r] = lo + column, ov[r] = sum. Returns the number of
// distinct columns. LDS: `lds` (wave_rank_lds bytes, 8-byte aligned) and
// scol (64*KPT 16-bit places).
template <int KPT>
__device__ __forceinline__ int wave_rank_emit(const uint32_t (&idx)[KPT], const double (&v)[KPT],
                                              int W, void* lds, double* vals, uint16_t* scol,
                                              int32_t lo, int32_t* oc, double* ov, bool numeric) {
    constexpr int CAP = kWave * KPT;
    const int lane = lane_id();
    const int ntw = W >= 4096 ? (W >> 11) : 1;  // top words: at most 32
    unsigned long long* bm = (unsigned long long*)lds;  // CAP masks
    int* bpre = (int*)(bm + CAP);                       // CAP bucket prefixes
    uint32_t* top = (uint32_t*)(bpre + CAP);            // ntw words
    int* tpre = (int*)(top + ntw);                      // ntw word prefixes
    if (lane < ntw) top[lane] = 0u;
#pragma unroll
    for (int k = 0; k < KPT; ++k) bm[k * kWave + lane] = 0ull;
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
        if (idx[k] < (uint32_t)W) {
            const uint32_t b = idx[k] >> 6;
            atomicOr(&top[b >> 5], 1u << (b & 31));
        }
    }
    wave_lds_sync();
    int nb;
    {
        const int pc = lane < ntw ? __popc(top[lane]) : 0;
        const int inc = wave_inclusive_scan(pc);
        if (lane < ntw) tpre[lane] = inc - pc;
        nb = __shfl(inc, kWave - 1, kWave);
    }
    wave_lds_sync();
    int cb[KPT];
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
        cb[k] = -1;
        if (idx[k] < (uint32_t)W) {
            const uint32_t b = idx[k] >> 6, w = b >> 5;
            cb[k] = tpre[w] + __popc(top[w] & ((1u << (b & 31)) - 1u));
            atomicOr(&bm[cb[k]], 1ull << (idx[k] & 63));
        }
    }
    wave_lds_sync();
    int nnz;
    {
        // lane l takes buckets l*KPT .. l*KPT + KPT - 1 (nb <= CAP of them)
        int pc = 0;
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            const int c = lane * KPT + k;
            if (c < nb) pc += __popcll(bm[c]);
        }
        const int inc = wave_inclusive_scan(pc);
        nnz = __shfl(inc, kWave - 1, kWave);
        int pre = inc - pc;
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            const int c = lane * KPT + k;
            if (c < nb) {
                bpre[c] = pre;
                pre += __popcll(bm[c]);
            }
            if (numeric) vals[k * kWave + lane] = 0.0;  // CAP places >= nnz
        }
    }
    wave_lds_sync();
    if (!numeric) return nnz;
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
        if (cb[k] >= 0) {
            const int r = bpre[cb[k]] + __popcll(bm[cb[k]] & ((1ull << (idx[k] & 63)) - 1ull));
            atomicAdd(&vals[r], v[k]);
            scol[r] = (uint16_t)idx[k];
        }
    }
    wave_lds_sync();
    for (int r = lane; r < nnz; r += kWave) {
        oc[r] = lo + scol[r];
        ov[r] = vals[r];
    }
    return nnz;
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
