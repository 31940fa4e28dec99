// Setup phase of Algorithm 3 on the gMAGNUS page: input validation,
// InterOffsets (per-row intermediate-product counts and their prefix sum)
// and ThreshPartition of the rows into heavy rows and light-row bins.
#include "kernels.h"
#include "primitives.h"

namespace sg {

__global__ void k_part_bin_starts(const int64_t* offs, int nb, int64_t nblocks, int64_t n,
                                  int64_t* bin_start) {
    int b = threadIdx.x;
    if (b < nb) bin_start[b] = offs[(int64_t)b * nblocks];
    // the elements placed (all n unless a bin function leaves some out)
    if (b == nb) bin_start[nb] = offs[(int64_t)nb * nblocks];
}

__global__ void k_tile_starts(const int64_t* a, int64_t n, int64_t step, int64_t ntiles,
                              int64_t* out) {
    int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g < ntiles) out[g] = upper_index(a, int64_t(0), n, g * step);
}

// ---------------------------------------------------------------- validation
__global__ void k_validate_rowptr(const int64_t* rp, int64_t n, int64_t nnz, int* flag) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; i <= n; i += stride) {
        int64_t v = rp[i];
        bool bad = (i == 0 && v != 0) || (i == n && v != nnz) || (i < n && rp[i + 1] < v) ||
                   v < 0 || v > nnz;
        if (bad) atomicOr(flag, 1);
    }
}

__global__ void k_validate_cols(const int32_t* col, int64_t nnz, int64_t ncols, int* flag) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    bool bad = false;
    for (; i < nnz; i += stride) {
        int32_t c = col[i];
        bad |= (c < 0) || ((int64_t)c >= ncols);
    }
    if (__ballot(bad) != 0 && lane_id() == 0) atomicOr(flag, 2);
}

void launch_validate(const DevCSR& M, int* flag, hipStream_t st) {
    int64_t blocks = std::min<int64_t>(ceil_div(M.n + 1, 256), 4096);
    hipLaunchKernelGGL(k_validate_rowptr, dim3(grid_1d(blocks)), dim3(256), 0, st, M.rp, M.n,
                       M.nnz, flag);
    SG_LAUNCH_CHECK();
    if (M.nnz > 0) {
        blocks = std::min<int64_t>(ceil_div(M.nnz, 256), 8192);
        hipLaunchKernelGGL(k_validate_cols, dim3(grid_1d(blocks)), dim3(256), 0, st, M.col, M.nnz,
                           M.m, flag);
        SG_LAUNCH_CHECK();
    }
}

// ---------------------------------------------------------------- InterOffsets
struct EntryProducts {
    const int32_t* acol;
    const int64_t* brp;
    __device__ int64_t operator()(int64_t q) const {
        int32_t k = acol[q];
        return brp[k + 1] - brp[k];
    }
};

void entry_prefix(const DevCSR& A, const DevCSR& B, int64_t* S, Arena& ar, hipStream_t st) {
    scan_exclusive(EntryProducts{A.col, B.rp}, A.nnz, S, ar, st);
}

// Sum over A's entries of the square of the entry's product count (its B
// row's length): with the products' sum, the mean B-row length that a
// product sees.
__global__ __launch_bounds__(256) void k_entry_len_sq(const int64_t* S, int64_t nnz, double* out) {
    __shared__ double sh[256 / kWave + 1];
    double acc = 0.0;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < nnz;
         q += (int64_t)gridDim.x * 256) {
        const double l = (double)(S[q + 1] - S[q]);
        acc += l * l;
    }
    acc = block_reduce_sum<256>(acc, sh);
    if (threadIdx.x == 0 && acc != 0.0) atomicAdd(out, acc);
}

void entry_len_sq(const int64_t* S, int64_t nnz, double* out, hipStream_t st) {
    fill<double>(out, 1, 0.0, st);
    if (nnz <= 0) return;
    hipLaunchKernelGGL(k_entry_len_sq, dim3(grid_1d(std::min<int64_t>(ceil_div(nnz, 256), 512))),
                       dim3(256), 0, st, S, nnz, out);
    SG_LAUNCH_CHECK();
}

// ---------------------------------------------------------------- B row spans
// One wavefront per B row: smallest and largest column of the row.
__global__ __launch_bounds__(256) void k_brow_minmax(const int64_t* rp, const int32_t* col,
                                                     int64_t n, int32_t* bmin, int32_t* bmax) {
    int64_t row = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    if (row >= n) return;
    int64_t s = rp[row], e = rp[row + 1];
    int32_t lo = 0x7fffffff, hi = -1;
    for (int64_t q = s + lane_id(); q < e; q += kWave) {
        int32_t c = col[q];
        lo = min(lo, c);
        hi = max(hi, c);
    }
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) {
        lo = min(lo, __shfl_xor(lo, d, kWave));
        hi = max(hi, __shfl_xor(hi, d, kWave));
    }
    if (lane_id() == 0) {
        bmin[row] = lo;
        bmax[row] = hi;
    }
}

void brow_minmax(const DevCSR& B, int32_t* bmin, int32_t* bmax, hipStream_t st) {
    if (B.n <= 0) return;
    int64_t blocks = ceil_div(B.n * kWave, 256);
    hipLaunchKernelGGL(k_brow_minmax, dim3(grid_1d(blocks)), dim3(256), 0, st, B.rp, B.col, B.n,
                       bmin, bmax);
    SG_LAUNCH_CHECK();
}

// ---------------------------------------------------------------- classification
// Per row: u(i), the row's output column span (from the B rows' spans), and
// its bin. Heavy rows (u > tau) are the rows whose intermediate products
// would overflow a local-memory accumulator (Section II-B, Eq. 4).
// Histogram bucket of u >= 0 for the p95 statistic: u < 64 exactly, above
// that 64 buckets per octave (the 6 bits below the leading one).
__device__ __forceinline__ int u_bucket(int64_t u) {
    if (u < 64) return (int)u;
    const int e = 63 - __clzll((unsigned long long)u);
    return 64 + (e - 6) * 64 + (int)((u >> (e - 6)) & 63);
}

// Grid-stride over rows, so the per-block sums below meet few work groups
// at the global counters (same-address atomics serialise at the L2).
constexpr int kClassifyMaxBlocks = 512;

__global__ __launch_bounds__(256) void k_classify_rows(const int64_t* arp, const int32_t* acol,
                                                       int64_t n, const int64_t* S,
                                                       const int32_t* bmin, const int32_t* bmax,
                                                       int64_t tau, uint8_t* bin, int32_t* rowlo,
                                                       int64_t* stats, int32_t* uhist) {
    __shared__ int64_t sh[8];
    __shared__ double shd[8];
    // the block's u histogram, added to the global one once at the end
    __shared__ int hb[kUHistBuckets];
    for (int b = threadIdx.x; b < kUHistBuckets; b += blockDim.x) hb[b] = 0;
    __syncthreads();
    int64_t su = 0, heavy = 0, hprod = 0, c512 = 0, c4k = 0, c32k = 0, mu = 0, alight = 0;
    double u2 = 0.0;
    for (int64_t base = (int64_t)blockIdx.x * 256; base < n; base += (int64_t)gridDim.x * 256) {
        const int64_t i = base + threadIdx.x;
        const bool in = i < n;
        int64_t u = 0;
        if (in) {
            const int64_t a0 = arp[i], a1 = arp[i + 1];
            u = S[a1] - S[a0];
            int b;
            if (u == 0) {
                b = RB_EMPTY;
            } else if (u > tau) {
                b = RB_HEAVY;
                heavy += 1;
                hprod += u;
            } else if (u <= kThreadMaxItems[2]) {
                b = u <= kThreadMaxItems[0] ? RB_T8 : (u <= kThreadMaxItems[1] ? RB_T16 : RB_T32);
                alight += a1 - a0;
            } else {
                alight += a1 - a0;
                // the row's B column range, eight entries' loads in flight
                int32_t lo = 0x7fffffff, hi = -1;
                for (int64_t qb = a0; qb < a1; qb += 8) {
                    int32_t k[8];
#pragma unroll
                    for (int t = 0; t < 8; ++t) k[t] = qb + t < a1 ? acol[qb + t] : -1;
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        if (k[t] >= 0) {
                            lo = min(lo, bmin[k[t]]);
                            hi = max(hi, bmax[k[t]]);
                        }
                    }
                }
                const int64_t span = (int64_t)hi - lo + 1;
                rowlo[i] = lo;
                if (span <= kWinSmall) {
                    b = RB_WIN64;
                } else if (span <= kWinLarge) {
                    b = RB_WIN1024;
                } else if (u <= kHashMaxItems[0]) {
                    b = RB_H128;
                } else if (u <= kHashMaxItems[1]) {
                    b = RB_H512;
                } else if (u <= kHashMaxItems[2]) {
                    b = RB_H2048;
                } else {
                    b = RB_H8192;
                }
            }
            bin[i] = (uint8_t)b;
            // the structural statistics of the rows' products: F_h counts and
            // the sum of squares (for the coefficient of variation)
            su += u;
            c512 += u <= 512;
            c4k += u <= 4096;
            c32k += u <= 32768;
            u2 += (double)u * (double)u;
            mu = u > mu ? u : mu;
        }
        // the u histogram: the lanes of a wave that share a bucket add once
        // (a banded matrix puts nearly every row in one bucket)
        const int bk = in ? u_bucket(u) : -1;
        uint64_t act = __ballot(bk >= 0);
        while (act) {
            const int leader = __ffsll((unsigned long long)act) - 1;
            const int lb = __shfl(bk, leader);
            const uint64_t m = __ballot(bk == lb);
            if (lane_id() == leader) atomicAdd(&hb[lb], __popcll(m));
            act &= ~m;
        }
    }
    su = block_reduce_sum<256>(su, sh);
    heavy = block_reduce_sum<256>(heavy, sh);
    hprod = block_reduce_sum<256>(hprod, sh);
    c512 = block_reduce_sum<256>(c512, sh);
    c4k = block_reduce_sum<256>(c4k, sh);
    c32k = block_reduce_sum<256>(c32k, sh);
    u2 = block_reduce_sum<256>(u2, shd);
    alight = block_reduce_sum<256>(alight, sh);
    // block_reduce_sum ends with a barrier: every wave's LDS histogram adds are in
    for (int b = threadIdx.x; b < kUHistBuckets; b += blockDim.x)
        if (hb[b]) atomicAdd(&uhist[b], hb[b]);
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) {
        const int64_t o = __shfl_xor(mu, d, kWave);
        mu = mu > o ? mu : o;
    }
    if (lane_id() == 0 && mu > 0)
        atomicMax((unsigned long long*)&stats[1], (unsigned long long)mu);
    if (threadIdx.x == 0) {
        atomicAdd((unsigned long long*)&stats[0], (unsigned long long)su);
        atomicAdd((unsigned long long*)&stats[2], (unsigned long long)heavy);
        atomicAdd((unsigned long long*)&stats[3], (unsigned long long)hprod);
        atomicAdd((unsigned long long*)&stats[4], (unsigned long long)c512);
        atomicAdd((unsigned long long*)&stats[5], (unsigned long long)c4k);
        atomicAdd((unsigned long long*)&stats[6], (unsigned long long)c32k);
        atomicAdd((double*)&stats[7], u2);
        atomicAdd((unsigned long long*)&stats[8], (unsigned long long)alight);
    }
}

// Sum of cnt[perm[j]] over j < n, added into *out (the light rows' output
// entries, for the light path's algorithmic bytes).
__global__ __launch_bounds__(256) void k_sum_rows(const int32_t* perm, int64_t n,
                                                  const int64_t* cnt, int64_t* out) {
    __shared__ int64_t sh[8];
    int64_t s = 0;
    for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < n;
         j += (int64_t)gridDim.x * 256)
        s += cnt[perm[j]];
    s = block_reduce_sum<256>(s, sh);
    if (threadIdx.x == 0 && s) atomicAdd((unsigned long long*)out, (unsigned long long)s);
}

void sum_rows(const int32_t* perm, int64_t n, const int64_t* cnt, int64_t* out, hipStream_t st) {
    fill<int64_t>(out, 1, 0, st);
    if (n <= 0) return;
    hipLaunchKernelGGL(k_sum_rows, dim3(grid_1d(std::min<int64_t>(ceil_div(n, 256), 256))),
                       dim3(256), 0, st, perm, n, cnt, out);
    SG_LAUNCH_CHECK();
}

struct RowBinOf {
    const uint8_t* bin;
    __device__ int operator()(int64_t i) const { return bin[i]; }
};

void classify_rows(const DevCSR& A, const int64_t* S, const int32_t* bmin, const int32_t* bmax,
                   int64_t tau, int32_t* rowlo, int32_t* perm, int64_t* bin_start,
                   int64_t* stats, int32_t* uhist, Arena& ar, hipStream_t st) {
    uint8_t* bin = ar.get<uint8_t>("row_bin", (size_t)A.n + 1);
    fill<int64_t>(stats, kRowStats, 0, st);
    fill<int32_t>(uhist, kUHistBuckets, 0, st);
    if (A.n > 0) {
        hipLaunchKernelGGL(k_classify_rows,
                           dim3(grid_1d(std::min<int64_t>(ceil_div(A.n, 256), kClassifyMaxBlocks))),
                           dim3(256), 0, st,
                           A.rp, A.col, A.n, S, bmin, bmax, tau, bin, rowlo, stats, uhist);
        SG_LAUNCH_CHECK();
    }
    partition(RowBinOf{bin}, A.n, RB_COUNT, perm, (int32_t*)nullptr, bin_start, ar, st);
}

}  // namespace sg
