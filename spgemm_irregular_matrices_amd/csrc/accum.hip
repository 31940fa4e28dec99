// Local-memory accumulators (gMAGNUS page, Section III-E).
//
// * Hash accumulator, for light rows of C (and light chunks too wide for a
//   bitmap): an LDS hash map keyed by column (multiplicative hashing,
//   linear probing, at least two slots per item element, i.e. alpha = 2);
//   the occupied slots are compacted and bitonic-sorted to emit the row
//   with ascending columns.
// * Bitmap-rank accumulator, for light chunks of C-hat-reord: after the
//   multisplit every chunk spans a bounded column width, so a one-bit-per-
//   column bitmap fits in LDS; a prefix sum over its word popcounts ranks
//   the present columns, values are summed at their rank, and the chunk
//   comes out sorted without a sort.
// * Dense window accumulator, for heavy chunks of the last multisplit level
//   and for light rows whose output columns fall in a short window (the
//   "shortened dense accumulator" of banded matrices, Section II-B): an LDS
//   array over the window plus the bitmap; the word-popcount prefix sum
//   over the bitmap gives each present column its output rank.
//
// The symbolic pass counts distinct columns per item; the numeric pass sums
// values and writes columns and values at the item's output offset.
#include "accum_util.h"
#include "kernels.h"
#include "primitives.h"

namespace sg {

enum { MODE_ROW = 0, MODE_CHUNK = 1 };

struct ItemHdr {
    int64_t count;  // products (rows) or elements (chunks)
    int64_t out;    // output index: row id, or chunk's map entry
    int64_t a0, a1, s0;  // row mode: A entry range and its product offset
    int64_t start;       // chunk mode: first element
};

template <int MODE>
__device__ __forceinline__ ItemHdr load_item(const RowItems& ri, const ChunkItems& ci,
                                             int64_t p) {
    ItemHdr h;
    if constexpr (MODE == MODE_ROW) {
        int32_t r = ri.perm[p];
        h.out = r;
        h.a0 = ri.A.rp[r];
        h.a1 = ri.A.rp[r + 1];
        h.s0 = ri.S[h.a0];
        h.count = ri.S[h.a1] - h.s0;
        h.start = 0;
    } else {
        h.start = ci.rp[p];
        h.count = ci.rp[p + 1] - h.start;
        h.out = ci.map[p];
        h.a0 = h.a1 = h.s0 = 0;
    }
    return h;
}

// Element t of an item. Row mode walks the products of row i in Gustavson
// order: the product's A entry is the last entry q whose product offset
// S[q] is <= s0 + t, and its B entry is t's distance from that offset.
// `cur` is a per-thread cursor over q (t only grows within a thread).
template <int MODE, bool NUM>
__device__ __forceinline__ void load_elem(const RowItems& ri, const ChunkItems& ci,
                                          const ItemHdr& h, int64_t t, int64_t& cur,
                                          int32_t lo, int32_t& col, double& val) {
    if constexpr (MODE == MODE_ROW) {
        int64_t target = h.s0 + t;
        int64_t q = upper_index(ri.S, cur, h.a1, target);
        cur = q;
        int32_t k = ri.A.col[q];
        int64_t b = ri.B.rp[k] + (target - ri.S[q]);
        col = ri.B.col[b];
        if constexpr (NUM) val = ri.A.val[q] * ri.B.val[b];
    } else {
        col = ci.bcol16 ? lo + (int32_t)ci.bcol16[h.start + t] : ci.bcol[h.start + t];
        if constexpr (NUM) val = ci.bval[h.start + t];
    }
}

// First column of a chunk's window: from the per-chunk base when columns are
// stored as 16-bit offsets, else from the chunk's first column rounded down
// to the chunk width.
__device__ __forceinline__ int32_t chunk_lo(const ChunkItems& ci, int64_t start, int64_t out,
                                            int64_t W) {
    return ci.bcol16 ? ci.colbase[out] : (int32_t)(ci.bcol[start] & ~(int32_t)(W - 1));
}

template <int MODE>
__device__ __forceinline__ int64_t out_offset(const RowItems& ri, const ChunkItems& ci,
                                              const ItemHdr& h) {
    if constexpr (MODE == MODE_ROW) return ri.Crp[h.out];
    else return ci.off[h.out];
}

template <int MODE>
__device__ __forceinline__ void write_count(const RowItems& ri, const ChunkItems& ci,
                                            const ItemHdr& h, int64_t n) {
    if constexpr (MODE == MODE_ROW) ri.cnt[h.out] = n;
    else ci.cnt[h.out] = n;
}

template <int MODE>
__device__ __forceinline__ int32_t* out_cols(const RowItems& ri, const ChunkItems& ci) {
    if constexpr (MODE == MODE_ROW) return ri.Ccol;
    else return ci.Ccol;
}
template <int MODE>
__device__ __forceinline__ double* out_vals(const RowItems& ri, const ChunkItems& ci) {
    if constexpr (MODE == MODE_ROW) return ri.Cval;
    else return ci.Cval;
}

// ---------------------------------------------------------------- light rows
// A light row's products are read round by round: up to TW of the row's A
// entries are staged in the team's LDS (B row start, A value, exclusive
// prefix of B row lengths), then each thread reads U products at a time,
// stride TW, each found by a search of the staged prefix, so that a product
// costs one dependent global read (its B entry) instead of a walk of the
// entry offsets in global memory.
template <int TW>
struct RowStage {
    int pre[TW + 1];
    int64_t b0[TW];
    double a[TW];
};

// Synchronises a team: one wave, or the whole work group.
template <int TW>
__device__ __forceinline__ void team_sync() {
    if constexpr (TW == kWave) wave_lds_sync();
    else __syncthreads();
}

// Last staged entry j in [j, ne) with pre[j] <= t (pre rises; pre[j] <= t).
__device__ __forceinline__ int stage_find(const int* pre, int ne, int t, int j) {
    int jh = ne;
    while (jh - j > 1) {
        const int mid = (j + jh) >> 1;
        if (pre[mid] <= t) j = mid; else jh = mid;
    }
    return j;
}

template <int TW, int U, bool NUM, class F>
__device__ __forceinline__ void row_products(const RowItems& ri, const ItemHdr& h,
                                             RowStage<TW>& sg_, int* red_sh, int tt, F&& f) {
    for (int64_t qb = h.a0; qb < h.a1; qb += TW) {
        const int ne = (int)min((int64_t)TW, h.a1 - qb);
        team_sync<TW>();  // the previous round's staging is consumed
        int len = 0;
        if (tt < ne) {
            const int64_t q = qb + tt;
            const int32_t k = ri.A.col[q];
            const int64_t b0 = ri.B.rp[k];
            len = (int)(ri.B.rp[k + 1] - b0);
            sg_.b0[tt] = b0;
            if constexpr (NUM) sg_.a[tt] = ri.A.val[q];
        }
        int tot;
        const int pre = team_exclusive_scan<TW>(len, red_sh, &tot);
        sg_.pre[tt] = pre;
        team_sync<TW>();
        int j = 0;
        for (int tb = tt; tb < tot; tb += TW * U) {
            int64_t bi[U];
            double av[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int t = tb + u * TW;
                bi[u] = -1;
                av[u] = 0.0;
                if (t < tot) {
                    j = stage_find(sg_.pre, ne, t, j);
                    bi[u] = sg_.b0[j] + (t - sg_.pre[j]);
                    if constexpr (NUM) av[u] = sg_.a[j];
                }
            }
            int32_t c[U];
            double v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                v[u] = 0.0;
                if (bi[u] >= 0) {
                    c[u] = ri.B.col[bi[u]];
                    if constexpr (NUM) v[u] = av[u] * ri.B.val[bi[u]];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (bi[u] >= 0) f(c[u], v[u]);
        }
    }
}

// ---------------------------------------------------------------- thread-local rows
// Rows with at most N products (N = 8, 16, 32) take one thread each: the
// products go into registers in Gustavson order, a bitonic network of
// compare-exchanges at fixed places sorts them by column (places past u hold
// an all-ones key and sort last), and runs of equal columns are summed on
// the way out. Every index is a compile-time constant after unrolling, so
// the arrays stay in registers.
template <bool NUM, int N>
__device__ __forceinline__ void bitonic_regs(uint32_t (&k)[N], double (&v)[N]) {
#pragma unroll
    for (int size = 2; size <= N; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int j = i ^ stride;
                if (j > i) {
                    const bool up = (i & size) == 0;
                    const uint32_t ki = k[i], kj = k[j];
                    const bool sw = up ? (ki > kj) : (ki < kj);
                    k[i] = sw ? kj : ki;
                    k[j] = sw ? ki : kj;
                    if constexpr (NUM) {
                        const double vi = v[i], vj = v[j];
                        v[i] = sw ? vj : vi;
                        v[j] = sw ? vi : vj;
                    }
                }
            }
        }
    }
}

template <bool NUM, int N>
__global__ __launch_bounds__(256) void k_acc_thread(RowItems ri, int64_t p0, int64_t nitems) {
    constexpr uint32_t kNone = 0xffffffffu;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= nitems) return;
    const int32_t r = ri.perm[p0 + i];
    const int64_t a1 = ri.A.rp[r + 1];
    int64_t q = ri.A.rp[r], b = 0, b1 = 0;
    double a = 0.0;
    uint32_t k[N];
    double v[N];
#pragma unroll
    for (int t = 0; t < N; ++t) {
        k[t] = kNone;
        v[t] = 0.0;
        while (b == b1 && q < a1) {  // next entry with products left
            const int32_t kk = ri.A.col[q];
            b = ri.B.rp[kk];
            b1 = ri.B.rp[kk + 1];
            if constexpr (NUM) a = ri.A.val[q];
            ++q;
        }
        if (b < b1) {
            k[t] = (uint32_t)ri.B.col[b];
            if constexpr (NUM) v[t] = a * ri.B.val[b];
            ++b;
        }
    }
    bitonic_regs<NUM, N>(k, v);
    if constexpr (!NUM) {
        int cnt = k[0] != kNone;
#pragma unroll
        for (int t = 1; t < N; ++t) cnt += k[t] != kNone && k[t] != k[t - 1];
        ri.cnt[r] = cnt;
    } else {
        const int64_t off = ri.Crp[r];
        int64_t w = off;
        uint32_t cur = k[0];
        double acc = v[0];
#pragma unroll
        for (int t = 1; t < N; ++t) {
            if (k[t] != cur) {
                if (cur != kNone) {
                    ri.Ccol[w] = (int32_t)cur;
                    ri.Cval[w] = acc;
                    ++w;
                }
                cur = k[t];
                acc = v[t];
            } else {
                acc += v[t];
            }
        }
        if (cur != kNone) {
            ri.Ccol[w] = (int32_t)cur;
            ri.Cval[w] = acc;
        }
    }
}

template <bool NUM, int N>
static void launch_thread(const RowItems& ri, int64_t p0, int64_t n, hipStream_t st) {
    hipLaunchKernelGGL((k_acc_thread<NUM, N>), dim3(grid_1d(ceil_div(n, 256))), dim3(256), 0, st,
                       ri, p0, n);
    SG_LAUNCH_CHECK();
}

// ---------------------------------------------------------------- hash
// Output of a hash row without a sort. The row's distinct columns (nnz of
// them, in the SPT table slots each thread holds in registers; empty slots
// hold ~0) are ranked through a two-level bitmap: bucket b = column / 64 is
// one bit of a top bitmap over the column range (tww words); a prefix of the
// top words' popcounts numbers the nonempty buckets in column order; each
// nonempty bucket has a 64-bit mask of its columns, and a prefix of the
// masks' popcounts gives every bucket its first rank. A column's rank is its
// bucket's first rank plus the columns below it in its mask, so it is
// written straight to its place in the row. Uses 12 * nnz + 8 * tww bytes of
// LDS at `lds` (the caller's table, free once read into registers).
template <int TW, int SPT>
__device__ __forceinline__ void emit_ranked(const uint32_t (&kk)[SPT], const double (&vv)[SPT],
                                            int nnz, int tww, int64_t* lds, int* red_sh,
                                            int32_t* oc, double* ov) {
    const int tt = threadIdx.x;
    uint64_t* bm = (uint64_t*)lds;           // nnz bucket masks
    int* bpre = (int*)(bm + nnz);            // nnz first ranks
    uint32_t* top = (uint32_t*)(bpre + nnz); // tww words: one bit per bucket
    int* tpre = (int*)(top + tww);           // tww word prefixes
    for (int w = tt; w < tww; w += TW) top[w] = 0u;
    for (int c = tt; c < nnz; c += TW) bm[c] = 0ull;
    team_sync<TW>();
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        if (kk[j] != 0xffffffffu) {
            const uint32_t b = kk[j] >> 6;
            atomicOr(&top[b >> 5], 1u << (b & 31));
        }
    }
    team_sync<TW>();
    // nonempty buckets before each top word (thread tt sums a run of words)
    int tot;
    {
        const int per = (tww + TW - 1) / TW;
        const int w0 = min(tww, tt * per), w1 = min(tww, w0 + per);
        int pc = 0;
        for (int w = w0; w < w1; ++w) pc += __popc(top[w]);
        int pre = team_exclusive_scan<TW>(pc, red_sh, &tot);
        for (int w = w0; w < w1; ++w) {
            tpre[w] = pre;
            pre += __popc(top[w]);
        }
    }
    team_sync<TW>();
    int cb[SPT];
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        cb[j] = -1;
        if (kk[j] != 0xffffffffu) {
            const uint32_t b = kk[j] >> 6, w = b >> 5;
            cb[j] = tpre[w] + __popc(top[w] & ((1u << (b & 31)) - 1u));
            atomicOr((unsigned long long*)&bm[cb[j]], 1ull << (kk[j] & 63));
        }
    }
    team_sync<TW>();
    // first rank of every nonempty bucket (tot <= nnz of them)
    {
        const int per = (tot + TW - 1) / TW;
        const int c0 = min(tot, tt * per), c1 = min(tot, c0 + per);
        int pc = 0;
        for (int c = c0; c < c1; ++c) pc += __popcll(bm[c]);
        int all;
        int pre = team_exclusive_scan<TW>(pc, red_sh, &all);
        for (int c = c0; c < c1; ++c) {
            bpre[c] = pre;
            pre += __popcll(bm[c]);
        }
    }
    team_sync<TW>();
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        if (cb[j] >= 0) {
            const int r = bpre[cb[j]] + __popcll(bm[cb[j]] & ((1ull << (kk[j] & 63)) - 1ull));
            oc[r] = (int32_t)kk[j];
            ov[r] = vv[j];
        }
    }
}

// One item per work group of TW threads; the table has S = 2^LOGS slots.
template <int MODE, bool NUM, int TW, int LOGS>
__global__ __launch_bounds__(TW) void k_acc_hash(RowItems ri, ChunkItems ci, int64_t p0,
                                                 int64_t nitems) {
    constexpr int S = 1 << LOGS;
    constexpr int SPT = S / TW;  // slots per thread in the compaction step
    static_assert(SPT >= 1 && SPT * TW == S, "table must be a multiple of the team");
    extern __shared__ int64_t lds_a[];
    uint32_t* keys = (uint32_t*)lds_a;
    double* vals = (double*)(keys + S);
    __shared__ int red_sh[TW / kWave + 1];
    const int tt = threadIdx.x;
    const int64_t item = blockIdx.x;
    if (item >= nitems) return;
    const ItemHdr h = load_item<MODE>(ri, ci, p0 + item);
    for (int s = tt; s < S; s += TW) {
        keys[s] = 0xffffffffu;
        if constexpr (NUM) vals[s] = 0.0;
    }
    __syncthreads();

    int fresh = 0;
    {
        constexpr uint32_t smask = (uint32_t)S - 1;
        auto insert = [&](int32_t c, double v) {
            uint32_t key = (uint32_t)c;
            uint32_t slot = (key * 2654435769u) >> (32 - LOGS);
            for (;;) {
                uint32_t old = atomicCAS(&keys[slot], 0xffffffffu, key);
                if (old == 0xffffffffu) {
                    ++fresh;
                    break;
                }
                if (old == key) break;
                slot = (slot + 1) & smask;
            }
            if constexpr (NUM) atomicAdd(&vals[slot], v);
        };
        if constexpr (MODE == MODE_ROW) {
            __shared__ RowStage<TW> stage;
            row_products<TW, 2, NUM>(ri, h, stage, red_sh, tt, insert);
        } else {
            int64_t cur = 0;
            for (int64_t t = tt; t < h.count; t += TW) {
                int32_t c;
                double v = 0.0;
                load_elem<MODE, NUM>(ri, ci, h, t, cur, 0, c, v);
                insert(c, v);
            }
        }
    }
    const int nnz = team_sum<TW>(fresh, red_sh);
    if constexpr (!NUM) {
        if (tt == 0) write_count<MODE>(ri, ci, h, nnz);
        return;
    } else {
        __syncthreads();
        uint32_t kk[SPT];
        double vv[SPT];
        int occ = 0;
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            kk[j] = keys[tt * SPT + j];
            vv[j] = vals[tt * SPT + j];
            occ += kk[j] != 0xffffffffu;
        }
        if constexpr (MODE == MODE_ROW) {
            // a row's columns lie in [0, B.ncols): when the two-level bitmap
            // over that range fits the table's LDS, rank without a sort
            const int tww = (int)((ri.B.m + 2047) >> 11);
            if (8 * (int64_t)tww + 12 * (int64_t)nnz <= 12 * (int64_t)S) {
                __syncthreads();  // the table is in registers: its LDS is reused
                const int64_t off = out_offset<MODE>(ri, ci, h);
                emit_ranked<TW, SPT>(kk, vv, nnz, tww, lds_a, red_sh, out_cols<MODE>(ri, ci) + off,
                                     out_vals<MODE>(ri, ci) + off);
                return;
            }
        }
        // compact the occupied slots to the front, in slot order
        int tot;
        int pre = team_exclusive_scan<TW>(occ, red_sh, &tot);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            if (kk[j] != 0xffffffffu) {
                keys[pre] = kk[j];
                vals[pre] = vv[j];
                ++pre;
            }
        }
        int P2 = 1;
        while (P2 < nnz) P2 <<= 1;
        __syncthreads();
        for (int s = nnz + tt; s < P2; s += TW) keys[s] = 0xffffffffu;
        __syncthreads();
        // bitonic sort of the next power of two above nnz. With distance
        // j <= 32, the 64 pairs of a wave lie in its own block of 128 keys
        // (the same blocks in every such step), so two such steps in a row
        // need only the wave's own LDS ordering, not a work-group barrier.
        for (int k = 2; k <= P2; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                for (int pi = tt; pi < (P2 >> 1); pi += TW) {
                    int i = ((pi & ~(j - 1)) << 1) | (pi & (j - 1));
                    int ix = i | j;
                    uint32_t ka = keys[i], kb = keys[ix];
                    bool asc = (i & k) == 0;
                    if ((ka > kb) == asc) {
                        keys[i] = kb;
                        keys[ix] = ka;
                        double va = vals[i];
                        vals[i] = vals[ix];
                        vals[ix] = va;
                    }
                }
                const int jn = j > 1 ? (j >> 1) : k;  // the next step's distance
                if (j <= kWave / 2 && jn <= kWave / 2) wave_lds_sync();
                else __syncthreads();
            }
        }
        __syncthreads();
        int64_t off = out_offset<MODE>(ri, ci, h);
        int32_t* oc = out_cols<MODE>(ri, ci);
        double* ov = out_vals<MODE>(ri, ci);
        for (int s = tt; s < nnz; s += TW) {
            oc[off + s] = (int32_t)keys[s];
            ov[off + s] = vals[s];
        }
    }
}

// ---------------------------------------------------------------- bitmap rank
// Chunks whose column width W is small enough for a one-bit-per-column
// bitmap in LDS. Pass 1 sets the bitmap from the chunk's columns (kept in
// registers); a prefix sum over the word popcounts gives every present
// column its rank, i.e. its place in the sorted output; pass 2 adds each
// value into a compact array at that rank. Each thread then writes the
// columns of its own bitmap words at their ranks into LDS, and the chunk is
// streamed out with coalesced writes.

// One chunk of at most TW*KPT elements, its columns (idx, ~0 for none) and
// values already in registers: bitmap, ranks, values summed at their rank,
// the chunk written sorted (or its distinct count, symbolic).
template <bool NUM, int TW, int KPT>
__device__ __forceinline__ void rank_chunk(const ChunkItems& ci, int W, const uint32_t (&idx)[KPT],
                                           double (&v)[KPT], int64_t out, int32_t lo,
                                           double* vals, uint32_t* bits, int* wpre,
                                           int32_t* scol, int* red_sh) {
    const int NWD = W >> 5;
    const int tt = threadIdx.x;
    // one-wave chunks are ranked through the two-level bitmap (work by
    // element); the larger ones through the chunk's full bitmap
    constexpr bool kTwoLevel = TW == kWave;
    // A numeric chunk whose W one-byte flags fit in its value array marks
    // its columns there with plain byte stores (lanes of a wave often share
    // a bitmap word, on which atomic ORs serialise), packed into the bitmap
    // afterwards; the values take the array over once the flags are packed.
    const bool flags = NUM && W <= TW * KPT * 8;
    if constexpr (!kTwoLevel) {
        if (flags) {
            const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
            for (int i = tt; i < W / 16; i += TW) ((uint4*)vals)[i] = z4;
        } else {
            for (int w = tt; w < NWD; w += TW) bits[w] = 0u;
        }
        __syncthreads();
    }
    if constexpr (kTwoLevel) {
        if constexpr (!NUM) {
#pragma unroll
            for (int k = 0; k < KPT; ++k) v[k] = 0.0;
        }
        // LDS from `bits` on: the two-level arrays, then the ranked columns
        uint16_t* scol16 = (uint16_t*)((char*)bits + wave_rank_lds(KPT, W));
        const int64_t off = NUM ? ci.off[out] : 0;
        const int nnz = wave_rank_emit<KPT>(idx, v, W, bits, vals, scol16, lo, ci.Ccol + off,
                                            ci.Cval + off, NUM);
        if constexpr (!NUM)
            if (tt == 0) ci.cnt[out] = nnz;
        return;
    }
    const int64_t off = NUM ? ci.off[out] : 0;
    const int per = (NWD + TW - 1) / TW;
    const int w0 = min(NWD, tt * per), w1 = min(NWD, w0 + per);
    int pc = 0;
    if (flags) {
        uint8_t* fb = (uint8_t*)vals;
#pragma unroll
        for (int k = 0; k < KPT; ++k)
            if (idx[k] < (uint32_t)W) fb[idx[k]] = 1;
        __syncthreads();
        for (int w = w0; w < w1; ++w) {
            const uint32_t m = pack_flags32((const uint32_t*)vals + w * 8);
            bits[w] = m;
            pc += __popc(m);
        }
    } else {
#pragma unroll
        for (int k = 0; k < KPT; ++k)
            if (idx[k] < (uint32_t)W) atomicOr(&bits[idx[k] >> 5], 1u << (idx[k] & 31));
        __syncthreads();
        for (int w = w0; w < w1; ++w) pc += __popc(bits[w]);
    }
    if constexpr (!NUM) {
        int tot = team_sum<TW>(pc, red_sh);
        if (tt == 0) ci.cnt[out] = tot;
    } else {
        // the scan's barrier also ends every thread's packing of the flags
        int tot;
        int pre = block_scan_first<TW>(pc, red_sh, &tot);
        for (int w = w0; w < w1; ++w) {
            wpre[w] = pre;
            pre += __popc(bits[w]);
        }
        for (int r = tt; r < tot; r += TW) vals[r] = 0.0;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            if (idx[k] < (uint32_t)W) {
                uint32_t w = idx[k] >> 5;
                int rank = wpre[w] + __popc(bits[w] & ((1u << (idx[k] & 31)) - 1u));
                atomicAdd(&vals[rank], v[k]);
            }
        }
        // the column of every rank, scattered into LDS from the bitmap words
        // (each thread walks the set bits of its own words), then streamed out
        for (int w = w0; w < w1; ++w) {
            uint32_t x = bits[w];
            int r = wpre[w];
            while (x) {
                const int b = __ffs(x) - 1;
                x &= x - 1;
                scol[r++] = lo + w * 32 + b;
            }
        }
        __syncthreads();
        for (int r = tt; r < tot; r += TW) {
            ci.Ccol[off + r] = scol[r];
            ci.Cval[off + r] = vals[r];
        }
    }
}

// IPG consecutive chunks of a class per work group, one after the other:
// every thread reads a chunk's first column itself (one address for the
// group), and all the chunks' elements are loaded before the first is
// ranked, so that no barrier stands between a chunk's header and its loads
// and the later chunks' loads are paid while the first one is ranked.
template <bool NUM, int TW, int KPT, int IPG>
__global__ __launch_bounds__(TW) void k_acc_rank(ChunkItems ci, int64_t p0, int64_t nitems,
                                                 int logW) {
    extern __shared__ __align__(16) int64_t lds_r[];
    const int W = 1 << logW;
    const int NWD = W >> 5;
    double* vals = (double*)lds_r;                                // TW*KPT (NUM)
    uint32_t* bits = (uint32_t*)(vals + (NUM ? TW * KPT : 0));    // NWD
    int* wpre = (int*)(bits + NWD);                               // NWD (NUM)
    int32_t* scol = (int32_t*)(wpre + NWD);                       // TW*KPT (NUM)
    __shared__ int red_sh[TW / kWave + 1];
    const int tt = threadIdx.x;
    const int64_t i0 = (int64_t)blockIdx.x * IPG;
    if (i0 >= nitems) return;
    const int nown = (int)min((int64_t)IPG, nitems - i0);  // uniform over the group
    int64_t start[IPG], out[IPG];
    int count[IPG];
    int32_t lo[IPG];
#pragma unroll
    for (int u = 0; u < IPG; ++u) {
        const int64_t it = p0 + i0 + min(u, nown - 1);
        start[u] = ci.rp[it];
        count[u] = (int)(ci.rp[it + 1] - start[u]);
        out[u] = ci.map[it];
    }
#pragma unroll
    for (int u = 0; u < IPG; ++u) lo[u] = chunk_lo(ci, start[u], out[u], W);
    uint32_t idx[IPG][KPT];
    double v[IPG][KPT];
#pragma unroll
    for (int u = 0; u < IPG; ++u) {
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            const int t = tt + k * TW;
            idx[u][k] = 0xffffffffu;
            v[u][k] = 0.0;
            if (t < count[u]) {
                idx[u][k] = ci.bcol16 ? (uint32_t)ci.bcol16[start[u] + t]
                                      : (uint32_t)(ci.bcol[start[u] + t] - lo[u]);
                if constexpr (NUM) v[u][k] = ci.bval[start[u] + t];
            }
        }
    }
#pragma unroll
    for (int u = 0; u < IPG; ++u) {
        if (u < nown) {
            // the previous chunk's output has read the LDS arrays
            if (u > 0) {
                if constexpr (TW == kWave) wave_lds_sync();
                else __syncthreads();
            }
            rank_chunk<NUM, TW, KPT>(ci, W, idx[u], v[u], out[u], lo[u], vals, bits, wpre, scol,
                                     red_sh);
        }
    }
}

// ---------------------------------------------------------------- dense window
// Light rows whose columns fall in a short window (rows of banded matrices):
// NI teams of TW threads per work group, one row each.
template <bool NUM, int TW, int NI>
__global__ __launch_bounds__(TW* NI) void k_acc_window(RowItems ri, int64_t p0, int64_t nitems,
                                                       int logW) {
    static_assert(TW == kWave || NI == 1, "block-wide teams hold one item");
    extern __shared__ int64_t lds_w[];
    const int W = 1 << logW;
    const int NWD = W >> 5;  // bitmap words
    const int team = threadIdx.x / TW;
    const int tt = threadIdx.x % TW;
    double* acc = (double*)lds_w + (NUM ? team * W : 0);
    uint32_t* flags = (uint32_t*)((double*)lds_w + (NUM ? NI * W : 0)) + team * NWD * 8;
    uint32_t* bits = (uint32_t*)((double*)lds_w + (NUM ? NI * W : 0)) + NI * NWD * 8 + team * NWD;
    int* wpre = (int*)((uint32_t*)((double*)lds_w + (NUM ? NI * W : 0)) + NI * NWD * 9) + team * NWD;
    __shared__ int red_sh[TW / kWave + 1];
    __shared__ int32_t lo_sh[NI];

    const int64_t item = (int64_t)blockIdx.x * NI + team;
    const bool active = item < nitems;
    ItemHdr h;
    if (active) h = load_item<MODE_ROW>(ri, ChunkItems{}, p0 + item);
    for (int w = tt; w < NWD * 8; w += TW) flags[w] = 0u;
    if constexpr (NUM)
        for (int s = tt; s < W; s += TW) acc[s] = 0.0;
    if (tt == 0 && active) lo_sh[team] = ri.rowlo[h.out];
    __syncthreads();
    const int32_t lo = active ? lo_sh[team] : 0;
    uint8_t* fb = (uint8_t*)flags;
    __shared__ RowStage<TW> stages[NI];
    if (active) {
        row_products<TW, 4, NUM>(ri, h, stages[team], red_sh, tt, [&](int32_t c, double v) {
            const uint32_t idx = (uint32_t)(c - lo);
            if (idx < (uint32_t)W) {
                fb[idx] = 1;
                if constexpr (NUM) atomicAdd(&acc[idx], v);
            }
        });
    }
    __syncthreads();
    // each thread owns a contiguous run of bitmap words
    const int per = (NWD + TW - 1) / TW;
    const int w0 = min(NWD, tt * per), w1 = min(NWD, w0 + per);
    int pc = 0;
    for (int w = w0; w < w1; ++w) {
        uint32_t m = pack_flags32(flags + w * 8);
        bits[w] = m;
        pc += __popc(m);
    }
    if constexpr (!NUM) {
        int tot = team_sum<TW>(pc, red_sh);
        if (active && tt == 0) ri.cnt[h.out] = tot;
    } else {
        int tot;
        int pre = team_exclusive_scan<TW>(pc, red_sh, &tot);
        for (int w = w0; w < w1; ++w) {
            wpre[w] = pre;
            pre += __popc(bits[w]);
        }
        __syncthreads();
        if (active) {
            const int64_t off = ri.Crp[h.out];
            for (int idx = tt; idx < W; idx += TW) {
                uint32_t word = bits[idx >> 5];
                uint32_t bit = 1u << (idx & 31);
                if (word & bit) {
                    int rank = wpre[idx >> 5] + __popc(word & (bit - 1));
                    ri.Ccol[off + rank] = lo + idx;
                    ri.Cval[off + rank] = acc[idx];
                }
            }
        }
    }
}

// Dense window of one heavy chunk: the chunk mode of the window
// accumulator in a kernel of its own. The first batch of elements is loaded
// before the window is cleared (16 bytes a store), so that the clearing
// runs while they arrive, and every thread reads the chunk's first column
// itself instead of waiting on a barrier for it.
constexpr int kChunkWinNT = 1024;

template <bool NUM>
__global__ __launch_bounds__(kChunkWinNT) void k_chunk_window(ChunkItems ci, int64_t p0,
                                                             int64_t nitems, int logW) {
    constexpr int TW = kChunkWinNT;
    constexpr int U = 4;  // loads in flight per thread
    extern __shared__ __align__(16) int64_t lds_c[];
    const int W = 1 << logW;
    const int NWD = W >> 5;  // bitmap words
    double* acc = (double*)lds_c;                        // W (numeric)
    uint32_t* flags = (uint32_t*)(acc + (NUM ? W : 0));  // W bytes
    uint32_t* bits = flags + NWD * 8;                    // NWD
    int* wpre = (int*)(bits + NWD);                      // NWD
    __shared__ int red_sh[TW / kWave + 1];
    const int tt = threadIdx.x;
    const int64_t item = blockIdx.x;
    if (item >= nitems) return;
    const int64_t start = ci.rp[p0 + item];
    const int64_t count = ci.rp[p0 + item + 1] - start;
    const int64_t out = ci.map[p0 + item];
    const int32_t lo = chunk_lo(ci, start, out, W);
    uint32_t c[U];
    double v[U];
    auto load = [&](int64_t t0) {
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
            const int64_t t = t0 + (int64_t)uu * TW;
            c[uu] = 0xffffffffu;  // past the window: skipped
            v[uu] = 0.0;
            if (t < count) {
                c[uu] = ci.bcol16 ? (uint32_t)ci.bcol16[start + t]
                                  : (uint32_t)(ci.bcol[start + t] - lo);
                if constexpr (NUM) v[uu] = ci.bval[start + t];
            }
        }
    };
    load(tt);
    // W is a power of two of at least 32: W bytes of flags are NWD * 2
    // 16-byte stores, W doubles W / 2 of them
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
    for (int i = tt; i < NWD * 2; i += TW) ((uint4*)flags)[i] = z4;
    if constexpr (NUM)
        for (int i = tt; i < W / 2; i += TW) ((uint4*)acc)[i] = z4;
    __syncthreads();
    uint8_t* fb = (uint8_t*)flags;
    for (int64_t t0 = tt; t0 < count; t0 += (int64_t)TW * U) {
        if (t0 != tt) load(t0);
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
            if (c[uu] < (uint32_t)W) {
                fb[c[uu]] = 1;
                if constexpr (NUM) atomicAdd(&acc[c[uu]], v[uu]);
            }
        }
    }
    __syncthreads();
    // each thread packs a contiguous run of bitmap words
    const int per = (NWD + TW - 1) / TW;
    const int w0 = min(NWD, tt * per), w1 = min(NWD, w0 + per);
    int pc = 0;
    for (int w = w0; w < w1; ++w) {
        const uint32_t m = pack_flags32(flags + w * 8);
        bits[w] = m;
        pc += __popc(m);
    }
    if constexpr (!NUM) {
        const int tot = team_sum<TW>(pc, red_sh);
        if (tt == 0) ci.cnt[out] = tot;
    } else {
        int tot;
        int pre = block_scan_first<TW>(pc, red_sh, &tot);
        for (int w = w0; w < w1; ++w) {
            wpre[w] = pre;
            pre += __popc(bits[w]);
        }
        __syncthreads();
        const int64_t off = ci.off[out];
        for (int i = tt; i < W; i += TW) {
            const uint32_t word = bits[i >> 5];
            const uint32_t bit = 1u << (i & 31);
            if (word & bit) {
                const int rank = wpre[i >> 5] + __popc(word & (bit - 1));
                ci.Ccol[off + rank] = lo + i;
                ci.Cval[off + rank] = acc[i];
            }
        }
    }
}

// ---------------------------------------------------------------- launchers
// chunks per work group of the bitmap-rank classes
constexpr int kRankIPG = 2;

template <int MODE, bool NUM, int TW, int LOGS>
static void launch_hash(const RowItems& ri, const ChunkItems& ci, int64_t p0, int64_t n,
                        hipStream_t st) {
    size_t lds = (size_t)(1 << LOGS) * (4 + (NUM ? 8 : 0));
    auto kern = k_acc_hash<MODE, NUM, TW, LOGS>;
    SG_HIP(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds));
    hipLaunchKernelGGL(kern, dim3(grid_1d(n)), dim3(TW), lds, st, ri, ci, p0, n);
    SG_LAUNCH_CHECK();
}

template <bool NUM, int TW, int KPT, int IPG = kRankIPG>
static void launch_rank(const ChunkItems& ci, int64_t p0, int64_t n, hipStream_t st) {
    const int64_t W = ci.width;
    size_t lds = (NUM ? (size_t)TW * KPT * 12 : 0) + (size_t)(W / 32) * 4 * (NUM ? 2 : 1);
    if (TW == kWave)  // the two-level arrays and 16-bit ranked columns after the values
        lds = (NUM ? (size_t)TW * KPT * 8 : 0) + (size_t)wave_rank_lds(KPT, W) +
              (size_t)TW * KPT * 2;
    auto kern = k_acc_rank<NUM, TW, KPT, IPG>;
    SG_HIP(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds));
    hipLaunchKernelGGL(kern, dim3(grid_1d(ceil_div(n, IPG))), dim3(TW), lds, st, ci, p0, n,
                       ilog2(W));
    SG_LAUNCH_CHECK();
}

template <bool NUM, int TW, int NI>
static void launch_window(const RowItems& ri, int64_t p0, int64_t n, int64_t W, hipStream_t st) {
    if (W < 32 || (W & (W - 1))) throw std::logic_error("window width must be a power of two >= 32");
    size_t lds = (size_t)NI * ((NUM ? W * 8 : 0) + W + (W / 32) * 4 * 2);
    if (lds > 160 * 1024) throw OverflowError("dense window exceeds LDS");
    auto kern = k_acc_window<NUM, TW, NI>;
    SG_HIP(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds));
    hipLaunchKernelGGL(kern, dim3(grid_1d(ceil_div(n, NI))), dim3(TW * NI), lds, st, ri, p0, n,
                       ilog2(W));
    SG_LAUNCH_CHECK();
}

template <int MODE, bool NUM>
static void launch_hash_bin(int hb, int top_logS, const RowItems& ri, const ChunkItems& ci,
                            int64_t p0, int64_t n, hipStream_t st) {
    switch (hb) {
        case 0: launch_hash<MODE, NUM, 64, 7>(ri, ci, p0, n, st); break;
        case 1: launch_hash<MODE, NUM, 64, 9>(ri, ci, p0, n, st); break;
        case 2: launch_hash<MODE, NUM, 256, 11>(ri, ci, p0, n, st); break;
        default:
            if (top_logS <= 12) launch_hash<MODE, NUM, 512, 12>(ri, ci, p0, n, st);
            else launch_hash<MODE, NUM, 512, 13>(ri, ci, p0, n, st);
            break;
    }
}

template <bool NUM>
static void launch_rank_bin(int hb, const ChunkItems& ci, int64_t p0, int64_t n, hipStream_t st) {
    switch (hb) {
        case 0: launch_rank<NUM, 64, 1>(ci, p0, n, st); break;
        case 1: launch_rank<NUM, 64, 4>(ci, p0, n, st); break;
        // four elements a thread in the block-sized classes: with eight, the
        // kernel reaches 64 VGPRs and LDS bounds its groups to 22 waves a CU
        case 2: launch_rank<NUM, 256, 4>(ci, p0, n, st); break;
        default:
            // the top light class holds chunks of at most tau elements
            if (ci.hash_top_logS <= 12) launch_rank<NUM, 512, 4>(ci, p0, n, st);
            else launch_rank<NUM, 512, 16, 1>(ci, p0, n, st);
            break;
    }
}

template <bool NUM>
static void rows_impl(const RowItems& it, int bin, int64_t p0, int64_t n, hipStream_t st) {
    ChunkItems none{};
    switch (bin) {
        case RB_T8: launch_thread<NUM, 8>(it, p0, n, st); break;
        case RB_T16: launch_thread<NUM, 16>(it, p0, n, st); break;
        case RB_T32: launch_thread<NUM, 32>(it, p0, n, st); break;
        case RB_WIN64: launch_window<NUM, 64, 4>(it, p0, n, kWinSmall, st); break;
        case RB_WIN1024:
            launch_window<NUM, 256, 1>(it, p0, n, kWinLarge, st);
            break;
        case RB_H128: launch_hash_bin<MODE_ROW, NUM>(0, it.hash_top_logS, it, none, p0, n, st); break;
        case RB_H512: launch_hash_bin<MODE_ROW, NUM>(1, it.hash_top_logS, it, none, p0, n, st); break;
        case RB_H2048: launch_hash_bin<MODE_ROW, NUM>(2, it.hash_top_logS, it, none, p0, n, st); break;
        case RB_H8192: launch_hash_bin<MODE_ROW, NUM>(3, it.hash_top_logS, it, none, p0, n, st); break;
        default: throw std::logic_error("not a light row bin");
    }
}

void accumulate_rows(const RowItems& it, int bin, int64_t p0, int64_t n, bool numeric,
                     hipStream_t st) {
    if (n <= 0) return;
    if (numeric) rows_impl<true>(it, bin, p0, n, st);
    else rows_impl<false>(it, bin, p0, n, st);
}

template <bool NUM>
static void chunks_impl(const ChunkItems& it, int bin, int64_t p0, int64_t n, hipStream_t st) {
    RowItems none{};
    switch (bin) {
        case CB_DENSE: {
            const int64_t W = it.width;
            if (W < 32 || (W & (W - 1)))
                throw std::logic_error("window width must be a power of two >= 32");
            const size_t lds = (size_t)((NUM ? W * 8 : 0) + W + (W / 32) * 4 * 2);
            if (lds > 160 * 1024) throw OverflowError("dense window exceeds LDS");
            auto kern = k_chunk_window<NUM>;
            SG_HIP(hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
            hipLaunchKernelGGL(kern, dim3(grid_1d(n)), dim3(kChunkWinNT), lds, st, it, p0, n,
                               ilog2(W));
            SG_LAUNCH_CHECK();
            break;
        }
        case CB_H128:
        case CB_H512:
        case CB_H2048:
        case CB_H8192:
            if (it.width <= kRankMaxWidth)
                launch_rank_bin<NUM>(bin - CB_H128, it, p0, n, st);
            else if (!it.bcol16)
                launch_hash_bin<MODE_CHUNK, NUM>(bin - CB_H128, it.hash_top_logS, none, it, p0, n,
                                                 st);
            else
                throw std::logic_error("16-bit chunk columns need chunks at most 2^16 wide");
            break;
        default: throw std::logic_error("not an accumulated chunk bin");
    }
}

void accumulate_chunks(const ChunkItems& it, int bin, int64_t p0, int64_t n, bool numeric,
                       hipStream_t st) {
    if (n <= 0) return;
    if (numeric) chunks_impl<true>(it, bin, p0, n, st);
    else chunks_impl<false>(it, bin, p0, n, st);
}

}  // namespace sg
