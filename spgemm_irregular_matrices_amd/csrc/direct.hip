// Direct accumulation of the heavy rows (numeric pass).
//
// The chunk of a product a_ik * b_kj is fixed by j alone, so the
// column-range split that the gMAGNUS page applies to C-hat (Section III-C,
// hierarchical multisplit) can be applied to B instead: every B row is
// partitioned once into the final chunks (slots of width W), and the split
// copy of B is laid out slot by slot: all rows' entries of slot 0, then of
// slot 1, and so on, each slot's entries in row order. spos[s*B.n + k]
// records where row k's entries of slot s start, so the products of heavy
// row i that fall into chunk s are the slices [spos[s*B.n + k],
// spos[s*B.n + k + 1]) for the B rows k of row i's entries, each scaled by
// its a_ik, and one slot's part of B is contiguous. One work group per
// (heavy row, chunk) item forms exactly those products and accumulates them
// in LDS with the page's accumulators
// (Section III-E): the bitmap-rank accumulator for items of at most
// kDirectDense products, the dense window above that. C-hat and
// C-hat-reord are never written; the per-item product and distinct-column
// counts come from the fused symbolic pass.
#include "accum_util.h"
#include "kernels.h"
#include "primitives.h"

namespace sg {

// ---------------------------------------------------------------- B split
// bslot (row-major, B.n x req) to slot-major (req x B.n), in 32 x 32 tiles;
// also the rows' occupancy words, row-major: bit t of roc[k * nw + w] is set
// if B row k has entries in slot 32 w + t (nw = ceil(req / 32) = gridDim.y;
// each half wave holds the 32 slots of one row).
__global__ __launch_bounds__(256) void k_bslot_transpose(const int32_t* bslot, int64_t nb, int req,
                                                         int32_t* bslotT, uint32_t* roc) {
    __shared__ int32_t tile[32][33];
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
    const int64_t k0 = (int64_t)blockIdx.x * 32;
    const int s0 = blockIdx.y * 32;
    for (int r = ty; r < 32; r += 8) {
        const int64_t k = k0 + r;
        const int sl = s0 + tx;
        const int32_t c = (k < nb && sl < req) ? bslot[k * req + sl] : 0;
        tile[r][tx] = c;
        const uint64_t m = __ballot(c != 0);
        if (tx == 0 && k < nb)
            roc[k * gridDim.y + blockIdx.y] = (uint32_t)(threadIdx.x & 32 ? m >> 32 : m);
    }
    __syncthreads();
    for (int r = ty; r < 32; r += 8) {
        const int sl = s0 + r;
        const int64_t k = k0 + tx;
        const int32_t c = tile[tx][r];
        if (sl < req && k < nb) bslotT[(int64_t)sl * nb + k] = c;
    }
}

// eocc[w * annz + q]: occupancy word w of B row Acol[q], for every A entry q,
// so that an item reads its entries' bits beside their columns, coalesced.
__global__ __launch_bounds__(256) void k_entry_occ(const int32_t* acol, int64_t annz, int nw,
                                                   const uint32_t* roc, uint32_t* eocc) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= annz) return;
    const int64_t k = acol[q];
    for (int w = 0; w < nw; ++w) eocc[(int64_t)w * annz + q] = roc[k * nw + w];
}

void direct_entry_occ(const int32_t* acol, int64_t annz, int req, const uint32_t* roc,
                      uint32_t* eocc, hipStream_t st) {
    if (annz <= 0) return;
    hipLaunchKernelGGL(k_entry_occ, dim3(grid_1d(ceil_div(annz, 256))), dim3(256), 0, st, acol,
                       annz, (int)ceil_div(req, 32), roc, eocc);
    SG_LAUNCH_CHECK();
}

struct LoadI32 {
    const int32_t* a;
    __device__ int64_t operator()(int64_t i) const { return a[i]; }
};

// One wavefront per B row: each entry goes to its slot's part of the split
// copy, at the row's start there plus its rank among the row's entries of
// that slot. Every lane reads its slot's start first (one round of loads
// for the batch); the wave then ranks each batch of 64 entries by peeling
// one distinct slot at a time (ballot of the lanes holding the first
// remaining lane's slot), touching only LDS, where the row's running counts
// per slot live.
constexpr int kBpartNT = 256;

__global__ __launch_bounds__(kBpartNT) void k_bpartition(const int64_t* brp, const int32_t* bcol,
                                                         int64_t nb, int logW, int req,
                                                         const int32_t* spos, int32_t* bperm,
                                                         uint16_t* bcol16) {
    extern __shared__ int lds_b[];
    const int w = threadIdx.x / kWave, lane = lane_id();
    int* run = lds_b + w * req;
    const int64_t k = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    if (k >= nb) return;  // whole waves leave together; no block barrier below
    for (int sl = lane; sl < req; sl += kWave) run[sl] = 0;
    const int64_t e0 = brp[k], e1 = brp[k + 1];
    const uint32_t wmask = (1u << logW) - 1u;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    for (int64_t eb = e0; eb < e1; eb += kWave) {
        const int64_t e = eb + lane;
        int32_t c = 0;
        int sl = -1;
        int32_t p0 = 0;
        if (e < e1) {
            c = bcol[e];
            sl = (int)((uint32_t)c >> logW);
            p0 = spos[(int64_t)sl * nb + k];
        }
        int rank = 0;
        uint64_t act = __ballot(sl >= 0);
        while (act) {
            const int leader = __builtin_ctzll(act);
            const int ls = __builtin_amdgcn_readlane(sl, leader);
            const uint64_t m = __ballot(sl == ls);
            const int base = run[ls];
            if (sl == ls) rank = base + __popcll(m & lt);
            if (lane == leader) run[ls] = base + __popcll(m);
            act &= ~m;
        }
        if (sl >= 0) {
            bperm[p0 + rank] = (int32_t)e;
            bcol16[p0 + rank] = (uint16_t)((uint32_t)c & wmask);
        }
    }
}

void direct_split_b(const DevCSR& B, const int32_t* bslot, int req, int64_t W, int32_t* spos,
                    uint32_t* roc, int32_t* bperm, uint16_t* bcol16, Arena& ar, hipStream_t st) {
    if (W > 65536 || req > kDirectMaxSlots || B.nnz > INT32_MAX)
        throw std::logic_error("direct split limits");
    const int64_t n = (int64_t)req * B.n;
    if (B.n <= 0) {
        fill<int32_t>(spos, 1, 0, st);
        return;
    }
    int32_t* bslotT = ar.get<int32_t>("bslotT", (size_t)n);
    hipLaunchKernelGGL(k_bslot_transpose, dim3(grid_1d(ceil_div(B.n, 32)), ceil_div(req, 32)),
                       dim3(256), 0, st, bslot, B.n, req, bslotT, roc);
    SG_LAUNCH_CHECK();
    scan_exclusive<LoadI32, int32_t>(LoadI32{bslotT}, n, spos, ar, st);
    if (B.nnz <= 0) return;
    const size_t lds = (size_t)(kBpartNT / kWave) * req * 4;
    SG_HIP(hipFuncSetAttribute((const void*)k_bpartition,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
    hipLaunchKernelGGL(k_bpartition, dim3(grid_1d(ceil_div(B.n * kWave, kBpartNT))),
                       dim3(kBpartNT), lds, st, B.rp, B.col, B.n, ilog2(W), req, spos, bperm,
                       bcol16);
    SG_LAUNCH_CHECK();
}

// ---------------------------------------------------------------- offsets
// off[h*req + s] = C.rowPtr of heavy row h + distinct columns of the row in
// slots before s (slots are in column order, so this is the item's place in
// the sorted output row). One wavefront per heavy row scans its slots.
__global__ __launch_bounds__(256) void k_direct_offsets(const int64_t* C_rp, const int32_t* hrows,
                                                       int64_t H, int req,
                                                       const int64_t* dist_fin, int64_t* off) {
    const int64_t h = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    if (h >= H) return;  // whole waves leave together
    const int lane = lane_id();
    int64_t run = C_rp[hrows[h]];
    for (int sb = 0; sb < req; sb += kWave) {
        const int sl = sb + lane;
        const int64_t c = sl < req ? dist_fin[h * req + sl] : 0;
        const int64_t inc = wave_inclusive_scan(c);
        if (sl < req) off[h * req + sl] = run + inc - c;
        run += __shfl(inc, kWave - 1, kWave);
    }
}

void direct_offsets(const int64_t* C_rp, const int32_t* hrows, int64_t H, int req,
                    const int64_t* dist_fin, int64_t* off, hipStream_t st) {
    if (H <= 0) return;
    hipLaunchKernelGGL(k_direct_offsets, dim3(grid_1d(ceil_div(H * kWave, 256))), dim3(256), 0, st,
                       C_rp, hrows, H, req, dist_fin, off);
    SG_LAUNCH_CHECK();
}

// ---------------------------------------------------------------- numeric
// kGatherU placement-map entries a thread, their value loads issued together
// (where B's columns are spread evenly over the slots, every load is a
// random line: their latency, not bytes, bounds the gather).
constexpr int kGatherU = 4;

__global__ __launch_bounds__(256) void k_gather_bval(const int32_t* bperm, const double* bval,
                                                     int64_t nnz, double* out) {
    const int64_t j0 = (int64_t)blockIdx.x * (256 * kGatherU) + threadIdx.x;
    int32_t src[kGatherU];
#pragma unroll
    for (int u = 0; u < kGatherU; ++u) {
        const int64_t j = j0 + u * 256;
        src[u] = j < nnz ? bperm[j] : -1;
    }
    double v[kGatherU];
#pragma unroll
    for (int u = 0; u < kGatherU; ++u) v[u] = src[u] >= 0 ? bval[src[u]] : 0.0;
#pragma unroll
    for (int u = 0; u < kGatherU; ++u) {
        const int64_t j = j0 + u * 256;
        if (j < nnz) out[j] = v[u];
    }
}

void direct_gather_values(const int32_t* bperm, const double* bval, int64_t nnz, double* out,
                          hipStream_t st) {
    if (nnz <= 0) return;
    hipLaunchKernelGGL(k_gather_bval, dim3(grid_1d(ceil_div(nnz, 256 * kGatherU))), dim3(256), 0,
                       st, bperm, bval, nnz, out);
    SG_LAUNCH_CHECK();
}

// One staged entry of a round: its slice's start in the partitioned B less
// the round's product prefix at the entry, so that the round's product p of
// the entry is B entry base + p, and its a value; 16 bytes, one LDS access.
// The direct path takes B with at most INT32_MAX entries, so B positions
// (and base, which lies above -2^31) are kept in 32 bits: fewer registers
// per product in flight.
struct alignas(16) StagedEntry {
    int32_t base;
    int32_t pad;
    double a;
};

// Staging of one round of an item's A entries (at most NE of them, taken by
// threads tt < NE): each entry's StagedEntry and the exclusive prefix of
// slice lengths (s_pre). Returns the products of the round. Threads past
// the item's entries add 0.
template <int TW, int NE, bool OCC>
__device__ __forceinline__ int direct_stage(const DirectArgs& d, int64_t q, int64_t q1, int s,
                                            int* s_pre, StagedEntry* s_e, int* red_sh) {
    const int tt = threadIdx.x;
    int len = 0;
    int32_t lo = 0;
    double a = 0.0;
    if (tt < NE && q < q1) {
        const int32_t k = d.Acol[q];
        a = d.Aval[q];
        // with the occupancy bits, an empty (B row, slot) slice reads no bounds
        if (!OCC || (d.eocc[(int64_t)(s >> 5) * d.annz + q] >> (s & 31)) & 1u) {
            const int32_t* sp = d.spos + (int64_t)s * d.nb + k;
            lo = sp[0];
            len = (int)(sp[1] - lo);
        }
    }
    int tot;
    int pre;
    if constexpr (NE < TW)
        pre = block_scan_first<NE>(len, red_sh, &tot);  // one barrier
    else
        pre = team_scan_fast<TW>(len, red_sh, &tot);
    if (tt < NE) {
        s_pre[tt] = pre;
        s_e[tt] = StagedEntry{(int32_t)(lo - pre), 0, a};
    }
    __syncthreads();
    return tot;
}

// The first staging round of an item, loaded into registers so that two
// items' loads can be in flight together: this thread's entry q (a valid
// index of the item's row; `valid` is false past the row's entries, whose
// slice then counts as empty).
template <bool OCC>
__device__ __forceinline__ void stage_load(const DirectArgs& d, int64_t q, bool valid, int s,
                                           double& a, int32_t& lo, int& len) {
    const int32_t k = d.Acol[q];
    a = d.Aval[q];
    lo = 0;
    len = 0;
    if (!OCC || (d.eocc[(int64_t)(s >> 5) * d.annz + q] >> (s & 31)) & 1u) {
        const int32_t* sp = d.spos + (int64_t)s * d.nb + k;
        lo = sp[0];
        len = (int)(sp[1] - lo);
    }
    if (!valid) len = 0;
}

// Puts a round loaded by stage_load into LDS as direct_stage does (one entry
// per thread of the team); returns the round's products.
template <int TW>
__device__ __forceinline__ int stage_commit(double a, int32_t lo, int len, int* s_pre,
                                            StagedEntry* s_e, int* red_sh) {
    const int tt = threadIdx.x;
    int tot;
    const int pre = team_scan_fast<TW>(len, red_sh, &tot);
    s_pre[tt] = pre;
    s_e[tt] = StagedEntry{(int32_t)(lo - pre), 0, a};
    __syncthreads();
    return tot;
}

// Entry of product p of a round: the last staged entry whose prefix is <= p,
// searched from `j` up (products are visited in increasing order per thread).
__device__ __forceinline__ int direct_find(const int* s_pre, int ne, int p, int j) {
    int jh = ne;
    while (jh - j > 1) {
        const int mid = (j + jh) >> 1;
        if (s_pre[mid] <= p) j = mid; else jh = mid;
    }
    return j;
}

// Entry of product base + lane for a chunk of 64 consecutive products whose
// first product lies in entry jc. Lane w reads the start of entry jc+1+w;
// with at most kWalkMax of them inside the chunk, each lane keeps the last
// one starting at or before its product (the ballot's bits taken lowest
// first, as starts rise); with more, lane w adds one to the byte of lane d_w
// in the wave's 16 LDS words `hw` (zero on entry and on exit) and a scan of
// the counts gives every lane the entries starting at or before it; if all
// 64 start inside the chunk, each lane searches the staged prefix.
constexpr int kWalkMax = 4;
__device__ __forceinline__ int chunk_entry_fast(const int* s_pre, int ne, int base, int jc, int lane,
                                                uint32_t* hw) {
    const int win = jc + 1 + lane;
    const int dw = win < ne ? s_pre[win] - base : kWave;
    uint64_t m = __ballot(dw < kWave);
    // 64 or more entries start inside the chunk (mostly empty slices, as
    // when B rows are short against the number of slots): a search per lane
    if (m == ~0ull) return direct_find(s_pre, ne, base + lane, jc);
    if (__popcll(m) <= kWalkMax) {
        int e = jc;
        while (m) {
            const int w = __ffsll((unsigned long long)m) - 1;
            if (lane >= __builtin_amdgcn_readlane(dw, w)) e = jc + 1 + w;
            m &= m - 1;
        }
        return e;
    }
    if (dw < kWave) atomicAdd(&hw[dw >> 2], 1u << ((dw & 3) * 8));
    wave_lds_sync();
    const int cnt = (int)((hw[lane >> 2] >> ((lane & 3) * 8)) & 0xffu);
    wave_lds_sync();
    if (lane < kWave / 4) hw[lane] = 0u;
    return jc + wave_inclusive_scan_i32(cnt);
}

// Bitmap-rank accumulation of one item with at most TW*KPT products: the
// products are formed into registers, then accumulated as in the chunk
// accumulator (bitmap of the chunk's columns, word-popcount prefix for the
// ranks, values summed at their rank) and written sorted. The first staging
// round arrives in registers (a0, lo0, len0: this thread's entry q0 + tt).
template <int TW, int KPT, bool OCC>
__device__ __forceinline__ void rank_item(const DirectArgs& d, int32_t x, int64_t q0, int64_t q1,
                                          int64_t off, double a0, int32_t lo0, int len0,
                                          double* vals, uint32_t* bits, int* wpre, int* s_pre,
                                          StagedEntry* s_e, int* red_sh) {
    const int W = 1 << d.logW;
    const int NWD = W >> 5;
    const int tt = threadIdx.x;
    const int s = (int)((uint32_t)x & (uint32_t)(d.req - 1));  // req is a power of two
    // one-wave items of at most 128 products are ranked through the
    // two-level bitmap (work by product); larger ones through the chunk's
    // full bitmap
    constexpr bool kTwoLevel = TW == kWave && KPT <= 2;
    if constexpr (!kTwoLevel)
        for (int wd = tt; wd < NWD; wd += TW) bits[wd] = 0u;

    uint32_t idx[KPT];
    double v[KPT];
#pragma unroll
    for (int k = 0; k < KPT; ++k) idx[k] = 0xffffffffu;
    int done = 0;
    for (int64_t qb = q0; qb < q1; qb += TW) {
        const int tot = qb == q0
                            ? stage_commit<TW>(a0, lo0, len0, s_pre, s_e, red_sh)
                            : direct_stage<TW, TW, OCC>(d, qb + tt, q1, s, s_pre, s_e, red_sh);
        const int ne = (int)min((int64_t)TW, q1 - qb);
        int32_t bi[KPT];
        double av[KPT];
        int j = 0;
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            const int p = k * TW + tt - done;
            bi[k] = -1;
            if (p >= 0 && p < tot) {
                j = direct_find(s_pre, ne, p, j);
                const StagedEntry se = s_e[j];
                bi[k] = se.base + p;
                av[k] = se.a;
            }
        }
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            if (bi[k] >= 0) {
                idx[k] = d.bcol16[bi[k]];
                v[k] = av[k] * d.bval[bi[k]];
            }
        }
        done += tot;
        __syncthreads();  // the next round restages
    }
    if constexpr (kTwoLevel) {
        // the staged entries are free once the products are formed
        wave_rank_emit<KPT>(idx, v, W, bits, vals, (uint16_t*)s_e, s << d.logW, d.Ccol + off,
                            d.Cval + off, true);
        return;
    }
#pragma unroll
    for (int k = 0; k < KPT; ++k)
        if (idx[k] < (uint32_t)W) atomicOr(&bits[idx[k] >> 5], 1u << (idx[k] & 31));
    __syncthreads();
    const int per = (NWD + TW - 1) / TW;
    const int w0 = min(NWD, tt * per), w1 = min(NWD, w0 + per);
    int pc = 0;
    for (int wd = w0; wd < w1; ++wd) pc += __popc(bits[wd]);
    int tot;
    int pre = team_scan_fast<TW>(pc, red_sh, &tot);
    for (int wd = w0; wd < w1; ++wd) {
        wpre[wd] = pre;
        pre += __popc(bits[wd]);
    }
    for (int r = tt; r < tot; r += TW) vals[r] = 0.0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
        if (idx[k] < (uint32_t)W) {
            const uint32_t wd = idx[k] >> 5;
            const int rank = wpre[wd] + __popc(bits[wd] & ((1u << (idx[k] & 31)) - 1u));
            atomicAdd(&vals[rank], v[k]);
        }
    }
    // each column at its rank, in the staging area (free once the products
    // are formed), so that columns and values are written out coalesced
    static_assert(KPT * 2 <= (int)sizeof(StagedEntry), "the ranked columns fit the staging area");
    uint16_t* scol = (uint16_t*)s_e;
    for (int wd = w0; wd < w1; ++wd) {
        uint32_t bw = bits[wd];
        int r = wpre[wd];
        while (bw) {
            const int b = __ffs(bw) - 1;
            bw &= bw - 1;
            scol[r++] = (uint16_t)(wd * 32 + b);
        }
    }
    __syncthreads();
    const int32_t lo = s << d.logW;
    for (int r = tt; r < tot; r += TW) {
        d.Ccol[off + r] = lo + scol[r];
        d.Cval[off + r] = vals[r];
    }
}

// IPG consecutive items of a class per work group, one after the other: all
// their headers, first-round A entries and slice bounds are loaded together
// before the first item is accumulated, so the later items' dependent-load
// chains are mostly paid while the first one runs.
template <int TW, int KPT, bool OCC, int IPG>
__global__ __launch_bounds__(TW) void k_direct_rank(DirectArgs d, int64_t p0, int64_t nitems) {
    extern __shared__ int64_t lds_r[];
    const int W = 1 << d.logW;
    double* vals = (double*)lds_r;                  // TW*KPT
    uint32_t* bits = (uint32_t*)(vals + TW * KPT);  // W/32
    int* wpre = (int*)(bits + (W >> 5));            // W/32
    __shared__ int s_pre[TW];
    __shared__ StagedEntry s_e[TW];
    __shared__ int red_sh[TW / kWave + 1];
    const int tt = threadIdx.x;
    const int64_t i0 = (int64_t)blockIdx.x * IPG;
    if (i0 >= nitems) return;
    const int nown = (int)min((int64_t)IPG, nitems - i0);  // uniform over the group
    int32_t x[IPG];
    int64_t q0[IPG], ne[IPG], off[IPG];
#pragma unroll
    for (int u = 0; u < IPG; ++u) {
        const int64_t i = p0 + i0 + min(u, nown - 1);
        x[u] = d.items[i];
        q0[u] = d.iq0[i];
        ne[u] = d.ine[i];
    }
    // the output offsets are read now, beside the items' entries, rather
    // than after the accumulation
#pragma unroll
    for (int u = 0; u < IPG; ++u) off[u] = d.off[x[u]];
    // A rank item has products, so its row has at least one entry; the
    // index is clamped into the row so that every thread's loads stay in
    // bounds. All loads of the items are issued before any is used.
    double a[IPG];
    int32_t lo[IPG];
    int len[IPG];
    if constexpr (!OCC) {
        int32_t k[IPG];
#pragma unroll
        for (int u = 0; u < IPG; ++u) {
            const int64_t q = q0[u] + min((int64_t)tt, ne[u] - 1);
            k[u] = d.Acol[q];
            a[u] = d.Aval[q];
        }
        int32_t hi[IPG];
#pragma unroll
        for (int u = 0; u < IPG; ++u) {
            const int s = (int)((uint32_t)x[u] & (uint32_t)(d.req - 1));
            const int32_t* sp = d.spos + (int64_t)s * d.nb + k[u];
            lo[u] = sp[0];
            hi[u] = sp[1];
        }
#pragma unroll
        for (int u = 0; u < IPG; ++u) len[u] = tt < ne[u] ? (int)(hi[u] - lo[u]) : 0;
    } else {
#pragma unroll
        for (int u = 0; u < IPG; ++u) {
            const int s = (int)((uint32_t)x[u] & (uint32_t)(d.req - 1));
            stage_load<OCC>(d, q0[u] + min((int64_t)tt, ne[u] - 1), tt < ne[u], s, a[u], lo[u],
                            len[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < IPG; ++u) {
        if (u < nown) {
            // the previous item's output has read the staging area and bitmap
            if (u > 0) __syncthreads();
            rank_item<TW, KPT, OCC>(d, x[u], q0[u], q0[u] + ne[u], off[u], a[u], lo[u], len[u],
                                    vals, bits, wpre, s_pre, s_e, red_sh);
        }
    }
}

// A run's products: each round gives every lane one (entry, slot) pair of
// the run, lane = j * nns + t for entry eb + j of the row and the t-th slot
// of the mask (epr = 64 / nns entries a round; the lanes past epr * nns
// idle), the slices are scanned and each lane forms up to two of the run's
// products. The two-level bitmap then ranks the run's columns over the
// span of its slots and writes the run's output, which is its items'
// outputs one after the other. The first round arrives in registers.
template <bool OCC>
__device__ __forceinline__ void run_item(const DirectArgs& d, int64_t hdr, int64_t q0, int ne,
                                         int64_t off, int jl, int ds, int epr, double a0,
                                         int32_t lo0, int len0, int WR, double* vals, void* rk,
                                         int* s_pre, StagedEntry* s_e, int* s_cb) {
    constexpr int KPT = kRunKPT;
    static_assert(kWave * KPT == kRunMax, "one wavefront holds a run's products");
    const int lane = lane_id();
    const int32_t x = (int32_t)hdr;
    const int s0 = (int)((uint32_t)x & (uint32_t)(d.req - 1));  // req is a power of two
    const int s = s0 + ds;
    s_cb[lane] = ds << d.logW;
    uint32_t idx[KPT];
    double v[KPT];
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
        idx[k] = 0xffffffffu;
        v[k] = 0.0;
    }
    int done = 0;
    for (int eb = 0; eb < ne; eb += epr) {
        double a = a0;
        int32_t lo = lo0;
        int len = len0;
        if (eb > 0) {
            const int j = eb + jl;
            const int64_t q = q0 + min(j, ne - 1);
            const int32_t k = d.Acol[q];
            a = d.Aval[q];
            lo = 0;
            len = 0;
            // with the occupancy bits, an empty slice reads no bounds
            if (!OCC || (d.eocc[(int64_t)(s >> 5) * d.annz + q] >> (s & 31)) & 1u) {
                const int32_t* sp = d.spos + (int64_t)s * d.nb + k;
                lo = sp[0];
                len = (jl < epr && j < ne) ? (int)(sp[1] - lo) : 0;
            }
        }
        const int inc = wave_inclusive_scan(len);
        const int tot = __shfl(inc, kWave - 1, kWave);
        s_pre[lane] = inc - len;
        s_e[lane] = StagedEntry{(int32_t)(lo - (inc - len)), 0, a};
        wave_lds_sync();
        int32_t bi[KPT];
        double av[KPT];
        int cb[KPT];
        int j = 0;
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            const int p = k * kWave + lane - done;
            bi[k] = -1;
            if (p >= 0 && p < tot) {
                j = direct_find(s_pre, kWave, p, j);
                const StagedEntry se = s_e[j];
                bi[k] = se.base + p;
                av[k] = se.a;
                cb[k] = s_cb[j];
            }
        }
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            if (bi[k] >= 0) {
                idx[k] = (uint32_t)cb[k] + d.bcol16[bi[k]];
                v[k] = av[k] * d.bval[bi[k]];
            }
        }
        done += tot;
        wave_lds_sync();  // the next round restages
    }
    // the staged entries are free once the products are formed
    wave_rank_emit<KPT>(idx, v, WR, rk, vals, (uint16_t*)s_e, s0 << d.logW, d.Ccol + off,
                        d.Cval + off, true);
}

// IPG runs per wavefront-sized work group: their headers, output offsets and
// first rounds are loaded together, as in k_direct_rank.
template <bool OCC, int IPG>
__global__ __launch_bounds__(kWave) void k_direct_runs(DirectArgs d, int64_t nruns) {
    extern __shared__ int64_t lds_u[];
    double* vals = (double*)lds_u;     // kRunMax
    void* rk = vals + kRunMax;         // wave_rank_lds(kRunKPT, run width)
    __shared__ int s_pre[kWave];
    __shared__ StagedEntry s_e[kWave];
    __shared__ int s_cb[kWave];
    const int lane = lane_id();
    const int64_t i0 = (int64_t)blockIdx.x * IPG;
    if (i0 >= nruns) return;
    const int nown = (int)min((int64_t)IPG, nruns - i0);  // uniform over the group
    const int WR = run_span(d.logW) << d.logW;
    int64_t hdr[IPG], q0[IPG], off[IPG];
    int ne[IPG];
#pragma unroll
    for (int u = 0; u < IPG; ++u) {
        const int64_t i = i0 + min(u, nown - 1);
        hdr[u] = d.rhdr[i];
        q0[u] = d.rq0[i];
        ne[u] = d.rne[i];
    }
#pragma unroll
    for (int u = 0; u < IPG; ++u) off[u] = d.off[(int32_t)hdr[u]];
    // lane roles: entry jl of each round, slot s0 + ds (t = lane mod nns < nns,
    // so the mask keeps a bit after t are cleared, also on idle lanes)
    int jl[IPG], ds[IPG], epr[IPG];
#pragma unroll
    for (int u = 0; u < IPG; ++u) {
        uint32_t m = (uint32_t)(hdr[u] >> 32);
        const int nns = __popc(m);
        epr[u] = kWave / nns;
        jl[u] = lane / nns;
        for (int t = lane - jl[u] * nns; t > 0; --t) m &= m - 1;
        ds[u] = __builtin_ctz(m);
    }
    // a run has products, so its row has an entry: the index is clamped
    // into the row and every load stays in bounds
    double a[IPG];
    int32_t lo[IPG];
    int len[IPG];
    int32_t k[IPG];
    int64_t q[IPG];
#pragma unroll
    for (int u = 0; u < IPG; ++u) {
        q[u] = q0[u] + min(jl[u], ne[u] - 1);
        k[u] = d.Acol[q[u]];
        a[u] = d.Aval[q[u]];
    }
    int32_t hi[IPG];
#pragma unroll
    for (int u = 0; u < IPG; ++u) {
        const int s = (int)((uint32_t)hdr[u] & (uint32_t)(d.req - 1)) + ds[u];
        lo[u] = 0;
        hi[u] = 0;
        if (!OCC || (d.eocc[(int64_t)(s >> 5) * d.annz + q[u]] >> (s & 31)) & 1u) {
            const int32_t* sp = d.spos + (int64_t)s * d.nb + k[u];
            lo[u] = sp[0];
            hi[u] = sp[1];
        }
    }
#pragma unroll
    for (int u = 0; u < IPG; ++u)
        len[u] = (jl[u] < epr[u] && jl[u] < ne[u]) ? (int)(hi[u] - lo[u]) : 0;
#pragma unroll
    for (int u = 0; u < IPG; ++u) {
        if (u < nown) {
            // the previous run's output has read the staging area
            if (u > 0) wave_lds_sync();
            run_item<OCC>(d, hdr[u], q0[u], ne[u], off[u], jl[u], ds[u], epr[u], a[u], lo[u],
                          len[u], WR, vals, rk, s_pre, s_e, s_cb);
        }
    }
}

// Dense window accumulation of the large items: the item's entries are
// staged kDirectNE at a time and their products streamed through an LDS
// array over the chunk's W columns (fp64 atomics) with one-byte presence
// flags; the flags then give every present column its rank in the sorted
// output, as in the chunk window accumulator.
constexpr int kDirectWinNT = 1024;
constexpr int kDirectNE = 256;
// one thread stages each entry of a round
static_assert(kDirectNE <= kDirectWinNT, "a staged round holds at most one entry per thread");
constexpr int kDirectU = 4;  // products in flight per thread
// per-wave entry-start counts: 16 words for each of the block's waves
constexpr int kWinHistWords = (kDirectWinNT / kWave) * (kWave / 4);

template <bool OCC>
__global__ __launch_bounds__(kDirectWinNT) void k_direct_window(DirectArgs d, int64_t p0,
                                                               int64_t nitems) {
    constexpr int TW = kDirectWinNT;
    extern __shared__ __align__(16) int64_t lds_w[];
    const int W = 1 << d.logW;
    const int NWD = W >> 5;
    double* acc = (double*)lds_w;                    // W
    uint32_t* flags = (uint32_t*)(acc + W);          // W bytes
    uint32_t* bits = flags + NWD * 8;                // NWD
    int* wpre = (int*)(bits + NWD);                  // NWD
    // while products accumulate, bits and wpre hold the waves' entry-start
    // counts (kWinHistWords words from bits on; the launch sizes them)
    uint32_t* hw_all = bits;
    __shared__ int s_pre[kDirectNE];
    __shared__ StagedEntry s_e[kDirectNE];
    __shared__ int red_sh[TW / kWave + 1];
    const int tt = threadIdx.x;
    const int64_t item = blockIdx.x;
    if (item >= nitems) return;
    const int32_t x = d.items[p0 + item];
    const int64_t q0 = d.iq0[p0 + item];
    const int64_t q1 = q0 + d.ine[p0 + item];
    const int64_t off = d.off[x];
    const int s = (int)((uint32_t)x & (uint32_t)(d.req - 1));  // req is a power of two
    // the first round's entries and slice bounds are loaded before the
    // window is cleared, so that the clearing runs while they arrive (a
    // dense item has entries: the index is clamped into its row)
    double a0 = 0.0;
    int32_t lo0 = 0;
    int len0 = 0;
    if (tt < kDirectNE)
        stage_load<OCC>(d, q0 + min((int64_t)tt, q1 - q0 - 1), q0 + tt < q1, s, a0, lo0, len0);
    // 16 bytes a store: W is a power of two of at least 32
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
    for (int i = tt; i < NWD * 2; i += TW) ((uint4*)flags)[i] = z4;
    for (int i = tt; i < W / 2; i += TW) ((uint4*)acc)[i] = z4;
    for (int i = tt; i < kWinHistWords; i += TW) hw_all[i] = 0u;
    uint8_t* fb = (uint8_t*)flags;
    // wave index and chunk bounds are uniform per wave: scalar registers
    const int wv = __builtin_amdgcn_readfirstlane(tt / kWave), lane = lane_id();
    uint32_t* hw = hw_all + wv * (kWave / 4);
    constexpr int NWV = TW / kWave;
    for (int64_t qb = q0; qb < q1; qb += kDirectNE) {
        __syncthreads();  // zeroing done / previous round's staging consumed
        int tot;
        if (qb == q0) {
            const int pre = block_scan_first<kDirectNE>(len0, red_sh, &tot);
            if (tt < kDirectNE) {
                s_pre[tt] = pre;
                s_e[tt] = StagedEntry{(int32_t)(lo0 - pre), 0, a0};
            }
            __syncthreads();
        } else {
            tot = direct_stage<TW, kDirectNE, OCC>(d, qb + tt, q1, s, s_pre, s_e, red_sh);
        }
        tot = __builtin_amdgcn_readfirstlane(tot);
        const int ne = (int)min((int64_t)kDirectNE, q1 - qb);
        // each wave takes a contiguous run of 64-product chunks; lane l of a
        // chunk takes product base + l
        const int nch = (tot + kWave - 1) / kWave;
        const int cpw = (nch + NWV - 1) / NWV;
        const int c0 = wv * cpw, c1 = min(nch, c0 + cpw);
        int jc = c0 < c1 ? direct_find(s_pre, ne, c0 * kWave, 0) : 0;
        for (int cb = c0; cb < c1; cb += kDirectU) {
            int32_t bi[kDirectU];
            double av[kDirectU];
#pragma unroll
            for (int u = 0; u < kDirectU; ++u) {
                bi[u] = -1;
                if (cb + u < c1) {
                    const int base = (cb + u) * kWave;
                    int e = chunk_entry_fast(s_pre, ne, base, jc, lane, hw);
                    // the chunk's last product's entry starts the next chunk
                    jc = __builtin_amdgcn_readlane(e, kWave - 1);
                    const int p = base + lane;
                    if (p < tot) {
                        const StagedEntry se = s_e[e];
                        bi[u] = se.base + p;
                        av[u] = se.a;
                    }
                }
            }
            uint32_t c[kDirectU];
            double bv[kDirectU];
#pragma unroll
            for (int u = 0; u < kDirectU; ++u) {
                if (bi[u] >= 0) {
                    c[u] = d.bcol16[bi[u]];
                    bv[u] = d.bval[bi[u]];
                }
            }
#pragma unroll
            for (int u = 0; u < kDirectU; ++u) {
                if (bi[u] >= 0) {
                    fb[c[u]] = 1;
                    atomicAdd(&acc[c[u]], av[u] * bv[u]);
                }
            }
        }
    }
    __syncthreads();
    const int per = (NWD + TW - 1) / TW;
    const int w0 = min(NWD, tt * per), w1 = min(NWD, w0 + per);
    int pc = 0;
    for (int wd = w0; wd < w1; ++wd) {
        const uint32_t m = pack_flags32(flags + wd * 8);
        bits[wd] = m;
        pc += __popc(m);
    }
    int tot;
    int pre = block_scan_first<TW>(pc, red_sh, &tot);
    for (int wd = w0; wd < w1; ++wd) {
        wpre[wd] = pre;
        pre += __popc(bits[wd]);
    }
    __syncthreads();
    const int32_t lo = s << d.logW;
    for (int i = tt; i < W; i += TW) {
        const uint32_t word = bits[i >> 5];
        const uint32_t bit = 1u << (i & 31);
        if (word & bit) {
            const int rank = wpre[i >> 5] + __popc(word & (bit - 1));
            d.Ccol[off + rank] = lo + i;
            d.Cval[off + rank] = acc[i];
        }
    }
}

// Per class of items (dense window / bitmap rank / runs): products, output
// entries, and A entries read (a dense or rank item reads all of its row's
// entries; the runs count theirs when they are formed), for the algorithmic
// byte counts. out8 = {dense: products, outputs, entries, rank: products,
// outputs, entries, runs: products, outputs}.
constexpr int kDirectTotals = 8;

__global__ __launch_bounds__(256) void k_direct_totals(const int64_t* hq0, const int64_t* hq1,
                                                      int64_t nitems, int logreq,
                                                      const int64_t* elem_fin,
                                                      const int64_t* dist_fin, int64_t* part) {
    __shared__ int64_t sh[256 / kWave + 1];
    int64_t v[kDirectTotals] = {};
    int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; x < nitems; x += stride) {
        const int64_t e = elem_fin[x];
        if (e == 0) continue;
        const int64_t h = x >> logreq;  // req is a power of two
        const int64_t o = dist_fin[x];
        if (e <= kRunMax) {
            v[6] += e;
            v[7] += o;
            continue;
        }
        const int c = e > kDirectDense ? 0 : 3;
        v[c] += e;
        v[c + 1] += o;
        v[c + 2] += hq1[h] - hq0[h];
    }
#pragma unroll
    for (int i = 0; i < kDirectTotals; ++i) {
        const int64_t r = block_reduce_sum<256>(v[i], sh);
        if (threadIdx.x == 0) part[(int64_t)i * gridDim.x + blockIdx.x] = r;
    }
}

// out[i] = sum of the groups' partial sums i, for i < nv (one work group).
__global__ __launch_bounds__(256) void k_sum_parts(const int64_t* part, int nparts, int nv,
                                                   int64_t* out) {
    __shared__ int64_t sh[256 / kWave + 1];
    for (int i = 0; i < nv; ++i) {
        int64_t v = 0;
        for (int b = threadIdx.x; b < nparts; b += 256) v += part[(int64_t)i * nparts + b];
        v = block_reduce_sum<256>(v, sh);
        if (threadIdx.x == 0) out[i] = v;
    }
}

void direct_totals(const int64_t* hq0, const int64_t* hq1, int64_t H, int req,
                   const int64_t* elem_fin, const int64_t* dist_fin, int64_t* out8, Arena& ar,
                   hipStream_t st) {
    const int64_t n = H * req;
    if (n <= 0) {
        fill<int64_t>(out8, kDirectTotals, 0, st);
        return;
    }
    // partial sums per group, then one group adds them: no shared counter
    const int blocks = (int)std::min<int64_t>(ceil_div(n, 256), 2048);
    int64_t* part = ar.get<int64_t>("dtot_parts", (size_t)kDirectTotals * blocks);
    hipLaunchKernelGGL(k_direct_totals, dim3(blocks), dim3(256), 0, st, hq0, hq1, n, ilog2(req),
                       elem_fin, dist_fin, part);
    SG_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_sum_parts, dim3(1), dim3(256), 0, st, part, blocks, kDirectTotals, out8);
    SG_LAUNCH_CHECK();
}

// ---------------------------------------------------------------- work lists
// One thread per heavy row walks its slots in order (16-slot batches of the
// item counts, 16 bytes a load) and
// - forms the row's runs (see run_span and kRunMax): markT (slot-major,
//   req x H bytes) receives the run's slot mask at (s0, h) and 0 at every
//   other slot, so that a scan in slot-major order numbers the runs slot by
//   slot;
// - writes each item's class among the listed rank classes (those the runs
//   do not take: 0 .. kListedRank - 1, else kNotListed) to clsT, slot-major;
// - counts the row's dense items (dcnt).
// part: per work group, the A entries and the (entry, slot) pairs its runs
// read. With `fill`, the walk instead lists the row's dense items at
// dpos[h] (items, and the row's first A entry and entry count).
constexpr int kRunBatch = 16;
constexpr int kListedRank = kNumRankClasses - kRunClasses;
constexpr uint8_t kNotListed = 0xff;

__device__ __forceinline__ uint8_t listed_rank_class(int64_t c) {
    if (c <= kRunMax || c > kDirectDense) return kNotListed;
    int r = 0;
#pragma unroll
    for (int j = kRunClasses; j + 1 < kNumRankClasses; ++j) r += c > kRankClassMax[j];
    return (uint8_t)r;
}

template <bool FILL>
__global__ __launch_bounds__(256) void k_items_walk(const int64_t* elem_fin, int64_t H, int req,
                                                    int span, const int64_t* hq0,
                                                    const int64_t* hq1, uint8_t* markT,
                                                    uint8_t* clsT, int64_t* dcnt, int64_t* part,
                                                    const int64_t* dpos, int32_t* items,
                                                    int64_t* iq0, int32_t* ine) {
    __shared__ int64_t sh[256 / kWave + 1];
    const int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t ent = 0, pairs = 0;
    if (h < H) {
        const int64_t q0 = hq0[h], ne = hq1[h] - q0;
        const int64_t* e = elem_fin + h * req;
        int64_t nd = 0, dp = FILL ? dpos[h] : 0;
        int s0 = -1;
        uint32_t mask = 0;
        int64_t cur = 0;
        for (int sb = 0; sb < req; sb += kRunBatch) {
            int64_t c[kRunBatch];
            if (req >= kRunBatch) {
                // req is a power of two: the batch is 128-byte aligned
                const uint4* e4 = (const uint4*)(e + sb);
#pragma unroll
                for (int t = 0; t < kRunBatch / 2; ++t) {
                    const uint4 v = e4[t];
                    c[2 * t] = (int64_t)(((uint64_t)v.y << 32) | v.x);
                    c[2 * t + 1] = (int64_t)(((uint64_t)v.w << 32) | v.z);
                }
            } else {
#pragma unroll
                for (int t = 0; t < kRunBatch; ++t) c[t] = t < req ? e[t] : 0;
            }
#pragma unroll
            for (int t = 0; t < kRunBatch; ++t) {
                const int s = sb + t;
                if (s >= req) break;
                const int64_t cs = c[t];
                if constexpr (FILL) {
                    if (cs > kDirectDense) {
                        items[dp] = (int32_t)(h * req + s);
                        iq0[dp] = q0;
                        ine[dp] = (int32_t)ne;
                        ++dp;
                    }
                    continue;
                }
                markT[(int64_t)s * H + h] = 0;
                clsT[(int64_t)s * H + h] = listed_rank_class(cs);
                nd += cs > kDirectDense;
                if (cs == 0) continue;
                // a larger item writes between: the run cannot span it
                const bool big = cs > kRunMax;
                if (s0 >= 0 && (big || cur + cs > kRunMax || s - s0 >= span)) {
                    markT[(int64_t)s0 * H + h] = (uint8_t)mask;
                    ent += ne;
                    pairs += ne * __popc(mask);
                    s0 = -1;
                }
                if (big) continue;
                if (s0 < 0) {
                    s0 = s;
                    mask = 0;
                    cur = 0;
                }
                cur += cs;
                mask |= 1u << (s - s0);
            }
        }
        if constexpr (!FILL) {
            if (s0 >= 0) {
                markT[(int64_t)s0 * H + h] = (uint8_t)mask;
                ent += ne;
                pairs += ne * __popc(mask);
            }
            dcnt[h] = nd;
        }
    }
    if constexpr (!FILL) {
        ent = block_reduce_sum<256>(ent, sh);
        pairs = block_reduce_sum<256>(pairs, sh);
        if (threadIdx.x == 0) {
            part[blockIdx.x] = ent;
            part[gridDim.x + blockIdx.x] = pairs;
        }
    }
}

struct RunStart {
    const uint8_t* markT;
    __device__ int64_t operator()(int64_t i) const { return markT[i] != 0; }
};

// Bin of slot-major position i for the partition of the listed rank
// classes (-1: not listed).
struct ListedClass {
    const uint8_t* clsT;
    __device__ int operator()(int64_t i) const {
        const int c = clsT[i];
        return c == kNotListed ? -1 : c;
    }
};

// rpos: exclusive scan of RunStart over req x H (+1).
__global__ __launch_bounds__(256) void k_runs_scatter(const uint8_t* markT, const int64_t* rpos,
                                                      int64_t H, int req, const int64_t* hq0,
                                                      const int64_t* hq1, int64_t* rhdr,
                                                      int64_t* rq0, int32_t* rne) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= H * req) return;
    const uint32_t m = markT[i];
    if (!m) return;
    const int64_t s0 = i / H, h = i - s0 * H;
    const int64_t j = rpos[i];
    const int64_t q0 = hq0[h];
    rhdr[j] = (h * req + s0) | ((int64_t)m << 32);
    rq0[j] = q0;
    rne[j] = (int32_t)(hq1[h] - q0);
}

// The listed rank classes' items after the dense ones: position p of the
// slot-major partition (perm: slot-major index) goes to items[ndense + p].
__global__ __launch_bounds__(256) void k_rank_items(const int32_t* perm, const int64_t* lbins,
                                                    const int64_t* dpos, int64_t H, int req,
                                                    const int64_t* hq0, const int64_t* hq1,
                                                    int32_t* items, int64_t* iq0, int32_t* ine) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= lbins[kListedRank]) return;
    const int64_t i = perm[p];
    const int64_t s = i / H, h = i - s * H;
    const int64_t d = dpos[H] + p;
    const int64_t q0 = hq0[h];
    items[d] = (int32_t)(h * req + s);
    iq0[d] = q0;
    ine[d] = (int32_t)(hq1[h] - q0);
}

// The class starts (DC_COUNT + 1: dense, the rank classes, empty; the run
// classes and the empty class are empty ranges) and the run count.
__global__ void k_class_bins(const int64_t* dpos, int64_t H, const int64_t* lbins,
                             const int64_t* rpos, int64_t n, int64_t* bins, int64_t* run_meta) {
    const int64_t nd = dpos[H];
    bins[DC_DENSE] = 0;
    for (int r = 0; r <= kRunClasses; ++r) bins[DC_RANK0 + r] = nd;
    for (int r = 1; r <= kListedRank; ++r) bins[DC_RANK0 + kRunClasses + r] = nd + lbins[r];
    bins[DC_COUNT] = nd + lbins[kListedRank];
    run_meta[0] = rpos[n];
}

void direct_classify(const int64_t* elem_fin, int64_t H, int req, int logW, const int64_t* hq0,
                     const int64_t* hq1, int32_t* items, int64_t* iq0, int32_t* ine,
                     int64_t* bins, int64_t* rhdr, int64_t* rq0, int32_t* rne, int64_t* run_meta,
                     Arena& ar, hipStream_t st) {
    static_assert(DC_RANK0 + kNumRankClasses == DC_EMPTY && DC_EMPTY + 1 == DC_COUNT,
                  "class layout");
    if (H <= 0) {
        fill<int64_t>(bins, DC_COUNT + 1, 0, st);
        fill<int64_t>(run_meta, 3, 0, st);
        return;
    }
    const int64_t n = H * req;
    const int64_t blocks = ceil_div(H, 256);
    uint8_t* markT = ar.get<uint8_t>("run_mark", (size_t)n);
    uint8_t* clsT = ar.get<uint8_t>("item_cls", (size_t)n);
    int64_t* dpos = ar.get<int64_t>("dense_pos", (size_t)H + 1);
    int64_t* part = ar.get<int64_t>("run_parts", (size_t)(2 * blocks));
    const int span = run_span(logW);
    hipLaunchKernelGGL(k_items_walk<false>, dim3(grid_1d(blocks)), dim3(256), 0, st, elem_fin, H,
                       req, span, hq0, hq1, markT, clsT, dpos, part, (const int64_t*)nullptr,
                       (int32_t*)nullptr, (int64_t*)nullptr, (int32_t*)nullptr);
    SG_LAUNCH_CHECK();
    // the dense items, row by row
    scan_exclusive(LoadI64{dpos}, H, dpos, ar, st);
    hipLaunchKernelGGL(k_items_walk<true>, dim3(grid_1d(blocks)), dim3(256), 0, st, elem_fin, H,
                       req, span, hq0, hq1, (uint8_t*)nullptr, (uint8_t*)nullptr,
                       (int64_t*)nullptr, (int64_t*)nullptr, (const int64_t*)dpos, items, iq0,
                       ine);
    SG_LAUNCH_CHECK();
    // the listed rank classes, slot by slot: items of one slot that run
    // together share that slot's slice starts and B entries in cache
    int32_t* perm = ar.get<int32_t>("item_perm", (size_t)n);
    int64_t* lbins = ar.get<int64_t>("item_lbins", (size_t)kListedRank + 1);
    partition(ListedClass{clsT}, n, kListedRank, perm, (int32_t*)nullptr, lbins, ar, st);
    hipLaunchKernelGGL(k_rank_items, dim3(grid_1d(ceil_div(n, 256))), dim3(256), 0, st, perm,
                       lbins, dpos, H, req, hq0, hq1, items, iq0, ine);
    SG_LAUNCH_CHECK();
    // the runs, in the order of their first slot
    int64_t* rpos = ar.get<int64_t>("run_pos", (size_t)n + 1);
    scan_exclusive(RunStart{markT}, n, rpos, ar, st);
    hipLaunchKernelGGL(k_runs_scatter, dim3(grid_1d(ceil_div(n, 256))), dim3(256), 0, st, markT,
                       rpos, H, req, hq0, hq1, rhdr, rq0, rne);
    SG_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_class_bins, dim3(1), dim3(1), 0, st, dpos, H, lbins, rpos, n, bins,
                       run_meta);
    SG_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_sum_parts, dim3(1), dim3(256), 0, st, part, (int)blocks, 2,
                       run_meta + 1);
    SG_LAUNCH_CHECK();
}

// items per work group of the rank classes: 4 where a thread forms one or
// two products, 2 where it forms four (their registers allow no more)
constexpr int RANK_IPG_S = 4, RANK_IPG_L = 2;

template <int TW, int KPT, int IPG>
static void launch_direct_rank(const DirectArgs& d, int64_t p0, int64_t n, hipStream_t st) {
    const int64_t W = int64_t(1) << d.logW;
    size_t lds = (size_t)TW * KPT * 8 + (size_t)(W / 32) * 8;
    if (TW == kWave && KPT <= 2)
        lds = std::max(lds, (size_t)TW * KPT * 8 + (size_t)wave_rank_lds(KPT, W));
    auto kern = d.occ ? k_direct_rank<TW, KPT, true, IPG> : k_direct_rank<TW, KPT, false, IPG>;
    SG_HIP(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds));
    hipLaunchKernelGGL(kern, dim3(grid_1d((n + IPG - 1) / IPG)), dim3(TW), lds, st, d, p0, n);
    SG_LAUNCH_CHECK();
}

void direct_accumulate_runs(const DirectArgs& d, int64_t nruns, hipStream_t st) {
    if (nruns <= 0) return;
    const int WR = run_span(d.logW) << d.logW;
    const size_t lds = (size_t)kRunMax * 8 + (size_t)wave_rank_lds(kRunKPT, WR);
    constexpr int IPG = 2;
    auto kern = d.eocc ? k_direct_runs<true, IPG> : k_direct_runs<false, IPG>;
    hipLaunchKernelGGL(kern, dim3(grid_1d(ceil_div(nruns, IPG))), dim3(kWave), lds, st, d, nruns);
    SG_LAUNCH_CHECK();
}

size_t direct_window_lds(int64_t W) {
    return (size_t)W * 9 + std::max<size_t>((size_t)(W / 32) * 8, (size_t)kWinHistWords * 4);
}

void direct_accumulate(const DirectArgs& d, int cls, int64_t p0, int64_t n, hipStream_t st) {
    if (n <= 0) return;
    // teams of TW threads with KPT products each: TW * KPT is the class's
    // largest item
    static_assert(kRankClassMax[0] == 64 * 1 && kRankClassMax[1] == 64 * 2 &&
                      kRankClassMax[2] == 64 * 4 && kRankClassMax[3] == 128 * 4 &&
                      kRankClassMax[4] == 256 * 4 && kRankClassMax[5] == 512 * 4,
                  "rank class table and kernel teams disagree");
    switch (cls) {
        case DC_DENSE: {
            const int64_t W = int64_t(1) << d.logW;
            const size_t lds = direct_window_lds(W);
            auto kern = d.occ ? k_direct_window<true> : k_direct_window<false>;
            SG_HIP(hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
            hipLaunchKernelGGL(kern, dim3(grid_1d(n)), dim3(kDirectWinNT), lds, st, d,
                               p0, n);
            SG_LAUNCH_CHECK();
            break;
        }
        case DC_RANK0 + 0: launch_direct_rank<64, 1, RANK_IPG_S>(d, p0, n, st); break;
        case DC_RANK0 + 1: launch_direct_rank<64, 2, RANK_IPG_S>(d, p0, n, st); break;
        case DC_RANK0 + 2: launch_direct_rank<64, 4, RANK_IPG_L>(d, p0, n, st); break;
        case DC_RANK0 + 3: launch_direct_rank<128, 4, RANK_IPG_L>(d, p0, n, st); break;
        case DC_RANK0 + 4: launch_direct_rank<256, 4, RANK_IPG_L>(d, p0, n, st); break;
        case DC_RANK0 + 5: launch_direct_rank<512, 4, RANK_IPG_L>(d, p0, n, st); break;
        default: throw std::logic_error("not a direct item class");
    }
}

}  // namespace sg
