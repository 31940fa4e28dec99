// Heavy-row path of the gMAGNUS page (the heavy branch of Algorithm 3):
// masked CSR-to-CSC of the heavy rows, the outer product into C-hat
// (Section III-B, Algorithm 4), and the hierarchical multisplit that
// reorders every heavy row into column-range chunks (Section III-C,
// Algorithm 5), plus the small kernels that turn chunk counts into C's
// row counts and chunk output offsets.
#include "kernels.h"
#include "primitives.h"

namespace sg {

// ---------------------------------------------------------------- C-hat rowptr
struct HeavyRowProducts {
    const int64_t* arp;
    const int64_t* S;
    const int32_t* hrows;
    __device__ int64_t operator()(int64_t h) const {
        int32_t r = hrows[h];
        return S[arp[r + 1]] - S[arp[r]];
    }
};

void heavy_rowptr(const DevCSR& A, const int64_t* S, const int32_t* hrows, int64_t H,
                  int64_t* chat_rp, Arena& ar, hipStream_t st) {
    scan_exclusive(HeavyRowProducts{A.rp, S, hrows}, H, chat_rp, ar, st);
}

// ---------------------------------------------------------------- masked CSR -> CSC
// One wavefront per heavy row walks its A entries. Entries whose B row is
// empty produce nothing and are dropped (they would be empty slices).
__global__ __launch_bounds__(256) void k_csc_count(const int64_t* arp, const int32_t* acol,
                                                   const int64_t* brp, const int32_t* hrows,
                                                   int64_t H, int32_t* colcnt) {
    int64_t h = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    if (h >= H) return;
    int32_t r = hrows[h];
    for (int64_t q = arp[r] + lane_id(); q < arp[r + 1]; q += kWave) {
        int32_t k = acol[q];
        if (brp[k + 1] > brp[k]) atomicAdd(&colcnt[k], 1);
    }
}

// The position of an entry's first product inside its C-hat row is the
// number of products of the entries before it in the same A row, which the
// InterOffsets prefix S already holds: no atomics on C-hat.rowPtr are needed.
__global__ __launch_bounds__(256) void k_csc_fill(const int64_t* arp, const int32_t* acol,
                                                  const int64_t* brp, const int32_t* hrows,
                                                  int64_t H, const int64_t* S,
                                                  const int64_t* chat_rp, int64_t dest_base,
                                                  unsigned long long* cursor, int32_t* ent_k,
                                                  int64_t* ent_q, int64_t* ent_dest) {
    int64_t h = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    if (h >= H) return;
    int32_t r = hrows[h];
    int64_t a0 = arp[r];
    int64_t base = chat_rp[h] - dest_base - S[a0];
    for (int64_t q = a0 + lane_id(); q < arp[r + 1]; q += kWave) {
        int32_t k = acol[q];
        if (brp[k + 1] > brp[k]) {
            int64_t slot = (int64_t)atomicAdd(&cursor[k], 1ull);
            ent_k[slot] = k;
            ent_q[slot] = q;
            ent_dest[slot] = base + S[q];
        }
    }
}

struct LoadI32AsI64 {
    const int32_t* p;
    __device__ int64_t operator()(int64_t i) const { return p[i]; }
};
// Pieces of 64 products (one per lane of a wavefront) per CSC entry.
struct SlicePieces {
    const int32_t* ent_k;
    const int64_t* brp;
    __device__ int64_t operator()(int64_t e) const {
        int32_t k = ent_k[e];
        return (brp[k + 1] - brp[k] + kWave - 1) / kWave;
    }
};

int64_t masked_csr2csc(const DevCSR& A, const DevCSR& B, const int64_t* S, const int32_t* hrows,
                       int64_t H, const int64_t* chat_rp, int64_t dest_base, int32_t* ent_k,
                       int64_t* ent_q, int64_t* ent_dest, int64_t ent_capacity, int64_t* P,
                       int64_t* total_pieces, Arena& ar, hipStream_t st) {
    int32_t* colcnt = ar.get<int32_t>("csc_colcnt", (size_t)A.m + 1);
    int64_t* colptr = ar.get<int64_t>("csc_colptr", (size_t)A.m + 1);
    fill<int32_t>(colcnt, A.m, 0, st);
    int64_t blocks = ceil_div(H * kWave, 256);
    hipLaunchKernelGGL(k_csc_count, dim3(grid_1d(blocks)), dim3(256), 0, st, A.rp, A.col, B.rp,
                       hrows, H, colcnt);
    SG_LAUNCH_CHECK();
    scan_exclusive(LoadI32AsI64{colcnt}, A.m, colptr, ar, st);
    int64_t ne = 0;
    SG_HIP(hipMemcpyAsync(&ne, colptr + A.m, sizeof(int64_t), hipMemcpyDeviceToHost, st));
    SG_HIP(hipStreamSynchronize(st));
    if (ne > ent_capacity) throw std::logic_error("CSC entry capacity exceeded");
    unsigned long long* cursor = ar.get<unsigned long long>("csc_cursor", (size_t)A.m + 1);
    copy<int64_t>((int64_t*)cursor, colptr, A.m, st);
    hipLaunchKernelGGL(k_csc_fill, dim3(grid_1d(blocks)), dim3(256), 0, st, A.rp, A.col, B.rp,
                       hrows, H, S, chat_rp, dest_base, cursor, ent_k, ent_q, ent_dest);
    SG_LAUNCH_CHECK();
    scan_exclusive(SlicePieces{ent_k, B.rp}, ne, P, ar, st);
    SG_HIP(hipMemcpyAsync(total_pieces, P + ne, sizeof(int64_t), hipMemcpyDeviceToHost, st));
    SG_HIP(hipStreamSynchronize(st));
    return ne;
}

// C-hat row pointers of one batch, relative to the batch's first element.
__global__ void k_sub_base(const int64_t* a, int64_t n, int64_t base, int64_t* out) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = a[i] - base;
}

void rebase(const int64_t* a, int64_t n, int64_t base, int64_t* out, hipStream_t st) {
    if (n <= 0) return;
    hipLaunchKernelGGL(k_sub_base, dim3(grid_1d(ceil_div(n, 256))), dim3(256), 0, st, a, n, base,
                       out);
    SG_LAUNCH_CHECK();
}

// ---------------------------------------------------------------- outer product
// Static partition of the flattened product space (Section III-B, Fig. 2).
// The space is cut into pieces of 64 products, one per lane: piece j of CSC
// entry e (slice k = ent_k[e], value a) covers products [64j, 64j+64) of
// B row k, scaled by a and written to the entry's contiguous run of its
// C-hat row. Work group g takes pieces [g*PPB, (g+1)*PPB): it stages the
// descriptors of the (at most PPB) entries those pieces belong to in LDS,
// then its waves take pieces in turn, several at once, so B reads and C-hat
// writes are coalesced and no element needs a search. Reads of B rows are
// shared across the entries of one slice (CSC order keeps them adjacent).
constexpr int kExpandNT = 256;
constexpr int kExpandPPB = 128;   // pieces per work group (8192 products at most)
constexpr int kExpandU = 2;       // pieces in flight per wave

template <bool NUM>
__global__ __launch_bounds__(kExpandNT) void k_expand(ExpandArgs a, int64_t total_pieces) {
    constexpr int NW = kExpandNT / kWave;
    __shared__ int64_t s_pp[kExpandPPB + 1];
    __shared__ int64_t s_dest[kExpandPPB];
    __shared__ int64_t s_bst[kExpandPPB];
    __shared__ int s_nb[kExpandPPB];
    __shared__ double s_a[kExpandPPB];
    __shared__ int64_t s_e0;
    __shared__ int s_ne;
    const int tt = threadIdx.x, w = tt / kWave, lane = lane_id();
    const int64_t P0 = (int64_t)blockIdx.x * kExpandPPB;
    const int64_t P1 = min(total_pieces, P0 + kExpandPPB);
    if (tt == 0) {
        // first entry of this tile and of the next: the last entry is the
        // next tile's first one unless that entry starts exactly at P1
        const int64_t e0 = a.tile_e0[blockIdx.x];
        int64_t e1 = a.ne - 1;
        if (P1 < total_pieces) {
            const int64_t en = a.tile_e0[blockIdx.x + 1];
            e1 = (a.P[en] == P1) ? en - 1 : en;
        }
        s_e0 = e0;
        s_ne = (int)(e1 - e0 + 1);
    }
    __syncthreads();
    const int64_t e0 = s_e0;
    const int ne = s_ne;
    for (int j = tt; j <= ne; j += kExpandNT) {
        const int64_t e = e0 + j;
        s_pp[j] = a.P[e];
        if (j < ne) {
            const int32_t k = a.ent_k[e];
            const int64_t b0 = a.Brp[k];
            s_bst[j] = b0;
            s_nb[j] = (int)(a.Brp[k + 1] - b0);
            s_dest[j] = a.ent_dest[e];
            if constexpr (NUM) s_a[j] = a.Aval[a.ent_q[e]];
        }
    }
    __syncthreads();
    int jj = 0;
    for (int64_t p = P0 + w; p < P1; p += (int64_t)NW * kExpandU) {
        int32_t col[kExpandU];
        double bv[kExpandU];
        int64_t dst[kExpandU];
        bool ok[kExpandU];
        double av[kExpandU];
#pragma unroll
        for (int u = 0; u < kExpandU; ++u) {
            const int64_t pu = p + (int64_t)u * NW;
            ok[u] = false;
            if (pu < P1) {
                while (s_pp[jj + 1] <= pu) ++jj;
                const int off = (int)(pu - s_pp[jj]) * kWave + lane;
                if (off < s_nb[jj]) {
                    ok[u] = true;
                    const int64_t bi = s_bst[jj] + off;
                    dst[u] = s_dest[jj] + off;
                    col[u] = a.Bcol[bi];
                    if constexpr (NUM) {
                        bv[u] = a.Bval[bi];
                        av[u] = s_a[jj];
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kExpandU; ++u) {
            if (ok[u]) {
                a.out_col[dst[u]] = col[u];
                if constexpr (NUM) a.out_val[dst[u]] = av[u] * bv[u];
            }
        }
    }
}

int64_t expand_tiles(int64_t total_pieces) { return ceil_div(total_pieces, kExpandPPB); }

void expand_tile_starts(const int64_t* P, int64_t ne, int64_t total_pieces, int64_t* tile_e0,
                        hipStream_t st) {
    tile_starts(P, ne, kExpandPPB, expand_tiles(total_pieces), tile_e0, st);
}

void expand(const ExpandArgs& a, hipStream_t st) {
    const int64_t total_pieces = a.total_pieces;
    if (a.ne <= 0 || total_pieces <= 0) return;
    int64_t blocks = ceil_div(total_pieces, kExpandPPB);
    if (a.out_val)
        hipLaunchKernelGGL(k_expand<true>, dim3(grid_1d(blocks)), dim3(kExpandNT), 0, st, a,
                           total_pieces);
    else
        hipLaunchKernelGGL(k_expand<false>, dim3(grid_1d(blocks)), dim3(kExpandNT), 0, st, a,
                           total_pieces);
    SG_LAUNCH_CHECK();
}

// ---------------------------------------------------------------- level geometry
// Rows of a level's input all hold more than tau elements, so a range of E
// consecutive elements touches at most this many rows (the ngroupRows of
// Section III-C).
inline int rows_per_range(int64_t E, int64_t tau) {
    return (int)((E + tau) / (tau + 1)) + 1;
}

// ---------------------------------------------------------------- histogram
constexpr int kHistNT = 256;

__global__ __launch_bounds__(kHistNT) void k_histogram(LevelGeom g, const int32_t* in_col,
                                                       int64_t* counts, const int64_t* tile_r0,
                                                       int64_t epb, int nr_max) {
    extern __shared__ int64_t lds_h[];
    int64_t* rb = lds_h;                          // nr_max + 1 row bounds
    int* hist = (int*)(lds_h + nr_max + 1);       // nr_max * nch counters
    __shared__ int64_t r0_sh;
    const int64_t g0 = (int64_t)blockIdx.x * epb;
    const int64_t g1 = min(g.total, g0 + epb);
    const int nkeys = nr_max * g.nch;
    if (threadIdx.x == 0) r0_sh = tile_r0[blockIdx.x];
    for (int x = threadIdx.x; x < nkeys; x += kHistNT) hist[x] = 0;
    __syncthreads();
    const int64_t r0 = r0_sh;
    for (int j = threadIdx.x; j <= nr_max; j += kHistNT)
        rb[j] = (r0 + j <= g.nrows) ? g.rp[r0 + j] : INT64_MAX;
    __syncthreads();
    int lr = 0;
    const int mask = g.nch - 1;
    for (int64_t t = g0 + threadIdx.x; t < g1; t += kHistNT) {
        while (lr + 1 < nr_max && t >= rb[lr + 1]) ++lr;
        int c = (in_col[t] >> g.shift) & mask;
        atomicAdd(&hist[lr * g.nch + c], 1);
    }
    __syncthreads();
    for (int x = threadIdx.x; x < nkeys; x += kHistNT) {
        int v = hist[x];
        if (v) {
            int64_t r = r0 + x / g.nch;
            atomicAdd((unsigned long long*)&counts[r * g.nch + (x & mask)],
                      (unsigned long long)v);
        }
    }
}

static int64_t hist_epb(int64_t tau, int nch, int* nr_max) {
    int64_t epb = 16384;
    while (epb > 256 && (int64_t)rows_per_range(epb, tau) * nch * 4 > 32768) epb /= 2;
    *nr_max = rows_per_range(epb, tau);
    return epb;
}

void histogram(const LevelGeom& g, const int32_t* in_col, int64_t* counts, Arena& ar,
               hipStream_t st) {
    if (g.total <= 0) return;
    int nr_max;
    int64_t epb = hist_epb(g.tau, g.nch, &nr_max);
    size_t lds = (size_t)(nr_max + 1) * 8 + (size_t)nr_max * g.nch * 4;
    int64_t blocks = ceil_div(g.total, epb);
    int64_t* tile_r0 = ar.get<int64_t>("hist_tile_r0", (size_t)blocks + 1);
    tile_starts(g.rp, g.nrows, epb, blocks, tile_r0, st);
    hipLaunchKernelGGL(k_histogram, dim3(grid_1d(blocks)), dim3(kHistNT), lds, st, g, in_col,
                       counts, tile_r0, epb, nr_max);
    SG_LAUNCH_CHECK();
}

// ---------------------------------------------------------------- chunk bins
struct ChunkBinOf {
    const int64_t* counts;
    int64_t tau;
    bool last;
    __device__ int operator()(int64_t x) const {
        int64_t c = counts[x];
        if (c == 0) return CB_EMPTY;
        if (c > tau) return last ? CB_DENSE : CB_NEXT;
        if (c <= kHashMaxItems[0]) return CB_H128;
        if (c <= kHashMaxItems[1]) return CB_H512;
        if (c <= kHashMaxItems[2]) return CB_H2048;
        return CB_H8192;
    }
};

void classify_chunks(const int64_t* counts, int64_t nchunks, int64_t tau, bool last_level,
                     int32_t* inv, int32_t* pos_of, int64_t* bin_start, Arena& ar,
                     hipStream_t st) {
    partition(ChunkBinOf{counts, tau, last_level}, nchunks, CB_COUNT, inv, pos_of, bin_start, ar,
              st);
}

struct CountAt {
    const int64_t* counts;
    const int32_t* inv;
    __device__ int64_t operator()(int64_t p) const { return counts[inv[p]]; }
};

void reord_rowptr(const int64_t* counts, const int32_t* inv, int64_t npos, int64_t* rp_out,
                  Arena& ar, hipStream_t st) {
    scan_exclusive(CountAt{counts, inv}, npos, rp_out, ar, st);
}

// ---------------------------------------------------------------- multisplit
// One work group per tile of E = NT*K consecutive input elements
// (Algorithm 5):
//  1. local histogram of (local row, chunk) keys. Each wave ranks its
//     elements by matching keys across lanes with ballots (one ballot per
//     key bit), so equal keys are found without LDS atomics; the first lane
//     of each key group adds the group to the wave's private histogram
//     (subgroup-private histograms, Section III-C);
//  2. per key: the waves' exclusive prefix, the key's offset in the tile
//     (block-wide scan) and one global reservation on the chunk's cursor in
//     C-hat-reord;
//  3. permute the elements into LDS, grouped by key, recording each slot's
//     key;
//  4. write the LDS buffer out in slot order: slot d goes to
//     (reserved base of its key) - (key's tile offset) + d, so consecutive
//     threads write consecutive slots of each chunk (the coalesced write of
//     Algorithm 5).
// Inside a tile, elements keep their input order within each chunk; across
// tiles the order follows the reservations.
// With FUSED, level 0 of the numeric pass takes its input straight from A
// and B instead of from C-hat: every thread forms the products of its own
// elements of the tile (the same C-hat range a plain multisplit tile would
// read). The tile's A entries are staged in LDS in rounds of kMsNT; an
// element's entry is found by a search over the staged product offsets,
// and its B entry is the entry's B row start plus the element's distance
// from the entry's first product. All loads of a round are issued together.
struct FusedSrc {
    const int64_t* hq0 = nullptr;   // per C-hat row: first A entry of its heavy row
    const int64_t* hq1 = nullptr;   // ... one past its last A entry
    const int64_t* hs0 = nullptr;   // ... InterOffsets at its first entry
    const int64_t* S = nullptr;     // InterOffsets over A's entries
    const int64_t* ebo = nullptr;   // per A entry: first entry of its B row
    const double* Aval = nullptr;
    const int32_t* Bcol = nullptr;
    const double* Bval = nullptr;
    const int64_t* tile_q0 = nullptr; // entry holding each tile's first product
    const int64_t* tile_r0 = nullptr; // C-hat row holding each tile's first product
    int64_t nblocks = 0;
};

template <bool NUM, bool OUT16, bool FUSED, int kMsNT, int kMsK>
__global__ __launch_bounds__(kMsNT) void k_multisplit(LevelGeom g, const int32_t* in_col,
                                                      const double* in_val,
                                                      const int32_t* pos_of,
                                                      unsigned long long* cursor,
                                                      int32_t* out_col, double* out_val,
                                                      const int64_t* tile_r0, int64_t epb,
                                                      int nr_max, FusedSrc fs) {
    static_assert(!FUSED || NUM, "the fused tile forms values");
    constexpr int NW = kMsNT / kWave;
    extern __shared__ int64_t lds_m[];
    const int nkeys = nr_max * g.nch;
    int64_t* delta = lds_m;                          // nkeys
    int64_t* rb = delta + nkeys;                     // nr_max + 1
    double* valbuf = (double*)(rb + nr_max + 1);     // epb (NUM only)
    int* whist = (int*)(valbuf + (NUM ? epb : 0));   // NW * nkeys
    int* loff = whist + NW * nkeys;                  // nkeys + 1
    int* colbuf = loff + nkeys + 1;                  // epb
    uint16_t* keybuf = (uint16_t*)(colbuf + epb);    // epb
    int* pos_sh = (int*)(keybuf + epb + (epb & 1));  // nkeys
    int* rbr = pos_sh + nkeys;                       // nr_max + 1: tile-relative row starts
    __shared__ int64_t r0_sh;
    __shared__ int scan_sh[NW + 1];

    const int tt = threadIdx.x, w = tt / kWave;
    const int64_t g0 = (int64_t)blockIdx.x * epb;
    const int64_t g1 = min(g.total, g0 + epb);
    const int n_wg = (int)(g1 - g0);
    const int mask = g.nch - 1;
    if (tt == 0) r0_sh = tile_r0[blockIdx.x];
    for (int x = tt; x < NW * nkeys; x += kMsNT) whist[x] = 0;
    __syncthreads();
    const int64_t r0 = r0_sh;
    for (int j = tt; j <= nr_max; j += kMsNT) {
        const int64_t v = (r0 + j <= g.nrows) ? g.rp[r0 + j] : INT64_MAX;
        rb[j] = v;
        // 32-bit copy relative to the tile, with a sentinel that ends the
        // row search at the last row slot
        rbr[j] = (j == nr_max || v - g0 >= (int64_t)INT32_MAX)
                     ? INT32_MAX
                     : (int)(v > g0 ? v - g0 : 0);
    }
    __syncthreads();

    // positions of this tile's (row, chunk) keys in the level's partition,
    // loaded now so that the reservations below wait on one load less
    for (int x = tt; x < nkeys; x += kMsNT) {
        const int64_t r = r0 + x / g.nch;
        pos_sh[x] = r < g.nrows ? pos_of[r * g.nch + (x & mask)] : -1;
    }

    int32_t col[kMsK];
    double val[kMsK];
    if constexpr (FUSED) {
        // 0. form the tile's products in registers, in the layout phase 1
        // reads: element t of the tile (C-hat order) lies in the last A
        // entry whose product range starts at or before t.
        // (offsets from the LDS base keep the pointers in the LDS address space)
        const int rq_off = (int)(((char*)(rbr + nr_max + 1) - (char*)lds_m + 7) & ~7);
        int64_t* rq0 = (int64_t*)((char*)lds_m + rq_off);                               // nr_max
        int64_t* rpre = rq0 + nr_max;                                                  // nr_max + 1
        int64_t* rrel = rpre + nr_max + 1;                                             // nr_max
        __shared__ int s_rel[kMsNT + 1];
        __shared__ int64_t s_bo[kMsNT + 1];  // the extra slot keeps the staging branch-free
        __shared__ double s_a[kMsNT + 1];
        // per row of the tile: first entry, entry count, and the tile-relative
        // position of the row's InterOffsets origin
        for (int j = tt; j < nr_max; j += kMsNT) {
            const int64_t r = r0 + j;
            int64_t cnt = 0, qs = 0, rel = 0;
            if (r < g.nrows && rb[j] < g1) {
                qs = (j == 0) ? fs.tile_q0[blockIdx.x] : fs.hq0[r];
                int64_t qe = fs.hq1[r];
                if (blockIdx.x + 1 < fs.nblocks && fs.tile_r0[blockIdx.x + 1] == r)
                    qe = fs.tile_q0[blockIdx.x + 1] + 1;
                cnt = qe > qs ? qe - qs : 0;
                rel = rb[j] - g0 - fs.hs0[r];
            }
            rq0[j] = qs;
            rpre[j + 1] = cnt;  // prefix formed below
            rrel[j] = rel;
        }
        __syncthreads();
        if (tt == 0) {
            rpre[0] = 0;
            for (int j = 0; j < nr_max; ++j) rpre[j + 1] += rpre[j];
        }
        __syncthreads();
        const int64_t E = rpre[nr_max];
        // entries in rounds of kMsNT; a round covers the elements from its
        // first entry's start to the next round's first entry's start
        for (int64_t eb = 0; eb < E; eb += kMsNT) {
            for (int x = tt; x <= kMsNT; x += kMsNT) {
                const int64_t e = eb + x;
                int cs = n_wg;
                if (e < E) {
                    int j = 0;
                    while (rpre[j + 1] <= e) ++j;
                    const int64_t q = rq0[j] + (e - rpre[j]);
                    // the three loads depend on q only: issue them together
                    const int64_t sq = fs.S[q];
                    const int64_t eq = fs.ebo[q];
                    const double aq = fs.Aval[q];
                    const int64_t rs = rrel[j] + sq;
                    cs = (int)(rs < 0 ? 0 : (rs > n_wg ? n_wg : rs));
                    s_bo[x] = eq + (cs - rs);
                    s_a[x] = aq;
                }
                s_rel[x] = cs;
            }
            __syncthreads();
            const int nst = (int)min((int64_t)kMsNT, E - eb);
            const int lo = s_rel[0], hi = s_rel[kMsNT];
            // B indices of this round's elements from LDS first, then every
            // load at once, then the products (a load per element waited on
            // in turn would serialise the round's latency kMsK times)
            int64_t bi[kMsK];
            double av[kMsK];
            int j = 0;
#pragma unroll
            for (int k = 0; k < kMsK; ++k) {
                const int t = k * kMsNT + tt;
                bi[k] = -1;
                if (t >= lo && t < hi) {
                    int jh = nst;  // largest j with s_rel[j] <= t, searched in [j, jh)
                    while (jh - j > 1) {
                        const int mid = (j + jh) >> 1;
                        if (s_rel[mid] <= t) j = mid; else jh = mid;
                    }
                    bi[k] = s_bo[j] + (t - s_rel[j]);
                    av[k] = s_a[j];
                }
            }
            int32_t bc[kMsK];
            double bv[kMsK];
#pragma unroll
            for (int k = 0; k < kMsK; ++k) {
                if (bi[k] >= 0) {
                    bc[k] = fs.Bcol[bi[k]];
                    bv[k] = fs.Bval[bi[k]];
                }
            }
#pragma unroll
            for (int k = 0; k < kMsK; ++k) {
                if (bi[k] >= 0) {
                    col[k] = bc[k];
                    val[k] = av[k] * bv[k];
                }
            }
            __syncthreads();
        }
    }

    // 1. load, key, rank within the wave. Keys of a wave's 64 elements are
    // few and clustered (consecutive products share a row and mostly a
    // chunk), so the wave peels them one distinct key at a time: the first
    // remaining lane's key is broadcast, a ballot finds the lanes holding it,
    // and each takes the wave's running count of the key plus its place
    // among those lanes.
    int key[kMsK];
    int rank[kMsK];
    if constexpr (!FUSED) {
#pragma unroll
        for (int k = 0; k < kMsK; ++k) {
            const int t = k * kMsNT + tt;
            if (t < n_wg) {
                col[k] = in_col[g0 + t];
                if constexpr (NUM) val[k] = in_val[g0 + t];
            }
        }
    }
    int lr = 0;
    int* myhist = whist + w * nkeys;
    const int lane = lane_id();
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
    for (int k = 0; k < kMsK; ++k) {
        const int t = k * kMsNT + tt;
        int kk = -1;
        if (t < n_wg) {
            while (t >= rbr[lr + 1]) ++lr;
            kk = lr * g.nch + ((col[k] >> g.shift) & mask);
        }
        key[k] = kk;
        int r = 0;
        uint64_t act = __ballot(kk >= 0);
        while (act) {
            const int leader = __builtin_ctzll(act);
            const int lk = __builtin_amdgcn_readlane(kk, leader);
            const uint64_t m = __ballot(kk == lk);
            const int base = myhist[lk];
            if (kk == lk) r = base + __popcll(m & lt);
            if (lane == leader) myhist[lk] = base + __popcll(m);
            act &= ~m;
        }
        rank[k] = r;
    }
    __syncthreads();

    // 2. per key: wave prefixes, tile offset (block scan) and reservation.
    // The reservation atomic of a thread's first key is only waited for
    // after the LDS permute, so its latency overlaps the permute (with
    // nkeys <= threads every key is such a first key).
    int64_t pend_v = 0;
    int pend_x = -1;
    {
        const int per = (nkeys + kMsNT - 1) / kMsNT;
        const int k0 = min(nkeys, tt * per);
        const int k1 = min(nkeys, k0 + per);
        int s = 0;
        for (int x = k0; x < k1; ++x) {
            int run = 0;
            for (int ww = 0; ww < NW; ++ww) {
                int c = whist[ww * nkeys + x];
                whist[ww * nkeys + x] = run;
                run += c;
            }
            loff[x] = run;  // total for now
            s += run;
        }
        int tot;
        int pre = block_exclusive_scan<kMsNT>(s, scan_sh, &tot);
        for (int x = k0; x < k1; ++x) {
            const int v = loff[x];
            if (v) {
                // each wave's slot base for the key now includes the key's
                // offset in the tile
                for (int ww = 0; ww < NW; ++ww) whist[ww * nkeys + x] += pre;
                const int p = pos_sh[x];
                const int64_t got = (int64_t)atomicAdd(&cursor[p], (unsigned long long)v) - pre;
                if (x == k0) {
                    pend_v = got;
                    pend_x = x;
                } else {
                    delta[x] = got;
                }
            }
            pre += v;
        }
    }
    __syncthreads();

    // 3. permute into LDS
#pragma unroll
    for (int k = 0; k < kMsK; ++k) {
        const int kk = key[k];
        if (kk >= 0) {
            const int d = myhist[kk] + rank[k];
            colbuf[d] = col[k];
            keybuf[d] = (uint16_t)kk;
            if constexpr (NUM) valbuf[d] = val[k];
        }
    }
    if (pend_x >= 0) delta[pend_x] = pend_v;
    __syncthreads();

    // 4. ordered write; at the last level the column is stored as its
    // 16-bit offset inside the chunk (chunks there are at most 2^16 wide)
    const int32_t lmask = (1 << g.shift) - 1;
    for (int d = tt; d < n_wg; d += kMsNT) {
        const int64_t ga = delta[keybuf[d]] + d;
        if constexpr (OUT16) ((uint16_t*)out_col)[ga] = (uint16_t)(colbuf[d] & lmask);
        else out_col[ga] = colbuf[d];
        if constexpr (NUM) out_val[ga] = valbuf[d];
    }
}

static size_t ms_lds(int64_t epb, int nr_max, int nch, bool num, int nw, bool fused) {
    size_t nkeys = (size_t)nr_max * nch;
    size_t b = nkeys * 8 + (size_t)(nr_max + 1) * 8 + (num ? (size_t)epb * 8 : 0) +
               (size_t)nw * nkeys * 4 + (nkeys + 1) * 4 + (size_t)epb * 4 + (size_t)epb * 2 + 8;
    b += nkeys * 4 + 4 + (size_t)(nr_max + 1) * 4;     // key positions (+ pad), row starts
    if (fused) b += 8 + (size_t)(3 * nr_max + 1) * 8;  // pad + per-row entry ranges
    return b;
}

// C-hat entry holding every tile's first product: the tile's first row is
// tile_r0[t]; inside the row the entry is found from InterOffsets.
__global__ void k_fused_tile_entries(const int64_t* chat_rp, const int64_t* hq0,
                                     const int64_t* hq1, const int64_t* hs0, const int64_t* S,
                                     const int64_t* tile_r0, int64_t epb, int64_t nblocks,
                                     int64_t* tile_q0) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= nblocks) return;
    const int64_t r = tile_r0[t];
    const int64_t target = hs0[r] + (t * epb - chat_rp[r]);
    tile_q0[t] = upper_index(S, hq0[r], hq1[r], target);
}

// Per heavy row: its A entry range and InterOffsets at its first entry.
__global__ void k_heavy_row_info(const int64_t* Arp, const int64_t* S, const int32_t* hrows,
                                 int64_t H, int64_t* hq0, int64_t* hq1, int64_t* hs0) {
    const int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= H) return;
    const int32_t i = hrows[h];
    const int64_t a0 = Arp[i];
    hq0[h] = a0;
    hq1[h] = Arp[i + 1];
    hs0[h] = S[a0];
}

// Per A entry: the first entry of the B row it multiplies.
__global__ void k_entry_bstart(const int32_t* Acol, const int64_t* Brp, int64_t nnz,
                               int64_t* ebo) {
    int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; q < nnz; q += stride) ebo[q] = Brp[Acol[q]];
}

void fused_setup(const DevCSR& A, const DevCSR& B, const int64_t* S, const int32_t* hrows,
                 int64_t H, int64_t* hq0, int64_t* hq1, int64_t* hs0, int64_t* ebo,
                 hipStream_t st) {
    if (H > 0) {
        hipLaunchKernelGGL(k_heavy_row_info, dim3(grid_1d(ceil_div(H, 256))), dim3(256), 0, st,
                           A.rp, S, hrows, H, hq0, hq1, hs0);
        SG_LAUNCH_CHECK();
    }
    if (A.nnz > 0) {
        int64_t blocks = std::min<int64_t>(ceil_div(A.nnz, 256), 8192);
        hipLaunchKernelGGL(k_entry_bstart, dim3(grid_1d(blocks)), dim3(256), 0, st, A.col, B.rp,
                           A.nnz, ebo);
        SG_LAUNCH_CHECK();
    }
}

template <bool NUM, bool OUT16, bool FUSED, int NT, int K>
static void ms_launch(const LevelGeom& g, const int32_t* in_col, const double* in_val,
                      const int32_t* pos_of, int64_t* cursor, int32_t* out_col, double* out_val,
                      FusedSrc fs, Arena& ar, hipStream_t st) {
    int64_t epb = (int64_t)NT * K;
    int nr_max = rows_per_range(epb, g.tau);
    while (epb > 64 && ms_lds(epb, nr_max, g.nch, NUM, NT / kWave, FUSED) > 65536) {
        epb /= 2;
        nr_max = rows_per_range(epb, g.tau);
    }
    if ((int64_t)nr_max * g.nch > 65535) throw OverflowError("multisplit keys exceed 16 bits");
    size_t lds = ms_lds(epb, nr_max, g.nch, NUM, NT / kWave, FUSED);
    if (lds > 160 * 1024) throw OverflowError("multisplit local histogram exceeds LDS");
    int64_t blocks = ceil_div(g.total, epb);
    int64_t* tile_r0 = ar.get<int64_t>("ms_tile_r0", (size_t)blocks + 1);
    tile_starts(g.rp, g.nrows, epb, blocks, tile_r0, st);
    if constexpr (FUSED) {
        int64_t* tile_q0 = ar.get<int64_t>("ms_tile_q0", (size_t)blocks + 1);
        hipLaunchKernelGGL(k_fused_tile_entries, dim3(grid_1d(ceil_div(blocks, 256))), dim3(256), 0,
                           st, g.rp, fs.hq0, fs.hq1, fs.hs0, fs.S, tile_r0, epb, blocks, tile_q0);
        SG_LAUNCH_CHECK();
        fs.tile_q0 = tile_q0;
        fs.tile_r0 = tile_r0;
        fs.nblocks = blocks;
    }
    auto kern = k_multisplit<NUM, OUT16, FUSED, NT, K>;
    SG_HIP(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds));
    hipLaunchKernelGGL(kern, dim3(grid_1d(blocks)), dim3(NT), lds, st, g, in_col, in_val, pos_of,
                       (unsigned long long*)cursor, out_col, out_val, tile_r0, epb, nr_max, fs);
    SG_LAUNCH_CHECK();
}

// 256 threads x 8 elements (2048 per group, about 25 KiB of LDS with values)
// measured fastest on MI355X among 128..1024 threads x 4..16 elements.
constexpr int kMsNT = 256;
constexpr int kMsK = 8;
constexpr int kMsKFused = 4;  // the tiles that form their own products

void multisplit(const LevelGeom& g, const int32_t* in_col, const double* in_val,
                const int32_t* pos_of, int64_t* cursor, int32_t* out_col, double* out_val,
                bool out16, Arena& ar, hipStream_t st) {
    if (g.total <= 0) return;
    if (out16 && g.shift > 16) throw std::logic_error("16-bit columns need chunks <= 2^16 wide");
    FusedSrc none{};
    if (out_val) {
        if (out16) ms_launch<true, true, false, kMsNT, kMsK>(g, in_col, in_val, pos_of, cursor, out_col, out_val, none, ar, st);
        else ms_launch<true, false, false, kMsNT, kMsK>(g, in_col, in_val, pos_of, cursor, out_col, out_val, none, ar, st);
    } else {
        if (out16) ms_launch<false, true, false, kMsNT, kMsK>(g, in_col, in_val, pos_of, cursor, out_col, nullptr, none, ar, st);
        else ms_launch<false, false, false, kMsNT, kMsK>(g, in_col, in_val, pos_of, cursor, out_col, nullptr, none, ar, st);
    }
}

void expand_multisplit(const LevelGeom& g, const FusedRows& fr, const DevCSR& A, const DevCSR& B,
                       const int64_t* S, const int32_t* pos_of, int64_t* cursor, int32_t* out_col,
                       double* out_val, bool out16, Arena& ar, hipStream_t st) {
    if (g.total <= 0) return;
    if (out16 && g.shift > 16) throw std::logic_error("16-bit columns need chunks <= 2^16 wide");
    FusedSrc fs{};
    fs.hq0 = fr.hq0;
    fs.hq1 = fr.hq1;
    fs.hs0 = fr.hs0;
    fs.ebo = fr.ebo;
    fs.S = S;
    fs.Aval = A.val;
    fs.Bcol = B.col;
    fs.Bval = B.val;
    // four elements a thread: with eight, forming the products in the tile
    // takes 96 VGPRs (five waves a SIMD); with four, 52 (eight)
    if (out16) ms_launch<true, true, true, kMsNT, kMsKFused>(g, nullptr, nullptr, pos_of, cursor, out_col, out_val, fs, ar, st);
    else ms_launch<true, false, true, kMsNT, kMsKFused>(g, nullptr, nullptr, pos_of, cursor, out_col, out_val, fs, ar, st);
}

// First column of every chunk of a level: level 0 chunk c of a row starts at
// c*W; a deeper chunk c of parent p starts at parent's start + c*W.
__global__ void k_chunk_colbase(int64_t nparents, int nch, int64_t width, const int32_t* parent_inv,
                                const int32_t* parent_base, int32_t* out) {
    int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= nparents * nch) return;
    int64_t p = x / nch;
    int c = (int)(x - p * nch);
    int64_t b = parent_inv ? parent_base[parent_inv[p]] : 0;
    out[x] = (int32_t)(b + c * width);
}

void chunk_colbase(int64_t nparents, int nch, int64_t width, const int32_t* parent_inv,
                   const int32_t* parent_base, int32_t* out, hipStream_t st) {
    int64_t n = nparents * nch;
    if (n <= 0) return;
    hipLaunchKernelGGL(k_chunk_colbase, dim3(grid_1d(ceil_div(n, 256))), dim3(256), 0, st,
                       nparents, nch, width, parent_inv, parent_base, out);
    SG_LAUNCH_CHECK();
}

// ---------------------------------------------------------------- fused symbolic
// Symbolic pass of the heavy rows without materialising C-hat-reord: the
// structure of every level (chunk element counts for Histogram, and the
// distinct columns per chunk that Symbolic counts on C-hat-reord) depends
// only on which columns each heavy row produces and how often, not on the
// order of elements inside a chunk. Counts per finest chunk slot (width
// W_fin) are enough: a chunk of any level is a run of consecutive slots.
//
// Element counts: B row k contributes the same per-slot counts to every
// row that uses it, so bslot[k][s] is counted once over B and each heavy
// row sums the vectors of its A entries.
__global__ void k_bslot_counts(const int64_t* brp, const int32_t* bcol, int64_t nb_rows,
                               int logW, int req, int32_t* bslot) {
    int64_t k = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    if (k >= nb_rows) return;
    for (int64_t e = brp[k] + lane_id(); e < brp[k + 1]; e += kWave)
        atomicAdd(&bslot[k * req + (bcol[e] >> logW)], 1);
}

// The same counts without global atomics: one wavefront per B row counts
// its slots in LDS, peeling one distinct slot of each 64-entry batch at a
// time (B rows are mostly sorted, so a batch holds few slots), then writes
// the row's counts.
constexpr int kBslotNT = 256;
constexpr int kBslotMaxReq = 4096;

__global__ __launch_bounds__(kBslotNT) void k_bslot_rows(const int64_t* brp, const int32_t* bcol,
                                                         int64_t nb, int logW, int req,
                                                         int32_t* bslot) {
    extern __shared__ int lds_c[];
    const int w = threadIdx.x / kWave, lane = lane_id();
    int* cnt = lds_c + w * req;
    const int64_t k = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    if (k >= nb) return;  // whole waves leave together; no block barrier below
    for (int s = lane; s < req; s += kWave) cnt[s] = 0;
    const int64_t e0 = brp[k], e1 = brp[k + 1];
    for (int64_t eb = e0; eb < e1; eb += kWave) {
        const int64_t e = eb + lane;
        const int s = e < e1 ? (int)((uint32_t)bcol[e] >> logW) : -1;
        uint64_t act = __ballot(s >= 0);
        while (act) {
            const int leader = __builtin_ctzll(act);
            const int ls = __builtin_amdgcn_readlane(s, leader);
            const uint64_t m = __ballot(s == ls);
            if (lane == leader) cnt[ls] += __popcll(m);
            act &= ~m;
        }
    }
    for (int s = lane; s < req; s += kWave) bslot[k * req + s] = cnt[s];
}

// Distinct columns: one work group per heavy row keeps a one-bit-per-column
// bitmap of the row's column range in LDS; the row's element counts per slot
// are the sums of its entries' B-row slot vectors. A row with far more
// products than a work group's share of the pass (power-law rows) is split
// by its product range over several work groups, which OR their bitmaps
// into a global one and add their element counts; a last pass counts the
// bits of the split rows. The row's A entries are taken in
// windows staged in LDS; each entry's B row is cut into pieces of 64
// products and the waves take pieces in turn, one product per lane, so the
// reads of B are coalesced and no product needs a search.
constexpr int kHsymNT = 1024;
constexpr int kHsymEW = 1024;  // entries per staged window (half with column parts)
// one thread stages each entry of a window
static_assert(kHsymEW <= kHsymNT, "a staged window holds at most one entry per thread");

constexpr int kHsymMaxSplit = 64;      // work groups per row at most
constexpr int64_t kHsymSplitMin = 16384;  // products per work group at least

// Per heavy row: (work groups) | (1 if split) << 32, for the exclusive scan
// that gives each row its first work group and its split-row index.
struct HsymSplitOf {
    const int64_t* arp;
    const int64_t* S;
    const int32_t* hrows;
    int64_t T;
    __device__ int64_t operator()(int64_t h) const {
        const int32_t r = hrows[h];
        const int64_t a0 = arp[r], a1 = arp[r + 1];
        const int64_t u = S[a1] - S[a0];
        int64_t ns = u > T ? (u + T - 1) / T : 1;
        ns = min(ns, (int64_t)kHsymMaxSplit);
        ns = max((int64_t)1, min(ns, a1 - a0));
        return ns | (ns > 1 ? (int64_t(1) << 32) : 0);
    }
};

__device__ __forceinline__ int64_t hsym_blocks(int64_t packed) { return packed & 0xffffffffLL; }
__device__ __forceinline__ int64_t hsym_split(int64_t packed) { return packed >> 32; }

// Work group -> heavy row map, split row -> heavy row map, and the split
// rows' element counts cleared (their work groups add into them).
__global__ void k_hsym_map(const int64_t* off, int64_t H, int req, int32_t* bmap, int32_t* smap,
                           int64_t* elem_fin) {
    const int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= H) return;
    const int64_t b0 = hsym_blocks(off[h]), b1 = hsym_blocks(off[h + 1]);
    for (int64_t b = b0; b < b1; ++b) bmap[b] = (int32_t)h;
    if (b1 - b0 > 1) {
        smap[hsym_split(off[h])] = (int32_t)h;
        for (int sl = 0; sl < req; ++sl) elem_fin[h * req + sl] = 0;
    }
}

// First entry e in [lo, hi] with S[e] >= x (S rises over a row's entries).
__device__ __forceinline__ int64_t first_at_or_above(const int64_t* S, int64_t lo, int64_t hi,
                                                     int64_t x) {
    while (lo < hi) {
        const int64_t mid = lo + ((hi - lo) >> 1);
        if (S[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// What one work group of the symbolic pass takes: A entries [a0, a1) of
// heavy row h, and the row's split index (-1: the row has one work group).
struct HsymGroup {
    int64_t a0, a1;
    int32_t h, sidx;
};

// One thread per work group, so that the searches of the split rows' entry
// ranges run side by side here rather than at the start of each group.
// off: packed scan of HsymSplitOf (H + 1) or null (one work group per row).
__global__ void k_hsym_groups(const int64_t* arp, const int32_t* hrows, const int64_t* S,
                              const int64_t* off, const int32_t* bmap, int64_t H,
                              int64_t ngroups, HsymGroup* grp) {
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= ngroups) return;
    HsymGroup g{0, 0, -1, -1};
    if (!off) {
        const int32_t r = hrows[b];
        g = HsymGroup{arp[r], arp[r + 1], (int32_t)b, -1};
    } else if (b < hsym_blocks(off[H])) {
        const int64_t h = bmap[b];
        const int64_t o = off[h];
        const int64_t ns = hsym_blocks(off[h + 1]) - hsym_blocks(o);
        const int32_t r = hrows[h];
        int64_t a0 = arp[r], a1 = arp[r + 1];
        int32_t sidx = -1;
        if (ns > 1) {
            // the entries whose products start in this group's 1/ns of the
            // row's product range
            const int64_t part = b - hsym_blocks(o);
            const int64_t s0 = S[a0], u = S[a1] - s0;
            const int64_t lo = s0 + u * part / ns, hi = s0 + u * (part + 1) / ns;
            const int64_t e0 = first_at_or_above(S, a0, a1, lo);
            a1 = part == ns - 1 ? a1 : first_at_or_above(S, a0, a1, hi);
            a0 = e0;
            sidx = (int32_t)hsym_split(o);
        }
        g = HsymGroup{a0, a1, (int32_t)h, sidx};
    }
    grp[b] = g;
}

// The row's column range may be taken in np parts, one launch each (when the
// whole bitmap would leave one work group per CU): part p keeps bitmap words
// [wlo, wlo + nwp) and slots [sl0, sl0 + reqp), reads every product of the
// row and skips those outside its columns. B32: B has fewer than 2^31
// entries, so B row starts are kept in 32 bits.
template <int EW, bool B32>
__global__ __launch_bounds__(kHsymNT) void k_heavy_symbolic(
    const HsymGroup* grp, const int32_t* acol, const int64_t* brp, const int32_t* bcol, int req,
    int nwords, int wlo, int nwp, int sl0, int reqp, const int32_t* bslot, int64_t* elem_fin,
    int64_t* dist_fin, uint32_t* gbits) {
    static_assert(EW <= kHsymNT, "a staged window holds at most one entry per thread");
    extern __shared__ __align__(16) int64_t lds_s[];
    constexpr int NW = kHsymNT / kWave;
    using BT = typename std::conditional<B32, uint32_t, int64_t>::type;
    uint32_t* bits = (uint32_t*)lds_s;                      // nwp, padded to 4 words
    BT* bst = (BT*)(bits + ((nwp + 3) & ~3));               // EW B row starts
    unsigned long long* esl = (unsigned long long*)(bst + EW);  // reqp element counts
    int* nbv = (int*)(esl + reqp);                          // EW B row lengths
    int* kst = nbv + EW;                                    // EW B rows
    int* ppre = kst + EW;                                   // EW + 1 piece prefix
    int* dsl = ppre + EW + 1;                               // reqp distinct counts
    __shared__ int scan_sh[NW + 1];
    const int tt = threadIdx.x;
    // the wave index and the loop bounds below are uniform per wave: kept in
    // scalar registers, the piece loop branches on them without exec masks
    const int w = __builtin_amdgcn_readfirstlane(tt / kWave), lane = lane_id();
    // words per slot, and the rotation group of the bitmap words
    const uint32_t gm = (uint32_t)min(32, nwords / req) - 1u;
    // the full staging window means a single column part (wlo = 0)
    const uint32_t wl = EW == kHsymEW ? 0u : (uint32_t)wlo;
    const HsymGroup g = grp[blockIdx.x];
    // the whole work group leaves together when the grid's bound exceeds the groups
    if (g.h < 0) return;
    const int64_t h = g.h, a0 = g.a0, a1 = g.a1;
    // the bitmap starts the 16-byte aligned LDS block: cleared 4 words a store
    for (int i = tt * 4; i < nwp; i += kHsymNT * 4) *(uint4*)&bits[i] = make_uint4(0, 0, 0, 0);
    for (int i = tt; i < reqp; i += kHsymNT) {
        dsl[i] = 0;
        esl[i] = 0ull;
    }
    __syncthreads();
    for (int64_t ew = a0; ew < a1; ew += EW) {
        const int ne = (int)min((int64_t)EW, a1 - ew);
        int pc = 0;
        if (tt < ne) {
            int32_t k = acol[ew + tt];
            int64_t b0 = brp[k];
            int nb = (int)(brp[k + 1] - b0);
            bst[tt] = (BT)b0;
            nbv[tt] = nb;
            kst[tt] = k;
            pc = (nb + kWave - 1) / kWave;
        }
        int tot;
        int pre = block_exclusive_scan<kHsymNT>(pc, scan_sh, &tot);
        tot = __builtin_amdgcn_readfirstlane(tot);
        if (tt < ne) ppre[tt] = pre;
        if (tt == 0) ppre[ne] = tot;
        __syncthreads();
        constexpr int U = 8;  // pieces in flight per wave
        // Each wave takes a contiguous run of the window's pieces, so that
        // consecutive pieces mostly continue the same entry (long B rows)
        // and its first piece, length and B start stay in scalar
        // registers; a piece past the entry's end looks its entry up with
        // a ballot over the first pieces of the next 64 entries (the
        // entries starting at or before it are a prefix of them, as the
        // prefixes rise; zero-piece entries are passed over).
        const int per = (tot + NW - 1) / NW;
        const int pb = min(tot, w * per), pe = min(tot, pb + per);
        auto entry_of = [&](int j, int pu) {
            for (;;) {
                const int wj = j + 1 + lane;
                const int pw = wj <= ne ? ppre[wj] : INT_MAX;
                const int cnt = __popcll(__ballot(pw <= pu));
                j += cnt;
                if (cnt < kWave) return j;
            }
        };
        // entry j's first piece, next entry's first piece, length and B
        // start, all uniform: kept in scalar registers
        int j = 0, pj = 0, pn = 0, nj = 0;
        int64_t bj = 0;
        auto load_entry = [&]() {
            pj = __builtin_amdgcn_readfirstlane(ppre[j]);
            pn = __builtin_amdgcn_readfirstlane(ppre[j + 1]);
            nj = __builtin_amdgcn_readfirstlane(nbv[j]);
            const BT b = bst[j];
            if constexpr (B32)
                bj = (uint32_t)__builtin_amdgcn_readfirstlane((int)b);
            else
                bj = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(
                                    (int)((uint64_t)b >> 32)) << 32) |
                               (uint32_t)__builtin_amdgcn_readfirstlane((int)b));
        };
        if (pb < pe) {
            j = entry_of(0, pb);
            load_entry();
            for (int p0 = pb; p0 < pe; p0 += U) {
                uint32_t c[U];
#pragma unroll
                for (int uu = 0; uu < U; ++uu) {
                    const int pu = p0 + uu;
                    c[uu] = 0xffffffffu;
                    if (pu < pe) {
                        if (pu >= pn) {
                            j = entry_of(j, pu);
                            load_entry();
                        }
                        // a scalar base and a 32-bit lane offset
                        const int32_t* rowp = bcol + bj;
                        const int off = (pu - pj) * kWave + lane;
                        if (off < nj) c[uu] = (uint32_t)rowp[(uint32_t)off];
                    }
                }
                // Column c = 32 q + r sets bit r of word q ^ (r & gm), a word
                // of q's aligned group of gm + 1 words (which never spans two
                // slots), so that the runs of nearby columns of a B row fall
                // into different words and banks; only per-slot counts are
                // read. (A lane without a product holds c = ~0: its word lies
                // far past any bitmap that fits LDS, so the bound test drops
                // it.)
#pragma unroll
                for (int uu = 0; uu < U; ++uu) {
                    const uint32_t q = c[uu] >> 5, r = c[uu] & 31;
                    const uint32_t wd = (q ^ (r & gm)) - wl;
                    if (wd < (uint32_t)nwp) atomicOr(&bits[wd], 1u << r);
                }
            }
        }
        // element counts per slot: the sum of the window's B-row slot vectors
        if (reqp <= kHsymNT) {
            const int sl = tt % reqp, step = kHsymNT / reqp;
            int64_t sum = 0;
            if (tt < step * reqp)
                for (int e = tt / reqp; e < ne; e += step)
                    sum += bslot[(int64_t)kst[e] * req + sl0 + sl];
            if (sum) atomicAdd(&esl[sl], (unsigned long long)sum);
        } else {
            for (int sl = tt; sl < reqp; sl += kHsymNT) {
                int64_t sum = 0;
                for (int e = 0; e < ne; ++e) sum += bslot[(int64_t)kst[e] * req + sl0 + sl];
                esl[sl] += (unsigned long long)sum;
            }
        }
        __syncthreads();
    }
    if (g.sidx >= 0) {
        // a part of a split row: add into the row's global counts and bitmap
        uint32_t* gb = gbits + g.sidx * (int64_t)nwords + wlo;
        for (int i = tt; i < nwp; i += kHsymNT)
            if (bits[i]) atomicOr(&gb[i], bits[i]);
        for (int sl = tt; sl < reqp; sl += kHsymNT)
            if (esl[sl])
                atomicAdd((unsigned long long*)&elem_fin[h * req + sl0 + sl], esl[sl]);
        return;
    }
    // distinct columns per finest slot: popcounts of the slot's words
    const int wps = nwp / reqp;  // words per slot (>= 1)
    if (wps >= 8) {
        // eight consecutive words per thread (all in one slot), summed over
        // the lps lanes that share the slot (the active lanes of a wave are
        // a prefix of whole slots: nwp and wps are powers of two); 16 or
        // more lanes a slot: each row of 16 lanes sums by DPP and adds once
        const int lps = min(wps / 8, kWave);
        const int lgw = __builtin_ctz(wps);
        for (int i0 = tt * 8; i0 < nwp; i0 += kHsymNT * 8) {
            const uint4 wa = *(const uint4*)&bits[i0];
            const uint4 wb = *(const uint4*)&bits[i0 + 4];
            int pc = __popc(wa.x) + __popc(wa.y) + __popc(wa.z) + __popc(wa.w) + __popc(wb.x) +
                     __popc(wb.y) + __popc(wb.z) + __popc(wb.w);
            if (lps >= 16) {
                pc = row16_sum_i32(pc);
                if ((lane & 15) == 15 && pc) atomicAdd(&dsl[i0 >> lgw], pc);
            } else {
                for (int dd = 1; dd < lps; dd <<= 1) pc += __shfl_xor(pc, dd, kWave);
                if ((lane & (lps - 1)) == 0 && pc) atomicAdd(&dsl[i0 >> lgw], pc);
            }
        }
    } else {
        for (int i = tt; i < nwp; i += kHsymNT) {
            const int pc = __popc(bits[i]);
            if (pc) atomicAdd(&dsl[i / wps], pc);
        }
    }
    __syncthreads();
    for (int sl = tt; sl < reqp; sl += kHsymNT) {
        dist_fin[h * req + sl0 + sl] = dsl[sl];
        elem_fin[h * req + sl0 + sl] = (int64_t)esl[sl];
    }
}

// Distinct columns of the split rows: popcounts of their global bitmaps.
__global__ __launch_bounds__(kHsymNT) void k_hsym_finalize(const int64_t* off, int64_t H,
                                                          const int32_t* smap,
                                                          const uint32_t* gbits, int req,
                                                          int nwords, int64_t* dist_fin) {
    extern __shared__ int dsl_f[];
    const int64_t b = blockIdx.x;
    if (b >= hsym_split(off[H])) return;
    const int tt = threadIdx.x, lane = lane_id();
    const int64_t h = smap[b];
    for (int i = tt; i < req; i += kHsymNT) dsl_f[i] = 0;
    __syncthreads();
    const uint32_t* g = gbits + b * (int64_t)nwords;
    const int wps = nwords / req;
    for (int i = tt; i < nwords; i += kHsymNT) {
        int pc = __popc(g[i]);
        if (wps >= kWave) {
            pc = wave_reduce_sum(pc);
            if (lane == 0 && pc) atomicAdd(&dsl_f[i / wps], pc);
        } else if (pc) {
            atomicAdd(&dsl_f[i / wps], pc);
        }
    }
    __syncthreads();
    for (int sl = tt; sl < req; sl += kHsymNT) dist_fin[h * req + sl] = dsl_f[sl];
}

// Column parts of B for a symbolic pass taken in np column parts: B's
// entries in part-major order (every row's entries of part 0, row by row,
// then part 1, ...; a row's order is kept inside a part), and the start of
// every (part, row) segment, so that the launch of part p reads only the
// columns it keeps instead of every product of the row. One wavefront per B
// row, its parts ranked by peeling as in k_bslot_rows; part of column c is
// c >> shift.
constexpr int kBpartNT = 256;

__global__ __launch_bounds__(kBpartNT) void k_bpart_count(const int64_t* brp,
                                                          const int32_t* bcol, int64_t nb,
                                                          int shift, int np, int64_t* cnt) {
    extern __shared__ int lds_p[];
    const int w = threadIdx.x / kWave, lane = lane_id();
    int* c = lds_p + w * np;
    const int64_t k = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    if (k >= nb) return;  // whole waves leave together; no block barrier below
    for (int p = lane; p < np; p += kWave) c[p] = 0;
    const int64_t e0 = brp[k], e1 = brp[k + 1];
    for (int64_t eb = e0; eb < e1; eb += kWave) {
        const int64_t e = eb + lane;
        const int pt = e < e1 ? (int)((uint32_t)bcol[e] >> shift) : -1;
        uint64_t act = __ballot(pt >= 0);
        while (act) {
            const int leader = __builtin_ctzll(act);
            const int lp = __builtin_amdgcn_readlane(pt, leader);
            const uint64_t m = __ballot(pt == lp);
            if (lane == leader) c[lp] += __popcll(m);
            act &= ~m;
        }
    }
    for (int p = lane; p < np; p += kWave) cnt[(int64_t)p * nb + k] = c[p];
}

// ppos: exclusive scan of the part-major counts (np * nb + 1 values).
__global__ __launch_bounds__(kBpartNT) void k_bpart_scatter(const int64_t* brp,
                                                            const int32_t* bcol, int64_t nb,
                                                            int shift, int np,
                                                            const int64_t* ppos, int32_t* pcol) {
    extern __shared__ int lds_p[];
    const int w = threadIdx.x / kWave, lane = lane_id();
    int* run = lds_p + w * np;
    const int64_t k = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    if (k >= nb) return;
    for (int p = lane; p < np; p += kWave) run[p] = 0;
    const int64_t e0 = brp[k], e1 = brp[k + 1];
    for (int64_t eb = e0; eb < e1; eb += kWave) {
        const int64_t e = eb + lane;
        const int32_t col = e < e1 ? bcol[e] : 0;
        const int pt = e < e1 ? (int)((uint32_t)col >> shift) : -1;
        // the segment starts are read before the ranking, one round a batch
        const int64_t p0 = pt >= 0 ? ppos[(int64_t)pt * nb + k] : 0;
        int rank = 0;
        uint64_t act = __ballot(pt >= 0);
        while (act) {
            const int leader = __builtin_ctzll(act);
            const int lp = __builtin_amdgcn_readlane(pt, leader);
            const uint64_t m = __ballot(pt == lp);
            const int base = run[lp];  // read by every lane before the leader adds
            if (pt == lp) rank = base + lane_prefix(m);
            wave_lds_sync();
            if (lane == leader) run[lp] = base + __popcll(m);
            wave_lds_sync();
            act &= ~m;
        }
        if (pt >= 0) pcol[p0 + rank] = col;
    }
}

static size_t hsym_lds(int ew, int64_t nwp, int64_t reqp) {
    return (size_t)ew * 8 + (size_t)reqp * 8 + (size_t)ew * 4 * 2 + (size_t)(ew + 1) * 4 +
           (size_t)reqp * 4 + (size_t)((nwp + 3) & ~int64_t(3)) * 4;
}

size_t heavy_symbolic_lds(int64_t ppow, int64_t req) { return hsym_lds(kHsymEW, ppow / 32, req); }

template <int EW, bool B32>
static void launch_hsym(size_t lds, int64_t grid, hipStream_t st, const HsymGroup* grp,
                        const DevCSR& A, const DevCSR& B, int64_t req, int nwords, int part,
                        int nwp, int reqp, const int32_t* bslot, int64_t* elem_fin,
                        int64_t* dist_fin, uint32_t* gbits) {
    auto kern = k_heavy_symbolic<EW, B32>;
    SG_HIP(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds));
    hipLaunchKernelGGL(kern, dim3(grid_1d(grid)), dim3(kHsymNT), lds, st, grp, A.col, B.rp, B.col,
                       (int)req, nwords, part * nwp, nwp, part * reqp, reqp, bslot, elem_fin,
                       dist_fin, gbits);
    SG_LAUNCH_CHECK();
}

void heavy_symbolic(const DevCSR& A, const DevCSR& B, const int64_t* S, const int32_t* hrows,
                    int64_t H, int64_t Nh, int64_t max_u, int ncu, int64_t dev_lds, int64_t ppow,
                    int64_t wfin, int32_t* bslot, int64_t* elem_fin, int64_t* dist_fin, Arena& ar,
                    hipStream_t st) {
    if (H <= 0) return;
    const int64_t req = ppow / wfin;
    const int logW = ilog2(wfin);
    if (req <= kBslotMaxReq) {
        if (B.n > 0) {
            const size_t lds = (size_t)(kBslotNT / kWave) * req * 4;
            SG_HIP(hipFuncSetAttribute((const void*)k_bslot_rows,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
            hipLaunchKernelGGL(k_bslot_rows, dim3(grid_1d(ceil_div(B.n * kWave, kBslotNT))),
                               dim3(kBslotNT), lds, st, B.rp, B.col, B.n, logW, (int)req, bslot);
            SG_LAUNCH_CHECK();
        }
    } else {
        fill<int32_t>(bslot, B.n * req, 0, st);
        if (B.n > 0) {
            hipLaunchKernelGGL(k_bslot_counts, dim3(grid_1d(ceil_div(B.n * kWave, 256))),
                               dim3(256), 0, st, B.rp, B.col, B.n, logW, (int)req, bslot);
            SG_LAUNCH_CHECK();
        }
    }
    const int nwords = (int)(ppow / 32);
    // the whole bitmap in one launch if two work groups fit a CU; else the
    // fewest column parts (with half the staging window) that do
    int np = 1, ew = kHsymEW;
    size_t lds = hsym_lds(kHsymEW, nwords, req);
    if (lds > (size_t)dev_lds / 2) {
        for (int cand = 2; cand <= req && cand <= 64; cand *= 2) {
            const size_t l = hsym_lds(kHsymEW / 2, nwords / cand, req / cand);
            if (l <= (size_t)dev_lds / 2) {
                np = cand;
                ew = kHsymEW / 2;
                lds = l;
                break;
            }
        }
    }
    // a work group's share: a quarter of the pass over the work groups the
    // device holds at once, and at least kHsymSplitMin products
    const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(2, dev_lds / (int64_t)lds));
    const int64_t T = std::max<int64_t>(kHsymSplitMin, ceil_div(Nh, 4 * (int64_t)ncu * per_cu));
    const int64_t* off = nullptr;
    const int32_t* bmap = nullptr;
    uint32_t* gbits = nullptr;
    int64_t grid = H, nsplit_max = 0;
    if (max_u > T) {
        // sum over rows of the work groups is at most H + Nh / T, and every
        // split row has more than T products
        nsplit_max = std::min<int64_t>(H, Nh / T);
        grid = H + Nh / T;
        int64_t* offw = ar.get<int64_t>("hsym_off", (size_t)H + 1);
        scan_exclusive(HsymSplitOf{A.rp, S, hrows, T}, H, offw, ar, st);
        int32_t* bmapw = ar.get<int32_t>("hsym_bmap", (size_t)grid);
        int32_t* smap = ar.get<int32_t>("hsym_smap", (size_t)nsplit_max + 1);
        gbits = ar.get<uint32_t>("hsym_gbits", (size_t)nsplit_max * nwords + 1);
        fill<uint32_t>(gbits, nsplit_max * (int64_t)nwords, 0u, st);
        hipLaunchKernelGGL(k_hsym_map, dim3(grid_1d(ceil_div(H, 256))), dim3(256), 0, st, offw, H,
                           (int)req, bmapw, smap, elem_fin);
        SG_LAUNCH_CHECK();
        off = offw;
        bmap = bmapw;
    }
    HsymGroup* grp = ar.get<HsymGroup>("hsym_grp", (size_t)grid);
    hipLaunchKernelGGL(k_hsym_groups, dim3(grid_1d(ceil_div(grid, 256))), dim3(256), 0, st, A.rp,
                       hrows, S, off, bmap, H, grid, grp);
    SG_LAUNCH_CHECK();
    const int nwp = nwords / np, reqp = (int)req / np;
    // with column parts, B's columns split by part once, so that each part's
    // launch reads only its own columns of every B row
    const int64_t* ppos = nullptr;
    const int32_t* pcol = nullptr;
    if (np > 1 && B.n > 0) {
        const int shift = ilog2((int64_t)nwp * 32);
        int64_t* cnt = ar.get<int64_t>("bpart_cnt", (size_t)np * B.n + 1);
        int64_t* pp = ar.get<int64_t>("bpart_pos", (size_t)np * B.n + 1);
        int32_t* pc = ar.get<int32_t>("bpart_col", (size_t)B.nnz + 1);
        const size_t plds = (size_t)(kBpartNT / kWave) * np * 4;
        const unsigned blocks = grid_1d(ceil_div(B.n * kWave, kBpartNT));
        hipLaunchKernelGGL(k_bpart_count, dim3(blocks), dim3(kBpartNT), plds, st, B.rp, B.col, B.n,
                           shift, np, cnt);
        SG_LAUNCH_CHECK();
        scan_exclusive(LoadI64{cnt}, (int64_t)np * B.n, pp, ar, st);
        hipLaunchKernelGGL(k_bpart_scatter, dim3(blocks), dim3(kBpartNT), plds, st, B.rp, B.col,
                           B.n, shift, np, (const int64_t*)pp, pc);
        SG_LAUNCH_CHECK();
        ppos = pp;
        pcol = pc;
    }
    for (int part = 0; part < np; ++part) {
        DevCSR Bp = B;
        if (ppos) {
            Bp.rp = ppos + (int64_t)part * B.n;  // [rp[k], rp[k+1]): row k's part-p columns
            Bp.col = pcol;
        }
        if (ew == kHsymEW) {
            if (B.nnz < (int64_t(1) << 31))
                launch_hsym<kHsymEW, true>(lds, grid, st, grp, A, Bp, req, nwords, part, nwp, reqp,
                                           bslot, elem_fin, dist_fin, gbits);
            else
                launch_hsym<kHsymEW, false>(lds, grid, st, grp, A, Bp, req, nwords, part, nwp, reqp,
                                            bslot, elem_fin, dist_fin, gbits);
        } else {
            if (B.nnz < (int64_t(1) << 31))
                launch_hsym<kHsymEW / 2, true>(lds, grid, st, grp, A, Bp, req, nwords, part, nwp,
                                               reqp, bslot, elem_fin, dist_fin, gbits);
            else
                launch_hsym<kHsymEW / 2, false>(lds, grid, st, grp, A, Bp, req, nwords, part, nwp,
                                                reqp, bslot, elem_fin, dist_fin, gbits);
        }
    }
    if (off && nsplit_max > 0) {
        hipLaunchKernelGGL(k_hsym_finalize, dim3(grid_1d(nsplit_max)), dim3(kHsymNT),
                           (size_t)req * 4, st, off, H, (const int32_t*)ar.get<int32_t>("hsym_smap", (size_t)nsplit_max + 1),
                           (const uint32_t*)gbits, (int)req, nwords, dist_fin);
        SG_LAUNCH_CHECK();
    }
}

// Per natural chunk of a level: its first finest slot, and its element and
// distinct-column counts as sums over its `g` finest slots. Level 0's
// parents are the heavy rows (slot base h*req); a deeper level's parents are
// the previous level's heavy chunks, found through that level's inv map.
__global__ void k_level_from_slots(const int64_t* parent_slot0, const int32_t* parent_inv,
                                   int64_t nparents, int nch, int g, int64_t req,
                                   const int64_t* elem_fin, const int64_t* dist_fin,
                                   int64_t* counts, int64_t* nnz, int64_t* slot0) {
    int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= nparents * nch) return;
    int64_t p = x / nch;
    int c = (int)(x - p * nch);
    int64_t ps = parent_inv ? parent_slot0[parent_inv[p]] : p * req;
    int64_t s = ps + (int64_t)c * g;
    int64_t e = 0, d = 0;
    for (int j = 0; j < g; ++j) {
        e += elem_fin[s + j];
        d += dist_fin[s + j];
    }
    counts[x] = e;
    nnz[x] = d;
    slot0[x] = s;
}

void level_from_slots(const int64_t* parent_slot0, const int32_t* parent_inv, int64_t nparents,
                      int nch, int g, int64_t req, const int64_t* elem_fin,
                      const int64_t* dist_fin, int64_t* counts, int64_t* nnz, int64_t* slot0,
                      hipStream_t st) {
    int64_t n = nparents * nch;
    if (n <= 0) return;
    hipLaunchKernelGGL(k_level_from_slots, dim3(grid_1d(ceil_div(n, 256))), dim3(256), 0, st,
                       parent_slot0, parent_inv, nparents, nch, g, req, elem_fin, dist_fin, counts,
                       nnz, slot0);
    SG_LAUNCH_CHECK();
}

// ---------------------------------------------------------------- chunk tree
__global__ void k_reduce_children(const int64_t* nnz_child, int nch, int64_t nparents,
                                  const int32_t* inv, int64_t* nnz_parent) {
    int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= nparents) return;
    int64_t s = 0;
    for (int c = 0; c < nch; ++c) s += nnz_child[p * nch + c];
    nnz_parent[inv ? inv[p] : p] = s;
}

void reduce_children(const int64_t* nnz_child, int nch, int64_t nparents, const int32_t* inv,
                     int64_t* nnz_parent, hipStream_t st) {
    if (nparents <= 0) return;
    hipLaunchKernelGGL(k_reduce_children, dim3(grid_1d(ceil_div(nparents, 256))), dim3(256), 0,
                       st, nnz_child, nch, nparents, inv, nnz_parent);
    SG_LAUNCH_CHECK();
}

__global__ void k_child_offsets(const int64_t* nnz_child, int nch, int64_t nparents,
                                const int32_t* map, const int64_t* base, int64_t* off_child) {
    int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= nparents) return;
    int64_t o = base[map[p]];
    for (int c = 0; c < nch; ++c) {
        off_child[p * nch + c] = o;
        o += nnz_child[p * nch + c];
    }
}

void child_offsets(const int64_t* nnz_child, int nch, int64_t nparents, const int32_t* map,
                   const int64_t* base, int64_t* off_child, hipStream_t st) {
    if (nparents <= 0) return;
    hipLaunchKernelGGL(k_child_offsets, dim3(grid_1d(ceil_div(nparents, 256))), dim3(256), 0, st,
                       nnz_child, nch, nparents, map, base, off_child);
    SG_LAUNCH_CHECK();
}

}  // namespace sg
