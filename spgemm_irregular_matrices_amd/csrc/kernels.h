// Launchers of the HIP kernels, called by the host orchestration (plan.cpp).
// Names follow the steps of Algorithm 3 on the gMAGNUS page.
#pragma once

#include "arena.h"
#include "common.h"

namespace sg {

struct DevCSR {
    int64_t n = 0, m = 0, nnz = 0;
    const int64_t* rp = nullptr;
    const int32_t* col = nullptr;
    const double* val = nullptr;
};

// Row bins: the light/heavy split of Algorithm 3 (ThreshPartition at tau)
// and the work-group-size binning of Section III-E. Partition order is
// bin order, so heavy rows come first.
enum RowBin : int {
    RB_HEAVY = 0,  // u > tau: outer product + multisplit path
    RB_T8,         // light, u <= 8: one thread per row, products sorted in registers
    RB_T16,        // light, u <= 16
    RB_T32,        // light, u <= 32
    RB_WIN64,      // light, output span <= 64: wave-per-row dense window
    RB_WIN1024,    // light, output span <= 1024: block dense window
    RB_H128,       // light hash bins by u (table slots >= 2u, alpha = 2)
    RB_H512,
    RB_H2048,
    RB_H8192,
    RB_EMPTY,      // u = 0
    RB_COUNT
};

// Chunk bins of one multisplit level. Heavy chunks (> tau) of a non-final
// level go first: they are the next level's input (Section III-A).
enum ChunkBin : int {
    CB_NEXT = 0,  // > tau, not the last level: split again
    CB_DENSE,     // > tau at the last level: dense LDS accumulation
    CB_H128,      // light chunks: LDS hash accumulation
    CB_H512,
    CB_H2048,
    CB_H8192,
    CB_EMPTY,
    CB_COUNT
};

// Hash-table slots per light bin and the largest item each bin takes.
constexpr int kHashSlots[4] = {128, 512, 2048, 8192};
constexpr int64_t kHashMaxItems[4] = {64, 256, 1024, 8191};
// Light chunks no wider than this use the bitmap-rank accumulator.
constexpr int64_t kRankMaxWidth = 65536;
// Largest u of each thread-local bin (one thread per row, registers only).
constexpr int64_t kThreadMaxItems[3] = {8, 16, 32};
constexpr int kWinSmall = 64;
constexpr int kWinLarge = 1024;

// ---------------------------------------------------------------- setup
// Validation: rowptr monotone with rowptr[0] = 0 and rowptr[n] = nnz, and
// every column in [0, ncols). Sets bit 1 (rowptr) or 2 (column) in *flag.
void launch_validate(const DevCSR& M, int* flag, hipStream_t st);

// S[q] = sum_{q' < q} nnz(B[A.col[q'],:]) for q in [0, A.nnz] (InterOffsets,
// Algorithm 3, at entry granularity: u(i) = S[rp[i+1]] - S[rp[i]]).
void entry_prefix(const DevCSR& A, const DevCSR& B, int64_t* S, Arena& ar, hipStream_t st);
// out[0] = sum over A entries q of (S[q+1] - S[q])^2.
void entry_len_sq(const int64_t* S, int64_t nnz, double* out, hipStream_t st);

// Per B row: smallest and largest column (INT32_MAX / -1 for empty rows).
void brow_minmax(const DevCSR& B, int32_t* bmin, int32_t* bmax, hipStream_t st);

// Row classification and stable partition into RowBins.
// stats[0]=sum u, [1]=max u, [2]=heavy rows, [3]=heavy products, [4..6]=rows
// with u <= 512, 4096, 32768, [7]=sum of u^2 (a double); uhist counts the
// rows per u bucket (kUHistBuckets: u < 64 exactly, then 64 per octave).
constexpr int kUHistBuckets = 4096;
// Entries of the row statistics record classify_rows fills: sum, max, heavy
// rows and products of u(i), the F_h counts, the sum of u(i)^2, the A
// entries of the light rows, and one word for the light rows' outputs.
constexpr int kRowStats = 10;
// out[0] = sum over j < n of cnt[perm[j]].
void sum_rows(const int32_t* perm, int64_t n, const int64_t* cnt, int64_t* out, hipStream_t st);
void classify_rows(const DevCSR& A, const int64_t* S, const int32_t* bmin, const int32_t* bmax,
                   int64_t tau, int32_t* rowlo, int32_t* perm, int64_t* bin_start,
                   int64_t* stats, int32_t* uhist, Arena& ar, hipStream_t st);

// ---------------------------------------------------------------- heavy path
// C-hat row pointers: exclusive scan of u over the heavy rows perm[0..H).
void heavy_rowptr(const DevCSR& A, const int64_t* S, const int32_t* hrows, int64_t H,
                  int64_t* chat_rp, Arena& ar, hipStream_t st);

// Masked CSR-to-CSC of A[heavy rows, :] for the heavy rows hrows[0..H) of
// one batch, keeping only entries whose B row is nonempty. ent_k = column of
// A (the slice), ent_q = A entry index, ent_dest = position, relative to
// dest_base, of the entry's first product in C-hat (chat_rp holds the
// batch's C-hat row starts); P = exclusive scan of the entries' piece counts
// ceil(nnz(B[ent_k,:]) / 64), the flattened slice offsets in units of
// 64-product pieces. Outputs go to caller buffers of ent_capacity entries
// (P: one more). Returns the entry count.
int64_t masked_csr2csc(const DevCSR& A, const DevCSR& B, const int64_t* S, const int32_t* hrows,
                       int64_t H, const int64_t* chat_rp, int64_t dest_base, int32_t* ent_k,
                       int64_t* ent_q, int64_t* ent_dest, int64_t ent_capacity, int64_t* P,
                       int64_t* total_pieces, Arena& ar, hipStream_t st);
// out[i] = a[i] - base for i < n.
void rebase(const int64_t* a, int64_t n, int64_t base, int64_t* out, hipStream_t st);

struct ExpandArgs {
    const int32_t* ent_k;
    const int64_t* ent_q;
    const int64_t* ent_dest;
    const int64_t* P;
    int64_t ne;
    const double* Aval;
    const int64_t* Brp;
    const int32_t* Bcol;
    const double* Bval;
    int32_t* out_col;
    double* out_val;  // null: columns only
    int64_t total_pieces;    // P[ne]
    const int64_t* tile_e0;  // first entry of every tile (expand_tile_starts)
};
// Number of expand tiles, and their first entries (cached between calls).
int64_t expand_tiles(int64_t total_pieces);
void expand_tile_starts(const int64_t* P, int64_t ne, int64_t total_pieces, int64_t* tile_e0,
                        hipStream_t st);
// OuterProduct (Algorithm 4): every (a, B-row) pair of every slice written
// to its C-hat position.
void expand(const ExpandArgs& a, hipStream_t st);

struct LevelGeom {
    const int64_t* rp;  // input row pointers, nrows+1
    int64_t nrows;
    int64_t total;      // rp[nrows]
    int shift;          // log2 of this level's chunk width
    int nch;            // chunks per input row (power of two)
    int64_t tau;        // every input row has > tau elements
};

// Histogram (Section III-C): counts[r*nch + c] += elements of row r in chunk c.
void histogram(const LevelGeom& g, const int32_t* in_col, int64_t* counts, Arena& ar,
               hipStream_t st);

// Classify the level's chunks and partition them (CB_* order). inv[pos] =
// natural chunk index, pos_of[natural] = pos. bin_start has CB_COUNT+1.
void classify_chunks(const int64_t* counts, int64_t nchunks, int64_t tau, bool last_level,
                     int32_t* inv, int32_t* pos_of, int64_t* bin_start, Arena& ar,
                     hipStream_t st);

// rp_out[p] = exclusive scan of counts[inv[p]] over p in [0, npos).
void reord_rowptr(const int64_t* counts, const int32_t* inv, int64_t npos, int64_t* rp_out,
                  Arena& ar, hipStream_t st);

// Multisplit (Algorithm 5): permute the level's input into C-hat-reord.
// cursor[pos] starts at rp_out[pos] and is advanced by reservations.
// With out16 the output columns are 16-bit offsets inside each chunk
// (written to out_col's memory as uint16), for levels whose chunks are at
// most 2^16 columns wide.
void multisplit(const LevelGeom& g, const int32_t* in_col, const double* in_val,
                const int32_t* pos_of, int64_t* cursor, int32_t* out_col, double* out_val,
                bool out16, Arena& ar, hipStream_t st);
// Outer product and first multisplit level in one pass (numeric): the
// products of the C-hat rows g.rp are formed from A, B and InterOffsets S
// tile by tile and multisplit as they are formed, without writing C-hat.
struct FusedRows {
    const int64_t* hq0;  // per C-hat row of the batch: first A entry
    const int64_t* hq1;  // one past the last A entry
    const int64_t* hs0;  // InterOffsets at the first entry
    const int64_t* ebo;  // per A entry (all of A): first entry of its B row
};
void fused_setup(const DevCSR& A, const DevCSR& B, const int64_t* S, const int32_t* hrows,
                 int64_t H, int64_t* hq0, int64_t* hq1, int64_t* hs0, int64_t* ebo,
                 hipStream_t st);
void expand_multisplit(const LevelGeom& g, const FusedRows& fr, const DevCSR& A, const DevCSR& B,
                       const int64_t* S, const int32_t* pos_of, int64_t* cursor, int32_t* out_col,
                       double* out_val, bool out16, Arena& ar, hipStream_t st);
// out[p*nch + c] = (parent_inv ? parent_base[parent_inv[p]] : 0) + c*width.
void chunk_colbase(int64_t nparents, int nch, int64_t width, const int32_t* parent_inv,
                   const int32_t* parent_base, int32_t* out, hipStream_t st);

// Fused symbolic pass over the heavy rows (a work group per row, several for
// a row far above the average share): per finest chunk slot of width wfin,
// the element count and the number of distinct columns. Needs
// heavy_symbolic_lds(ppow, ppow/wfin) bytes of LDS.
size_t heavy_symbolic_lds(int64_t ppow, int64_t req);
// bslot (B.n * (ppow/wfin) int32) receives every B row's entries per slot.
// S is the entry product prefix, Nh the heavy rows' products, max_u the
// largest u(i); ncu and dev_lds size the per-work-group share.
void heavy_symbolic(const DevCSR& A, const DevCSR& B, const int64_t* S, const int32_t* hrows,
                    int64_t H, int64_t Nh, int64_t max_u, int ncu, int64_t dev_lds, int64_t ppow,
                    int64_t wfin, int32_t* bslot, int64_t* elem_fin, int64_t* dist_fin, Arena& ar,
                    hipStream_t st);
// Counts, distinct counts and first finest slot of every natural chunk of a
// level, summed from the finest slots (g slots per chunk).
void level_from_slots(const int64_t* parent_slot0, const int32_t* parent_inv, int64_t nparents,
                      int nch, int g, int64_t req, const int64_t* elem_fin,
                      const int64_t* dist_fin, int64_t* counts, int64_t* nnz, int64_t* slot0,
                      hipStream_t st);

// nnz_parent[inv[p]] = sum_c nnz_child[p*nch + c] for p < nparents.
void reduce_children(const int64_t* nnz_child, int nch, int64_t nparents, const int32_t* inv,
                     int64_t* nnz_parent, hipStream_t st);
// off_child[p*nch + c] = base[map[p]] + sum_{c'<c} nnz_child[p*nch + c'].
void child_offsets(const int64_t* nnz_child, int nch, int64_t nparents, const int32_t* map,
                   const int64_t* base, int64_t* off_child, hipStream_t st);

// ---------------------------------------------------------------- accumulation
// Light rows, straight from A and B (Gustavson, Algorithm 1 per row).
struct RowItems {
    DevCSR A, B;
    const int64_t* S;
    const int32_t* perm;   // row ids in bin order
    const int32_t* rowlo;  // window base per row (window bins)
    int64_t* cnt;          // symbolic: nnz per row
    const int64_t* Crp;    // numeric: row offsets
    int32_t* Ccol;
    double* Cval;
    int hash_top_logS;     // slots (log2) of the largest light hash table
};
void accumulate_rows(const RowItems& it, int bin, int64_t p0, int64_t n, bool numeric,
                     hipStream_t st);

// Chunks (or whole C-hat rows when no multisplit level is needed).
struct ChunkItems {
    const int64_t* rp;     // element range per position
    const int32_t* map;    // output index per position
    const int32_t* bcol;
    const double* bval;
    int64_t* cnt;          // symbolic: cnt[map[p]]
    const int64_t* off;    // numeric: off[map[p]]
    int32_t* Ccol;
    double* Cval;
    int64_t width;         // column width of every chunk (power of two)
    int hash_top_logS;     // slots (log2) of the largest light hash table
    const uint16_t* bcol16;  // if set: columns as 16-bit offsets from colbase[map[p]]
    const int32_t* colbase;
};
void accumulate_chunks(const ChunkItems& it, int bin, int64_t p0, int64_t n, bool numeric,
                       hipStream_t st);

// ---------------------------------------------------------------- direct
// Heavy rows accumulated per (heavy row, final chunk) item straight from A
// and a chunk-partitioned copy of B (no C-hat): items of more than
// kDirectDense products use the dense window, smaller ones the bitmap-rank
// accumulator. Slots per row are bounded so that every wave of the B
// partition keeps its slot offsets in LDS.
constexpr int64_t kDirectDense = 2048;
constexpr int kDirectMaxSlots = 4096;
// Item classes of the direct path: the dense window, then bitmap-rank
// classes by product count (class r takes items of at most
// kRankClassMax[r] products), then the empty items.
constexpr int kNumRankClasses = 6;
constexpr int64_t kRankClassMax[kNumRankClasses] = {64, 128, 256, 512, 1024, 2048};
static_assert(kRankClassMax[kNumRankClasses - 1] == kDirectDense, "rank classes end at the window");
enum DirectClass : int {
    DC_DENSE = 0,
    DC_RANK0 = 1,
    DC_EMPTY = DC_RANK0 + kNumRankClasses,
    DC_COUNT
};
struct DirectArgs {
    const int32_t* items;   // item ids h*req + s, in class order
    int req;                // final chunks (slots) per row
    int logW;               // log2 of the slot width
    const int64_t* hq0;     // per heavy row: first A entry
    const int64_t* hq1;     // one past its last A entry
    const int64_t* iq0;     // per position of items: its row's first A entry
    const int32_t* ine;     // per position of items: its row's A entries
    const int32_t* Acol;
    const double* Aval;
    const int32_t* spos;    // req x B.nrows (+1): where row k's part of slot s starts in split B
    int64_t nb;             // B.nrows
    const uint32_t* eocc;   // ceil(req/32) x A.nnz words: bit s & 31 of word
                            // (s >> 5) * annz + q set if B row Acol[q] has entries in slot s
    int64_t annz;           // A.nnz
    bool occ;               // dense and rank items test eocc (runs always do)
    const uint16_t* bcol16; // partitioned B: column offset inside the slot
    const double* bval;     // partitioned B: values
    const int64_t* off;     // per item: output offset in C
    int32_t* Ccol;
    double* Cval;
    const int64_t* rhdr;    // per run: first item id h*req + s0 | slot mask << 32
    const int64_t* rq0;     // per run: its row's first A entry
    const int32_t* rne;     // per run: its row's A entries
};
// Runs: a heavy row's items of at most kRunMax products, taken together by
// one wavefront. A run starts at a small item's slot s0 and holds the row's
// next small items while their products stay within kRunMax, their slots
// within s0 + run_span(logW), and no larger item lies between them; bit t
// of its mask marks slot s0 + t. Its output is the concatenation of its
// items' outputs (slots in column order, the empty ones write nothing).
constexpr int kRunClasses = 2;  // the smallest rank classes that runs take
constexpr int64_t kRunMax = kRankClassMax[kRunClasses - 1];
constexpr int kRunKPT = (int)(kRunMax / 64);  // products per lane of a run
__host__ __device__ constexpr int run_span(int logW) {
    return (65536 >> logW) < 8 ? (65536 >> logW) : 8;
}
// The split copy of B, slot by slot (B.nnz < 2^31): spos (req*B.n + 1) from the
// per-row slot counts bslot; bperm[p] = B entry placed at p, bcol16[p] its
// column inside its slot; roc (B.n x ceil(req/32) words): bit t of word
// k * ceil(req/32) + w set if B row k has entries in slot 32 w + t.
void direct_split_b(const DevCSR& B, const int32_t* bslot, int req, int64_t W, int32_t* spos,
                    uint32_t* roc, int32_t* bperm, uint16_t* bcol16, Arena& ar, hipStream_t st);
// The occupancy words of every A entry's B row, slot-word-major (see
// DirectArgs::eocc).
void direct_entry_occ(const int32_t* acol, int64_t annz, int req, const uint32_t* roc,
                      uint32_t* eocc, hipStream_t st);
// Items test the occupancy bits before reading a slice's bounds when the B
// rows that the products come from average fewer than req / kOccSparse
// entries (a product-weighted mean), so that most (B row, slot) slices of
// an item are empty.
constexpr int kOccSparse = 4;
void direct_offsets(const int64_t* C_rp, const int32_t* hrows, int64_t H, int req,
                    const int64_t* dist_fin, int64_t* off, hipStream_t st);
// The direct path's work lists, from the exact product count of every item
// (elem_fin, H x req): items[0, ndense) the dense items in row order, then
// the bitmap-rank classes that the runs do not take, each in slot order
// (all rows' items of slot 0 first), with per position the item's row's
// first A entry and entry count (iq0, ine); bins: DC_COUNT + 1 class starts
// (the run classes and the empty class are empty ranges); the runs
// (rhdr, rq0, rne; at most H*req) in the order of their first slot; and
// run_meta = {runs, A entries read, (entry, slot) slice bounds read}.
void direct_classify(const int64_t* elem_fin, int64_t H, int req, int logW, const int64_t* hq0,
                     const int64_t* hq1, int32_t* items, int64_t* iq0, int32_t* ine,
                     int64_t* bins, int64_t* rhdr, int64_t* rq0, int32_t* rne, int64_t* run_meta,
                     Arena& ar, hipStream_t st);
void direct_gather_values(const int32_t* bperm, const double* bval, int64_t nnz, double* out,
                          hipStream_t st);
// out8 = {dense items: products, outputs, A entries read; rank items of more
// than kRunMax products: the same; items of at most kRunMax: products,
// outputs}.
void direct_totals(const int64_t* hq0, const int64_t* hq1, int64_t H, int req,
                   const int64_t* elem_fin, const int64_t* dist_fin, int64_t* out8, Arena& ar,
                   hipStream_t st);
size_t direct_window_lds(int64_t W);
void direct_accumulate(const DirectArgs& d, int cls, int64_t p0, int64_t n, hipStream_t st);
void direct_accumulate_runs(const DirectArgs& d, int64_t nruns, hipStream_t st);

}  // namespace sg
