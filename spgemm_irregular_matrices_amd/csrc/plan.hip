// Host orchestration and the C ABI (include/spgemm.h).
//
// spgemm_symbolic runs Algorithm 3 of the gMAGNUS page up to and including
// the prefix sum of C.rowPtr; spgemm_numeric runs the heavy path with values
// and then the accumulation steps. The structure the symbolic pass finds (row
// bins, the masked CSC, every level's chunk partition, C-hat-reord row
// pointers and chunk output offsets) is kept in the plan, so the numeric
// pass does no histogramming, partitioning or blocking host reads.
//
// Heavy rows are processed in batches of consecutive heavy rows whose
// intermediate products fit a budget (max_batch_products; one batch by
// default). Each batch has its own masked CSC, C-hat, levels and chunk
// partitions, so C-hat and C-hat-reord need buffers of one batch's size.
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/spgemm.h"
#include "kernels.h"
#include "primitives.h"

using namespace sg;

namespace {

constexpr int kMaxLevels = SPGEMM_MAX_LEVELS;

// Parameters of Section III-D (GetMagnusParams) for one product.
struct Params {
    int64_t slm = 0;      // local memory per work group (s_LM)
    int64_t tau = 0;      // heavy threshold, Eq. (4)
    int64_t wdense = 0;   // dense accumulator width (power of two)
    int64_t ppow = 0;     // column range rounded up to a power of two
    int nlevels = 0;
    int vchunks[kMaxLevels] = {};
    int64_t width[kMaxLevels] = {};  // chunk width after level l
    int64_t final_width = 0;
    int64_t nchunks_required = 1;
    int64_t nchunks_max = 0;
    int hash_top_logS = 13;  // slots of the largest light hash table (log2)
};

// One multisplit level of one batch. Natural chunk indices of the level are
// local to the batch (parent * nch + chunk); the level's arrays hold every
// batch, the batch's part starting at nat_off (and its C-hat-reord row
// pointers at rp_off).
struct LevelState {
    int64_t R = 0;         // input rows (C-hat rows or the previous level's heavy chunks)
    int64_t total_in = 0;  // input elements
    int nch = 0;
    int shift = 0;
    int64_t nnat = 0;      // R * nch
    int64_t npos = 0;      // nonempty chunks
    int64_t bins[CB_COUNT + 1] = {};
    int64_t final_elems = 0;  // elements of this level's accumulated (non-split) chunks
    int64_t nat_off = 0;
    int64_t rp_off = 0;
    int64_t nheavy() const { return bins[CB_NEXT + 1] - bins[CB_NEXT]; }
};

// A run of consecutive heavy rows [h0, h1) processed together.
struct BatchState {
    int64_t h0 = 0, h1 = 0;
    int64_t N = 0;          // intermediate products (C-hat elements)
    int64_t chat_base = 0;  // C-hat offset of the batch's first row
    int64_t ent0 = 0, ne = 0;   // masked CSC entries
    int64_t P0 = 0;             // offset of the batch's piece prefix (ne + 1 values)
    int64_t npieces = 0;
    int64_t tile0 = 0;          // offset of the batch's expand tile starts
    int64_t crp0 = 0;           // offset of the batch's rebased C-hat row pointers (R + 1)
    int L = 0;
    LevelState lv[kMaxLevels];
};

}  // namespace

// Pinned host words: 64 for small scalars, then the u histogram (int32).
constexpr int kHostWords = 64 + sg::kUHistBuckets / 2;
// The direct path's metadata, read back in one copy: its class starts
// (DC_COUNT + 1), the totals of direct_totals (8), the product-weighted
// B-row length sum (a double), and the runs' count, A entries and
// (entry, slot) pairs.
constexpr int kDirTot = sg::DC_COUNT + 1;
constexpr int kDirLenSq = kDirTot + 8;
constexpr int kDirRuns = kDirLenSq + 1;
constexpr int kDirMeta = kDirRuns + 3;

struct spgemm_plan_s {
    spgemm_options opt{};
    Arena ar;
    int device = 0;
    int64_t dev_lds = 0;
    int dev_cus = 1;
    int64_t* host = nullptr;  // pinned staging for small device-to-host reads (kHostWords)
    // the light rows' numeric pass runs on a stream of its own, beside the
    // heavy rows (the two queues of Algorithm 3), joined before returning
    hipStream_t lst = nullptr;
    hipEvent_t ev_fork = nullptr, ev_join = nullptr;
    // state of the last successful symbolic call
    bool ready = false;
    int64_t An = 0, Am = 0, Annz = 0, Bn = 0, Bm = 0, Bnnz = 0, Cnnz = 0;
    Params prm;
    int64_t row_bins[RB_COUNT + 1] = {};
    int64_t H = 0, Nh = 0;
    int L = 0;  // deepest level used by any batch
    std::vector<BatchState> batches;
    int64_t maxN = 0;                         // largest batch (C-hat buffer size)
    int64_t cap_nat[kMaxLevels] = {}, cap_rp[kMaxLevels] = {};
    int64_t cap_ent = 0, cap_P = 0, cap_tiles = 0, cap_crp = 0;
    spgemm_stats stats{};
    // timing
    struct Ev {
        int pass, phase;
        hipEvent_t a, b;
    };
    std::vector<hipEvent_t> evpool;
    size_t evnext = 0;
    std::vector<Ev> evs;
    bool fused_sym = false;
    bool fused_num = false;  // numeric level 0 forms its products itself (no C-hat)
    bool direct = false;     // heavy rows accumulated per (row, final chunk) from A and split B
    int direct_req = 0;      // final chunks per heavy row on the direct path
    bool direct_occ = false;  // items test the slices' occupancy bits
    int64_t direct_W = 0;    // their width
    int64_t dir_bins[DC_COUNT + 1] = {};
    // dense / rank items: products, outputs, A entries read; runs: products, outputs
    int64_t dir_tot[8] = {};
    int64_t dir_runs[3] = {};  // runs, their A entries and (entry, slot) pairs read
    int64_t light_annz = 0;   // A entries of the light rows
    int64_t light_cnnz = 0;   // output entries of the light rows
    // debug dumps (kept for single-batch products)
    bool dbg_valid = false;
    bool dbg_chat = false;  // C-hat was dumped (separate outer product only)
    bool dbg_has_val = false;       // levels were dumped with values
    bool dbg_chat_val = false;      // C-hat was dumped with values
};

namespace {

hipEvent_t next_event(spgemm_plan p) {
    if (p->evnext == p->evpool.size()) {
        hipEvent_t e;
        SG_HIP(hipEventCreate(&e));
        p->evpool.push_back(e);
    }
    return p->evpool[p->evnext++];
}

// Records HIP events around one phase on the phase's stream.
struct PhaseScope {
    spgemm_plan p;
    int pass, phase;
    hipStream_t st;
    hipEvent_t a = nullptr;
    PhaseScope(spgemm_plan p_, int pass_, int phase_, hipStream_t st_)
        : p(p_), pass(pass_), phase(phase_), st(st_) {
        if (p->opt.timing) {
            a = next_event(p);
            SG_HIP(hipEventRecord(a, st));
        }
    }
    ~PhaseScope() {
        if (p->opt.timing && a) {
            try {
                hipEvent_t b = next_event(p);
                if (hipEventRecord(b, st) == hipSuccess) p->evs.push_back({pass, phase, a, b});
            } catch (...) {
            }
        }
    }
};

void add_bytes(spgemm_plan p, int pass, int phase, double bytes) {
    p->stats.phase_bytes[pass][phase] += bytes;
}

int64_t* d2h(spgemm_plan p, const int64_t* dsrc, int64_t n, hipStream_t st) {
    if (n > 64) throw std::logic_error("staging buffer too small");
    SG_HIP(hipMemcpyAsync(p->host, dsrc, (size_t)n * sizeof(int64_t), hipMemcpyDeviceToHost, st));
    SG_HIP(hipStreamSynchronize(st));
    return p->host;
}

// Self-checks of a debug plan (debug_dump), on the host.
// A level's chunk sizes add up to its input: every element of the level's
// rows (Sigma u of the heavy rows at level 0, the heavy chunks' elements
// below) falls in exactly one chunk. rp is the level's exclusive scan of the
// sizes of its npos nonempty chunks.
void check_level_sizes(spgemm_plan p, const int64_t* rp, int64_t npos, int64_t total, int l,
                       hipStream_t st) {
    if (!p->opt.debug_dump) return;
    const int64_t sum = d2h(p, rp + npos, 1, st)[0];
    if (sum != total)
        throw InternalError("multisplit level " + std::to_string(l) + ": chunk sizes add up to " +
                            std::to_string(sum) + ", the level's input is " +
                            std::to_string(total));
}

// After a multisplit every chunk's cursor has moved from its start to the
// next chunk's start: no element was lost or placed twice.
void check_cursors(spgemm_plan p, const int64_t* cursor, const int64_t* rp, int64_t npos, int l,
                   hipStream_t st) {
    if (!p->opt.debug_dump || npos <= 0) return;
    std::vector<int64_t> cur((size_t)npos), end((size_t)npos);
    SG_HIP(hipMemcpyAsync(cur.data(), cursor, (size_t)npos * sizeof(int64_t),
                          hipMemcpyDeviceToHost, st));
    SG_HIP(hipMemcpyAsync(end.data(), rp + 1, (size_t)npos * sizeof(int64_t),
                          hipMemcpyDeviceToHost, st));
    SG_HIP(hipStreamSynchronize(st));
    for (int64_t i = 0; i < npos; ++i)
        if (cur[(size_t)i] != end[(size_t)i])
            throw InternalError("multisplit level " + std::to_string(l) + ": chunk " +
                                std::to_string(i) + " filled to " +
                                std::to_string(cur[(size_t)i]) + ", it ends at " +
                                std::to_string(end[(size_t)i]));
}

// GetMagnusParams (Section III-D). Readings of the garbled formulas:
// Eq. (4): tau = s_LM / (alpha * (s_col + s_val)), alpha = 2, so that a hash
// table of tau entries at load factor 1/alpha fills the local memory;
// because this library's hash tables have power-of-two sizes, tau is the
// half of the largest such table that fits in s_LM;
// n_denseNumeric = s_LM / (s_val + s_bitmap), with a one-byte flag per
// column; the dense width is floored to a power of two and the required
// chunk count is the column range (rounded up to a power of two) divided by
// it; nchunksMax follows Eq. (6) for the multisplit's own LDS arrays and is
// capped; nlevels is the smallest count with nchunksMax^nlevels >=
// nchunksRequired (Eq. 7), every level but the last uses nchunksMax and the
// last takes the remaining factor nchunksRequired / nchunksMax^(nlevels-1).
// s_LM defaults to half of a compute unit's LDS: two work groups of each
// LDS-heavy kernel stay resident per CU, so one group's memory phase
// overlaps the other's LDS phase.
Params get_params(spgemm_plan p, int64_t ncols_c) {
    Params q;
    const spgemm_options& o = p->opt;
    q.slm = o.lds_budget_bytes > 0 ? std::min(o.lds_budget_bytes, p->dev_lds) : p->dev_lds / 2;
    const int64_t s_col = 4, s_val = 8, alpha = 2, s_bitmap = 1, s_histo = 4, s_rowptr = 8;
    int64_t table = std::min<int64_t>(floor_pow2(q.slm / (s_col + s_val)), 8192);
    table = std::max<int64_t>(table, 2048);
    q.tau = std::min(q.slm / (alpha * (s_col + s_val)), table / alpha);
    if (o.tau_override > 0) q.tau = o.tau_override;
    q.tau = std::min<int64_t>(q.tau, kHashMaxItems[3]);
    q.tau = std::max<int64_t>(q.tau, 1);
    q.hash_top_logS = q.tau * alpha <= 4096 ? 12 : 13;
    int64_t ndense = q.slm / (s_val + s_bitmap);
    q.wdense = floor_pow2(ndense);
    // the dense-window kernel also keeps a 4-byte word prefix per 32 columns
    while (q.wdense > 32 && q.wdense * 8 + (q.wdense / 32) * 8 > std::max(q.slm, int64_t(4096)))
        q.wdense /= 2;
    if (o.chunk_width_override > 0) q.wdense = std::min(q.wdense, o.chunk_width_override);
    q.ppow = std::max<int64_t>(ceil_pow2(std::max<int64_t>(ncols_c, 1)), 32);
    const int64_t nmin = q.slm / (2 * (s_col + s_val));
    const int64_t ngroup_rows = 2, nsub = 1;
    int64_t eq6 = (q.slm - nmin * (s_col + s_val) - s_histo) /
                  (ngroup_rows * (nsub * s_histo + s_rowptr));
    int64_t cap = o.nchunks_cap > 0 ? o.nchunks_cap : 32;
    q.nchunks_max = std::max<int64_t>(2, std::min(floor_pow2(std::max<int64_t>(eq6, 2)), cap));
    if (q.ppow <= q.wdense) {
        q.nlevels = 0;
        q.final_width = q.ppow;
        q.nchunks_required = 1;
        return q;
    }
    q.nchunks_required = q.ppow / q.wdense;
    int lr = ilog2(q.nchunks_required), lm = ilog2(q.nchunks_max);
    q.nlevels = (lr + lm - 1) / lm;
    if (q.nlevels > kMaxLevels) throw OverflowError("more multisplit levels than supported");
    int64_t w = q.ppow;
    for (int l = 0; l < q.nlevels; ++l) {
        int64_t v = (l < q.nlevels - 1) ? q.nchunks_max
                                        : q.nchunks_required >> (lm * (q.nlevels - 1));
        q.vchunks[l] = (int)v;
        w /= v;
        q.width[l] = w;
    }
    q.final_width = w;
    return q;
}

DevCSR to_dev(const spgemm_csr* M) {
    DevCSR d;
    d.n = M->nrows;
    d.m = M->ncols;
    d.nnz = M->nnz;
    d.rp = M->rowptr;
    d.col = M->col;
    d.val = M->val;
    return d;
}

int check_csr(const spgemm_csr* M, bool need_val) {
    if (!M) return SPGEMM_ERR_INVALID_ARG;
    if (M->nrows < 0 || M->ncols < 0 || M->nnz < 0) return SPGEMM_ERR_INVALID_ARG;
    if (!M->rowptr) return SPGEMM_ERR_INVALID_ARG;
    if (M->nnz > 0 && (!M->col || (need_val && !M->val))) return SPGEMM_ERR_INVALID_ARG;
    if (M->ncols > 0x7fffffffLL || M->nrows >= 0x7fffffffLL) return SPGEMM_ERR_OVERFLOW;
    return SPGEMM_OK;
}

std::string lvname(const char* what, int l) { return std::string("lv") + std::to_string(l) + what; }

// A level's array of natural-chunk values (every batch), or of row pointers.
template <class T>
T* lvarr(spgemm_plan p, int l, const char* what, bool rowptrs = false) {
    const int64_t cap = rowptrs ? p->cap_rp[l] : p->cap_nat[l];
    return p->ar.get<T>(lvname(what, l), (size_t)cap + 1);
}

__global__ void k_i32_to_i64(const int32_t* a, int64_t n, int64_t* b) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) b[i] = a[i];
}

void debug_copy_chat(spgemm_plan p, const BatchState& bt, const int64_t* crp, const int32_t* col,
                     const double* val, const int32_t* hrows, hipStream_t st) {
    Arena& ar = p->ar;
    const int64_t R = bt.h1 - bt.h0;
    copy<int64_t>(ar.get<int64_t>("dbg_m1_rp", (size_t)R + 1), crp, R + 1, st);
    copy<int32_t>(ar.get<int32_t>("dbg_m1_col", (size_t)bt.N), col, bt.N, st);
    if (val) copy<double>(ar.get<double>("dbg_m1_val", (size_t)bt.N), val, bt.N, st);
    int64_t* key = ar.get<int64_t>("dbg_m1_key", (size_t)R + 1);
    hipLaunchKernelGGL(k_i32_to_i64, dim3(grid_1d(ceil_div(R, 256))), dim3(256), 0, st, hrows, R,
                       key);
    SG_LAUNCH_CHECK();
    p->dbg_valid = true;
    p->dbg_chat = true;
    p->dbg_chat_val = val != nullptr;
}

void debug_copy_level(spgemm_plan p, int l, const LevelState& S_l, const int64_t* rp,
                      const int32_t* col, const double* val, const int32_t* inv, hipStream_t st) {
    Arena& ar = p->ar;
    int64_t nnz = d2h(p, rp + S_l.npos, 1, st)[0];
    std::string b = "dbg_l" + std::to_string(l);
    copy<int64_t>(ar.get<int64_t>(b + "_rp", (size_t)S_l.npos + 1), rp, S_l.npos + 1, st);
    copy<int32_t>(ar.get<int32_t>(b + "_col", (size_t)nnz), col, nnz, st);
    if (val) copy<double>(ar.get<double>(b + "_val", (size_t)nnz), val, nnz, st);
    int64_t* key = ar.get<int64_t>(b + "_key", (size_t)S_l.npos + 1);
    p->dbg_valid = true;
    p->dbg_has_val = val != nullptr;
    if (S_l.npos > 0) {
        hipLaunchKernelGGL(k_i32_to_i64, dim3(grid_1d(ceil_div(S_l.npos, 256))), dim3(256), 0, st,
                           inv, S_l.npos, key);
        SG_LAUNCH_CHECK();
    }
}

// ---------------------------------------------------------------- batches
// Consecutive heavy rows whose products fit max_batch_products (a row larger
// than the budget is a batch of its own); one batch when there is no budget.
void plan_batches(spgemm_plan p, const int64_t* chat_rp, hipStream_t st) {
    p->batches.clear();
    const int64_t budget = p->opt.max_batch_products;
    if (budget <= 0 || p->Nh <= budget) {
        BatchState b;
        b.h0 = 0;
        b.h1 = p->H;
        b.N = p->Nh;
        p->batches.push_back(b);
    } else {
        std::vector<int64_t> h((size_t)p->H + 1);
        SG_HIP(hipMemcpyAsync(h.data(), chat_rp, h.size() * sizeof(int64_t),
                              hipMemcpyDeviceToHost, st));
        SG_HIP(hipStreamSynchronize(st));
        int64_t h0 = 0;
        while (h0 < p->H) {
            int64_t h1 = h0 + 1;
            while (h1 < p->H && h[h1 + 1] - h[h0] <= budget) ++h1;
            BatchState b;
            b.h0 = h0;
            b.h1 = h1;
            b.N = h[h1] - h[h0];
            b.chat_base = h[h0];
            p->batches.push_back(b);
            h0 = h1;
        }
    }
    p->maxN = 0;
    for (auto& b : p->batches) p->maxN = std::max(p->maxN, b.N);
}

// Upper bounds of the arrays that hold every batch: a batch's level-l input
// rows (l >= 1) each hold more than tau elements, so their number is at
// most N_b / (tau + 1).
void plan_capacities(spgemm_plan p, const DevCSR& A) {
    const Params& q = p->prm;
    const int64_t nb = (int64_t)p->batches.size();
    for (int l = 0; l < kMaxLevels; ++l) p->cap_nat[l] = p->cap_rp[l] = 0;
    for (int l = 0; l < q.nlevels; ++l) {
        const int64_t rows = l == 0 ? p->H : p->Nh / (q.tau + 1);
        p->cap_nat[l] = rows * q.vchunks[l];
        p->cap_rp[l] = p->cap_nat[l] + nb;
        if (p->cap_nat[l] >= (int64_t(1) << 31)) throw OverflowError("too many chunks in a level");
    }
    p->cap_ent = A.nnz;
    p->cap_P = A.nnz + nb;
    p->cap_tiles = (A.nnz + p->Nh / 64 + nb) / 128 + 2 * nb + 2;
    p->cap_crp = p->H + nb;
}

struct CscBufs {
    int32_t* ent_k;
    int64_t* ent_q;
    int64_t* ent_dest;
    int64_t* P;
    int64_t* tiles;
    int64_t* crp;
};

CscBufs csc_bufs(spgemm_plan p) {
    Arena& ar = p->ar;
    return {ar.get<int32_t>("csc_ent_k", (size_t)p->cap_ent + 1),
            ar.get<int64_t>("csc_ent_q", (size_t)p->cap_ent + 1),
            ar.get<int64_t>("csc_ent_dest", (size_t)p->cap_ent + 1),
            ar.get<int64_t>("csc_slice_off", (size_t)p->cap_P + 1),
            ar.get<int64_t>("expand_tiles", (size_t)p->cap_tiles + 1),
            ar.get<int64_t>("chat_rp_local", (size_t)p->cap_crp + 1)};
}

ExpandArgs expand_args(spgemm_plan p, const BatchState& bt, const DevCSR& A, const DevCSR& B,
                       int32_t* out_col, double* out_val) {
    CscBufs c = csc_bufs(p);
    return ExpandArgs{c.ent_k + bt.ent0, c.ent_q + bt.ent0, c.ent_dest + bt.ent0, c.P + bt.P0,
                      bt.ne, A.val, B.rp, B.col, B.val, out_col, out_val, bt.npieces,
                      c.tiles + bt.tile0};
}

// ---------------------------------------------------------------- symbolic, heavy rows
// Symbolic pass of one batch the way Algorithm 3 lays it out: expand C-hat
// (columns only), then per level Histogram, ThreshPartition and Multisplit,
// and count distinct columns of every final chunk.
void symbolic_batch_multisplit(spgemm_plan p, BatchState& bt, const DevCSR& A, const DevCSR& B,
                               const int32_t* hrows, int64_t* cnt_row, int64_t* nat_cur,
                               int64_t* rp_cur, hipStream_t st) {
    Arena& ar = p->ar;
    const Params& q = p->prm;
    const int64_t R0 = bt.h1 - bt.h0;
    CscBufs c = csc_bufs(p);
    int32_t* buf0c = ar.get<int32_t>("buf0c", (size_t)p->maxN);
    {
        PhaseScope ps(p, 0, SPGEMM_PHASE_OUTER_PROD, st);
        expand(expand_args(p, bt, A, B, buf0c, nullptr), st);
        add_bytes(p, 0, SPGEMM_PHASE_OUTER_PROD, 4.0 * bt.N + 20.0 * bt.ne);
    }
    const bool dump = p->opt.debug_dump && p->batches.size() == 1;
    if (dump) debug_copy_chat(p, bt, c.crp + bt.crp0, buf0c, nullptr, hrows + bt.h0, st);
    if (q.nlevels == 0) {
        ChunkItems ci{};
        ci.hash_top_logS = q.hash_top_logS;
        ci.rp = c.crp + bt.crp0;
        ci.map = hrows + bt.h0;
        ci.bcol = buf0c;
        ci.cnt = cnt_row;
        ci.width = q.final_width;
        PhaseScope ps(p, 0, SPGEMM_PHASE_HEAVY_ACCUM, st);
        accumulate_chunks(ci, CB_DENSE, 0, R0, false, st);
        add_bytes(p, 0, SPGEMM_PHASE_HEAVY_ACCUM, 4.0 * bt.N);
        return;
    }
    int32_t* bufc[2] = {buf0c, ar.get<int32_t>("buf1c", (size_t)p->maxN)};
    const int64_t* rp_in = c.crp + bt.crp0;
    int64_t R = R0, total = bt.N;
    for (int l = 0; l < q.nlevels; ++l) {
        const bool last = (l == q.nlevels - 1);
        LevelState& S_l = bt.lv[l];
        S_l.R = R;
        S_l.total_in = total;
        S_l.nch = q.vchunks[l];
        S_l.shift = ilog2(q.width[l]);
        S_l.nnat = R * S_l.nch;
        S_l.nat_off = nat_cur[l];
        S_l.rp_off = rp_cur[l];
        if (S_l.nat_off + S_l.nnat > p->cap_nat[l]) throw std::logic_error("level capacity");
        int64_t* counts = lvarr<int64_t>(p, l, "_counts") + S_l.nat_off;
        int32_t* inv = lvarr<int32_t>(p, l, "_inv") + S_l.nat_off;
        int32_t* pos = lvarr<int32_t>(p, l, "_pos") + S_l.nat_off;
        int64_t* nnz_l = lvarr<int64_t>(p, l, "_nnz") + S_l.nat_off;
        int64_t* bins = ar.get<int64_t>("chunk_bins", CB_COUNT + 1);
        LevelGeom g{rp_in, R, total, S_l.shift, S_l.nch, q.tau};
        {
            PhaseScope ps(p, 0, SPGEMM_PHASE_HISTO, st);
            fill<int64_t>(counts, S_l.nnat, 0, st);
            histogram(g, bufc[l & 1], counts, ar, st);
            classify_chunks(counts, S_l.nnat, q.tau, last, inv, pos, bins, ar, st);
            add_bytes(p, 0, SPGEMM_PHASE_HISTO, 4.0 * total + 8.0 * (R + 1) + 8.0 * S_l.nnat);
        }
        int64_t* hb = d2h(p, bins, CB_COUNT + 1, st);
        for (int b = 0; b <= CB_COUNT; ++b) S_l.bins[b] = hb[b];
        S_l.npos = S_l.bins[CB_EMPTY];
        int64_t* rp = lvarr<int64_t>(p, l, "_rp", true) + S_l.rp_off;
        int64_t* cursor = ar.get<int64_t>("cursor", (size_t)p->cap_rp[l] + 1);
        {
            PhaseScope ps(p, 0, SPGEMM_PHASE_HISTO, st);
            reord_rowptr(counts, inv, S_l.npos, rp, ar, st);
            copy<int64_t>(cursor, rp, S_l.npos, st);
        }
        check_level_sizes(p, rp, S_l.npos, total, l, st);
        int32_t* out = bufc[(l + 1) & 1];
        {
            PhaseScope ps(p, 0, SPGEMM_PHASE_MULTISPLIT, st);
            multisplit(g, bufc[l & 1], nullptr, pos, cursor, out, nullptr, false, ar, st);
            add_bytes(p, 0, SPGEMM_PHASE_MULTISPLIT, 8.0 * total + 8.0 * (R + 1));
        }
        check_cursors(p, cursor, rp, S_l.npos, l, st);
        if (dump) debug_copy_level(p, l, S_l, rp, out, nullptr, inv, st);
        fill<int64_t>(nnz_l, S_l.nnat, 0, st);
        {
            ChunkItems ci{};
            ci.hash_top_logS = q.hash_top_logS;
            ci.rp = rp;
            ci.map = inv;
            ci.bcol = out;
            ci.cnt = nnz_l;
            ci.width = q.width[l];
            PhaseScope ps(p, 0, SPGEMM_PHASE_HEAVY_ACCUM, st);
            for (int b = CB_DENSE; b <= CB_H8192; ++b)
                accumulate_chunks(ci, b, S_l.bins[b], S_l.bins[b + 1] - S_l.bins[b], false, st);
        }
        nat_cur[l] += S_l.nnat;
        rp_cur[l] += S_l.npos + 1;
        bt.L = l + 1;
        const int64_t nheavy = S_l.nheavy();
        if (nheavy == 0) {
            S_l.final_elems = total;
            add_bytes(p, 0, SPGEMM_PHASE_HEAVY_ACCUM, 4.0 * total);
            break;
        }
        const int64_t elems_heavy = d2h(p, rp + nheavy, 1, st)[0];
        S_l.final_elems = total - elems_heavy;
        add_bytes(p, 0, SPGEMM_PHASE_HEAVY_ACCUM, 4.0 * S_l.final_elems);
        rp_in = rp;
        R = nheavy;
        total = elems_heavy;
    }
    // bottom-up: a heavy chunk's count is the sum of its sub-chunks' counts
    PhaseScope ps(p, 0, SPGEMM_PHASE_PREFIX_SUM, st);
    for (int l = bt.L - 2; l >= 0; --l) {
        const LevelState& a = bt.lv[l];
        const LevelState& c1 = bt.lv[l + 1];
        reduce_children(lvarr<int64_t>(p, l + 1, "_nnz") + c1.nat_off, c1.nch, a.nheavy(),
                        lvarr<int32_t>(p, l, "_inv") + a.nat_off,
                        lvarr<int64_t>(p, l, "_nnz") + a.nat_off, st);
    }
}

// Symbolic pass of one batch without C-hat: every level's chunk counts (the
// Histogram of Algorithm 3) and distinct counts (its Symbolic) are sums of
// the finest-slot counts of one bitmap pass per heavy row; ThreshPartition
// then orders each level's chunks exactly as the multisplit path would.
void symbolic_batch_fused(spgemm_plan p, BatchState& bt, const int64_t* elem_fin,
                          const int64_t* dist_fin, int64_t* nat_cur, int64_t* rp_cur,
                          hipStream_t st) {
    Arena& ar = p->ar;
    const Params& q = p->prm;
    const int64_t req = q.nchunks_required;
    const int64_t* elem = elem_fin + bt.h0 * req;
    const int64_t* dist = dist_fin + bt.h0 * req;
    const int64_t* parent_slot0 = nullptr;
    const int32_t* parent_inv = nullptr;
    int64_t R = bt.h1 - bt.h0, total = bt.N;
    int64_t slots_per_chunk = req;
    for (int l = 0; l < q.nlevels; ++l) {
        const bool last = (l == q.nlevels - 1);
        LevelState& S_l = bt.lv[l];
        S_l.R = R;
        S_l.total_in = total;
        S_l.nch = q.vchunks[l];
        S_l.shift = ilog2(q.width[l]);
        S_l.nnat = R * S_l.nch;
        S_l.nat_off = nat_cur[l];
        S_l.rp_off = rp_cur[l];
        if (S_l.nat_off + S_l.nnat > p->cap_nat[l]) throw std::logic_error("level capacity");
        slots_per_chunk /= S_l.nch;
        int64_t* counts = lvarr<int64_t>(p, l, "_counts") + S_l.nat_off;
        int64_t* nnz_l = lvarr<int64_t>(p, l, "_nnz") + S_l.nat_off;
        int64_t* slot0 = lvarr<int64_t>(p, l, "_slot0") + S_l.nat_off;
        int32_t* inv = lvarr<int32_t>(p, l, "_inv") + S_l.nat_off;
        int32_t* pos = lvarr<int32_t>(p, l, "_pos") + S_l.nat_off;
        int64_t* bins = ar.get<int64_t>("chunk_bins", CB_COUNT + 1);
        {
            PhaseScope ps(p, 0, SPGEMM_PHASE_HISTO, st);
            level_from_slots(parent_slot0, parent_inv, R, S_l.nch, (int)slots_per_chunk, req,
                             elem, dist, counts, nnz_l, slot0, st);
            classify_chunks(counts, S_l.nnat, q.tau, last, inv, pos, bins, ar, st);
        }
        int64_t* hb = d2h(p, bins, CB_COUNT + 1, st);
        for (int b = 0; b <= CB_COUNT; ++b) S_l.bins[b] = hb[b];
        S_l.npos = S_l.bins[CB_EMPTY];
        int64_t* rp = lvarr<int64_t>(p, l, "_rp", true) + S_l.rp_off;
        {
            PhaseScope ps(p, 0, SPGEMM_PHASE_HISTO, st);
            reord_rowptr(counts, inv, S_l.npos, rp, ar, st);
        }
        check_level_sizes(p, rp, S_l.npos, total, l, st);
        nat_cur[l] += S_l.nnat;
        rp_cur[l] += S_l.npos + 1;
        bt.L = l + 1;
        const int64_t nheavy = S_l.nheavy();
        if (nheavy == 0) {
            S_l.final_elems = total;
            break;
        }
        const int64_t elems_heavy = d2h(p, rp + nheavy, 1, st)[0];
        S_l.final_elems = total - elems_heavy;
        parent_slot0 = slot0;
        parent_inv = inv;
        R = nheavy;
        total = elems_heavy;
    }
}

// Chunk output offsets, top-down: level 0 from C.rowPtr of the heavy rows,
// every deeper level from its parent chunk's offset.
void heavy_offsets(spgemm_plan p, const int32_t* hrows, const int64_t* C_rp, hipStream_t st) {
    if (p->prm.nlevels == 0 || p->H == 0) return;
    PhaseScope ps(p, 0, SPGEMM_PHASE_PREFIX_SUM, st);
    child_offsets(lvarr<int64_t>(p, 0, "_nnz"), p->prm.vchunks[0], p->H, hrows, C_rp,
                  lvarr<int64_t>(p, 0, "_off"), st);
    // first column of every chunk, for levels whose columns are stored as
    // 16-bit offsets inside the chunk
    chunk_colbase(p->H, p->prm.vchunks[0], p->prm.width[0], nullptr, nullptr,
                  lvarr<int32_t>(p, 0, "_cb"), st);
    for (const BatchState& bt : p->batches) {
        for (int l = 0; l + 1 < bt.L; ++l) {
            const LevelState& a = bt.lv[l];
            const LevelState& c1 = bt.lv[l + 1];
            child_offsets(lvarr<int64_t>(p, l + 1, "_nnz") + c1.nat_off, c1.nch, a.nheavy(),
                          lvarr<int32_t>(p, l, "_inv") + a.nat_off,
                          lvarr<int64_t>(p, l, "_off") + a.nat_off,
                          lvarr<int64_t>(p, l + 1, "_off") + c1.nat_off, st);
            chunk_colbase(a.nheavy(), c1.nch, p->prm.width[l + 1],
                          lvarr<int32_t>(p, l, "_inv") + a.nat_off,
                          lvarr<int32_t>(p, l, "_cb") + a.nat_off,
                          lvarr<int32_t>(p, l + 1, "_cb") + c1.nat_off, st);
        }
    }
}

// ---------------------------------------------------------------- row statistics
// The structural statistics of the products the SparseDitto page uses as
// operator features (Section 3.1, Eqs. 5 and 6): p95 and coefficient of
// variation of u(i), the fractions F_h of rows with u(i) <= h for h = 512,
// 4K, 32K; gamma (sum u / nnz(C)) is set once nnz(C) is known.
static void row_statistics(spgemm_plan p, int64_t n, const int32_t* hist) {
    spgemm_stats& S = p->stats;
    double u2;
    memcpy(&u2, &p->host[23], sizeof(double));
    const double mean = n > 0 ? (double)S.sum_products / (double)n : 0.0;
    const double var = n > 0 ? u2 / (double)n - mean * mean : 0.0;
    S.u_cv = mean > 0 ? std::sqrt(var > 0 ? var : 0.0) / mean : 0.0;
    for (int k = 0; k < 3; ++k) S.f_u_le[k] = n > 0 ? (double)p->host[20 + k] / (double)n : 0.0;
    // p95: the upper end of the first bucket at which 95% of the rows are reached
    const int64_t need = (n * 95 + 99) / 100;
    int64_t run = 0;
    S.u_p95 = 0;
    for (int b = 0; b < kUHistBuckets && n > 0; ++b) {
        run += hist[b];
        if (run >= need) {
            if (b < 64) {
                S.u_p95 = b;
            } else {
                const int e = (b - 64) / 64 + 6, f = (b - 64) % 64;
                S.u_p95 = ((int64_t)(64 + f + 1) << (e - 6)) - 1;
            }
            break;
        }
    }
}

// ---------------------------------------------------------------- symbolic
int64_t symbolic_impl(spgemm_plan p, const DevCSR& A, const DevCSR& B, int64_t* C_rp,
                      hipStream_t st) {
    Arena& ar = p->ar;
    p->ready = false;
    p->dbg_valid = false;
    p->dbg_chat = false;
    p->evnext = 0;
    p->evs.clear();
    memset(&p->stats, 0, sizeof(p->stats));
    const Params q = get_params(p, B.m);
    p->prm = q;
    const int64_t n = A.n;

    int* vflag = ar.get<int>("vflag", 4);
    if (p->opt.validate_inputs) {
        PhaseScope ps(p, 0, SPGEMM_PHASE_VALIDATE, st);
        fill<int>(vflag, 1, 0, st);
        launch_validate(A, vflag, st);
        launch_validate(B, vflag, st);
    }
    if (p->opt.validate_inputs) {
        SG_HIP(hipMemcpyAsync(p->host, vflag, sizeof(int), hipMemcpyDeviceToHost, st));
        SG_HIP(hipStreamSynchronize(st));
        if (*(int*)p->host != 0) return -1;
    }

    int64_t* S = ar.get<int64_t>("S", (size_t)A.nnz + 1);
    {
        PhaseScope ps(p, 0, SPGEMM_PHASE_INTER_PROD_SIZE, st);
        entry_prefix(A, B, S, ar, st);
        add_bytes(p, 0, SPGEMM_PHASE_INTER_PROD_SIZE, 4.0 * A.nnz + 16.0 * A.nnz);
    }
    int32_t* rowlo = ar.get<int32_t>("rowlo", (size_t)n + 1);
    int32_t* rowperm = ar.get<int32_t>("rowperm", (size_t)n + 1);
    int64_t* rowbins = ar.get<int64_t>("rowbins", RB_COUNT + 1);
    int64_t* st4 = ar.get<int64_t>("stats4", kRowStats);
    int32_t* uhist = ar.get<int32_t>("uhist", kUHistBuckets);
    {
        PhaseScope ps(p, 0, SPGEMM_PHASE_BINNING, st);
        int32_t* bmin = ar.get<int32_t>("bmin", (size_t)B.n + 1);
        int32_t* bmax = ar.get<int32_t>("bmax", (size_t)B.n + 1);
        brow_minmax(B, bmin, bmax, st);
        classify_rows(A, S, bmin, bmax, q.tau, rowlo, rowperm, rowbins, st4, uhist, ar, st);
        add_bytes(p, 0, SPGEMM_PHASE_BINNING, 8.0 * (n + 1) + 8.0 * n + 4.0 * n);
    }
    // the Synchronize() after ThreshPartition in Algorithm 3: workspace is sized from these
    {
        SG_HIP(hipMemcpyAsync(p->host, rowbins, (RB_COUNT + 1) * sizeof(int64_t),
                              hipMemcpyDeviceToHost, st));
        SG_HIP(hipMemcpyAsync(p->host + 16, st4, 9 * sizeof(int64_t), hipMemcpyDeviceToHost, st));
        int32_t* hist = (int32_t*)(p->host + 64);
        SG_HIP(hipMemcpyAsync(hist, uhist, kUHistBuckets * sizeof(int32_t),
                              hipMemcpyDeviceToHost, st));
        SG_HIP(hipStreamSynchronize(st));
        for (int b = 0; b <= RB_COUNT; ++b) p->row_bins[b] = p->host[b];
        p->stats.sum_products = p->host[16];
        p->stats.max_products = p->host[17];
        p->stats.heavy_rows = p->host[18];
        p->stats.heavy_products = p->host[19];
        p->light_annz = p->host[24];
        row_statistics(p, n, hist);
    }
    p->H = p->row_bins[RB_HEAVY + 1] - p->row_bins[RB_HEAVY];
    p->Nh = p->stats.heavy_products;
    const int32_t* hrows = rowperm + p->row_bins[RB_HEAVY];

    int64_t* cnt_row = ar.get<int64_t>("cnt_row", (size_t)n + 1);
    fill<int64_t>(cnt_row, n, 0, st);

    // light rows (Algorithm 3, the light-row symbolic step)
    RowItems ri{};
    ri.A = A;
    ri.B = B;
    ri.S = S;
    ri.perm = rowperm;
    ri.rowlo = rowlo;
    ri.cnt = cnt_row;
    ri.hash_top_logS = q.hash_top_logS;
    {
        PhaseScope ps(p, 0, SPGEMM_PHASE_LIGHT_ACCUM, st);
        for (int b = RB_T8; b <= RB_H8192; ++b)
            accumulate_rows(ri, b, p->row_bins[b], p->row_bins[b + 1] - p->row_bins[b], false, st);
        // per light row: its A and C row pointers and bin entry (28 B); per A
        // entry: column and B row bounds (20 B); per product: its B column
        const int64_t nl = p->row_bins[RB_H8192 + 1] - p->row_bins[RB_T8];
        add_bytes(p, 0, SPGEMM_PHASE_LIGHT_ACCUM,
                  28.0 * nl + 20.0 * p->light_annz +
                      4.0 * (p->stats.sum_products - p->stats.heavy_products));
        sum_rows(rowperm + p->row_bins[RB_T8], nl, cnt_row, st4 + 9, st);
    }

    // heavy rows (Algorithm 3, the heavy-row branch), batch by batch
    p->L = 0;
    p->batches.clear();
    if (p->H > 0) {
        p->stats.chat_bytes = 12 * p->Nh + 8 * (p->H + 1);
        const int64_t req = q.nlevels == 0 ? 1 : q.nchunks_required;
        // the fused pass needs the row's bitmap in LDS and a per-B-row slot
        // histogram (B.nrows x slots int32) in HBM
        const bool fused_fits = heavy_symbolic_lds(q.ppow, req) <= (size_t)p->dev_lds &&
                                B.n * req <= (int64_t(1) << 28);
        p->fused_sym = p->opt.symbolic_mode == 1 || (p->opt.symbolic_mode == 0 && fused_fits);
        // the direct path needs the fused pass's per-slot counts, 16-bit
        // columns inside a slot and a dense window of one slot in LDS (of
        // at least one 32-bit bitmap word)
        const int64_t wfin_d = q.nlevels == 0 ? q.ppow : q.final_width;
        const bool direct_ok = p->fused_sym && wfin_d >= 32 && wfin_d <= 65536 &&
                               req <= kDirectMaxSlots &&
                               direct_window_lds(wfin_d) + 8192 <= (size_t)p->dev_lds &&
                               p->H * req < (int64_t(1) << 31) && B.nnz <= INT32_MAX;
        p->direct = direct_ok && (p->opt.numeric_mode == 3 ||
                                  (p->opt.numeric_mode == 0 && !p->opt.debug_dump));
        p->direct_req = (int)req;
        p->direct_W = wfin_d;
        p->fused_num = !p->direct && q.nlevels > 0 &&
                       (p->opt.numeric_mode == 1 || p->opt.numeric_mode == 3 ||
                        (p->opt.numeric_mode == 0 && !p->opt.debug_dump));
        // the masked CSC feeds the separate outer product only
        const bool need_csc = !(p->fused_num || p->direct) || !p->fused_sym;
        // C-hat's row pointers, the row batches and the capacities of the
        // per-batch arrays serve the paths that build C-hat-reord; the
        // direct path forms every (row, final chunk) item from A and the
        // split B in one pass, so it has one batch and none of these arrays
        int64_t* chat_rp = nullptr;
        if (p->direct) {
            BatchState b;
            b.h0 = 0;
            b.h1 = p->H;
            b.N = p->Nh;
            p->batches.push_back(b);
            p->maxN = 0;
        } else {
            chat_rp = ar.get<int64_t>("chat_rp", (size_t)p->H + 1);
            {
                PhaseScope ps(p, 0, SPGEMM_PHASE_CSR_TO_CSC, st);
                heavy_rowptr(A, S, hrows, p->H, chat_rp, ar, st);
            }
            plan_batches(p, chat_rp, st);
            plan_capacities(p, A);
        }
        if (p->fused_num || p->direct) {
            PhaseScope ps(p, 0, SPGEMM_PHASE_CSR_TO_CSC, st);
            fused_setup(A, B, S, hrows, p->H, ar.get<int64_t>("h_q0", (size_t)p->H),
                        ar.get<int64_t>("h_q1", (size_t)p->H), ar.get<int64_t>("h_s0", (size_t)p->H),
                        ar.get<int64_t>("ebo", (size_t)A.nnz + 1), st);
            add_bytes(p, 0, SPGEMM_PHASE_CSR_TO_CSC, 28.0 * p->H + 20.0 * A.nnz);
        }
        if (p->fused_sym && !fused_fits)
            throw OverflowError("fused symbolic pass needs more LDS than the device has");
        int64_t* elem_fin = nullptr;
        int64_t* dist_fin = nullptr;
        if (p->fused_sym) {
            const int64_t wfin = q.nlevels == 0 ? q.ppow : q.final_width;
            elem_fin = ar.get<int64_t>("elem_fin", (size_t)(p->H * req));
            dist_fin = ar.get<int64_t>("dist_fin", (size_t)(p->H * req));
            PhaseScope ps(p, 0, SPGEMM_PHASE_HISTO, st);
            int32_t* bslot = ar.get<int32_t>("bslot", (size_t)(B.n * req + 1));
            heavy_symbolic(A, B, S, hrows, p->H, p->Nh, p->stats.max_products, p->dev_cus,
                           p->dev_lds, q.ppow, wfin, bslot, elem_fin, dist_fin, ar, st);
            add_bytes(p, 0, SPGEMM_PHASE_HISTO, 4.0 * p->Nh + 16.0 * p->H * req);
        }
        if (p->direct) {
            // B partitioned into the final chunks (the column-range split
            // applied to B rather than to C-hat), and the items by class
            PhaseScope ps(p, 0, SPGEMM_PHASE_HISTO, st);
            int32_t* bslot = ar.get<int32_t>("bslot", (size_t)(B.n * req + 1));
            direct_split_b(B, bslot, (int)req, wfin_d,
                           ar.get<int32_t>("spos", (size_t)(B.n * req + 1)),
                           ar.get<uint32_t>("roc", (size_t)(B.n * ceil_div(req, 32) + 1)),
                           ar.get<int32_t>("bperm", (size_t)B.nnz + 1),
                           ar.get<uint16_t>("bcol16", (size_t)B.nnz + 1), ar, st);
            // class starts, totals and the runs' counts side by side, read
            // back with nnz(C)
            int64_t* bins = ar.get<int64_t>("dmeta", kDirMeta);
            entry_len_sq(S, A.nnz, (double*)(bins + kDirLenSq), st);
            // the work lists: dense items, the rank classes, and the items
            // of at most kRunMax products merged per row into runs
            direct_classify(elem_fin, p->H, (int)req, ilog2(wfin_d),
                            ar.get<int64_t>("h_q0", (size_t)p->H),
                            ar.get<int64_t>("h_q1", (size_t)p->H),
                            ar.get<int32_t>("ditems", (size_t)(p->H * req)),
                            ar.get<int64_t>("diq0", (size_t)(p->H * req)),
                            ar.get<int32_t>("dine", (size_t)(p->H * req)), bins,
                            ar.get<int64_t>("rhdr", (size_t)(p->H * req)),
                            ar.get<int64_t>("rq0", (size_t)(p->H * req)),
                            ar.get<int32_t>("rne", (size_t)(p->H * req)), bins + kDirRuns, ar, st);
            direct_totals(ar.get<int64_t>("h_q0", (size_t)p->H), ar.get<int64_t>("h_q1", (size_t)p->H),
                          p->H, (int)req, elem_fin, dist_fin, bins + kDirTot, ar, st);
            add_bytes(p, 0, SPGEMM_PHASE_HISTO, 20.0 * B.nnz + 4.0 * B.n * (req + 1) +
                                                    24.0 * p->H * req);
        }
        if (p->direct) {
            // the items are the final chunks: C-hat's row pointers and the
            // per-level chunk classes are not needed, and a heavy row's
            // count is the sum of its items' distinct columns
            p->L = q.nlevels;
            for (int l = 0; l < q.nlevels; ++l) p->stats.vchunks[l] = q.vchunks[l];
            PhaseScope ps(p, 0, SPGEMM_PHASE_PREFIX_SUM, st);
            reduce_children(dist_fin, (int)req, p->H, hrows, cnt_row, st);
        }
        CscBufs c{};
        if (!p->direct) c = csc_bufs(p);
        int64_t ent_cur = 0, P_cur = 0, tile_cur = 0, crp_cur = 0;
        int64_t nat_cur[kMaxLevels] = {}, rp_cur[kMaxLevels] = {};
        for (BatchState& bt : p->batches) {
            if (p->direct) break;
            const int64_t R0 = bt.h1 - bt.h0;
            {
                PhaseScope ps(p, 0, SPGEMM_PHASE_CSR_TO_CSC, st);
                bt.ent0 = ent_cur;
                bt.P0 = P_cur;
                bt.tile0 = tile_cur;
                bt.ne = 0;
                bt.npieces = 0;
                if (need_csc) {
                    bt.ne = masked_csr2csc(A, B, S, hrows + bt.h0, R0, chat_rp + bt.h0,
                                           bt.chat_base, c.ent_k + ent_cur, c.ent_q + ent_cur,
                                           c.ent_dest + ent_cur, p->cap_ent - ent_cur,
                                           c.P + P_cur, &bt.npieces, ar, st);
                    ent_cur += bt.ne;
                    P_cur += bt.ne + 1;
                    if (tile_cur + expand_tiles(bt.npieces) + 1 > p->cap_tiles)
                        throw std::logic_error("expand tile capacity");
                    expand_tile_starts(c.P + bt.P0, bt.ne, bt.npieces, c.tiles + bt.tile0, st);
                    tile_cur += expand_tiles(bt.npieces) + 1;
                    add_bytes(p, 0, SPGEMM_PHASE_CSR_TO_CSC, 36.0 * bt.ne);
                }
                bt.crp0 = crp_cur;
                rebase(chat_rp + bt.h0, R0 + 1, bt.chat_base, c.crp + bt.crp0, st);
                crp_cur += R0 + 1;
            }
            if (p->fused_sym) {
                if (q.nlevels > 0)
                    symbolic_batch_fused(p, bt, elem_fin, dist_fin, nat_cur, rp_cur, st);
            } else {
                symbolic_batch_multisplit(p, bt, A, B, hrows, cnt_row, nat_cur, rp_cur, st);
            }
            p->L = std::max(p->L, bt.L);
            for (int l = 0; l < bt.L; ++l) {
                const LevelState& S_l = bt.lv[l];
                p->stats.vchunks[l] = S_l.nch;
                p->stats.level_in_elems[l] += S_l.total_in;
                p->stats.level_heavy_chunks[l] += S_l.nheavy();
                p->stats.level_final_chunks[l] += S_l.bins[CB_EMPTY] - S_l.bins[CB_DENSE];
            }
        }
        // row counts of the heavy rows
        if (!p->direct) {
            PhaseScope ps(p, 0, SPGEMM_PHASE_PREFIX_SUM, st);
            if (q.nlevels == 0) {
                if (p->fused_sym) reduce_children(dist_fin, 1, p->H, hrows, cnt_row, st);
            } else {
                reduce_children(lvarr<int64_t>(p, 0, "_nnz"), q.vchunks[0], p->H, hrows, cnt_row,
                                st);
            }
        }
    }

    // C.rowPtr (Algorithm 3, the closing PrefixSum)
    {
        PhaseScope ps(p, 0, SPGEMM_PHASE_PREFIX_SUM, st);
        scan_exclusive(LoadI64{cnt_row}, n, C_rp, ar, st);
        add_bytes(p, 0, SPGEMM_PHASE_PREFIX_SUM, 16.0 * n);
    }
    int64_t nnz_c = 0;
    // the light rows' output entries, read back with nnz(C)
    SG_HIP(hipMemcpyAsync(p->host + 40, st4 + 9, sizeof(int64_t), hipMemcpyDeviceToHost, st));
    if (p->direct) {
        // nnz(C) and the direct path's class starts, totals and runs in one wait
        static_assert(1 + kDirMeta <= 40, "staging buffer");
        SG_HIP(hipMemcpyAsync(p->host + 1, ar.get<int64_t>("dmeta", kDirMeta),
                              kDirMeta * sizeof(int64_t), hipMemcpyDeviceToHost, st));
        const int64_t* h = d2h(p, C_rp + n, 1, st);
        nnz_c = h[0];
        for (int b = 0; b <= DC_COUNT; ++b) p->dir_bins[b] = h[1 + b];
        for (int i = 0; i < 8; ++i) p->dir_tot[i] = h[1 + kDirTot + i];
        for (int i = 0; i < 3; ++i) p->dir_runs[i] = h[1 + kDirRuns + i];
        double len_sq;
        memcpy(&len_sq, &h[1 + kDirLenSq], sizeof(double));
        // the mean B-row length a product sees, against the slots per row
        const double seen = p->stats.sum_products > 0 ? len_sq / (double)p->stats.sum_products : 0.0;
        p->direct_occ = seen * kOccSparse < (double)p->direct_req;
        if (p->H > 0) {
            // the runs test the bits always; the other items when most of
            // their slices are empty
            PhaseScope ps(p, 0, SPGEMM_PHASE_HISTO, st);
            const int64_t req = p->direct_req;
            direct_entry_occ(A.col, A.nnz, (int)req,
                             ar.get<uint32_t>("roc", (size_t)(B.n * ceil_div(req, 32) + 1)),
                             ar.get<uint32_t>("eocc", (size_t)(ceil_div(req, 32) * A.nnz + 1)), st);
            add_bytes(p, 0, SPGEMM_PHASE_HISTO, (4.0 + 8.0 * ceil_div(req, 32)) * A.nnz);
        }
    } else {
        nnz_c = d2h(p, C_rp + n, 1, st)[0];
    }
    if (!p->direct) heavy_offsets(p, hrows, C_rp, st);
    if (p->direct) {
        PhaseScope ps(p, 0, SPGEMM_PHASE_PREFIX_SUM, st);
        direct_offsets(C_rp, hrows, p->H, p->direct_req,
                       ar.get<int64_t>("dist_fin", (size_t)(p->H * p->direct_req)),
                       ar.get<int64_t>("doff", (size_t)(p->H * p->direct_req)), st);
    }
    p->light_cnnz = p->host[40];
    p->stats.numeric_path = p->H == 0 ? 0 : (p->direct ? 3 : (p->fused_num ? 1 : 2));
    p->stats.nrows = n;
    p->stats.ncols_c = B.m;
    p->stats.nnz_c = nnz_c;
    p->stats.tau = q.tau;
    p->stats.final_chunk_width = q.final_width;
    p->stats.nlevels = p->L;
    p->stats.nbatches = (int32_t)p->batches.size();
    p->stats.lds_bytes = q.slm;
    p->stats.light_rows = p->row_bins[RB_EMPTY] - p->row_bins[RB_T8];
    p->stats.light_products = p->stats.sum_products - p->stats.heavy_products;
    p->stats.gamma = nnz_c > 0 ? (double)p->stats.sum_products / (double)nnz_c : 0.0;
    return nnz_c;
}

// ---------------------------------------------------------------- numeric
void numeric_impl(spgemm_plan p, const DevCSR& A, const DevCSR& B, const int64_t* C_rp,
                  int32_t* C_col, double* C_val, hipStream_t st) {
    Arena& ar = p->ar;
    const Params& q = p->prm;
    const int64_t n = A.n;
    // drop the numeric events of an earlier numeric call after this symbolic
    {
        std::vector<spgemm_plan_s::Ev> keep;
        for (auto& e : p->evs)
            if (e.pass == 0) keep.push_back(e);
        p->evs.swap(keep);
        for (int ph = 0; ph < SPGEMM_NUM_PHASES; ++ph) p->stats.phase_bytes[1][ph] = 0;
    }
    int64_t* S = ar.get<int64_t>("S", (size_t)A.nnz + 1);
    int32_t* rowlo = ar.get<int32_t>("rowlo", (size_t)n + 1);
    int32_t* rowperm = ar.get<int32_t>("rowperm", (size_t)n + 1);
    const int32_t* hrows = rowperm + p->row_bins[RB_HEAVY];

    RowItems ri{};
    ri.A = A;
    ri.B = B;
    ri.S = S;
    ri.perm = rowperm;
    ri.rowlo = rowlo;
    ri.hash_top_logS = q.hash_top_logS;
    ri.Crp = C_rp;
    ri.Ccol = C_col;
    ri.Cval = C_val;
    // light rows on the plan's second stream when there are heavy rows to
    // overlap with; the caller's stream waits for them on every way out
    const bool fork = p->lst != nullptr && p->H > 0 && p->row_bins[RB_H8192 + 1] > p->row_bins[RB_T8];
    // Armed as soon as the side stream has forked: whatever was queued on
    // it, also when a later launch throws, is waited for by the caller's
    // stream when this function returns.
    struct Join {
        bool on;
        hipStream_t st, side;
        hipEvent_t ev;
        ~Join() {
            if (on && hipEventRecord(ev, side) == hipSuccess) (void)hipStreamWaitEvent(st, ev, 0);
        }
    } join{false, st, p->lst, p->ev_join};
    const hipStream_t lst = fork ? p->lst : st;
    // The light rows start beside the direct path's items at once. Beside
    // the page's dataflow they start with its first accumulation, so that
    // they share the GPU with the latency-bound accumulators rather than
    // with the outer product and multisplit, which stream at HBM speed.
    bool light_queued = false;
    auto queue_light = [&]() {
        if (light_queued) return;
        light_queued = true;
        if (fork) {
            SG_HIP(hipEventRecord(p->ev_fork, st));
            SG_HIP(hipStreamWaitEvent(p->lst, p->ev_fork, 0));
            join.on = true;
        }
        PhaseScope ps(p, 1, SPGEMM_PHASE_LIGHT_ACCUM, lst);
        for (int b = RB_T8; b <= RB_H8192; ++b)
            accumulate_rows(ri, b, p->row_bins[b], p->row_bins[b + 1] - p->row_bins[b], true, lst);
        // per light row: A and C row pointers and bin entry (28 B); per A
        // entry: column, value and B row bounds (28 B); per product: its B
        // column and value (12 B); per output entry: column and value (12 B)
        const int64_t nl = p->row_bins[RB_H8192 + 1] - p->row_bins[RB_T8];
        add_bytes(p, 1, SPGEMM_PHASE_LIGHT_ACCUM,
                  28.0 * nl + 28.0 * p->light_annz + 12.0 * p->stats.light_products +
                      12.0 * p->light_cnnz);
    };
    if (p->H == 0 || p->direct) queue_light();
    if (p->H == 0) return;

    if (p->direct) {
        const int req = p->direct_req;
        double* bpval = ar.get<double>("bpval", (size_t)B.nnz + 1);
        DirectArgs d{};
        d.items = ar.get<int32_t>("ditems", (size_t)(p->H * req));
        d.req = req;
        d.logW = ilog2(p->direct_W);
        d.hq0 = ar.get<int64_t>("h_q0", (size_t)p->H);
        d.hq1 = ar.get<int64_t>("h_q1", (size_t)p->H);
        d.iq0 = ar.get<int64_t>("diq0", (size_t)(p->H * req));
        d.ine = ar.get<int32_t>("dine", (size_t)(p->H * req));
        d.Acol = A.col;
        d.Aval = A.val;
        d.spos = ar.get<int32_t>("spos", (size_t)(B.n * req + 1));
        d.nb = B.n;
        d.annz = A.nnz;
        d.eocc = ar.get<uint32_t>("eocc", (size_t)(ceil_div(req, 32) * A.nnz + 1));
        d.occ = p->direct_occ;
        d.bcol16 = ar.get<uint16_t>("bcol16", (size_t)B.nnz + 1);
        d.bval = bpval;
        d.off = ar.get<int64_t>("doff", (size_t)(p->H * req));
        d.Ccol = C_col;
        d.Cval = C_val;
        d.rhdr = ar.get<int64_t>("rhdr", (size_t)(p->H * req));
        d.rq0 = ar.get<int64_t>("rq0", (size_t)(p->H * req));
        d.rne = ar.get<int32_t>("rne", (size_t)(p->H * req));
        // Bytes per class: every product's B operand (16-bit column and
        // value, read once), every output entry written once (12 B), and
        // each item's reads of its row's entries (column and value, 12 B)
        // with their slice bounds (two 32-bit starts, 8 B).
        {
            PhaseScope ps(p, 1, SPGEMM_PHASE_DIRECT_RANK, st);
            // B's values in the split order (values may change between
            // numeric calls; the structure may not)
            direct_gather_values(ar.get<int32_t>("bperm", (size_t)B.nnz + 1), B.val, B.nnz, bpval,
                                 st);
            // the smallest classes are taken by the runs
            direct_accumulate_runs(d, p->dir_runs[0], st);
            for (int b = DC_RANK0 + kRunClasses; b < DC_EMPTY; ++b)
                direct_accumulate(d, b, p->dir_bins[b], p->dir_bins[b + 1] - p->dir_bins[b], st);
            // the gather of B's values: its placement map (4 B), a value read
            // and written (16 B) per B entry. Runs read their row's entries
            // (12 B) and an occupancy word per (entry, slot) pair (4 B); the
            // bounds of the nonempty slices they then read are not counted.
            add_bytes(p, 1, SPGEMM_PHASE_DIRECT_RANK,
                      20.0 * B.nnz + 10.0 * (p->dir_tot[3] + p->dir_tot[6]) +
                          12.0 * (p->dir_tot[4] + p->dir_tot[7]) + 20.0 * p->dir_tot[5] +
                          12.0 * p->dir_runs[1] + 4.0 * p->dir_runs[2]);
        }
        {
            PhaseScope ps(p, 1, SPGEMM_PHASE_DIRECT_DENSE, st);
            direct_accumulate(d, DC_DENSE, p->dir_bins[DC_DENSE],
                              p->dir_bins[DC_DENSE + 1] - p->dir_bins[DC_DENSE], st);
            add_bytes(p, 1, SPGEMM_PHASE_DIRECT_DENSE,
                      10.0 * p->dir_tot[0] + 12.0 * p->dir_tot[1] + 20.0 * p->dir_tot[2]);
        }
        return;
    }

    CscBufs c = csc_bufs(p);
    // C-hat (buffer 0) is written only by the separate outer product; with
    // the fused first level, buffer 0 holds level 1's output if there is one
    int32_t* bufc[2] = {nullptr, nullptr};
    double* bufv[2] = {nullptr, nullptr};
    if (!p->fused_num || p->L > 1) {
        bufc[0] = ar.get<int32_t>("buf0c", (size_t)p->maxN);
        bufv[0] = ar.get<double>("buf0v", (size_t)p->maxN);
    }
    if (q.nlevels > 0) {
        bufc[1] = ar.get<int32_t>("buf1c", (size_t)p->maxN);
        bufv[1] = ar.get<double>("buf1v", (size_t)p->maxN);
    }
    const bool dump = p->opt.debug_dump && p->batches.size() == 1;
    for (const BatchState& bt : p->batches) {
        const int64_t R0 = bt.h1 - bt.h0;
        if (!p->fused_num) {
            {
                PhaseScope ps(p, 1, SPGEMM_PHASE_OUTER_PROD, st);
                expand(expand_args(p, bt, A, B, bufc[0], bufv[0]), st);
                add_bytes(p, 1, SPGEMM_PHASE_OUTER_PROD, 12.0 * bt.N + 28.0 * bt.ne);
            }
            if (dump) debug_copy_chat(p, bt, c.crp + bt.crp0, bufc[0], bufv[0], hrows + bt.h0, st);
        }
        if (q.nlevels == 0) {
            ChunkItems ci{};
            ci.hash_top_logS = q.hash_top_logS;
            ci.rp = c.crp + bt.crp0;
            ci.map = hrows + bt.h0;
            ci.bcol = bufc[0];
            ci.bval = bufv[0];
            ci.off = C_rp;
            ci.Ccol = C_col;
            ci.Cval = C_val;
            ci.width = q.final_width;
            queue_light();
            PhaseScope ps(p, 1, SPGEMM_PHASE_HEAVY_ACCUM, st);
            accumulate_chunks(ci, CB_DENSE, 0, R0, true, st);
            add_bytes(p, 1, SPGEMM_PHASE_HEAVY_ACCUM, 12.0 * bt.N);
            continue;
        }
        const int64_t* rp_in = c.crp + bt.crp0;
        for (int l = 0; l < bt.L; ++l) {
            const LevelState& S_l = bt.lv[l];
            int32_t* inv = lvarr<int32_t>(p, l, "_inv") + S_l.nat_off;
            int32_t* pos = lvarr<int32_t>(p, l, "_pos") + S_l.nat_off;
            int64_t* off = lvarr<int64_t>(p, l, "_off") + S_l.nat_off;
            int64_t* rp = lvarr<int64_t>(p, l, "_rp", true) + S_l.rp_off;
            int64_t* cursor = ar.get<int64_t>("cursor", (size_t)p->cap_rp[l] + 1);
            copy<int64_t>(cursor, rp, S_l.npos, st);
            LevelGeom g{rp_in, S_l.R, S_l.total_in, S_l.shift, S_l.nch, q.tau};
            const int in = l & 1, outb = (l + 1) & 1;
            // A level with no chunk for a further level feeds only the
            // accumulators: its columns go out as 16-bit offsets in the chunk.
            const bool c16 = !dump && S_l.nheavy() == 0 && q.width[l] <= (int64_t(1) << 16);
            {
                PhaseScope ps(p, 1, SPGEMM_PHASE_MULTISPLIT, st);
                if (l == 0 && p->fused_num) {
                    // products formed in the tile: the Ĉreord write, one read
                    // of the B rows and the row pointers are the minimum
                    FusedRows fr{ar.get<int64_t>("h_q0", (size_t)p->H) + bt.h0,
                                 ar.get<int64_t>("h_q1", (size_t)p->H) + bt.h0,
                                 ar.get<int64_t>("h_s0", (size_t)p->H) + bt.h0,
                                 ar.get<int64_t>("ebo", (size_t)A.nnz + 1)};
                    expand_multisplit(g, fr, A, B, S, pos, cursor, bufc[outb], bufv[outb], c16,
                                      ar, st);
                    add_bytes(p, 1, SPGEMM_PHASE_MULTISPLIT,
                              (c16 ? 10.0 : 12.0) * S_l.total_in + 12.0 * B.nnz +
                                  8.0 * (S_l.R + 1));
                } else {
                    multisplit(g, bufc[in], bufv[in], pos, cursor, bufc[outb], bufv[outb], c16,
                               ar, st);
                    add_bytes(p, 1, SPGEMM_PHASE_MULTISPLIT,
                              (c16 ? 22.0 : 24.0) * S_l.total_in + 8.0 * (S_l.R + 1));
                }
            }
            check_cursors(p, cursor, rp, S_l.npos, l, st);
            if (dump) debug_copy_level(p, l, S_l, rp, bufc[outb], bufv[outb], inv, st);
            {
                ChunkItems ci{};
                ci.hash_top_logS = q.hash_top_logS;
                ci.rp = rp;
                ci.map = inv;
                ci.bcol = bufc[outb];
                if (c16) {
                    ci.bcol16 = (const uint16_t*)bufc[outb];
                    ci.colbase = lvarr<int32_t>(p, l, "_cb") + S_l.nat_off;
                }
                ci.bval = bufv[outb];
                ci.off = off;
                ci.Ccol = C_col;
                ci.Cval = C_val;
                ci.width = q.width[l];
                queue_light();
                PhaseScope ps(p, 1, SPGEMM_PHASE_HEAVY_ACCUM, st);
                for (int b = CB_DENSE; b <= CB_H8192; ++b)
                    accumulate_chunks(ci, b, S_l.bins[b], S_l.bins[b + 1] - S_l.bins[b], true, st);
                add_bytes(p, 1, SPGEMM_PHASE_HEAVY_ACCUM, (c16 ? 10.0 : 12.0) * S_l.final_elems);
            }
            rp_in = rp;
        }
    }
    queue_light();
    // every heavy row's output entries, written once by the accumulators
    // (column and value, 12 B)
    add_bytes(p, 1, SPGEMM_PHASE_HEAVY_ACCUM, 12.0 * (p->stats.nnz_c - p->light_cnnz));
}

template <class F>
int guarded(F&& f) {
    try {
        return f();
    } catch (const OomError&) {
        return SPGEMM_ERR_OUT_OF_MEMORY;
    } catch (const OverflowError&) {
        return SPGEMM_ERR_OVERFLOW;
    } catch (const ScratchError&) {
        return SPGEMM_ERR_SCRATCH_LIMIT;
    } catch (const InternalError&) {
        return SPGEMM_ERR_INTERNAL;
    } catch (const HipError& e) {
        if (e.code == hipErrorOutOfMemory) return SPGEMM_ERR_OUT_OF_MEMORY;
        return SPGEMM_ERR_HIP;
    } catch (const std::bad_alloc&) {
        return SPGEMM_ERR_OUT_OF_MEMORY;
    } catch (...) {
        return SPGEMM_ERR_HIP;
    }
}

// After OUT_OF_MEMORY the plan gives back all of its workspace (hipFree
// waits for the device, so no queued kernel still uses it) and needs a new
// symbolic call: the caller can free memory of its own and retry.
int release_on_oom(spgemm_plan p, int rc) {
    if (rc == SPGEMM_ERR_OUT_OF_MEMORY) {
        p->ready = false;
        p->dbg_valid = false;
        p->ar.release();
    }
    return rc;
}

bool options_valid(const spgemm_options& o) {
    if (o.lds_budget_bytes < 0 || o.tau_override < 0 || o.chunk_width_override < 0 ||
        o.nchunks_cap < 0 || o.max_batch_products < 0 || o.workspace_limit_bytes < 0)
        return false;
    if (o.symbolic_mode < 0 || o.symbolic_mode > 2 || o.numeric_mode < 0 || o.numeric_mode > 3)
        return false;
    if (o.chunk_width_override > 0 &&
        (o.chunk_width_override < 32 || (o.chunk_width_override & (o.chunk_width_override - 1))))
        return false;
    if (o.nchunks_cap > 0 && (o.nchunks_cap < 2 || (o.nchunks_cap & (o.nchunks_cap - 1))))
        return false;
    return true;
}

// ---------------------------------------------------------------- allocation-free calls
// The device scratch of spgemm_multiply_noalloc. In host code this name is
// only a stand-in for the symbol: its device address, which differs per
// device, comes from hipGetSymbolAddress once per device and is the only
// form host code passes on.
static __device__ __align__(256) unsigned char scratch[SPGEMM_NOALLOC_SCRATCH_BYTES];

constexpr int kNoallocDevices = 64;

// Per device: the scratch address and the plan state that lives on it.
struct NoallocDevice {
    std::mutex mu;            // one host thread at a time in a device's call
    bool ready = false;
    void* ptr = nullptr;      // device address of `scratch` on this device
    spgemm_plan_s plan;       // its arena carves buffers out of ptr
    int64_t host[kHostWords]; // staging for the plan's small device-to-host reads
};

NoallocDevice g_noalloc[kNoallocDevices];

// Set-up on the first call on the current device: the scratch address (with
// the device current) and the plan's device properties; no stream, event or
// memory is created.
int noalloc_setup(NoallocDevice& d, int device) {
    if (d.ready) return SPGEMM_OK;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
        (void)hipGetLastError();
        return SPGEMM_ERR_HIP;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return SPGEMM_ERR_HIP;
    d.ptr = ptr;
    spgemm_plan_s& p = d.plan;
    p.device = device;
    p.dev_lds = (int64_t)prop.sharedMemPerBlock;
    p.dev_cus = std::max(1, prop.multiProcessorCount);
    p.host = d.host;
    p.lst = nullptr;  // the light rows run on the caller's stream
    p.ar.use_region(d.ptr, (size_t)SPGEMM_NOALLOC_SCRATCH_BYTES);
    d.ready = true;
    return SPGEMM_OK;
}

}  // namespace

// ============================================================================
// C ABI
// ============================================================================
extern "C" {

SPGEMM_API void spgemm_options_default(spgemm_options* opt) {
    if (!opt) return;
    memset(opt, 0, sizeof(*opt));
    opt->validate_inputs = 1;
}

SPGEMM_API int spgemm_plan_create(spgemm_plan* out, const spgemm_options* opt) {
    if (!out) return SPGEMM_ERR_INVALID_ARG;
    *out = nullptr;
    spgemm_options o;
    spgemm_options_default(&o);
    if (opt) o = *opt;
    if (!options_valid(o)) return SPGEMM_ERR_INVALID_ARG;
    return guarded([&]() -> int {
        auto* p = new spgemm_plan_s();
        p->opt = o;
        p->ar.set_limit((size_t)o.workspace_limit_bytes);
        p->ar.set_poison(o.debug_dump != 0);
        if (hipGetDevice(&p->device) != hipSuccess) {
            delete p;
            return SPGEMM_ERR_HIP;
        }
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, p->device) != hipSuccess) {
            delete p;
            return SPGEMM_ERR_HIP;
        }
        p->dev_lds = (int64_t)prop.sharedMemPerBlock;
        p->dev_cus = std::max(1, prop.multiProcessorCount);
        if (hipHostMalloc((void**)&p->host, kHostWords * sizeof(int64_t), hipHostMallocDefault) !=
            hipSuccess) {
            delete p;
            return SPGEMM_ERR_HIP;
        }
        if (hipStreamCreateWithFlags(&p->lst, hipStreamNonBlocking) != hipSuccess ||
            hipEventCreateWithFlags(&p->ev_fork, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&p->ev_join, hipEventDisableTiming) != hipSuccess) {
            spgemm_plan_destroy(p);
            return SPGEMM_ERR_HIP;
        }
        *out = p;
        return SPGEMM_OK;
    });
}

SPGEMM_API void spgemm_plan_destroy(spgemm_plan p) {
    if (!p) return;
    (void)hipDeviceSynchronize();
    for (auto e : p->evpool) (void)hipEventDestroy(e);
    if (p->ev_fork) (void)hipEventDestroy(p->ev_fork);
    if (p->ev_join) (void)hipEventDestroy(p->ev_join);
    if (p->lst) (void)hipStreamDestroy(p->lst);
    if (p->host) (void)hipHostFree(p->host);
    p->ar.release();
    delete p;
}

SPGEMM_API int spgemm_symbolic(spgemm_plan p, const spgemm_csr* A, const spgemm_csr* B,
                               int64_t* C_rowptr, int64_t* C_nnz, void* stream) {
    if (!p || !C_rowptr || !C_nnz) return SPGEMM_ERR_INVALID_ARG;
    int rc = check_csr(A, false);
    if (rc) return rc;
    rc = check_csr(B, false);
    if (rc) return rc;
    if (A->ncols != B->nrows) return SPGEMM_ERR_DIM_MISMATCH;
    p->ready = false;
    hipStream_t st = (hipStream_t)stream;
    return release_on_oom(p, guarded([&]() -> int {
        int64_t nnz = symbolic_impl(p, to_dev(A), to_dev(B), C_rowptr, st);
        if (nnz < 0) return SPGEMM_ERR_INDEX_RANGE;
        *C_nnz = nnz;
        p->An = A->nrows;
        p->Am = A->ncols;
        p->Annz = A->nnz;
        p->Bn = B->nrows;
        p->Bm = B->ncols;
        p->Bnnz = B->nnz;
        p->Cnnz = nnz;
        p->ready = true;
        return SPGEMM_OK;
    }));
}

SPGEMM_API int spgemm_numeric(spgemm_plan p, const spgemm_csr* A, const spgemm_csr* B,
                              const int64_t* C_rowptr, int32_t* C_col, double* C_val,
                              void* stream) {
    if (!p || !C_rowptr) return SPGEMM_ERR_INVALID_ARG;
    int rc = check_csr(A, true);
    if (rc) return rc;
    rc = check_csr(B, true);
    if (rc) return rc;
    if (!p->ready) return SPGEMM_ERR_NOT_READY;
    if (A->nrows != p->An || A->ncols != p->Am || A->nnz != p->Annz || B->nrows != p->Bn ||
        B->ncols != p->Bm || B->nnz != p->Bnnz)
        return SPGEMM_ERR_PLAN_MISMATCH;
    if (p->Cnnz > 0 && (!C_col || !C_val)) return SPGEMM_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    return release_on_oom(p, guarded([&]() -> int {
        numeric_impl(p, to_dev(A), to_dev(B), C_rowptr, C_col, C_val, st);
        return SPGEMM_OK;
    }));
}

SPGEMM_API int spgemm_multiply(spgemm_plan p, const spgemm_csr* A, const spgemm_csr* B,
                               int64_t* C_rowptr, int32_t* C_col, double* C_val,
                               int64_t capacity, int64_t* C_nnz, void* stream) {
    if (!p || !C_nnz || capacity < 0) return SPGEMM_ERR_INVALID_ARG;
    int rc = spgemm_symbolic(p, A, B, C_rowptr, C_nnz, stream);
    if (rc != SPGEMM_OK) return rc;
    if (*C_nnz > capacity) return SPGEMM_ERR_CAPACITY;
    return spgemm_numeric(p, A, B, C_rowptr, C_col, C_val, stream);
}

SPGEMM_API int spgemm_multiply_noalloc(const spgemm_options* opt, const spgemm_csr* A,
                                       const spgemm_csr* B, int64_t* C_rowptr, int32_t* C_col,
                                       double* C_val, int64_t capacity, int64_t* C_nnz,
                                       void* stream) {
    if (!C_rowptr || !C_nnz || capacity < 0) return SPGEMM_ERR_INVALID_ARG;
    spgemm_options o;
    spgemm_options_default(&o);
    if (opt) o = *opt;
    if (!options_valid(o) || o.timing || o.debug_dump) return SPGEMM_ERR_INVALID_ARG;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return SPGEMM_ERR_HIP;
    if (device < 0 || device >= kNoallocDevices) return SPGEMM_ERR_HIP;
    NoallocDevice& d = g_noalloc[device];
    std::lock_guard<std::mutex> lock(d.mu);
    int rc = noalloc_setup(d, device);
    if (rc != SPGEMM_OK) return rc;
    spgemm_plan p = &d.plan;
    p->opt = o;
    p->opt.workspace_limit_bytes = 0;
    p->ready = false;
    p->ar.release();  // a fresh layout inside the scratch for this call
    return spgemm_multiply(p, A, B, C_rowptr, C_col, C_val, capacity, C_nnz, stream);
}

SPGEMM_API int spgemm_plan_stats(spgemm_plan p, spgemm_stats* out) {
    if (!p || !out) return SPGEMM_ERR_INVALID_ARG;
    return guarded([&]() -> int {
        spgemm_stats s = p->stats;
        for (int pass = 0; pass < 2; ++pass)
            for (int ph = 0; ph < SPGEMM_NUM_PHASES; ++ph) {
                s.phase_ms[pass][ph] = 0;
                s.phase_launches[pass][ph] = 0;
            }
        for (auto& e : p->evs) {
            SG_HIP(hipEventSynchronize(e.b));
            float ms = 0;
            SG_HIP(hipEventElapsedTime(&ms, e.a, e.b));
            s.phase_ms[e.pass][e.phase] += ms;
            s.phase_launches[e.pass][e.phase] += 1;
        }
        *out = s;
        return SPGEMM_OK;
    });
}

SPGEMM_API int spgemm_plan_debug(spgemm_plan p, int which, spgemm_debug_matrix* out) {
    if (!p || !out || !p->opt.debug_dump || !p->dbg_valid || p->batches.size() != 1)
        return SPGEMM_ERR_INVALID_ARG;
    return guarded([&]() -> int {
        Arena& ar = p->ar;
        const BatchState& bt = p->batches[0];
        memset(out, 0, sizeof(*out));
        if (which == -1) {
            if (!p->dbg_chat) return SPGEMM_ERR_INVALID_ARG;
            const int64_t R = bt.h1 - bt.h0;
            out->nrows = R;
            out->nnz = bt.N;
            out->rowptr = ar.get<int64_t>("dbg_m1_rp", (size_t)R + 1);
            out->col = ar.get<int32_t>("dbg_m1_col", (size_t)bt.N);
            out->val = p->dbg_chat_val ? ar.get<double>("dbg_m1_val", (size_t)bt.N) : nullptr;
            out->row_key = ar.get<int64_t>("dbg_m1_key", (size_t)R + 1);
            out->chunk_width = p->prm.ppow;
            return SPGEMM_OK;
        }
        if (which < 0 || which >= bt.L) return SPGEMM_ERR_INVALID_ARG;
        const LevelState& S_l = bt.lv[which];
        std::string b = "dbg_l" + std::to_string(which);
        SG_HIP(hipDeviceSynchronize());
        int64_t* rp = ar.get<int64_t>(b + "_rp", (size_t)S_l.npos + 1);
        int64_t nnz = 0;
        SG_HIP(hipMemcpy(&nnz, rp + S_l.npos, sizeof(int64_t), hipMemcpyDeviceToHost));
        out->nrows = S_l.npos;
        out->nnz = nnz;
        out->rowptr = rp;
        out->col = ar.get<int32_t>(b + "_col", (size_t)nnz);
        out->val = p->dbg_has_val ? ar.get<double>(b + "_val", (size_t)nnz) : nullptr;
        out->row_key = ar.get<int64_t>(b + "_key", (size_t)S_l.npos + 1);
        out->chunk_width = p->prm.width[which];
        return SPGEMM_OK;
    });
}

SPGEMM_API const char* spgemm_status_string(int status) {
    switch (status) {
        case SPGEMM_OK: return "success";
        case SPGEMM_ERR_INVALID_ARG: return "invalid argument";
        case SPGEMM_ERR_DIM_MISMATCH: return "inner dimensions differ (A.ncols != B.nrows)";
        case SPGEMM_ERR_INDEX_RANGE: return "row pointer or column index out of range";
        case SPGEMM_ERR_OVERFLOW: return "size exceeds a supported limit";
        case SPGEMM_ERR_OUT_OF_MEMORY: return "device memory exhausted";
        case SPGEMM_ERR_PLAN_MISMATCH: return "numeric call does not match the symbolic call";
        case SPGEMM_ERR_HIP: return "HIP runtime error";
        case SPGEMM_ERR_NOT_READY: return "numeric called before a successful symbolic";
        case SPGEMM_ERR_CAPACITY: return "C has more entries than the room given";
        case SPGEMM_ERR_SCRATCH_LIMIT:
            return "product needs more workspace than the fixed scratch buffer holds";
        case SPGEMM_ERR_INTERNAL: return "internal self-check failed (debug plan)";
        default: return "unknown status";
    }
}

}  // extern "C"
