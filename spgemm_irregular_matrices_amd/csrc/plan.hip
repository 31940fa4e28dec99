// Host orchestration and the C ABI (include/spgemm.h).
//
// spgemm_symbolic runs Algorithm 3 of the gMAGNUS page up to the prefix sum
// of C.rowPtr (lines 1-25) with columns only; spgemm_numeric reruns the
// heavy path with values and accumulates (lines 26-27). The structure the
// symbolic pass finds (row bins, C-hat and C-hat-reord row pointers, chunk
// partitions and chunk output offsets) is kept in the plan, so the numeric
// pass does no histogramming, partitioning or blocking host reads.
#include <string.h>

#include <algorithm>
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

struct LevelState {
    int64_t R = 0;         // input rows (C-hat rows or the previous level's heavy chunks)
    int64_t total_in = 0;  // input elements
    int nch = 0;
    int shift = 0;
    int64_t nnat = 0;      // R * nch
    int64_t npos = 0;      // nonempty chunks
    int64_t bins[CB_COUNT + 1] = {};
    int in_buf = 0;        // which double buffer holds the input
    int64_t final_elems = 0;  // elements of this level's accumulated (non-split) chunks
};

}  // namespace

struct spgemm_plan_s {
    spgemm_options opt{};
    Arena ar;
    int device = 0;
    int64_t dev_lds = 0;
    int64_t* host = nullptr;  // pinned staging for small device-to-host reads
    // state of the last successful symbolic call
    bool ready = false;
    int64_t An = 0, Am = 0, Annz = 0, Bn = 0, Bm = 0, Bnnz = 0, Cnnz = 0;
    Params prm;
    int64_t row_bins[RB_COUNT + 1] = {};
    int64_t H = 0, Nh = 0, ne = 0, npieces = 0;
    int L = 0;
    LevelState lv[kMaxLevels];
    spgemm_stats stats{};
    // timing
    struct Ev {
        int pass, phase;
        hipEvent_t a, b;
    };
    std::vector<hipEvent_t> evpool;
    size_t evnext = 0;
    std::vector<Ev> evs;
    // debug dumps
    bool fused_sym = false;
    bool dbg_valid = false;
    bool dbg_has_val = false;
    int dbg_levels = 0;
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

void debug_copy_chat(spgemm_plan p, const int64_t* chat_rp, const int32_t* col, const double* val,
                     const int32_t* hrows, hipStream_t st);
void debug_copy_level(spgemm_plan p, int l, const int64_t* rp, int64_t npos, const int32_t* col,
                      const double* val, const int32_t* inv, hipStream_t st);

__global__ void k_i32_to_i64(const int32_t* a, int64_t n, int64_t* b) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) b[i] = a[i];
}

// Symbolic pass of the heavy rows the way Algorithm 3 lays it out: expand
// C-hat (columns only), then per level Histogram, ThreshPartition and
// Multisplit, and count distinct columns of every final chunk.
void heavy_symbolic_multisplit(spgemm_plan p, const DevCSR& A, const DevCSR& B,
                               const int64_t* chat_rp, const int32_t* ent_k, const int64_t* ent_q,
                               const int64_t* ent_dest, const int64_t* P, const int32_t* hrows,
                               int64_t* cnt_row, hipStream_t st) {
    Arena& ar = p->ar;
    const Params& q = p->prm;
    int32_t* buf0c = ar.get<int32_t>("buf0c", (size_t)p->Nh);
    {
        ExpandArgs ea{ent_k, ent_q, ent_dest, P, p->ne, A.val, B.rp, B.col, B.val, buf0c,
                      nullptr, p->npieces,
                      ar.get<int64_t>("expand_tiles", (size_t)expand_tiles(p->npieces) + 1)};
        PhaseScope ps(p, 0, SPGEMM_PHASE_OUTER_PROD, st);
        expand(ea, st);
        add_bytes(p, 0, SPGEMM_PHASE_OUTER_PROD, 4.0 * p->Nh + 20.0 * p->ne);
    }
    if (p->opt.debug_dump) debug_copy_chat(p, chat_rp, buf0c, nullptr, hrows, st);

    if (q.nlevels == 0) {
        ChunkItems ci{};
            ci.hash_top_logS = p->prm.hash_top_logS;
        ci.rp = chat_rp;
        ci.map = hrows;
        ci.bcol = buf0c;
        ci.cnt = cnt_row;
        ci.width = q.final_width;
        PhaseScope ps(p, 0, SPGEMM_PHASE_HEAVY_ACCUM, st);
        accumulate_chunks(ci, CB_DENSE, 0, p->H, false, st);
        add_bytes(p, 0, SPGEMM_PHASE_HEAVY_ACCUM, 4.0 * p->Nh);
    } else {
        int32_t* bufc[2] = {buf0c, ar.get<int32_t>("buf1c", (size_t)p->Nh)};
        const int64_t* rp_in = chat_rp;
        int64_t R = p->H, total = p->Nh;
        int L = 0;
        for (int l = 0; l < q.nlevels; ++l) {
            const bool last = (l == q.nlevels - 1);
            LevelState& S_l = p->lv[l];
            S_l.R = R;
            S_l.total_in = total;
            S_l.nch = q.vchunks[l];
            S_l.shift = ilog2(q.width[l]);
            S_l.nnat = R * S_l.nch;
            S_l.in_buf = l & 1;
            if (S_l.nnat >= (int64_t(1) << 31)) throw OverflowError("too many chunks in a level");
            int64_t* counts = ar.get<int64_t>(lvname("_counts", l), (size_t)S_l.nnat);
            int32_t* inv = ar.get<int32_t>(lvname("_inv", l), (size_t)S_l.nnat);
            int32_t* pos = ar.get<int32_t>(lvname("_pos", l), (size_t)S_l.nnat);
            int64_t* bins = ar.get<int64_t>(lvname("_bins", l), CB_COUNT + 1);
            LevelGeom g{rp_in, R, total, S_l.shift, S_l.nch, q.tau};
            {
                PhaseScope ps(p, 0, SPGEMM_PHASE_HISTO, st);
                fill<int64_t>(counts, S_l.nnat, 0, st);
                histogram(g, bufc[l & 1], counts, ar, st);
                classify_chunks(counts, S_l.nnat, q.tau, last, inv, pos, bins, ar, st);
                add_bytes(p, 0, SPGEMM_PHASE_HISTO,
                          4.0 * total + 8.0 * (R + 1) + 8.0 * S_l.nnat);
            }
            int64_t* hb = d2h(p, bins, CB_COUNT + 1, st);
            for (int b = 0; b <= CB_COUNT; ++b) S_l.bins[b] = hb[b];
            S_l.npos = S_l.bins[CB_EMPTY];
            int64_t* rp = ar.get<int64_t>(lvname("_rp", l), (size_t)S_l.npos + 1);
            int64_t* cursor = ar.get<int64_t>("cursor", (size_t)S_l.npos + 1);
            {
                PhaseScope ps(p, 0, SPGEMM_PHASE_HISTO, st);
                reord_rowptr(counts, inv, S_l.npos, rp, ar, st);
                copy<int64_t>(cursor, rp, S_l.npos, st);
            }
            int32_t* out = bufc[(l + 1) & 1];
            {
                PhaseScope ps(p, 0, SPGEMM_PHASE_MULTISPLIT, st);
                multisplit(g, bufc[l & 1], nullptr, pos, cursor, out, nullptr, ar, st);
                add_bytes(p, 0, SPGEMM_PHASE_MULTISPLIT, 8.0 * total + 8.0 * (R + 1));
            }
            if (p->opt.debug_dump) debug_copy_level(p, l, rp, S_l.npos, out, nullptr, inv, st);
            int64_t* nnz_l = ar.get<int64_t>(lvname("_nnz", l), (size_t)S_l.nnat);
            fill<int64_t>(nnz_l, S_l.nnat, 0, st);
            const int64_t nheavy = S_l.bins[CB_NEXT + 1] - S_l.bins[CB_NEXT];
            {
                ChunkItems ci{};
            ci.hash_top_logS = p->prm.hash_top_logS;
                ci.rp = rp;
                ci.map = inv;
                ci.bcol = out;
                ci.cnt = nnz_l;
                ci.width = q.width[l];
                PhaseScope ps(p, 0, SPGEMM_PHASE_HEAVY_ACCUM, st);
                for (int b = CB_DENSE; b <= CB_H8192; ++b)
                    accumulate_chunks(ci, b, S_l.bins[b], S_l.bins[b + 1] - S_l.bins[b], false,
                                      st);
            }
            p->stats.vchunks[l] = S_l.nch;
            p->stats.level_in_elems[l] = total;
            p->stats.level_heavy_chunks[l] = nheavy;
            p->stats.level_final_chunks[l] = S_l.bins[CB_EMPTY] - S_l.bins[CB_DENSE];
            L = l + 1;
            if (nheavy == 0) {
                S_l.final_elems = total;
                add_bytes(p, 0, SPGEMM_PHASE_HEAVY_ACCUM, 4.0 * total);
                break;
            }
            int64_t elems_heavy = d2h(p, rp + nheavy, 1, st)[0];
            S_l.final_elems = total - elems_heavy;
            add_bytes(p, 0, SPGEMM_PHASE_HEAVY_ACCUM, 4.0 * S_l.final_elems);
            rp_in = rp;
            R = nheavy;
            total = elems_heavy;
        }
        p->L = L;
        // bottom-up: a heavy chunk's count is the sum of its sub-chunks' counts
        {
            PhaseScope ps(p, 0, SPGEMM_PHASE_PREFIX_SUM, st);
            for (int l = L - 2; l >= 0; --l) {
                LevelState& a = p->lv[l];
                const int64_t nheavy = a.bins[CB_NEXT + 1] - a.bins[CB_NEXT];
                reduce_children(ar.get<int64_t>(lvname("_nnz", l + 1), 1), p->lv[l + 1].nch,
                                nheavy, ar.get<int32_t>(lvname("_inv", l), 1),
                                ar.get<int64_t>(lvname("_nnz", l), 1), st);
            }
            reduce_children(ar.get<int64_t>(lvname("_nnz", 0), 1), p->lv[0].nch, p->H, hrows,
                            cnt_row, st);
        }
    }
}

// Symbolic pass of the heavy rows without C-hat: per finest chunk slot, the
// element and distinct-column counts from one bitmap pass per heavy row;
// every level's chunk counts (the Histogram of Algorithm 3) and distinct
// counts (its Symbolic) are sums over slots. ThreshPartition then orders
// each level's chunks exactly as the multisplit path would.
void heavy_symbolic_fused(spgemm_plan p, const DevCSR& A, const DevCSR& B, const int64_t* S,
                          const int32_t* hrows, int64_t* cnt_row, hipStream_t st) {
    Arena& ar = p->ar;
    const Params& q = p->prm;
    const int64_t req = q.nlevels == 0 ? 1 : q.nchunks_required;
    const int64_t wfin = q.nlevels == 0 ? q.ppow : q.final_width;
    int64_t* elem_fin = ar.get<int64_t>("elem_fin", (size_t)(p->H * req));
    int64_t* dist_fin = ar.get<int64_t>("dist_fin", (size_t)(p->H * req));
    {
        PhaseScope ps(p, 0, SPGEMM_PHASE_HISTO, st);
        int32_t* bslot = ar.get<int32_t>("bslot", (size_t)(B.n * req + 1));
        heavy_symbolic(A, B, hrows, p->H, q.ppow, wfin, bslot, elem_fin, dist_fin, st);
        add_bytes(p, 0, SPGEMM_PHASE_HISTO, 4.0 * p->Nh + 16.0 * p->H * req);
    }
    if (q.nlevels == 0) {
        PhaseScope ps(p, 0, SPGEMM_PHASE_PREFIX_SUM, st);
        reduce_children(dist_fin, 1, p->H, hrows, cnt_row, st);
        return;
    }
    const int64_t* parent_slot0 = nullptr;
    const int32_t* parent_inv = nullptr;
    int64_t R = p->H, total = p->Nh;
    int64_t slots_per_chunk = req;
    int L = 0;
    for (int l = 0; l < q.nlevels; ++l) {
        const bool last = (l == q.nlevels - 1);
        LevelState& S_l = p->lv[l];
        S_l.R = R;
        S_l.total_in = total;
        S_l.nch = q.vchunks[l];
        S_l.shift = ilog2(q.width[l]);
        S_l.nnat = R * S_l.nch;
        S_l.in_buf = l & 1;
        if (S_l.nnat >= (int64_t(1) << 31)) throw OverflowError("too many chunks in a level");
        slots_per_chunk /= S_l.nch;
        int64_t* counts = ar.get<int64_t>(lvname("_counts", l), (size_t)S_l.nnat);
        int64_t* nnz_l = ar.get<int64_t>(lvname("_nnz", l), (size_t)S_l.nnat);
        int64_t* slot0 = ar.get<int64_t>(lvname("_slot0", l), (size_t)S_l.nnat);
        int32_t* inv = ar.get<int32_t>(lvname("_inv", l), (size_t)S_l.nnat);
        int32_t* pos = ar.get<int32_t>(lvname("_pos", l), (size_t)S_l.nnat);
        int64_t* bins = ar.get<int64_t>(lvname("_bins", l), CB_COUNT + 1);
        {
            PhaseScope ps(p, 0, SPGEMM_PHASE_HISTO, st);
            level_from_slots(parent_slot0, parent_inv, R, S_l.nch, (int)slots_per_chunk, req,
                             elem_fin, dist_fin, counts, nnz_l, slot0, st);
            classify_chunks(counts, S_l.nnat, q.tau, last, inv, pos, bins, ar, st);
        }
        int64_t* hb = d2h(p, bins, CB_COUNT + 1, st);
        for (int b = 0; b <= CB_COUNT; ++b) S_l.bins[b] = hb[b];
        S_l.npos = S_l.bins[CB_EMPTY];
        int64_t* rp = ar.get<int64_t>(lvname("_rp", l), (size_t)S_l.npos + 1);
        {
            PhaseScope ps(p, 0, SPGEMM_PHASE_HISTO, st);
            reord_rowptr(counts, inv, S_l.npos, rp, ar, st);
        }
        const int64_t nheavy = S_l.bins[CB_NEXT + 1] - S_l.bins[CB_NEXT];
        p->stats.vchunks[l] = S_l.nch;
        p->stats.level_in_elems[l] = total;
        p->stats.level_heavy_chunks[l] = nheavy;
        p->stats.level_final_chunks[l] = S_l.bins[CB_EMPTY] - S_l.bins[CB_DENSE];
        L = l + 1;
        if (nheavy == 0) {
            S_l.final_elems = total;
            break;
        }
        int64_t elems_heavy = d2h(p, rp + nheavy, 1, st)[0];
        S_l.final_elems = total - elems_heavy;
        parent_slot0 = slot0;
        parent_inv = inv;
        R = nheavy;
        total = elems_heavy;
    }
    p->L = L;
    PhaseScope ps(p, 0, SPGEMM_PHASE_PREFIX_SUM, st);
    reduce_children(ar.get<int64_t>(lvname("_nnz", 0), 1), p->lv[0].nch, p->H, hrows, cnt_row, st);
}

// ---------------------------------------------------------------- symbolic
int64_t symbolic_impl(spgemm_plan p, const DevCSR& A, const DevCSR& B, int64_t* C_rp,
                      hipStream_t st) {
    Arena& ar = p->ar;
    p->ready = false;
    p->dbg_valid = false;
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
    int64_t* st4 = ar.get<int64_t>("stats4", 4);
    {
        PhaseScope ps(p, 0, SPGEMM_PHASE_BINNING, st);
        int32_t* bmin = ar.get<int32_t>("bmin", (size_t)B.n + 1);
        int32_t* bmax = ar.get<int32_t>("bmax", (size_t)B.n + 1);
        brow_minmax(B, bmin, bmax, st);
        classify_rows(A, S, bmin, bmax, q.tau, rowlo, rowperm, rowbins, st4, ar, st);
        add_bytes(p, 0, SPGEMM_PHASE_BINNING, 8.0 * (n + 1) + 8.0 * n + 4.0 * n);
    }
    // Synchronize() of Algorithm 3 line 5: workspace is sized from these
    {
        SG_HIP(hipMemcpyAsync(p->host, rowbins, (RB_COUNT + 1) * sizeof(int64_t),
                              hipMemcpyDeviceToHost, st));
        SG_HIP(hipMemcpyAsync(p->host + 16, st4, 4 * sizeof(int64_t), hipMemcpyDeviceToHost, st));
        SG_HIP(hipStreamSynchronize(st));
        for (int b = 0; b <= RB_COUNT; ++b) p->row_bins[b] = p->host[b];
        p->stats.sum_products = p->host[16];
        p->stats.max_products = p->host[17];
        p->stats.heavy_rows = p->host[18];
        p->stats.heavy_products = p->host[19];
    }
    p->H = p->row_bins[RB_HEAVY + 1] - p->row_bins[RB_HEAVY];
    p->Nh = p->stats.heavy_products;
    const int32_t* hrows = rowperm + p->row_bins[RB_HEAVY];

    int64_t* cnt_row = ar.get<int64_t>("cnt_row", (size_t)n + 1);
    fill<int64_t>(cnt_row, n, 0, st);

    // light rows (Algorithm 3 line 22)
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
        for (int b = RB_WIN64; b <= RB_H8192; ++b)
            accumulate_rows(ri, b, p->row_bins[b], p->row_bins[b + 1] - p->row_bins[b], false, st);
    }

    // heavy rows (Algorithm 3 lines 6-21)
    p->L = 0;
    if (p->H > 0) {
        int64_t* chat_rp = ar.get<int64_t>("chat_rp", (size_t)p->H + 1);
        int32_t *ent_k = nullptr;
        int64_t *ent_q = nullptr, *ent_dest = nullptr, *P = nullptr;
        {
            PhaseScope ps(p, 0, SPGEMM_PHASE_CSR_TO_CSC, st);
            heavy_rowptr(A, S, hrows, p->H, chat_rp, ar, st);
            p->ne = masked_csr2csc(A, B, S, hrows, p->H, chat_rp, &ent_k, &ent_q, &ent_dest, &P,
                                   &p->npieces, ar, st);
            expand_tile_starts(P, p->ne, p->npieces,
                               ar.get<int64_t>("expand_tiles", (size_t)expand_tiles(p->npieces) + 1),
                               st);
            add_bytes(p, 0, SPGEMM_PHASE_CSR_TO_CSC, 36.0 * p->ne);
        }
        p->stats.chat_bytes = 12 * p->Nh + 8 * (p->H + 1);
        const int64_t req = q.nlevels == 0 ? 1 : q.nchunks_required;
        // the fused pass needs the row's bitmap in LDS and a per-B-row slot
        // histogram (B.nrows x slots int32) in HBM
        const bool fused_fits = heavy_symbolic_lds(q.ppow, req) <= (size_t)p->dev_lds &&
                                B.n * req <= (int64_t(1) << 28);
        p->fused_sym = p->opt.symbolic_mode == 1 || (p->opt.symbolic_mode == 0 && fused_fits);
        if (p->fused_sym && !fused_fits)
            throw OverflowError("fused symbolic pass needs more LDS than the device has");
        if (p->fused_sym)
            heavy_symbolic_fused(p, A, B, S, hrows, cnt_row, st);
        else
            heavy_symbolic_multisplit(p, A, B, chat_rp, ent_k, ent_q, ent_dest, P, hrows, cnt_row,
                                      st);
    }

    // C.rowPtr (Algorithm 3 lines 23-25)
    int64_t nnz_c;
    {
        PhaseScope ps(p, 0, SPGEMM_PHASE_PREFIX_SUM, st);
        scan_exclusive(LoadI64{cnt_row}, n, C_rp, ar, st);
        add_bytes(p, 0, SPGEMM_PHASE_PREFIX_SUM, 16.0 * n);
    }
    nnz_c = d2h(p, C_rp + n, 1, st)[0];
    // chunk output offsets, top-down
    if (p->H > 0 && p->L > 0) {
        PhaseScope ps(p, 0, SPGEMM_PHASE_PREFIX_SUM, st);
        child_offsets(ar.get<int64_t>(lvname("_nnz", 0), 1), p->lv[0].nch, p->H, hrows, C_rp,
                      ar.get<int64_t>(lvname("_off", 0), (size_t)p->lv[0].nnat), st);
        for (int l = 0; l + 1 < p->L; ++l) {
            const int64_t nheavy = p->lv[l].bins[CB_NEXT + 1] - p->lv[l].bins[CB_NEXT];
            child_offsets(ar.get<int64_t>(lvname("_nnz", l + 1), 1), p->lv[l + 1].nch, nheavy,
                          ar.get<int32_t>(lvname("_inv", l), 1),
                          ar.get<int64_t>(lvname("_off", l), 1),
                          ar.get<int64_t>(lvname("_off", l + 1), (size_t)p->lv[l + 1].nnat), st);
        }
    }
    p->stats.nrows = n;
    p->stats.ncols_c = B.m;
    p->stats.nnz_c = nnz_c;
    p->stats.tau = q.tau;
    p->stats.final_chunk_width = q.final_width;
    p->stats.nlevels = p->L;
    p->stats.nbatches = p->H > 0 ? 1 : 0;
    p->stats.lds_bytes = q.slm;
    p->stats.light_rows = p->row_bins[RB_EMPTY] - p->row_bins[RB_WIN64];
    p->stats.light_products = p->stats.sum_products - p->stats.heavy_products;
    if (p->H > 0 && q.nlevels == 0) p->stats.nlevels = 0;
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
    {
        PhaseScope ps(p, 1, SPGEMM_PHASE_LIGHT_ACCUM, st);
        for (int b = RB_WIN64; b <= RB_H8192; ++b)
            accumulate_rows(ri, b, p->row_bins[b], p->row_bins[b + 1] - p->row_bins[b], true, st);
    }
    if (p->H == 0) return;

    int64_t* chat_rp = ar.get<int64_t>("chat_rp", (size_t)p->H + 1);
    int32_t* ent_k = ar.get<int32_t>("csc_ent_k", (size_t)p->ne);
    int64_t* ent_q = ar.get<int64_t>("csc_ent_q", (size_t)p->ne);
    int64_t* ent_dest = ar.get<int64_t>("csc_ent_dest", (size_t)p->ne);
    int64_t* P = ar.get<int64_t>("csc_slice_off", (size_t)p->ne + 1);
    int32_t* bufc[2] = {ar.get<int32_t>("buf0c", (size_t)p->Nh), nullptr};
    double* bufv[2] = {ar.get<double>("buf0v", (size_t)p->Nh), nullptr};
    {
        ExpandArgs ea{ent_k, ent_q, ent_dest, P, p->ne, A.val, B.rp, B.col, B.val, bufc[0],
                      bufv[0], p->npieces,
                      ar.get<int64_t>("expand_tiles", (size_t)expand_tiles(p->npieces) + 1)};
        PhaseScope ps(p, 1, SPGEMM_PHASE_OUTER_PROD, st);
        expand(ea, st);
        add_bytes(p, 1, SPGEMM_PHASE_OUTER_PROD, 12.0 * p->Nh + 28.0 * p->ne);
    }
    if (p->opt.debug_dump) debug_copy_chat(p, chat_rp, bufc[0], bufv[0], hrows, st);

    if (q.nlevels == 0) {
        ChunkItems ci{};
            ci.hash_top_logS = p->prm.hash_top_logS;
        ci.rp = chat_rp;
        ci.map = hrows;
        ci.bcol = bufc[0];
        ci.bval = bufv[0];
        ci.off = C_rp;
        ci.Ccol = C_col;
        ci.Cval = C_val;
        ci.width = q.final_width;
        PhaseScope ps(p, 1, SPGEMM_PHASE_HEAVY_ACCUM, st);
        accumulate_chunks(ci, CB_DENSE, 0, p->H, true, st);
        add_bytes(p, 1, SPGEMM_PHASE_HEAVY_ACCUM, 12.0 * p->Nh);
        return;
    }
    bufc[1] = ar.get<int32_t>("buf1c", (size_t)p->Nh);
    bufv[1] = ar.get<double>("buf1v", (size_t)p->Nh);
    const int64_t* rp_in = chat_rp;
    for (int l = 0; l < p->L; ++l) {
        LevelState& S_l = p->lv[l];
        int32_t* inv = ar.get<int32_t>(lvname("_inv", l), (size_t)S_l.nnat);
        int32_t* pos = ar.get<int32_t>(lvname("_pos", l), (size_t)S_l.nnat);
        int64_t* rp = ar.get<int64_t>(lvname("_rp", l), (size_t)S_l.npos + 1);
        int64_t* off = ar.get<int64_t>(lvname("_off", l), (size_t)S_l.nnat);
        int64_t* cursor = ar.get<int64_t>("cursor", (size_t)S_l.npos + 1);
        copy<int64_t>(cursor, rp, S_l.npos, st);
        LevelGeom g{rp_in, S_l.R, S_l.total_in, S_l.shift, S_l.nch, q.tau};
        const int in = l & 1, outb = (l + 1) & 1;
        {
            PhaseScope ps(p, 1, SPGEMM_PHASE_MULTISPLIT, st);
            multisplit(g, bufc[in], bufv[in], pos, cursor, bufc[outb], bufv[outb], ar, st);
            add_bytes(p, 1, SPGEMM_PHASE_MULTISPLIT, 24.0 * S_l.total_in + 8.0 * (S_l.R + 1));
        }
        if (p->opt.debug_dump) debug_copy_level(p, l, rp, S_l.npos, bufc[outb], bufv[outb], inv, st);
        {
            ChunkItems ci{};
            ci.hash_top_logS = p->prm.hash_top_logS;
            ci.rp = rp;
            ci.map = inv;
            ci.bcol = bufc[outb];
            ci.bval = bufv[outb];
            ci.off = off;
            ci.Ccol = C_col;
            ci.Cval = C_val;
            ci.width = p->prm.width[l];
            PhaseScope ps(p, 1, SPGEMM_PHASE_HEAVY_ACCUM, st);
            for (int b = CB_DENSE; b <= CB_H8192; ++b)
                accumulate_chunks(ci, b, S_l.bins[b], S_l.bins[b + 1] - S_l.bins[b], true, st);
            add_bytes(p, 1, SPGEMM_PHASE_HEAVY_ACCUM, 12.0 * S_l.final_elems);
        }
        rp_in = rp;
    }
}

// ---------------------------------------------------------------- debug dumps
void debug_copy_chat(spgemm_plan p, const int64_t* chat_rp, const int32_t* col, const double* val,
                     const int32_t* hrows, hipStream_t st) {
    Arena& ar = p->ar;
    copy<int64_t>(ar.get<int64_t>("dbg_m1_rp", (size_t)p->H + 1), chat_rp, p->H + 1, st);
    copy<int32_t>(ar.get<int32_t>("dbg_m1_col", (size_t)p->Nh), col, p->Nh, st);
    if (val) copy<double>(ar.get<double>("dbg_m1_val", (size_t)p->Nh), val, p->Nh, st);
    int64_t* key = ar.get<int64_t>("dbg_m1_key", (size_t)p->H + 1);
    hipLaunchKernelGGL(k_i32_to_i64, dim3(grid_1d(ceil_div(p->H, 256))), dim3(256), 0, st, hrows,
                       p->H, key);
    SG_LAUNCH_CHECK();
    p->dbg_valid = true;
    p->dbg_has_val = val != nullptr;
}

void debug_copy_level(spgemm_plan p, int l, const int64_t* rp, int64_t npos, const int32_t* col,
                      const double* val, const int32_t* inv, hipStream_t st) {
    Arena& ar = p->ar;
    int64_t nnz = d2h(p, rp + npos, 1, st)[0];
    std::string b = "dbg_l" + std::to_string(l);
    copy<int64_t>(ar.get<int64_t>(b + "_rp", (size_t)npos + 1), rp, npos + 1, st);
    copy<int32_t>(ar.get<int32_t>(b + "_col", (size_t)nnz), col, nnz, st);
    if (val) copy<double>(ar.get<double>(b + "_val", (size_t)nnz), val, nnz, st);
    int64_t* key = ar.get<int64_t>(b + "_key", (size_t)npos + 1);
    if (npos > 0) {
        hipLaunchKernelGGL(k_i32_to_i64, dim3(grid_1d(ceil_div(npos, 256))), dim3(256), 0, st,
                           inv, npos, key);
        SG_LAUNCH_CHECK();
    }
    p->dbg_levels = std::max(p->dbg_levels, l + 1);
}

template <class F>
int guarded(F&& f) {
    try {
        return f();
    } catch (const OomError&) {
        return SPGEMM_ERR_OUT_OF_MEMORY;
    } catch (const OverflowError&) {
        return SPGEMM_ERR_OVERFLOW;
    } catch (const HipError& e) {
        if (e.code == hipErrorOutOfMemory) return SPGEMM_ERR_OUT_OF_MEMORY;
        return SPGEMM_ERR_HIP;
    } catch (const std::bad_alloc&) {
        return SPGEMM_ERR_OUT_OF_MEMORY;
    } catch (...) {
        return SPGEMM_ERR_HIP;
    }
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
    if (o.lds_budget_bytes < 0 || o.tau_override < 0 || o.chunk_width_override < 0 ||
        o.nchunks_cap < 0 || o.max_batch_products < 0)
        return SPGEMM_ERR_INVALID_ARG;
    if (o.chunk_width_override > 0 &&
        (o.chunk_width_override < 32 || (o.chunk_width_override & (o.chunk_width_override - 1))))
        return SPGEMM_ERR_INVALID_ARG;
    if (o.nchunks_cap > 0 && (o.nchunks_cap < 2 || (o.nchunks_cap & (o.nchunks_cap - 1))))
        return SPGEMM_ERR_INVALID_ARG;
    return guarded([&]() -> int {
        auto* p = new spgemm_plan_s();
        p->opt = o;
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
        if (hipHostMalloc((void**)&p->host, 64 * sizeof(int64_t), hipHostMallocDefault) !=
            hipSuccess) {
            delete p;
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
    return guarded([&]() -> int {
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
    });
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
    return guarded([&]() -> int {
        numeric_impl(p, to_dev(A), to_dev(B), C_rowptr, C_col, C_val, st);
        return SPGEMM_OK;
    });
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
    if (!p || !out || !p->opt.debug_dump || !p->dbg_valid) return SPGEMM_ERR_INVALID_ARG;
    return guarded([&]() -> int {
        Arena& ar = p->ar;
        memset(out, 0, sizeof(*out));
        if (which == -1) {
            out->nrows = p->H;
            out->nnz = p->Nh;
            out->rowptr = ar.get<int64_t>("dbg_m1_rp", (size_t)p->H + 1);
            out->col = ar.get<int32_t>("dbg_m1_col", (size_t)p->Nh);
            out->val = p->dbg_has_val ? ar.get<double>("dbg_m1_val", (size_t)p->Nh) : nullptr;
            out->row_key = ar.get<int64_t>("dbg_m1_key", (size_t)p->H + 1);
            out->chunk_width = p->prm.ppow;
            return SPGEMM_OK;
        }
        if (which < 0 || which >= p->L) return SPGEMM_ERR_INVALID_ARG;
        const LevelState& S_l = p->lv[which];
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
        default: return "unknown status";
    }
}

}  // extern "C"
