/*
 * spgemm.h -- C ABI of the MI355X (gfx950) sparse product C = A * B.
 *
 * The operation is sparse general matrix-matrix multiplication on CSR
 * matrices, as defined on the gMAGNUS page (Wolfson-Pou, Helal, Petrini,
 * "gMAGNUS: Fast SpGEMM on GPUs for Irregular Matrices via Hierarchical
 * Multisplit"): Section II-A gives the CSR layout (rowPtr / col / val,
 * sub-ranges [start:end)), Section II-B Eq. (1) the row-wise definition
 * C[i,:] = sum_j A[i,j] * B[j,:], and the split of the work into a symbolic
 * phase (C.rowPtr and C.nnz) and a numeric phase (C.col and C.val, given
 * C.rowPtr) that Algorithm 1 takes as its inputs and outputs. Internally the
 * library follows Algorithm 3 of that page: per-row intermediate-product
 * counts, a light/heavy row split at the threshold tau of Eq. (4), the
 * column-range chunk hierarchy of Section III-D (Eqs. 5-7), and
 * local-memory accumulation of every chunk and light row (Section III-E).
 * The heavy rows' numeric pass has three dataflows (spgemm_options
 * numeric_mode). The page's own: an outer product (Algorithm 4) expands the
 * heavy rows into C-hat and a hierarchical multisplit (Algorithm 5, Section
 * III-C) cuts them into chunks; or the same with the first multisplit level
 * forming its own products, so that C-hat is never written. The default,
 * where it applies: the column-range split is applied once to B's rows
 * instead of to C-hat, and every (heavy row, final chunk) is accumulated
 * straight from A and the split B, so neither C-hat nor its reordered copy
 * is built; the chunk sets, and so the result, are the same.
 *
 * Conventions for every entry point
 *   - Matrix and output arrays are DEVICE pointers on the current HIP
 *     device. Row pointers are int64, column indices int32, values fp64.
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued
 *     on it; spgemm_symbolic blocks until C_nnz is known, spgemm_numeric
 *     returns without waiting.
 *   - Every call returns an spgemm_status (0 = success, negative = error).
 *     No C++ exception crosses this boundary. After an error the outputs are
 *     unspecified, and the plan can still be destroyed or reused.
 *   - A plan is not thread-safe; separate plans are independent.
 */
#ifndef SPGEMM_H
#define SPGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPGEMM_API __attribute__((visibility("default")))

typedef enum {
    SPGEMM_OK = 0,
    SPGEMM_ERR_INVALID_ARG = -1,   /* null pointer, negative size, bad option      */
    SPGEMM_ERR_DIM_MISMATCH = -2,  /* A.ncols != B.nrows                           */
    SPGEMM_ERR_INDEX_RANGE = -3,   /* column index outside [0, ncols) or bad rowptr */
    SPGEMM_ERR_OVERFLOW = -4,      /* a size exceeds int32 columns / int64 offsets  */
    SPGEMM_ERR_OUT_OF_MEMORY = -5, /* device workspace could not be allocated       */
    SPGEMM_ERR_PLAN_MISMATCH = -6, /* numeric called with other shapes than symbolic */
    SPGEMM_ERR_HIP = -7,           /* a HIP runtime call failed                     */
    SPGEMM_ERR_NOT_READY = -8,     /* numeric called before a successful symbolic   */
    SPGEMM_ERR_CAPACITY = -9,      /* spgemm_multiply: C has more entries than room */
    SPGEMM_ERR_SCRATCH_LIMIT = -10, /* spgemm_multiply_noalloc: the product needs more
                                       workspace than its fixed scratch buffer holds */
    SPGEMM_ERR_INTERNAL = -11       /* a self-check of a plan with debug_dump = 1 failed:
                                       a multisplit level's chunk sizes do not add up to
                                       its input (a library bug, not a caller error)  */
} spgemm_status;

/* A CSR matrix (gMAGNUS page, Section II-A). `rowptr` has nrows+1 entries
 * with rowptr[0] = 0 and rowptr[nrows] = nnz; `col` and `val` have nnz
 * entries. Columns need not be sorted within a row. A repeated column in one
 * row acts as a sum of the two entries (the product is linear). `val` may
 * be NULL for spgemm_symbolic, which reads structure only. */
typedef struct {
    int64_t nrows;
    int64_t ncols;
    int64_t nnz;
    const int64_t* rowptr;
    const int32_t* col;
    const double* val;
} spgemm_csr;

/* Tuning and debugging options. Zero means "derive it", following the
 * parameter rules of the gMAGNUS page, Section III-D. None of them changes
 * the result: they move work between the light path, the heavy path and the
 * multisplit levels. */
typedef struct {
    int64_t lds_budget_bytes;     /* s_LM of Eq. (4)-(6); 0 = device's LDS per work group */
    int64_t tau_override;         /* heavy threshold tau; 0 = Eq. (4)                     */
    int64_t chunk_width_override; /* final chunk width (power of two >= 32); 0 = derived  */
    int32_t nchunks_cap;          /* cap on chunks per level (power of two >= 2); 0 = 32  */
    int32_t validate_inputs;      /* 1 = check rowptr and column ranges (default 1)       */
    int32_t debug_dump;           /* 1 = keep copies of C-hat and each C-hat-reord level,
                                     fill new value workspace with NaN, and check after
                                     each multisplit level that its chunk sizes add up to
                                     the level's input (Sigma u of the heavy rows at level
                                     0); a failed check returns INTERNAL                  */
    int32_t timing;               /* 1 = time every phase with HIP events                 */
    int64_t max_batch_products;   /* heavy products per row batch; 0 = one batch          */
    int32_t symbolic_mode;        /* heavy-row symbolic pass: 0 = auto, 1 = fused per-row
                                     bitmap pass, 2 = multisplit of column-only C-hat      */
    int32_t numeric_mode;         /* heavy-row numeric pass: 0 = auto (3 where it applies,
                                     else 1; 2 when debug_dump is set, so that C-hat and
                                     the levels can be dumped),
                                     1 = products formed inside the first multisplit level
                                     (C-hat is never written), 2 = outer product into C-hat
                                     then multisplit, 3 = direct: B's rows split into the
                                     final chunks once, and every (heavy row, chunk) item
                                     accumulated straight from A and the split B (needs
                                     the fused symbolic pass; else 1 runs)                 */
    int64_t workspace_limit_bytes; /* most device workspace the plan may hold; a call that
                                     needs more returns OUT_OF_MEMORY (0 = no limit)      */
} spgemm_options;

/* Phases, named after the gMAGNUS page's phase breakdown (Section IV-C,
 * Figs. 5 and 7), plus the light path and setup pieces of Algorithm 3. */
typedef enum {
    SPGEMM_PHASE_VALIDATE = 0,
    SPGEMM_PHASE_INTER_PROD_SIZE, /* InterOffsets: u(i) and its prefix sum        */
    SPGEMM_PHASE_BINNING,         /* ThreshPartition of rows into heavy / bins    */
    SPGEMM_PHASE_CSR_TO_CSC,      /* MaskedCsr2Csc of the heavy rows              */
    SPGEMM_PHASE_OUTER_PROD,      /* OuterProduct into C-hat                       */
    SPGEMM_PHASE_HISTO,           /* Histogram + chunk partition + prefix sum      */
    SPGEMM_PHASE_MULTISPLIT,      /* Multisplit into C-hat-reord                   */
    SPGEMM_PHASE_HEAVY_ACCUM,     /* dense / hash accumulation of chunks           */
    SPGEMM_PHASE_LIGHT_ACCUM,     /* accumulation of light rows                    */
    SPGEMM_PHASE_PREFIX_SUM,      /* C.rowPtr prefix sum and chunk offsets         */
    SPGEMM_PHASE_DIRECT_DENSE,    /* direct numeric path: dense-window items       */
    SPGEMM_PHASE_DIRECT_RANK,     /* direct numeric path: bitmap-rank items and
                                     B's values in split order                     */
    SPGEMM_NUM_PHASES
} spgemm_phase;

#define SPGEMM_MAX_LEVELS 8

/* What spgemm_plan_stats reports: the columns of the gMAGNUS page's runtime
 * parameter tables (Tables V and VI: C-hat size, heavy intermediate-product
 * and heavy-row fractions, chunks per level), plus timing per phase. Byte
 * counts are the algorithmic minimum each phase must move, in the style of
 * Eq. (8). Times and bytes cover the last symbolic + numeric pair. */
typedef struct {
    int64_t nrows, ncols_c, nnz_c;
    int64_t sum_products;         /* sum of u(i) over all rows                   */
    int64_t max_products;         /* max of u(i)                                 */
    int64_t heavy_rows;           /* rows with u(i) > tau                        */
    int64_t heavy_products;       /* sum of u(i) over heavy rows                 */
    int64_t tau;
    int64_t final_chunk_width;
    int32_t nlevels;              /* multisplit levels (0 = heavy rows fit LDS)  */
    int32_t nbatches;
    int32_t vchunks[SPGEMM_MAX_LEVELS];        /* chunks per row per level      */
    int64_t level_in_elems[SPGEMM_MAX_LEVELS]; /* elements reordered per level  */
    int64_t level_heavy_chunks[SPGEMM_MAX_LEVELS];
    int64_t level_final_chunks[SPGEMM_MAX_LEVELS];
    int64_t chat_bytes;           /* bytes of C-hat (col + val + rowptr)         */
    /* [0] = symbolic pass, [1] = numeric pass; zero unless timing = 1 */
    double phase_ms[2][SPGEMM_NUM_PHASES];
    int64_t phase_launches[2][SPGEMM_NUM_PHASES];
    double phase_bytes[2][SPGEMM_NUM_PHASES];
    int64_t lds_bytes;            /* s_LM used                                    */
    int64_t light_rows;           /* rows with 0 < u(i) <= tau                    */
    int64_t light_products;
    int32_t numeric_path;         /* heavy rows' numeric pass that ran: 0 = none,
                                     1 = first level formed in the multisplit tiles,
                                     2 = outer product into C-hat, 3 = direct          */
    int32_t reserved_stats;
    /* Structural statistics of the product over all rows of A (the operator
     * features of the SparseDitto page, Section 3.1, Eqs. 5 and 6): */
    int64_t u_p95;                /* 95th percentile of u(i), as the upper end of the
                                     histogram bucket that holds it: exact below 64,
                                     then buckets 1/64 of an octave wide             */
    double u_cv;                  /* coefficient of variation of u(i)             */
    double f_u_le[3];             /* F_h: fraction of rows with u(i) <= h for
                                     h = 512, 4096, 32768                         */
    double gamma;                 /* sum of u(i) / nnz(C): products per output    */
} spgemm_stats;

/* One intermediate matrix kept by a plan with debug_dump = 1. */
typedef struct {
    int64_t nrows;                /* rows of C-hat, or chunks of the level     */
    int64_t nnz;
    const int64_t* rowptr;        /* device, nrows+1                           */
    const int32_t* col;           /* device, global column indices             */
    const double* val;            /* device; NULL when only symbolic ran       */
    const int64_t* row_key;       /* device, nrows: see spgemm_plan_debug      */
    int64_t chunk_width;          /* column width of every row of this matrix */
} spgemm_debug_matrix;

typedef struct spgemm_plan_s* spgemm_plan;

/* Fill `opt` with the defaults (all derived, validation on). */
SPGEMM_API void spgemm_options_default(spgemm_options* opt);

/* Create a plan that owns all device workspace and the structure cached
 * between symbolic and numeric (Algorithm 3's setup state). `opt` may be
 * NULL for defaults. The caller owns *out and frees it with
 * spgemm_plan_destroy. Errors: INVALID_ARG (bad option), HIP (no device). */
SPGEMM_API int spgemm_plan_create(spgemm_plan* out, const spgemm_options* opt);

/* Free the plan and every device buffer it holds. NULL is a no-op. */
SPGEMM_API void spgemm_plan_destroy(spgemm_plan plan);

/* Symbolic phase (gMAGNUS page, Section II-B and Algorithm 3 up to the
 * PrefixSum of C.rowPtr):
 * computes C_rowptr (device, A.nrows+1 int64, caller-allocated) and the
 * total C_nnz (host out). The structure is the symbolic product: every
 * (i, j) reachable through a stored A[i,k] and a stored B[k,j], including
 * entries whose values later cancel to zero. Reads A and B structure only.
 * Blocks the calling thread until C_nnz is known. Errors: INVALID_ARG,
 * DIM_MISMATCH, INDEX_RANGE (validation on), OVERFLOW (A.ncols or B.ncols
 * above INT32_MAX, A.nrows of INT32_MAX or more), OUT_OF_MEMORY (device
 * memory, or the plan's workspace_limit_bytes, exhausted), HIP. */
SPGEMM_API int spgemm_symbolic(spgemm_plan plan, const spgemm_csr* A, const spgemm_csr* B,
                               int64_t* C_rowptr, int64_t* C_nnz, void* stream);

/* Numeric phase (gMAGNUS page, Algorithm 1 outputs; the numeric steps
 * that close Algorithm 3): fills C_col (int32) and C_val (fp64), C_nnz entries each,
 * caller-allocated device buffers, given the C_rowptr that
 * spgemm_symbolic produced for the same A and B structure. Columns come out
 * strictly ascending within each row. Values are recomputed from A.val and
 * B.val, so new values on the same structure need only a new numeric call.
 * Each value is a sum of the entry's products in an unspecified order.
 * Asynchronous on `stream`. Errors: INVALID_ARG, NOT_READY (no symbolic
 * yet), PLAN_MISMATCH (shapes or nnz differ from the symbolic call), HIP. */
SPGEMM_API int spgemm_numeric(spgemm_plan plan, const spgemm_csr* A, const spgemm_csr* B,
                              const int64_t* C_rowptr, int32_t* C_col, double* C_val,
                              void* stream);

/* Both phases in one call (gMAGNUS page, Algorithm 3 run through in one
 * go): the symbolic phase fills C_rowptr and *C_nnz; if *C_nnz <= capacity
 * (entries of room in the caller's C_col and C_val, device buffers) the
 * numeric phase fills them as spgemm_numeric would and the call returns OK.
 * Otherwise it returns CAPACITY with C_rowptr and *C_nnz valid and the plan
 * ready, so the caller can allocate *C_nnz entries and call spgemm_numeric
 * for the same A and B. Blocks until *C_nnz is known; the numeric part is
 * asynchronous on `stream`. Errors: those of spgemm_symbolic and
 * spgemm_numeric, INVALID_ARG (capacity < 0), CAPACITY. */
SPGEMM_API int spgemm_multiply(spgemm_plan plan, const spgemm_csr* A, const spgemm_csr* B,
                               int64_t* C_rowptr, int32_t* C_col, double* C_val,
                               int64_t capacity, int64_t* C_nnz, void* stream);

/* Size of the fixed device scratch buffer of spgemm_multiply_noalloc. */
#define SPGEMM_NOALLOC_SCRATCH_BYTES ((int64_t)64 << 20)

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * Computes C = A * B as spgemm_multiply does on a fresh plan created with
 * `opt` (NULL = defaults; timing and debug_dump must be 0, else
 * INVALID_ARG), into the caller's C_rowptr (A.nrows+1 int64), C_col and
 * C_val (`capacity` entries each), all device buffers. Every other piece of
 * device memory the call needs comes from one buffer of
 * SPGEMM_NOALLOC_SCRATCH_BYTES inside the library, which each device the
 * library runs on holds from the first call until the process ends; no
 * hipMalloc, hipFree or other device or pinned-host allocation is made (the
 * host bookkeeping of the call uses the C++ heap). The light and heavy rows
 * run on `stream` alone. Returns SCRATCH_LIMIT, with the outputs
 * unspecified, when the product needs more workspace than the buffer holds,
 * and CAPACITY, with C_rowptr and *C_nnz valid, when C does not fit
 * `capacity` (call again with room for *C_nnz entries). Every call on a
 * device shares that device's buffer and keeps the last call's contents
 * there: calls that overlap on one device race, so the caller orders them
 * (one stream, or a wait for the previous call's stream) and makes them
 * from one host thread at a time. Blocks until *C_nnz is known; the numeric
 * part is asynchronous on `stream`. Errors: those of spgemm_multiply (but
 * never OUT_OF_MEMORY), SCRATCH_LIMIT. */
SPGEMM_API int spgemm_multiply_noalloc(const spgemm_options* opt, const spgemm_csr* A,
                                       const spgemm_csr* B, int64_t* C_rowptr, int32_t* C_col,
                                       double* C_val, int64_t capacity, int64_t* C_nnz,
                                       void* stream);

/* Copy the statistics of the last symbolic + numeric pair into *out
 * (synchronises on pending timing events). Errors: INVALID_ARG. */
SPGEMM_API int spgemm_plan_stats(spgemm_plan plan, spgemm_stats* out);

/* With debug_dump = 1: describe C-hat (which = -1; row_key = original row
 * of each heavy row) or the reordered matrix of multisplit level `which`
 * (row_key = the chunk's parent row of the level's input times the level's
 * chunk count plus the chunk number, i.e. the chunk's natural index; rows
 * are in the level's output order). Pointers stay valid until the next
 * symbolic or numeric call or plan destruction. Errors: INVALID_ARG
 * (no dump kept, or no such level). */
SPGEMM_API int spgemm_plan_debug(spgemm_plan plan, int which, spgemm_debug_matrix* out);

/* A static English description of a status code. */
SPGEMM_API const char* spgemm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPGEMM_H */
