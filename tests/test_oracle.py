"""Pins for the CPU oracle: each test ties it to something other than itself.

The oracle (``oracle/``) is checked against
* the worked example the gMAGNUS page prints (Figure 1), for C, C-hat and
  the chunked C-hat-reord;
* brute-force dense products (numpy float64 within a rounding bound, and
  exact int64 products for small-integer values);
* identity, permutation, rank-1 and diagonal products (exact);
* the closed form of the all-ones banded square;
* the row-sum identity C*1 = A*(B*1);
* scipy.sparse's product;
* brute-force u(i) = sum of nnz(B[k,:]) over row i of A;
* closed forms of the structural statistics (SparseDitto page, Section 3.1,
  Eqs. 5 and 6) on a staircase product whose u(i) = i * L is known.
A plausible mistake (a dropped term, a wrong index, a transposed operand,
an unsorted or merged-away column) breaks at least one of these.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.sparse as sp

import oracle
from oracle import stages
from spgemm_irregular_matrices_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BOUND = 1e-12


def setup_module(_m):
    oracle.build(force=False)


def _dense_pattern(M):
    d = np.zeros((M.nrows, M.ncols), dtype=np.int64)
    rows = np.repeat(np.arange(M.nrows), np.diff(M.rowptr))
    d[rows, M.col] = 1
    return d


def _oracle_dense(rp, col, val, n, p):
    d = np.zeros((n, p))
    pat = np.zeros((n, p), dtype=bool)
    rows = np.repeat(np.arange(n), np.diff(rp))
    d[rows, col] = val
    pat[rows, col] = True
    return d, pat


def _check_sorted_rows(rp, col):
    for i in range(rp.size - 1):
        c = col[rp[i]:rp[i + 1]]
        assert np.all(np.diff(c) > 0), f"row {i} not strictly ascending"


# ---------------------------------------------------------------- Figure 1
def _fig1():
    with open(os.path.join(GOLDEN, "fig1_heavy_rows.json")) as f:
        g = json.load(f)
    na, ma = g["shape_A"]
    nb, mb = g["shape_B"]
    arows = [g["A_rows"].get(str(i), []) for i in range(na)]
    brows = [g["B_rows"].get(str(i), []) for i in range(nb)]
    return g, arows, brows, (na, ma), (nb, mb)


def _term_value(term, Ad, Bd):
    # "A15B53" -> A[1,5] * B[5,3]
    a_i, a_k, b_k, b_j = int(term[1]), int(term[2]), int(term[4]), int(term[5])
    assert a_k == b_k
    return Ad[a_i, a_k] * Bd[b_k, b_j]


@pytest.mark.parametrize("kind", ["uniform", "int"])
def test_fig1_product(kind):
    g, arows, brows, (na, ma), (nb, mb) = _fig1()
    A0 = synth.from_rows(na, ma, arows)
    B0 = synth.from_rows(nb, mb, brows)
    A = synth.CSR(na, ma, A0.rowptr, A0.col, synth._values(kind, 11, A0.nnz))
    B = synth.CSR(nb, mb, B0.rowptr, B0.col, synth._values(kind, 12, B0.nnz))
    Ad, Bd = A.to_dense(), B.to_dense()
    res = oracle.spgemm_rows(A, B, g["heavy_rows"])
    for x, i in enumerate(g["heavy_rows"]):
        col, val, absum = res.row(x)
        exp = g["C"][str(i)]
        assert col.tolist() == exp["col"]
        for y, terms in enumerate(exp["terms"]):
            vals = [_term_value(t, Ad, Bd) for t in terms]
            ref = math.fsum(vals)
            if kind == "int":
                assert val[y] == ref
            else:
                assert abs(val[y] - ref) <= BOUND * sum(abs(v) for v in vals)
            assert absum[y] == pytest.approx(sum(abs(v) for v in vals), rel=1e-15)
    # row 0 of A is empty, so row 0 of C is empty
    assert oracle.spgemm_rows(A, B, [0]).nnz == 0


def test_fig1_stages():
    g, arows, brows, (na, ma), (nb, mb) = _fig1()
    A0 = synth.from_rows(na, ma, arows)
    B0 = synth.from_rows(nb, mb, brows)
    A = synth.CSR(na, ma, A0.rowptr, A0.col, synth._values("uniform", 13, A0.nnz))
    B = synth.CSR(nb, mb, B0.rowptr, B0.col, synth._values("uniform", 14, B0.nnz))
    Ad, Bd = A.to_dense(), B.to_dense()
    rp, col, val = stages.expand(A, B, g["heavy_rows"])
    assert rp.tolist() == g["C_hat"]["rowptr"]
    assert col.tolist() == g["C_hat"]["col"]
    assert val.tolist() == [_term_value(t, Ad, Bd) for t in g["C_hat"]["val"]]
    W, nch = g["chunk_width"], g["nchunks"]
    k = 0
    for x, _i in enumerate(g["heavy_rows"]):
        s, e = rp[x], rp[x + 1]
        chunks = stages.split_by_width(col[s:e], val[s:e], W, 0, nch)
        for c, (cc, vv) in enumerate(chunks):
            assert list(g["C_hat_reord"]["rows"][k]) == [g["heavy_rows"][x], c]
            exp_cols = g["C_hat_reord"]["local_col"][k]
            exp_vals = [_term_value(t, Ad, Bd) for t in g["C_hat_reord"]["val"][k]]
            # elements inside a chunk are unordered: compare multisets
            assert sorted(zip((cc - c * W).tolist(), vv.tolist())) == sorted(zip(exp_cols, exp_vals))
            k += 1


# ---------------------------------------------------------------- counts
def test_row_products_bruteforce():
    A = synth.random_csr(300, 200, seed=7, value_seed=8, mean_len=6, skew=1.5)
    B = synth.random_csr(200, 250, seed=9, value_seed=10, mean_len=5, skew=1.2)
    u = oracle.row_products(A, B)
    for i in range(A.nrows):
        exp = 0
        for q in range(A.rowptr[i], A.rowptr[i + 1]):
            k = A.col[q]
            exp += B.rowptr[k + 1] - B.rowptr[k]
        assert u[i] == exp
    res = oracle.spgemm_rows(A, B)
    assert np.array_equal(res.u, u)
    # every distinct column is at most one product, so nnz(C_i) <= u(i)
    assert np.all(np.diff(res.rowptr) <= u)


# ---------------------------------------------------------------- dense checks
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_dense_random(seed):
    A = synth.random_csr(150, 120, seed=seed, value_seed=100 + seed, mean_len=8, skew=1.3,
                         empty_frac=0.1)
    B = synth.random_csr(120, 170, seed=seed + 50, value_seed=200 + seed, mean_len=6, skew=1.1)
    rp, col, val, absum = oracle.spgemm(A, B)
    _check_sorted_rows(rp, col)
    Ad, Bd = A.to_dense(), B.to_dense()
    ref = Ad @ Bd  # BLAS: error <= n*eps*sum|a||b|, far inside the bound
    absref = np.abs(Ad) @ np.abs(Bd)
    d, pat = _oracle_dense(rp, col, val, A.nrows, B.ncols)
    # structure is the boolean product of the patterns
    assert np.array_equal(pat, (_dense_pattern(A) @ _dense_pattern(B)) > 0)
    assert np.all(np.abs(d - ref) <= BOUND * absref)
    ab, _ = _oracle_dense(rp, col, absum, A.nrows, B.ncols)
    assert np.allclose(ab, absref, rtol=1e-13, atol=0)


def test_dense_transposed_operand_fails():
    """A*B differs from B^T-style misuse: the dense pin separates the two orders."""
    A = synth.random_csr(40, 40, seed=21, value_seed=22, mean_len=5)
    B = synth.random_csr(40, 40, seed=23, value_seed=24, mean_len=5)
    rp, col, val, _ = oracle.spgemm(A, B)
    d, _ = _oracle_dense(rp, col, val, 40, 40)
    assert not np.allclose(d, B.to_dense() @ A.to_dense())
    assert np.allclose(d, A.to_dense() @ B.to_dense(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", [4, 5])
def test_small_integer_exact(seed):
    A = synth.random_csr(200, 180, seed=seed, value_seed=300 + seed, mean_len=10, skew=1.2,
                         values="int")
    B = synth.random_csr(180, 160, seed=seed + 9, value_seed=400 + seed, mean_len=8, skew=1.2,
                         values="int")
    rp, col, val, _ = oracle.spgemm(A, B)
    Ai = A.to_dense().astype(np.int64)
    Bi = B.to_dense().astype(np.int64)
    ref = Ai @ Bi
    d, pat = _oracle_dense(rp, col, val, A.nrows, B.ncols)
    assert np.array_equal(pat, (_dense_pattern(A) @ _dense_pattern(B)) > 0)
    assert np.array_equal(d.astype(np.int64), ref)  # bit-exact
    # entries that cancel to zero are kept in the structure
    zeros = int(np.sum(pat & (ref == 0)))
    assert zeros > 0


def test_cancellation_kept():
    A = synth.from_rows(1, 2, [[0, 1]], [[1.0, 1.0]])
    B = synth.from_rows(2, 3, [[0, 2], [0]], [[2.5, 1.0], [-2.5]])
    rp, col, val, absum = oracle.spgemm(A, B)
    assert rp.tolist() == [0, 2]
    assert col.tolist() == [0, 2]
    assert val.tolist() == [0.0, 1.0]
    assert absum.tolist() == [5.0, 1.0]


def test_rmat_tiny_dense_gemm():
    """The 1024 x 1024 R-MAT square against a dense 1024^3 product."""
    A, B = synth.workload("rmat10_ef8")
    rp, col, val, _ = oracle.spgemm(A, B)
    Ad = A.to_dense()
    ref = Ad @ Ad
    absref = np.abs(Ad) @ np.abs(Ad)
    d, pat = _oracle_dense(rp, col, val, A.nrows, A.ncols)
    pA = _dense_pattern(A)
    assert np.array_equal(pat, (pA @ pA) > 0)
    assert np.all(np.abs(d - ref) <= BOUND * absref)


# ---------------------------------------------------------------- exact products
def test_identity_and_permutation_exact():
    A = synth.random_csr(120, 90, seed=31, value_seed=32, mean_len=7, skew=1.4)
    rp, col, val, _ = oracle.spgemm(synth.identity(120), A)
    assert np.array_equal(rp, A.rowptr) and np.array_equal(col, A.col) and np.array_equal(val, A.val)
    rp, col, val, _ = oracle.spgemm(A, synth.identity(90))
    assert np.array_equal(rp, A.rowptr) and np.array_equal(col, A.col) and np.array_equal(val, A.val)
    P = synth.permutation(120, 33)
    rp, col, val, _ = oracle.spgemm(P, A)   # row i of P*A is row perm[i] of A
    for i in range(120):
        k = P.col[i]
        s, e = A.rowptr[k], A.rowptr[k + 1]
        assert np.array_equal(col[rp[i]:rp[i + 1]], A.col[s:e])
        assert np.array_equal(val[rp[i]:rp[i + 1]], A.val[s:e])
    Q = synth.permutation(90, 34)
    rp, col, val, _ = oracle.spgemm(A, Q)   # column k of A moves to column Q.col[k]
    Ad = A.to_dense()
    d, _ = _oracle_dense(rp, col, val, 120, 90)
    exp = np.zeros_like(Ad)
    exp[:, Q.col] = Ad
    assert np.array_equal(d, exp)


def test_rank1_and_diagonal_exact():
    x = synth.random_csr(50, 1, seed=41, value_seed=42, mean_len=1)
    y = synth.random_csr(1, 60, seed=43, value_seed=44, mean_len=20)
    rp, col, val, _ = oracle.spgemm(x, y)
    d, _ = _oracle_dense(rp, col, val, 50, 60)
    assert np.array_equal(d, x.to_dense() @ y.to_dense())
    D1 = synth.CSR(64, 64, np.arange(65, dtype=np.int64), np.arange(64, dtype=np.int32),
                   synth.uniform_values(45, 64))
    D2 = synth.CSR(64, 64, np.arange(65, dtype=np.int64), np.arange(64, dtype=np.int32),
                   synth.uniform_values(46, 64))
    rp, col, val, _ = oracle.spgemm(D1, D2)
    assert np.array_equal(col, np.arange(64)) and np.array_equal(val, D1.val * D2.val)


def test_banded_all_ones_closed_form():
    n, h = 300, 8
    A = synth.banded(n, h, value_seed=0, values="ones")
    rp, col, val, _ = oracle.spgemm(A, A)
    assert rp[-1] == 33 * n - 272   # row i spans max(0,i-16)..min(n-1,i+16)
    for i in range(n):
        c = col[rp[i]:rp[i + 1]]
        assert c.tolist() == list(range(max(0, i - 2 * h), min(n - 1, i + 2 * h) + 1))
        for j, v in zip(c, val[rp[i]:rp[i + 1]]):
            exp = sum(1 for k in range(n) if abs(i - k) <= h and abs(k - j) <= h)
            assert v == exp
            if 2 * h <= i < n - 2 * h:
                assert v == 2 * h + 1 - abs(i - j)


def test_rowsum_identity():
    A = synth.rmat(11, 8, seed=51, value_seed=52)
    B = synth.rmat(11, 8, seed=53, value_seed=54)
    rp, col, val, _ = oracle.spgemm(A, B)
    Ad, Bd = A.to_dense(), B.to_dense()
    lhs = np.array([math.fsum(val[rp[i]:rp[i + 1]]) for i in range(A.nrows)])
    rhs = Ad @ Bd.sum(axis=1)
    bound = np.abs(Ad) @ np.abs(Bd).sum(axis=1)
    assert np.all(np.abs(lhs - rhs) <= BOUND * bound + 1e-300)


def test_scipy_product():
    A = synth.random_csr(400, 350, seed=61, value_seed=62, mean_len=9, skew=1.2)
    B = synth.random_csr(350, 500, seed=63, value_seed=64, mean_len=7, skew=1.1)
    rp, col, val, absum = oracle.spgemm(A, B)
    sa = sp.csr_matrix((A.val, A.col, A.rowptr), shape=(A.nrows, A.ncols))
    sb = sp.csr_matrix((B.val, B.col, B.rowptr), shape=(B.nrows, B.ncols))
    sc = (sa @ sb).tocsr()
    sc.sort_indices()
    # continuous values: no exact cancellation, so scipy keeps the same pattern
    assert np.array_equal(sc.indptr, rp) and np.array_equal(sc.indices, col)
    assert np.all(np.abs(sc.data - val) <= BOUND * absum)


# ---------------------------------------------------------------- edge cases
def test_edge_cases():
    E = synth.CSR(0, 5, np.zeros(1, np.int64), np.zeros(0, np.int32), np.zeros(0))
    B = synth.random_csr(5, 7, seed=71, value_seed=72, mean_len=2)
    rp, col, val, _ = oracle.spgemm(E, B)
    assert rp.tolist() == [0] and col.size == 0
    # inner dimension zero: every row is empty
    A0 = synth.CSR(4, 0, np.zeros(5, np.int64), np.zeros(0, np.int32), np.zeros(0))
    B0 = synth.CSR(0, 6, np.zeros(1, np.int64), np.zeros(0, np.int32), np.zeros(0))
    rp, col, val, _ = oracle.spgemm(A0, B0)
    assert rp.tolist() == [0] * 5
    # 1x1
    one = synth.CSR(1, 1, np.array([0, 1], np.int64), np.array([0], np.int32), np.array([-3.0]))
    rp, col, val, _ = oracle.spgemm(one, one)
    assert col.tolist() == [0] and val.tolist() == [9.0]
    # empty rows of A and of B
    A = synth.random_csr(30, 20, seed=73, value_seed=74, mean_len=3, empty_frac=0.5)
    B = synth.random_csr(20, 25, seed=75, value_seed=76, mean_len=3, empty_frac=0.5)
    rp, col, val, _ = oracle.spgemm(A, B)
    d, _ = _oracle_dense(rp, col, val, 30, 25)
    assert np.allclose(d, A.to_dense() @ B.to_dense(), rtol=0, atol=1e-14)
    with pytest.raises(ValueError):
        oracle.spgemm(A, A)


def test_row_subset_matches_full():
    A = synth.random_csr(200, 150, seed=81, value_seed=82, mean_len=6, skew=1.3)
    B = synth.random_csr(150, 180, seed=83, value_seed=84, mean_len=6, skew=1.3)
    full = oracle.spgemm_rows(A, B)
    sel = np.array([199, 0, 17, 17, 5, 150], dtype=np.int64)
    sub = oracle.spgemm_rows(A, B, sel, nthreads=3)
    for x, i in enumerate(sel):
        c1, v1, a1 = full.row(int(i))
        c2, v2, a2 = sub.row(x)
        assert np.array_equal(c1, c2) and np.array_equal(v1, v2) and np.array_equal(a1, a2)


def test_stage_chunks_partition_rows():
    A = synth.random_csr(60, 80, seed=91, value_seed=92, mean_len=10)
    B = synth.random_csr(80, 256, seed=93, value_seed=94, mean_len=12)
    full = oracle.spgemm_rows(A, B)
    for i in range(A.nrows):
        cols, vals = stages.expand_row(A, B, i)
        assert cols.size == full.u[i]
        W, nch = 32, 8
        parts = stages.split_by_width(cols, vals, W, 0, nch)
        assert sum(p[0].size for p in parts) == cols.size
        dist = stages.distinct_per_chunk(cols, W, 0, nch)
        c, _, _ = full.row(i)
        assert dist.sum() == c.size
        assert np.array_equal(stages.chunk_counts(cols, W, 0, nch),
                              np.bincount(cols // W, minlength=nch))


# ---------------------------------------------------------------- structural statistics
def _staircase(L):
    """Row i of A (100 rows) holds columns 0..i-1; every row of B holds columns
    0..L-1. So u(i) = i*L, C's row i has L entries for i > 0, nnz(C) = 99*L."""
    m = 100
    lens = np.arange(m, dtype=np.int64)
    arp = np.zeros(m + 1, dtype=np.int64)
    np.cumsum(lens, out=arp[1:])
    acol = np.concatenate([np.arange(i, dtype=np.int32) for i in range(m)])
    A = synth.CSR(m, m, arp, acol, np.ones(acol.size))
    brp = np.arange(m + 1, dtype=np.int64) * L
    bcol = np.tile(np.arange(L, dtype=np.int32), m)
    B = synth.CSR(m, L, brp, bcol, np.ones(bcol.size))
    return A, B


@pytest.mark.parametrize("L", [32, 512])
def test_structural_stats_closed_form(L):
    A, B = _staircase(L)
    u = oracle.row_products(A, B)
    assert np.array_equal(u, np.arange(100) * L)
    rp, _, _, _ = oracle.spgemm(A, B)
    assert rp[-1] == 99 * L
    st = oracle.structural_stats(u, int(rp[-1]))
    assert st["sum"] == 4950 * L and st["max"] == 99 * L
    # nearest rank: the 95th smallest of 0, L, ..., 99L is 94L
    assert st["p95"] == 94 * L
    # mean 49.5 L, population variance (100^2 - 1)/12 * L^2
    assert st["cv"] == pytest.approx(math.sqrt(9999 / 12) / 49.5, rel=1e-14)
    # F_h counts rows with i*L <= h, the bound included
    exp = [(min(h // L, 99) + 1) / 100 for h in (512, 4096, 32768)]
    assert st["f"] == exp
    assert exp[0] == (0.17 if L == 32 else 0.02)
    assert st["gamma"] == 50.0


def test_structural_stats_degenerate():
    st = oracle.structural_stats(np.zeros(0, dtype=np.int64), 0)
    assert st == {"sum": 0, "max": 0, "p95": 0, "cv": 0.0, "f": [0.0, 0.0, 0.0], "gamma": 0.0}
    st = oracle.structural_stats(np.full(20, 7), 140)
    assert st["p95"] == 7 and st["cv"] == 0.0 and st["f"] == [1.0, 1.0, 1.0] and st["gamma"] == 1.0
