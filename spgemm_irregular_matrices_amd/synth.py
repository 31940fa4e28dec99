"""Seeded synthetic sparse inputs (CSR, int64 row pointers, int32 columns, fp64 values).

This module only draws random structure and values. It holds none of the
product's arithmetic, so both the HIP path and the CPU oracle take their inputs
from here and nothing else.

Random numbers come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) used as a counter-based
generator: draw ``i`` of stream ``seed`` is ``mix64(seed + (i + 1) * GAMMA)``,
which is the ``i``-th output of a SplitMix64 generator seeded with ``seed``.
A uniform double in [0, 1) is ``(x >> 11) * 2**-53``.

Workload shapes follow the matrices the gMAGNUS page (Wolfson-Pou, Helal,
Petrini, "gMAGNUS: Fast SpGEMM on GPUs for Irregular Matrices via Hierarchical
Multisplit") evaluates in Section IV-A: recursive power-law (R-MAT) matrices
with the Graph500 quadrant probabilities a=0.57, b=c=0.19 (d=0.05), plus a
banded matrix (the structured case of Section II-B) and a rectangular
Zipf-row-length product whose heavy rows span the full column range.
"""
from __future__ import annotations

import dataclasses

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


@dataclasses.dataclass
class CSR:
    """A CSR matrix on the host: ``rowptr`` int64[n+1], ``col`` int32[nnz], ``val`` f64[nnz]."""

    nrows: int
    ncols: int
    rowptr: np.ndarray
    col: np.ndarray
    val: np.ndarray

    @property
    def nnz(self) -> int:
        return int(self.rowptr[-1])

    def check(self) -> "CSR":
        assert self.rowptr.dtype == np.int64 and self.col.dtype == np.int32
        assert self.val.dtype == np.float64
        assert self.rowptr.shape == (self.nrows + 1,)
        assert self.rowptr[0] == 0 and self.col.shape == (self.nnz,) == self.val.shape
        assert np.all(np.diff(self.rowptr) >= 0)
        if self.nnz:
            assert int(self.col.min()) >= 0 and int(self.col.max()) < self.ncols
        return self

    def row_lengths(self) -> np.ndarray:
        return np.diff(self.rowptr)

    def to_dense(self) -> np.ndarray:
        d = np.zeros((self.nrows, self.ncols), dtype=np.float64)
        rows = np.repeat(np.arange(self.nrows), np.diff(self.rowptr))
        np.add.at(d, (rows, self.col.astype(np.int64)), self.val)
        return d


# --------------------------------------------------------------------------
# counter-based SplitMix64
# --------------------------------------------------------------------------
def splitmix64(seed: int, idx: np.ndarray) -> np.ndarray:
    """Draw ``idx`` (uint64 array) of the SplitMix64 stream seeded with ``seed``."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + (idx + np.uint64(1)) * GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def uniform01(seed: int, idx: np.ndarray) -> np.ndarray:
    """Uniform doubles in [0, 1) with 53 random bits."""
    return (splitmix64(seed, idx) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def uniform_values(seed: int, n: int, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    """``n`` values uniform in [lo, hi), drawn in index order from stream ``seed``."""
    out = np.empty(n, dtype=np.float64)
    step = 1 << 24
    for s in range(0, n, step):
        e = min(n, s + step)
        out[s:e] = lo + (hi - lo) * uniform01(seed, np.arange(s, e, dtype=np.uint64))
    return out


def small_int_values(seed: int, n: int, k: int = 3) -> np.ndarray:
    """``n`` integers in [-k, k] as doubles (products and sums stay exact in fp64)."""
    x = splitmix64(seed, np.arange(n, dtype=np.uint64))
    return ((x % np.uint64(2 * k + 1)).astype(np.int64) - k).astype(np.float64)


def _csr_from_sorted_keys(keys: np.ndarray, nrows: int, ncols: int, vals: np.ndarray) -> CSR:
    rows = (keys // ncols).astype(np.int64)
    cols = (keys % ncols).astype(np.int32)
    rowptr = np.zeros(nrows + 1, dtype=np.int64)
    np.cumsum(np.bincount(rows, minlength=nrows), out=rowptr[1:])
    return CSR(nrows, ncols, rowptr, cols, vals).check()


# --------------------------------------------------------------------------
# R-MAT
# --------------------------------------------------------------------------
def rmat(scale: int, edge_factor: int, seed: int, value_seed: int,
         probs=(0.57, 0.19, 0.19, 0.05), values: str = "uniform") -> CSR:
    """Plain R-MAT graph as a 2^scale x 2^scale CSR matrix.

    Each of ``edge_factor * 2^scale`` edges picks one quadrant per level
    (``scale`` levels, most significant bit first): draw ``u`` from stream
    ``seed`` at index ``edge*scale + level``; u < a gives (0,0), u < a+b gives
    (0,1), u < a+b+c gives (1,0), otherwise (1,1). There is no noise and no
    vertex permutation, and self-loops are kept. Duplicate edges are merged,
    and values are drawn after merging, in CSR order, from ``value_seed``.
    """
    a, b, c, _ = probs
    n = 1 << scale
    nedges = edge_factor * n
    t1, t2, t3 = a, a + b, a + b + c
    keys_parts = []
    step = 1 << 22
    for s in range(0, nedges, step):
        e = np.arange(s, min(nedges, s + step), dtype=np.uint64)
        row = np.zeros(e.shape, dtype=np.int64)
        col = np.zeros(e.shape, dtype=np.int64)
        for lvl in range(scale):
            u = uniform01(seed, e * np.uint64(scale) + np.uint64(lvl))
            rbit = (u >= t2).astype(np.int64)
            cbit = (((u >= t1) & (u < t2)) | (u >= t3)).astype(np.int64)
            sh = scale - 1 - lvl
            row |= rbit << sh
            col |= cbit << sh
        keys_parts.append(row * n + col)
    keys = np.unique(np.concatenate(keys_parts))
    vals = _values(values, value_seed, keys.size)
    return _csr_from_sorted_keys(keys, n, n, vals)


def _values(kind: str, seed: int, n: int) -> np.ndarray:
    if kind == "uniform":
        return uniform_values(seed, n)
    if kind == "int":
        return small_int_values(seed, n)
    if kind == "ones":
        return np.ones(n, dtype=np.float64)
    raise ValueError(kind)


# --------------------------------------------------------------------------
# banded
# --------------------------------------------------------------------------
def banded(n: int, half_width: int, value_seed: int, values: str = "uniform") -> CSR:
    """n x n matrix with the diagonals -half_width..+half_width, cut at the edges."""
    i = np.arange(n, dtype=np.int64)
    lo = np.maximum(0, i - half_width)
    hi = np.minimum(n - 1, i + half_width)
    lens = hi - lo + 1
    rowptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(lens, out=rowptr[1:])
    nnz = int(rowptr[-1])
    rows = np.repeat(i, lens)
    col = (lo[rows] + (np.arange(nnz, dtype=np.int64) - rowptr[rows])).astype(np.int32)
    return CSR(n, n, rowptr, col, _values(values, value_seed, nnz)).check()


# --------------------------------------------------------------------------
# rows of distinct uniform columns (Zipf row lengths for the rectangular case)
# --------------------------------------------------------------------------
def zipf_lengths(n: int, alpha: float, cap: int, seed: int) -> np.ndarray:
    """``n`` row lengths with P(L=k) proportional to k^-alpha (k >= 1), clipped at ``cap``.

    Sampled by inverse CDF: the masses of 1..cap-1 are exact, and all mass at
    k >= cap (a Hurwitz zeta tail) sits on ``cap``.
    """
    from scipy.special import zeta

    k = np.arange(1, cap, dtype=np.float64)
    total = float(zeta(alpha, 1.0))
    pmf = np.empty(cap, dtype=np.float64)
    pmf[: cap - 1] = k ** (-alpha) / total
    pmf[cap - 1] = float(zeta(alpha, float(cap))) / total
    cdf = np.cumsum(pmf)
    cdf /= cdf[-1]
    u = uniform01(seed, np.arange(n, dtype=np.uint64))
    return np.minimum(np.searchsorted(cdf, u, side="right") + 1, cap).astype(np.int64)


def distinct_uniform_rows(lengths: np.ndarray, ncols: int, seed: int,
                          value_seed: int, values: str = "uniform") -> CSR:
    """Row i holds the first ``lengths[i]`` distinct values of its own column stream.

    Draw j of row i is ``floor(u * ncols)`` with u from stream ``seed`` at
    index ``i * 2^32 + j``. Columns are stored sorted.
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    n = lengths.size
    assert np.all(lengths <= ncols)
    have = np.zeros(0, dtype=np.int64)  # sorted unique keys row*ncols+col
    next_draw = np.zeros(n, dtype=np.int64)
    need = lengths.copy()
    while True:
        rows = np.nonzero(need > 0)[0]
        if rows.size == 0:
            break
        cnt = need[rows]
        r = np.repeat(rows, cnt)
        start = np.repeat(next_draw[rows] - np.cumsum(cnt) + cnt, cnt)
        j = start + np.arange(r.size, dtype=np.int64)
        u = uniform01(seed, (r.astype(np.uint64) << np.uint64(32)) + j.astype(np.uint64))
        c = np.minimum((u * ncols).astype(np.int64), ncols - 1)
        next_draw[rows] += cnt
        have = np.unique(np.concatenate([have, r * ncols + c]))
        got = np.bincount(have // ncols, minlength=n)
        need = lengths - got
        assert np.all(need >= 0)
    vals = _values(values, value_seed, have.size)
    return _csr_from_sorted_keys(have, n, ncols, vals)


# --------------------------------------------------------------------------
# small and edge-case matrices for tests
# --------------------------------------------------------------------------
def random_csr(nrows: int, ncols: int, seed: int, value_seed: int, mean_len: float = 4.0,
               skew: float = 0.0, max_len: int | None = None, empty_frac: float = 0.0,
               values: str = "uniform") -> CSR:
    """Random CSR with distinct columns per row.

    Row lengths are drawn as floor(mean_len * x^skew_pow) style power-law
    samples when ``skew`` > 0 (a Pareto tail with exponent ``skew``), else
    uniform in [0, 2*mean_len]. ``empty_frac`` of rows are forced empty.
    """
    u = uniform01(seed ^ 0x5A5A, np.arange(nrows, dtype=np.uint64))
    if skew > 0:
        lens = np.floor(mean_len * (1.0 - u) ** (-1.0 / skew) - mean_len + 1).astype(np.int64)
    else:
        lens = np.floor(u * (2 * mean_len + 1)).astype(np.int64)
    cap = ncols if max_len is None else min(ncols, max_len)
    lens = np.clip(lens, 0, cap)
    if empty_frac > 0:
        e = uniform01(seed ^ 0xA5A5, np.arange(nrows, dtype=np.uint64))
        lens[e < empty_frac] = 0
    if ncols == 0:
        lens[:] = 0
    return distinct_uniform_rows(lens, max(ncols, 1), seed, value_seed, values) if ncols else CSR(
        nrows, 0, np.zeros(nrows + 1, np.int64), np.zeros(0, np.int32), np.zeros(0, np.float64))


def from_dense(d: np.ndarray) -> CSR:
    """CSR of the nonzero pattern of a dense array (values copied)."""
    d = np.asarray(d, dtype=np.float64)
    r, c = np.nonzero(d)
    rowptr = np.zeros(d.shape[0] + 1, dtype=np.int64)
    np.cumsum(np.bincount(r, minlength=d.shape[0]), out=rowptr[1:])
    return CSR(d.shape[0], d.shape[1], rowptr, c.astype(np.int32), d[r, c].copy()).check()


def from_rows(nrows: int, ncols: int, rows: list, vals: list | None = None) -> CSR:
    """CSR from explicit per-row column lists (kept in the given order)."""
    rowptr = np.zeros(nrows + 1, dtype=np.int64)
    rowptr[1:] = np.cumsum([len(r) for r in rows])
    col = np.array([c for r in rows for c in r], dtype=np.int32)
    if vals is None:
        val = np.ones(col.size, dtype=np.float64)
    else:
        val = np.array([v for r in vals for v in r], dtype=np.float64)
    return CSR(nrows, ncols, rowptr, col, val).check()


def transpose(M: CSR) -> CSR:
    """The transpose of M; each of its rows lists entries in ascending column order."""
    rows = np.repeat(np.arange(M.nrows, dtype=np.int64), np.diff(M.rowptr))
    order = np.argsort(M.col.astype(np.int64) * max(M.nrows, 1) + rows, kind="stable")
    rowptr = np.zeros(M.ncols + 1, dtype=np.int64)
    np.cumsum(np.bincount(M.col, minlength=M.ncols), out=rowptr[1:])
    return CSR(M.ncols, M.nrows, rowptr, rows[order].astype(np.int32),
               M.val[order].copy()).check()


def identity(n: int) -> CSR:
    return CSR(n, n, np.arange(n + 1, dtype=np.int64), np.arange(n, dtype=np.int32),
               np.ones(n, dtype=np.float64))


def permutation(n: int, seed: int) -> CSR:
    """Permutation matrix P with P[i, perm[i]] = 1, perm from a seeded shuffle."""
    keys = splitmix64(seed, np.arange(n, dtype=np.uint64))
    perm = np.argsort(keys, kind="stable").astype(np.int32)
    return CSR(n, n, np.arange(n + 1, dtype=np.int64), perm, np.ones(n, dtype=np.float64))


# --------------------------------------------------------------------------
# the benchmark workloads
# --------------------------------------------------------------------------
WORKLOADS = {
    "rmat10_ef8": "R-MAT A*A, 1024 x 1024, edge factor 8, (0.57,0.19,0.19,0.05)",
    "banded_n1M_17diag": "banded A*A, n=1,048,576, diagonals -8..+8",
    "rmat18_ef16": "R-MAT A*A, 262,144 x 262,144, edge factor 16",
    "rmat20_ef8": "R-MAT A*A, 1,048,576 x 1,048,576, edge factor 8",
    "rect_zipf2.1_x_uniform16": "A 1,048,576 x 262,144 Zipf(2.1) rows capped 65,536; "
                                "B 262,144 x 1,048,576 with 16 uniform nnz/row",
}


# The gMAGNUS page's RMat set (Sec. IV-A, Table III): A of scale s with
# A.nnz/A.n in {4, 8, 16, 32} times an independent B of the same scale with
# B.nnz/B.n = 8, at the scales the table fills for each A density.
TABLE3_CELLS = [(s, a) for a, top in ((4, 20), (8, 19), (16, 18), (32, 18))
                for s in range(15, top + 1)]


def rmat_pair(scale: int, a_density: int, b_density: int = 8):
    """A seeded pair of independent plain R-MATs (A, B) of one scale."""
    A = rmat(scale, a_density, seed=700 + 10 * scale + a_density,
             value_seed=800 + 10 * scale + a_density)
    B = rmat(scale, b_density, seed=900 + scale + 100 * b_density,
             value_seed=950 + scale + 100 * b_density)
    return A, B


def pair_name(scale: int, a_density: int, b_density: int = 8) -> str:
    return f"rmat_pair_s{scale}_a{a_density}_b{b_density}"


def describe(name: str) -> str:
    """One-line description of a named workload."""
    if name.startswith("rmat_pair_"):
        s, a, b = (int(x[1:]) for x in name[len("rmat_pair_"):].split("_"))
        return (f"R-MAT A*B, independent A and B of scale {s} (2^{s} square), "
                f"A.nnz/A.n = {a}, B.nnz/B.n = {b}, (0.57,0.19,0.19,0.05)")
    return WORKLOADS[name]


def workload(name: str, values: str = "uniform"):
    """Return (A, B) for one of the named workloads (B is A for the A*A cases);
    rmat_pair_s<S>_a<A>_b<B> names an independent R-MAT pair (rmat_pair)."""
    if name.startswith("rmat_pair_"):
        s, a, b = (int(x[1:]) for x in name[len("rmat_pair_"):].split("_"))
        return rmat_pair(s, a, b)
    if name == "rmat10_ef8":
        A = rmat(10, 8, seed=1, value_seed=101, values=values)
        return A, A
    if name == "banded_n1M_17diag":
        A = banded(1 << 20, 8, value_seed=102, values=values)
        return A, A
    if name == "rmat18_ef16":
        A = rmat(18, 16, seed=3, value_seed=103, values=values)
        return A, A
    if name == "rmat20_ef8":
        A = rmat(20, 8, seed=4, value_seed=104, values=values)
        return A, A
    if name == "rect_zipf2.1_x_uniform16":
        lens = zipf_lengths(1 << 20, 2.1, 65536, seed=5)
        A = distinct_uniform_rows(lens, 1 << 18, seed=5, value_seed=105, values=values)
        B = distinct_uniform_rows(np.full(1 << 18, 16, dtype=np.int64), 1 << 20, seed=6,
                                  value_seed=106, values=values)
        return A, B
    raise KeyError(name)
