"""CPU oracle for C = A*B (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package. The GPU library never calls it.
It shares no code with the HIP path: the product is computed by ``oracle.c``
(plain C, threads over rows, long-double sums), and the stage helpers in
``stages.py`` are plain numpy.

Every function here is pinned by ``tests/test_oracle.py`` against values the
gMAGNUS page prints for its worked example (Figure 1), closed forms, exact
integer arithmetic, dense products and library routines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (returns the path)."""
    src = os.path.join(_HERE, "oracle.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-o", tmp, src])
        os.replace(tmp, _SO)
    return _SO


class _Result(ctypes.Structure):
    _fields_ = [("nsel", ctypes.c_int64), ("nnz", ctypes.c_int64),
                ("rowptr", ctypes.POINTER(ctypes.c_int64)),
                ("col", ctypes.POINTER(ctypes.c_int32)),
                ("val", ctypes.POINTER(ctypes.c_double)),
                ("abssum", ctypes.POINTER(ctypes.c_double)),
                ("u", ctypes.POINTER(ctypes.c_int64))]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        lib.oracle_spgemm_rows.argtypes = [ctypes.c_int64, ctypes.c_int64, P, P, P,
                                           ctypes.c_int64, ctypes.c_int64, P, P, P, P,
                                           ctypes.c_int64, ctypes.c_int, ctypes.POINTER(_Result)]
        lib.oracle_spgemm_rows.restype = ctypes.c_int
        lib.oracle_free.argtypes = [ctypes.POINTER(_Result)]
        lib.oracle_free.restype = None
        lib.oracle_row_products.argtypes = [ctypes.c_int64, P, P, P, P]
        lib.oracle_row_products.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def row_products(A, B) -> np.ndarray:
    """u(i) = sum over k in row i of A of nnz(B[k,:]) for every row of A."""
    lib = _load()
    out = np.zeros(A.nrows, dtype=np.int64)
    arp = np.ascontiguousarray(A.rowptr)
    acol = np.ascontiguousarray(A.col)
    brp = np.ascontiguousarray(B.rowptr)
    lib.oracle_row_products(A.nrows, _ptr(arp), _ptr(acol), _ptr(brp), _ptr(out))
    return out


class OracleRows:
    """Rows ``rows`` of C = A*B: CSR arrays over the selected rows plus per-entry abssum."""

    def __init__(self, rows, rowptr, col, val, abssum, u):
        self.rows, self.rowptr, self.col, self.val, self.abssum, self.u = (
            rows, rowptr, col, val, abssum, u)

    @property
    def nnz(self) -> int:
        return int(self.rowptr[-1])

    def row(self, x: int):
        s, e = int(self.rowptr[x]), int(self.rowptr[x + 1])
        return self.col[s:e], self.val[s:e], self.abssum[s:e]


def spgemm_rows(A, B, rows=None, nthreads: int | None = None) -> OracleRows:
    """Compute the listed rows of C = A*B (all rows when ``rows`` is None)."""
    if A.ncols != B.nrows:
        raise ValueError("inner dimensions differ")
    lib = _load()
    if rows is None:
        rows = np.arange(A.nrows, dtype=np.int64)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    arrs = [np.ascontiguousarray(x) for x in (A.rowptr, A.col, A.val, B.rowptr, B.col, B.val)]
    res = _Result()
    rc = lib.oracle_spgemm_rows(A.nrows, A.ncols, *[_ptr(x) for x in arrs[:3]],
                                B.nrows, B.ncols, *[_ptr(x) for x in arrs[3:]],
                                _ptr(rows), rows.size, int(nthreads), ctypes.byref(res))
    if rc != 0:
        raise RuntimeError(f"oracle_spgemm_rows failed ({rc})")
    try:
        nsel, nnz = int(res.nsel), int(res.nnz)
        rowptr = np.ctypeslib.as_array(res.rowptr, shape=(nsel + 1,)).copy()
        u = np.ctypeslib.as_array(res.u, shape=(max(nsel, 1),))[:nsel].copy()
        if nnz:
            col = np.ctypeslib.as_array(res.col, shape=(nnz,)).copy()
            val = np.ctypeslib.as_array(res.val, shape=(nnz,)).copy()
            absum = np.ctypeslib.as_array(res.abssum, shape=(nnz,)).copy()
        else:
            col = np.zeros(0, np.int32)
            val = np.zeros(0, np.float64)
            absum = np.zeros(0, np.float64)
    finally:
        lib.oracle_free(ctypes.byref(res))
    return OracleRows(rows, rowptr, col, val, absum, u)


def spgemm(A, B, nthreads: int | None = None):
    """All of C = A*B as (rowptr int64, col int32, val f64, abssum f64)."""
    r = spgemm_rows(A, B, None, nthreads)
    return r.rowptr, r.col, r.val, r.abssum


def structural_stats(u: np.ndarray, nnz_c: int) -> dict:
    """The operator-induced features of the SparseDitto page (Section 3.1):
    total, maximum, 95th percentile and coefficient of variation of u(i), the
    accumulator-fit fractions F_h = (1/m) * #{i : u(i) <= h} for h = 512, 4K
    and 32K (Eq. 5), and gamma = sum_i u(i) / nnz(C) (Eq. 6). m counts every
    row of A. The percentile is the nearest-rank one: the smallest value v
    with at least 95% of the rows at u(i) <= v. The CV is the population
    standard deviation over the mean (0 when the mean is 0).
    """
    u = np.asarray(u, dtype=np.int64)
    m = u.size
    total = int(u.sum())
    out = {"sum": total, "max": int(u.max()) if m else 0}
    if m == 0:
        out.update(p95=0, cv=0.0, f=[0.0, 0.0, 0.0], gamma=0.0)
        return out
    srt = np.sort(u)
    rank = -(-95 * m // 100)  # ceil(0.95 m), 1-based
    out["p95"] = int(srt[rank - 1])
    mean = total / m
    dev = u.astype(np.float64) - mean
    out["cv"] = float(np.sqrt(np.mean(dev * dev)) / mean) if mean > 0 else 0.0
    out["f"] = [float(np.count_nonzero(u <= h)) / m for h in (512, 4096, 32768)]
    out["gamma"] = total / nnz_c if nnz_c > 0 else 0.0
    return out
