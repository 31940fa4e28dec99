"""Oracle for the intermediate stages of the heavy-row path (TEST INFRASTRUCTURE ONLY).

These follow the gMAGNUS page, Section III-A and Figure 1:

* the intermediate matrix C-hat holds, for each heavy row i, every product
  (j, A[i,k]*B[k,j]) of that row, one entry per product; its row length is
  u(i) (Section III-B builds it by outer product, Eq. 2; which product lands
  where inside a row is free, so the oracle returns rows in Gustavson
  emission order and tests compare multisets or that order where the path
  fixes it);
* a multisplit level with chunk width W cuts a row (or a heavy chunk) into
  the column ranges [c*W, (c+1)*W); the chunk is the row's entries in that
  range, and elements inside a chunk are unordered (Section III-A, III-C);
* the reordered matrix C-hat-reord has one row per (row, chunk) pair, e.g.
  two heavy rows cut into two chunks each give four rows (Figure 1).

Plain numpy; nothing here is shared with the GPU library.
"""
from __future__ import annotations

import numpy as np


def expand_row(A, B, i: int):
    """Products of row i of A*B in emission order: (cols int32, prods f64)."""
    cols, prods = [], []
    for q in range(int(A.rowptr[i]), int(A.rowptr[i + 1])):
        k = int(A.col[q])
        s, e = int(B.rowptr[k]), int(B.rowptr[k + 1])
        cols.append(B.col[s:e])
        prods.append(A.val[q] * B.val[s:e])
    if not cols:
        return np.zeros(0, np.int32), np.zeros(0, np.float64)
    return np.concatenate(cols).astype(np.int32), np.concatenate(prods)


def expand(A, B, rows):
    """C-hat over ``rows`` (in the given order): rowptr int64, col int32, val f64."""
    parts = [expand_row(A, B, int(i)) for i in rows]
    rowptr = np.zeros(len(parts) + 1, dtype=np.int64)
    rowptr[1:] = np.cumsum([p[0].size for p in parts])
    col = np.concatenate([p[0] for p in parts]) if parts else np.zeros(0, np.int32)
    val = np.concatenate([p[1] for p in parts]) if parts else np.zeros(0, np.float64)
    return rowptr, col.astype(np.int32), val


def split_by_width(cols: np.ndarray, vals: np.ndarray, width: int, col_base: int, nchunks: int):
    """Cut one row's entries into ``nchunks`` column ranges of ``width`` starting at ``col_base``.

    Returns a list of (cols, vals) per chunk, each in the row's original order.
    """
    out = []
    for c in range(nchunks):
        lo, hi = col_base + c * width, col_base + (c + 1) * width
        m = (cols >= lo) & (cols < hi)
        out.append((cols[m], vals[m]))
    assert sum(x[0].size for x in out) == cols.size, "entries outside the row's range"
    return out


def chunk_counts(cols: np.ndarray, width: int, col_base: int, nchunks: int) -> np.ndarray:
    """Entries per chunk of one row (a histogram over the column ranges)."""
    return np.array([x[0].size for x in split_by_width(cols, np.zeros(cols.size), width,
                                                       col_base, nchunks)], dtype=np.int64)


def distinct_per_chunk(cols: np.ndarray, width: int, col_base: int, nchunks: int) -> np.ndarray:
    """Distinct columns per chunk: the symbolic count of each chunk's output."""
    return np.array([np.unique(x[0]).size for x in split_by_width(
        cols, np.zeros(cols.size), width, col_base, nchunks)], dtype=np.int64)
