"""Shared helpers for the GPU parity tests: run the HIP path, compare with the oracle."""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

import oracle
from spgemm_irregular_matrices_amd import synth

BOUND = 1e-12  # |c_gpu - c_ref| <= BOUND * sum|a_ik * b_kj| for every entry


def gather_ranges(starts: np.ndarray, lens: np.ndarray) -> np.ndarray:
    """Concatenation of arange(starts[i], starts[i]+lens[i]) over i (vectorised)."""
    starts = np.asarray(starts, dtype=np.int64)
    lens = np.asarray(lens, dtype=np.int64)
    total = int(lens.sum())
    if total == 0:
        return np.zeros(0, dtype=np.int64)
    excl = np.cumsum(lens) - lens
    return np.repeat(starts - excl, lens) + np.arange(total, dtype=np.int64)


def run_gpu(A, B, **plan_kwargs):
    """C = A*B on the GPU through the C ABI; returns host arrays and the plan's stats."""
    import torch
    from spgemm_irregular_matrices_amd import binding

    dA = binding.DeviceCSR.from_host(A)
    dB = dA if B is A else binding.DeviceCSR.from_host(B)
    with binding.Plan(**plan_kwargs) as p:
        C = p.multiply(dA, dB)
        torch.cuda.synchronize()
        stats = p.stats()
    return (C.rowptr.cpu().numpy(), C.col.cpu().numpy(), C.val.cpu().numpy(), stats)


def compare(A, B, rp, col, val, rows=None, nthreads=None, check_all_rowptr=True,
            exact_values=False):
    """Check GPU output rows against the oracle; returns the worst error ratio.

    Structure must match bit for bit; each value must sit within
    BOUND * abssum of the oracle's (or equal it when ``exact_values``).
    """
    n = A.nrows
    assert rp.shape == (n + 1,) and rp[0] == 0
    assert np.all(np.diff(rp) >= 0)
    assert col.shape == val.shape == (int(rp[-1]),)
    assert not np.any(np.isnan(val)) and not np.any(np.isinf(val))
    if rows is None:
        rows = np.arange(n, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    ref = oracle.spgemm_rows(A, B, rows, nthreads=nthreads)
    glen = rp[rows + 1] - rp[rows]
    rlen = np.diff(ref.rowptr)
    bad = np.nonzero(glen != rlen)[0]
    assert bad.size == 0, f"row lengths differ at rows {rows[bad[:10]]}: gpu {glen[bad[:10]]} ref {rlen[bad[:10]]}"
    gi = gather_ranges(rp[rows], glen)
    gcol = col[gi]
    gval = val[gi]
    badc = np.nonzero(gcol != ref.col)[0]
    assert badc.size == 0, f"{badc.size} column mismatches, first at entry {badc[0]}"
    err = np.abs(gval - ref.val)
    if exact_values:
        badv = np.nonzero(err != 0)[0]
        assert badv.size == 0, f"{badv.size} inexact values (first err {err[badv[0]]})"
        worst = 0.0
    else:
        lim = BOUND * ref.abssum
        badv = np.nonzero(err > lim)[0]
        assert badv.size == 0, (f"{badv.size} values outside the bound, first: gpu {gval[badv[0]]} "
                                f"ref {ref.val[badv[0]]} abssum {ref.abssum[badv[0]]}")
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = np.where(lim > 0, err / np.where(lim > 0, lim, 1), 0.0)
        worst = float(ratio.max()) if ratio.size else 0.0
    if check_all_rowptr and rows.size == n:
        assert np.array_equal(rp[1:], np.cumsum(rlen))
    return worst


def sample_rows(A, B, n_heavy=8, n_random=200, seed=0, tau=6826):
    """Row sample for full-size checks: the heaviest rows, rows near tau and random rows."""
    u = oracle.row_products(A, B)
    order = np.argsort(-u, kind="stable")
    heavy = order[:n_heavy]
    near = np.nonzero((u > tau * 0.8) & (u < tau * 1.5))[0][:n_heavy]
    rnd = (synth.splitmix64(seed, np.arange(n_random, dtype=np.uint64)) % np.uint64(A.nrows)).astype(np.int64)
    rows = np.unique(np.concatenate([heavy, near, rnd, [0, A.nrows - 1]]))
    return rows.astype(np.int64), u


BLOCK_PRODUCTS = 1 << 27  # oracle work per row block of compare_every_row


def oracle_threads() -> int:
    """Host threads for the oracle: the cores this process may use, at most 16
    (a one-GPU machine gives a process 16 threads whatever the mask shows)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def row_blocks(u, r0, r1):
    """Consecutive row blocks of [r0, r1) with about BLOCK_PRODUCTS products each."""
    cu = np.cumsum(u[r0:r1], dtype=np.int64)
    out = []
    a = 0
    n = r1 - r0
    while a < n:
        base = int(cu[a - 1]) if a else 0
        b = int(np.searchsorted(cu, base + BLOCK_PRODUCTS, side="right"))
        b = max(b, a + 1)
        out.append((r0 + a, r0 + min(b, n)))
        a = b
    return out


def _check_piece(gcol, gval, rcol, rval, rabs):
    """(columns equal, index of the first value outside the bound or -1)."""
    if not np.array_equal(gcol, rcol):
        return False, -1
    ok = np.abs(gval - rval) <= BOUND * rabs  # NaN or Inf fails
    if ok.all():
        return True, -1
    return True, int(np.argmin(ok))


def _compare_block(pool, res, ref, r0, r1):
    rp = res["rp"]
    C = res["C"]
    glen = np.diff(rp[r0:r1 + 1])
    rlen = np.diff(ref.rowptr)
    bad = np.nonzero(glen != rlen)[0]
    assert bad.size == 0, (f"[{res['label']}] row lengths differ at rows {r0 + bad[:10]}: "
                           f"gpu {glen[bad[:10]]} oracle {rlen[bad[:10]]}")
    s, e = int(rp[r0]), int(rp[r1])
    gcol = C.col[s:e].cpu().numpy()
    gval = C.val[s:e].cpu().numpy()
    nn = e - s
    cuts = np.linspace(0, nn, num=min(oracle_threads(), max(1, nn // (1 << 16))) + 1).astype(np.int64)
    futs = [pool.submit(_check_piece, gcol[a:b], gval[a:b], ref.col[a:b], ref.val[a:b],
                        ref.abssum[a:b]) for a, b in zip(cuts[:-1], cuts[1:])]
    for a, f in zip(cuts[:-1], futs):
        cols_ok, first_bad = f.result()
        if not cols_ok:
            j = a + int(np.argmax(gcol[a:] != ref.col[a:]))
            row = r0 + int(np.searchsorted(ref.rowptr, j, side="right")) - 1
            raise AssertionError(f"[{res['label']}] column mismatch at row {row}: gpu {gcol[j]} "
                                 f"oracle {ref.col[j]}")
        if first_bad >= 0:
            j = a + first_bad
            row = r0 + int(np.searchsorted(ref.rowptr, j, side="right")) - 1
            raise AssertionError(f"[{res['label']}] value outside the bound at row {row} col "
                                 f"{gcol[j]}: gpu {gval[j]!r} oracle {ref.val[j]!r} "
                                 f"abssum {ref.abssum[j]!r}")


def compare_every_row(A, B, results, u, r0=0, r1=None):
    """Rows [r0, r1) of every GPU result against one oracle pass, in row blocks.

    results: dicts with "label", "C" (the product on the device: col and val
    tensors) and "rp" (its row pointers on the host). Row lengths and columns
    must match bit for bit; values within BOUND * abssum.
    """
    if r1 is None:
        r1 = A.nrows
    nthr = oracle_threads()
    with cf.ThreadPoolExecutor(max_workers=nthr) as pool:
        for a, b in row_blocks(u, r0, r1):
            ref = oracle.spgemm_rows(A, B, np.arange(a, b, dtype=np.int64), nthreads=nthr)
            for res in results:
                _compare_block(pool, res, ref, a, b)
            del ref
