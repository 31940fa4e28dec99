"""GPU parity at the benchmark workloads' full sizes, every row of C.

Each workload runs through the C ABI in the launch configuration bench.py
times (default plan options, numeric path 3), and again with the gMAGNUS
page's own dataflow (numeric path 2: outer product into C-hat, the
hierarchical multisplit, dense accumulation of the chunks; Alg. 3-5,
Sec. III-B/C). The 2^18 R-MAT square runs the page's dataflow in one batch,
so C-hat positions pass 2^31, and also with the fused first level (path 1);
the 2^20 R-MAT square runs it in row batches of at most 2^31 - 1 products.

The oracle then computes every row in row blocks balanced by intermediate
products, and each block is compared with every GPU result: row lengths and
columns bit for bit, every value within 1e-12 * sum|a*b| of its entry. The
large workloads are split into several tests so that each one reports within
a minute or so.
"""
import numpy as np
import pytest

import oracle
from spgemm_irregular_matrices_amd import synth
from tests.helpers import compare, compare_every_row, oracle_threads

pytestmark = pytest.mark.gpu

BATCH_2G = (1 << 31) - 1

# workload -> (label, plan options, numeric path that must have run, batches)
RUNS = {
    "rmat18_ef16": [
        ("default", {}, 3, 1),
        ("page_dataflow_one_batch", {"numeric_mode": 2}, 2, 1),
        ("fused_first_level", {"numeric_mode": 1}, 1, 1),
    ],
    "rmat20_ef8": [
        ("default", {}, 3, 1),
        ("page_dataflow_batched", {"numeric_mode": 2, "max_batch_products": BATCH_2G}, 2, 3),
    ],
    "rect_zipf2.1_x_uniform16": [
        ("default", {}, 3, 1),
        ("page_dataflow_one_batch", {"numeric_mode": 2}, 2, 1),
    ],
}
PARTS = {"rmat18_ef16": 4, "rmat20_ef8": 8, "rect_zipf2.1_x_uniform16": 1}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    from spgemm_irregular_matrices_amd import binding
    binding.load()


def _multiply(A, B, **plan_kwargs):
    import torch
    from spgemm_irregular_matrices_amd import binding
    dA = binding.DeviceCSR.from_host(A)
    dB = dA if B is A else binding.DeviceCSR.from_host(B)
    with binding.Plan(**plan_kwargs) as p:
        C = p.multiply(dA, dB)
        torch.cuda.synchronize()
        st = p.stats()
    del dA, dB
    return C, st


def _bucket_upper(v: int) -> int:
    """Upper end of the stats record's u-histogram bucket holding v: exact
    below 64, then 64 buckets per octave."""
    if v < 64:
        return v
    e = v.bit_length() - 1
    f = (v >> (e - 6)) & 63
    return ((64 + f + 1) << (e - 6)) - 1


def _check_structural_stats(st, u):
    """The stats record's structural statistics against the oracle's, on all rows."""
    ref = oracle.structural_stats(u, st["nnz_c"])
    assert st["sum_products"] == ref["sum"] and st["max_products"] == ref["max"]
    assert st["u_p95"] == _bucket_upper(ref["p95"])
    assert st["u_cv"] == pytest.approx(ref["cv"], rel=1e-9, abs=1e-12)
    assert st["f_u_le"] == ref["f"]
    assert st["gamma"] == ref["gamma"]


def test_rmat10_all_rows():
    A, B = synth.workload("rmat10_ef8")
    C, st = _multiply(A, B)
    compare(A, B, C.rowptr.cpu().numpy(), C.col.cpu().numpy(), C.val.cpu().numpy())
    _check_structural_stats(st, oracle.row_products(A, B))


def test_banded_1M_all_rows():
    A, B = synth.workload("banded_n1M_17diag")
    C, st = _multiply(A, B)
    n = A.nrows
    assert st["heavy_rows"] == 0
    assert st["nnz_c"] == 33 * n - 272
    rp = C.rowptr.cpu().numpy()
    i = np.arange(n)
    exp = np.minimum(n - 1, i + 16) - np.maximum(0, i - 16) + 1
    assert np.array_equal(np.diff(rp), exp)
    compare(A, B, rp, C.col.cpu().numpy(), C.val.cpu().numpy(), nthreads=oracle_threads())
    _check_structural_stats(st, oracle.row_products(A, B))


# ---------------------------------------------------------------- large workloads
_cache: dict = {}


def _workload_results(name):
    """Inputs, u(i) and every GPU result of one workload (kept while its parts run)."""
    import torch
    if _cache.get("name") != name:
        _cache.clear()
        torch.cuda.empty_cache()
        A, B = synth.workload(name)
        u = oracle.row_products(A, B)
        res = []
        for label, kw, path, nbatches in RUNS[name]:
            C, st = _multiply(A, B, **kw)
            res.append({"label": label, "C": C, "rp": C.rowptr.cpu().numpy(), "st": st,
                        "path": path, "nbatches": nbatches})
            torch.cuda.empty_cache()
        _cache.update(name=name, A=A, B=B, u=u, cu=np.cumsum(u), res=res)
    return _cache


def _part_rows(cu, parts, k):
    """Rows [r0, r1) of part k of `parts`, balanced by intermediate products."""
    n = cu.size
    tot = int(cu[-1]) if n else 0
    b = [0] + [int(np.searchsorted(cu, tot * j // parts, side="right")) for j in range(1, parts)] + [n]
    return b[k], max(b[k], b[k + 1])


CASES = [(name, k) for name in RUNS for k in range(PARTS[name])]


@pytest.mark.parametrize("name,part", CASES, ids=[f"{n}-part{k}" for n, k in CASES])
def test_large_every_row(name, part):
    w = _workload_results(name)
    A, B, u = w["A"], w["B"], w["u"]
    for res in w["res"]:
        st = res["st"]
        assert st["numeric_path"] == res["path"], (res["label"], st["numeric_path"])
        if res["nbatches"] == 1:
            assert st["nbatches"] == 1, (res["label"], st["nbatches"])
        else:
            assert st["nbatches"] >= res["nbatches"], (res["label"], st["nbatches"])
        assert st["sum_products"] == int(u.sum())
        assert st["heavy_rows"] > 0
        assert st["heavy_products"] == int(u[u > st["tau"]].sum())
        rp = res["rp"]
        assert rp[0] == 0 and rp[-1] == st["nnz_c"]
    if part == 0:
        # the results agree on C's size; the stats record's statistics hold
        nnz = {r["st"]["nnz_c"] for r in w["res"]}
        assert len(nnz) == 1, nnz
        _check_structural_stats(w["res"][0]["st"], u)
        if name == "rmat18_ef16":
            # one batch of the page's dataflow holds more than 2^31 products
            assert w["res"][1]["st"]["heavy_products"] > (1 << 31)
        if name == "rmat20_ef8":
            assert w["res"][0]["st"]["nnz_c"] > (1 << 31)
    r0, r1 = _part_rows(w["cu"], PARTS[name], part)
    compare_every_row(A, B, w["res"], u, r0, r1)
    if part == PARTS[name] - 1:
        _cache.clear()
