"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Structure (row pointers and columns) must match bit for bit; every value
must be within 1e-12 * sum|a*b| of the oracle's long-double sum, or equal
to it for small-integer inputs where every partial sum is exact. Forced
parameters (tau, final chunk width, chunks per level) push small inputs
through the heavy path with one to five multisplit levels, so every kernel
runs at sizes the oracle checks in seconds.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import stages
from spgemm_irregular_matrices_amd import synth
from tests.helpers import compare, run_gpu

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    from spgemm_irregular_matrices_amd import binding
    binding.load()


def _rmat10():
    return synth.workload("rmat10_ef8")[0]


def test_rmat10_default_and_all_light():
    A = _rmat10()
    rp, col, val, st = run_gpu(A, A)
    compare(A, A, rp, col, val)
    rp, col, val, st = run_gpu(A, A, tau_override=6000)  # max u of this matrix is 4557
    assert st["heavy_rows"] == 0
    compare(A, A, rp, col, val)


# (symbolic, numeric) modes: fused bitmap symbolic or multisplit symbolic;
# products formed inside the first multisplit level, a separate C-hat, or
# direct accumulation from A and the chunk-split B
MODES = [(1, 1), (2, 2), (1, 2), (1, 3)]


def _expected_path(mode, nlevels):
    if mode[1] == 3:
        return 3
    return 1 if mode[1] == 1 and nlevels > 0 else 2


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("tau,width,cap,levels", [
    (64, 0, 0, 0),        # heavy rows accumulate densely without any multisplit
    (64, 256, 32, 1),     # one level of 4 chunks
    (64, 64, 4, 2),       # 16 chunks over two levels
    (16, 32, 2, 5),       # 32 chunks over five levels of 2
    (200, 128, 8, 1),
])
def test_rmat10_forced_heavy(tau, width, cap, levels, mode):
    A = _rmat10()
    rp, col, val, st = run_gpu(A, A, tau_override=tau, chunk_width_override=width,
                               nchunks_cap=cap, symbolic_mode=mode[0], numeric_mode=mode[1])
    assert st["heavy_rows"] > 0
    assert st["nlevels"] == levels, st
    assert st["numeric_path"] == _expected_path(mode, levels)
    compare(A, A, rp, col, val)


def _power_law_rows(p=1 << 17):
    """Rows far above the symbolic pass's per-work-group share: 128K, 48K and
    24K products, plus a 3-entry row whose first B row holds 60,000 entries
    (split into three parts by product range, the middle one empty). With
    p = 2^19 columns the row bitmap no longer lets two work groups share a
    CU, so the symbolic pass also takes the columns in parts."""
    n, m = 3000, 1 << 15
    lens = synth.zipf_lengths(n, 2.1, 20, seed=61)
    lens[:4] = [8000, 3000, 1500, 3]
    A = synth.distinct_uniform_rows(lens, m, seed=62, value_seed=63)
    blens = np.full(m, 16, dtype=np.int64)
    c = A.col[A.rowptr[3]:A.rowptr[4]]
    blens[c[0]], blens[c[1]], blens[c[2]] = 60000, 1, 1
    B = synth.distinct_uniform_rows(blens, p, seed=64, value_seed=65)
    return A, B


@pytest.mark.parametrize("cols", [1 << 17, 1 << 19])
@pytest.mark.parametrize("mode", MODES)
def test_power_law_rows_split_over_work_groups(mode, cols):
    A, B = _power_law_rows(cols)
    u = oracle.row_products(A, B)
    assert u[0] == 128000 and u[3] == 60002
    rp, col, val, st = run_gpu(A, B, symbolic_mode=mode[0], numeric_mode=mode[1])
    assert st["heavy_rows"] >= 4 and st["max_products"] == int(u.max())
    compare(A, B, rp, col, val)


def _thread_bin_rows():
    """Rows at and around the thread-local bin bounds (u = 8, 16, 32), with
    entries on empty B rows, repeated columns across entries, and a row whose
    products all fall in one column; small integer values, so sums are exact."""
    m, p = 64, 40
    rng = np.random.default_rng(71)
    brows = [[] for _ in range(m)]
    for k in range(1, m):
        ln = [1, 3, 5, 8, 16][k % 5]
        brows[k] = sorted(rng.choice(p, size=ln, replace=False).tolist())
    brows[7] = []            # another empty B row
    brows[9] = [5]           # single column 5
    brows[11] = [5]
    arows = []
    for target in (1, 7, 8, 9, 15, 16, 17, 31, 32, 33):
        row, u = [0], 0      # entry on the empty B row 0 first
        for k in rng.permutation(np.arange(1, m)):
            ln = len(brows[k])
            if ln and u + ln <= target:
                row.append(int(k))
                u += ln
            if u == target:
                break
        row.insert(len(row) // 2, 7)
        arows.append(row)
    arows.append([9, 7])                       # one product
    arows.append([9, 0, 11, 7])                # two products in one column, empty rows between
    A0 = synth.from_rows(len(arows), m, arows)
    B0 = synth.from_rows(m, p, brows)
    A = synth.CSR(A0.nrows, m, A0.rowptr, A0.col, synth.small_int_values(72, A0.nnz))
    B = synth.CSR(m, p, B0.rowptr, B0.col, synth.small_int_values(73, B0.nnz))
    return A, B


def test_thread_local_bins_exact():
    A, B = _thread_bin_rows()
    u = oracle.row_products(A, B)
    assert {8, 9, 16, 17, 32, 33} <= set(u.tolist())
    rp, col, val, st = run_gpu(A, B)
    assert st["heavy_rows"] == 0
    compare(A, B, rp, col, val, exact_values=True)
    # all products in one column: a single output
    assert rp[-1] - rp[-2] == 1


def _class_bound_items():
    """Heavy rows whose (row, slot) items hold product counts at and around
    every bound of the direct path's item classes (64, 128, 256, 512, 1 K and
    2 K products, then the dense window): B row j holds targets[j] distinct
    columns inside slot j mod 8 of a 65,536-column range (eight slots of
    8192). Row i takes B rows i..i+7 (one per slot, so each item's count is
    one target); row 24 + i takes three B rows of one slot, whose columns
    overlap. The last rows take n single-column B rows of slot 0 each (n =
    100 ... 2100), so that their items stage their entries over several
    rounds of the teams (and repeat columns)."""
    W, req = 8192, 8
    targets = [1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512, 513,
               1023, 1024, 1025, 2047, 2048, 2049, 3000, 4095, 5000, 8192]
    nt = len(targets)
    rng = np.random.default_rng(81)
    brows = [sorted(((j % req) * W + rng.choice(W, size=L, replace=False)).tolist())
             for j, L in enumerate(targets)]
    many = (100, 300, 600, 1500, 2100)
    brows += [[int(c)] for c in rng.integers(0, W, size=max(many))]
    arows = [[(i + t) % nt for t in range(req)] for i in range(nt)]
    arows += [sorted({i, (i + req) % nt, (i + 2 * req) % nt}) for i in range(nt)]
    arows += [list(range(nt, nt + n)) for n in many]
    nb = len(brows)
    A0 = synth.from_rows(len(arows), nb, arows)
    B0 = synth.from_rows(nb, W * req, brows)
    A = synth.CSR(A0.nrows, nb, A0.rowptr, A0.col, synth.uniform_values(82, A0.nnz))
    B = synth.CSR(nb, W * req, B0.rowptr, B0.col, synth.uniform_values(83, B0.nnz))
    return A, B, targets


def test_direct_item_class_bounds():
    A, B, targets = _class_bound_items()
    rp, col, val, st = run_gpu(A, B, tau_override=16)
    assert st["numeric_path"] == 3 and st["final_chunk_width"] == 8192, st
    assert st["heavy_rows"] == A.nrows
    compare(A, B, rp, col, val)


@pytest.mark.parametrize("counts", [(5, 3, 1, 2, 3, 7), (1, 1, 1, 1, 1, 1), (4, 6, 2, 8, 6, 3)])
def test_rank_classes_with_partial_groups(counts):
    """A work group of a rank class takes several consecutive items (four in
    the two smallest classes, two in the others), so a class whose item count
    is not a multiple of that ends in a partly filled group. counts[c] heavy
    rows each hold one item of class c: a single B row of L distinct columns
    inside one slot (L = 40, 100, 200, 400, 900, 1800, one per class)."""
    W, req = 8192, 8
    sizes = (40, 100, 200, 400, 900, 1800)
    rng = np.random.default_rng(101)
    brows, arows = [], []
    for L, n in zip(sizes, counts):
        for _ in range(n):
            j = len(brows)
            brows.append(sorted(((j % req) * W + rng.choice(W, size=L, replace=False)).tolist()))
            arows.append([j])
    nb = len(brows)
    A0 = synth.from_rows(len(arows), nb, arows)
    B0 = synth.from_rows(nb, W * req, brows)
    A = synth.CSR(A0.nrows, nb, A0.rowptr, A0.col, synth.uniform_values(102, A0.nnz))
    B = synth.CSR(nb, W * req, B0.rowptr, B0.col, synth.uniform_values(103, B0.nnz))
    rp, col, val, st = run_gpu(A, B, tau_override=16)
    assert st["numeric_path"] == 3 and st["final_chunk_width"] == W, st
    assert st["heavy_rows"] == A.nrows
    compare(A, B, rp, col, val)


# (row pattern {slot: products}, one B row per product?) for the runs test
RUN_PATTERNS = [
    ({0: 5, 2: 7, 5: 9, 6: 3, 10: 2, 11: 1, 20: 4}, False),  # gaps, span breaks
    ({0: 60, 1: 50, 2: 30, 3: 100, 4: 128, 5: 1}, False),    # product cap breaks
    ({0: 10, 1: 200, 2: 10, 3: 10, 4: 3000, 5: 10}, False),  # larger items between
    ({s: 2 for s in range(9)}, True),                        # nine one-product slots
    ({s: 5 for s in range(8)}, True),                        # 40 entries x 8 slots
    ({0: 35, 3: 35}, True),                                  # 70 entries x 2 slots
    ({30: 4, 31: 23}, False),                                # the last slots
    ({s: 2 for s in range(16)}, False),                      # two full spans
]


def _run_rows(W, ncols, seed):
    """Heavy rows whose (row, slot) items hold given product counts: each
    item is formed by B rows whose distinct columns all lie in that slot
    (one product each when split, else at most W each), and one extra row
    of 20 entries whose B rows each hold a column in slots 0, 1 and 3."""
    rng = np.random.default_rng(seed)
    brows, arows = [], []
    for pat, split in RUN_PATTERNS:
        row = []
        for s, c in sorted(pat.items()):
            pieces = [1] * c if split else [min(W, c - i) for i in range(0, c, W)]
            for L in pieces:
                row.append(len(brows))
                brows.append(sorted((s * W + rng.choice(W, size=L, replace=False)).tolist()))
        arows.append(row)
    row = []
    for _ in range(20):
        row.append(len(brows))
        brows.append([int(s * W + rng.integers(W)) for s in (0, 1, 3)])
    arows.append(row)
    nb = len(brows)
    A0 = synth.from_rows(len(arows), nb, arows)
    B0 = synth.from_rows(nb, ncols, brows)
    A = synth.CSR(A0.nrows, nb, A0.rowptr, A0.col, synth.uniform_values(111, A0.nnz))
    B = synth.CSR(nb, ncols, B0.rowptr, B0.col, synth.uniform_values(112, B0.nnz))
    return A, B


@pytest.mark.parametrize("W", [64, 1024, 8192, 16384])
def test_runs_of_small_items(W):
    """The items of at most 128 products are accumulated in runs: a run holds
    a row's next small items while their products stay within 128, their
    slots within min(8, 65536 / W) of its first and no larger item lies
    between them. The rows cover runs with empty slots inside, breaks at the
    product cap, at the span and at larger items, and runs whose (entry, slot)
    pairs take several rounds; every row is heavy, over 32 slots of width W."""
    A, B = _run_rows(W, 32 * W, seed=110 + W)
    # a width of 16384 needs the whole 160 KiB of a CU's LDS for the window
    lds = 160 * 1024 if W > 8192 else 0
    rp, col, val, st = run_gpu(A, B, tau_override=16, chunk_width_override=W,
                               lds_budget_bytes=lds)
    assert st["numeric_path"] == 3 and st["final_chunk_width"] == W, st
    assert st["heavy_rows"] == A.nrows
    compare(A, B, rp, col, val)


@pytest.mark.parametrize("W", [8192, 16384])
def test_page_dataflow_chunk_classes(W):
    """The page's dataflow (outer product into C-hat, multisplit, chunk
    accumulation) with final chunks of 257-1024, 1025-2048 and more than
    tau = 2048 elements: the 256- and 512-thread rank teams and the chunk
    window. At W = 8192 both rank teams mark columns with byte flags in
    their value arrays; at W = 16384 the 256-thread team's flags no longer
    fit there and it sets the bitmap with atomic ORs."""
    ncols, nb = 4 * W, 2048
    B = synth.distinct_uniform_rows(np.full(nb, 30, dtype=np.int64), ncols, seed=121,
                                    value_seed=122)
    lens = np.array([100] * 20 + [200] * 20 + [400] * 5 + [3] * 50, dtype=np.int64)
    A = synth.distinct_uniform_rows(lens, nb, seed=123, value_seed=124)
    # products per (heavy row, final chunk): every class above is populated
    blen = np.diff(B.rowptr)
    sizes = []
    for i in range(A.nrows):
        ks = A.col[A.rowptr[i]:A.rowptr[i + 1]]
        cols = np.concatenate([B.col[B.rowptr[k]:B.rowptr[k + 1]] for k in ks])
        if blen[ks].sum() > 2048:
            sizes += np.bincount(cols // W, minlength=4).tolist()
    sizes = np.array(sizes)
    for lo, hi in ((256, 1024), (1024, 2048), (2048, 1 << 30)):
        assert ((sizes > lo) & (sizes <= hi)).any(), (lo, hi)
    lds = 160 * 1024 if W > 8192 else 0
    rp, col, val, st = run_gpu(A, B, tau_override=2048, chunk_width_override=W,
                               lds_budget_bytes=lds, numeric_mode=2)
    assert st["numeric_path"] == 2 and st["final_chunk_width"] == W, st
    assert st["heavy_rows"] == 45
    compare(A, B, rp, col, val)


def test_short_b_rows_over_many_slots():
    """B rows of 4 entries over 2^18 columns (32 slots): most (B row, slot)
    slices of a heavy row's items are empty, so the items test the slices'
    occupancy bits before reading their bounds."""
    lens = synth.zipf_lengths(3000, 2.1, 1200, seed=91)
    lens[:3] = [1200, 900, 700]
    A = synth.distinct_uniform_rows(lens, 4096, seed=92, value_seed=93)
    B = synth.distinct_uniform_rows(np.full(4096, 4, dtype=np.int64), 1 << 18, seed=94,
                                    value_seed=95)
    rp, col, val, st = run_gpu(A, B)
    assert st["numeric_path"] == 3 and st["heavy_rows"] >= 3, st
    compare(A, B, rp, col, val)


def test_multiply_in_one_call():
    """spgemm_multiply: with room for C, both phases in one call equal the
    two-call product; with too little room it returns CAPACITY with a valid
    row pointer and nnz, and a numeric call into right-sized buffers finishes."""
    import torch
    from spgemm_irregular_matrices_amd import binding
    A = synth.workload("rmat10_ef8")[0]
    dA = binding.DeviceCSR.from_host(A)
    with binding.Plan(tau_override=200) as p:
        ref = p.multiply(dA, dA)
        C, fit = p.multiply_once(dA, dA, capacity=int(ref.col.numel()) + 5)
        torch.cuda.synchronize()
        assert fit
        assert torch.equal(C.rowptr, ref.rowptr) and torch.equal(C.col, ref.col)
        compare(A, A, C.rowptr.cpu().numpy(), C.col.cpu().numpy(), C.val.cpu().numpy())
        C2, fit2 = p.multiply_once(dA, dA, capacity=10)
        assert not fit2 and C2.col.numel() == ref.col.numel()
        assert torch.equal(C2.rowptr, ref.rowptr)
        p.numeric(dA, dA, C2.rowptr, C2.col, C2.val)
        torch.cuda.synchronize()
        compare(A, A, C2.rowptr.cpu().numpy(), C2.col.cpu().numpy(), C2.val.cpu().numpy())
        with pytest.raises(binding.SpgemmError):
            p.multiply_once(dA, dA, capacity=-1)


def test_fig1_stages_and_product():
    with open(os.path.join(GOLDEN, "fig1_heavy_rows.json")) as f:
        g = json.load(f)
    na, ma = g["shape_A"]
    nb, mb = g["shape_B"]
    A0 = synth.from_rows(na, ma, [g["A_rows"].get(str(i), []) for i in range(na)])
    B0 = synth.from_rows(nb, mb, [g["B_rows"].get(str(i), []) for i in range(nb)])
    A = synth.CSR(na, ma, A0.rowptr, A0.col, synth.uniform_values(31, A0.nnz))
    B = synth.CSR(nb, mb, B0.rowptr, B0.col, synth.uniform_values(32, B0.nnz))
    import torch
    from spgemm_irregular_matrices_amd import binding
    dA, dB = binding.DeviceCSR.from_host(A), binding.DeviceCSR.from_host(B)
    # tau=2: rows 1 (7 products) and 2 (3 products) are heavy; width 4 over C.m=8
    # gives the figure's two chunks in one level (the window floor is 32, so
    # the chunk width is forced through the column range: see below)
    with binding.Plan(tau_override=2, chunk_width_override=32, debug_dump=True) as p:
        C = p.multiply(dA, dB)
        torch.cuda.synchronize()
        chat = p.debug(-1)
        st = p.stats()
    assert st["heavy_rows"] == 2
    # C-hat in the figure's order (Gustavson order inside each heavy row)
    assert chat["rowptr"].tolist() == g["C_hat"]["rowptr"]
    assert chat["col"].tolist() == g["C_hat"]["col"]
    assert chat["row_key"].tolist() == g["heavy_rows"]
    Ad, Bd = A.to_dense(), B.to_dense()
    exp_vals = [Ad[int(t[1]), int(t[2])] * Bd[int(t[4]), int(t[5])] for t in g["C_hat"]["val"]]
    assert chat["val"].tolist() == exp_vals  # one IEEE multiply each: bit-exact
    compare(A, B, C.rowptr.cpu().numpy(), C.col.cpu().numpy(), C.val.cpu().numpy())


def test_fig1_chunks_on_wider_columns():
    """The figure's chunking (two chunks per heavy row) on a column range of 64.

    Columns are scaled by 8 so that the figure's width-4 chunks become the
    width-32 chunks of the smallest dense window; the multisets of each
    (row, chunk) must be the figure's.
    """
    with open(os.path.join(GOLDEN, "fig1_heavy_rows.json")) as f:
        g = json.load(f)
    na, ma = g["shape_A"]
    nb, _ = g["shape_B"]
    scale = 8
    brows = [[c * scale for c in g["B_rows"].get(str(i), [])] for i in range(nb)]
    A0 = synth.from_rows(na, ma, [g["A_rows"].get(str(i), []) for i in range(na)])
    B0 = synth.from_rows(nb, 8 * scale, brows)
    A = synth.CSR(na, ma, A0.rowptr, A0.col, synth.uniform_values(33, A0.nnz))
    B = synth.CSR(nb, 8 * scale, B0.rowptr, B0.col, synth.uniform_values(34, B0.nnz))
    import torch
    from spgemm_irregular_matrices_amd import binding
    dA, dB = binding.DeviceCSR.from_host(A), binding.DeviceCSR.from_host(B)
    with binding.Plan(tau_override=2, chunk_width_override=32, nchunks_cap=2,
                      debug_dump=True) as p:
        C = p.multiply(dA, dB)
        torch.cuda.synchronize()
        lvl = p.debug(0)
        st = p.stats()
    assert st["nlevels"] == 1 and st["vchunks"] == [2]
    Ad, Bd = A.to_dense(), B.to_dense()
    got = {}
    for r in range(lvl["rowptr"].size - 1):
        key = int(lvl["row_key"][r])            # natural index: heavy row * 2 + chunk
        s, e = lvl["rowptr"][r], lvl["rowptr"][r + 1]
        got[key] = sorted(zip(((lvl["col"][s:e] % (4 * scale)) // scale).tolist(),
                              lvl["val"][s:e].tolist()))
    for k, (row, chunk) in enumerate(g["C_hat_reord"]["rows"]):
        h = g["heavy_rows"].index(row)
        vals = [Ad[int(t[1]), int(t[2])] * Bd[int(t[4]), int(t[5]) * scale]
                for t in g["C_hat_reord"]["val"][k]]
        assert got[h * 2 + chunk] == sorted(zip(g["C_hat_reord"]["local_col"][k], vals))
    compare(A, B, C.rowptr.cpu().numpy(), C.col.cpu().numpy(), C.val.cpu().numpy())


@pytest.mark.parametrize("numeric_mode", [2, 1])
def test_chat_stage_matches_oracle(numeric_mode):
    """C-hat rows are bit-exact against the oracle's expansion, in Gustavson order,
    and level 0 holds each heavy row's products split by column range.

    With the products formed inside the first multisplit level (numeric
    mode 1) C-hat is never written: its columns come from the multisplit
    symbolic pass and carry no values.
    """
    A = synth.random_csr(400, 300, seed=41, value_seed=42, mean_len=10, skew=1.2)
    B = synth.random_csr(300, 500, seed=43, value_seed=44, mean_len=8, skew=1.2)
    import torch
    from spgemm_irregular_matrices_amd import binding
    dA, dB = binding.DeviceCSR.from_host(A), binding.DeviceCSR.from_host(B)
    tau = 40
    with binding.Plan(tau_override=tau, chunk_width_override=64, nchunks_cap=2,
                      debug_dump=True, symbolic_mode=2, numeric_mode=numeric_mode) as p:
        C = p.multiply(dA, dB)
        torch.cuda.synchronize()
        levels = [p.debug(l) for l in range(p.stats()["nlevels"])]
        chat = p.debug(-1)
    u = oracle.row_products(A, B)
    rows = np.nonzero(u > tau)[0]
    rp, col, val = stages.expand(A, B, rows)
    assert np.array_equal(chat["row_key"], rows)
    assert np.array_equal(chat["rowptr"], rp)
    assert np.array_equal(chat["col"], col)
    if numeric_mode == 2:
        assert np.array_equal(chat["val"], val)
    else:
        assert chat["val"] is None
    # level 0: each chunk is its parent row's entries in that column range
    l0 = levels[0]
    W = l0["chunk_width"]
    nch = 512 // W  # B.ncols=500 rounds up to 512
    seen = 0
    for r in range(l0["rowptr"].size - 1):
        key = int(l0["row_key"][r])
        h, c = divmod(key, nch)
        s, e = rp[h], rp[h + 1]
        m = (col[s:e] >= c * W) & (col[s:e] < (c + 1) * W)
        exp = sorted(zip(col[s:e][m].tolist(), val[s:e][m].tolist()))
        a, b = l0["rowptr"][r], l0["rowptr"][r + 1]
        assert sorted(zip(l0["col"][a:b].tolist(), l0["val"][a:b].tolist())) == exp
        seen += b - a
    assert seen == rp[-1]
    compare(A, B, C.rowptr.cpu().numpy(), C.col.cpu().numpy(), C.val.cpu().numpy())


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("tau", [6826, 1, 20, 300])
@pytest.mark.parametrize("seed", [1, 2])
def test_random_skewed_paths(tau, seed, mode):
    A = synth.random_csr(600, 500, seed=seed, value_seed=seed + 10, mean_len=12, skew=1.1,
                         empty_frac=0.05)
    B = synth.random_csr(500, 700, seed=seed + 20, value_seed=seed + 30, mean_len=9, skew=1.1,
                         empty_frac=0.05)
    rp, col, val, st = run_gpu(A, B, tau_override=tau, chunk_width_override=32, nchunks_cap=4,
                               symbolic_mode=mode[0], numeric_mode=mode[1])
    compare(A, B, rp, col, val)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("budget,width,cap", [(1, 64, 4), (700, 64, 4), (5000, 32, 2), (20000, 0, 0)])
def test_row_batches(budget, width, cap, mode):
    """Heavy rows processed in batches of bounded products (one row per batch at
    budget 1). The direct path (numeric mode 3) builds no C-hat, so the budget
    does not apply to it: it runs one batch."""
    A = synth.rmat(11, 8, seed=121, value_seed=122)
    rp, col, val, st = run_gpu(A, A, tau_override=64, chunk_width_override=width, nchunks_cap=cap,
                               max_batch_products=budget, symbolic_mode=mode[0],
                               numeric_mode=mode[1])
    if st["numeric_path"] == 3:
        assert st["nbatches"] == 1
    else:
        assert st["nbatches"] > 1
    compare(A, A, rp, col, val)


def test_small_integer_values_exact():
    A = synth.rmat(11, 8, seed=61, value_seed=62, values="int")
    for mode in MODES:
        rp, col, val, st = run_gpu(A, A, tau_override=100, chunk_width_override=64, nchunks_cap=4,
                                   symbolic_mode=mode[0], numeric_mode=mode[1])
        assert st["heavy_rows"] > 0 and st["nlevels"] >= 2
        compare(A, A, rp, col, val, exact_values=True)
    rp, col, val, st = run_gpu(A, A)
    compare(A, A, rp, col, val, exact_values=True)


def test_banded_window_path():
    A = synth.banded(20000, 8, value_seed=71)
    rp, col, val, st = run_gpu(A, A)
    assert st["heavy_rows"] == 0
    assert rp[-1] == 33 * 20000 - 272
    compare(A, A, rp, col, val)
    Aw = synth.banded(3000, 200, value_seed=72)   # spans of 801 columns: the larger window
    rp, col, val, st = run_gpu(Aw, Aw, tau_override=8191)
    compare(Aw, Aw, rp, col, val)


def test_banded_forced_heavy():
    A = synth.banded(4096, 8, value_seed=73)
    rp, col, val, st = run_gpu(A, A, tau_override=100, chunk_width_override=32, nchunks_cap=8)
    assert st["heavy_rows"] > 0
    compare(A, A, rp, col, val)


def test_edge_cases():
    from spgemm_irregular_matrices_amd import binding
    # no rows
    E = synth.CSR(0, 5, np.zeros(1, np.int64), np.zeros(0, np.int32), np.zeros(0))
    B = synth.random_csr(5, 7, seed=81, value_seed=82, mean_len=2)
    rp, col, val, _ = run_gpu(E, B)
    assert rp.tolist() == [0] and col.size == 0
    # inner dimension zero
    A0 = synth.CSR(4, 0, np.zeros(5, np.int64), np.zeros(0, np.int32), np.zeros(0))
    B0 = synth.CSR(0, 6, np.zeros(1, np.int64), np.zeros(0, np.int32), np.zeros(0))
    rp, col, val, _ = run_gpu(A0, B0)
    assert rp.tolist() == [0] * 5
    # 1x1
    one = synth.CSR(1, 1, np.array([0, 1], np.int64), np.array([0], np.int32), np.array([-3.0]))
    rp, col, val, _ = run_gpu(one, one)
    assert col.tolist() == [0] and val.tolist() == [9.0]
    # rank one, forced heavy
    x = synth.random_csr(50, 1, seed=83, value_seed=84, mean_len=1)
    y = synth.random_csr(1, 3000, seed=85, value_seed=86, mean_len=1500)
    for kw in ({}, {"tau_override": 10, "chunk_width_override": 64, "nchunks_cap": 4}):
        rp, col, val, _ = run_gpu(x, y, **kw)
        compare(x, y, rp, col, val)
    # empty rows everywhere
    A = synth.random_csr(300, 200, seed=87, value_seed=88, mean_len=6, empty_frac=0.6)
    Bm = synth.random_csr(200, 260, seed=89, value_seed=90, mean_len=6, empty_frac=0.6)
    for kw in ({}, {"tau_override": 3, "chunk_width_override": 32, "nchunks_cap": 2}):
        rp, col, val, _ = run_gpu(A, Bm, **kw)
        compare(A, Bm, rp, col, val)
    # cancellation zeros stay in the structure
    Ac = synth.from_rows(1, 2, [[0, 1]], [[1.0, 1.0]])
    Bc = synth.from_rows(2, 3, [[0, 2], [0]], [[2.5, 1.0], [-2.5]])
    rp, col, val, _ = run_gpu(Ac, Bc)
    assert rp.tolist() == [0, 2] and col.tolist() == [0, 2] and val.tolist() == [0.0, 1.0]


def test_rectangular_and_unsorted_input_columns():
    A = synth.random_csr(700, 90, seed=91, value_seed=92, mean_len=20, skew=1.3)
    B = synth.random_csr(90, 3000, seed=93, value_seed=94, mean_len=60, skew=1.3)
    # shuffle columns inside every row of A and B: the product must not care
    for M, sd in ((A, 95), (B, 96)):
        keys = synth.splitmix64(sd, np.arange(M.nnz, dtype=np.uint64))
        rows = np.repeat(np.arange(M.nrows), np.diff(M.rowptr))
        order = np.lexsort((keys, rows))
        M.col = M.col[order].copy()
        M.val = M.val[order].copy()
    for kw in ({}, {"tau_override": 200, "chunk_width_override": 128, "nchunks_cap": 4}):
        rp, col, val, _ = run_gpu(A, B, **kw)
        compare(A, B, rp, col, val)


def test_numeric_rerun_with_new_values_and_determinism():
    import torch
    from spgemm_irregular_matrices_amd import binding
    A = synth.rmat(11, 8, seed=101, value_seed=102)
    A2 = synth.CSR(A.nrows, A.ncols, A.rowptr, A.col, synth.uniform_values(103, A.nnz))
    dA = binding.DeviceCSR.from_host(A)
    dA2 = binding.DeviceCSR.from_host(A2)
    with binding.Plan(tau_override=80, chunk_width_override=64, nchunks_cap=4) as p:
        rp, nnz = p.symbolic(dA, dA)
        col = torch.empty(nnz, dtype=torch.int32, device="cuda")
        val = torch.empty(nnz, dtype=torch.float64, device="cuda")
        p.numeric(dA, dA, rp, col, val)
        torch.cuda.synchronize()
        compare(A, A, rp.cpu().numpy(), col.cpu().numpy(), val.cpu().numpy())
        p.numeric(dA2, dA2, rp, col, val)   # same structure, new values
        torch.cuda.synchronize()
        compare(A2, A2, rp.cpu().numpy(), col.cpu().numpy(), val.cpu().numpy())
        first = (rp.cpu().numpy().copy(), col.cpu().numpy().copy())
        for _ in range(5):
            rp2, nnz2 = p.symbolic(dA, dA)
            p.numeric(dA, dA, rp2, col, val)
            torch.cuda.synchronize()
            assert nnz2 == nnz
            assert np.array_equal(rp2.cpu().numpy(), first[0])
            assert np.array_equal(col.cpu().numpy(), first[1])


def test_error_paths():
    import torch
    from spgemm_irregular_matrices_amd import binding
    A = synth.random_csr(50, 40, seed=111, value_seed=112, mean_len=4)
    B = synth.random_csr(30, 60, seed=113, value_seed=114, mean_len=4)
    dA, dB = binding.DeviceCSR.from_host(A), binding.DeviceCSR.from_host(B)
    with binding.Plan() as p:
        with pytest.raises(binding.SpgemmError) as e:
            p.symbolic(dA, dB)
        assert e.value.code == -2
        rp = torch.zeros(51, dtype=torch.int64, device="cuda")
        with pytest.raises(binding.SpgemmError) as e:
            p.numeric(dA, dA, rp, None, None)
        assert e.value.code in (-8, -6)
    # out-of-range column is caught by validation before any kernel uses it
    Bb = synth.random_csr(40, 60, seed=115, value_seed=116, mean_len=4)
    bad = Bb.col.copy()
    bad[3] = 60
    dBb = binding.DeviceCSR(Bb.nrows, Bb.ncols, torch.from_numpy(Bb.rowptr).cuda(),
                            torch.from_numpy(bad).cuda(), torch.from_numpy(Bb.val).cuda())
    with binding.Plan() as p:
        with pytest.raises(binding.SpgemmError) as e:
            p.symbolic(dA, dBb)
        assert e.value.code == -3
    # a broken row pointer is caught too
    badrp = Bb.rowptr.copy()
    badrp[5] = badrp[6] + 1
    dBr = binding.DeviceCSR(Bb.nrows, Bb.ncols, torch.from_numpy(badrp).cuda(),
                            torch.from_numpy(Bb.col).cuda(), torch.from_numpy(Bb.val).cuda())
    with binding.Plan() as p:
        with pytest.raises(binding.SpgemmError) as e:
            p.symbolic(dA, dBr)
        assert e.value.code == -3
        # the plan stays usable after an error
        dBg = binding.DeviceCSR.from_host(Bb)
        C = p.multiply(dA, dBg)
        torch.cuda.synchronize()
        compare(A, Bb, C.rowptr.cpu().numpy(), C.col.cpu().numpy(), C.val.cpu().numpy())
        # numeric with other shapes than symbolic
        A51 = binding.DeviceCSR.from_host(synth.random_csr(51, 40, seed=117, value_seed=118,
                                                           mean_len=4))
        with pytest.raises(binding.SpgemmError) as e:
            p.numeric(A51, dBg, C.rowptr, C.col, C.val)
        assert e.value.code == -6
    for kw in ({"chunk_width_override": 48}, {"numeric_mode": 4}, {"symbolic_mode": -1}):
        with pytest.raises(binding.SpgemmError) as e:
            binding.Plan(**kw)
        assert e.value.code == -1


def _with_duplicates(M, seed):
    """M with every stored entry repeated once under a new value, the entries of
    each row shuffled: a repeated column must act as the sum of its entries."""
    rows = np.repeat(np.arange(M.nrows), np.diff(M.rowptr))
    rows2 = np.concatenate([rows, rows])
    col2 = np.concatenate([M.col, M.col])
    val2 = np.concatenate([M.val, synth.uniform_values(seed, M.nnz)])
    keys = synth.splitmix64(seed + 1, np.arange(col2.size, dtype=np.uint64))
    order = np.lexsort((keys, rows2))
    rp = np.zeros(M.nrows + 1, dtype=np.int64)
    rp[1:] = np.cumsum(2 * np.diff(M.rowptr))
    return synth.CSR(M.nrows, M.ncols, rp, col2[order].astype(np.int32), val2[order].copy())


@pytest.mark.parametrize("kw", [
    {},                                                               # light bins only
    {"tau_override": 40, "chunk_width_override": 64, "nchunks_cap": 4},  # heavy, path 3
    {"tau_override": 40, "chunk_width_override": 64, "nchunks_cap": 4,
     "symbolic_mode": 2, "numeric_mode": 2},                           # the page's dataflow
    {"tau_override": 40, "chunk_width_override": 64, "nchunks_cap": 4, "numeric_mode": 1},
])
def test_duplicate_entries_in_rows(kw):
    """A and B with every (row, column) stored twice: the oracle sums every
    stored entry's products, and so must each path."""
    A = _with_duplicates(synth.rmat(10, 4, seed=131, value_seed=132), 133)
    B = _with_duplicates(synth.random_csr(1024, 900, seed=134, value_seed=135, mean_len=5,
                                          skew=1.2), 136)
    rp, col, val, st = run_gpu(A, B, **kw)
    if kw:
        assert st["heavy_rows"] > 0
    compare(A, B, rp, col, val)
    Ai = _with_duplicates(synth.rmat(10, 4, seed=137, value_seed=138), 139)
    Ai.val = synth.small_int_values(140, Ai.nnz)  # every partial sum is an exact integer
    rp, col, val, st = run_gpu(Ai, Ai, **kw)
    compare(Ai, Ai, rp, col, val, exact_values=True)


def test_overflow_rejected_before_any_kernel():
    """More than INT32_MAX columns cannot be indexed by int32 columns: OVERFLOW."""
    import torch
    from spgemm_irregular_matrices_amd import binding
    big = (1 << 31)
    rp5 = torch.zeros(6, dtype=torch.int64, device="cuda")
    rp4 = torch.zeros(5, dtype=torch.int64, device="cuda")
    empty_i = torch.zeros(0, dtype=torch.int32, device="cuda")
    empty_v = torch.zeros(0, dtype=torch.float64, device="cuda")
    A = binding.DeviceCSR(4, 5, rp4, empty_i, empty_v)
    B = binding.DeviceCSR(5, big, rp5, empty_i, empty_v)
    with binding.Plan() as p:
        with pytest.raises(binding.SpgemmError) as e:
            p.symbolic(A, B)
        assert e.value.code == -4
        # A with more columns than int32 holds, B with as many rows
        Aw = binding.DeviceCSR(4, big, rp4, empty_i, empty_v)
        Bw = binding.DeviceCSR(big, 3, torch.zeros(1, dtype=torch.int64, device="cuda"),
                               empty_i, empty_v)
        with pytest.raises(binding.SpgemmError) as e:
            p.symbolic(Aw, Bw)
        assert e.value.code == -4
        # the plan still works
        S = synth.random_csr(40, 40, seed=141, value_seed=142, mean_len=4)
        dS = binding.DeviceCSR.from_host(S)
        C = p.multiply(dS, dS)
        torch.cuda.synchronize()
        compare(S, S, C.rowptr.cpu().numpy(), C.col.cpu().numpy(), C.val.cpu().numpy())


def test_workspace_limit_gives_out_of_memory():
    """A plan whose workspace limit is below what a product needs returns
    OUT_OF_MEMORY, frees its workspace, and can then run a product that fits."""
    import torch
    from spgemm_irregular_matrices_amd import binding
    A = synth.rmat(12, 16, seed=143, value_seed=144)
    dA = binding.DeviceCSR.from_host(A)
    tiny = synth.from_rows(2, 2, [[0, 1], [1]], [[2.0, -1.0], [3.0]])
    dT = binding.DeviceCSR.from_host(tiny)
    with binding.Plan(workspace_limit_bytes=64 << 10) as p:
        with pytest.raises(binding.SpgemmError) as e:
            p.multiply(dA, dA)
        assert e.value.code == -5
        # the numeric pass needs a successful symbolic pass again
        rp = torch.zeros(A.nrows + 1, dtype=torch.int64, device="cuda")
        with pytest.raises(binding.SpgemmError) as e:
            p.numeric(dA, dA, rp, None, None)
        assert e.value.code == -8
        C = p.multiply(dT, dT)
        torch.cuda.synchronize()
        assert C.rowptr.cpu().tolist() == [0, 2, 3]
        assert C.col.cpu().tolist() == [0, 1, 1]
        assert C.val.cpu().tolist() == [4.0, -5.0, 9.0]
    rp, col, val, st = run_gpu(A, A, workspace_limit_bytes=1 << 30)
    compare(A, A, rp, col, val)


def _check_levels_against_oracle(A, B, tau, chat, levels):
    """Every multisplit level, level by level, against the oracle's C-hat cut
    by oracle.stages.split_by_width.

    Level l's rows are the nonempty chunks of its input rows (the heavy rows
    of C-hat at level 0, else the heavy chunks of level l-1, which come first
    in that level's output); row_key = input row * chunks + chunk. Each row
    must hold exactly the entries of its parent's column range (a multiset:
    order inside a chunk is free), and a level's first rows are exactly its
    chunks with more than tau elements when a further level follows.
    """
    u = oracle.row_products(A, B)
    rows = np.nonzero(u > tau)[0]
    crp, ccol, cval = stages.expand(A, B, rows)
    # parents of level 0: the heavy rows of C-hat, covering [0, ppow)
    par_cols = [ccol[crp[h]:crp[h + 1]] for h in range(rows.size)]
    par_vals = [cval[crp[h]:crp[h + 1]] for h in range(rows.size)]
    par_base = [0] * rows.size
    width_in = chat["chunk_width"]
    for l, lv in enumerate(levels):
        W = lv["chunk_width"]
        nch = width_in // W
        keys = lv["row_key"]
        lrp = lv["rowptr"]
        assert np.unique(keys).size == keys.size
        by_key = {int(k): r for r, k in enumerate(keys)}
        nxt_cols, nxt_vals, nxt_base = {}, {}, {}
        seen = 0
        for p_idx in range(len(par_cols)):
            pieces = stages.split_by_width(par_cols[p_idx], par_vals[p_idx], W, par_base[p_idx], nch)
            for c, (ec, ev) in enumerate(pieces):
                key = p_idx * nch + c
                if ec.size == 0:
                    assert key not in by_key, f"level {l}: empty chunk {key} present"
                    continue
                r = by_key[key]
                a, b = int(lrp[r]), int(lrp[r + 1])
                got = sorted(zip(lv["col"][a:b].tolist(), lv["val"][a:b].tolist()))
                assert got == sorted(zip(ec.tolist(), ev.tolist())), f"level {l} chunk {key}"
                seen += b - a
                nxt_cols[r], nxt_vals[r], nxt_base[r] = ec, ev, par_base[p_idx] + c * W
        assert seen == int(lrp[-1]) and len(by_key) == len(nxt_cols)
        counts = np.diff(lrp)
        if l + 1 < len(levels):
            nheavy = int(np.count_nonzero(counts > tau))
            assert np.all(counts[:nheavy] > tau) and np.all(counts[nheavy:] <= tau)
            par_cols = [nxt_cols[r] for r in range(nheavy)]
            par_vals = [nxt_vals[r] for r in range(nheavy)]
            par_base = [nxt_base[r] for r in range(nheavy)]
        width_in = W


@pytest.mark.parametrize("numeric_mode", [2, 1])
@pytest.mark.parametrize("width,cap,nlevels", [(64, 2, 3), (32, 4, 2), (32, 2, 4)])
def test_every_multisplit_level_matches_oracle(numeric_mode, width, cap, nlevels):
    """Stage parity of every multisplit level (not only the first)."""
    import torch
    from spgemm_irregular_matrices_amd import binding
    A = synth.random_csr(300, 200, seed=151, value_seed=152, mean_len=10, skew=1.3)
    B = synth.random_csr(200, 500, seed=153, value_seed=154, mean_len=12, skew=1.3)
    tau = 24
    dA, dB = binding.DeviceCSR.from_host(A), binding.DeviceCSR.from_host(B)
    with binding.Plan(tau_override=tau, chunk_width_override=width, nchunks_cap=cap,
                      debug_dump=True, symbolic_mode=2, numeric_mode=numeric_mode) as p:
        C = p.multiply(dA, dB)
        torch.cuda.synchronize()
        st = p.stats()
        assert st["nlevels"] == nlevels, st
        levels = [p.debug(l) for l in range(st["nlevels"])]
        chat = p.debug(-1)
    assert all(lv["val"] is not None for lv in levels)
    _check_levels_against_oracle(A, B, tau, chat, levels)
    compare(A, B, C.rowptr.cpu().numpy(), C.col.cpu().numpy(), C.val.cpu().numpy())


@pytest.mark.parametrize("modes", [(1, 1), (1, 2), (2, 1), (2, 2)])
def test_debug_plan_self_checks(modes):
    """A debug plan (debug_dump) fills new floating-point workspace with NaN
    and checks on the host, after every multisplit level, that the level's
    chunk sizes add up to its input and that every chunk was filled to its
    end. Over three levels, in both symbolic and both level-forming numeric
    modes, the checks pass (the call returns OK), with row batches too, and
    the product still meets the oracle: no value was read from workspace
    that nothing wrote."""
    import torch
    from spgemm_irregular_matrices_amd import binding
    A = synth.random_csr(400, 300, seed=171, value_seed=172, mean_len=12, skew=1.3)
    B = synth.random_csr(300, 700, seed=173, value_seed=174, mean_len=14, skew=1.3)
    dA, dB = binding.DeviceCSR.from_host(A), binding.DeviceCSR.from_host(B)
    for budget in (0, 4000):
        with binding.Plan(tau_override=24, chunk_width_override=32, nchunks_cap=4,
                          debug_dump=True, symbolic_mode=modes[0], numeric_mode=modes[1],
                          max_batch_products=budget) as p:
            C = p.multiply(dA, dB)
            torch.cuda.synchronize()
            st = p.stats()
        assert st["nlevels"] == 3 and st["numeric_path"] == modes[1], st
        assert (st["nbatches"] > 1) == (budget > 0), st
        val = C.val.cpu().numpy()
        assert not np.isnan(val).any()
        compare(A, B, C.rowptr.cpu().numpy(), C.col.cpu().numpy(), val)


def test_heavy_rows_beyond_the_direct_slots():
    """Heavy rows over 2^26 columns: 8192 final chunks of 8192 columns are more
    than the direct path's 4096 slots and the row bitmap of the fused
    symbolic pass does not fit LDS, so the default options take the
    multisplit symbolic pass and the fused first level (path 1). The
    heaviest row (2.4 M products) needs all three levels (32 x 32 x 8
    chunks); the one-entry rows stay light."""
    lens = np.array([2000, 1800, 1500, 1200] + [1] * 200, dtype=np.int64)
    A = synth.distinct_uniform_rows(lens, 2000, seed=182, value_seed=183)
    B = synth.distinct_uniform_rows(np.full(2000, 1200, dtype=np.int64), 1 << 26, seed=184,
                                    value_seed=185)
    rp, col, val, st = run_gpu(A, B)
    assert st["numeric_path"] == 1 and st["nlevels"] == 3, st
    assert st["heavy_rows"] == 4 and st["vchunks"][:3] == [32, 32, 8], st
    compare(A, B, rp, col, val)


@pytest.mark.parametrize("ncols", [1 << 12, 1 << 20, 1 << 24])
def test_light_hash_rows_wide_columns(ncols):
    """Light rows whose columns spread over the whole range take the hash bins.
    Up to about 6 M columns their output is ranked through the two-level
    bitmap (no sort); at 2^24 columns the bitmap does not fit next to the
    table and the rows are sorted instead. Both against the oracle."""
    A = synth.random_csr(3000, 2000, seed=161, value_seed=162, mean_len=12, skew=1.2)
    B = synth.random_csr(2000, ncols, seed=163, value_seed=164, mean_len=40, skew=1.1)
    rp, col, val, st = run_gpu(A, B)
    u = oracle.row_products(A, B)
    assert st["heavy_rows"] == int(np.count_nonzero(u > st["tau"]))
    assert np.count_nonzero((u > 64) & (u <= st["tau"])) > 100  # hash-bin rows
    compare(A, B, rp, col, val)
