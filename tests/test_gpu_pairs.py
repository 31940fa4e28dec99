"""GPU parity on a second workload family: products of two independent
R-MAT matrices over the gMAGNUS page's grid of sizes and densities (Sec. IV-A:
scales 15-20, A.nnz/A.n from 4 to 64, B.nnz/B.n from 4 to 16, here at the
smaller scales the oracle checks row by row in seconds), and A*A^T for a
rectangular power-law A. Every row is compared with the oracle, with the
default heavy path and with the page's own dataflow (outer product into
C-hat, multisplit), at the default threshold and with heavy rows forced.
"""
import pytest

import oracle
from spgemm_irregular_matrices_amd import synth
from tests.helpers import compare, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    from spgemm_irregular_matrices_amd import binding
    binding.load()


PATHS = [{}, {"numeric_mode": 2},
         {"tau_override": 64, "chunk_width_override": 256, "nchunks_cap": 4},
         {"tau_override": 64, "chunk_width_override": 256, "nchunks_cap": 4, "numeric_mode": 2}]


@pytest.mark.parametrize("scale,efa,efb", [(12, 4, 16), (13, 16, 8), (12, 64, 4), (14, 8, 12)])
def test_rmat_pairs(scale, efa, efb):
    A = synth.rmat(scale, efa, seed=200 + scale, value_seed=300 + scale)
    B = synth.rmat(scale, efb, seed=400 + scale, value_seed=500 + scale)
    for kw in PATHS:
        rp, col, val, st = run_gpu(A, B, **kw)
        if kw.get("tau_override"):
            assert st["heavy_rows"] > 0
        compare(A, B, rp, col, val)


def test_rectangular_a_at():
    lens = synth.zipf_lengths(1 << 13, 2.1, 2048, seed=61)
    A = synth.distinct_uniform_rows(lens, 1 << 12, seed=61, value_seed=62)
    At = synth.transpose(A)
    for kw in PATHS:
        rp, col, val, st = run_gpu(A, At, **kw)
        assert st["heavy_rows"] > 0
        compare(A, At, rp, col, val)
