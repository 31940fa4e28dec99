"""The input generators' structural helpers (CPU)."""
import numpy as np

from spgemm_irregular_matrices_amd import synth


def test_transpose():
    M = synth.random_csr(37, 53, seed=7, value_seed=8, mean_len=5, skew=1.2)
    T = synth.transpose(M)
    assert (T.nrows, T.ncols) == (53, 37)
    assert np.array_equal(T.to_dense(), M.to_dense().T)
    assert np.array_equal(synth.transpose(T).to_dense(), M.to_dense())
    for i in range(T.nrows):
        assert np.all(np.diff(T.col[T.rowptr[i]:T.rowptr[i + 1]]) > 0)
