"""The committed golden files still match the oracle (regression guard)."""
import os

import numpy as np

from oracle import dion_oracle as O
from workloads import fp32_64x128

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_fp32_golden():
    out, _ = O.orthogonalize(fp32_64x128(), n_iter=5)
    ref = np.load(os.path.join(HERE, "fp32_64x128_out.npy"))
    assert O.rel_frobenius(out, ref) < 1e-13


def test_rowsubset_golden():
    g = np.load(os.path.join(HERE, "rowsubset_32x20.npz"))
    E = np.zeros((32, 20), np.float32)
    for t in range(3):
        (E,), (o,), (idx,) = O.rowsubset_step([E], [g[f"G{t}"]], 0.95, n_iter=5,
                                              restart_every=2, row_frac=0.25)
        assert np.array_equal(E, g[f"E{t}"])
        assert np.array_equal(idx, g[f"idx{t}"])
        assert O.rel_frobenius(o, g[f"out{t}"]) < 1e-13
