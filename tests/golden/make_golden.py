"""Writes the stored expected values under tests/golden/.

Every value here comes from the fp64 oracle (oracle/) applied to the seeded
inputs of workloads.py; nothing comes from the GPU path.  Re-run with
``python tests/golden/make_golden.py`` after a change to the oracle's
arithmetic, and say in the commit which passage of the pages justifies it.
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import dion_oracle as O  # noqa: E402
from workloads import fp32_64x128, lowrank_np, round_bf16  # noqa: E402


def main():
    M = fp32_64x128()
    out, _ = O.orthogonalize(M, n_iter=5)
    np.save(os.path.join(HERE, "fp32_64x128_out.npy"), out)

    # a small row-subset case: 3 fp32 momentum steps, top 1/4 rows of a 32x20
    E = np.zeros((32, 20), np.float32)
    rec = {}
    for t in range(3):
        G = round_bf16(lowrank_np((4, t, 0, 0), 32, 20, 3, 0.05, log_scale=(-3.0, 0.0)))
        (E,), (o,), (idx,) = O.rowsubset_step([E], [G], 0.95, n_iter=5, restart_every=2, row_frac=0.25)
        rec[f"G{t}"], rec[f"E{t}"], rec[f"out{t}"], rec[f"idx{t}"] = G, E, o, idx
    np.savez(os.path.join(HERE, "rowsubset_32x20.npz"), **rec)


if __name__ == "__main__":
    main()
