"""A randomized sweep of the batched call against the fp64 oracle.

Shapes, schedule (restart period, mask or threshold), safety factor, row
fraction, element type, precision and keep_schedule are drawn from a fixed
seed, so every run checks the same cases: the planner's tile tables, buffer
slots and restart forms meet here in combinations the hand-written cases do
not.  Gates as elsewhere: selected rows bit-exact (up to exchanges of rows whose
fp64 keys agree to 4 ulps), unselected rows copied exactly, the update within
1e-4 (FP64 path) or 2e-2 (MFMA16 path) relative Frobenius error per matrix.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import dion_oracle as O  # noqa: E402
from workloads import lowrank_np  # noqa: E402

pytestmark = pytest.mark.gpu

DIMS = [1, 3, 17, 64, 65, 128, 200, 255, 256, 257, 384, 511, 600]
N_CASES = 40


@pytest.fixture(scope="module")
def dion():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import orthogonalized_optimizer_step_amd as d
    return d


def draw(i):
    rng = np.random.default_rng([7, i])
    shapes = [(int(rng.choice(DIMS)), int(rng.choice(DIMS))) for _ in range(int(rng.integers(1, 6)))]
    K = int(rng.integers(1, 9))
    kind = int(rng.integers(0, 3))
    if kind == 0:
        sched = {"restart_every": int(rng.integers(0, 4))}
    elif kind == 1:
        sched = {"restart_mask": int(rng.integers(0, 1 << max(K - 1, 1)))}
    else:
        sched = {"restart_threshold": float(rng.choice([5.0, 100.0, 1000.0]))}
    kw = dict(n_iter=K, safety=float(rng.choice([1.0, 1.01, 1.05])),
              row_frac=float(rng.choice([1.0, 0.5, 0.25, 1.0 / 3])), **sched)
    dt = str(rng.choice(["bf16", "fp16", "fp32"]))
    prec = str(rng.choice(["auto", "mfma16"])) if dt == "fp32" else "auto"
    keep = bool(rng.integers(0, 2))
    return shapes, kw, dt, prec, keep


def longest_run(dion, kw):
    pts = dion.restart_points(**{k: v for k, v in kw.items() if k != "row_frac"})
    ends = pts + [kw["n_iter"]]
    return max(b - a for a, b in zip([0] + pts, ends))


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_config(dion, case):
    shapes, kw, dt, prec, keep = draw(case)
    if keep and longest_run(dion, kw) > 5:
        keep = False   # two-term runs longer than five iterations are outside the MFMA16 gate
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dt]
    dev = []
    for j, (r, c) in enumerate(shapes):
        M = lowrank_np((7, case, j), r, c, max(1, min(r, c) // 8), 0.1, log_scale=(-3.0, 0.0))
        dev.append(torch.from_numpy(M).to(tdt).cuda())
    fp64_path = dt == "fp32" and prec == "auto"
    tol = 1e-4 if fp64_path else 2e-2
    print(f"case {case}: {shapes} {dt} {prec} keep={keep} {kw}", flush=True)
    outs, idxs = dion.orth_batched(dev, precision=prec, keep_schedule=keep, return_indices=True, **kw)
    for M_dev, o, idx, s in zip(dev, outs, idxs, shapes):
        M = M_dev.float().cpu().numpy()
        ref, ref_idx = O.orthogonalize(M, **kw)
        got_idx = idx.cpu().numpy().astype(np.int64)
        if not np.array_equal(got_idx, ref_idx):
            keys = O.row_keys(M)
            diff = np.setxor1d(got_idx, ref_idx)
            assert np.max(keys[diff]) - np.min(keys[diff]) <= 4 * np.spacing(np.max(keys[diff])), (s, diff)
        got = o.float().cpu().numpy().astype(np.float64)
        rest = np.setdiff1d(np.arange(s[0]), got_idx)
        assert np.array_equal(got[rest], M[rest].astype(np.float64)), (s, "unselected rows")
        err = O.rel_frobenius(got[got_idx], ref[got_idx]) if np.array_equal(got_idx, ref_idx) else \
            O.rel_frobenius(got[ref_idx], ref[ref_idx])
        assert err <= tol, (s, dt, prec, keep, kw, err)
