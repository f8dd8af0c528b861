"""A randomized sweep of the batched call and the row-subset step against the fp64 oracle.

Shapes, schedule (restart period, mask or threshold), safety factor, row
fraction, element type, precision and keep_schedule are drawn from a fixed
seed, so every run checks the same cases: the planner's tile tables, buffer
slots and restart forms meet here in combinations the hand-written cases do
not.  Gates as elsewhere: selected rows bit-exact, unselected rows copied
exactly, every output of every matrix checked, the update within 1e-4 (FP64
path) or 2e-2 (MFMA16 path) relative Frobenius error per matrix.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import dion_oracle as O  # noqa: E402
from workloads import lowrank_np, round_bf16  # noqa: E402

pytestmark = pytest.mark.gpu

DIMS = [1, 3, 17, 64, 65, 128, 200, 255, 256, 257, 384, 511, 600]
N_CASES = 300
N_STEP_CASES = 100


@pytest.fixture(scope="module")
def dion():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import orthogonalized_optimizer_step_amd as d
    return d


# per-iteration coefficient schedules (n_coeff_sets = n_iter): the cubic
# Newton-Schulz map, a steeper first iteration followed by the quintic
# Newton-Schulz map (15x - 10x^3 + 3x^5) / 8, and the fixed quintic followed
# by that map
NS_CUBIC = (1.5, -0.5, 0.0)
NS_QUINTIC = (1.875, -1.25, 0.375)
STEEP_FIRST = (4.0, -5.5, 2.3)
QUINTIC = (3.4445, -4.7750, 2.0315)


def coefficient_draw(rng, K):
    kind = int(rng.integers(0, 6))
    if kind == 0:
        return [NS_CUBIC] * K
    if kind == 1:
        return [STEEP_FIRST] + [NS_QUINTIC] * (K - 1)
    if kind == 2:
        h = (K + 1) // 2
        return [QUINTIC] * h + [NS_QUINTIC] * (K - h)
    return None   # the fixed quintic


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
    co = coefficient_draw(rng, K)
    if co is not None:
        kw["coeffs"] = co
    dt = str(rng.choice(["bf16", "fp16", "fp32"]))
    prec = str(rng.choice(["auto", "mfma16"])) if dt == "fp32" else "auto"
    keep = bool(rng.integers(0, 2))
    return shapes, kw, dt, prec, keep


def longest_run(dion, kw):
    pts = dion.restart_points(**{k: v for k, v in kw.items() if k != "row_frac"})
    ends = pts + [kw["n_iter"]]
    return max(b - a for a, b in zip([0] + pts, ends))


def kept_in_range(dion, kw):
    """Whether keep_schedule is inside the MFMA16 path's range for this schedule:
    runs of at most two iterations are never cut (keep changes nothing); a longer
    run is kept only if no run exceeds five iterations and the slopes a_k / s of the
    whole schedule multiply to at most six iterations of the fixed quintic's."""
    run = longest_run(dion, kw)
    if run <= 2:
        return True
    co = kw.get("coeffs", [QUINTIC] * kw["n_iter"])
    gain = float(np.prod([max(1.0, abs(c[0]) / kw["safety"]) for c in co]))
    return run <= 5 and gain <= 3.4445 ** 6 * (1 + 1e-9)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_config(dion, case):
    shapes, kw, dt, prec, keep = draw(case)
    if keep and not kept_in_range(dion, kw):
        keep = False   # outside the range where the MFMA16 gate holds for kept runs
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
        assert np.array_equal(got_idx, ref_idx), (s, np.setxor1d(got_idx, ref_idx))
        got = o.float().cpu().numpy().astype(np.float64)
        rest = np.setdiff1d(np.arange(s[0]), ref_idx)
        assert np.array_equal(got[rest], M[rest].astype(np.float64)), (s, "unselected rows")
        err = O.rel_frobenius(got[ref_idx], ref[ref_idx])
        assert err <= tol, (s, dt, prec, keep, kw, err)


def same_selection(got_idx, ref_idx):
    """Indices bit-exact: both sides rank rows by the exact sum of squares rounded once."""
    assert np.array_equal(got_idx, ref_idx), np.setxor1d(got_idx, ref_idx)


@pytest.mark.parametrize("case", range(N_STEP_CASES))
def test_random_rowsubset_steps(dion, case):
    """Two consecutive row-subset steps: the fp32 buffer bit-exact (both error-feedback
    forms), indices as the oracle's, unselected rows exact, selected rows within 2e-2."""
    rng = np.random.default_rng([8, case])
    shapes = [(int(rng.choice(DIMS)), int(rng.choice(DIMS))) for _ in range(int(rng.integers(1, 5)))]
    _, kw, _, _, keep = draw(case + 1000)
    kw["row_frac"] = float(rng.choice([1.0, 0.5, 0.25, 1.0 / 3, 0.125]))
    if keep and not kept_in_range(dion, kw):
        keep = False
    ef = str(rng.choice(["raw", "carry"]))
    gdt = str(rng.choice(["bf16", "fp32"]))
    beta = float(rng.choice([0.9, 0.95]))
    print(f"step case {case}: {shapes} grad {gdt} ef={ef} beta={beta} keep={keep} {kw}", flush=True)
    E_host = [np.zeros(s, np.float32) for s in shapes]
    E_dev = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    for t in range(2):
        G = []
        for j, (r, c) in enumerate(shapes):
            g = lowrank_np((8, case, t, j), r, c, max(1, min(r, c) // 8), 0.05, log_scale=(-3.0, 0.0))
            G.append(round_bf16(g) if gdt == "bf16" else g.astype(np.float32))
        G_dev = [torch.from_numpy(np.ascontiguousarray(g)).cuda().to(torch.bfloat16 if gdt == "bf16" else torch.float32)
                 for g in G]
        outs, idxs = dion.rowsubset_step(E_dev, G_dev, beta, return_indices=True, ef=ef, keep_schedule=keep, **kw)
        newE, ref_outs, ref_idxs = O.rowsubset_step(E_host, G, beta, ef=ef, **kw)
        for i, s in enumerate(shapes):
            B = np.add(np.multiply(np.float32(beta), E_host[i], dtype=np.float32) if ef == "raw" else E_host[i], G[i],
                       dtype=np.float32)
            got_idx = idxs[i].cpu().numpy().astype(np.int64)
            same_selection(got_idx, ref_idxs[i])
            E_got = E_dev[i].cpu().numpy()
            assert np.array_equal(E_got.view(np.uint32), newE[i].view(np.uint32)), (s, t, "buffer")
            got = outs[i].float().cpu().numpy().astype(np.float64)
            rest = np.setdiff1d(np.arange(s[0]), got_idx)
            want_rest = round_bf16(B[rest]).astype(np.float64) if ef == "raw" else np.zeros((len(rest), s[1]))
            assert np.array_equal(got[rest], want_rest), (s, t, "unselected rows")
            err = O.rel_frobenius(got[ref_idxs[i]], ref_outs[i][ref_idxs[i]])
            assert err <= 2e-2, (s, t, gdt, ef, keep, kw, err)
            E_host[i] = E_got


N_LOWRANK_CASES = 40


@pytest.mark.parametrize("case", range(N_LOWRANK_CASES))
def test_random_lowrank_step(dion, case):
    """The low-rank Dion / Orth-Dion step on random shapes, ranks, beta, modes and
    gradient types: buffer (relative to ||B||), right factor and fp32 update within 1e-4,
    or within cond * 2^-24 where the factored matrix F (B Q for P, W for the QR form of
    Q') has a condition number cond above 2^24 * 1e-4 ~ 1700.  An orthogonal factor of F
    is determined by fp32-accurate data only to about cond(F) * 2^-24: a Gaussian right
    factor of full rank r = C is a square Gaussian matrix, whose condition number reaches
    1e3-1e5 (the step's own Q' is orthonormal, so only a first step from a random
    factor meets this)."""
    from oracle import orthdion_oracle as L
    rng = np.random.default_rng([9, case])
    shapes = [(int(rng.choice(DIMS[1:])), int(rng.choice(DIMS[1:]))) for _ in range(int(rng.integers(1, 5)))]
    rank = int(rng.choice([1, 4, 16, 33, 64, 128]))
    beta = float(rng.choice([0.0, 0.1, 0.5, 1.0]))
    mode = str(rng.choice(["qr", "colnorm"]))
    gdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[str(rng.choice(["bf16", "fp16", "fp32"]))]
    print(f"lowrank case {case}: {shapes} rank {rank} beta {beta} {mode} {gdt}", flush=True)
    Ms, Gs, Qs = [], [], []
    for R, C in shapes:
        r = min(rank, R, C)
        A = rng.standard_normal((R, 8)) @ rng.standard_normal((8, C)) + 0.3 * rng.standard_normal((R, C))
        Ms.append(A.astype(np.float32))
        Gs.append(torch.from_numpy((0.5 * rng.standard_normal((R, C))).astype(np.float32)).to(gdt))
        Qs.append(rng.standard_normal((C, r)).astype(np.float32))
    dM = [torch.from_numpy(M.copy()).cuda() for M in Ms]
    dQ = [torch.from_numpy(Q.copy()).cuda() for Q in Qs]
    outs = dion.lowrank_step(dM, [g.cuda() for g in Gs], dQ, beta, mode=mode, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for i, s in enumerate(shapes):
        G = Gs[i].float().numpy()
        M_ref, Q_ref, P_ref, D_ref = L.lowrank_step(Ms[i], G, Qs[i], beta, mode)
        B = L.accumulate(Ms[i], G).astype(np.float64)
        eb = float(np.linalg.norm(dM[i].cpu().numpy().astype(np.float64) - M_ref) / max(np.linalg.norm(B), 1e-300))
        eq = O.rel_frobenius(dQ[i].cpu().numpy().astype(np.float64), Q_ref)
        ed = O.rel_frobenius(outs[i].cpu().numpy().astype(np.float64), D_ref)
        c_p = np.linalg.cond(B @ Qs[i].astype(np.float64))
        c_w = np.linalg.cond(B.T @ P_ref) if mode == "qr" else 1.0
        tol_q = max(1e-4, c_w * 2.0 ** -24)
        tol_d = max(1e-4, max(c_p, c_w) * 2.0 ** -24)
        assert eb <= 1e-4 and eq <= tol_q and ed <= tol_d, (s, rank, beta, mode, gdt, eb, eq, ed, c_p, c_w)


N_UPDATE_CASES = 40


@pytest.mark.parametrize("case", range(N_UPDATE_CASES))
def test_random_fused_update(dion, case):
    """The row-subset step with the fused weight update on random draws: buffer, indices
    and the unselected weight rows bit-exact (both error-feedback forms, bf16 or fp32
    weights); selected rows within 2e-2 of the oracle's update (plus bf16 rounding)."""
    rng = np.random.default_rng([10, case])
    shapes = [(int(rng.choice(DIMS)), int(rng.choice(DIMS))) for _ in range(int(rng.integers(1, 5)))]
    _, kw, _, _, keep_s = draw(case + 2000)
    kw["row_frac"] = float(rng.choice([1.0, 0.5, 0.25, 1.0 / 3, 0.125]))
    if keep_s and not kept_in_range(dion, kw):
        keep_s = False
    ef = str(rng.choice(["raw", "carry"]))
    wbf16 = bool(rng.integers(0, 2))
    beta, wd = float(rng.choice([0.9, 0.95])), float(rng.choice([0.0, 0.01, 0.1]))
    alphas = [float(rng.choice([0.01, 0.02])) * float(np.sqrt(max(1.0, r / c))) for r, c in shapes]
    print(f"update case {case}: {shapes} wbf16={wbf16} ef={ef} wd={wd} keep={keep_s} {kw}", flush=True)
    W_host = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in shapes]
    if wbf16:
        W_host = [O.round_to_bf16(w) for w in W_host]
    W_dev = [torch.from_numpy(w).cuda().to(torch.bfloat16 if wbf16 else torch.float32) for w in W_host]
    E_host = [np.zeros(s, np.float32) for s in shapes]
    E_dev = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    keep = float(np.float32(1.0) - np.float32(wd))
    for t in range(2):
        G = [round_bf16(lowrank_np((10, case, t, j), r, c, max(1, min(r, c) // 8), 0.05, log_scale=(-3.0, 0.0)))
             for j, (r, c) in enumerate(shapes)]
        G_dev = [torch.from_numpy(np.ascontiguousarray(g)).cuda().to(torch.bfloat16) for g in G]
        _, idxs = dion.rowsubset_step_update(E_dev, G_dev, W_dev, beta, alphas, wd, return_indices=True, ef=ef,
                                             keep_schedule=keep_s, **kw)
        newE, newW, ref_idxs = O.rowsubset_step_update(E_host, G, W_host, beta, alphas, wd, bf16=wbf16, ef=ef, **kw)
        for i, s in enumerate(shapes):
            B = np.add(np.multiply(np.float32(beta), E_host[i], dtype=np.float32) if ef == "raw" else E_host[i], G[i],
                       dtype=np.float32)
            got_idx = idxs[i].cpu().numpy().astype(np.int64)
            same_selection(got_idx, ref_idxs[i])
            assert np.array_equal(E_dev[i].cpu().numpy().view(np.uint32), newE[i].view(np.uint32)), (s, t)
            got = W_dev[i].float().cpu().numpy().astype(np.float64)
            ix = ref_idxs[i]
            rest = np.setdiff1d(np.arange(s[0]), ix)
            assert np.array_equal(got[rest], newW[i][rest]), (s, t, "unselected weight rows")
            base = W_host[i][ix].astype(np.float64) * keep
            d_ref = newW[i][ix] - base
            if wbf16:
                err = np.linalg.norm(got[ix] - newW[i][ix])
                assert err <= 2.0 ** -9 * 1.01 * np.linalg.norm(newW[i][ix]) + 2e-2 * np.linalg.norm(d_ref), (s, t)
            else:
                assert O.rel_frobenius(got[ix] - base, d_ref) <= 2e-2, (s, t)
        E_host = [e.cpu().numpy() for e in E_dev]
        W_host = [w.float().cpu().numpy() for w in W_dev]


def test_large_megabatch(dion):
    """One call over 400 matrices of mixed shapes (1 ... 600 per side): the megabatch's
    tile tables, matrix lookup and per-XCD tile ranges at a size where every phase spans
    hundreds of matrices; every output against the oracle."""
    rng = np.random.default_rng(11)
    shapes = [(int(rng.choice(DIMS)), int(rng.choice(DIMS))) for _ in range(400)]
    kw = dict(n_iter=5, restart_every=2, row_frac=0.5)
    Ms = [lowrank_np((11, j), r, c, max(1, min(r, c) // 8), 0.1, log_scale=(-3.0, 0.0)) for j, (r, c) in enumerate(shapes)]
    dev = [torch.from_numpy(M).to(torch.bfloat16).cuda() for M in Ms]
    outs, idxs = dion.orth_batched(dev, return_indices=True, **kw)
    worst = 0.0
    for M_dev, o, idx, s in zip(dev, outs, idxs, shapes):
        M = M_dev.float().cpu().numpy()
        ref, ref_idx = O.orthogonalize(M, **kw)
        got_idx = idx.cpu().numpy().astype(np.int64)
        same_selection(got_idx, ref_idx)
        got = o.float().cpu().numpy().astype(np.float64)
        rest = np.setdiff1d(np.arange(s[0]), got_idx)
        assert np.array_equal(got[rest], M[rest].astype(np.float64)), s
        worst = max(worst, O.rel_frobenius(got[got_idx], ref[got_idx]))
    print(f"400 matrices: worst {worst:.2e}", flush=True)
    assert worst <= 2e-2
