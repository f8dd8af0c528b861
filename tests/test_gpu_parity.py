"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Gates: selected rows and the fp32 momentum buffer bit-exact; the update within
a relative Frobenius error of 1e-4 on the FP64 path (fp32 data) and 2e-2 on
the MFMA16 path (bf16 data), per matrix, against the oracle's fp64 result.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import dion_oracle as O  # noqa: E402
from workloads import (WORKLOADS, fp32_64x128, gpt2_small_np, bf16_bits_to_f32, lowrank_np,  # noqa: E402
                       round_bf16, LLAMA3_8B_LAYER)

pytestmark = pytest.mark.gpu

TOL_MFMA16 = 2e-2
TOL_FP64 = 1e-4


@pytest.fixture(scope="module")
def dion():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import orthogonalized_optimizer_step_amd as d
    return d


def to_dev_bf16(a32):
    return torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).cuda().to(torch.bfloat16)


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_selection(idx_gpu, M, frac):
    """Bit-exact against the oracle's selection: both sides rank rows by the
    exact sum of squares rounded once, so the selection is unique."""
    ref = O.select_rows(M, frac)
    got = np.asarray(idx_gpu, dtype=np.int64)
    assert np.array_equal(got, ref), f"selection differs: {np.setxor1d(got, ref)}"


# ------------------------------------------------------------ fp64 path
def test_fp32_64x128_fp64_path(dion):
    M = fp32_64x128()
    out = dion.orth_batched([torch.from_numpy(M).cuda()], n_iter=5)[0]
    ref, _ = O.orthogonalize(M, n_iter=5)
    err = O.rel_frobenius(to_np(out), ref)
    print(f"fp32 64x128 FP64 path: rel err {err:.3e}")
    assert err <= TOL_FP64
    assert err < 1e-6  # fp64 internals, fp32 output rounding only


SMALL_SHAPES = [(7, 33), (33, 7), (300, 200), (200, 520), (1, 5), (5, 1), (256, 256), (257, 511), (64, 64)]


def small_batch(seed, dtype_bf16=True):
    Ms = []
    for i, (r, c) in enumerate(SMALL_SHAPES):
        M = lowrank_np((seed, i), r, c, max(1, min(r, c) // 8), 0.1, log_scale=(-3.0, 0.0))
        Ms.append(round_bf16(M) if dtype_bf16 else M)
    return Ms


@pytest.mark.parametrize("sched", [dict(), dict(restart_every=2), dict(restart_mask=0b10, safety=1.01),
                                   dict(n_iter=6, restart_every=2, safety=1.05),
                                   dict(n_iter=6, restart_threshold=116.0, safety=1.05)])
def test_small_ragged_fp64_path(dion, sched):
    Ms = small_batch(11)
    outs = dion.orth_batched([torch.from_numpy(M).cuda() for M in Ms], precision="fp64",
                             **{"n_iter": 5, **sched})
    for M, o in zip(Ms, outs):
        ref, _ = O.orthogonalize(M, **{"n_iter": 5, **sched})
        err = O.rel_frobenius(to_np(o), ref)
        assert err < 1e-6, (M.shape, err)


# ---------------------------------------------------------- MFMA16 path
@pytest.mark.parametrize("sched", [dict(), dict(restart_every=2), dict(restart_mask=0b10, safety=1.01),
                                   dict(n_iter=6, restart_every=2, safety=1.05), dict(restart_every=1),
                                   dict(n_iter=6, restart_every=1), dict(restart_threshold=1000.0),
                                   dict(n_iter=6, restart_threshold=116.0, safety=1.05),
                                   dict(n_iter=6, restart_threshold=5.0)])
def test_small_ragged_mfma16(dion, sched):
    Ms = small_batch(12)
    kw = {"n_iter": 5, **sched}
    outs = dion.orth_batched([to_dev_bf16(M) for M in Ms], **kw)
    errs = []
    for M, o in zip(Ms, outs):
        ref, _ = O.orthogonalize(M, **kw)
        errs.append(O.rel_frobenius(to_np(o), ref))
    print("MFMA16 small ragged", sched, " ".join(f"{e:.2e}" for e in errs), flush=True)
    assert max(errs) <= TOL_MFMA16


@pytest.mark.parametrize("sched", [dict(), dict(restart_mask=0b10, safety=1.01), dict(n_iter=6, restart_mask=0b1),
                                   dict(n_iter=6, restart_threshold=1e5)])
def test_long_runs_cut_or_kept(dion, sched):
    """Schedules with runs of more than two iterations between restarts: cut by extra
    restarts (the default) or run as given with two-term operands (keep_schedule).  Both
    against the oracle of the schedule as given, since a restart does not change the exact
    result; the kept plan forms one Gram per run of the schedule, the cut one more."""
    Ms = small_batch(15)
    kw = {"n_iter": 5, **sched}
    dev = [to_dev_bf16(M) for M in Ms]
    refs = [O.orthogonalize(M, **kw)[0] for M in Ms]
    grams, worst = {}, {}
    for keep in (False, True):
        dion.profile_enable(True)
        outs = dion.orth_batched(dev, keep_schedule=keep, **kw)
        names = [r[0] for r in dion.profile_records()]
        dion.profile_enable(False)
        errs = [O.rel_frobenius(to_np(o), ref) for o, ref in zip(outs, refs)]
        grams[keep], worst[keep] = names.count("syrk"), max(errs)
        assert max(errs) <= TOL_MFMA16, (sched, keep, errs)
    runs = len(dion.restart_points(**{k: v for k, v in kw.items() if k != "row_frac"})) + 1
    assert grams[True] == runs and grams[False] > runs, (grams, runs)
    print("long runs", sched, f"cut {worst[False]:.2e} kept {worst[True]:.2e}", flush=True)


def test_profile_algorithmic_flops(dion):
    """Per-launch FLOP accounting of a two-restart schedule (K = 5, restarts after 2
    and 4), against counts written out from the shapes: useful FLOPs over the call
    equal dion_useful_flops; every launch's algorithmic FLOPs equal its useful ones
    except the accumulated restart factor's, which counts m^2 (m + 1) per matrix
    restarting from X0 in the algorithmic figure and nothing in the useful one."""
    shapes = [(256, 640), (640, 256), (384, 384), (1024, 512)]
    Ms = [round_bf16(lowrank_np((33, i), r, c, 16, 0.1)) for i, (r, c) in enumerate(shapes)]
    dev = [to_dev_bf16(M) for M in Ms]
    dion.profile_enable(True)
    dion.orth_batched(dev, restart_every=2)
    recs = dion.profile_records()
    dion.profile_enable(False)
    useful = sum(r[3] for r in recs)
    assert useful == pytest.approx(dion.useful_flops(shapes, restart_every=2), rel=1e-12)
    acc = [r for r in recs if r[0] == "acc_product"]
    assert len(acc) == 1, [r[0] for r in recs]
    assert acc[0][3] == 0.0
    # every matrix here has a Gram side of at least 128 and restarts from X0
    assert acc[0][6] == pytest.approx(sum(float(min(r, c)) ** 2 * (min(r, c) + 1) for r, c in shapes), rel=1e-12)
    for r in recs:
        if r[0] != "acc_product":
            assert r[6] == pytest.approx(r[3], rel=1e-12), r


def test_keep_schedule_no_effect_on_short_runs(dion):
    """Runs of at most two iterations are never cut: the same plan, bit-identical outputs."""
    dev = [to_dev_bf16(M) for M in small_batch(16)]
    for kw in (dict(restart_every=2), dict(n_iter=6, restart_every=2, safety=1.05), dict(n_iter=2)):
        a = dion.orth_batched(dev, **kw)
        b = dion.orth_batched(dev, keep_schedule=True, **kw)
        for x, y in zip(a, b):
            assert torch.equal(x, y), kw


def test_restart_threshold_same_plan_as_mask(dion):
    """A threshold only chooses the restart points: tau = 100 with the fixed quintic
    plans restarts {2, 4}, so the output is bit-identical to restart_every = 2."""
    Ms = small_batch(14)
    dev = [to_dev_bf16(M) for M in Ms]
    a = dion.orth_batched(dev, restart_threshold=100.0)
    b = dion.orth_batched(dev, restart_every=2)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_fp32_input_mfma16(dion):
    """fp32 momentum on the MFMA16 path (two-term operands for X0)."""
    Ms = small_batch(13, dtype_bf16=False)
    outs = dion.orth_batched([torch.from_numpy(M).cuda() for M in Ms], precision="mfma16", restart_every=2)
    for M, o in zip(Ms, outs):
        ref, _ = O.orthogonalize(M, restart_every=2)
        assert O.rel_frobenius(to_np(o), ref) <= TOL_MFMA16


def test_gpt2_small_full(dion):
    wl = WORKLOADS["gpt2_small"]
    Ms = [bf16_bits_to_f32(b) for b in gpt2_small_np()]
    outs = dion.orth_batched([to_dev_bf16(M) for M in Ms], **wl.ns_kwargs())
    errs = []
    for M, o in zip(Ms, outs):
        ref, _ = O.orthogonalize(M, **wl.ns_kwargs())
        errs.append(O.rel_frobenius(to_np(o), ref))
    print(f"gpt2_small: max rel err {max(errs):.3e}, mean {np.mean(errs):.3e}")
    assert max(errs) <= TOL_MFMA16


def test_determinism(dion):
    Ms = [to_dev_bf16(M) for M in small_batch(14)]
    a = dion.orth_batched(Ms, restart_every=2, row_frac=0.5)
    b = dion.orth_batched(Ms, restart_every=2, row_frac=0.5)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_zero_matrix(dion):
    for prec, dt in (("mfma16", torch.bfloat16), ("fp64", torch.float32)):
        Ms = [torch.zeros((12, 40), dtype=dt, device="cuda"), torch.zeros((40, 12), dtype=dt, device="cuda")]
        outs, idx = dion.orth_batched(Ms, row_frac=0.25, precision=prec, return_indices=True)
        for o in outs:
            assert torch.count_nonzero(o) == 0
        assert idx[0].tolist() == [0, 1, 2] and idx[1].tolist() == list(range(10))


# ---------------------------------------------------------- row subset
@pytest.mark.parametrize("frac", [0.25, 0.5, 0.125, 1.0 / 37])
@pytest.mark.parametrize("prec", ["mfma16", "fp64"])
def test_row_subset_ties(dion, frac, prec):
    rng = np.random.default_rng(int(frac * 1000))
    shapes = [(37, 16), (64, 20), (16, 300), (520, 40)]
    Ms = []
    for r, c in shapes:
        M = rng.integers(-4, 5, size=(r, c)).astype(np.float32)
        M[rng.integers(0, r, size=r // 4)] = 0.0
        M[r // 2] = M[0]
        M[r - 1] = M[1]
        Ms.append(M)
    dt = torch.bfloat16 if prec == "mfma16" else torch.float32
    dev = [torch.from_numpy(M).cuda().to(dt) for M in Ms]
    outs, idxs = dion.orth_batched(dev, restart_every=2, row_frac=frac, precision=prec, return_indices=True)
    for M, o, ix in zip(Ms, outs, idxs):
        ref_out, ref_idx = O.orthogonalize(M, restart_every=2, row_frac=frac)
        assert np.array_equal(ix.cpu().numpy(), ref_idx)          # integer keys: exact
        got = to_np(o)
        rest = np.setdiff1d(np.arange(M.shape[0]), ref_idx)
        assert np.array_equal(got[rest], M[rest].astype(np.float64))
        tol = TOL_MFMA16 if prec == "mfma16" else 1e-6
        assert O.rel_frobenius(got[ref_idx], ref_out[ref_idx]) <= tol


def test_rowsubset_step_small(dion):
    shapes = [(32, 20), (64, 48), (40, 200), (300, 64)]
    beta = 0.95
    E_host = [np.zeros(s, np.float32) for s in shapes]
    E_dev = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    for t in range(3):
        G = [round_bf16(lowrank_np((4, t, i, 0), r, c, 3, 0.05, log_scale=(-3.0, 0.0)))
             for i, (r, c) in enumerate(shapes)]
        outs, idxs = dion.rowsubset_step(E_dev, [to_dev_bf16(g) for g in G], beta, restart_every=2,
                                         row_frac=0.25, return_indices=True)
        newE, ref_outs, ref_idxs = O.rowsubset_step(E_host, G, beta, n_iter=5, restart_every=2, row_frac=0.25)
        for i in range(len(shapes)):
            assert np.array_equal(E_dev[i].cpu().numpy().view(np.uint32), newE[i].view(np.uint32))
            assert_selection(idxs[i].cpu().numpy(), newE[i], 0.25)
            got = to_np(outs[i])
            ix = ref_idxs[i]
            rest = np.setdiff1d(np.arange(shapes[i][0]), ix)
            assert np.array_equal(got[rest], round_bf16(newE[i][rest]).astype(np.float64))
            assert O.rel_frobenius(got[ix], ref_outs[i][ix]) <= TOL_MFMA16
        E_host = newE


@pytest.mark.parametrize("keep", [False, True])
def test_long_runs_fp32_operands(dion, keep):
    """fp32 inputs on the MFMA16 path (two-term X0) and the row-subset step's fp32 buffer,
    with no restarts in K = 5: the cut plan restarts from the two-term iterate; both plans
    against the oracle of the schedule as given."""
    Ms = small_batch(17, dtype_bf16=False)
    outs = dion.orth_batched([torch.from_numpy(M).cuda() for M in Ms], precision="mfma16", keep_schedule=keep)
    for M, o in zip(Ms, outs):
        assert O.rel_frobenius(to_np(o), O.orthogonalize(M)[0]) <= TOL_MFMA16, (M.shape, keep)
    shapes = [(64, 48), (40, 200), (300, 64), (257, 511)]
    E_host = [np.zeros(s, np.float32) for s in shapes]
    E_dev = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    for t in range(2):
        G = [round_bf16(lowrank_np((4, t, i, 6), r, c, 3, 0.05)) for i, (r, c) in enumerate(shapes)]
        outs = dion.rowsubset_step(E_dev, [to_dev_bf16(g) for g in G], 0.95, row_frac=0.25, keep_schedule=keep)
        E_host, ref_outs, ref_idxs = O.rowsubset_step(E_host, G, 0.95, n_iter=5, row_frac=0.25)
        for i, ix in enumerate(ref_idxs):
            assert O.rel_frobenius(to_np(outs[i])[ix], ref_outs[i][ix]) <= TOL_MFMA16, (shapes[i], t, keep)


# -------------------------------------------------- fused weight update
@pytest.mark.parametrize("wbf16", [False, True])
def test_rowsubset_step_update(dion, wbf16):
    """Momentum + selection + Gram-NS + weight update in one call, three steps.

    E and the rows left out by the selection are fixed bit for bit (their
    update is the exact fp32 momentum).  Selected rows: fp32 weights gate the
    update W_new - W keep against -alpha O at 2e-2; bf16 weights add their
    rounding, 2^-9 relative per element."""
    shapes = [(32, 20), (64, 48), (40, 200), (300, 64)]
    beta, wd = 0.95, 0.01
    alphas = [0.02 * float(np.sqrt(max(1.0, r / c))) for r, c in shapes]
    keep = float(np.float32(1.0) - np.float32(wd))
    rng = np.random.default_rng(7)
    W_host = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in shapes]
    if wbf16:
        W_host = [O.round_to_bf16(w) for w in W_host]
    wdt = torch.bfloat16 if wbf16 else torch.float32
    W_dev = [torch.from_numpy(w).cuda().to(wdt) for w in W_host]
    E_host = [np.zeros(s, np.float32) for s in shapes]
    E_dev = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    for t in range(3):
        G = [round_bf16(lowrank_np((4, t, i, 1), r, c, 3, 0.05, log_scale=(-3.0, 0.0)))
             for i, (r, c) in enumerate(shapes)]
        _, idxs = dion.rowsubset_step_update(E_dev, [to_dev_bf16(g) for g in G], W_dev, beta, alphas, wd,
                                             restart_every=2, row_frac=0.25, return_indices=True)
        newE, newW, ref_idxs = O.rowsubset_step_update(E_host, G, W_host, beta, alphas, wd, bf16=wbf16, n_iter=5,
                                                       restart_every=2, row_frac=0.25)
        for i in range(len(shapes)):
            assert np.array_equal(E_dev[i].cpu().numpy().view(np.uint32), newE[i].view(np.uint32))
            assert_selection(idxs[i].cpu().numpy(), newE[i], 0.25)
            got = to_np(W_dev[i])
            ix = ref_idxs[i]
            rest = np.setdiff1d(np.arange(shapes[i][0]), ix)
            assert np.array_equal(got[rest], newW[i][rest])
            base = W_host[i][ix].astype(np.float64) * keep
            d_ref = newW[i][ix] - base
            if wbf16:
                err = np.linalg.norm(got[ix] - newW[i][ix])
                assert err <= 2.0 ** -9 * 1.01 * np.linalg.norm(newW[i][ix]) + TOL_MFMA16 * np.linalg.norm(d_ref)
            else:
                assert O.rel_frobenius(got[ix] - base, d_ref) <= TOL_MFMA16
        E_host = newE
        W_host = [to_np(w).astype(np.float32) for w in W_dev]   # selected rows follow the GPU's own values


def test_dion3_optimizer_step(dion):
    """The optimizer class: one step on two fp32 weights equals the fused call
    with alpha = lr * sqrt(max(1, rows / cols)) and decay lr * weight_decay."""
    torch.manual_seed(0)
    shapes = [(96, 64), (64, 160)]
    params = [torch.nn.Parameter(torch.randn(s, device="cuda") * 0.02) for s in shapes]
    W0 = [p.detach().cpu().numpy().copy() for p in params]
    G = [round_bf16(lowrank_np((8, i), r, c, 4, 0.05)) for i, (r, c) in enumerate(shapes)]
    for p, g in zip(params, G):
        p.grad = torch.from_numpy(g).cuda()
    opt = dion.Dion3(params, lr=0.02, momentum=0.95, row_frac=0.5, weight_decay=0.1, restart_every=2)
    opt.step()
    alphas = [0.02 * float(np.sqrt(max(1.0, r / c))) for r, c in shapes]
    newE, newW, idxs = O.rowsubset_step_update([np.zeros(s, np.float32) for s in shapes], G, W0, 0.95, alphas,
                                               0.02 * 0.1, n_iter=5, restart_every=2, row_frac=0.5)
    keep = float(np.float32(1.0) - np.float32(0.02 * 0.1))
    for p, E, W, ix, w0 in zip(params, newE, newW, idxs, W0):
        assert np.array_equal(opt.state[p]["momentum_buffer"].cpu().numpy(), E)
        got = p.detach().cpu().numpy().astype(np.float64)
        rest = np.setdiff1d(np.arange(W.shape[0]), ix)
        assert np.array_equal(got[rest], W[rest])
        base = w0[ix].astype(np.float64) * keep
        assert O.rel_frobenius(got[ix] - base, W[ix] - base) <= TOL_MFMA16


# ------------------------------------------------------------ fp16 I/O
def f16_batch(seed):
    return [lowrank_np((seed, i), r, c, max(1, min(r, c) // 8), 0.1, log_scale=(-3.0, 0.0)).astype(np.float16)
            .astype(np.float32) for i, (r, c) in enumerate(SMALL_SHAPES)]


@pytest.mark.parametrize("prec,tol", [("mfma16", TOL_MFMA16), ("fp64", 2.0 ** -10)])
def test_small_ragged_fp16_io(dion, prec, tol):
    """fp16 momentum in, fp16 update out.  MFMA16: the bf16-path gate (fp16
    values are exact in one fp16 term); FP64: only the fp16 output rounding,
    at most 2^-11 relative per element."""
    Ms = f16_batch(31)
    kw = {"n_iter": 5, "restart_every": 2}
    outs, idx = dion.orth_batched([torch.from_numpy(M).cuda().to(torch.float16) for M in Ms], precision=prec,
                                  row_frac=0.5, return_indices=True, **kw)
    errs = []
    for M, o, ix in zip(Ms, outs, idx):
        assert o.dtype == torch.float16
        ref, ref_idx = O.orthogonalize(M, row_frac=0.5, **kw)
        assert np.array_equal(ix.cpu().numpy(), ref_idx)
        got = to_np(o)
        rest = np.setdiff1d(np.arange(M.shape[0]), ref_idx)
        assert np.array_equal(got[rest], M[rest].astype(np.float64))
        errs.append(O.rel_frobenius(got[ref_idx], ref[ref_idx]))
    print(f"fp16 I/O {prec}:", " ".join(f"{e:.1e}" for e in errs), flush=True)
    assert max(errs) <= tol


def test_fp16_full_size(dion):
    """A Llama-3-8B down-projection-shaped fp16 matrix (4096 x 14336), restarts every 2."""
    M = lowrank_np((3, 0, 6), 4096, 14336, 64, 0.05, log_scale=(-3, 0)).astype(np.float16).astype(np.float32)
    out = dion.orth_batched([torch.from_numpy(M).cuda().to(torch.float16)], n_iter=5, restart_every=2)[0]
    ref, _ = O.orthogonalize(M, n_iter=5, restart_every=2)
    err = O.rel_frobenius(to_np(out), ref)
    print(f"fp16 4096x14336: rel err {err:.3e}", flush=True)
    assert err <= TOL_MFMA16


@pytest.mark.parametrize("prec", ["mfma16", "fp64"])
def test_batch_order_independence(dion, prec):
    """A tile's arithmetic does not depend on which XCD or CU runs it, so permuting
    the batch (which moves the work-balanced per-XCD tile ranges) leaves every
    matrix's output bit-identical.  Shapes mix reduction depths from 512 to 8192;
    on the MFMA16 path four 4096 x 4096 matrices push the symmetric phases onto
    256-row tiles."""
    rng = np.random.default_rng(77)
    if prec == "mfma16":
        shapes = [(4096, 4096)] * 4 + [(1024, 8192)] * 3 + [(8192, 1024), (300, 500), (512, 512), (2048, 600)]
        Ms = [to_dev_bf16(rng.standard_normal(s).astype(np.float32)) for s in shapes]
    else:
        shapes = [(96, 700), (64, 64), (500, 130), (40, 1200), (256, 256), (130, 333)]
        Ms = [torch.from_numpy(rng.standard_normal(s).astype(np.float32)).cuda() for s in shapes]
    kw = dict(n_iter=5, restart_every=2, precision=prec)
    base = dion.orth_batched(Ms, **kw)
    for perm in (list(range(len(Ms)))[::-1], list(rng.permutation(len(Ms)))):
        outs = dion.orth_batched([Ms[i] for i in perm], **kw)
        for o, i in zip(outs, perm):
            assert torch.equal(o, base[i]), (prec, shapes[i], perm)


TINY_SHAPES = [(64, 128), (128, 64), (1, 5), (5, 1), (40, 40), (64, 1024), (1024, 64), (3, 700), (63, 65)]
TINY_TOL = {"fp32": 1e-6, "bf16": 2.0 ** -8, "fp16": 2.0 ** -10}


@pytest.mark.parametrize("sched", [dict(), dict(restart_every=2), dict(restart_mask=0b10, safety=1.01),
                                   dict(n_iter=6, restart_every=1), dict(restart_threshold=100.0)])
@pytest.mark.parametrize("dt", ["fp32", "bf16", "fp16"])
def test_tiny_batch_one_launch(dion, sched, dt):
    """Every matrix with Gram side <= 64 and long side <= 1024: keys, selection and one fp64
    launch for the whole iteration; the output carries only its own rounding."""
    rng = np.random.default_rng(31)
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[dt]
    dev = [torch.from_numpy(rng.standard_normal(s).astype(np.float32)).to(tdt).cuda() for s in TINY_SHAPES]
    kw = {"n_iter": 5, **sched}
    dion.profile_enable(True)
    outs = dion.orth_batched(dev, **kw)
    names = [r[0] for r in dion.profile_records()]
    dion.profile_enable(False)
    assert "tiny" in names and "syrk" not in names, names
    for M, o, s in zip(dev, outs, TINY_SHAPES):
        ref, _ = O.orthogonalize(M.float().cpu().numpy(), **kw)
        err = O.rel_frobenius(to_np(o), ref)
        assert err <= TINY_TOL[dt], (s, dt, err)


@pytest.mark.parametrize("frac", [0.125, 0.25, 1.0 / 3])
def test_tiny_row_subset(dion, frac):
    """Row subsets on the one-launch path: indices as the oracle's, unselected rows copied exactly."""
    rng = np.random.default_rng(32)
    shapes = [(512, 64), (256, 300), (96, 8), (40, 1000)]
    Ms = [round_bf16(rng.standard_normal(s).astype(np.float32)) for s in shapes]
    outs, idxs = dion.orth_batched([to_dev_bf16(M) for M in Ms], row_frac=frac, restart_every=2,
                                   return_indices=True)
    for M, o, ix, s in zip(Ms, outs, idxs, shapes):
        assert_selection(ix.cpu().numpy(), M, frac)
        ref, idx = O.orthogonalize(M, row_frac=frac, restart_every=2)
        on = to_np(o)
        unsel = np.setdiff1d(np.arange(s[0]), idx)
        assert np.array_equal(on[unsel], M[unsel].astype(np.float64)), s
        assert O.rel_frobenius(on[idx], ref[idx]) <= 2.0 ** -8, s


# ---------------------------------------- carry form of error feedback
def test_rowsubset_carry_steps(dion):
    """ef="carry", three steps: the buffer bit-exact (unselected rows carried
    undecayed, selected rows fl32(beta B)), indices as the oracle's on
    B = fl32(E + G), unselected output rows exactly zero."""
    shapes = [(32, 20), (64, 48), (40, 200), (300, 64)]
    beta = 0.95
    E_host = [np.zeros(s, np.float32) for s in shapes]
    E_dev = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    for t in range(3):
        G = [round_bf16(lowrank_np((4, t, i, 2), r, c, 3, 0.05, log_scale=(-3.0, 0.0)))
             for i, (r, c) in enumerate(shapes)]
        outs, idxs = dion.rowsubset_step(E_dev, [to_dev_bf16(g) for g in G], beta, restart_every=2,
                                         row_frac=0.25, return_indices=True, ef="carry")
        newE, ref_outs, ref_idxs = O.rowsubset_step(E_host, G, beta, ef="carry", n_iter=5, restart_every=2,
                                                    row_frac=0.25)
        for i in range(len(shapes)):
            B = np.add(E_host[i], G[i], dtype=np.float32)
            assert np.array_equal(E_dev[i].cpu().numpy().view(np.uint32), newE[i].view(np.uint32))
            assert_selection(idxs[i].cpu().numpy(), B, 0.25)
            got = to_np(outs[i])
            ix = ref_idxs[i]
            rest = np.setdiff1d(np.arange(shapes[i][0]), ix)
            assert np.all(got[rest] == 0.0)
            assert O.rel_frobenius(got[ix], ref_outs[i][ix]) <= TOL_MFMA16
        E_host = newE


def test_rowsubset_carry_update(dion):
    """ef="carry" with the fused weight update: unselected weight rows take only the
    decay, fl32(W keep) rounded to bf16, bit for bit; the buffer bit-exact."""
    shapes = [(32, 20), (64, 48), (300, 64)]
    beta, wd = 0.9, 0.01
    alphas = [0.02 * float(np.sqrt(max(1.0, r / c))) for r, c in shapes]
    rng = np.random.default_rng(8)
    W_host = [O.round_to_bf16((rng.standard_normal(s) * 0.02).astype(np.float32)) for s in shapes]
    W_dev = [torch.from_numpy(w).cuda().to(torch.bfloat16) for w in W_host]
    E_host = [np.zeros(s, np.float32) for s in shapes]
    E_dev = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    for t in range(2):
        G = [round_bf16(lowrank_np((4, t, i, 3), r, c, 3, 0.05)) for i, (r, c) in enumerate(shapes)]
        dion.rowsubset_step_update(E_dev, [to_dev_bf16(g) for g in G], W_dev, beta, alphas, wd,
                                   restart_every=2, row_frac=0.25, ef="carry")
        newE, newW, ref_idxs = O.rowsubset_step_update(E_host, G, W_host, beta, alphas, wd, bf16=True, n_iter=5,
                                                       restart_every=2, row_frac=0.25, ef="carry")
        for i in range(len(shapes)):
            assert np.array_equal(E_dev[i].cpu().numpy().view(np.uint32), newE[i].view(np.uint32))
            rest = np.setdiff1d(np.arange(shapes[i][0]), ref_idxs[i])
            assert np.array_equal(to_np(W_dev[i])[rest], newW[i][rest])
        E_host = newE
        W_host = [to_np(w).astype(np.float32) for w in W_dev]


def test_rowsubset_carry_equals_raw_at_full_rows(dion):
    """row_frac = 1: carry and raw run the same momentum sequence, so their outputs are
    bit-identical over several steps, and carry's buffer is fl32(beta * raw's)."""
    shapes = [(64, 48), (40, 200)]
    beta = 0.95
    Er = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    Ec = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    for t in range(3):
        G = [to_dev_bf16(round_bf16(lowrank_np((4, t, i, 4), r, c, 3, 0.05))) for i, (r, c) in enumerate(shapes)]
        o_r = dion.rowsubset_step(Er, G, beta, restart_every=2, row_frac=1.0)
        o_c = dion.rowsubset_step(Ec, G, beta, restart_every=2, row_frac=1.0, ef="carry")
        for i in range(len(shapes)):
            assert torch.equal(o_r[i], o_c[i])
            want = np.multiply(np.float32(beta), Er[i].cpu().numpy(), dtype=np.float32)
            assert np.array_equal(Ec[i].cpu().numpy().view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("sched", [dict(n_iter=12, restart_every=2), dict(n_iter=9, restart_every=2),
                                   dict(n_iter=8, restart_mask=0b1010101)])
def test_many_restarts(dion, sched):
    """Three to five restarts of two-iteration segments, wide and tall matrices among them
    (n >= 1.5 m): with more than two restarts every matrix restarts from the two-term iterate,
    since the accumulated restart factor's rounding would compound.  Row subsets, bf16,
    against the oracle."""
    rng = np.random.default_rng(41)
    shapes = [(92, 43), (280, 85), (196, 298), (83, 114), (200, 640), (640, 200), (128, 128)]
    Ms = [round_bf16(rng.standard_normal(s).astype(np.float32)) for s in shapes]
    kw = dict(row_frac=0.5, **sched)
    outs = dion.orth_batched([to_dev_bf16(M) for M in Ms], **kw)
    for M, o, s in zip(Ms, outs, shapes):
        ref, idx = O.orthogonalize(M, **kw)
        assert O.rel_frobenius(to_np(o)[idx], ref[idx]) <= TOL_MFMA16, (s, sched)


@pytest.mark.parametrize("ef", ["raw", "carry"])
def test_rowsubset_resume_from_host_copy(dion, ef):
    """The caller's fp32 buffer is the only state across steps: ten consecutive steps equal
    five steps, a round trip of the buffer through host memory into fresh device tensors,
    and five more steps, bit for bit (buffer, indices and outputs)."""
    shapes = [(64, 48), (40, 200), (300, 64)]
    grads = [[to_dev_bf16(round_bf16(lowrank_np((4, t, i, 5), r, c, 3, 0.05))) for i, (r, c) in enumerate(shapes)]
             for t in range(10)]
    kw = dict(restart_every=2, row_frac=0.25, return_indices=True, ef=ef)
    E1 = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    run1 = [dion.rowsubset_step(E1, grads[t], 0.95, **kw) for t in range(10)]
    E2 = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    run2 = [dion.rowsubset_step(E2, grads[t], 0.95, **kw) for t in range(5)]
    host = [e.cpu().numpy().copy() for e in E2]
    del E2
    E3 = [torch.from_numpy(h).cuda() for h in host]
    run2 += [dion.rowsubset_step(E3, grads[t], 0.95, **kw) for t in range(5, 10)]
    for a, b in zip(E1, E3):
        assert torch.equal(a, b)
    for (oa, ia), (ob, ib) in zip(run1, run2):
        for x, y in zip(oa, ob):
            assert torch.equal(x, y)
        for x, y in zip(ia, ib):
            assert torch.equal(x, y)


# ----------------------------------- small Gram sides with long rows (tiny route)
LONG_THIN = [(2, 16384), (16384, 3), (16, 16384), (17, 8192), (64, 16384), (65, 8192), (8192, 33), (1, 16384),
             (300, 200)]


@pytest.mark.parametrize("dt,frac", [("bf16", 1.0), ("bf16", 0.25), ("fp32", 1.0), ("fp32", 0.25)])
def test_small_gram_side_long_rows(dion, dt, frac):
    """Gram sides of 1 to 65 rows beside long sides up to 16384, in one call:
    sides up to 16 (any length) and up to 64 (length up to 1024) take the
    one-launch fp64 kernel, the others the GEMM path.  Indices bit-exact,
    unselected rows copied, each matrix within its path's gate (bf16 output:
    2e-2 on the GEMM path; fp32 on the FP64 path: 1e-4)."""
    Ms = [lowrank_np((31, i), r, c, max(1, min(r, c) // 4), 0.1, log_scale=(-3.0, 0.0))
          for i, (r, c) in enumerate(LONG_THIN)]
    if dt == "bf16":
        Ms = [round_bf16(M) for M in Ms]
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    outs, idxs = dion.orth_batched([torch.from_numpy(M).cuda().to(tdt) for M in Ms], restart_every=2,
                                   row_frac=frac, return_indices=True)
    for M, o, ix in zip(Ms, outs, idxs):
        ref, ref_idx = O.orthogonalize(M, restart_every=2, row_frac=frac)
        assert np.array_equal(ix.cpu().numpy(), ref_idx), M.shape
        got = to_np(o)
        rest = np.setdiff1d(np.arange(M.shape[0]), ref_idx)
        assert np.array_equal(got[rest], M[rest].astype(np.float64)), M.shape
        err = O.rel_frobenius(got[ref_idx], ref[ref_idx])
        print(f"{dt} {M.shape} rho {frac}: rel err {err:.2e}", flush=True)
        assert err <= (TOL_MFMA16 if dt == "bf16" else TOL_FP64), (M.shape, err)


# row-subset blocks of 3, 64, 17, 13, 12 (tall) and 5 rows at rho = 1/8
STEP_THIN = [(24, 16384), (512, 16384), (130, 8192), (100, 4096), (16384, 12), (40, 600)]


@pytest.mark.parametrize("ef", ["raw", "carry"])
def test_rowsubset_step_small_blocks(dion, ef):
    """Two row-subset steps whose selected blocks have Gram sides of 3 to 64 rows
    and long sides up to 16384: buffer and indices bit-exact, unselected output
    rows the raw momentum (raw) or zero (carry), selected rows within 2e-2."""
    beta, frac = 0.95, 0.125
    E_host = [np.zeros(s, np.float32) for s in STEP_THIN]
    E_dev = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in STEP_THIN]
    for t in range(2):
        G = [round_bf16(lowrank_np((32, t, i), r, c, 4, 0.05, log_scale=(-3.0, 0.0)))
             for i, (r, c) in enumerate(STEP_THIN)]
        outs, idxs = dion.rowsubset_step(E_dev, [to_dev_bf16(g) for g in G], beta, restart_every=2,
                                         row_frac=frac, return_indices=True, ef=ef)
        newE, ref_outs, ref_idxs = O.rowsubset_step(E_host, G, beta, ef=ef, n_iter=5, restart_every=2,
                                                    row_frac=frac)
        for i, s in enumerate(STEP_THIN):
            assert np.array_equal(E_dev[i].cpu().numpy().view(np.uint32), newE[i].view(np.uint32)), (s, t)
            assert_selection(idxs[i].cpu().numpy(), newE[i] if ef == "raw" else
                             np.add(E_host[i], G[i], dtype=np.float32), frac)
            got = to_np(outs[i])
            ix = ref_idxs[i]
            rest = np.setdiff1d(np.arange(s[0]), ix)
            want = round_bf16(newE[i][rest]).astype(np.float64) if ef == "raw" else np.zeros((len(rest), s[1]))
            assert np.array_equal(got[rest], want), (s, t)
            err = O.rel_frobenius(got[ix], ref_outs[i][ix])
            print(f"step {t} {s} ({ef}): selected rows rel err {err:.2e}", flush=True)
            assert err <= TOL_MFMA16, (s, t, err)
        E_host = newE


@pytest.mark.parametrize("wbf16,ef", [(True, "raw"), (False, "carry")])
def test_rowsubset_step_update_small_blocks(dion, wbf16, ef):
    """The fused weight update on the same small blocks: unselected weight rows
    bit-exact, selected rows within 2e-2 of the oracle's update (plus bf16 rounding)."""
    beta, wd, frac = 0.95, 0.01, 0.125
    alphas = [0.02 * float(np.sqrt(max(1.0, r / c))) for r, c in STEP_THIN]
    keep = float(np.float32(1.0) - np.float32(wd))
    rng = np.random.default_rng(12)
    W_host = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in STEP_THIN]
    if wbf16:
        W_host = [O.round_to_bf16(w) for w in W_host]
    W_dev = [torch.from_numpy(w).cuda().to(torch.bfloat16 if wbf16 else torch.float32) for w in W_host]
    E_host = [np.zeros(s, np.float32) for s in STEP_THIN]
    E_dev = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in STEP_THIN]
    for t in range(2):
        G = [round_bf16(lowrank_np((33, t, i), r, c, 4, 0.05, log_scale=(-3.0, 0.0)))
             for i, (r, c) in enumerate(STEP_THIN)]
        _, idxs = dion.rowsubset_step_update(E_dev, [to_dev_bf16(g) for g in G], W_dev, beta, alphas, wd,
                                             restart_every=2, row_frac=frac, return_indices=True, ef=ef)
        newE, newW, ref_idxs = O.rowsubset_step_update(E_host, G, W_host, beta, alphas, wd, bf16=wbf16, ef=ef,
                                                       n_iter=5, restart_every=2, row_frac=frac)
        for i, s in enumerate(STEP_THIN):
            assert np.array_equal(E_dev[i].cpu().numpy().view(np.uint32), newE[i].view(np.uint32)), (s, t)
            assert np.array_equal(idxs[i].cpu().numpy(), ref_idxs[i]), (s, t)
            got = to_np(W_dev[i])
            ix = ref_idxs[i]
            rest = np.setdiff1d(np.arange(s[0]), ix)
            assert np.array_equal(got[rest], newW[i][rest]), (s, t)
            base = W_host[i][ix].astype(np.float64) * keep
            d_ref = newW[i][ix] - base
            if wbf16:
                err = np.linalg.norm(got[ix] - newW[i][ix])
                assert err <= 2.0 ** -9 * 1.01 * np.linalg.norm(newW[i][ix]) + TOL_MFMA16 * np.linalg.norm(d_ref)
            else:
                assert O.rel_frobenius(got[ix] - base, d_ref) <= TOL_MFMA16, (s, t)
        E_host = newE
        W_host = [to_np(w).astype(np.float32) for w in W_dev]


def test_calls_never_block_the_host(dion):
    """Eight calls enqueued back to back return while the device is still on
    the first ones: the plan upload never waits on the host (a ring of pinned
    buffers, then kernel-argument uploads once the host is eight calls ahead)."""
    import time
    shapes = [(4096, 4096)] * 4
    Ms = [torch.from_numpy(round_bf16(lowrank_np((41, j), r, c, 64, 0.05))).cuda().to(torch.bfloat16)
          for j, (r, c) in enumerate(shapes)]
    outs = [torch.empty_like(M) for M in Ms]
    orth = dion.Orthogonalizer(shapes, "bf16", restart_every=2)
    for _ in range(10):            # warm up, and let the ring grow
        orth(Ms, outs)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    for n_calls in (8, 12):        # 12: beyond the ring, kernel-argument uploads
        t0 = time.perf_counter()
        for _ in range(n_calls):
            orth(Ms, outs)
        t_host = time.perf_counter() - t0
        pending = not torch.cuda.current_stream().query()
        torch.cuda.synchronize()
        t_all = time.perf_counter() - t0
        print(f"{n_calls} calls: enqueued in {1e3 * t_host:.1f} ms, done after {1e3 * t_all:.1f} ms", flush=True)
        assert pending and t_host < 0.25 * t_all
        for o, r in zip(outs, ref):
            assert torch.equal(o, r)


# ------------------------------------------------------ workspace in waves
def test_waves_bit_identical(dion):
    """A workspace smaller than the whole plan runs the batch in waves of
    consecutive matrices: outputs, indices, buffers and weights are bit-identical
    to one wave, for the batched call and both row-subset entry points."""
    from workloads import LLAMA3_8B_LAYER
    shapes = [(r // 4, c // 4) for _ in range(2) for _, r, c in LLAMA3_8B_LAYER] + [(5, 700), (3000, 40)]
    Ms = [torch.from_numpy(round_bf16(lowrank_np((42, j), r, c, 16, 0.05, log_scale=(-3.0, 0.0)))).cuda()
          .to(torch.bfloat16) for j, (r, c) in enumerate(shapes)]
    full = dion.workspace_size(shapes, "bf16", restart_every=2, row_frac=0.5)
    for budget in (full // 3, full // 6):
        need = dion.workspace_size(shapes, "bf16", restart_every=2, row_frac=0.5, budget=budget)
        assert need <= budget < full
        a, ia = dion.orth_batched(Ms, restart_every=2, row_frac=0.5, return_indices=True)
        b, ib = dion.orth_batched(Ms, restart_every=2, row_frac=0.5, return_indices=True, workspace_budget=budget)
        for x, y, u, v in zip(a, b, ia, ib):
            assert torch.equal(u, v) and torch.equal(x.view(torch.int16), y.view(torch.int16))
        print(f"orth waves at {budget / full:.2f} of the full workspace: bit-identical", flush=True)
    # the row-subset step and its fused update, two steps each
    Es = [[torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes] for _ in range(2)]
    Ws = [[torch.full(s, 0.01, dtype=torch.bfloat16, device="cuda") for s in shapes] for _ in range(2)]
    alphas = [0.02] * len(shapes)
    full_s = dion.workspace_size(shapes, "fp32", restart_every=2, row_frac=0.125, precision="mfma16")
    orths = [dion.Orthogonalizer(shapes, "fp32", restart_every=2, row_frac=0.125, precision="mfma16",
                                 step_mode=True, workspace_budget=b) for b in (None, full_s // 4)]
    assert orths[1].ws_bytes < full_s
    for t in range(2):
        G = [torch.from_numpy(round_bf16(lowrank_np((43, t, j), r, c, 8, 0.05))).cuda().to(torch.bfloat16)
             for j, (r, c) in enumerate(shapes)]
        outs = [[torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes] for _ in range(2)]
        sels = [torch.empty(orths[0].total_selected, dtype=torch.int32, device="cuda") for _ in range(2)]
        for k in range(2):
            orths[k].step(Es[k], G, outs[k], 0.95, sels[k])
        assert torch.equal(sels[0], sels[1])
        for x, y, e, f in zip(outs[0], outs[1], Es[0], Es[1]):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16)) and torch.equal(e, f)
        for k in range(2):
            orths[k].step_update(Es[k], G, Ws[k], 0.95, alphas, 0.01, sels[k])
        assert torch.equal(sels[0], sels[1])
        for x, y in zip(Ws[0], Ws[1]):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    print("row-subset waves: bit-identical", flush=True)
