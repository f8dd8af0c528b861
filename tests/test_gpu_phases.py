"""Parity of the phase entry points (one step of the path on its own, through
the C ABI) with the oracle's single steps: row keys and top-k, the Gram
matrix, the Gram polynomial and the apply on the Gram side.

Gates, derived from the arithmetic of each path:
  keys     bit-exact: both sides round the exact sum of squares once;
           selected rows bit-exact
  MFMA16   bf16 operands are exact in fp16 and products accumulate in fp32:
           relative Frobenius 2e-5 on fp32 outputs; fp32 operands of the Gram
           product take one fp16 term (2^-11 relative each): 2e-3; two-term
           operands (Q, G, fp32 X of the apply): 2e-5
  bf16 out round to nearest even: at most 2^-8 relative per element, so
           relative Frobenius 2^-8 + 2e-5
  FP64     only the final fp32 rounding: 1e-7
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import dion_oracle as O  # noqa: E402
from workloads import lowrank_np, round_bf16  # noqa: E402

pytestmark = pytest.mark.gpu

QUINTIC = (3.4445, -4.7750, 2.0315)
TOL_ACC = 2e-5
TOL_GRAM_FP32_ONE_TERM = 2e-3
TOL_BF16_OUT = 2.0 ** -8 + 2e-5
TOL_FP64 = 1e-7

SHAPES = [(7, 33), (33, 7), (300, 200), (200, 520), (1, 5), (5, 1), (257, 511), (64, 64)]


@pytest.fixture(scope="module")
def dion():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import orthogonalized_optimizer_step_amd as d
    return d


def dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(dt)


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def batch(seed, shapes, bf16=True):
    out = []
    for i, (r, c) in enumerate(shapes):
        M = lowrank_np((seed, i), r, c, max(1, min(r, c) // 8), 0.1, log_scale=(-3.0, 0.0))
        out.append(round_bf16(M) if bf16 else M.astype(np.float32))
    return out


def sym_unit_gram(seed, m):
    """Symmetric PSD fp32 matrix with spectral norm <= 1: the Gram matrix of a
    Frobenius-normalized random block, symmetrized before rounding."""
    S = lowrank_np((seed, m), m, m + 37, max(1, m // 4), 0.2)
    S = S / np.linalg.norm(S.astype(np.float64))
    G = O.gram(S)
    return ((G + G.T) / 2).astype(np.float32)


def assert_selection(idx_gpu, M, frac):
    ref = O.select_rows(M, frac)
    got = np.asarray(idx_gpu, dtype=np.int64)
    assert np.array_equal(got, ref), np.setxor1d(got, ref)


# ------------------------------------------------------------ rowkeys + top-k
@pytest.mark.parametrize("frac", [1.0, 0.5, 0.125, 1.0 / 37])
@pytest.mark.parametrize("bf16", [True, False])
def test_rowkeys_topk_random(dion, frac, bf16):
    Ms = batch(21, SHAPES, bf16)
    dt = torch.bfloat16 if bf16 else torch.float32
    keys, idx = dion.rowkeys_topk([dev(M, dt) for M in Ms], row_frac=frac)
    for M, k, ix in zip(Ms, keys, idx):
        ref = O.row_keys(M)
        got = k.cpu().numpy()
        assert np.array_equal(got.view(np.uint64), ref.view(np.uint64)), M.shape   # rounded once from the exact sum
        assert_selection(ix.cpu().numpy(), M, frac)


def test_rowkeys_topk_ties_and_zero_rows(dion):
    """Integer entries: keys are exact integers on both sides, so the
    selection (ties to the lower row index) must match bit for bit."""
    rng = np.random.default_rng(5)
    Ms = []
    for r, c in [(37, 16), (64, 20), (16, 300), (520, 40)]:
        M = rng.integers(-4, 5, size=(r, c)).astype(np.float32)
        M[rng.integers(0, r, size=r // 4)] = 0.0
        M[r // 2] = M[0]
        M[r - 1] = M[1]
        Ms.append(M)
    for frac in (0.25, 0.5, 1.0 / 37):
        keys, idx = dion.rowkeys_topk([dev(M, torch.bfloat16) for M in Ms], row_frac=frac)
        for M, k, ix in zip(Ms, keys, idx):
            assert np.array_equal(k.cpu().numpy(), O.row_keys(M))
            assert np.array_equal(ix.cpu().numpy(), O.select_rows(M, frac))


def test_rowkeys_topk_full_size(dion):
    """Llama-3-8B q and gate shapes at 1/8 of the rows, as the row-subset step selects."""
    Ms = [round_bf16(lowrank_np((3, 0, 0), 4096, 4096, 64, 0.05, log_scale=(-3, 0))),
          round_bf16(lowrank_np((3, 0, 4), 14336, 4096, 64, 0.05, log_scale=(-3, 0)))]
    keys, idx = dion.rowkeys_topk([dev(M, torch.bfloat16) for M in Ms], row_frac=0.125)
    for M, k, ix in zip(Ms, keys, idx):
        ref = O.row_keys(M)
        assert np.array_equal(k.cpu().numpy().view(np.uint64), ref.view(np.uint64))
        assert_selection(ix.cpu().numpy(), M, 0.125)


T27 = 2.0 ** -27   # T27^2 = 2^-54: two such squares add exactly half an ulp of 1.0


def adversarial_matrix(dtype, cols, seed):
    """Rows of random values mixed with rows whose exact sum of squares sits on
    a rounding midpoint of the doubles, a hair above one (only an exact sum
    tells), or spreads over hundreds of bits, placed at varied columns so that
    different lanes hold them; all values exact in `dtype`."""
    rng = np.random.default_rng(seed)
    if dtype == "fp16":   # fp16 squares span 2^-48 .. 2^32: ties against 2^30
        big, t, tiny, far = 32768.0, 2.0 ** -12, 2.0 ** -24, 2.0 ** -24
    else:                 # bf16 and fp32 share the exponent range
        big, t, tiny, far = 1.0, T27, 2.0 ** -100, 2.0 ** (-133 if dtype == "bf16" else -149)
    rows = []
    for j in range(24):
        r = np.zeros(cols, np.float32)
        c = rng.choice(cols, size=4, replace=False)
        kind = j % 6
        if kind == 0:
            r[:] = rng.standard_normal(cols)
        elif kind == 1:                          # a tie: ties to even
            r[c[:3]] = [big, t, t]
        elif kind == 2:                          # just above the tie
            r[c] = [big, t, t, tiny]
        elif kind == 3:                          # squares spread far apart
            r[c] = [big * 1.5, far, tiny, -t]
        elif kind == 4:                          # random values plus one far below them
            r[:] = rng.standard_normal(cols)
            r[c[0]] = far
        else:                                    # equal to a tie row's key: ties to the lower row
            r[c[0]] = big
        rows.append(r)
    # random rows with one value far below the others: for 16-bit inputs the
    # eight values of its 16-byte load no longer sum exactly in one double, and
    # are added one at a time
    for e in ((16, 20) if dtype == "fp16" else (20, 40)):
        r = rng.standard_normal(cols).astype(np.float32)
        r[rng.integers(cols)] = np.float32(2.0 ** -e)
        rows.append(r)
    if cols > 4096:
        # random rows whose columns from 4096 on are scaled by a power of two:
        # each load holds values of one scale and sums exactly on its own, and
        # the loads' sums, up to 2^52 apart, meet only in the exact pair
        for e in ((6, 12) if dtype == "fp16" else (8, 14, 20, 26)):
            r = rng.standard_normal(cols).astype(np.float32)
            r[4096:] *= np.float32(2.0 ** -e)
            rows.append(r)
    A = np.stack(rows)
    if dtype == "bf16":
        A = round_bf16(A)
    elif dtype == "fp16":
        A = A.astype(np.float16).astype(np.float32)
    return A


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("cols", [9216, 640, 333, 64, 5])
def test_rowkeys_exact_rounding(dion, dtype, cols):
    """Keys bit-equal to the exact sum of squares rounded once, on rows built to
    defeat any fixed summation order (ties, a hair above a tie, squares hundreds
    of bits apart): the first exercise the exact fast paths, the others the
    exact integer fallback; 9216, 640 and 64 columns take 16-byte loads (at 9216
    eighteen per lane), 333 and 5 do not."""
    A = adversarial_matrix(dtype, cols, seed=cols)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dtype]
    for frac in (1.0 / 8, 0.5):
        keys, idx = dion.rowkeys_topk([dev(A, tdt)], row_frac=frac)
        ref = O.row_keys(A)
        got = keys[0].cpu().numpy()
        assert np.array_equal(got.view(np.uint64), ref.view(np.uint64)), np.flatnonzero(got != ref)
        assert_selection(idx[0].cpu().numpy(), A, frac)


@pytest.mark.parametrize("gdt", ["bf16", "fp32"])
def test_momentum_keys_exact_rounding(dion, gdt):
    """The momentum pass's keys decide the row-subset step's selection: with
    beta = 0 the new buffer is the gradient itself, built from adversarial rows;
    the selection must match the oracle's exactly and the buffer bit for bit."""
    A = adversarial_matrix("bf16" if gdt == "bf16" else "fp32", 640, seed=9)
    E = torch.zeros(A.shape, dtype=torch.float32, device="cuda")
    G = dev(A, torch.bfloat16 if gdt == "bf16" else torch.float32)
    for frac in (1.0 / 8, 1.0 / 3):
        outs, idx = dion.rowsubset_step([E], [G], 0.0, row_frac=frac, return_indices=True)
        assert np.array_equal(E.cpu().numpy().view(np.uint32), A.view(np.uint32))
        assert_selection(idx[0].cpu().numpy(), A, frac)


# ------------------------------------------------------------------- Gram
@pytest.mark.parametrize("prec,bf16,tol", [("mfma16", True, TOL_ACC), ("mfma16", False, TOL_GRAM_FP32_ONE_TERM),
                                           ("fp64", False, TOL_FP64), ("fp64", True, TOL_FP64)])
def test_syrk_ragged(dion, prec, bf16, tol):
    Ms = batch(22, SHAPES, bf16)
    dt = torch.bfloat16 if bf16 else torch.float32
    Gs = dion.syrk([dev(M, dt) for M in Ms], precision=prec)
    errs = [O.rel_frobenius(to_np(G), O.gram(M)) for M, G in zip(Ms, Gs)]
    print(f"syrk {prec} {'bf16' if bf16 else 'fp32'}:", " ".join(f"{e:.1e}" for e in errs), flush=True)
    assert max(errs) <= tol


def test_syrk_zero_matrix(dion):
    Gs = dion.syrk([torch.zeros((12, 40), dtype=torch.bfloat16, device="cuda")], precision="mfma16")
    assert torch.count_nonzero(Gs[0]) == 0 and tuple(Gs[0].shape) == (12, 12)


def test_syrk_full_size(dion):
    """Three 4096 x 4096 and one 14336 x 4096 (tall: X^T X) bf16 matrices:
    544 upper-triangle tiles, so the 256 x 256 tile kernel the benchmark runs."""
    shapes = [(4096, 4096)] * 3 + [(14336, 4096)]
    Ms = [round_bf16(lowrank_np((3, 0, j), r, c, 64, 0.05, log_scale=(-3, 0))) for j, (r, c) in enumerate(shapes)]
    Gs = dion.syrk([dev(M, torch.bfloat16) for M in Ms], precision="mfma16")
    errs = [O.rel_frobenius(to_np(G), O.gram(M)) for M, G in zip(Ms, Gs)]
    print("syrk full size:", " ".join(f"{e:.1e}" for e in errs), flush=True)
    assert max(errs) <= TOL_ACC


# -------------------------------------------------------- Gram polynomial
@pytest.mark.parametrize("prec,tol", [("mfma16", TOL_ACC), ("fp64", TOL_FP64)])
@pytest.mark.parametrize("coeffs", [QUINTIC, (1.5, -0.5, 0.0), (3.4445 / 1.05, -4.7750 / 1.05 ** 3,
                                                                 2.0315 / 1.05 ** 5)])
def test_sympoly(dion, prec, tol, coeffs):
    Gs = [sym_unit_gram(23, m) for m in (1, 7, 64, 257, 300)]
    Ps = dion.sympoly([torch.from_numpy(G).cuda() for G in Gs], coeffs=coeffs, precision=prec)
    errs = [O.rel_frobenius(to_np(P), O.gram_polynomial(G, *coeffs)) for G, P in zip(Gs, Ps)]
    print(f"sympoly {prec} {coeffs}:", " ".join(f"{e:.1e}" for e in errs), flush=True)
    assert max(errs) <= tol


def test_sympoly_full_size(dion):
    """Four 4096 x 4096 Gram matrices (544 upper tiles: the 256-tile kernel)."""
    Gs = [sym_unit_gram(24 + i, 4096) for i in range(4)]
    Ps = dion.sympoly([torch.from_numpy(G).cuda() for G in Gs], precision="mfma16")
    errs = [O.rel_frobenius(to_np(P), O.gram_polynomial(G, *QUINTIC)) for G, P in zip(Gs, Ps)]
    print("sympoly full size:", " ".join(f"{e:.1e}" for e in errs), flush=True)
    assert max(errs) <= TOL_ACC


# ------------------------------------------------------------------ apply
def general_factor(seed, m):
    """A nonsymmetric fp32 m x m factor: a transposed operand changes the result."""
    rng = np.random.default_rng([seed, m])
    return (rng.standard_normal((m, m)) / np.sqrt(m) + np.eye(m)).astype(np.float32)


@pytest.mark.parametrize("prec,bf16,tol", [("mfma16", True, TOL_BF16_OUT), ("mfma16", False, TOL_ACC),
                                           ("fp64", False, TOL_FP64)])
def test_apply_ragged(dion, prec, bf16, tol):
    Xs = batch(25, SHAPES, bf16)
    Qs = [general_factor(25, min(X.shape)) for X in Xs]
    dt = torch.bfloat16 if bf16 else torch.float32
    Ys = dion.apply([torch.from_numpy(Q).cuda() for Q in Qs], [dev(X, dt) for X in Xs], precision=prec)
    errs = [O.rel_frobenius(to_np(Y), O.apply_factor(Q, X)) for Q, X, Y in zip(Qs, Xs, Ys)]
    print(f"apply {prec} {'bf16' if bf16 else 'fp32'}:", " ".join(f"{e:.1e}" for e in errs), flush=True)
    assert max(errs) <= tol
    if bf16:  # elementwise: within 2^-8 of each exact value, plus the accumulation
        for Q, X, Y in zip(Qs, Xs, Ys):
            ref = O.apply_factor(Q, X)
            assert np.all(np.abs(to_np(Y) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5 * np.abs(ref).max())


def test_apply_zero_operand(dion):
    X = torch.zeros((12, 40), dtype=torch.bfloat16, device="cuda")
    Q = torch.from_numpy(general_factor(1, 12)).cuda()
    Y = dion.apply([Q], [X], precision="mfma16")[0]
    assert torch.count_nonzero(Y) == 0


def test_apply_full_size(dion):
    """The down (4096 x 14336, Q X) and gate (14336 x 4096, X Q) shapes with
    4096 x 4096 factors: 896 tiles each, the 256-tile kernel."""
    Xs = [round_bf16(lowrank_np((3, 0, 6), 4096, 14336, 64, 0.05, log_scale=(-3, 0))),
          round_bf16(lowrank_np((3, 0, 4), 14336, 4096, 64, 0.05, log_scale=(-3, 0)))]
    Qs = [general_factor(26, 4096), general_factor(27, 4096)]
    Ys = dion.apply([torch.from_numpy(Q).cuda() for Q in Qs], [dev(X, torch.bfloat16) for X in Xs],
                    precision="mfma16")
    errs = [O.rel_frobenius(to_np(Y), O.apply_factor(Q, X)) for Q, X, Y in zip(Qs, Xs, Ys)]
    print("apply full size:", " ".join(f"{e:.1e}" for e in errs), flush=True)
    assert max(errs) <= TOL_BF16_OUT


def test_phases_fp16(dion):
    """The phase entry points on fp16 inputs (exact in one fp16 term)."""
    Ms = [M.astype(np.float16).astype(np.float32) for M in batch(27, SHAPES, bf16=False)]
    dev16 = [torch.from_numpy(M).cuda().to(torch.float16) for M in Ms]
    keys, idx = dion.rowkeys_topk(dev16, row_frac=0.25)
    for M, k, ix in zip(Ms, keys, idx):
        ref = O.row_keys(M)
        assert np.all(np.abs(k.cpu().numpy() - ref) <= 1e-12 * ref + 1e-300)
        assert_selection(ix.cpu().numpy(), M, 0.25)
    Gs = dion.syrk(dev16, precision="mfma16")
    assert max(O.rel_frobenius(to_np(G), O.gram(M)) for M, G in zip(Ms, Gs)) <= TOL_ACC
    Qs = [general_factor(28, min(M.shape)) for M in Ms]
    Ys = dion.apply([torch.from_numpy(Q).cuda() for Q in Qs], dev16, precision="mfma16")
    errs = [O.rel_frobenius(to_np(Y), O.apply_factor(Q, M)) for Q, M, Y in zip(Qs, Ms, Ys)]
    assert all(Y.dtype == torch.float16 for Y in Ys)
    assert max(errs) <= 2.0 ** -11 + TOL_ACC   # fp16 output rounding plus the accumulation
