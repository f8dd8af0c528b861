"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test names what it pins.  None retypes the oracle's iteration: the
references are the SVD closed form, a library polar factor, exact rational
arithmetic, the plain (non-Gram) Newton-Schulz iteration, invariances, brute
force and scalar IEEE emulation.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

from oracle import dion_oracle as O
from workloads import QUINTIC, fp32_64x128, heavytail_np, lowrank_np, round_bf16

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------- helpers
def scalar_map(x, coeffs, n_iter, safety=1.0):
    """The NS polynomial applied to a singular value: x <- f(x / s), K times."""
    trip = np.tile(np.asarray(coeffs, float), (n_iter, 1)) if np.ndim(coeffs) == 1 else np.asarray(coeffs)
    y = np.asarray(x, dtype=np.float64)
    for a, b, c in trip:
        t = y / safety
        y = a * t + b * t ** 3 + c * t ** 5
    return y


def svd_closed_form(M, coeffs, n_iter, safety=1.0):
    """U diag(f^K(sigma / ||M||_F)) V^T, the exact-arithmetic output of NS."""
    M = np.asarray(M, dtype=np.float64)
    U, s, Vt = np.linalg.svd(M, full_matrices=False)
    nu = np.linalg.norm(M)
    return (U * scalar_map(s / nu, coeffs, n_iter, safety)) @ Vt


def exact_f(x: Fraction, coeffs, n_iter, safety=Fraction(1)) -> Fraction:
    a, b, c = (Fraction(str(v)) for v in coeffs)
    for _ in range(n_iter):
        t = x / safety
        x = a * t + b * t ** 3 + c * t ** 5
    return x


def f32(x: float) -> float:
    return struct.unpack("f", struct.pack("f", x))[0]


def rand_lowrank(R, C, rank, noise, rng=RNG):
    return rng.standard_normal((R, rank)) @ rng.standard_normal((rank, C)) + noise * rng.standard_normal((R, C))


# ------------------------------------------------- P6: exact scalar values
def test_scalar_map_exact_values():
    """f^5(1) for the fixed quintic, by exact rational arithmetic, matches the
    value worked out independently (0.696436409469752), and the fp64 scalar
    loop used by the SVD pin reproduces it."""
    v = exact_f(Fraction(1), QUINTIC, 5)
    assert abs(float(v) - 0.696436409469752) < 1e-14
    assert abs(scalar_map(1.0, QUINTIC, 5) - float(v)) < 1e-13
    v101 = exact_f(Fraction(1), QUINTIC, 5, Fraction("1.01"))
    assert abs(float(v101) - 0.709030164453003) < 1e-14
    v6 = exact_f(Fraction(1), QUINTIC, 6, Fraction("1.05"))
    assert abs(float(v6) - 1.136014264217548) < 1e-14
    v8 = exact_f(Fraction(1, 8), QUINTIC, 5)
    assert abs(float(v8) - 0.688139855776055) < 1e-14


def test_scalar_map_textbook_cubic_converges():
    """Cubic NS (1.5, -0.5, 0) is the textbook polar iteration: from 0.1 it
    reaches 1 to 1e-15 within 11 steps, and fixes 1 exactly."""
    assert abs(float(exact_f(Fraction(1), (1.5, -0.5, 0.0), 7)) - 1.0) == 0.0
    assert abs(scalar_map(0.1, (1.5, -0.5, 0.0), 11) - 1.0) < 1e-15


# -------------------------------------------------- P1: SVD closed form
@pytest.mark.parametrize("shape", [(64, 128), (128, 64), (48, 48), (7, 33), (33, 7), (1, 9), (9, 1)])
@pytest.mark.parametrize("sched", [dict(), dict(restart_every=2), dict(restart_mask=0b10),
                                   dict(restart_every=1)])
@pytest.mark.parametrize("ns", [(5, 1.0), (5, 1.01), (6, 1.05)])
def test_svd_closed_form(shape, sched, ns):
    n_iter, safety = ns
    M = rand_lowrank(*shape, rank=min(4, *shape), noise=0.1)
    out, idx = O.orthogonalize(M, n_iter=n_iter, safety=safety, **sched)
    ref = svd_closed_form(M, QUINTIC, n_iter, safety)
    assert list(idx) == list(range(shape[0]))
    assert O.rel_frobenius(out, ref) < 1e-10


def test_svd_closed_form_fp32_workload():
    """The fp32 64x128 workload: oracle vs SVD closed form."""
    M = fp32_64x128()
    out, _ = O.orthogonalize(M, n_iter=5)
    assert O.rel_frobenius(out, svd_closed_form(M, QUINTIC, 5)) < 1e-11


def test_per_iteration_coefficients():
    """A per-iteration schedule is applied in order (closed form per step)."""
    sched = [(3.4445, -4.7750, 2.0315), (2.0, -1.5, 0.5), (1.5, -0.5, 0.0)]
    M = rand_lowrank(20, 30, 3, 0.2)
    out, _ = O.orthogonalize(M, coeffs=sched, n_iter=3, restart_every=1, safety=1.02)
    assert O.rel_frobenius(out, svd_closed_form(M, sched, 3, 1.02)) < 1e-11
    out_rev, _ = O.orthogonalize(M, coeffs=sched[::-1], n_iter=3, safety=1.02)
    assert O.rel_frobenius(out_rev, out) > 1e-3


# ------------------------------------------------ P2: textbook polar factor
@pytest.mark.parametrize("shape", [(6, 10), (10, 6), (8, 8)])
def test_polar_factor_cubic(shape):
    """With the cubic (1.5, -0.5, 0) the iteration converges to the polar
    factor; scipy's polar decomposition is the independent reference."""
    R, C = shape
    r = min(R, C)
    U, _ = np.linalg.qr(RNG.standard_normal((R, r)))
    V, _ = np.linalg.qr(RNG.standard_normal((C, r)))
    s = np.linspace(0.2, 1.0, r)
    M = (U * s) @ V.T          # normalized singular values in [0.1, 0.6]
    out, _ = O.orthogonalize(M, coeffs=(1.5, -0.5, 0.0), n_iter=40, restart_every=3)
    if R >= C:
        Up, _ = scipy.linalg.polar(M, side="right")
    else:
        Up, _ = scipy.linalg.polar(M.T, side="right")
        Up = Up.T
    assert np.max(np.abs(out - Up)) < 1e-12


# ------------------------------------------------------ P3: band invariant
THR = {(5, 1.0): 1.505e-3, (5, 1.01): 1.582e-3, (5, 1.05): 1.922e-3,
       (6, 1.0): 4.37e-4, (6, 1.01): 4.64e-4, (6, 1.05): 5.86e-4}


@pytest.mark.parametrize("ns", sorted(THR))
def test_band_invariant(ns):
    """Output singular values never exceed 1.20237, and those whose
    normalized input is above the capture threshold land in
    [0.68183, 1.20237]."""
    n_iter, safety = ns
    for shape in [(40, 90), (90, 40)]:
        r = min(shape)
        U, _ = np.linalg.qr(RNG.standard_normal((shape[0], r)))
        V, _ = np.linalg.qr(RNG.standard_normal((shape[1], r)))
        s = np.geomspace(1e-5, 1.0, r)
        M = (U * s) @ V.T
        out, _ = O.orthogonalize(M, n_iter=n_iter, restart_every=2, safety=safety)
        s0 = np.linalg.svd(M, compute_uv=False) / np.linalg.norm(M)
        s1 = np.linalg.svd(out, compute_uv=False)
        assert s1.max() <= 1.20237 + 1e-9
        # singular values keep their order under the monotone-on-[0,1] map
        captured = s1[s0 >= THR[ns]]
        assert captured.size > 0
        assert captured.min() >= 0.68183 - 1e-9 and captured.max() <= 1.20237 + 1e-9


# -------------------------------------------- P4: Gram NS == plain NS
def plain_ns(M, coeffs, n_iter, safety):
    """Muon-style Newton-Schulz on the full matrix: X <- aX + (bA + cA^2)X."""
    X = np.asarray(M, float)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    X = X / np.linalg.norm(X)
    for _ in range(n_iter):
        a, b, c = coeffs[0] / safety, coeffs[1] / safety ** 3, coeffs[2] / safety ** 5
        A = X @ X.T
        X = a * X + b * (A @ X) + c * (A @ (A @ X))
    return X.T if tall else X


@pytest.mark.parametrize("sched", [dict(), dict(restart_every=2), dict(restart_mask=0b101)])
@pytest.mark.parametrize("shape", [(30, 70), (70, 30)])
def test_gram_equals_plain_ns(sched, shape):
    M = rand_lowrank(*shape, rank=5, noise=0.05)
    out, _ = O.orthogonalize(M, n_iter=5, safety=1.01, **sched)
    assert O.rel_frobenius(out, plain_ns(M, QUINTIC, 5, 1.01)) < 1e-12


# ------------------------------------------------------- P5: invariances
def test_invariances():
    M = rand_lowrank(24, 40, 3, 0.1)
    kw = dict(n_iter=5, restart_every=2)
    base, _ = O.orthogonalize(M, **kw)
    assert O.rel_frobenius(O.orthogonalize(7.3e-3 * M, **kw)[0], base) < 1e-12
    assert O.rel_frobenius(O.orthogonalize(-M, **kw)[0], -base) < 1e-12
    assert O.rel_frobenius(O.orthogonalize(M.T, **kw)[0], base.T) < 1e-12
    U1, _ = np.linalg.qr(RNG.standard_normal((24, 24)))
    V1, _ = np.linalg.qr(RNG.standard_normal((40, 40)))
    rot, _ = O.orthogonalize(U1 @ M @ V1.T, **kw)
    assert O.rel_frobenius(rot, U1 @ base @ V1.T) < 1e-11
    perm = RNG.permutation(24)
    assert O.rel_frobenius(O.orthogonalize(M[perm], **kw)[0], base[perm]) < 1e-12


# ------------------------------------------- P6: special cases, exact values
def test_rank_one_exact():
    u = RNG.standard_normal(17)
    v = RNG.standard_normal(29)
    out, _ = O.orthogonalize(np.outer(u, v), n_iter=5, restart_every=2)
    expect = 0.696436409469752 * np.outer(u / np.linalg.norm(u), v / np.linalg.norm(v))
    assert np.max(np.abs(out - expect)) < 1e-13


def test_orthonormal_rows_exact():
    Q, _ = np.linalg.qr(RNG.standard_normal((200, 64)))
    M = 3.0 * Q.T                            # 64 orthonormal rows, scaled
    out, _ = O.orthogonalize(M, n_iter=5)
    assert np.max(np.abs(out - 0.688139855776055 * Q.T)) < 1e-13


def test_diagonal_worked_example():
    """[[3,0,0],[0,4,0]]: nu = 5, singular values 0.6, 0.8 map separately."""
    M = np.array([[3.0, 0, 0], [0, 4.0, 0]])
    out, _ = O.orthogonalize(M, n_iter=5)
    e6 = float(exact_f(Fraction(3, 5), QUINTIC, 5))
    e8 = float(exact_f(Fraction(4, 5), QUINTIC, 5))
    assert np.max(np.abs(out - np.array([[e6, 0, 0], [0, e8, 0]]))) < 1e-14


def test_zero_matrix():
    out, idx = O.orthogonalize(np.zeros((5, 7)), n_iter=5, row_frac=0.4)
    assert np.all(out == 0) and list(idx) == [0, 1]


# -------------------------------------------------- P7: row selection
def brute_force_select(M, k):
    keys = [sum(int(v) * int(v) for v in row) for row in np.asarray(M)]
    order = sorted(range(len(keys)), key=lambda j: (-keys[j], j))
    return sorted(order[:k])


@pytest.mark.parametrize("R,C,frac", [(16, 5, 0.25), (37, 4, 0.5), (8, 3, 1 / 8), (40, 6, 1.0),
                                      (9, 9, 1 / 9), (64, 2, 0.125), (12, 30, 0.75)])
def test_selection_brute_force_with_ties(R, C, frac):
    rng = np.random.default_rng(R * 100 + C)
    M = rng.integers(-3, 4, size=(R, C)).astype(np.float64)
    M[rng.integers(0, R, size=R // 3)] = 0.0           # zero rows
    M[R // 2] = M[0]                                    # exact duplicates
    M[R - 1] = M[1]
    k = O.selected_count(R, frac)
    assert list(O.select_rows(M, frac)) == brute_force_select(M, k)


# ------------------------------------ P7: row keys, rounded once from the exact sum
def exact_key(row) -> float:
    """The exact sum of the squares as a Fraction, rounded once by float():
    CPython's int / int true division is correctly rounded, ties to even."""
    s = sum((Fraction(float(v)) ** 2 for v in row), Fraction(0))
    return float(s)


T27 = 2.0 ** -27   # T27^2 = 2^-54: two of them add exactly half an ulp of 1.0
ADVERSARIAL_ROWS = [
    ([1.0, T27, T27], "tie"),                              # 1 + 2^-53: ties to even -> 1
    ([1.0, T27, T27, 2.0 ** -100], "above"),               # a hair above the tie -> 1 + 2^-52
    ([1.0, 3 * 2.0 ** -26, T27, T27], "tie"),              # 1 + 2^-49 + 2^-52 + 2^-53: odd below -> up
    ([T27, 1.0, T27], "tie"),                              # the same tie in another order
    ([2.0 ** -149, 2.0 ** -149, 2.0 ** -140], "small"),    # subnormal squares (2^-298)
    ([1.5 * 2.0 ** 127, 2.0 ** -100, 2.0 ** -149, -(2.0 ** 126)], "spread"),   # squares over 550 bits
    ([0.0, -0.0, 0.0], "zero"),
    ([-1.0, -T27, -T27], "tie"),                           # signs do not matter
]


def _is_midpoint(row):
    s = sum((Fraction(float(v)) ** 2 for v in row), Fraction(0))
    r = float(s)
    if Fraction(r) == s:
        return False
    lo, hi = (r, math.nextafter(r, math.inf)) if Fraction(r) < s else (math.nextafter(r, 0.0), r)
    return 2 * s == Fraction(lo) + Fraction(hi)


def test_row_keys_adversarial_exact():
    """Rows on a rounding midpoint of the doubles (ties to even), a hair off one,
    with subnormal squares and with squares spread over 550 bits: the keys equal
    the exact sum rounded once (Fraction) and the fsum definition."""
    width = max(len(r) for r, _ in ADVERSARIAL_ROWS)
    M = np.zeros((len(ADVERSARIAL_ROWS), width), np.float32)
    for i, (r, kind) in enumerate(ADVERSARIAL_ROWS):
        M[i, :len(r)] = np.float32(r)
        assert np.array_equal(M[i, :len(r)].astype(np.float64), np.asarray(r)), "inputs must be float32 values"
        assert _is_midpoint(r) == (kind == "tie"), (i, kind)
    got = O.row_keys(M)
    want = np.array([exact_key(row) for row in M])
    assert np.array_equal(got.view(np.uint64), want.view(np.uint64))
    assert np.array_equal(got.view(np.uint64), O.row_keys_fsum(M).view(np.uint64))
    assert got[0] == 1.0 and got[1] == 1.0 + 2.0 ** -52 and got[2] == 1.0 + 2.0 ** -49 + 2.0 ** -51
    # the plain fp64 sum in row order rounds the first tie away from the exact answer's neighbour
    assert float(np.sum(np.float64(M[2]) ** 2)) != got[2] or float(np.sum(np.float64(M[1]) ** 2)) != got[1]


@pytest.mark.parametrize("kind", ["normal", "bf16", "fp16", "wide", "sparse", "fp64"])
def test_row_keys_equal_fsum_and_fractions(kind):
    """On random float32 data of several kinds, bit-equal to math.fsum of the exact
    squares, and (on a subset) to the Fraction sum rounded once; permuting the
    columns changes no key (the definition has no summation order)."""
    rng = np.random.default_rng({"normal": 1, "bf16": 2, "fp16": 3, "wide": 4, "sparse": 5, "fp64": 6}[kind])
    A = rng.standard_normal((200, 333)).astype(np.float32)
    if kind == "fp64":   # doubles that are not float32 values: the Veltkamp-split fsum branch
        A = rng.standard_normal((200, 333)) * 10.0 ** rng.uniform(-100, 100, (200, 333))
    if kind == "bf16":
        A = round_bf16(A * 10.0 ** rng.uniform(-3, 3, (200, 1)))
    elif kind == "fp16":
        A = (A * 10.0 ** rng.uniform(-6, 4, A.shape)).astype(np.float16).astype(np.float32)
    elif kind == "wide":
        A = (A * 10.0 ** rng.uniform(-45, 38, A.shape)).astype(np.float32)
    elif kind == "sparse":
        A[rng.random(A.shape) < 0.9] = 0.0
        A[:5] = 0.0
    got = O.row_keys(A)
    assert np.array_equal(got.view(np.uint64), O.row_keys_fsum(A).view(np.uint64))
    for i in range(0, 200, 40):
        assert got[i] == exact_key(A[i])
    perm = rng.permutation(A.shape[1])
    assert np.array_equal(O.row_keys(A[:, perm]).view(np.uint64), got.view(np.uint64))
    if kind == "normal":   # einsum's summation order differs from the rounded exact sum on most rows
        assert np.count_nonzero(np.einsum("ij,ij->i", A.astype(np.float64), A.astype(np.float64)) != got) > 20


def test_selection_follows_rounded_exact_keys():
    """Rows whose exact sums differ below the doubles' spacing rank by their rounded
    keys, and equal keys rank by row index (brute force on Fraction keys)."""
    rows = [[1.0, T27, T27], [1.0], [1.0, T27, T27, 2.0 ** -100], [0.5, 0.5, 0.5, 0.5], [1.0, 2.0 ** -120]]
    M = np.zeros((len(rows), 4), np.float32)
    for i, r in enumerate(rows):
        M[i, :len(r)] = r
    keys = [exact_key(r) for r in M]
    for k in range(1, len(rows) + 1):
        order = sorted(range(len(rows)), key=lambda j: (-keys[j], j))
        assert list(O.select_rows(M, k / len(rows))) == sorted(order[:k])
    assert list(O.select_rows(M, 0.2)) == [2]         # the one key above 1.0
    assert list(O.select_rows(M, 0.4)) == [0, 2]      # then the first of four keys equal to 1.0


def test_selected_count():
    assert O.selected_count(4096, 0.125) == 512
    assert O.selected_count(14336, 0.125) == 1792
    assert O.selected_count(28672, 0.25) == 7168
    assert O.selected_count(1000, float(np.float32(0.1))) == 100
    assert O.selected_count(7, 0.5) == 4
    assert O.selected_count(5, 1e-6) == 1
    assert O.selected_count(5, 1.0) == 5


def test_rowsubset_output_structure():
    """Unselected rows are copied; the selected block (tall here: 12 > 8
    columns) equals the closed form of that block alone."""
    M = rand_lowrank(24, 8, 2, 0.3)
    out, idx = O.orthogonalize(M, n_iter=5, restart_every=2, row_frac=0.5)
    keys = np.sum(M * M, axis=1)
    assert set(idx) == set(np.argsort(-keys, kind="stable")[:12])
    rest = np.setdiff1d(np.arange(24), idx)
    assert np.array_equal(out[rest], M[rest])
    assert O.rel_frobenius(out[idx], svd_closed_form(M[idx], QUINTIC, 5)) < 1e-11


# ------------------------------------------- P8: fp32 momentum, bit exact
def test_momentum_bit_exact_scalar_emulation():
    rng = np.random.default_rng(7)
    E = (rng.standard_normal(3000) * 10.0 ** rng.uniform(-40, 30, 3000)).astype(np.float32)
    G = round_bf16((rng.standard_normal(3000) * 10.0 ** rng.uniform(-40, 30, 3000)).astype(np.float32))
    E[:5] = [0.0, -0.0, 1.0, 1e-45, 3.4e38]
    got = O.momentum_update(E, G, 0.95)
    beta = f32(0.95)
    for e, g, r in zip(E.tolist(), G.tolist(), got.tolist()):
        want = f32(f32(beta * e) + g)      # each op exact in fp64, rounded once
        assert struct.pack("f", want) == struct.pack("f", r)


def test_momentum_is_not_fma():
    """Two roundings differ from a fused multiply-add on some inputs."""
    rng = np.random.default_rng(11)
    E = rng.standard_normal(200000).astype(np.float32)
    G = round_bf16(rng.standard_normal(200000).astype(np.float32))
    got = O.momentum_update(E, G, 0.95)
    fma = (np.float64(np.float32(0.95)) * E.astype(np.float64) + G.astype(np.float64)).astype(np.float32)
    assert np.any(got != fma)


def test_momentum_steps_recurrence():
    """Two steps of the batch rule: E_t = M_t and out = orth(M_t)."""
    E = [np.zeros((16, 24), np.float32)]
    for t in range(2):
        G = [round_bf16(lowrank_np((9, t), 16, 24, 2, 0.1))]
        newE, outs, idxs = O.rowsubset_step(E, G, 0.95, n_iter=5, restart_every=2, row_frac=0.25)
        Mt = O.momentum_update(E[0], G[0], 0.95)
        assert np.array_equal(newE[0], Mt)
        assert np.array_equal(outs[0][np.setdiff1d(np.arange(16), idxs[0])],
                              Mt[np.setdiff1d(np.arange(16), idxs[0])].astype(np.float64))
        E = newE


# ------------------------------------------ workload shapes and sanity
def test_heavytail_generator_spectrum():
    M = heavytail_np((5, 0, 0), 60, 40)
    s = np.linalg.svd(M.astype(np.float64), compute_uv=False)
    assert np.allclose(s, np.arange(1, 41) ** -0.5, rtol=1e-5)


def test_hyperparameter_expansion():
    assert O.restart_points(5, restart_every=2) == [2, 4]
    assert O.restart_points(6, restart_every=2) == [2, 4]
    assert O.restart_points(5, restart_mask=0b10) == [2]
    assert O.restart_points(5, restart_mask=0b10000) == []
    assert O.restart_points(5) == []
    sch = O.coefficient_schedule(QUINTIC, 2, 1.05)
    assert sch[0] == (3.4445 / 1.05, -4.7750 / 1.05 ** 3, 2.0315 / 1.05 ** 5)
    with pytest.raises(ValueError):
        O.coefficient_schedule([QUINTIC, QUINTIC], 3)
    assert math.isclose(O.rel_frobenius(np.ones(3), np.ones(3) * 2), 0.5)


@pytest.mark.parametrize("tau,safety,n_iter", [(100.0, 1.0, 5), (100.0, 1.0, 9), (1000.0, 1.0, 7), (5.0, 1.0, 4),
                                                 (1e4, 1.0, 5), (116.0, 1.0, 6), (116.0, 1.05, 6), (1e30, 1.0, 5)])
def test_restart_threshold_closed_form(tau, safety, n_iter):
    """Reading R12 with one fixed triple: the growth per iteration is the constant
    (a/s)^2, so segments have the length L = ceil(ln tau / ln (a/s)^2) and the
    restarts fall on the multiples of L below K (taus chosen away from ties)."""
    g = (QUINTIC[0] / safety) ** 2
    L = max(1, math.ceil(math.log(tau) / math.log(g)))
    expect = [k for k in range(L, n_iter, L)]
    sched = O.coefficient_schedule(QUINTIC, n_iter, safety)
    assert O.restart_points(n_iter, restart_threshold=tau, coeff_list=sched) == expect


def test_restart_threshold_safety_lengthens_segments():
    """tau = 116 lies between the two-iteration growths (3.4445/1.05)^4 = 115.8 and
    3.4445^4 = 140.8: segments of 2 at s = 1, of 3 at s = 1.05."""
    assert (3.4445 / 1.05) ** 4 < 116 < 3.4445 ** 4
    assert O.restart_points(6, restart_threshold=116, coeff_list=O.coefficient_schedule(QUINTIC, 6, 1.0)) == [2, 4]
    assert O.restart_points(6, restart_threshold=116, coeff_list=O.coefficient_schedule(QUINTIC, 6, 1.05)) == [3]


def test_restart_threshold_schedule_by_hand():
    """Per-iteration slopes a = 2, 2, 4, 1.5, 3 give growths 4, 4, 16, 2.25, 9; with
    tau = 15 the products since the last restart are 4, 16 (restart), 16 (restart),
    2.25, then the last iteration, which never restarts."""
    sched = [(2.0, 0.0, 0.0), (2.0, 0.0, 0.0), (4.0, 0.0, 0.0), (1.5, 0.0, 0.0), (3.0, 0.0, 0.0)]
    assert O.restart_points(5, restart_threshold=15.0, coeff_list=sched) == [2, 3]
    # a mask still wins over the threshold; a threshold wins over restart_every
    assert O.restart_points(5, restart_mask=0b1, restart_threshold=15.0, coeff_list=sched) == [1]
    assert O.restart_points(5, restart_every=1, restart_threshold=15.0, coeff_list=sched) == [2, 3]
    with pytest.raises(ValueError):
        O.restart_points(5, restart_threshold=15.0)


def test_restart_threshold_growth_factor_is_a_squared():
    """The premise of R12, checked on the oracle's own polynomial step: an error of
    size eps in a null direction of G comes out of one Gram update P G P multiplied
    by a^2 (to first order), with P = a I + b G + c G^2."""
    a, b, c = QUINTIC
    lam = np.array([0.0, 0.3, 0.9, 1.2])
    G = np.diag(lam)
    eps = 1e-9
    dG = np.zeros_like(G)
    dG[0, 0] = eps

    def step(H):
        P = O.gram_polynomial(H, a, b, c)
        return P @ H @ P

    grown = (step(G + dG) - step(G))[0, 0]
    assert abs(grown / eps - a * a) < 1e-6 * a * a


def test_restart_threshold_keeps_exact_output():
    """Restarts change only rounding: with threshold-chosen restarts the fp64 output
    still equals the SVD closed form."""
    M = RNG.standard_normal((24, 40))
    ref = svd_closed_form(M, QUINTIC, 6)
    for tau in (5.0, 100.0, 1e3):
        out, _ = O.orthogonalize(M, n_iter=6, restart_threshold=tau)
        assert np.abs(out - ref).max() < 1e-12


# ------------------------------------- the single steps of one iteration
@pytest.mark.parametrize("shape", [(7, 33), (33, 7), (40, 40), (1, 9), (9, 1)])
def test_gram_spectrum_is_squared_singular_values(shape):
    """gram(S) is symmetric PSD on the smaller side, with eigenvalues sigma_i^2
    (LAPACK SVD of S) and eigenvectors the left (wide) / right (tall) singular vectors."""
    S = RNG.standard_normal(shape)
    G = O.gram(S)
    m = min(shape)
    assert G.shape == (m, m)
    U, s, Vt = np.linalg.svd(S, full_matrices=False)
    W = U if shape[0] <= shape[1] else Vt.T
    assert np.allclose(G, (W * s ** 2) @ W.T, atol=1e-12 * max(1.0, s[0] ** 2))
    assert np.allclose(np.sort(np.linalg.eigvalsh(G)), np.sort(s ** 2), atol=1e-12 * s[0] ** 2)


def test_gram_polynomial_spectral_form():
    """For G = V diag(lam) V^T (V orthogonal from a seeded QR), a I + b G + c G^2
    = V diag(a + b lam + c lam^2) V^T."""
    m = 24
    V, _ = np.linalg.qr(RNG.standard_normal((m, m)))
    lam = RNG.uniform(-1.0, 1.0, m)
    G = (V * lam) @ V.T
    a, b, c = QUINTIC
    P = O.gram_polynomial(G, a, b, c)
    assert np.allclose(P, (V * (a + b * lam + c * lam ** 2)) @ V.T, atol=1e-12)
    # the identity term sits on the diagonal only
    assert np.allclose(O.gram_polynomial(np.zeros((3, 3)), 2.0, 5.0, 7.0), 2.0 * np.eye(3))


@pytest.mark.parametrize("shape", [(12, 30), (30, 12)])
def test_one_step_composition_is_one_ns_iteration(shape):
    """apply_factor(gram_polynomial(gram(X)), X) on a normalized X is one
    Newton-Schulz iteration: the SVD closed form with K = 1."""
    S = RNG.standard_normal(shape)
    X = S / np.linalg.norm(S)
    a, b, c = QUINTIC
    Y = O.apply_factor(O.gram_polynomial(O.gram(X), a, b, c), X)
    assert np.allclose(Y, svd_closed_form(S, QUINTIC, 1), atol=1e-13)
    assert np.array_equal(O.apply_factor(np.eye(min(shape)), X), X)


# ------------------------------------------------------ weight update (R11)
def f32_bits_to_bf16_rne(x: float) -> float:
    """Scalar round-to-nearest-even of an fp32 value to bfloat16, by its bits."""
    u = struct.unpack("<I", struct.pack("<f", x))[0]
    lower = u & 0xFFFF
    up = u >> 16
    if lower > 0x8000 or (lower == 0x8000 and (up & 1)):
        up += 1
    return struct.unpack("<f", struct.pack("<I", (up & 0xFFFF) << 16))[0]


def test_bf16_rounding_ties_to_even():
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, -(1.0 + 2.0 ** -8),
                     3.0, 0.0], dtype=np.float32)
    got = O.round_to_bf16(vals)
    assert got.tolist() == [1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -1.0, 3.0, 0.0]
    x = RNG.standard_normal(2000).astype(np.float32) * 10.0 ** RNG.uniform(-5, 3, 2000).astype(np.float32)
    assert np.array_equal(O.round_to_bf16(x), np.array([f32_bits_to_bf16_rne(float(v)) for v in x], np.float32))


@pytest.mark.parametrize("wd,bf16", [(0.0, False), (0.01, False), (0.01, True)])
def test_weight_update_scalar_emulation(wd, bf16):
    """fl32(fl32(W keep) - fl32(alpha U)) reproduced with struct-rounded fp64 scalars."""
    W = (RNG.standard_normal(500) * 0.02).astype(np.float32)
    U = (RNG.standard_normal(500) * 0.05).astype(np.float32)
    alpha = 0.02 * 1.7
    got = O.weight_update_f32(W, U, alpha, wd, bf16)
    keep = f32(1.0 - f32(wd))
    a32 = f32(alpha)
    for i in range(500):
        v = f32(f32(float(W[i]) * keep) - f32(a32 * float(U[i])))
        if bf16:
            v = f32_bits_to_bf16_rne(v)
        assert got[i] == v


def _svd_orth_rows(Mt, idx, **ns):
    """The selected block's exact output from the SVD closed form."""
    return svd_closed_form(np.asarray(Mt, np.float64)[idx], ns.get("coeffs", QUINTIC), ns["n_iter"],
                           ns.get("safety", 1.0))


def _scalar_update(W, U, alpha, wd, bf16=False):
    """fl32(fl32(W keep) - fl32(alpha U)) with struct-rounded fp64 scalars."""
    keep = f32(1.0 - f32(wd))
    a32 = f32(alpha)
    out = np.array([[f32(f32(float(w) * keep) - f32(a32 * float(u))) for w, u in zip(rw, ru)]
                    for rw, ru in zip(np.asarray(W), np.asarray(U))], np.float32)
    return O.round_to_bf16(out) if bf16 else out


def _brute_idx(M, frac):
    keys = [exact_key(r) for r in np.asarray(M)]
    k = O.selected_count(len(keys), frac)
    return sorted(sorted(range(len(keys)), key=lambda j: (-keys[j], j))[:k])


@pytest.mark.parametrize("ef", ["raw", "carry"])
def test_rowsubset_step_update_alpha_zero_keeps_decayed_weights(ef):
    """alpha = 0: every row becomes W (1 - wd); the selected rows exactly (fp64),
    the others as the fp32 update fl32(W keep) (scalar emulation)."""
    rng = np.random.default_rng(21)
    E = [rng.standard_normal((16, 24)).astype(np.float32)]
    G = [round_bf16(rng.standard_normal((16, 24)).astype(np.float32))]
    W = [(rng.standard_normal((16, 24)) * 0.02).astype(np.float32)]
    _, newW, idxs = O.rowsubset_step_update(E, G, W, 0.9, [0.0], 0.01, ef=ef, row_frac=0.25, n_iter=5)
    keep = f32(1.0 - f32(0.01))
    idx, rest = idxs[0], np.setdiff1d(np.arange(16), idxs[0])
    exact = np.array([[float(Fraction(float(w)) * Fraction(keep)) for w in row] for row in W[0][idx]])
    assert np.array_equal(newW[0][idx], exact)
    assert np.array_equal(newW[0][rest], _scalar_update(W[0][rest], np.zeros((len(rest), 24)), 0.0, 0.01))


@pytest.mark.parametrize("ef,shape,frac", [("raw", (24, 10), 0.25), ("raw", (12, 30), 0.5),
                                           ("carry", (24, 10), 0.25), ("carry", (12, 30), 1 / 3)])
def test_rowsubset_step_update_from_zero_weights(ef, shape, frac):
    """W = 0, no decay: the selected rows are -alpha times the SVD closed form of the
    selected block of the buffer the step orthogonalizes, the rows chosen by brute
    force on exact keys; the others are -fl32(alpha M_t) (raw) or zero (carry).
    The buffer the step orthogonalizes is fl32(fl32(beta E) + G) (raw) or
    fl32(E + G) (carry), each rebuilt by scalar emulation."""
    rng = np.random.default_rng(hash((ef, shape)) % 2 ** 32)
    E = rng.standard_normal(shape).astype(np.float32)
    G = round_bf16(rng.standard_normal(shape).astype(np.float32))
    W0 = np.zeros(shape, np.float32)
    beta, alpha = 0.9, 0.05
    ns = dict(n_iter=5, restart_every=2)
    _, newW, idxs = O.rowsubset_step_update([E], [G], [W0], beta, [alpha], 0.0, ef=ef, row_frac=frac, **ns)
    if ef == "raw":
        B = np.array([[f32(f32(f32(beta) * float(e)) + float(g)) for e, g in zip(re_, rg)] for re_, rg in zip(E, G)],
                     np.float32)
    else:
        B = np.array([[f32(float(e) + float(g)) for e, g in zip(re_, rg)] for re_, rg in zip(E, G)], np.float32)
    idx = _brute_idx(B, frac)
    assert list(idxs[0]) == idx
    rest = np.setdiff1d(np.arange(shape[0]), idx)
    want = -f32(alpha) * _svd_orth_rows(B, idx, **ns)
    assert O.rel_frobenius(newW[0][idx], want) < 1e-11
    if ef == "raw":
        assert np.array_equal(newW[0][rest], _scalar_update(W0[rest], B[rest], alpha, 0.0))
        assert np.all(newW[0][rest] == -np.array([[f32(f32(alpha) * float(b)) for b in r] for r in B[rest]]))
    else:
        assert np.all(newW[0][rest] == 0.0)


def test_rowsubset_step_update_carry_routes_zero_update():
    """Carry with weights and decay: unselected rows take the zero update,
    fl32(W keep) bit for bit; selected rows W keep - alpha O (closed form)."""
    rng = np.random.default_rng(33)
    E = rng.standard_normal((20, 9)).astype(np.float32)
    G = round_bf16(rng.standard_normal((20, 9)).astype(np.float32))
    W = (rng.standard_normal((20, 9)) * 0.05).astype(np.float32)
    ns = dict(n_iter=4, restart_every=2)
    _, newW, idxs = O.rowsubset_step_update([E], [G], [W], 0.95, [0.02], 0.1, ef="carry", row_frac=0.3, **ns)
    B = np.array([[f32(float(e) + float(g)) for e, g in zip(re_, rg)] for re_, rg in zip(E, G)], np.float32)
    idx = _brute_idx(B, 0.3)
    assert list(idxs[0]) == idx
    rest = np.setdiff1d(np.arange(20), idx)
    keep = f32(1.0 - f32(0.1))
    assert np.array_equal(newW[0][rest], np.array([[f32(float(w) * keep) for w in r] for r in W[rest]], np.float32))
    want = W[idx].astype(np.float64) * keep - f32(0.02) * _svd_orth_rows(B, idx, **ns)
    assert O.rel_frobenius(newW[0][idx], want) < 1e-11


def _carry_inputs(shape=(48, 20), steps=3, seed=5):
    rng = np.random.default_rng(seed)
    return [round_bf16(rng.standard_normal(shape).astype(np.float32)) for _ in range(steps)]


def test_carry_equals_raw_at_full_rows():
    """rho = 1: both readings run the same momentum sequence.  Carry's buffer is
    fl32(beta M_t) where raw keeps M_t, and the next step forms fl32(fl32(beta M_t) + G)
    either way, so the outputs agree bit for bit over several steps."""
    Gs = _carry_inputs()
    Er = [np.zeros(Gs[0].shape, np.float32)]
    Ec = [np.zeros(Gs[0].shape, np.float32)]
    for G in Gs:
        Er, outr, _ = O.rowsubset_step(Er, [G], 0.95, row_frac=1.0, n_iter=5)
        Ec, outc, _ = O.rowsubset_step(Ec, [G], 0.95, ef="carry", row_frac=1.0, n_iter=5)
        assert np.array_equal(outr[0], outc[0])
        assert np.array_equal(Ec[0], np.multiply(np.float32(0.95), Er[0], dtype=np.float32))


def test_carry_with_beta_one_differs_only_in_unselected_output_rows():
    """beta = 1: fl32(1 E) = E, so both buffers are fl32(E + G) and the selected
    output rows agree; the unselected rows are the momentum (raw) or zero (carry)."""
    Gs = _carry_inputs()
    Er = [np.zeros(Gs[0].shape, np.float32)]
    Ec = [np.zeros(Gs[0].shape, np.float32)]
    for G in Gs:
        Er, outr, idr = O.rowsubset_step(Er, [G], 1.0, row_frac=0.25, n_iter=5)
        Ec, outc, idc = O.rowsubset_step(Ec, [G], 1.0, ef="carry", row_frac=0.25, n_iter=5)
        assert np.array_equal(Er[0], Ec[0]) and np.array_equal(idr[0], idc[0])
        rest = np.setdiff1d(np.arange(G.shape[0]), idr[0])
        assert np.array_equal(outr[0][idr[0]], outc[0][idc[0]])
        assert np.all(outc[0][rest] == 0.0) and np.array_equal(outr[0][rest], Er[0][rest].astype(np.float64))


def test_carry_keeps_unselected_rows_undecayed():
    """Carry: unselected buffer rows are B = fl32(E + G) exactly (scalar IEEE
    emulation), selected rows fl32(beta B); the update's unselected rows are zero."""
    rng = np.random.default_rng(6)
    E = rng.standard_normal((30, 12)).astype(np.float32)
    G = round_bf16(rng.standard_normal((30, 12)).astype(np.float32))
    (Et,), (out,), (idx,) = O.rowsubset_step([E], [G], 0.9, ef="carry", row_frac=0.2, n_iter=3)
    def f32(x):
        return struct.unpack("f", struct.pack("f", x))[0]
    B = np.array([[f32(float(a) + float(b)) for a, b in zip(r1, r2)] for r1, r2 in zip(E, G)], np.float32)
    rest = np.setdiff1d(np.arange(30), idx)
    assert np.array_equal(Et[rest].view(np.uint32), B[rest].view(np.uint32))
    decayed = np.array([[f32(f32(0.9) * float(v)) for v in row] for row in B[idx]], np.float32)
    assert np.array_equal(Et[idx].view(np.uint32), decayed.view(np.uint32))
    assert np.all(out[rest] == 0.0)
    assert np.array_equal(idx, O.select_rows(B, 0.2))
    with pytest.raises(ValueError):
        O.rowsubset_step([E], [G], 0.9, ef="dion")
