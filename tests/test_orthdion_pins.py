"""Pins of the low-rank (Dion / Orth-Dion) oracle against facts that do not come
from the oracle: an independent Gram-Schmidt, the SVD of the input, singular
values of the update, error-feedback identities and scalar IEEE emulation."""
import struct

import numpy as np
import pytest

from oracle import orthdion_oracle as L

RNG = np.random.default_rng(4321)


def gram_schmidt(A):
    """Modified Gram-Schmidt in fp64 (positive diagonal by construction)."""
    A = np.array(A, dtype=np.float64)
    n, r = A.shape
    Q = np.zeros_like(A)
    for j in range(r):
        v = A[:, j].copy()
        for i in range(j):
            v -= (Q[:, i] @ v) * Q[:, i]
        Q[:, j] = v / np.linalg.norm(v)
    return Q


@pytest.mark.parametrize("shape", [(9, 4), (40, 7), (7, 7), (300, 16)])
def test_qr_positive_matches_gram_schmidt(shape):
    A = RNG.standard_normal(shape)
    Q = L.qr_positive(A)
    assert np.abs(Q - gram_schmidt(A)).max() < 1e-10
    R = Q.T @ A
    assert np.abs(np.tril(R, -1)).max() < 1e-10 and np.all(np.diag(R) > 0)
    assert np.abs(Q.T @ Q - np.eye(shape[1])).max() < 1e-12


def test_column_normalize():
    W = RNG.standard_normal((12, 5))
    W[:, 2] = 0.0
    N = L.column_normalize(W)
    norms = np.linalg.norm(N, axis=0)
    assert np.allclose(norms[[0, 1, 3, 4]], 1.0, atol=1e-14) and norms[2] == 0.0
    for j in (0, 1, 3, 4):   # same direction
        assert abs(N[:, j] @ W[:, j] - np.linalg.norm(W[:, j])) < 1e-12


def test_accumulate_scalar_emulation():
    """fl32(M + G) against struct-rounded fp64 sums, including a tie case."""
    def f32(x):
        return struct.unpack("f", struct.pack("f", x))[0]
    M = RNG.standard_normal(200).astype(np.float32)
    G = RNG.standard_normal(200).astype(np.float32)
    M[0], G[0] = np.float32(1.0), np.float32(2.0 ** -24)   # exact tie: rounds to even (1.0)
    got = L.accumulate(M, G)
    want = np.array([f32(float(a) + float(b)) for a, b in zip(M, G)], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert got[0] == np.float32(1.0)


@pytest.mark.parametrize("shape,r", [((60, 40), 5), ((40, 60), 8), ((50, 50), 50), ((128, 96), 16)])
@pytest.mark.parametrize("mode", ["qr", "colnorm"])
def test_exact_recovery_of_polar_factor(shape, r, mode):
    """With Q = the top-r right singular vectors of B, one step returns the rank-r
    polar factor U_r V_r^T of B (both normalizations), P = U_r and Q' = V_r."""
    M = RNG.standard_normal(shape).astype(np.float32)
    G = np.zeros(shape, np.float32)
    B = L.accumulate(M, G).astype(np.float64)
    U, s, Vt = np.linalg.svd(B, full_matrices=False)
    Q = Vt[:r].T
    _, Qn, P, D = L.lowrank_step(M, G, Q, beta=1.0, mode=mode)
    assert np.abs(D - U[:, :r] @ Vt[:r]).max() < 1e-9
    assert np.abs(P - U[:, :r]).max() < 1e-9
    assert np.abs(Qn - Vt[:r].T).max() < 1e-9


@pytest.mark.parametrize("shape,r", [((70, 30), 6), ((30, 70), 6), ((64, 64), 20)])
def test_orthdion_update_is_partial_isometry(shape, r):
    """Orth-Dion: P and Q' have orthonormal columns, so D has exactly r singular
    values equal to one (the Ky Fan dual factor is one)."""
    M = RNG.standard_normal(shape).astype(np.float32)
    G = RNG.standard_normal(shape).astype(np.float32)
    Q = RNG.standard_normal((shape[1], r))
    _, Qn, P, D = L.lowrank_step(M, G, Q, beta=0.5, mode="qr")
    sv = np.linalg.svd(D, compute_uv=False)
    assert np.abs(sv[:r] - 1.0).max() < 1e-10 and np.abs(sv[r:]).max() < 1e-10
    assert np.abs(Qn.T @ Qn - np.eye(r)).max() < 1e-12
    # Q' spans the columns of W = B^T P
    B = L.accumulate(M, G).astype(np.float64)
    W = B.T @ P
    assert np.abs(Qn @ (Qn.T @ W) - W).max() < 1e-9 * np.abs(W).max()


def test_dion_colnorm_update_norm_bounds():
    """Dion: unit columns of Q'; the update's spectral norm lies in [1, sqrt(r)]."""
    r = 12
    M = (RNG.standard_normal((80, 50)) @ np.diag(np.linspace(3, 0.1, 50))).astype(np.float32)
    G = np.zeros_like(M)
    Q = RNG.standard_normal((50, r))
    _, Qn, P, D = L.lowrank_step(M, G, Q, beta=1.0, mode="colnorm")
    assert np.allclose(np.linalg.norm(Qn, axis=0), 1.0, atol=1e-12)
    s1 = np.linalg.norm(D, 2)
    assert 1.0 - 1e-12 <= s1 <= np.sqrt(r) + 1e-12


def test_error_feedback_identities():
    """beta = 1: the buffer keeps only what P does not capture (P^T M' = 0);
    beta = 0: the buffer is B unchanged; linear in beta in between."""
    M = RNG.standard_normal((45, 33)).astype(np.float32)
    G = RNG.standard_normal((45, 33)).astype(np.float32)
    Q = RNG.standard_normal((33, 7))
    B = L.accumulate(M, G).astype(np.float64)
    M1, _, P, _ = L.lowrank_step(M, G, Q, beta=1.0)
    assert np.abs(P.T @ M1).max() < 1e-12 * np.abs(B).max() * 45
    M0, _, _, _ = L.lowrank_step(M, G, Q, beta=0.0)
    assert np.array_equal(M0, B)
    Mh, _, _, _ = L.lowrank_step(M, G, Q, beta=0.25)
    assert np.abs(Mh - (0.75 * B + 0.25 * M1)).max() < 1e-12 * np.abs(B).max()


def test_rank_clamped_and_modes_checked():
    M = RNG.standard_normal((5, 9)).astype(np.float32)
    G = np.zeros_like(M)
    Q = RNG.standard_normal((9, 8))
    _, Qn, P, D = L.lowrank_step(M, G, Q, beta=1.0)
    assert P.shape == (5, 5) and Qn.shape == (9, 5)
    with pytest.raises(ValueError):
        L.lowrank_step(M, G, Q, beta=1.0, mode="svd")


@pytest.mark.parametrize("cond", [1e1, 1e3, 1e5])
def test_qr_factor_sensitivity_to_fp32_accurate_data(cond):
    """The orthogonal QR factor of F moves by up to about cond(F) * u under a relative
    perturbation u of F (QR perturbation theory), so data that is only fp32-accurate
    (u = 2^-24) determines P = orth(B Q) to about cond(B Q) * 2^-24: at cond 1e5 that
    exceeds 1e-4 even with every later step exact.  This is why the randomized low-rank
    sweep gates the factor and the update at max(1e-4, cond * 2^-24)."""
    rng = np.random.default_rng(int(np.log10(cond)))
    R, C = 300, 12
    U, _ = np.linalg.qr(rng.standard_normal((R, C)))
    V, _ = np.linalg.qr(rng.standard_normal((C, C)))
    F = (U * np.logspace(0, -np.log10(cond), C)) @ V.T
    assert np.isclose(np.linalg.cond(F), cond, rtol=1e-6)
    P = L.qr_positive(F)
    u = 2.0 ** -24
    worst = 0.0
    for t in range(20):
        E = rng.standard_normal(F.shape)
        E *= u * np.linalg.norm(F) / np.linalg.norm(E)
        d = np.linalg.norm(L.qr_positive(F + E) - P) / np.linalg.norm(P)
        worst = max(worst, d)
    assert worst <= 4 * cond * u            # bounded by the condition number ...
    assert worst >= 0.01 * cond * u         # ... and that bound is attained in order of magnitude
    if cond >= 1e5:
        assert worst > 1e-4
