"""Oracle for the low-rank Dion / Orth-Dion update: plain, slow, fp64, CPU only.

TEST INFRASTRUCTURE ONLY.  Only the test suite and the benchmark's CPU-baseline
leg may import or run this module.  The product path never imports it, and it
imports nothing from the product path.

Pages: the English explainer of Orth-Dion (technical summary: Problem
Statement, Methodology "The Geometric Insight" and "Orth-Dion", Theoretical
Contributions "Error Feedback Analysis", Key Results "Error Feedback Tuning").

* Dion approximates the orthogonalized momentum with rank-r factors from one
  step of power iteration, keeps a residual (error-feedback) buffer, and
  normalizes the right factor's columns (Problem Statement; Geometric Insight).
* Orth-Dion keeps all of that and replaces the column normalization of the
  right factor by QR orthogonalization, so the update is a partial isometry
  (Methodology, "Orth-Dion").
* The error-feedback coefficient beta below 1 leaves part of the captured
  component in the buffer (Error Feedback Analysis; Error Feedback Tuning).

The pages print no formula for the step.  The readings taken here are:

  D1  The buffer accumulates the gradient: B = fl32(M + G) (one fp32 rounding;
      M is the persistent fp32 buffer, G the gradient as stored).
  D2  One power-iteration step from the previous right factor Q (C x r):
      P = orth(B Q), where orth is the reduced QR factor normalized so that
      the triangular factor has a positive diagonal.
  D3  The right factor is W = B^T P (C x r).
  D4  Error feedback: the buffer keeps B - beta P W^T (beta = 1 removes the
      captured rank-r part; smaller beta leaves a share of it in the buffer).
  D5  Normalization of the right factor: Q' = orth(W) (Orth-Dion) or each
      column of W divided by its L2 norm (Dion, "colnorm"; a zero column
      stays zero).  Q' is returned as the next step's right factor.
  D6  The update is D = P Q'^T (R x C), unscaled: learning rate and shape
      factors belong to the weight update.
  D7  The matrix is used as stored (rows = dim 0); the rank is
      r = min(rank, R, C).  Inputs of rank below r (B Q or W rank-deficient)
      are outside the method's contract: the factorization is not unique.

Readings without a formula on the pages: D1 and D4 (the buffer's
accumulation and the error-feedback form) and D5's QR sign convention.  The
pages print no value to check them against; the functions are pinned against
the mathematics below.

Parity pins (in tests/test_orthdion_pins.py): orthonormal factors and the
positive-diagonal QR convention against LAPACK, exact recovery of the rank-r
polar factor U V^T when Q spans the top right singular vectors, the update's
singular values (all one for Orth-Dion, spectral norm in [1, sqrt(r)] for
Dion), the error-feedback identities for beta = 1 and beta = 0, and the fp32
accumulation by scalar emulation.
"""
from __future__ import annotations

import numpy as np


def qr_positive(A) -> np.ndarray:
    """Reduced QR factor of A (n x r, n >= r) with the triangular factor's
    diagonal made positive (D2).  LAPACK's QR is the library step."""
    A = np.asarray(A, dtype=np.float64)
    Q, R = np.linalg.qr(A, mode="reduced")
    s = np.sign(np.diag(R))
    s[s == 0] = 1.0
    return Q * s


def column_normalize(W) -> np.ndarray:
    """Each column divided by its L2 norm; zero columns stay zero (D5, Dion)."""
    W = np.asarray(W, dtype=np.float64)
    n = np.sqrt(np.sum(W * W, axis=0))
    out = np.zeros_like(W)
    nz = n > 0
    out[:, nz] = W[:, nz] / n[nz]
    return out


def accumulate(M, G) -> np.ndarray:
    """B = fl32(M + G): one correctly rounded fp32 addition per element (D1)."""
    return (np.asarray(M, dtype=np.float32) + np.asarray(G, dtype=np.float32)).astype(np.float32)


def lowrank_step(M, G, Q, beta: float, mode: str = "qr"):
    """One Dion / Orth-Dion step on one matrix (D1-D6).

    M  R x C fp32 buffer (not modified), G  R x C gradient, Q  C x r' previous
    right factor (r' >= the rank used).  Returns (M_new fp64, Q_new C x r,
    P R x r, D R x C) with r = Q's column count, clamped to min(R, C).
    """
    if mode not in ("qr", "colnorm"):
        raise ValueError("mode must be 'qr' or 'colnorm'")
    B = accumulate(M, G).astype(np.float64)
    R_, C_ = B.shape
    Q = np.asarray(Q, dtype=np.float64)
    r = min(Q.shape[1], R_, C_)
    Q = Q[:, :r]
    P = qr_positive(B @ Q)                       # D2
    W = B.T @ P                                  # D3
    M_new = B - beta * (P @ W.T)                 # D4
    Q_new = qr_positive(W) if mode == "qr" else column_normalize(W)   # D5
    D = P @ Q_new.T                              # D6
    return M_new, Q_new, P, D
