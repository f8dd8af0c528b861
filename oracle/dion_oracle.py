"""Oracle for the Dion3 orthogonalization hot path: plain, slow, fp64, CPU only.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import or run this module.  The product
path (the HIP library and its Python binding) never imports it, and this module
imports nothing from the product path.

What it computes, and where the pages state it
----------------------------------------------
Pages: "Dion3: Full-Stack Orthogonal Updates" (arXiv abstract mirror), section
Abstract; and the Chinese summary "Dion3：全栈正交更新", sections 方法 / 核心模块
(method, core modules), 输入输出流程 (input/output flow), 核心洞察 (insights) and
局限 (limitations).

* The update rule picks a fraction of the momentum matrix's rows and
  orthogonalizes only those; the other rows keep the raw momentum update
  (Abstract; 核心模块, "Dion3 更新规则" bullet).
* Orthogonalization is Newton-Schulz run on the Gram matrix of the momentum,
  with restarts and a safety factor (Abstract; 核心模块, "Gram Newton-Schulz"
  bullet; 局限, first bullet).
* The flow is: update momentum, select rows, Gram Newton-Schulz, update weights
  (输入输出流程).  The weight update is outside this path.

The pages print no coefficients, normalization, restart schedule, safety
formula, selection criterion or worked example.  The readings taken here are:

  R1  Coefficients: the fixed quintic (3.4445, -4.7750, 2.0315) unless a
      per-iteration list is given.
  R2  Normalization: X0 = S / ||S||_F (Frobenius norm of the selected rows,
      no epsilon); a zero matrix gives zero output rows.
  R3  The Gram matrix is formed on the smaller side (m = min(k, C)); when the
      selected block is tall it is transposed, processed, and transposed back.
  R4  Safety factor s scales the polynomial's argument at every iteration:
      f_s(x) = f(x / s), i.e. (a, b, c) -> (a/s, b/s^3, c/s^5).
  R5  A restart after iteration k (never after the last) re-forms the Gram
      matrix from the current iterate X_k = Q X and resets Q to I.
  R6  Rows are ranked by squared L2 norm: the exact sum of the squares of the
      stored values rounded once to the nearest double (ties to even), so the
      ranking does not depend on a summation order; larger first, ties (equal
      doubles) to the lower row index; k = ceil(row_frac * R),
      clamped to [1, R]; selected rows are processed in ascending order.
  R7  No output scaling (learning rate and shape factors belong to the
      weight update).
  R8  Error feedback / momentum: E is the persistent fp32 momentum buffer;
      M_t = fl32(fl32(beta * E_{t-1}) + G_t) (two correctly rounded fp32
      operations, heavy-ball form) and E_t = M_t; unselected rows of the
      output carry M_t unchanged.
  R11 Weight update (the step's last stage, 输入输出流程): W <- W (1 - wd) -
      alpha U with U the step's output and alpha the learning rate times a
      per-matrix shape scale chosen by the caller; in fp32 arithmetic with one
      rounding per operation, then round-to-nearest-even for bf16 weights.
  R14 Error feedback, "carry" alternative (ef="carry"): Dion's recurrence
      with only the selected rows captured.  The buffer takes the gradient,
      B = fl32(E + G); the update is the orthogonalized selected rows and
      zero elsewhere; the buffer keeps fl32(beta * B) on the selected rows and
      B unchanged on the others (carried undecayed).  The default remains R8.
  R12 Restart threshold tau (局限 names it as a hyperparameter; the same
      passage ties restarts to spurious negative eigenvalues of the
      intermediate matrices): in the smallest singular directions P is close
      to a_k I, so one iteration scales an error of the Gram matrix there by
      a_k^2.  A restart is taken after the iteration at which the product of
      these factors since the last restart first reaches tau.

Readings without a formula on the pages: R4 (where the safety factor acts),
R8 and R14 (the error-feedback form), R11 (the weight update and its shape
scale) and R12 (what the restart threshold measures).  The pages print no
value to check them against; the functions implementing them are pinned
against the mathematics below (closed forms, identities, scalar emulation).

Parity pins (in tests/): SVD closed form U f^K(Sigma) V^T, textbook polar
factor via the cubic Newton-Schulz map, the NS band invariant, equivalence with
plain (non-Gram) Newton-Schulz, invariances, exact rank-1 / orthonormal-row
values, brute-force selection with ties, and bit-exact fp32 momentum.  Every
function below is pinned by at least one of them.
"""
from __future__ import annotations

import math

import numpy as np

# R1: the fixed quintic used by every workload unless a schedule is supplied.
DEFAULT_COEFFS = (3.4445, -4.7750, 2.0315)


# --------------------------------------------------------------------------
# Hyperparameter expansion (readings R1, R4, R5)
# --------------------------------------------------------------------------
def coefficient_schedule(coeffs, n_iter: int, safety: float = 1.0):
    """Per-iteration (a, b, c) with the safety factor folded in (R1, R4).

    ``coeffs`` is either one triple (used at every iteration) or a list of
    ``n_iter`` triples.  The safety factor rescales the polynomial's argument:
    f_s(x) = a (x/s) + b (x/s)^3 + c (x/s)^5.
    Pages: Dion3 summary, 核心模块 (safety factors named, no formula); 局限.
    """
    arr = np.asarray(coeffs, dtype=np.float64)
    if arr.ndim == 1:
        if arr.shape[0] != 3:
            raise ValueError("a single coefficient set must have 3 entries")
        arr = np.tile(arr, (n_iter, 1))
    if arr.shape != (n_iter, 3):
        raise ValueError(f"need 1 or {n_iter} coefficient triples, got {arr.shape}")
    s = float(safety)
    if not s > 0:
        raise ValueError("safety must be > 0")
    return [(float(a) / s, float(b) / s ** 3, float(c) / s ** 5) for a, b, c in arr]


def restart_points(n_iter: int, restart_every: int = 0, restart_mask: int = 0,
                   restart_threshold: float = 0.0, coeff_list=None):
    """Iterations k (1-based) after which the Gram matrix is re-formed (R5, R12).

    A nonzero ``restart_mask`` wins: bit (k-1) set means restart after k.
    Otherwise a positive ``restart_threshold`` tau applies R12: the growth
    factor a_k^2 of every iteration since the last restart (``coeff_list``
    holds the safety-folded triples) is multiplied up, and the iteration at
    which the product first reaches tau restarts.  Otherwise every
    ``restart_every``-th iteration restarts.  No restart is ever taken after
    the last iteration.
    Pages: Dion3 summary, 核心模块 (restart strategy) and 局限 (restart
    threshold; spurious negative eigenvalues of the intermediate matrices).
    """
    if restart_mask:
        pts = {k for k in range(1, n_iter + 1) if (restart_mask >> (k - 1)) & 1}
    elif restart_threshold and restart_threshold > 0:
        if coeff_list is None or len(coeff_list) != n_iter:
            raise ValueError("the restart threshold needs the per-iteration coefficients")
        pts, growth = set(), 1.0
        for k in range(1, n_iter + 1):
            a = coeff_list[k - 1][0]
            growth *= a * a
            if growth >= restart_threshold:
                pts.add(k)
                growth = 1.0
    elif restart_every and restart_every > 0:
        pts = set(range(restart_every, n_iter + 1, restart_every))
    else:
        pts = set()
    return sorted(k for k in pts if k < n_iter)


# --------------------------------------------------------------------------
# Row selection (reading R6)
# --------------------------------------------------------------------------
def row_keys(M) -> np.ndarray:
    """Squared L2 norm of every row (R6): the exact sum of the squares of the
    stored values, rounded once to the nearest double (ties to even).

    A correctly rounded sum does not depend on the order of summation, so the
    selection it decides is the same for every implementation that rounds the
    exact sum once.  For float32 values (the stored bf16, fp16 and fp32
    inputs) it is computed with integer arithmetic in the oracle's C part
    (exact_keys.c); other doubles go through ``row_keys_fsum``, the same
    definition through Python's correctly rounded ``math.fsum``.  The two are
    pinned equal.
    """
    A = np.asarray(M)
    with np.errstate(over="ignore", invalid="ignore"):
        A32 = np.ascontiguousarray(A, dtype=np.float32)
    if A.dtype == np.float32 or np.array_equal(A32.astype(A.dtype), A):
        from . import native
        return native.row_sumsq_f32(A32)
    return row_keys_fsum(A)


def row_keys_fsum(M) -> np.ndarray:
    """``row_keys`` from its definition: math.fsum (correctly rounded) of the
    exact squares.  Each value x is split as x = h + l with h and l of at most
    26 significant bits (Veltkamp's split), so that x^2 = h^2 + 2hl + l^2 with
    every term exact in fp64.  Slow; for pins and fp64 data."""
    A = np.asarray(M, dtype=np.float64)
    c = A * 134217729.0            # 2^27 + 1
    h = c - (c - A)
    lo = A - h
    terms = np.stack([h * h, 2.0 * h * lo, lo * lo], axis=-1).reshape(A.shape[0], -1)
    return np.array([math.fsum(row) for row in terms.tolist()], dtype=np.float64)


def selected_count(n_rows: int, row_frac: float) -> int:
    """k = ceil(row_frac * R) clamped to [1, R] (R6).

    The fraction arrives as a float; x = row_frac * R is shrunk by a relative
    1e-6 before the ceiling so that the float rounding of a decimal fraction
    (0.1f * 1000 = 100.0000015) does not add a row.
    """
    if not (0.0 < row_frac <= 1.0):
        raise ValueError("row_frac must be in (0, 1]")
    x = float(row_frac) * n_rows
    k = int(math.ceil(x * (1.0 - 1e-6)))
    return max(1, min(n_rows, k))


def select_rows(M, row_frac: float) -> np.ndarray:
    """Indices of the selected rows, ascending (R6).

    The top-k rows by squared norm, larger first, ties to the lower index.
    Pages: Dion3 abstract (select a fraction of the momentum rows);
    Dion3 summary, 核心模块, "Dion3 更新规则" bullet (e.g. 1/8 of the rows).
    """
    R = np.asarray(M).shape[0]
    k = selected_count(R, row_frac)
    if k == R:
        return np.arange(R, dtype=np.int64)
    keys = row_keys(M)
    # stable sort on (-key) keeps equal keys in ascending row order
    order = np.argsort(-keys, kind="stable")
    return np.sort(order[:k]).astype(np.int64)


# --------------------------------------------------------------------------
# The single steps of one iteration, on the Gram side (reading R3)
# --------------------------------------------------------------------------
def gram(S) -> np.ndarray:
    """Gram matrix on the Gram side: X X^T with X = S (wide) or S^T (tall, R3).

    Pages: Dion3 summary, 核心模块, "Gram Newton-Schulz" bullet (the iteration
    runs on the Gram matrix) and CuteDSL bullet (symmetric products).
    """
    X = np.asarray(S, dtype=np.float64)
    if X.shape[0] > X.shape[1]:
        X = X.T
    return X @ X.T


def gram_polynomial(G, a: float, b: float, c: float) -> np.ndarray:
    """P = a I + b G + c G^2: the iteration's polynomial in the Gram matrix.

    One Newton-Schulz step X <- a X + b A X + c A^2 X (A = X X^T) is X <- P X
    with this P.  Pages: Dion3 summary, 核心模块, "Gram Newton-Schulz" bullet
    and CuteDSL bullet (the polynomial fused into the product as GEMM + add).
    """
    G = np.asarray(G, dtype=np.float64)
    return a * np.eye(G.shape[0]) + b * G + c * (G @ G)


def apply_factor(Q, S) -> np.ndarray:
    """The factor applied on the Gram side: Q S for a wide block, S Q for a tall one."""
    Q = np.asarray(Q, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    return S @ Q if S.shape[0] > S.shape[1] else Q @ S


# --------------------------------------------------------------------------
# Gram Newton-Schulz (readings R2-R5)
# --------------------------------------------------------------------------
def gram_newton_schulz(X, coeff_list, restarts) -> np.ndarray:
    """Gram Newton-Schulz on a wide, already normalized X (m <= n), fp64.

    Plain Newton-Schulz steps X <- (a I + b A + c A^2) X with A = X X^T.  The
    Gram form never updates X inside a segment: it keeps G (the Gram matrix of
    the current iterate) and Q (the accumulated left factor, current iterate =
    Q X), and uses that A_{k+1} = P A_k P because P is a polynomial in A_k.
    A restart re-forms G from the current iterate and resets Q.
    Pages: Dion3 summary, 核心模块, "Gram Newton-Schulz" bullet; 核心洞察, third
    bullet (restarts and safety factors make the Gram form stable).
    """
    X = np.array(X, dtype=np.float64)
    m = X.shape[0]
    eye = np.eye(m)
    G = X @ X.T
    Q = eye.copy()
    K = len(coeff_list)
    restart_set = set(restarts)
    for k in range(1, K + 1):
        a, b, c = coeff_list[k - 1]
        P = gram_polynomial(G, a, b, c)
        Q = P @ Q
        if k == K:
            break
        if k in restart_set:
            X = Q @ X
            G = X @ X.T
            Q = eye.copy()
        else:
            G = P @ G @ P
    return Q @ X


def orthogonalize(M, coeffs=DEFAULT_COEFFS, n_iter: int = 5, restart_every: int = 0,
                  restart_mask: int = 0, safety: float = 1.0, row_frac: float = 1.0,
                  restart_threshold: float = 0.0):
    """One matrix of the hot path.  Returns (out fp64 R x C, idx int64[k]).

    out[idx] is the orthogonalized selected block; the other rows are the
    input rows unchanged (R6, R8).  Inputs are taken exactly as stored.
    """
    M64 = np.asarray(M, dtype=np.float64)
    if M64.ndim != 2:
        raise ValueError("M must be 2-D")
    R, C = M64.shape
    idx = select_rows(M64, row_frac)
    S = M64[idx, :]
    coeff_list = coefficient_schedule(coeffs, n_iter, safety)
    restarts = restart_points(n_iter, restart_every, restart_mask, restart_threshold, coeff_list)

    tall = S.shape[0] > C                       # R3
    X = S.T if tall else S
    nu = math.sqrt(float(np.sum(X * X)))        # R2
    if nu == 0.0:
        O = np.zeros_like(X)
    else:
        O = gram_newton_schulz(X / nu, coeff_list, restarts)
    if tall:
        O = O.T
    out = M64.copy()
    out[idx, :] = O
    return out, idx


def orthogonalize_batch(Ms, **kw):
    """The megabatch is just the list of independent per-matrix results."""
    return [orthogonalize(M, **kw) for M in Ms]


# --------------------------------------------------------------------------
# Error feedback / momentum (reading R8)
# --------------------------------------------------------------------------
def momentum_update(E, G, beta: float) -> np.ndarray:
    """M_t = fl32(fl32(beta * E) + G): two separately rounded fp32 operations.

    ``E`` is the fp32 buffer, ``G`` the gradient (bf16 values held exactly in
    fp32).  numpy float32 ufuncs are correctly rounded IEEE operations with no
    contraction, so each line is one rounding.
    Pages: Dion3 summary, 输入输出流程 (momentum update comes first) and
    核心模块 ("Dion3 更新规则" bullet: the row rule comes with error feedback
    and handling of finite precision).
    """
    E32 = np.asarray(E, dtype=np.float32)
    G32 = np.asarray(G, dtype=np.float32)
    b = np.float32(beta)
    t = np.multiply(b, E32, dtype=np.float32)
    return np.add(t, G32, dtype=np.float32)


# --------------------------------------------------------------------------
# Weight update (reading R11)
# --------------------------------------------------------------------------
def round_to_bf16(x) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16, ties to even (as float32)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return (u & 0xFFFFFFFF).astype(np.uint32).view(np.float32)


def weight_update_f32(W, U, alpha: float, weight_decay: float = 0.0, bf16: bool = False) -> np.ndarray:
    """W <- fl32(fl32(W * keep) - fl32(alpha * U)), keep = fl32(1 - weight_decay),
    then rounded to bfloat16 when the weight is stored in bf16 (R11).

    Each numpy float32 operation is one IEEE rounding.  The rounding of the
    stored weight decides its bits, so this is computed in the precision the
    weight is stored and updated in (fp32).
    Pages: Dion3 summary, 输入输出流程 (the weight update ends the step).
    """
    W32 = np.asarray(W, dtype=np.float32)
    U32 = np.asarray(U, dtype=np.float32)
    keep = np.subtract(np.float32(1.0), np.float32(weight_decay), dtype=np.float32)
    a = np.multiply(W32, keep, dtype=np.float32)
    b = np.multiply(np.float32(alpha), U32, dtype=np.float32)
    out = np.subtract(a, b, dtype=np.float32)
    return round_to_bf16(out) if bf16 else out


def rowsubset_step_update(Es, grads, Ws, beta: float, alphas, weight_decay: float = 0.0, bf16: bool = False,
                          **kw):
    """One row-subset step followed by the weight update (R8, R11).

    Returns (new E list, new W list (fp64), idx list).  Selected rows take the
    exact update: W * (1 - weight_decay) - alpha * O in fp64; the other rows
    take the raw momentum through ``weight_update_f32`` (their update is an
    exact fp32 value, so their stored result is fixed bit for bit).
    """
    ef = kw.get("ef", "raw")
    newE, outs, idxs = rowsubset_step(Es, grads, beta, **kw)
    newW = []
    for W, Mt, out, idx, alpha in zip(Ws, newE, outs, idxs, alphas):
        W64 = np.asarray(W, dtype=np.float64)
        keep = float(np.subtract(np.float32(1.0), np.float32(weight_decay), dtype=np.float32))
        res = W64 * keep - float(np.float32(alpha)) * out
        rest = np.setdiff1d(np.arange(W64.shape[0]), idx)
        # unselected rows: the raw momentum (R8), or a zero update under "carry" (R14)
        U = Mt[rest] if ef == "raw" else np.zeros_like(Mt[rest])
        res[rest] = weight_update_f32(np.asarray(W)[rest], U, alpha, weight_decay, bf16)
        newW.append(res)
    return newE, newW, idxs


def rowsubset_step(Es, grads, beta: float, ef: str = "raw", **kw):
    """One step of the row-subset rule over a batch.

    Returns (new E list (fp32), out list (fp64), idx list).
    ef="raw" (R8): E_t = M_t = fl32(fl32(beta E) + G), and the output is
    orthogonalize(M_t) with unselected rows = M_t.
    ef="carry" (R14): B = fl32(E + G); the output is orthogonalize(B) with
    unselected rows zero; E_t = fl32(beta B) on the selected rows, B elsewhere.
    """
    if ef not in ("raw", "carry"):
        raise ValueError("ef must be 'raw' or 'carry'")
    newE, outs, idxs = [], [], []
    for E, G in zip(Es, grads):
        if ef == "raw":
            Mt = momentum_update(E, G, beta)
            out, idx = orthogonalize(Mt, **kw)
            newE.append(Mt)
        else:
            B = np.add(np.asarray(E, dtype=np.float32), np.asarray(G, dtype=np.float32), dtype=np.float32)
            out, idx = orthogonalize(B, **kw)
            rest = np.setdiff1d(np.arange(B.shape[0]), idx)
            out[rest] = 0.0
            Et = B.copy()
            Et[idx] = np.multiply(np.float32(beta), B[idx], dtype=np.float32)
            newE.append(Et)
        outs.append(out)
        idxs.append(idx)
    return newE, outs, idxs


# --------------------------------------------------------------------------
# Error metric used by every parity gate
# --------------------------------------------------------------------------
def rel_frobenius(approx, exact) -> float:
    """||approx - exact||_F / ||exact||_F (0 when both are zero)."""
    A = np.asarray(approx, dtype=np.float64)
    B = np.asarray(exact, dtype=np.float64)
    den = float(np.linalg.norm(B))
    num = float(np.linalg.norm(A - B))
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return num / den
