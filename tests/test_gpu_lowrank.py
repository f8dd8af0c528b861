"""Parity of the low-rank Dion / Orth-Dion step (through the C ABI) with the
fp64 oracle.

Gates: the accumulated buffer B = fl32(M + G) bit-exact (checked with beta = 0,
where the buffer is B); the new right factor and an fp32 update within 1e-4
relative Frobenius error of the oracle (fp32 GEMMs and shifted CholeskyQR3 with an
fp64 Cholesky factor); the new buffer B - beta P W^T within 1e-4 of ||B||, the
scale of its operands (at full rank and beta = 1 it is zero up to rounding, so
an error relative to itself says nothing); a bf16 update within its rounding
(2^-8 relative) plus 1e-4.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import orthdion_oracle as L  # noqa: E402
from oracle.dion_oracle import rel_frobenius  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = 1e-4


@pytest.fixture(scope="module")
def dion():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import orthogonalized_optimizer_step_amd as d
    return d


def make(shapes, rank, seed, grad_dtype=torch.bfloat16, scale=1.0):
    rng = np.random.default_rng(seed)
    Ms, Gs, Qs = [], [], []
    for R, C in shapes:
        r = min(rank, R, C)
        # a decaying spectrum keeps B Q and W well conditioned
        A = rng.standard_normal((R, 8)) @ rng.standard_normal((8, C)) + 0.3 * rng.standard_normal((R, C))
        Ms.append((scale * A).astype(np.float32))
        g = torch.from_numpy((0.5 * scale * rng.standard_normal((R, C))).astype(np.float32)).to(grad_dtype)
        Gs.append(g)
        Qs.append(rng.standard_normal((C, r)).astype(np.float32))
    return Ms, Gs, Qs


def run(dion, Ms, Gs, Qs, beta, mode, out_dtype=torch.float32):
    dM = [torch.from_numpy(M.copy()).cuda() for M in Ms]
    dG = [g.cuda() for g in Gs]
    dQ = [torch.from_numpy(Q.copy()).cuda() for Q in Qs]
    outs = dion.lowrank_step(dM, dG, dQ, beta, mode=mode, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return dM, dQ, outs


def as64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def buf_err(gpu, ref, M, G):
    """Frobenius error of the new buffer relative to ||B||, B = fl32(M + G)."""
    B = L.accumulate(M, G).astype(np.float64)
    return float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(B), 1e-300))


SHAPES = [(64, 48), (48, 64), (130, 70), (70, 130), (200, 200), (33, 257), (257, 33), (9, 5)]


@pytest.mark.parametrize("mode", ["qr", "colnorm"])
@pytest.mark.parametrize("beta", [1.0, 0.1])
@pytest.mark.parametrize("grad_dtype", [torch.bfloat16, torch.float32, torch.float16])
def test_lowrank_small_ragged(dion, mode, beta, grad_dtype):
    Ms, Gs, Qs = make(SHAPES, 16, 11, grad_dtype)
    dM, dQ, outs = run(dion, Ms, Gs, Qs, beta, mode)
    errs = []
    for i in range(len(Ms)):
        G = Gs[i].float().numpy()
        M_ref, Q_ref, _, D_ref = L.lowrank_step(Ms[i], G, Qs[i], beta, mode)
        e = (buf_err(as64(dM[i]), M_ref, Ms[i], G), rel_frobenius(as64(dQ[i]), Q_ref),
             rel_frobenius(as64(outs[i]), D_ref))
        errs.append(max(e))
        assert max(e) <= TOL, (SHAPES[i], e)
    print("lowrank", mode, beta, grad_dtype, f"max err {max(errs):.2e}", flush=True)


def test_lowrank_buffer_bit_exact_beta0(dion):
    """beta = 0 leaves the buffer at B = fl32(M + G): bit-exact (reading D1)."""
    Ms, Gs, Qs = make(SHAPES, 8, 12, torch.bfloat16)
    dM, _, _ = run(dion, Ms, Gs, Qs, 0.0, "qr")
    for i, M in enumerate(Ms):
        B = L.accumulate(M, Gs[i].float().numpy())
        assert np.array_equal(dM[i].cpu().numpy().view(np.uint32), B.view(np.uint32)), SHAPES[i]


@pytest.mark.parametrize("mode", ["qr", "colnorm"])
@pytest.mark.parametrize("grad_dtype", [torch.bfloat16, torch.float16])
def test_lowrank_formed_buffer_matches_stored_buffer(dion, mode, grad_dtype):
    """16-bit gradients have B = fl32(M + G) formed where it is read; fp32
    gradients have it stored by a pass first.  The same gradient values given
    both ways must give bit-identical buffers, right factors and updates (the
    ragged shapes take the masked loads, the 256-multiples the vector ones)."""
    shapes = SHAPES + [(512, 384), (384, 512), (1024, 256)]
    Ms, Gs, Qs = make(shapes, 64, 14, grad_dtype)
    G32 = [g.float() for g in Gs]   # exact: every 16-bit value is an fp32 value
    for beta in (0.1, 1.0):
        a = run(dion, Ms, Gs, Qs, beta, mode, out_dtype=torch.bfloat16)
        b = run(dion, Ms, G32, Qs, beta, mode, out_dtype=torch.bfloat16)
        for x, y in zip(a, b):
            for i, s in enumerate(shapes):
                assert torch.equal(x[i].view(torch.int16) if x[i].dtype == torch.bfloat16 else x[i].view(torch.int32),
                                   y[i].view(torch.int16) if y[i].dtype == torch.bfloat16 else y[i].view(torch.int32)), \
                    (s, beta, mode, grad_dtype)


@pytest.mark.parametrize("mode", ["qr", "colnorm"])
def test_lowrank_bf16_output_and_partial_isometry(dion, mode):
    shapes = [(300, 200), (200, 300), (512, 512)]
    Ms, Gs, Qs = make(shapes, 24, 13)
    _, _, outs = run(dion, Ms, Gs, Qs, 1.0, mode, out_dtype=torch.bfloat16)
    for i, s in enumerate(shapes):
        _, _, _, D_ref = L.lowrank_step(Ms[i], Gs[i].float().numpy(), Qs[i], 1.0, mode)
        assert rel_frobenius(as64(outs[i]), D_ref) <= 2.0 ** -8 + TOL, s
        if mode == "qr":   # Orth-Dion: r singular values equal to one (within bf16 rounding)
            sv = np.linalg.svd(as64(outs[i]), compute_uv=False)
            assert np.abs(sv[:24] - 1.0).max() < 2e-2 and sv[24] < 2e-2


@pytest.mark.parametrize("mode", ["qr", "colnorm"])
@pytest.mark.parametrize("beta", [1.0, 0.1])
def test_lowrank_bf16_update_from_hi_terms(dion, mode, beta):
    """A bf16 update is computed from the fp16 hi terms of P and Q' alone (one
    product).  Against the oracle its error may exceed the bf16 rounding of the
    exact update by at most a quarter (the one-term product's error is about a
    tenth of it), on ragged shapes and at ranks 16 and 64; the buffer and the
    right factor are those of the fp32-output call, bit for bit."""
    shapes = SHAPES + [(512, 384), (384, 512), (1024, 256)]
    for rank, seed in ((16, 21), (64, 22)):
        Ms, Gs, Qs = make(shapes, rank, seed)
        dM, dQ, outs = run(dion, Ms, Gs, Qs, beta, mode, out_dtype=torch.bfloat16)
        dM32, dQ32, _ = run(dion, Ms, Gs, Qs, beta, mode, out_dtype=torch.float32)
        worst = 0.0
        for i, s in enumerate(shapes):
            assert torch.equal(dM[i].view(torch.int32), dM32[i].view(torch.int32)), s
            assert torch.equal(dQ[i].view(torch.int32), dQ32[i].view(torch.int32)), s
            _, _, _, D_ref = L.lowrank_step(Ms[i], Gs[i].float().numpy(), Qs[i], beta, mode)
            rounded = torch.from_numpy(D_ref.astype(np.float32)).to(torch.bfloat16).float().numpy()
            e_round = rel_frobenius(rounded.astype(np.float64), D_ref)
            e = rel_frobenius(as64(outs[i]), D_ref)
            worst = max(worst, e / max(e_round, 1e-300))
            assert e <= 1.25 * e_round + 1e-6, (s, rank, e, e_round)
        print(f"lowrank bf16 update {mode} beta {beta} rank {rank}: error / bf16 rounding at most {worst:.3f}",
              flush=True)


def test_lowrank_exact_recovery(dion):
    """With Q = the top-r right singular vectors of B, the update is U_r V_r^T."""
    shapes = [(120, 80), (80, 120)]
    Ms, Gs, _ = make(shapes, 10, 14)
    Gs = [torch.zeros(s, dtype=torch.float32) for s in shapes]
    Qs = []
    for M in Ms:
        _, _, Vt = np.linalg.svd(M.astype(np.float64), full_matrices=False)
        Qs.append(Vt[:10].T.astype(np.float32))
    _, _, outs = run(dion, Ms, Gs, Qs, 1.0, "qr")
    for i, M in enumerate(Ms):
        U, _, Vt = np.linalg.svd(M.astype(np.float64), full_matrices=False)
        assert rel_frobenius(as64(outs[i]), U[:, :10] @ Vt[:10]) < 1e-4


def test_lowrank_three_steps(dion):
    """Three chained steps (buffer and right factor carried) track the oracle's chain."""
    shapes = [(96, 64), (64, 96), (150, 150)]
    Ms, _, Qs = make(shapes, 12, 15)
    rng = np.random.default_rng(16)
    dM = [torch.from_numpy(M.copy()).cuda() for M in Ms]
    dQ = [torch.from_numpy(Q.copy()).cuda() for Q in Qs]
    refM = [M.astype(np.float32) for M in Ms]
    refQ = [Q.astype(np.float64) for Q in Qs]
    for t in range(3):
        Gs = [torch.from_numpy(rng.standard_normal(s).astype(np.float32)).to(torch.bfloat16) for s in shapes]
        outs = dion.lowrank_step(dM, [g.cuda() for g in Gs], dQ, 0.5, mode="qr", out_dtype=torch.float32)
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            Mn, Qn, _, D = L.lowrank_step(refM[i], Gs[i].float().numpy(), refQ[i], 0.5, "qr")
            assert rel_frobenius(as64(outs[i]), D) < 1e-3, (t, shapes[i])
            assert buf_err(as64(dM[i]), Mn, refM[i], Gs[i].float().numpy()) < 1e-4
            assert rel_frobenius(as64(dQ[i]), Qn) < 1e-4
            refM[i] = as64(dM[i]).astype(np.float32)   # continue from the GPU's buffer (fp32 state)
            refQ[i] = as64(dQ[i])


def test_lowrank_full_size(dion):
    """Llama-3-8B MLP shapes at rank 256, fp32 update: every element against the
    oracle; and the bf16 update from the hi terms (the benchmarked form) within a
    quarter above the bf16 rounding of the exact update."""
    shapes = [(4096, 14336), (14336, 4096)]
    Ms, Gs, Qs = make(shapes, 256, 17)
    dM, dQ, outs = run(dion, Ms, Gs, Qs, 1.0, "qr")
    _, _, outs16 = run(dion, Ms, Gs, Qs, 1.0, "qr", out_dtype=torch.bfloat16)
    for i, s in enumerate(shapes):
        M_ref, Q_ref, _, D_ref = L.lowrank_step(Ms[i], Gs[i].float().numpy(), Qs[i], 1.0, "qr")
        e = (buf_err(as64(dM[i]), M_ref, Ms[i], Gs[i].float().numpy()), rel_frobenius(as64(dQ[i]), Q_ref),
             rel_frobenius(as64(outs[i]), D_ref))
        rounded = torch.from_numpy(D_ref.astype(np.float32)).to(torch.bfloat16).float().numpy()
        e_round = rel_frobenius(rounded.astype(np.float64), D_ref)
        e16 = rel_frobenius(as64(outs16[i]), D_ref)
        print("lowrank full", s, " ".join(f"{x:.2e}" for x in e), f"bf16 {e16:.3e} (rounding {e_round:.3e})",
              flush=True)
        assert max(e) <= TOL, (s, e)
        assert e16 <= 1.25 * e_round + 1e-6, (s, e16, e_round)


def test_lowrank_zero_input_is_finite(dion):
    shapes = [(64, 32), (32, 64)]
    dM = [torch.zeros(s, device="cuda") for s in shapes]
    dG = [torch.zeros(s, device="cuda", dtype=torch.bfloat16) for s in shapes]
    dQ = [torch.randn(s[1], 8, device="cuda") for s in shapes]
    outs = dion.lowrank_step(dM, dG, dQ, 1.0, mode="qr", out_dtype=torch.float32)
    torch.cuda.synchronize()
    for o, M in zip(outs, dM):
        assert torch.isfinite(o).all() and torch.isfinite(M).all()


@pytest.mark.parametrize("mode", ["qr", "colnorm"])
def test_lowrank_rank_above_256(dion, mode):
    """Ranks 257..512 factor the Gram matrix with the general (scratch-memory) kernel."""
    shapes = [(700, 400), (400, 700), (520, 520)]
    Ms, Gs, Qs = make(shapes, 300, 18)
    dM, dQ, outs = run(dion, Ms, Gs, Qs, 1.0, mode)
    for i, s in enumerate(shapes):
        G = Gs[i].float().numpy()
        M_ref, Q_ref, _, D_ref = L.lowrank_step(Ms[i], G, Qs[i], 1.0, mode)
        e = (buf_err(as64(dM[i]), M_ref, Ms[i], G), rel_frobenius(as64(dQ[i]), Q_ref),
             rel_frobenius(as64(outs[i]), D_ref))
        assert max(e) <= TOL, (s, e)
