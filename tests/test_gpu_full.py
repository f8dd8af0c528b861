"""Full-size parity: the workloads at their real shapes, launched exactly as
bench.py launches them (one megabatched call over every matrix), checked on
sampled matrices that the fp64 oracle computes one by one."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import dion_oracle as O  # noqa: E402
from workloads import WORKLOADS, LLAMA3_8B_LAYER, llama3_8b_torch  # noqa: E402

pytestmark = pytest.mark.gpu
TOL = 2e-2


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.fixture(scope="module")
def llama8b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import orthogonalized_optimizer_step_amd as dion
    wl = WORKLOADS["llama3_8b"]
    Ms = llama3_8b_torch()
    outs = [torch.empty_like(M) for M in Ms]
    orth = dion.Orthogonalizer(wl.shapes, "bf16", wl.coeffs, wl.n_iter, wl.restart_every, wl.restart_mask,
                               wl.safety, wl.row_frac)
    print("llama3_8b: inputs ready, running the megabatch", flush=True)
    orth(Ms, outs)
    torch.cuda.synchronize()
    print("llama3_8b: megabatch done", flush=True)
    del orth   # module fixtures live until the module ends: release the 127 GiB workspace now
    torch.cuda.empty_cache()
    yield wl, Ms, outs
    del Ms, outs
    torch.cuda.empty_cache()


# layer 0 q (square), k (1024x4096), gate (tall 14336x4096), down (wide 4096x14336); layer 31 v
@pytest.mark.parametrize("i", [1, 0, 4, 6, 31 * 7 + 2])
def test_llama3_8b_sampled(llama8b, i):
    wl, Ms, outs = llama8b
    M = Ms[i].float().cpu().numpy()
    ref, _ = O.orthogonalize(M, **wl.ns_kwargs())
    err = O.rel_frobenius(to_np(outs[i]), ref)
    print(f"llama3_8b matrix {i} {M.shape}: rel err {err:.3e}")
    assert err <= TOL


def test_llama3_8b_all_outputs_sane(llama8b):
    """Every output of the megabatch is finite with spectral mass in the NS
    band: Frobenius norm^2 between (#captured) * 0.68^2 and m * 1.21^2."""
    wl, Ms, outs = llama8b
    for o in outs:
        assert torch.isfinite(o.float()).all()
        fro2 = float(o.float().pow(2).sum())
        m = min(o.shape)
        assert 64 * 0.68 ** 2 * 0.9 < fro2 < m * 1.21 ** 2


def selection_ok(idx_gpu, E, frac):
    """Bit-exact against the oracle (keys are the exact sums of squares rounded
    once on both sides, so the selection is unique)."""
    return np.array_equal(np.asarray(idx_gpu, dtype=np.int64), O.select_rows(E, frac))


@pytest.fixture(scope="module")
def llama8b_rows():
    """Ten steps of the row-subset rule over the whole megabatch; layers 0 and
    31 are followed on the host with the oracle step by step."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import orthogonalized_optimizer_step_amd as dion
    from workloads import round_bf16
    wl = WORKLOADS["llama3_8b_rows"]
    sample = list(range(7)) + list(range(31 * 7, 32 * 7))
    Es = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in wl.shapes]
    outs = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in wl.shapes]
    orth = dion.Orthogonalizer(wl.shapes, "bf16", wl.coeffs, wl.n_iter, wl.restart_every, wl.restart_mask,
                               wl.safety, wl.row_frac, "mfma16", step_mode=True)
    sel = torch.empty(orth.total_selected, dtype=torch.int32, device="cuda")
    offs = np.concatenate([[0], np.cumsum(orth.selected)])
    E_host = {i: np.zeros(wl.shapes[i], np.float32) for i in sample}
    res = {"E": [], "idx": [], "rest": [], "err": {}}
    for t in range(1, wl.steps + 1):
        G = llama3_8b_torch(step=t)
        orth.step(Es, G, outs, wl.beta, sel)
        torch.cuda.synchronize()
        print(f"llama3_8b_rows: step {t} done on the GPU, checking", flush=True)
        sel_h = sel.cpu().numpy()
        for i in sample:
            E_host[i] = O.momentum_update(E_host[i], G[i].float().cpu().numpy(), wl.beta)
            E_gpu = Es[i].cpu().numpy()
            res["E"].append(((i, t), np.array_equal(E_host[i].view(np.uint32), E_gpu.view(np.uint32))))
            idx_gpu = sel_h[offs[i]:offs[i + 1]]
            res["idx"].append(((i, t), selection_ok(idx_gpu, E_host[i], wl.row_frac)))
            out_gpu = outs[i].float().cpu().numpy()
            rest = np.setdiff1d(np.arange(wl.shapes[i][0]), idx_gpu)
            res["rest"].append(((i, t), np.array_equal(out_gpu[rest], round_bf16(E_host[i][rest]))))
            if t in (1, wl.steps) and i < 7:
                ref, ridx = O.orthogonalize(E_host[i], **wl.ns_kwargs())
                res["err"][(i, t)] = O.rel_frobenius(out_gpu[ridx].astype(np.float64), ref[ridx])
        del G
    del Es, outs, orth, sel
    torch.cuda.empty_cache()
    yield wl, res


def test_llama3_8b_rows_momentum_bit_exact(llama8b_rows):
    """The fp32 buffer is bit-exact on layers 0 and 31 at all 10 steps."""
    wl, res = llama8b_rows
    bad = [k for k, ok in res["E"] if not ok]
    assert not bad, bad


def test_llama3_8b_rows_selection_bit_exact(llama8b_rows):
    wl, res = llama8b_rows
    bad = [k for k, ok in res["idx"] if not ok]
    assert not bad, bad


def test_llama3_8b_rows_unselected_rows_raw(llama8b_rows):
    """Unselected rows carry bf16(M_t) exactly."""
    wl, res = llama8b_rows
    bad = [k for k, ok in res["rest"] if not ok]
    assert not bad, bad


def test_llama3_8b_rows_update_parity(llama8b_rows):
    """Selected rows within 2e-2 of the oracle at steps 1 and 10 (layer 0)."""
    wl, res = llama8b_rows
    print("llama3_8b_rows selected-row rel err:", {k: f"{v:.2e}" for k, v in res["err"].items()})
    assert len(res["err"]) == 14
    assert max(res["err"].values()) <= TOL


@pytest.fixture(scope="module")
def llama70b_batch():
    """The Llama-3-70B-shaped stress as configured and as bench.py times it: 16
    matrices each of 8192x8192, 1024x8192, 28672x8192 and 8192x28672 (64 in one
    megabatched call), heavy-tailed spectrum k^-1/2 with random orthogonal
    factors from seeded QR (one pair per shape, each copy with its own order and
    signs of the spectrum); K=6, restarts every 2, safety 1.05, top 1/4 of rows."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import orthogonalized_optimizer_step_amd as dion
    from workloads import LLAMA3_70B_SHAPES, heavytail_copies_torch
    wl = WORKLOADS["llama3_70b"]
    Ms = []
    for si, (r, c) in enumerate(LLAMA3_70B_SHAPES):
        Ms.extend(heavytail_copies_torch((5, si), r, c, 16))
        torch.cuda.synchronize()
        print(f"llama3_70b: generated 16 of {r}x{c}", flush=True)
    assert [tuple(M.shape) for M in Ms] == list(wl.shapes)
    outs = [torch.empty_like(M) for M in Ms]
    orth = dion.Orthogonalizer(wl.shapes, "bf16", wl.coeffs, wl.n_iter, wl.restart_every, wl.restart_mask,
                               wl.safety, wl.row_frac)
    sel = torch.empty(orth.total_selected, dtype=torch.int32, device="cuda")
    orth(Ms, outs, sel)
    torch.cuda.synchronize()
    print("llama3_70b: 64-matrix megabatch done", flush=True)
    offs = np.concatenate([[0], np.cumsum(orth.selected)])
    idx = [sel[offs[i]:offs[i + 1]].cpu().numpy() for i in range(len(Ms))]
    del orth, sel
    torch.cuda.empty_cache()
    yield wl, Ms, outs, idx
    del Ms, outs
    torch.cuda.empty_cache()


# per shape: copy 5 against the full oracle (selection, copied rows, Gram-NS)
@pytest.mark.parametrize("i", [16 + 5, 0 + 5, 48 + 5, 32 + 5])
def test_llama3_70b_sampled(llama70b_batch, i):
    wl, Ms, outs, idx = llama70b_batch
    M = Ms[i].float().cpu().numpy()
    assert selection_ok(idx[i], M, wl.row_frac)
    ref, ref_idx = O.orthogonalize(M, **wl.ns_kwargs())
    got = to_np(outs[i])
    rest = np.setdiff1d(np.arange(M.shape[0]), ref_idx)
    assert np.array_equal(got[rest], M[rest].astype(np.float64))   # raw rows carried verbatim
    err = O.rel_frobenius(got[ref_idx], ref[ref_idx])
    print(f"llama3_70b matrix {i} {M.shape}: selected-row rel err {err:.3e}", flush=True)
    assert err <= TOL


def test_llama3_70b_selection_and_copies(llama70b_batch):
    """Selection bit-exact and unselected rows copied on every 1024x8192 matrix and
    on the first and last copy of each other shape; every output finite, with the
    selected rows' spectral mass in the NS band."""
    wl, Ms, outs, idx = llama70b_batch
    check = list(range(16, 32)) + [0, 15, 32, 47, 48, 63]
    for i in check:
        M = Ms[i].float().cpu().numpy()
        assert selection_ok(idx[i], M, wl.row_frac), i
        got = outs[i].float().cpu().numpy()
        rest = np.setdiff1d(np.arange(M.shape[0]), idx[i])
        assert np.array_equal(got[rest], M[rest]), i
        print(f"llama3_70b matrix {i}: selection and copies exact", flush=True)
    for i, o in enumerate(outs):
        sel = o[torch.from_numpy(idx[i].astype(np.int64)).cuda()].float()
        assert torch.isfinite(sel).all(), i
        fro2 = float(sel.pow(2).sum())
        m = min(sel.shape)
        assert m * 0.68 ** 2 * 0.95 < fro2 < m * 1.21 ** 2, (i, fro2, m)
