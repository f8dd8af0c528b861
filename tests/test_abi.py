"""C ABI checks that need no GPU: the library loads, exports every function
declared in include/dion.h, and its host-side functions (workspace sizing,
FLOP count, selected-row count, argument validation) behave as documented.
No kernel is launched here."""
import ctypes
import os
import re

import pytest

import orthogonalized_optimizer_step_amd as dion
from orthogonalized_optimizer_step_amd import _lib
from oracle import dion_oracle as O
from workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "dion.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dion_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert len(names) >= 9
    cdll = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(cdll, n), n
    assert set(names) == set(_lib.EXPORTS)


def test_no_internal_symbol_left_undefined():
    """Every function of the library's own namespace is defined in it: a shared
    library links with undefined symbols, which would fail only when loaded
    lazily on first use."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", "-C", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    missing = [ln.strip() for ln in out.splitlines() if "dion::" in ln or " dion_" in ln]
    assert not missing, missing


def test_profile_get_algorithmic_index_checked():
    """The algorithmic-FLOP query rejects an index outside the records."""
    lib = _lib.lib
    lib.dion_profile_enable(1)
    lib.dion_profile_enable(0)
    v = ctypes.c_double(-1.0)
    assert lib.dion_profile_count() == 0
    assert lib.dion_profile_get_algorithmic(0, ctypes.byref(v)) == -1
    assert lib.dion_profile_get_algorithmic(-1, None) == -1
    assert v.value == -1.0


def test_version():
    assert _lib.lib.dion_version() == 100


@pytest.mark.parametrize("R,frac", [(4096, 0.125), (14336, 0.125), (28672, 0.25), (1000, 0.1), (7, 0.5),
                                    (5, 1e-6), (5, 1.0), (8192, 0.25), (3, 0.34)])
def test_selected_rows_matches_oracle(R, frac):
    f32 = ctypes.c_float(frac).value
    assert _lib.lib.dion_selected_rows(R, ctypes.c_float(frac)) == O.selected_count(R, f32)


def test_useful_flops_formula():
    # m=64, n=128, K=5, no restart: one segment of length 5
    m, n = 64, 128
    expect = n * m * (m + 1) + 2 * m * m * n + (4 * 5 - 3) * m * m * (m + 1)
    assert dion.useful_flops([(64, 128)]) == expect
    # restarts every 2 with K=5: segments 2, 2, 1
    seg = lambda L: n * m * (m + 1) + 2 * m * m * n + (4 * L - 3) * m * m * (m + 1)
    assert dion.useful_flops([(128, 64)], restart_every=2) == 2 * seg(2) + seg(1)
    wl = WORKLOADS["llama3_8b"]
    assert abs(dion.useful_flops(wl.shapes, restart_every=2) / 1e12 - 371.617) < 0.01


def test_workspace_size_monotone_and_invalid():
    small = dion.workspace_size([(64, 128)])
    big = dion.workspace_size([(64, 128), (300, 200)])
    assert 0 < small < big
    assert dion.workspace_size([(64, 128)], "fp32") > 0
    with pytest.raises(dion.DionError):
        dion.workspace_size([(0, 5)])
    with pytest.raises(dion.DionError):
        dion.workspace_size([(5, 5)], row_frac=0.0)
    with pytest.raises(dion.DionError):
        dion.workspace_size([(5, 5)], n_iter=0)
    with pytest.raises(dion.DionError):
        dion.workspace_size([(5, 5)], coeffs=[(1, 2, 3), (1, 2, 3)], n_iter=3)


def _params(**kw):
    base = dict(coeffs=dion.QUINTIC, n_iter=5, restart_every=0, restart_mask=0, safety=1.0, row_frac=1.0,
                precision="auto")
    base.update(kw)
    return dion._params(**base)


def test_orth_validation_errors_before_launch():
    """Invalid calls return an error code on the host; nothing is launched."""
    lib = _lib.lib
    shp = dion._shapes([(4, 4)])
    fake = (ctypes.c_void_p * 1)(0x1000)
    fake_out = (ctypes.c_void_p * 1)(0x2000)
    p, keep = _params()
    # NULL matrix pointer
    null = (ctypes.c_void_p * 1)(None)
    assert lib.dion_orth_batched(null, fake_out, shp, 1, 0, ctypes.byref(p), None, ctypes.c_void_p(0x10000),
                                 1 << 30, None) == -1
    # out overlapping M
    assert lib.dion_orth_batched(fake, fake, shp, 1, 0, ctypes.byref(p), None, ctypes.c_void_p(0x10000),
                                 1 << 30, None) == -1
    # misaligned / small / NULL workspace
    assert lib.dion_orth_batched(fake, fake_out, shp, 1, 0, ctypes.byref(p), None, ctypes.c_void_p(0x10001),
                                 1 << 30, None) == -3
    assert lib.dion_orth_batched(fake, fake_out, shp, 1, 0, ctypes.byref(p), None, ctypes.c_void_p(0x10000),
                                 16, None) == -3
    assert lib.dion_orth_batched(fake, fake_out, shp, 1, 0, ctypes.byref(p), None, None, 1 << 30, None) == -3
    assert b"workspace" in lib.dion_last_error()
    # bad params
    for bad in (dict(safety=0.0), dict(row_frac=1.5), dict(n_iter=65), dict(precision=7)):
        pb, keep2 = _params(**bad)
        assert lib.dion_orth_batched(fake, fake_out, shp, 1, 0, ctypes.byref(pb), None,
                                     ctypes.c_void_p(0x10000), 1 << 30, None) == -1
    # bad dtype, bad batch
    assert lib.dion_orth_batched(fake, fake_out, shp, 1, 7, ctypes.byref(p), None, ctypes.c_void_p(0x10000),
                                 1 << 30, None) == -1
    assert lib.dion_orth_batched(fake, fake_out, shp, 0, 0, ctypes.byref(p), None, ctypes.c_void_p(0x10000),
                                 1 << 30, None) == -1
    # the step refuses the FP64 path
    pf, keep3 = _params(precision="fp64")
    E = (ctypes.c_void_p * 1)(0x3000)
    g = (ctypes.c_void_p * 1)(0x4000)
    assert lib.dion_rowsubset_step(E, g, fake_out, shp, 1, 0, ctypes.c_float(0.9), ctypes.byref(pf), None,
                                   ctypes.c_void_p(0x10000), 1 << 30, None) == -2
    assert lib.dion_strerror(-2) == b"unsupported combination"


def test_phase_workspace_sizes_and_validation():
    """Host-side checks of the phase entry points: sizes, and argument errors
    returned before any launch (NULL pointers, non-square polynomial input)."""
    L = _lib.lib
    shp = dion._shapes([(300, 200), (64, 640)])
    for ph in (1, 2, 4):
        assert L.dion_phase_workspace_size(ph, shp, 2, _lib.DION_BF16, 1, ctypes.c_float(0.5)) > 0
    assert L.dion_phase_workspace_size(3, shp, 2, _lib.DION_FP32, 1, ctypes.c_float(1.0)) == 0  # not square
    assert L.dion_phase_workspace_size(3, dion._shapes([(64, 64)]), 1, _lib.DION_FP32, 2, ctypes.c_float(1.0)) > 0
    assert L.dion_phase_workspace_size(9, shp, 2, _lib.DION_BF16, 1, ctypes.c_float(1.0)) == 0   # no such phase
    assert L.dion_phase_workspace_size(2, shp, 2, 7, 1, ctypes.c_float(1.0)) == 0                  # bad dtype
    null2 = (ctypes.c_void_p * 2)(None, None)
    assert L.dion_syrk_batched(null2, null2, shp, 2, _lib.DION_BF16, 1, None, 0, None) == -1
    assert L.dion_apply_batched(null2, null2, null2, shp, 2, _lib.DION_BF16, 1, None, 0, None) == -1
    assert L.dion_rowkeys_topk_batched(null2, shp, 2, _lib.DION_BF16, ctypes.c_float(0.0), None, None, None, 0,
                                       None) == -1                                              # row_frac 0
    ms = (ctypes.c_int32 * 1)(0)
    assert L.dion_sympoly_batched(null2, null2, ms, 1, None, 1, None, 0, None) == -1             # m = 0


@pytest.mark.parametrize("n_iter", [1, 2, 5, 6, 9, 40])
@pytest.mark.parametrize("tau", [5.0, 100.0, 116.0, 1000.0, 1e4, 1e30])
@pytest.mark.parametrize("safety", [1.0, 1.05])
def test_restart_threshold_matches_oracle(n_iter, tau, safety):
    """The planner's restart points for a threshold equal the oracle's (reading R12)."""
    got = dion.restart_points(n_iter=n_iter, safety=safety, restart_threshold=tau)
    want = O.restart_points(n_iter, restart_threshold=tau,
                            coeff_list=O.coefficient_schedule(dion.QUINTIC, n_iter, safety))
    assert got == want


def test_restart_points_schedules_and_precedence():
    sched = [(2.0, -1.0, 0.5), (2.0, -1.0, 0.5), (4.0, -1.0, 0.5), (1.5, -1.0, 0.5), (3.0, -1.0, 0.5)]
    want = O.restart_points(5, restart_threshold=15.0, coeff_list=O.coefficient_schedule(sched, 5))
    assert want == [2, 3]
    assert dion.restart_points(coeffs=sched, n_iter=5, restart_threshold=15.0) == want
    assert dion.restart_points(coeffs=sched, n_iter=5, restart_every=1, restart_threshold=15.0) == want
    assert dion.restart_points(coeffs=sched, n_iter=5, restart_mask=0b1, restart_threshold=15.0) == [1]
    assert dion.restart_points(n_iter=6, restart_every=2) == O.restart_points(6, restart_every=2)
    assert dion.restart_points(n_iter=5, restart_mask=0b10) == [2]
    assert dion.restart_points(n_iter=40, restart_mask=1 << 31) == [32]
    assert dion.restart_points(n_iter=5) == []


def test_restart_threshold_flops_and_validation():
    shapes = [(4096, 4096), (1024, 4096), (4096, 14336)]
    assert dion.useful_flops(shapes, restart_threshold=100.0) == dion.useful_flops(shapes, restart_every=2)
    assert dion.useful_flops(shapes, restart_threshold=1000.0) == dion.useful_flops(shapes, restart_mask=0b100)
    for bad in (-1.0, float("nan"), float("inf")):
        with pytest.raises(dion.DionError):
            dion.restart_points(n_iter=5, restart_threshold=bad)
        with pytest.raises(dion.DionError):
            dion.workspace_size(shapes, restart_threshold=bad)


def test_lowrank_validation_errors_before_launch():
    """The low-rank entry point rejects bad arguments on the host (fake device pointers, no device work)."""
    shp = (_lib.DionShape * 2)()
    shp[0].rows, shp[0].cols, shp[1].rows, shp[1].cols = 64, 32, 32, 64
    def ptrs(*v):
        return (ctypes.c_void_p * 2)(*v)
    M, G, Q, O = ptrs(0x10000, 0x20000), ptrs(0x30000, 0x40000), ptrs(0x50000, 0x60000), ptrs(0x70000, 0x80000)
    need = dion.lowrank_workspace_size([(64, 32), (32, 64)], 8)
    # the update is written in its dtype by the last product: no fp32 staging buffer
    assert need > 0 and dion.lowrank_workspace_size([(64, 32), (32, 64)], 8, "fp32") == need

    def call(M=M, G=G, Q=Q, O=O, rank=8, beta=1.0, mode=0, gdt=0, odt=0, ws=0x100000, nbytes=need, batch=2):
        return _lib.lib.dion_lowrank_step(M, G, Q, O, shp, batch, gdt, odt, rank, beta, mode,
                                          ctypes.c_void_p(ws), nbytes, None)
    assert call(rank=0) == -1
    assert call(rank=513) == -2
    assert call(mode=2) == -1
    assert call(gdt=7) == -1
    assert call(odt=7) == -1
    assert call(beta=float("nan")) == -1
    assert call(batch=0) == -1
    assert call(O=ptrs(0x10000, 0x80000)) == -1          # out overlaps M
    assert call(Q=ptrs(0x10000 + 64, 0x60000)) == -1     # Q overlaps M
    assert call(G=ptrs(0x10000 + 128, 0x40000)) == -1    # grad overlaps M
    assert call(M=ptrs(0, 0x20000)) == -1                # NULL matrix
    assert call(nbytes=need - 1) == -3                   # workspace too small
    assert call(ws=0x100001) == -3                       # misaligned
    assert call(ws=0) == -3


def test_ef_carry_validation():
    """ef_carry is 0 or 1; anything else is rejected when the parameters are parsed."""
    shp = [(64, 32)]
    assert dion.workspace_size(shp, "fp32", row_frac=0.25) > 0
    p, keep = dion._params(dion.QUINTIC, 5, 2, 0, 1.0, 0.25, "mfma16", 0.0, "carry")
    assert p.ef_carry == 1
    p.ef_carry = 2
    assert _lib.lib.dion_workspace_size(dion._shapes(shp), 1, _lib.DION_FP32, ctypes.byref(p)) == 0
    assert "ef_carry" in _lib.lib.dion_last_error().decode()


def test_keep_schedule_validation_and_plan():
    """keep_schedule is 0 or 1.  Left at 0, a run of more than two iterations between
    restarts is cut by extra restarts on the MFMA16 path: the plan then holds the second
    restart buffer, and where the cut makes exactly two restarts on a wide matrix the
    accumulated-factor buffers too, so it needs more workspace; the fp64 path and short-run
    schedules plan the same either way.  Useful FLOPs follow the schedule as given."""
    shp = [(768, 3072), (768, 768)]
    p, keep = dion._params(dion.QUINTIC, 5, 0, 0, 1.0, 1.0, "auto", 0.0, "raw", True)
    assert p.keep_schedule == 1
    p.keep_schedule = 2
    assert _lib.lib.dion_workspace_size(dion._shapes(shp), 2, _lib.DION_BF16, ctypes.byref(p)) == 0
    assert "keep_schedule" in _lib.lib.dion_last_error().decode()
    # no restart -> {2, 4}; {2} -> {2, 4}; {1} of 6 -> {1, 3, 5} (three restarts: no
    # accumulated factor, and the second restart buffer was there already)
    for sched, grows in ((dict(), True), (dict(restart_mask=0b10), True), (dict(n_iter=6, restart_mask=0b1), False)):
        split = dion.workspace_size(shp, "bf16", **sched)
        kept = dion.workspace_size(shp, "bf16", keep_schedule=True, **sched)
        assert (split > kept) if grows else (split == kept), sched
        assert dion.workspace_size(shp, "fp32", precision="fp64", **sched) == \
            dion.workspace_size(shp, "fp32", precision="fp64", keep_schedule=True, **sched)
    for sched in (dict(restart_every=2), dict(n_iter=2), dict(restart_every=1)):
        assert dion.workspace_size(shp, "bf16", **sched) == dion.workspace_size(shp, "bf16", keep_schedule=True,
                                                                                 **sched), sched
    assert dion.restart_points(n_iter=5) == []


def _orth_rc(shapes, dtype=_lib.DION_BF16, **kw):
    """dion_orth_batched's status for these hyper-parameters with placeholder
    pointers: the plan is checked before any pointer is used."""
    p, keep = dion._params(kw.pop("coeffs", dion.QUINTIC), kw.pop("n_iter", 5), kw.pop("restart_every", 0),
                           kw.pop("restart_mask", 0), kw.pop("safety", 1.0), 1.0, kw.pop("precision", "auto"),
                           keep_schedule=kw.pop("keep_schedule", False))
    assert not kw
    n = len(shapes)
    fake = (ctypes.c_void_p * n)(*[0x10000 * (i + 1) for i in range(n)])
    out = (ctypes.c_void_p * n)(*[0x90000000 + 0x10000 * i for i in range(n)])
    return _lib.lib.dion_orth_batched(fake, out, dion._shapes(shapes), n, dtype, ctypes.byref(p), None, None, 0,
                                      None)


def test_mfma16_iteration_range_guard():
    """The MFMA16 path refuses schedules beyond the range its 2e-2 error bound is
    established for (more than 12 iterations, slopes multiplying to more than
    3.4445^12, or a kept run of more than two iterations where a run exceeds 5
    iterations or the slopes multiply to more than 3.4445^6), with
    DION_E_UNSUPPORTED before any launch; the FP64 path and matrices that take
    the one-launch fp64 kernel (Gram side <= 64 and long side <= 1024, or Gram
    side <= 16) accept them."""
    big = [(256, 512)]
    tiny = [(64, 1024), (16, 20000), (30000, 9)]
    ws = -3   # DION_E_WORKSPACE: the plan was accepted, the (absent) workspace was not
    assert _orth_rc(big, n_iter=12, restart_every=2) == ws
    for kw in (dict(n_iter=13, restart_every=2), dict(n_iter=20), dict(coeffs=(5.0, -6.0, 2.0), n_iter=10),
               dict(n_iter=6, keep_schedule=True), dict(n_iter=8, restart_mask=0b1, keep_schedule=True),
               dict(n_iter=8, restart_mask=0b100100, keep_schedule=True),
               dict(n_iter=7, restart_mask=0b10000, keep_schedule=True)):
        assert _orth_rc(big, **kw) == -2, kw
        assert _orth_rc(big, precision="fp64", **kw) == ws, kw
        assert _orth_rc(tiny, **kw) == ws, kw
        with pytest.raises(dion.DionError):
            dion.workspace_size(big, "bf16", **kw)
    # slopes below the quintic's pass; the safety factor divides the slopes
    assert _orth_rc(big, coeffs=(1.5, -0.5, 0.0), n_iter=12) == ws
    assert _orth_rc(big, coeffs=(3.6, -4.8, 2.0), n_iter=12, safety=1.05) == ws
    assert _orth_rc(big, coeffs=(3.6, -4.8, 2.0), n_iter=12) == -2
    assert _orth_rc(big, n_iter=5, keep_schedule=True) == ws
    # kept runs: accepted up to six iterations of the fixed quintic, with lower
    # slopes, or where no run is longer than two (keep changes nothing)
    assert _orth_rc(big, n_iter=6, restart_mask=0b1, keep_schedule=True) == ws
    assert _orth_rc(big, coeffs=(1.5, -0.5, 0.0), n_iter=8, restart_mask=0b100100, keep_schedule=True) == ws
    assert _orth_rc(big, n_iter=8, restart_every=2, keep_schedule=True) == ws
    # the row-subset step (MFMA16 only) refuses the same schedules
    p, keep = dion._params(dion.QUINTIC, 13, 2, 0, 1.0, 0.125, "mfma16")
    fake = (ctypes.c_void_p * 1)(0x10000)
    rc = _lib.lib.dion_rowsubset_step(fake, (ctypes.c_void_p * 1)(0x20000), (ctypes.c_void_p * 1)(0x90000000),
                                      dion._shapes([(2048, 512)]), 1, _lib.DION_BF16, 0.9, ctypes.byref(p), None, None, 0,
                                      None)
    assert rc == -2


def test_binding_refuses_mismatched_batches():
    """The binding checks tensor lists against the planned batch before any C
    call: count, shapes, dtype, the entry point the batch was planned for and
    the index buffer (the C library would otherwise read past the pointer
    arrays or the tensors)."""
    import torch
    shapes = [(4, 6), (8, 3)]
    orth = dion.Orthogonalizer(shapes, "bf16", device="cpu")
    ok = [torch.zeros(s, dtype=torch.bfloat16) for s in shapes]
    for Ms, outs, msg in [
        (ok[:1], ok, "1 tensors for a batch of 2"),
        (ok, ok + ok[:1], "3 tensors for a batch of 2"),
        ([ok[0], torch.zeros((3, 8), dtype=torch.bfloat16)], ok, "planned (8, 3)"),
        ([torch.zeros(s) for s in shapes], ok, "expected torch.bfloat16"),
        (ok, ok, "on the GPU"),                    # right shapes, but host tensors
    ]:
        with pytest.raises(dion.DionError, match=msg.replace("(", r"\(").replace(")", r"\)")):
            orth(Ms, outs)
    with pytest.raises(dion.DionError, match="row-subset step"):
        orth.step(ok, ok, ok, 0.9)
    step = dion.Orthogonalizer(shapes, "fp32", precision="mfma16", device="cpu", step_mode=True, row_frac=0.5)
    E = [torch.zeros(s) for s in shapes]
    with pytest.raises(dion.DionError, match="planned for the row-subset step"):
        step(E, E)
    with pytest.raises(dion.DionError, match="2 tensors for a batch of 2|planned"):
        step.step(E, [torch.zeros((4, 6), dtype=torch.bfloat16)] * 2, ok, 0.9)
    with pytest.raises(dion.DionError, match="alphas"):
        step.step_update(E, ok, ok, 0.9, [0.1])


def test_workspace_cap_sizes():
    """dion_workspace_size_capped: the full size when it fits the cap, otherwise
    the largest wave's plan (at most the cap, at least one matrix's); 0 when one
    matrix alone exceeds the cap (the bound counts the whole call's header, so a
    cap of exactly one matrix's own plan is not enough)."""
    wl = WORKLOADS["llama3_8b"]
    full = dion.workspace_size(wl.shapes, "bf16", restart_every=2)
    assert dion.workspace_size(wl.shapes, "bf16", restart_every=2, budget=full) == full
    one = dion.workspace_size([wl.shapes[4]], "bf16", restart_every=2)   # a 14336 x 4096 matrix alone
    prev = 0
    for cap in (one + (64 << 20), 2 * one, 8 << 30, 32 << 30, full - 1):
        need = dion.workspace_size(wl.shapes, "bf16", restart_every=2, budget=cap)
        assert one <= need <= cap and need >= prev
        prev = need
    with pytest.raises(dion.DionError):
        dion.workspace_size(wl.shapes, "bf16", restart_every=2, budget=one - 1)
    # a workspace below one matrix's need is still refused by the call itself
    p, keep = dion._params(dion.QUINTIC, 5, 2, 0, 1.0, 1.0, "auto")
    fake = (ctypes.c_void_p * 1)(0x10000)
    out = (ctypes.c_void_p * 1)(0x90000000)
    rc = _lib.lib.dion_orth_batched(fake, out, dion._shapes([(4096, 4096)]), 1, _lib.DION_BF16, ctypes.byref(p), None,
                                    ctypes.c_void_p(1 << 20), 1 << 20, None)
    assert rc == -3 and b"alone needs" in _lib.lib.dion_last_error()
