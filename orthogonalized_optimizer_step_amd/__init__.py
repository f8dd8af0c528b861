"""MI355X-native Gram Newton-Schulz orthogonalization (Dion3 hot path).

Thin Python binding over the C ABI in include/dion.h.  Every step of the
path runs in the HIP kernels of libdion.so; this module only marshals
pointers, shapes and parameters, and uses PyTorch for device memory and the
current stream.
"""
from __future__ import annotations

import ctypes

from ._lib import DION_BF16, DION_FP16, DION_FP32, PHASE, PREC, DionError, DionParams, DionShape, check, lib

__all__ = ["orth_batched", "rowsubset_step", "workspace_size", "useful_flops", "Orthogonalizer",
           "DionError", "QUINTIC", "profile_enable", "profile_records", "rowkeys_topk", "syrk", "sympoly",
           "apply", "rowsubset_step_update", "Dion3", "restart_points", "lowrank_step",
           "lowrank_workspace_size", "orth_batched_noalloc", "NOALLOC_SCRATCH_BYTES"]

QUINTIC = (3.4445, -4.7750, 2.0315)


EF = {"raw": 0, "carry": 1}


def _params(coeffs, n_iter, restart_every, restart_mask, safety, row_frac, precision, restart_threshold=0.0,
            ef="raw", keep_schedule=False):
    flat = [float(x) for trip in ([coeffs] if len(coeffs) == 3 and not hasattr(coeffs[0], "__len__")
                                  else coeffs) for x in trip]
    arr = (ctypes.c_float * len(flat))(*flat)
    p = DionParams(ctypes.cast(arr, ctypes.POINTER(ctypes.c_float)), len(flat) // 3, int(n_iter),
                   int(restart_every), int(restart_mask), float(safety), float(row_frac),
                   PREC[precision] if isinstance(precision, str) else int(precision), float(restart_threshold),
                   EF[ef] if isinstance(ef, str) else int(ef), int(bool(keep_schedule)))
    return p, arr


def _shapes(shapes):
    arr = (DionShape * len(shapes))()
    for i, (r, c) in enumerate(shapes):
        arr[i].rows, arr[i].cols = int(r), int(c)
    return arr


def _dtype_code(dt):
    import torch
    if dt == torch.bfloat16:
        return DION_BF16
    if dt == torch.float32:
        return DION_FP32
    if dt == torch.float16:
        return DION_FP16
    raise DionError(-1, f"unsupported dtype {dt}")


def _ptrs(tensors):
    return (ctypes.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])


def _check_tensors(ts, dtype=None, shapes=None, what="matrices", device=True):
    """Refuse, before any C call, a list that does not match the batch the
    call was planned for: its length and each shape (when ``shapes`` is
    given), the dtype, and (with ``device``) 2-D contiguous device tensors."""
    ts = list(ts)
    if shapes is not None:
        if len(ts) != len(shapes):
            raise DionError(-1, f"{what}: {len(ts)} tensors for a batch of {len(shapes)}")
        for i, (t, sh) in enumerate(zip(ts, shapes)):
            if tuple(t.shape) != tuple(sh):
                raise DionError(-1, f"{what}[{i}]: shape {tuple(t.shape)}, planned {tuple(sh)}")
    for t in ts:
        if dtype is not None and t.dtype != dtype:
            raise DionError(-1, f"{what}: expected {dtype}, got {t.dtype}")
        if device and (t.dim() != 2 or not t.is_cuda or not t.is_contiguous()):
            raise DionError(-1, f"{what} must be 2-D, contiguous, on the GPU")


def workspace_size(shapes, dtype="bf16", coeffs=QUINTIC, n_iter=5, restart_every=0, restart_mask=0,
                   safety=1.0, row_frac=1.0, precision="auto", restart_threshold=0.0, keep_schedule=False,
                   budget=None) -> int:
    """Workspace bytes of a call; with ``budget``, of the call run in waves that
    fit it (dion_workspace_size_capped)."""
    p, keep = _params(coeffs, n_iter, restart_every, restart_mask, safety, row_frac, precision, restart_threshold,
                      keep_schedule=keep_schedule)
    code = {"bf16": DION_BF16, "fp32": DION_FP32, "fp16": DION_FP16}.get(dtype, dtype)
    if budget is None:
        n = lib.dion_workspace_size(_shapes(shapes), len(shapes), code, ctypes.byref(p))
    else:
        n = lib.dion_workspace_size_capped(_shapes(shapes), len(shapes), code, ctypes.byref(p), int(budget))
    if n == 0:
        raise DionError(-1, lib.dion_last_error().decode())
    return int(n)


def useful_flops(shapes, coeffs=QUINTIC, n_iter=5, restart_every=0, restart_mask=0, safety=1.0,
                 row_frac=1.0, restart_threshold=0.0) -> float:
    p, keep = _params(coeffs, n_iter, restart_every, restart_mask, safety, row_frac, "auto", restart_threshold)
    return float(lib.dion_useful_flops(_shapes(shapes), len(shapes), ctypes.byref(p)))


def restart_points(coeffs=QUINTIC, n_iter=5, restart_every=0, restart_mask=0, safety=1.0,
                   restart_threshold=0.0) -> list:
    """The iterations (1-based) after which these hyper-parameters restart, as the library plans them."""
    p, keep = _params(coeffs, n_iter, restart_every, restart_mask, safety, 1.0, "auto", restart_threshold)
    buf = (ctypes.c_int32 * 64)()
    n = lib.dion_restart_points(ctypes.byref(p), buf, 64)
    check(n if n < 0 else 0)
    return [int(buf[i]) for i in range(n)]


def _workspace(nbytes, device, workspace, stream=None):
    """The caller's workspace, or a new one.  A new one is allocated in the
    stream the call runs on, so that the caching allocator does not hand its
    memory to other work before that stream has finished with it."""
    import torch
    if workspace is None:
        if stream is not None and str(device) != "cpu":
            with torch.cuda.stream(stream):
                workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        else:
            workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-workspace.data_ptr()) % 256
    if workspace.numel() - off < nbytes:
        raise DionError(-3, f"workspace too small: need {nbytes} bytes")
    return workspace, workspace.data_ptr() + off, workspace.numel() - off


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(stream, *tensors):
    """Tensors this binding allocated and a call on a stream other than the
    current one writes: tell the caching allocator that stream uses them."""
    if stream is None:
        return
    for t in tensors:
        if t is None:
            continue
        for x in (t if isinstance(t, (list, tuple)) else [t]):
            x.record_stream(stream)


def _dtype_of(dtype):
    import torch
    return {"bf16": torch.bfloat16, "fp32": torch.float32, "fp16": torch.float16, DION_BF16: torch.bfloat16,
            DION_FP32: torch.float32, DION_FP16: torch.float16}.get(dtype, dtype)


def _sel_check(sel_idx, n):
    if sel_idx is not None:
        import torch
        if sel_idx.dtype != torch.int32 or sel_idx.numel() < n or not sel_idx.is_cuda or not sel_idx.is_contiguous():
            raise DionError(-1, f"sel_idx must be a contiguous int32 GPU tensor of at least {n} entries")


class Orthogonalizer:
    """A reusable megabatch: fixed shapes, dtype and hyper-parameters, with
    its own workspace, so repeated calls only marshal pointers."""

    def __init__(self, shapes, dtype="bf16", coeffs=QUINTIC, n_iter=5, restart_every=0, restart_mask=0,
                 safety=1.0, row_frac=1.0, precision="auto", device="cuda", step_mode=False, restart_threshold=0.0,
                 ef="raw", keep_schedule=False, stream=None, workspace_budget=None):
        import torch
        self.shapes = [tuple(int(x) for x in s) for s in shapes]
        self.dtype = dtype
        self.step_mode = step_mode
        self._p, self._keep = _params(coeffs, n_iter, restart_every, restart_mask, safety, row_frac, precision,
                                      restart_threshold, ef, keep_schedule)
        self._shp = _shapes(self.shapes)
        code = DION_FP32 if step_mode else {"bf16": DION_BF16, "fp32": DION_FP32, "fp16": DION_FP16}.get(dtype, dtype)
        if workspace_budget is None:
            self.ws_bytes = lib.dion_workspace_size(self._shp, len(self.shapes), code, ctypes.byref(self._p))
        else:   # waves of matrices that fit the budget
            self.ws_bytes = lib.dion_workspace_size_capped(self._shp, len(self.shapes), code, ctypes.byref(self._p),
                                                           int(workspace_budget))
        if self.ws_bytes == 0:
            raise DionError(-1, lib.dion_last_error().decode())
        self._ws_tensor, self._ws, self._ws_len = _workspace(self.ws_bytes, device, None, stream)
        self.selected = [int(lib.dion_selected_rows(r, ctypes.c_float(float(row_frac)))) for r, _ in self.shapes]
        self.total_selected = sum(self.selected)

    def useful_flops(self):
        return float(lib.dion_useful_flops(self._shp, len(self.shapes), ctypes.byref(self._p)))

    def __call__(self, Ms, outs, sel_idx=None, stream=None):
        if self.step_mode:
            raise DionError(-1, "this batch was planned for the row-subset step: use step() or step_update()")
        dt = _dtype_of(self.dtype)
        for ts, what in ((Ms, "Ms"), (outs, "outs")):
            _check_tensors(ts, dt, self.shapes, what, device=False)
        for ts, what in ((Ms, "Ms"), (outs, "outs")):
            _check_tensors(ts, dt, self.shapes, what)
        _sel_check(sel_idx, self.total_selected)
        code = _dtype_code(Ms[0].dtype)
        rc = lib.dion_orth_batched(_ptrs(Ms), _ptrs(outs), self._shp, len(self.shapes), code, ctypes.byref(self._p),
                                   ctypes.c_void_p(sel_idx.data_ptr() if sel_idx is not None else None),
                                   ctypes.c_void_p(self._ws), self._ws_len, _stream(stream))
        check(rc)
        return outs

    def step_update(self, Es, grads, Ws, beta, alphas, weight_decay=0.0, sel_idx=None, stream=None):
        """Row-subset step with the fused weight update W <- W (1 - wd) - alpha_i U."""
        import torch
        if not self.step_mode:
            raise DionError(-1, "this batch was not planned for the row-subset step")
        if len(alphas) != len(self.shapes):
            raise DionError(-1, f"{len(alphas)} alphas for a batch of {len(self.shapes)}")
        lists = ((Es, torch.float32, "Es"), (grads, grads[0].dtype if len(grads) else None, "grads"),
                 (Ws, Ws[0].dtype if len(Ws) else None, "Ws"))
        for dev in (False, True):
            for ts, dt, what in lists:
                _check_tensors(ts, dt, self.shapes, what, device=dev)
        _sel_check(sel_idx, self.total_selected)
        gcode = _dtype_code(grads[0].dtype)
        wcode = _dtype_code(Ws[0].dtype)
        al = (ctypes.c_float * len(alphas))(*[float(a) for a in alphas])
        rc = lib.dion_rowsubset_step_update(_ptrs(Es), _ptrs(grads), _ptrs(Ws), self._shp, len(self.shapes), gcode,
                                            wcode, float(beta), al, float(weight_decay), ctypes.byref(self._p),
                                            ctypes.c_void_p(sel_idx.data_ptr() if sel_idx is not None else None),
                                            ctypes.c_void_p(self._ws), self._ws_len, _stream(stream))
        check(rc)
        return Ws

    def step(self, Es, grads, outs, beta, sel_idx=None, stream=None):
        import torch
        if not self.step_mode:
            raise DionError(-1, "this batch was not planned for the row-subset step")
        lists = ((Es, torch.float32, "Es"), (grads, grads[0].dtype if len(grads) else None, "grads"),
                 (outs, torch.bfloat16, "outs"))
        for dev in (False, True):
            for ts, dt, what in lists:
                _check_tensors(ts, dt, self.shapes, what, device=dev)
        _sel_check(sel_idx, self.total_selected)
        code = _dtype_code(grads[0].dtype)
        rc = lib.dion_rowsubset_step(_ptrs(Es), _ptrs(grads), _ptrs(outs), self._shp, len(self.shapes), code,
                                     float(beta), ctypes.byref(self._p),
                                     ctypes.c_void_p(sel_idx.data_ptr() if sel_idx is not None else None),
                                     ctypes.c_void_p(self._ws), self._ws_len, _stream(stream))
        check(rc)
        return outs


def orth_batched(Ms, outs=None, coeffs=QUINTIC, n_iter=5, restart_every=0, restart_mask=0, safety=1.0,
                 row_frac=1.0, precision="auto", return_indices=False, stream=None, restart_threshold=0.0,
                 keep_schedule=False, workspace_budget=None):
    """Orthogonalize a list of 2-D bf16 or fp32 CUDA tensors in one megabatched call.

    Returns the list of outputs (same shapes and dtype), and with
    ``return_indices`` also the per-matrix selected rows (int32, ascending).
    """
    import torch
    _check_tensors(Ms, Ms[0].dtype)
    dt = {torch.bfloat16: "bf16", torch.float16: "fp16"}.get(Ms[0].dtype, "fp32")
    orth = Orthogonalizer([tuple(M.shape) for M in Ms], dt, coeffs, n_iter, restart_every, restart_mask,
                          safety, row_frac, precision, device=Ms[0].device, restart_threshold=restart_threshold,
                          keep_schedule=keep_schedule, stream=stream, workspace_budget=workspace_budget)
    new_outs = outs is None
    if new_outs:
        outs = [torch.empty_like(M) for M in Ms]
    _check_tensors(outs, Ms[0].dtype)
    sel = torch.empty(orth.total_selected, dtype=torch.int32, device=Ms[0].device) if return_indices else None
    orth(Ms, outs, sel, stream)
    _on_stream(stream, outs if new_outs else None, sel)
    if not return_indices:
        return outs
    return outs, list(torch.split(sel, orth.selected))


NOALLOC_SCRATCH_BYTES = 256 << 20   # DION_NOALLOC_SCRATCH_BYTES


def orth_batched_noalloc(Ms, outs, coeffs=QUINTIC, n_iter=5, restart_every=0, restart_mask=0, safety=1.0,
                         row_frac=1.0, precision="auto", sel_idx=None, stream=None, restart_threshold=0.0,
                         keep_schedule=False):
    """dion_orth_batched_noalloc: orth_batched with the library's fixed scratch
    array (no workspace, no device allocation in the call).  ``outs`` (and
    ``sel_idx``, int32 of the total selected rows) are the caller's."""
    _check_tensors(Ms, Ms[0].dtype)
    _check_tensors(outs, Ms[0].dtype)
    shapes = [tuple(M.shape) for M in Ms]
    if [tuple(o.shape) for o in outs] != shapes:
        raise DionError(-1, "outs must match the inputs' shapes")
    p, keep = _params(coeffs, n_iter, restart_every, restart_mask, safety, row_frac, precision, restart_threshold,
                      keep_schedule=keep_schedule)
    check(lib.dion_orth_batched_noalloc(_ptrs(Ms), _ptrs(outs), _shapes(shapes), len(Ms), _dtype_code(Ms[0].dtype),
                                        ctypes.byref(p), ctypes.c_void_p(sel_idx.data_ptr() if sel_idx is not None
                                                                         else None), _stream(stream)))
    return outs


def rowsubset_step(Es, grads, beta, outs=None, coeffs=QUINTIC, n_iter=5, restart_every=0, restart_mask=0,
                   safety=1.0, row_frac=0.125, return_indices=False, stream=None, restart_threshold=0.0, ef="raw",
                   keep_schedule=False):
    """One row-subset step; returns bf16 outputs.

    ef="raw": E <- fl32(fl32(beta E) + grad) in place, unselected output rows are E.
    ef="carry": E <- fl32(E + grad), then the selected rows of E decay to fl32(beta E)
    and the unselected output rows are zero (the carry form of error feedback).
    """
    import torch
    _check_tensors(Es, torch.float32)
    _check_tensors(grads, grads[0].dtype)
    orth = Orthogonalizer([tuple(E.shape) for E in Es], "fp32", coeffs, n_iter, restart_every, restart_mask,
                          safety, row_frac, "mfma16", device=Es[0].device, step_mode=True,
                          restart_threshold=restart_threshold, ef=ef, keep_schedule=keep_schedule, stream=stream)
    new_outs = outs is None
    if new_outs:
        outs = [torch.empty(E.shape, dtype=torch.bfloat16, device=E.device) for E in Es]
    _check_tensors(outs, torch.bfloat16)
    sel = torch.empty(orth.total_selected, dtype=torch.int32, device=Es[0].device) if return_indices else None
    orth.step(Es, grads, outs, beta, sel, stream)
    _on_stream(stream, outs if new_outs else None, sel)
    if not return_indices:
        return outs
    return outs, list(torch.split(sel, orth.selected))


# ------------------------------------------------------------ phase entry points
def _phase_ws(phase, shapes, dtype_code, precision, row_frac, device, stream=None):
    n = lib.dion_phase_workspace_size(PHASE[phase], _shapes(shapes), len(shapes), dtype_code,
                                      PREC[precision] if isinstance(precision, str) else int(precision),
                                      ctypes.c_float(float(row_frac)))
    if n == 0:
        raise DionError(-1, lib.dion_last_error().decode())
    return _workspace(n, device, None, stream)


def _gram_side(shape):
    return min(int(shape[0]), int(shape[1]))


def rowkeys_topk(Ms, row_frac=1.0, stream=None):
    """Squared L2 norm of every row (fp64) and the selected rows of each matrix
    (int32, ascending).  Returns (list of key vectors, list of index vectors)."""
    import torch
    _check_tensors(Ms, Ms[0].dtype)
    shapes = [tuple(M.shape) for M in Ms]
    code = _dtype_code(Ms[0].dtype)
    keep, ws, wl = _phase_ws("rowkeys_topk", shapes, code, "mfma16", row_frac, Ms[0].device, stream)
    ks = [int(lib.dion_selected_rows(r, ctypes.c_float(float(row_frac)))) for r, _ in shapes]
    keys = torch.empty(sum(r for r, _ in shapes), dtype=torch.float64, device=Ms[0].device)
    idx = torch.empty(sum(ks), dtype=torch.int32, device=Ms[0].device)
    check(lib.dion_rowkeys_topk_batched(_ptrs(Ms), _shapes(shapes), len(Ms), code, ctypes.c_float(float(row_frac)),
                                        ctypes.c_void_p(keys.data_ptr()), ctypes.c_void_p(idx.data_ptr()),
                                        ctypes.c_void_p(ws), wl, _stream(stream)))
    _on_stream(stream, keys, idx)
    return list(torch.split(keys, [r for r, _ in shapes])), list(torch.split(idx, ks))


def syrk(Xs, precision="auto", stream=None):
    """Gram matrix on the Gram side of each matrix (X X^T if wide, X^T X if tall), fp32."""
    import torch
    _check_tensors(Xs, Xs[0].dtype)
    shapes = [tuple(X.shape) for X in Xs]
    code = _dtype_code(Xs[0].dtype)
    keep, ws, wl = _phase_ws("syrk", shapes, code, precision, 1.0, Xs[0].device, stream)
    Gs = [torch.empty((_gram_side(s), _gram_side(s)), dtype=torch.float32, device=Xs[0].device) for s in shapes]
    check(lib.dion_syrk_batched(_ptrs(Xs), _ptrs(Gs), _shapes(shapes), len(Xs), code,
                                PREC[precision] if isinstance(precision, str) else int(precision),
                                ctypes.c_void_p(ws), wl, _stream(stream)))
    _on_stream(stream, Gs)
    return Gs


def sympoly(Gs, coeffs=QUINTIC, precision="auto", stream=None):
    """a I + b G + c G^2 for symmetric fp32 G with spectral norm <= 1."""
    import torch
    _check_tensors(Gs, torch.float32)
    ms = [int(G.shape[0]) for G in Gs]
    if any(G.shape[0] != G.shape[1] for G in Gs):
        raise DionError(-1, "G must be square")
    keep, ws, wl = _phase_ws("sympoly", [(m, m) for m in ms], DION_FP32, precision, 1.0, Gs[0].device, stream)
    Ps = [torch.empty_like(G) for G in Gs]
    co = (ctypes.c_float * 3)(*[float(x) for x in coeffs])
    check(lib.dion_sympoly_batched(_ptrs(Gs), _ptrs(Ps), (ctypes.c_int32 * len(ms))(*ms), len(Gs), co,
                                   PREC[precision] if isinstance(precision, str) else int(precision),
                                   ctypes.c_void_p(ws), wl, _stream(stream)))
    _on_stream(stream, Ps)
    return Ps


def apply(Qs, Xs, precision="auto", stream=None):
    """Q X (wide X) or X Q (tall X) with Q the fp32 m x m factor on the Gram side."""
    import torch
    _check_tensors(Xs, Xs[0].dtype)
    _check_tensors(Qs, torch.float32)
    shapes = [tuple(X.shape) for X in Xs]
    for Q, s in zip(Qs, shapes):
        if tuple(Q.shape) != (_gram_side(s), _gram_side(s)):
            raise DionError(-1, f"Q must be {_gram_side(s)} x {_gram_side(s)} for X of shape {s}")
    code = _dtype_code(Xs[0].dtype)
    keep, ws, wl = _phase_ws("apply", shapes, code, precision, 1.0, Xs[0].device, stream)
    Ys = [torch.empty_like(X) for X in Xs]
    check(lib.dion_apply_batched(_ptrs(Qs), _ptrs(Xs), _ptrs(Ys), _shapes(shapes), len(Xs), code,
                                 PREC[precision] if isinstance(precision, str) else int(precision),
                                 ctypes.c_void_p(ws), wl, _stream(stream)))
    _on_stream(stream, Ys)
    return Ys


def rowsubset_step_update(Es, grads, Ws, beta, alphas, weight_decay=0.0, coeffs=QUINTIC, n_iter=5,
                          restart_every=0, restart_mask=0, safety=1.0, row_frac=0.125, return_indices=False,
                          stream=None, restart_threshold=0.0, ef="raw", keep_schedule=False):
    """One row-subset step fused with the weight update; E and W are updated in place."""
    import torch
    _check_tensors(Es, torch.float32)
    _check_tensors(grads, grads[0].dtype)
    _check_tensors(Ws, Ws[0].dtype)
    orth = Orthogonalizer([tuple(E.shape) for E in Es], "fp32", coeffs, n_iter, restart_every, restart_mask,
                          safety, row_frac, "mfma16", device=Es[0].device, step_mode=True,
                          restart_threshold=restart_threshold, ef=ef, keep_schedule=keep_schedule, stream=stream)
    sel = torch.empty(orth.total_selected, dtype=torch.int32, device=Es[0].device) if return_indices else None
    orth.step_update(Es, grads, Ws, beta, alphas, weight_decay, sel, stream)
    _on_stream(stream, sel)
    if not return_indices:
        return Ws
    return Ws, list(torch.split(sel, orth.selected))


LOWRANK_MODE = {"qr": 0, "colnorm": 1}


def lowrank_workspace_size(shapes, rank, out_dtype="bf16") -> int:
    code = {"bf16": DION_BF16, "fp32": DION_FP32, "fp16": DION_FP16}.get(out_dtype, out_dtype)
    n = lib.dion_lowrank_workspace_size(_shapes(shapes), len(shapes), int(rank), code)
    if n == 0:
        raise DionError(-1, lib.dion_last_error().decode())
    return int(n)


def lowrank_step(Ms, grads, Qs, beta, mode="qr", outs=None, out_dtype=None, workspace=None, stream=None):
    """One Dion ("colnorm") or Orth-Dion ("qr") low-rank step over a batch.

    Ms: fp32 R x C buffers (updated in place); grads: R x C gradients (bf16,
    fp32 or fp16); Qs: fp32 C x r right factors, r = min(rank, R, C) with one
    rank for the batch (read, then overwritten with the new factors).
    Returns the R x C updates P Q^T (bf16 unless out_dtype or outs say
    otherwise).
    """
    import torch
    _check_tensors(Ms, torch.float32)
    _check_tensors(grads, grads[0].dtype)
    _check_tensors(Qs, torch.float32)
    shapes = [tuple(M.shape) for M in Ms]
    rank = max(int(Q.shape[1]) for Q in Qs)
    for (R, C), Q in zip(shapes, Qs):
        if tuple(Q.shape) != (C, min(rank, R, C)):
            raise DionError(-1, f"Q must be {C} x {min(rank, R, C)} for a {R} x {C} matrix at rank {rank}")
    new_outs = outs is None
    if new_outs:
        dt = out_dtype if out_dtype is not None else torch.bfloat16
        outs = [torch.empty(s, dtype=dt, device=Ms[0].device) for s in shapes]
    _check_tensors(outs, outs[0].dtype)
    ocode = _dtype_code(outs[0].dtype)
    nbytes = lib.dion_lowrank_workspace_size(_shapes(shapes), len(shapes), rank, ocode)
    if nbytes == 0:
        raise DionError(-1, lib.dion_last_error().decode())
    keep, ws, wl = _workspace(nbytes, Ms[0].device, workspace, stream)
    check(lib.dion_lowrank_step(_ptrs(Ms), _ptrs(grads), _ptrs(Qs), _ptrs(outs), _shapes(shapes), len(Ms),
                                _dtype_code(grads[0].dtype), ocode, rank, float(beta),
                                LOWRANK_MODE[mode] if isinstance(mode, str) else int(mode),
                                ctypes.c_void_p(ws), wl, _stream(stream)))
    _on_stream(stream, outs if new_outs else None)
    return outs


def profile_enable(on=True) -> bool:
    """Start (clearing old records) or stop per-phase event profiling on this thread."""
    return bool(lib.dion_profile_enable(1 if on else 0))


def profile_records():
    """[(name, kernel, ms, useful_flops, mfma_flops, bytes, algorithmic_flops)] of the phases
    enqueued while profiling."""
    recs = []
    name, kern = ctypes.c_char_p(), ctypes.c_char_p()
    ms = ctypes.c_float()
    u, r, b, a = ctypes.c_double(), ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    for i in range(lib.dion_profile_count()):
        check(lib.dion_profile_get(i, ctypes.byref(name), ctypes.byref(kern), ctypes.byref(ms), ctypes.byref(u),
                                   ctypes.byref(r), ctypes.byref(b)))
        check(lib.dion_profile_get_algorithmic(i, ctypes.byref(a)))
        recs.append((name.value.decode(), kern.value.decode(), ms.value, u.value, r.value, b.value, a.value))
    return recs


from .optim import Dion3  # noqa: E402
