"""ctypes loader for libdion.so (the HIP library built in-tree by build.py).

There is no fallback: if the library is missing or fails to load, importing
the package raises, so nothing can silently run elsewhere.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdion.so")

DION_BF16, DION_FP32, DION_FP16 = 0, 1, 2
PHASE = {"rowkeys_topk": 1, "syrk": 2, "sympoly": 3, "apply": 4}
PREC = {"auto": 0, "mfma16": 1, "fp64": 2}


class DionShape(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int32), ("cols", ctypes.c_int32)]


class DionParams(ctypes.Structure):
    _fields_ = [
        ("ns_coeffs", ctypes.POINTER(ctypes.c_float)),
        ("n_coeff_sets", ctypes.c_int32),
        ("n_iter", ctypes.c_int32),
        ("restart_every", ctypes.c_int32),
        ("restart_mask", ctypes.c_uint32),
        ("safety", ctypes.c_float),
        ("row_frac", ctypes.c_float),
        ("precision", ctypes.c_int32),
        ("restart_threshold", ctypes.c_float),
        ("ef_carry", ctypes.c_int32),
        ("keep_schedule", ctypes.c_int32),
    ]


# every symbol declared in include/dion.h
EXPORTS = (
    "dion_workspace_size", "dion_orth_batched", "dion_orth_batched_simple",
    "dion_rowsubset_step", "dion_useful_flops", "dion_selected_rows", "dion_strerror",
    "dion_last_error", "dion_version", "dion_profile_enable", "dion_profile_count",
    "dion_profile_get", "dion_phase_workspace_size", "dion_rowkeys_topk_batched", "dion_syrk_batched",
    "dion_sympoly_batched", "dion_apply_batched", "dion_rowsubset_step_update", "dion_restart_points",
    "dion_lowrank_workspace_size", "dion_lowrank_step", "dion_orth_batched_noalloc", "dion_workspace_size_capped",
    "dion_profile_get_algorithmic",
)


class DionError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dion error {code}: {msg}")
        self.code = code


def _load():
    # PyTorch bundles its own HIP runtime (libamdhip64, libhsa-runtime64) under
    # a file name that the dynamic linker does not match against ours: loading
    # libdion.so first would bring /opt/rocm's runtime and torch would then add
    # a second one to the process (the second sees no device).  Importing torch
    # first makes libdion.so bind to the runtime already loaded.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python orthogonalized_optimizer_step_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    pp = ctypes.POINTER(ctypes.c_void_p)
    shp = ctypes.POINTER(DionShape)
    prm = ctypes.POINTER(DionParams)
    lib.dion_workspace_size.argtypes = [shp, i32, i32, prm]
    lib.dion_workspace_size.restype = sz
    lib.dion_orth_batched.argtypes = [pp, pp, shp, i32, i32, prm, vp, vp, sz, vp]
    lib.dion_orth_batched.restype = ctypes.c_int
    lib.dion_workspace_size_capped.argtypes = [shp, i32, i32, prm, sz]
    lib.dion_workspace_size_capped.restype = sz
    lib.dion_orth_batched_noalloc.argtypes = [pp, pp, shp, i32, i32, prm, vp, vp]
    lib.dion_orth_batched_noalloc.restype = ctypes.c_int
    lib.dion_orth_batched_simple.argtypes = [pp, pp, shp, i32, i32, ctypes.POINTER(ctypes.c_float), i32, i32,
                                             ctypes.c_float, ctypes.c_float, vp, sz, vp]
    lib.dion_orth_batched_simple.restype = ctypes.c_int
    lib.dion_rowsubset_step.argtypes = [pp, pp, pp, shp, i32, i32, ctypes.c_float, prm, vp, vp, sz, vp]
    lib.dion_rowsubset_step.restype = ctypes.c_int
    lib.dion_useful_flops.argtypes = [shp, i32, prm]
    lib.dion_useful_flops.restype = ctypes.c_double
    lib.dion_selected_rows.argtypes = [i32, ctypes.c_float]
    lib.dion_selected_rows.restype = i32
    lib.dion_restart_points.argtypes = [prm, ctypes.POINTER(i32), i32]
    lib.dion_restart_points.restype = ctypes.c_int
    lib.dion_lowrank_workspace_size.argtypes = [shp, i32, i32, i32]
    lib.dion_lowrank_workspace_size.restype = sz
    lib.dion_lowrank_step.argtypes = [pp, pp, pp, pp, shp, i32, i32, i32, i32, ctypes.c_float, i32, vp, sz, vp]
    lib.dion_lowrank_step.restype = ctypes.c_int
    lib.dion_strerror.argtypes = [ctypes.c_int]
    lib.dion_strerror.restype = ctypes.c_char_p
    lib.dion_last_error.argtypes = []
    lib.dion_last_error.restype = ctypes.c_char_p
    lib.dion_profile_enable.argtypes = [ctypes.c_int]
    lib.dion_profile_enable.restype = ctypes.c_int
    lib.dion_profile_count.argtypes = []
    lib.dion_profile_count.restype = ctypes.c_int
    dp = ctypes.POINTER(ctypes.c_double)
    lib.dion_profile_get.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_char_p),
                                     ctypes.POINTER(ctypes.c_float), dp, dp, dp]
    lib.dion_profile_get.restype = ctypes.c_int
    lib.dion_profile_get_algorithmic.argtypes = [ctypes.c_int, dp]
    lib.dion_profile_get_algorithmic.restype = ctypes.c_int
    lib.dion_version.argtypes = []
    lib.dion_version.restype = ctypes.c_int
    fp = ctypes.POINTER(ctypes.c_float)
    lib.dion_phase_workspace_size.argtypes = [i32, shp, i32, i32, i32, ctypes.c_float]
    lib.dion_phase_workspace_size.restype = sz
    lib.dion_rowkeys_topk_batched.argtypes = [pp, shp, i32, i32, ctypes.c_float, vp, vp, vp, sz, vp]
    lib.dion_rowkeys_topk_batched.restype = ctypes.c_int
    lib.dion_syrk_batched.argtypes = [pp, pp, shp, i32, i32, i32, vp, sz, vp]
    lib.dion_syrk_batched.restype = ctypes.c_int
    lib.dion_sympoly_batched.argtypes = [pp, pp, ctypes.POINTER(i32), i32, fp, i32, vp, sz, vp]
    lib.dion_sympoly_batched.restype = ctypes.c_int
    lib.dion_apply_batched.argtypes = [pp, pp, pp, shp, i32, i32, i32, vp, sz, vp]
    lib.dion_apply_batched.restype = ctypes.c_int
    lib.dion_rowsubset_step_update.argtypes = [pp, pp, pp, shp, i32, i32, i32, ctypes.c_float, fp, ctypes.c_float,
                                               prm, vp, vp, sz, vp]
    lib.dion_rowsubset_step_update.restype = ctypes.c_int
    return lib


lib = _load()


def check(rc: int):
    if rc != 0:
        raise DionError(rc, f"{lib.dion_strerror(rc).decode()}: {lib.dion_last_error().decode()}")
