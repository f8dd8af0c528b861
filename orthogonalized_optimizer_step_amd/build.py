"""Builds the HIP library in-tree: orthogonalized_optimizer_step_amd/libdion.so (gfx950).

    python orthogonalized_optimizer_step_amd/build.py

(run as a script: importing the package needs the library it builds)

Every source is compiled with hipcc for gfx950 only.  The momentum kernel's
two fp32 roundings rely on explicit round-to-nearest intrinsics; the
stream-kernel unit is additionally built with contraction off.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libdion.so")
ARCH = "gfx950"

SOURCES = [
    ("gemm_kernels.hip", []),
    ("stream_kernels.hip", ["-ffp-contract=off"]),
    ("lowrank_kernels.hip", ["-ffp-contract=off"]),
    ("lowrank_gemm.hip", []),
    ("tiny_kernels.hip", []),
    ("dion_api.cpp", []),
]

BASE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs, procs = [], []
    for src, extra in SOURCES:   # the units compile concurrently
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [cc] + BASE_FLAGS + extra + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    failed = []
    for src, pr in procs:
        out, err = pr.communicate()
        if pr.returncode != 0:
            failed.append(f"hipcc failed on {src}:\n{out}\n{err}")
    if failed:
        raise RuntimeError("\n".join(failed))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
