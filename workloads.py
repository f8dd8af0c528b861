"""Seeded synthetic inputs and workload definitions.

This module holds no arithmetic of the method: it only draws random numbers,
rounds them to the stored dtype and describes the five workloads (shapes and
hyper-parameters).  Both sides of every parity check take their inputs from
here: the GPU path receives the device tensors, the oracle receives copies of
the very same bytes.

Workloads (the pages name no benchmark or dataset, so these synthetic,
transformer-shaped momentum matrices stand in for one):

  fp32_64x128      one fp32 64x128 matrix, rank-8 + 0.1 noise, K=5, no restart
  gpt2_small       36 bf16 matrices (12 each of 768x768, 768x3072, 3072x768),
                   rank-32 + 0.1 noise; K=5, one restart after iteration 2,
                   safety 1.01
  llama3_8b        Llama-3-8B layer set x 32 layers (q,o 4096x4096; k,v
                   1024x4096; gate,up 14336x4096; down 4096x14336), bf16,
                   rank-64 + 0.05 noise, per-matrix scale 10^U(-3,0); K=5,
                   restart every 2
  llama3_8b_rows   same layer set, row-subset mode: top 1/8 rows, fp32
                   momentum buffer (beta 0.95), 10 steps of fresh gradients
  llama3_70b       16 copies each of 8192x8192, 1024x8192, 28672x8192,
                   8192x28672, singular values k^-1/2 with random orthogonal
                   factors; K=6, restart every 2, safety 1.05, top 1/4 rows
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

QUINTIC = (3.4445, -4.7750, 2.0315)

LLAMA3_8B_LAYER = (
    ("q", 4096, 4096),
    ("k", 1024, 4096),
    ("v", 1024, 4096),
    ("o", 4096, 4096),
    ("gate", 14336, 4096),
    ("up", 14336, 4096),
    ("down", 4096, 14336),
)
LLAMA3_70B_SHAPES = ((8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672))


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shapes: tuple           # ((rows, cols), ...) in batch order
    dtype: str              # stored dtype of the momentum: "bf16" or "fp32"
    n_iter: int
    restart_every: int = 0
    restart_mask: int = 0
    safety: float = 1.0
    row_frac: float = 1.0
    coeffs: tuple = QUINTIC
    beta: float = 0.0       # row-subset mode only
    steps: int = 1          # row-subset mode only

    def ns_kwargs(self):
        return dict(coeffs=self.coeffs, n_iter=self.n_iter,
                    restart_every=self.restart_every, restart_mask=self.restart_mask,
                    safety=self.safety, row_frac=self.row_frac)

    @property
    def params(self) -> int:
        return int(sum(r * c for r, c in self.shapes))


def _llama8b_shapes(n_layers=32):
    return tuple((r, c) for _ in range(n_layers) for _, r, c in LLAMA3_8B_LAYER)


WORKLOADS = {
    "fp32_64x128": Workload("fp32_64x128", ((64, 128),), "fp32", n_iter=5),
    "gpt2_small": Workload(
        "gpt2_small", ((768, 768),) * 12 + ((768, 3072),) * 12 + ((3072, 768),) * 12,
        "bf16", n_iter=5, restart_mask=0b10, safety=1.01),
    "llama3_8b": Workload("llama3_8b", _llama8b_shapes(), "bf16", n_iter=5, restart_every=2),
    "llama3_8b_rows": Workload("llama3_8b_rows", _llama8b_shapes(), "bf16", n_iter=5,
                               restart_every=2, row_frac=0.125, beta=0.95, steps=10),
    "llama3_70b": Workload(
        "llama3_70b", tuple(s for s in LLAMA3_70B_SHAPES for _ in range(16)), "bf16",
        n_iter=6, restart_every=2, safety=1.05, row_frac=0.25),
}


# --------------------------------------------------------------------------
# bf16 helpers (round-to-nearest-even, as a storage format only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x) -> np.ndarray:
    """fp32 array whose values are exactly the bf16 rounding of x."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def seed_of(*key) -> int:
    """A 63-bit seed derived from a key tuple (used for torch generators)."""
    h = hashlib.sha256(repr(tuple(key)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


# --------------------------------------------------------------------------
# Host (numpy) generators: exact recipes for the small workloads
# --------------------------------------------------------------------------
def fp32_64x128() -> np.ndarray:
    """M = A B^T + 0.1 N with A 64x8, B 128x8, N 64x128 ~ N(0,1), seed 0, fp32."""
    rng = np.random.default_rng(0)
    A = rng.standard_normal((64, 8))
    B = rng.standard_normal((128, 8))
    N = rng.standard_normal((64, 128))
    return (A @ B.T + 0.1 * N).astype(np.float32)


def lowrank_np(key, rows, cols, rank, noise, log_scale=None) -> np.ndarray:
    """scale * (A B^T + noise N), fp32, from numpy PCG64 keyed by ``key``.

    A rows x rank, B cols x rank, N rows x cols ~ N(0,1); with ``log_scale =
    (lo, hi)`` the scale is 10^U(lo, hi) drawn from the same stream first.
    """
    rng = np.random.default_rng(list(key))
    scale = 1.0
    if log_scale is not None:
        scale = 10.0 ** rng.uniform(*log_scale)
    A = rng.standard_normal((rows, rank), dtype=np.float32)
    B = rng.standard_normal((cols, rank), dtype=np.float32)
    N = rng.standard_normal((rows, cols), dtype=np.float32)
    return (np.float32(scale) * (A @ B.T + np.float32(noise) * N)).astype(np.float32)


def gpt2_small_np():
    """The 36 bf16 matrices of the GPT-2-small batch, as bf16 bit arrays."""
    wl = WORKLOADS["gpt2_small"]
    return [f32_to_bf16_bits(lowrank_np((2, i), r, c, 32, 0.1)) for i, (r, c) in enumerate(wl.shapes)]


def heavytail_np(key, rows, cols, exponent=0.5) -> np.ndarray:
    """U diag(k^-exponent) V^T with U, V from QR of Gaussians (host, small sizes)."""
    rng = np.random.default_rng(list(key))
    r = min(rows, cols)
    U, _ = np.linalg.qr(rng.standard_normal((rows, r)))
    V, _ = np.linalg.qr(rng.standard_normal((cols, r)))
    s = np.arange(1, r + 1, dtype=np.float64) ** (-exponent)
    return ((U * s) @ V.T).astype(np.float32)


# --------------------------------------------------------------------------
# Device (torch) generators: the large workloads, drawn where they are used
# --------------------------------------------------------------------------
def lowrank_torch(key, rows, cols, rank, noise, log_scale=None, device="cuda", out_dtype=None):
    """Same recipe as ``lowrank_np`` drawn with a torch generator on ``device``.

    Returns a tensor of ``out_dtype`` (default bfloat16, rounded to nearest
    even by the dtype conversion).
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*key))
    scale = 1.0
    if log_scale is not None:
        u = torch.rand((1,), generator=g, device=device, dtype=torch.float64).item()
        scale = 10.0 ** (log_scale[0] + (log_scale[1] - log_scale[0]) * u)
    A = torch.randn((rows, rank), generator=g, device=device, dtype=torch.float32)
    B = torch.randn((cols, rank), generator=g, device=device, dtype=torch.float32)
    M = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)
    M.mul_(noise)
    M.addmm_(A, B.t())
    M.mul_(scale)
    return M.to(out_dtype or torch.bfloat16)


def heavytail_copies_torch(key, rows, cols, copies, exponent=0.5, device="cuda", out_dtype=None):
    """`copies` matrices U diag(d_c) V^T sharing U and V, the Q factors of
    seeded Gaussians (fp32): d_c is the spectrum k^-exponent in a seeded
    random order with random signs, so every copy has the same singular
    values, assigned to different pairs of singular vectors.  (Two QRs per
    shape rather than per copy: the QR of a 28672 x 8192 Gaussian takes
    seconds.)"""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*key))
    r = min(rows, cols)
    U, _ = torch.linalg.qr(torch.randn((rows, r), generator=g, device=device, dtype=torch.float32))
    V, _ = torch.linalg.qr(torch.randn((cols, r), generator=g, device=device, dtype=torch.float32))
    s = torch.arange(1, r + 1, device=device, dtype=torch.float32).pow(-exponent)
    out = []
    for _ in range(copies):
        perm = torch.randperm(r, generator=g, device=device)
        sign = torch.randint(0, 2, (r,), generator=g, device=device).to(torch.float32).mul_(2.0).sub_(1.0)
        out.append(((U * (s[perm] * sign)) @ V.t()).to(out_dtype or torch.bfloat16))
    del U, V
    return out


def llama3_8b_torch(step=None, n_layers=32, device="cuda"):
    """The Llama-3-8B layer-set momentum (or the gradients of one step)."""
    mats = []
    for layer in range(n_layers):
        for j, (_, r, c) in enumerate(LLAMA3_8B_LAYER):
            key = (3, layer, j) if step is None else (4, step, layer, j)
            mats.append(lowrank_torch(key, r, c, 64, 0.05, log_scale=(-3.0, 0.0), device=device))
    return mats


def llama3_70b_torch(copies=16, device="cuda"):
    """The Llama-3-70B-shaped stress: `copies` heavy-tailed matrices of each shape."""
    mats = []
    for si, (r, c) in enumerate(LLAMA3_70B_SHAPES):
        mats.extend(heavytail_copies_torch((5, si), r, c, copies, device=device))
    return mats
