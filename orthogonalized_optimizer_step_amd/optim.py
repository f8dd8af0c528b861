"""A Muon-style torch optimizer on the Dion3 hot path.

Per step and parameter group, one megabatched library call runs the whole
path for every 2-D parameter: the fp32 momentum update, the row-subset
selection, Gram Newton-Schulz and the weight update (the flow of the Dion3
summary, 输入输出流程; the pages present Dion3 as a drop-in replacement for
Muon, swapping only the optimizer class).  This module only gathers pointers,
learning-rate scales and the persistent momentum buffers; the arithmetic runs
in libdion.so.
"""
from __future__ import annotations

import math

import torch

QUINTIC = (3.4445, -4.7750, 2.0315)


def rows_over_cols_scale(shape) -> float:
    """sqrt(max(1, rows / cols)): the learning-rate factor that gives tall
    matrices an update of the same per-element size as square ones."""
    r, c = int(shape[0]), int(shape[1])
    return math.sqrt(max(1.0, r / c))


class Dion3(torch.optim.Optimizer):
    """Row-subset Gram Newton-Schulz optimizer for 2-D parameters.

    Arguments
      lr            learning rate
      momentum      heavy-ball factor beta of the fp32 momentum buffer
                    (M <- beta M + grad, two fp32 roundings)
      row_frac      fraction of each momentum matrix's rows orthogonalized per
                    step (largest L2 norms); the other rows apply the raw momentum
      weight_decay  decoupled: W <- W (1 - lr * weight_decay) - lr * scale * update
      ns_coeffs, n_iter, restart_every, safety, restart_threshold
                    the Gram Newton-Schulz schedule (a positive restart_threshold
                    replaces restart_every: restart once the product of a_k^2
                    since the last restart reaches it)
      ef            "raw" (the buffer keeps the momentum; unselected rows step with it)
                    or "carry" (unselected rows are carried in the buffer undecayed
                    and do not step; only the selected rows decay by momentum)
      shape_scale   callable(shape) -> float, or None for 1 (default:
                    sqrt(max(1, rows / cols)))

    Parameters must be 2-D CUDA tensors (bf16 or fp32); gradients bf16 or
    fp32.  Parameters of a group are batched by (gradient dtype, weight
    dtype) into one library call each.
    """

    def __init__(self, params, lr=0.02, momentum=0.95, row_frac=0.125, weight_decay=0.0, ns_coeffs=QUINTIC,
                 n_iter=5, restart_every=2, safety=1.0, shape_scale=rows_over_cols_scale, restart_threshold=0.0,
                 ef="raw"):
        if lr < 0 or not 0 < row_frac <= 1 or weight_decay < 0:
            raise ValueError("invalid lr, row_frac or weight_decay")
        defaults = dict(lr=lr, momentum=momentum, row_frac=row_frac, weight_decay=weight_decay,
                        ns_coeffs=tuple(ns_coeffs), n_iter=n_iter, restart_every=restart_every, safety=safety,
                        shape_scale=shape_scale, restart_threshold=restart_threshold, ef=ef)
        super().__init__(params, defaults)
        for g in self.param_groups:
            for p in g["params"]:
                if p.dim() != 2:
                    raise ValueError("Dion3 takes 2-D parameters only; give the others to another optimizer")
        self._orth = {}

    def _orthogonalizer(self, shapes, g):
        from . import Orthogonalizer
        key = (tuple(shapes), g["ns_coeffs"], g["n_iter"], g["restart_every"], g["safety"], g["row_frac"],
               g["restart_threshold"], g["ef"])
        orth = self._orth.get(key)
        if orth is None:
            orth = Orthogonalizer(shapes, "fp32", g["ns_coeffs"], g["n_iter"], g["restart_every"], 0, g["safety"],
                                  g["row_frac"], "mfma16", device="cuda", step_mode=True,
                                  restart_threshold=g["restart_threshold"], ef=g["ef"])
            self._orth[key] = orth
        return orth

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        for g in self.param_groups:
            batches = {}
            for p in g["params"]:
                if p.grad is None:
                    continue
                if not p.is_contiguous() or not p.grad.is_contiguous():
                    raise ValueError("Dion3 needs contiguous parameters and gradients")
                st = self.state[p]
                if "momentum_buffer" not in st:
                    st["momentum_buffer"] = torch.zeros(p.shape, dtype=torch.float32, device=p.device)
                batches.setdefault((p.grad.dtype, p.dtype), []).append(p)
            scale = g["shape_scale"] or (lambda shape: 1.0)
            for ps in batches.values():
                shapes = [tuple(p.shape) for p in ps]
                orth = self._orthogonalizer(shapes, g)
                alphas = [g["lr"] * scale(s) for s in shapes]
                orth.step_update([self.state[p]["momentum_buffer"] for p in ps], [p.grad for p in ps], ps,
                                 g["momentum"], alphas, g["lr"] * g["weight_decay"])
        return loss
