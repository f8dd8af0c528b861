"""Out-of-bounds writes: every path runs with guard bands of a known byte
pattern around its workspace (the library may write only the first
workspace_size bytes) and around each output matrix; the bands must come back
untouched."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

PAT = 0xA5
GUARD = 1 << 20


@pytest.fixture(scope="module")
def dion():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import orthogonalized_optimizer_step_amd as d
    return d


class Guarded:
    """A device byte buffer of `nbytes` (256-byte aligned) between two guard bands."""

    def __init__(self, nbytes):
        self.raw = torch.full((nbytes + 2 * GUARD + 256,), PAT, dtype=torch.uint8, device="cuda")
        base = self.raw.data_ptr()
        self.off = GUARD + (-(base + GUARD)) % 256
        self.n = nbytes
        self.ptr = base + self.off

    def intact(self):
        torch.cuda.synchronize()
        head = self.raw[: self.off]
        tail = self.raw[self.off + self.n:]
        return bool((head == PAT).all()) and bool((tail == PAT).all())


def guarded_like(shape, dtype):
    """An output tensor inside a guarded allocation, and its guard."""
    es = torch.tensor([], dtype=dtype).element_size()
    n = int(np.prod(shape)) * es
    g = Guarded(n)
    t = g.raw[g.off:g.off + n].view(dtype).view(shape)
    return t, g


def use_workspace(orth, g):
    orth._ws_tensor, orth._ws, orth._ws_len = g.raw, g.ptr, g.n + GUARD   # length past the plan: writes there are bugs


def rand(shape, dtype, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    return torch.randn(shape, generator=gen, device="cuda").to(dtype)


@pytest.mark.parametrize("case", ["mfma16", "mfma16_rows", "fp64", "tiny"])
def test_orth_paths_write_in_bounds(dion, case):
    shapes = {"mfma16": [(300, 520), (520, 300), (700, 700)],
              "mfma16_rows": [(512, 384), (384, 900), (1000, 260)],
              "fp64": [(130, 250), (250, 130), (96, 96)],
              "tiny": [(64, 128), (128, 64), (5, 1000)]}[case]
    dt = torch.float32 if case in ("fp64", "tiny") else torch.bfloat16
    frac = 0.5 if case == "mfma16_rows" else 1.0
    orth = dion.Orthogonalizer(shapes, "fp32" if dt == torch.float32 else "bf16", n_iter=5, restart_every=2,
                               row_frac=frac)
    g = Guarded(orth.ws_bytes)
    use_workspace(orth, g)
    Ms = [rand(s, dt, i) for i, s in enumerate(shapes)]
    outs, guards = zip(*[guarded_like(s, dt) for s in shapes])
    orth(Ms, list(outs))
    assert g.intact(), "workspace guard overwritten"
    for s, og in zip(shapes, guards):
        assert og.intact(), f"output guard of {s} overwritten"


@pytest.mark.parametrize("update", [False, True])
def test_rowsubset_step_writes_in_bounds(dion, update):
    shapes = [(256, 200), (200, 520), (640, 128)]
    orth = dion.Orthogonalizer(shapes, "fp32", n_iter=5, restart_every=2, row_frac=0.25, precision="mfma16",
                               step_mode=True)
    g = Guarded(orth.ws_bytes)
    use_workspace(orth, g)
    Es, eg = zip(*[guarded_like(s, torch.float32) for s in shapes])
    for e in Es:
        e.zero_()
    grads = [rand(s, torch.bfloat16, 10 + i) for i, s in enumerate(shapes)]
    if update:
        Ws, wg = zip(*[guarded_like(s, torch.bfloat16) for s in shapes])
        for w, s in zip(Ws, shapes):
            w.copy_(rand(s, torch.bfloat16, 20) * 0.02)
        orth.step_update(list(Es), grads, list(Ws), 0.95, [0.02] * len(shapes), 0.01)
        others = wg
    else:
        outs, og = zip(*[guarded_like(s, torch.bfloat16) for s in shapes])
        orth.step(list(Es), grads, list(outs), 0.95)
        others = og
    assert g.intact(), "workspace guard overwritten"
    for x in list(eg) + list(others):
        assert x.intact(), "buffer guard overwritten"


@pytest.mark.parametrize("mode", ["qr", "colnorm"])
def test_lowrank_step_writes_in_bounds(dion, mode):
    shapes = [(300, 200), (200, 300), (520, 520)]
    rank = 24
    need = dion.lowrank_workspace_size(shapes, rank)
    g = Guarded(need)
    ws = g.raw[g.off:g.off + need + GUARD]   # the library may use only the first `need` bytes
    Ms, mg = zip(*[guarded_like(s, torch.float32) for s in shapes])
    for m in Ms:
        m.zero_()
    Qs, qg = zip(*[guarded_like((s[1], min(rank, *s)), torch.float32) for s in shapes])
    for i, q in enumerate(Qs):
        q.copy_(rand(q.shape, torch.float32, 30 + i))
    outs, og = zip(*[guarded_like(s, torch.bfloat16) for s in shapes])
    grads = [rand(s, torch.bfloat16, 40 + i) for i, s in enumerate(shapes)]
    dion.lowrank_step(list(Ms), grads, list(Qs), 0.5, mode=mode, outs=list(outs), workspace=ws)
    assert g.intact(), "workspace guard overwritten"
    for x in list(mg) + list(qg) + list(og):
        assert x.intact(), "buffer guard overwritten"
