"""Helpers for the GPU parity tests: input upload, step runners and the
comparison rules.

Comparison rules (tolerances from the layer's numerics contract):
* integer outputs (expert ids, counts, offsets, slots, row sources) and the
  permuted copy x_perm: bit-exact;
* gate logits H: bit-exact (both sides evaluate the same fp32 operations);
* gates: absolute error within 1e-5 (fp32 layers) or 1e-4 (bf16 layers, whose
  certified tokens use gates from the MFMA logits);
* float outputs (FFN rows, y, aux): relative error per tensor
  ||Y - Y_ref||_F / ||Y_ref||_F and per non-zero row ||Y_t - Y_ref_t|| /
  ||Y_ref_t|| within 2e-2 for bf16 and 1e-5 for fp32; rows whose every slot
  was dropped must be exactly zero.
"""

from __future__ import annotations

import sys

import numpy as np

from synthetic import bf16_bits_to_f32

TOL = {"bf16": 2e-2, "f32": 1e-5}
# Gates: fp32 layers (and canonical-logit gates) within 1e-5; bf16 layers take
# the gates of certified tokens from the MFMA logits, which differ from the
# canonical ones at the rounding level (|dH| ~ 1e-5), hence 1e-4.
GATE_ATOL = {"bf16": 1e-4, "f32": 1e-5}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def as_f64(a, dtype):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def rel_rows_ok(got, ref, tol, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    nref = np.linalg.norm(ref)
    if nref > 0:
        rel = np.linalg.norm(got - ref) / nref
        assert rel <= tol, f"{what}: tensor relative error {rel:.3e} > {tol}"
    rn = np.linalg.norm(ref, axis=1)
    dn = np.linalg.norm(got - ref, axis=1)
    nz = rn > 0
    if nz.any():
        worst = (dn[nz] / rn[nz]).max()
        assert worst <= tol, f"{what}: worst row relative error {worst:.3e} > {tol}"
    assert np.all(got[~nz] == 0.0), f"{what}: rows that must be zero are not"


def aux_ok(got, ref, tol, what="aux"):
    got = np.asarray(got, np.float64)[:3]
    ref = np.asarray(ref, np.float64)[:3]
    for i, (g, r) in enumerate(zip(got, ref)):
        if np.isnan(r):
            assert np.isnan(g), f"{what}[{i}]: expected NaN, got {g}"
        elif r == 0:
            assert abs(g) <= tol, f"{what}[{i}]: {g} vs 0"
        else:
            assert abs(g - r) / abs(r) <= tol, f"{what}[{i}]: {g} vs {r} (rel {abs(g - r) / abs(r):.2e})"


def sample_rows(offsets: np.ndarray, n_random: int, seed: int = 0) -> np.ndarray:
    """Rows to check in a large permuted batch: the first and last row of every
    non-empty expert segment (the ragged edges of the GEMM tiles) plus random
    rows."""
    R = int(offsets[-1])
    if R == 0:
        return np.zeros(0, np.int64)
    edges = []
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            edges += [a, b - 1]
    rng = np.random.default_rng(seed)
    rows = np.concatenate([np.array(edges, np.int64), rng.integers(0, R, n_random)])
    return np.unique(rows)


GUARD = 4096
PAT = 0xA5


class Arena:
    """Output buffers as views between guard bands of the byte PAT (GUARD bytes on each
    side, the view 256-byte aligned); check() asserts that no guard byte changed."""

    def __init__(self, dev):
        self.dev = dev
        self.bufs = []

    def alloc(self, shape, dtype, fill=float("nan")):
        import torch

        shape = tuple(int(s) for s in shape)
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        raw = torch.full((n + 2 * GUARD + 256,), PAT, dtype=torch.uint8, device=self.dev)
        off = GUARD + (-(raw.data_ptr() + GUARD)) % 256  # 256-byte aligned view
        view = raw[off:off + n].view(dtype).view(shape)
        if fill is not None and n:
            view.fill_(fill if dtype.is_floating_point else -1)
        self.bufs.append((raw, off, n))
        return view

    def workspace(self, nbytes):
        import torch

        return self.alloc((max(int(nbytes), 1),), torch.uint8, fill=None)

    def check(self, what):
        import torch

        if any(raw.is_cuda for raw, _, _ in self.bufs):
            torch.cuda.synchronize()
        for i, (raw, off, n) in enumerate(self.bufs):
            h = raw.cpu().numpy()
            lo = np.flatnonzero(h[:off] != PAT)
            hi = np.flatnonzero(h[off + n:] != PAT)
            assert lo.size == 0 and hi.size == 0, (
                f"{what}: buffer {i} ({n} bytes): guard bytes changed, {lo.size} before it "
                f"(first at -{off - lo[-1] if lo.size else 0}), {hi.size} after it (first at +{hi[0] if hi.size else 0})")
