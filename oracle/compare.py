"""Acceptance test of a GPU result against the fp64 oracle.

TEST INFRASTRUCTURE (see oracle/layer.py).

A result passes when both hold, element by element and over the whole tensor:
  max |g - o| <= 2e-2 * (1 + |o|)      and      ||g - o||_F / ||o||_F <= 5e-3
for bf16 inputs with fp32 accumulation. The Frobenius bound is the binding one for small-magnitude
tensors (input gradients), where the elementwise bound is loose.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

ELEM_TOL = 2e-2
FRO_TOL = 5e-3


@dataclass
class Verdict:
    name: str
    ok: bool
    max_abs_err: float
    worst_index: tuple
    rel_fro: float
    max_err_over_rms: float
    n_elem_violations: int

    def __str__(self):
        return (f"{self.name}: {'PASS' if self.ok else 'FAIL'} max|g-o|={self.max_abs_err:.3e} "
                f"at {self.worst_index} rel_fro={self.rel_fro:.3e} "
                f"max_err/rms(o)={self.max_err_over_rms:.3e} elem_violations={self.n_elem_violations}")


def compare(g, o, name: str = "out", elem_tol: float = ELEM_TOL, fro_tol: float = FRO_TOL) -> Verdict:
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    if g.shape != o.shape:
        raise ValueError(f"{name}: shape {g.shape} != {o.shape}")
    if g.size == 0:
        return Verdict(name, True, 0.0, (), 0.0, 0.0, 0)
    d = np.abs(g - o)
    finite = bool(np.all(np.isfinite(g)))
    worst = np.unravel_index(int(np.argmax(d)), d.shape) if finite else ()
    viol = int(np.count_nonzero(~(d <= elem_tol * (1.0 + np.abs(o)))))
    no = float(np.linalg.norm(o))
    nd = float(np.linalg.norm(g - o)) if finite else float("inf")
    rel = nd / no if no > 0 else (0.0 if nd == 0 else float("inf"))
    rms = no / np.sqrt(o.size)
    mx = float(d.max()) if finite else float("inf")
    ok = finite and viol == 0 and rel <= fro_tol
    return Verdict(name, ok, mx, tuple(int(i) for i in worst), rel,
                   mx / rms if rms > 0 else (0.0 if mx == 0 else float("inf")), viol)
