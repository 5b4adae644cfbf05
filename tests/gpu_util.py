"""Helpers for the GPU parity tests (imported by tests only)."""
from __future__ import annotations

import sys

import numpy as np
import torch

# Tolerances: |gpu - oracle| <= TOL * (1 + |oracle|) elementwise, i.e. atol = rtol.
# 1e-3 for float32 I/O and 2e-2 for float16 / bfloat16 I/O, with float32
# arithmetic in the kernels and float64 in the oracle.
TOL = {torch.float32: 1e-3, torch.float16: 2e-2, torch.bfloat16: 2e-2}


def note(msg: str) -> None:
    """Name the case on stderr before it touches the GPU."""
    sys.stderr.write("[gpu case] %s\n" % msg)
    sys.stderr.flush()


def dev() -> torch.device:
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X")
    return torch.device("cuda", 0)


def to_dev(d: dict) -> dict:
    return {k: (v.to(dev()) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def assert_close(got, ref: np.ndarray, io_dtype, what: str, where=None) -> float:
    """Elementwise |got - ref| <= tol * (1 + |ref|); NaN positions must agree.
    ``where`` restricts the comparison to a boolean mask.  Returns the largest
    scaled error seen."""
    g = f64(got) if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    if where is not None:
        g, r = g[where], r[where]
    assert np.array_equal(np.isnan(g), np.isnan(r)), what + ": NaN positions differ"
    ok = ~np.isnan(r)
    tol = TOL[io_dtype]
    err = np.abs(g[ok] - r[ok]) / (1.0 + np.abs(r[ok]))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, "%s: worst scaled error %.3e > %.1e" % (what, worst, tol)
    return worst


def step_mask(mask, B: int, T: int) -> np.ndarray:
    """Boolean [B, T] of active steps (all True for a NULL mask)."""
    if mask is None:
        return np.ones((B, T), dtype=bool)
    return mask.cpu().numpy() > 0
