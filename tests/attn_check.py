"""The attention parity check (reading C4 of the tolerance "relative 2e-2 for
bf16 inputs, 1e-5 for fp32 inputs"), shared by the GPU parity tests and by the
CPU test that pins its sensitivity.

Per (request, node, q-head) row both must hold:
  * ||o - o_ref||_2 / ||o_ref||_2 <= tol                   (row norm)
  * max_d |o[d] - o_ref[d]| <= tol * max_d |o_ref[d]|       (element-wise)
"""
from __future__ import annotations

import numpy as np

TOL = {"bf16": 2e-2, "f32": 1e-5}


def row_errors(o, ref) -> tuple[np.ndarray, np.ndarray]:
    """Row-norm and element-wise relative errors of rows [..., D] (float64)."""
    o = np.asarray(o, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = o - ref
    den = np.maximum(np.linalg.norm(ref, axis=-1), 1e-300)
    row = np.linalg.norm(diff, axis=-1) / den
    elem = np.abs(diff).max(axis=-1) / np.maximum(np.abs(ref).max(axis=-1), 1e-300)
    return row, elem


def worst_errors(o, ref) -> tuple[float, float]:
    row, elem = row_errors(o, ref)
    return float(row.max(initial=0.0)), float(elem.max(initial=0.0))


def passes(o, ref, tol: float) -> bool:
    row, elem = worst_errors(o, ref)
    return row <= tol and elem <= tol
