"""Helpers of the GPU parity tests: tolerances, the normwise error metric and the
near-tie exclusion rule. Host-side only; compares HIP outputs with oracle values
computed from the same seeded inputs.

Tolerances. Layer outputs: per-token normwise relative error
max_t ||y_t - y*_t||_inf / ||y*_t||_inf <= 2e-2 (bf16 path) or 1e-4 (fp32 path).
Tokens whose routing is within a probability margin of 1e-5 of another selection
(the oracle computes the margin) are near ties: without capacity they alone are left
out of the selection and output comparisons (their GPU selection is checked to be a
valid one, and dispatch is compared on the GPU's own selection); with capacity the
oracle routes from the GPU's fp32 logits and nothing is left out.
"""
from __future__ import annotations

import numpy as np
import torch

TOL_Y = {"bf16": 2e-2, "f32": 1e-4}
MARGIN = 1e-5


def host(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            t = t.float()
        return t.numpy()
    return np.asarray(t)


def normwise_err(y, ref) -> np.ndarray:
    """Per-row ||y - ref||_inf / ||ref||_inf (rows with ref = 0 give |y|_inf)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(y - ref), axis=1)
    den = np.max(np.abs(ref), axis=1)
    out = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return out


def assert_rows_close(y, ref, tol, what="rows"):
    err = normwise_err(y, ref)
    worst = int(np.argmax(err)) if err.size else -1
    assert err.size == 0 or err.max() <= tol, f"{what}: max normwise error {err.max():.3e} at row {worst} > {tol}"
    return float(err.max()) if err.size else 0.0


def ambiguous_tokens(routing) -> np.ndarray:
    return np.nonzero(routing.margin < MARGIN)[0]
