"""Shared helpers of the GPU parity tests: conversions and the tolerance rule."""

from __future__ import annotations

import os

import numpy as np
import torch

BF16_TOL = 2e-2
F32_TOL = 1e-4
TIE = 1e-6          # oracle logit gap below which an integer decision is a near-tie


def host(t: torch.Tensor) -> np.ndarray:
    """Host copy for the oracle: bf16 -> uint16 bit patterns, others as they are."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def tol_for(t: torch.Tensor) -> float:
    return BF16_TOL if t.dtype == torch.bfloat16 else F32_TOL


# (test, what, elementwise error, max|d| / max|ref|, tolerance) of every float
# comparison, printed at the end of the run so that the headroom under each
# tolerance is visible, not only pass / fail
ACHIEVED: list = []


def assert_close(got, ref, tol, what=""):
    """max|d|/max(1,|ref|) <= tol elementwise, and max|d| <= tol * max|ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if ref.size == 0:
        return
    d = np.abs(got - ref)
    rel = (d / np.maximum(1.0, np.abs(ref))).max()
    scale0 = np.abs(ref).max()
    ACHIEVED.append((os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], what, float(rel),
                     float(d.max() / scale0) if scale0 > 0 else 0.0, tol))
    assert rel <= tol, f"{what}: max|d|/max(1,|ref|) = {rel:.3e} > {tol:.1e}"
    scale = np.abs(ref).max()
    assert d.max() <= tol * max(scale, 1e-30), f"{what}: max|d| = {d.max():.3e} > {tol:.1e} * max|ref| ({scale:.3e})"


def compare_ids(got, ref, gaps, what=""):
    """Bit-exact integer decisions, except rows whose oracle gap is a near-tie.
    Returns (number of flagged rows, boolean mask of flagged rows)."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    gaps = np.asarray(gaps)
    flagged = gaps < TIE
    rows_diff = (got != ref).reshape(got.shape[0], -1).any(axis=1)
    bad = rows_diff & ~flagged
    assert not bad.any(), f"{what}: {bad.sum()} rows differ without a near-tie, first at {np.nonzero(bad)[0][:5]}"
    return int(flagged.sum()), flagged
