"""Shared helpers for the GPU parity tests (HIP path vs. the float64 oracle).

Tolerances (max-abs for outputs, relative Frobenius norm for gradients):
  * O and lse, bf16: 1e-2; fp16: 2e-3 (the stated bounds; lse takes the bound
    of O for its dtype).
  * dQ, dK, dV, bf16: ||g - g_ref|| / ||g_ref|| <= 5e-2 per tensor; fp16:
    1e-2 (fp16 carries three more mantissa bits than bf16, so the same
    arithmetic gives an error about 8x smaller; 1e-2 keeps a 1.6x margin).
    A gradient that is exactly zero in exact arithmetic (a single key: every
    row of dS = P o (dP - D) cancels) has no relative scale, so the check is
    ||g - g_ref|| <= tol ||g_ref|| + GRAD_ATOL_RMS sqrt(numel): fp32 rounding
    of the cancelling terms is about 1e-7 per element.
Each failure message also reports the storage-type rounding floor
max|round(ref) - ref|, the error a perfectly rounded result would have.
check_rel_norm_blocks applies the gradient bound to every block of 32 rows
separately (one row block of a wave), so that a wrong row or block, which
barely moves a whole-tensor norm, still fails.
"""
import sys

import numpy as np
import torch

TOL_O = {torch.bfloat16: 1e-2, torch.float16: 2e-3}
TOL_GRAD = {torch.bfloat16: 5e-2, torch.float16: 1e-2}
GRAD_ATOL_RMS = 1e-5


def announce(msg: str) -> None:
    """Name the case on the real stderr (not captured), flushed before GPU work."""
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def rounding_floor(ref: np.ndarray, dtype: torch.dtype) -> float:
    r = torch.from_numpy(np.ascontiguousarray(ref)).to(dtype).to(torch.float64).numpy()
    return float(np.max(np.abs(r - ref))) if ref.size else 0.0


def check_max_abs(got: np.ndarray, ref: np.ndarray, dtype, what: str, tol=None) -> float:
    tol = TOL_O[dtype] if tol is None else tol
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values (unwritten or overflow)"
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert err <= tol, (f"{what}: max-abs error {err:.4e} > {tol:.1e} "
                        f"(rounding floor {rounding_floor(ref, dtype):.4e})")
    return err


def check_rel_norm(got: np.ndarray, ref: np.ndarray, dtype, what: str) -> float:
    tol = TOL_GRAD[dtype]
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    den = float(np.linalg.norm(ref))
    diff = float(np.linalg.norm(got - ref))
    err = diff / max(den, 1e-30)
    assert diff <= tol * den + GRAD_ATOL_RMS * np.sqrt(ref.size), (
        f"{what}: relative norm error {err:.4e} > {tol:.1e} (||ref|| = {den:.3e})")
    return err


def nan_like(t: torch.Tensor) -> torch.Tensor:
    return torch.full_like(t, float("nan"))


def check_rel_norm_blocks(got: np.ndarray, ref: np.ndarray, dtype, what: str,
                          rows: int = 32) -> float:
    """The gradient bound of check_rel_norm on every block of `rows` rows (axis -2)."""
    tol = TOL_GRAD[dtype]
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    n = ref.shape[-2]
    worst = 0.0
    for r0 in range(0, n, rows):
        g, r = got[..., r0:r0 + rows, :], ref[..., r0:r0 + rows, :]
        den = float(np.linalg.norm(r))
        diff = float(np.linalg.norm(g - r))
        assert diff <= tol * den + GRAD_ATOL_RMS * np.sqrt(r.size), (
            f"{what}: rows {r0}..{r0 + r.shape[-2] - 1}: relative norm error "
            f"{diff / max(den, 1e-30):.4e} > {tol:.1e} (||ref|| = {den:.3e})")
        worst = max(worst, diff / max(den, 1e-30))
    return worst
