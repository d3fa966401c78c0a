"""Shared pieces of the GPU parity tests: tolerances, device transfer, compare.

Tolerances (the stated accuracy targets of the method on this hardware):
  float32 path:           max |dO| <= 1e-5
  bf16 inputs, fp32 acc:  max |dO| <= 1e-2 and mean |dO| <= 1e-3
  log-sum-exp:            max |dLSE| <= 1e-3 (every dtype)
All differences are against the float64 oracle on the same (bf16-rounded)
inputs; the bf16 output rounding alone is at most half an ulp of |O|.

Gradients (bf16 backward): the absolute bounds above are for O, whose entries
are convex combinations of V rows.  Gradients have no fixed scale (dK and dV
sum over every query row that sees a key), so the same bounds are applied to
each gradient divided by its own scale, max|G_ref| for the maximum error and
mean|G_ref| for the mean:
  max |dG| <= GRAD_MAX_REL * max |G_ref|,  mean |dG| <= GRAD_MEAN_REL * mean |G_ref|.
Where the error comes from: every product on the MFMA takes bf16 operands, so
P (for dV) and dS (for dQ, dK) are rounded to bf16.  bf16 keeps 8 significant
bits, unit roundoff u = 2^-8; over mantissas spread log-uniformly the rounding
error is u/sqrt(3) * 0.74 ~ 1.7e-3 relative (rms) and u/2 * 0.72 ~ 1.4e-3
(mean).  A sum of n such terms of random sign is off by about 1.7e-3 of its
own rms size; the bf16 result then adds its own ~1.4e-3.  Together mean|dG| /
mean|G| ~ sqrt(1.7^2 + 1.4^2) e-3 ~ 2.2e-3 (measured 1.9e-3 to 2.4e-3), and
the largest error, about 4.5 rms of the first term plus one rounding of the
largest entry, ~ 5e-3 of max|G|.  tests/test_grad_tolerance.py checks this
on the CPU, without the kernels: the same formulas in float64 with exactly
those roundings give mean 2.2e-3 to 2.3e-3 and max 2.3e-3 to 5.0e-3 of the
gradients' scale, and the bounds are asserted to sit 1.3x (mean) and 1.5x
(max) or more above that model, and within 2.5x (mean) and 6x (max) of it.
"""
import sys
import zlib

import numpy as np

F32_MAX_O = 1e-5
BF16_MAX_O = 1e-2
BF16_MEAN_O = 1e-3
MAX_LSE = 1e-3
GRAD_MAX_REL = 1e-2
GRAD_MEAN_REL = 3.5e-3
GRAD_ZERO_ABS = 1e-4


def seed_of(name: str) -> int:
    return zlib.crc32(name.encode()) & 0x7FFFFFFF


def announce(msg: str) -> None:
    """Name the case on stdout before a GPU step (visible if the step dies)."""
    print(f"\n[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_np(t) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def check_o(o_gpu: np.ndarray, o_ref: np.ndarray, dtype: str, what: str = ""):
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    err = np.abs(o_gpu - o_ref)
    mx, mean = float(err.max()), float(err.mean())
    if dtype == "f32":
        assert mx <= F32_MAX_O, f"{what}: max|dO| {mx:.3g} > {F32_MAX_O}"
    else:
        assert mx <= BF16_MAX_O, f"{what}: max|dO| {mx:.3g} > {BF16_MAX_O}"
        assert mean <= BF16_MEAN_O, f"{what}: mean|dO| {mean:.3g} > {BF16_MEAN_O}"
    return mx, mean


def check_lse(lse_gpu: np.ndarray, lse_ref: np.ndarray, what: str = ""):
    assert np.all(np.isfinite(lse_gpu)), f"{what}: non-finite LSE"
    mx = float(np.abs(lse_gpu - lse_ref).max())
    assert mx <= MAX_LSE, f"{what}: max|dLSE| {mx:.3g} > {MAX_LSE}"
    return mx


def check_grad(g_gpu: np.ndarray, g_ref: np.ndarray, what: str = ""):
    """Gradient error relative to the gradient's own scale (see the module docstring)."""
    assert np.all(np.isfinite(g_gpu)), f"{what}: non-finite gradient"
    err = np.abs(g_gpu - g_ref)
    scale_max, scale_mean = float(np.abs(g_ref).max()), float(np.abs(g_ref).mean())
    if scale_max < 1e-12:
        # an exactly vanishing gradient (one visible key: dS = P (dP - D) = 0) is
        # reached on the GPU up to fp32 rounding of dP - D, two sums of the same
        # products taken in different orders
        assert float(err.max()) <= GRAD_ZERO_ABS, f"{what}: |G| {err.max():.3g} where 0 is exact"
        return float(err.max()), float(err.mean())
    rmax, rmean = float(err.max()) / scale_max, float(err.mean()) / scale_mean
    assert rmax <= GRAD_MAX_REL, f"{what}: max|dG|/max|G| {rmax:.3g} > {GRAD_MAX_REL}"
    assert rmean <= GRAD_MEAN_REL, f"{what}: mean|dG|/mean|G| {rmean:.3g} > {GRAD_MEAN_REL}"
    return rmax, rmean
