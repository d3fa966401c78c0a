"""Shared pieces of the GPU parity tests: tolerances, device transfer, compare.

Tolerances (the stated accuracy targets of the method on this hardware):
  float32 path:           max |dO| <= 1e-5
  bf16 inputs, fp32 acc:  max |dO| <= 1e-2 and mean |dO| <= 1e-3
  log-sum-exp:            max |dLSE| <= 1e-3 (every dtype)
All differences are against the float64 oracle on the same (bf16-rounded)
inputs; the bf16 output rounding alone is at most half an ulp of |O|.
"""
import sys
import zlib

import numpy as np

F32_MAX_O = 1e-5
BF16_MAX_O = 1e-2
BF16_MEAN_O = 1e-3
MAX_LSE = 1e-3


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
