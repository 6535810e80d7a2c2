"""Helpers shared by the GPU parity tests: moving stored values between torch
and NumPy without conversion, and the tolerance check against the oracle."""
from __future__ import annotations

import numpy as np
import torch

# Tolerances (decode output vs the unrounded fp64 oracle):
#   fp32 caches: max-abs 1e-5;  bf16 caches: |err| <= 2e-2 + 1e-2 * |ref|.
TOL = {"f32": (1e-5, 0.0), "bf16": (2e-2, 1e-2)}


def stored_np(t: torch.Tensor) -> np.ndarray:
    """The stored values of ``t`` on the host: float32 as is, bfloat16 as its
    16-bit patterns (the oracle widens those exactly)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def out_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def assert_matches_oracle(gpu_out: torch.Tensor, ref: np.ndarray, dtype: str, what: str = "") -> float:
    got = out_f64(gpu_out)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    atol, rtol = TOL[dtype]
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = ~(err <= bound)            # NaN counts as bad
    if bad.any():
        idx = np.argwhere(bad)[:5].tolist()
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outputs outside tolerance "
            f"(atol {atol}, rtol {rtol}); max err {np.nanmax(err):.3e}; first at {idx}: "
            f"got {[got[tuple(i)] for i in idx]} want {[ref[tuple(i)] for i in idx]}")
    return float(err.max()) if err.size else 0.0
