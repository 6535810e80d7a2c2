"""Helpers shared by the GPU parity tests: moving stored values between torch
and NumPy without conversion, running the oracle over every sequence of a
batch, and the tolerance check against the oracle."""
from __future__ import annotations

import numpy as np
import torch

from synth import stored_np  # noqa: F401  (re-exported for the tests)

# Tolerances (decode output vs the unrounded fp64 oracle):
#   fp32 caches: max-abs 1e-5;  bf16 caches: |err| <= 2e-2 + 1e-2 * |ref|.
TOL = {"f32": (1e-5, 0.0), "bf16": (2e-2, 1e-2)}


def oracle_per_sequence(fn, B: int, threads: int = 0):
    """Stack fn(b0, b1) -> rows of sequences b0 .. b1-1 over every sequence,
    the blocks of sequences spread over host threads (NumPy releases the GIL
    inside its kernels).  fn calls an oracle function on that slice of the
    batch; sequences are independent in the definition, so the stacked result
    is the oracle's on the whole batch."""
    import concurrent.futures as cf
    import os

    threads = threads or max(1, min(8, len(os.sched_getaffinity(0)), B))
    step = max(1, -(-B // (4 * threads)))
    spans = [(b, min(B, b + step)) for b in range(0, B, step)]
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        parts = list(ex.map(lambda s: fn(*s), spans))
    return np.concatenate(parts, axis=0)


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
