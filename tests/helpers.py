"""Shared helpers of the GPU parity tests: marshal tensors to the oracle and
compare results element by element."""
from __future__ import annotations

import numpy as np

# Tolerances against the unrounded fp64 oracle.
BF16_MAX_ABS = 2e-2      # bf16 output: max |O_gpu - O_ref|
BF16_MEAN_ABS = 2e-3     # bf16 output: mean |O_gpu - O_ref|
BF16_LSE_ABS = 1e-4      # fp32 lse from bf16 inputs
F32_MAX_ABS = 1e-5       # fp32 path, output and lse


def to_np(t):
    import torch
    return t.detach().to("cpu", torch.float32).numpy()


def report(name, got, ref):
    err = np.abs(got.astype(np.float64) - ref)
    idx = np.unravel_index(int(np.argmax(err)), err.shape) if err.size else ()
    return (f"{name}: max_abs={err.max() if err.size else 0:.3e} at {idx} "
            f"(got {got[idx] if err.size else None}, ref {ref[idx] if err.size else None}), "
            f"mean_abs={err.mean() if err.size else 0:.3e}")


def check_o(got, ref, max_abs, mean_abs=None, name="O"):
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all() == np.isfinite(ref).all(), name + ": non-finite values differ"
    err = np.abs(got - ref)
    msg = report(name, got, ref)
    print(msg)
    assert err.max(initial=0.0) <= max_abs, msg
    if mean_abs is not None and err.size:
        assert err.mean() <= mean_abs, msg


def check_lse(got, ref, max_abs, name="lse"):
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), name + ": -inf pattern differs"
    assert np.all(got[~fin] == ref[~fin])
    if fin.any():
        err = np.abs(got[fin] - ref[fin])
        msg = report(name, got[fin], ref[fin])
        print(msg)
        assert err.max() <= max_abs, msg
