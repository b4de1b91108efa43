"""Helpers for the GPU parity tests (no arithmetic of the scan here)."""
import sys

import numpy as np
import torch

# Tolerances of the normwise max relative error max|g - r| / max|r|:
TOL_F32 = 1e-4      # fp32 activations
TOL_BF16 = 2e-2     # bf16 activations (inputs and stored outputs in bf16)
TOL_STATE = 1e-5    # fp32 state after a long run of decode steps


def f64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, np.float64)


def rel_err(got, ref):
    got, ref = f64(got), f64(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    den = np.abs(ref).max()
    if den == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / den)


def dev(d):
    """Move every tensor of a dict (or a tensor) to the GPU."""
    if isinstance(d, dict):
        return {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    return d.to("cuda")


def announce(*parts):
    """Name the case on stdout before a GPU step, so a fault names it."""
    print("[case]", *parts, flush=True)
    sys.stdout.flush()
