"""Shared helpers for the GPU parity tests (HIP library vs float64 oracle)."""

import numpy as np
import pytest
import torch

DEV = "cuda:0"


def have_gpu():
    return torch.cuda.is_available()


def require_gpu():
    if not have_gpu():
        pytest.skip("no GPU")
    import sparse_attention_long_hca_amd as sa

    sa.lib()  # loud failure if the library is missing
    return sa


def f64(t):
    """Device/host tensor -> float64 numpy (exact upcast of bf16/fp32)."""
    return t.detach().to("cpu", torch.float64).numpy()


def max_abs_err(got, want):
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))))


def rel_err_normwise(got, want):
    want = np.asarray(want, np.float64)
    return max_abs_err(got, want) / max(float(np.max(np.abs(want))), 1e-300)


# Tolerances (stated in the task's parity contract):
#  fp32 configs: normwise relative error <= 1e-5.
#  bf16 configs: max-abs error <= 2e-2 on unit-variance inputs; for the
#  configs' own scaled inputs the bound is scaled by the value std.
F32_REL_TOL = 1e-5
BF16_ABS_TOL = 2e-2
