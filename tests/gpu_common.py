"""Shared helpers for the GPU parity tests (comparison metrics and tolerances)."""
from __future__ import annotations

import sys

import numpy as np
import torch

# Tolerances against the fp64 oracle: bf16 inputs with fp32 accumulation, and fp32 inputs.
BF16_REL_L2 = 2e-3
BF16_MAX_ABS = 1e-2
F32_REL_L2 = 1e-5


def metrics(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in the GPU output"
    err = got - ref
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))
    return rel, float(np.abs(err).max()) if err.size else 0.0


def assert_close(got, ref, dtype: str, label: str = ""):
    rel, mx = metrics(got, ref)
    print(f"[parity] {label} rel_l2={rel:.3e} max_abs={mx:.3e}", flush=True)
    if dtype == "bf16":
        assert rel <= BF16_REL_L2 and mx <= BF16_MAX_ABS, f"{label}: rel_l2={rel:.3e} max_abs={mx:.3e}"
    else:
        assert rel <= F32_REL_L2, f"{label}: rel_l2={rel:.3e}"
    return rel, mx


def announce(msg: str):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def gpu_available() -> bool:
    return torch.cuda.is_available()
