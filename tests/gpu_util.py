"""Helpers for the GPU parity tests: device transfer and the error metric."""
from __future__ import annotations

import sys

import numpy as np
import torch

# Normwise tolerances: max |x - ref| / max |ref| per tensor (fp32 accumulate in both).
TOL = {"fp32": 1e-4, "bf16": 2e-2}


def say(*a):
    """Name the case before a GPU step (flushed, so it survives a lost box)."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def dev_tensor(x: np.ndarray, dtype: str, device="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.to(device)


def host64(t) -> np.ndarray:
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def rel_err(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    return num / max(den, 1e-30)


def assert_close(name, x, ref, tol):
    e = rel_err(x, ref)
    print(f"  {name}: normwise max rel err {e:.3e} (tol {tol:.0e})", flush=True)
    assert np.all(np.isfinite(np.asarray(x, np.float64))), f"{name}: non-finite values"
    assert e <= tol, f"{name}: normwise max rel err {e:.3e} > {tol:.0e}"
