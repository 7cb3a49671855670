"""Helpers shared by the GPU parity tests: device transfer, error metrics,
tolerances.  No arithmetic of the method lives here."""
from __future__ import annotations

import numpy as np
import torch

# Normwise relative error bound per (b, h) slice and per output tensor:
# 1e-4 for fp32 I/O, 2e-2 for bf16 I/O (fp32 state and accumulation).
TOL = {"f32": 1e-4, "bf16": 2e-2}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 array holding exact I/O-dtype values -> contiguous device tensor."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda").to(TORCH_DT[dtype]).contiguous()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def normwise_rel(x: np.ndarray, ref: np.ndarray, lead: int = 2) -> float:
    """max over the leading `lead` axes (the (b, h) slices) of ||x - ref|| / ||ref||."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    n = int(np.prod(ref.shape[:lead]))
    d = np.linalg.norm((x - ref).reshape(n, -1), axis=1)
    r = np.linalg.norm(ref.reshape(n, -1), axis=1)
    return float((d / np.maximum(r, 1e-300)).max())


def floored_rel(x: np.ndarray, ref: np.ndarray) -> float:
    """Elementwise |x - ref| / (|ref| + mean|ref|), max (reported, not gated)."""
    ref = np.asarray(ref, np.float64)
    return float((np.abs(x - ref) / (np.abs(ref) + np.abs(ref).mean())).max())


def check(name: str, x: np.ndarray, ref: np.ndarray, dtype: str, lead: int = 2):
    assert np.isfinite(x).all(), f"{name}: non-finite output"
    e = normwise_rel(x, ref, lead)
    print(f"  {name}: normwise rel err {e:.3e} (tol {TOL[dtype]:.0e}), floored elementwise {floored_rel(x, ref):.3e}",
          flush=True)
    assert e <= TOL[dtype], f"{name}: normwise rel err {e:.3e} > {TOL[dtype]:.0e}"
    return e
