"""Helpers shared by the GPU parity tests: device transfer, error metrics,
tolerances.  No arithmetic of the method lives here.

The gate (``check``) bounds two normwise relative errors by the same
tolerance (1e-4 for fp32 I/O, 2e-2 for bf16 I/O):
  * per (b, h) slice: ||x - ref|| / ||ref|| over the whole slice;
  * per chunk: ||x_c - ref_c|| / ||ref_c|| over every run of 16 consecutive
    rows (tokens) of every slice, so that rows of small norm (outputs shrink
    like 1/sqrt(i) along the sequence) are gated as strictly as the large
    early ones.  Gradients whose rows can cancel to nearly zero (dQ, dK) take
    ``floor=True``: a chunk's denominator is then at least sqrt(rows) times
    FLOOR_FRAC of the slice's mean row norm.  The fraction is small on
    purpose: on the seeded long-sequence inputs the rows of dQ, dK and dV are
    largest at the start of the sequence (tens of times the mean) and the last
    chunks of dK and dV sit near 1/64 of it, so a floor at the mean itself
    would hide errors in exactly the late rows the gate is meant to see; 1/64
    only binds where a chunk really cancels (dQ of a first token is exactly 0).
"""
from __future__ import annotations

import numpy as np

try:   # the metrics below are plain numpy; torch is needed only for device transfer
    import torch
except ImportError:   # pragma: no cover
    torch = None

# Normwise relative error bound per (b, h) slice, per 16-row chunk and per
# output tensor: 1e-4 for fp32 I/O, 2e-2 for bf16 I/O (fp32 state and
# accumulation).
TOL = {"f32": 1e-4, "bf16": 2e-2}
CHUNK = 16
FLOOR_FRAC = 1.0 / 64.0


def _torch_dt(dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def dev(x: np.ndarray, dtype: str):
    """float32 array holding exact I/O-dtype values -> contiguous device tensor."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda").to(_torch_dt(dtype)).contiguous()


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def normwise_rel(x: np.ndarray, ref: np.ndarray, lead: int = 2) -> float:
    """max over the leading `lead` axes (the (b, h) slices) of ||x - ref|| / ||ref||."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    n = int(np.prod(ref.shape[:lead]))
    d = np.linalg.norm((x - ref).reshape(n, -1), axis=1)
    r = np.linalg.norm(ref.reshape(n, -1), axis=1)
    return float((d / np.maximum(r, 1e-300)).max())


def chunk_rel(x: np.ndarray, ref: np.ndarray, lead: int = 2, chunk: int = CHUNK, floor: bool = False):
    """Worst normwise relative error over every run of `chunk` consecutive rows
    (axis `lead`, the tokens) of every slice (the leading `lead` axes), and
    where it is: returns (error, slice index, first row).  With `floor` a
    chunk's denominator is at least sqrt(rows in it) times FLOOR_FRAC of the
    slice's mean row norm."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    n = int(np.prod(ref.shape[:lead]))
    rows = ref.shape[lead] if ref.ndim > lead else 1
    d2 = ((x - ref) ** 2).reshape(n, rows, -1).sum(2)
    r2 = (ref ** 2).reshape(n, rows, -1).sum(2)
    nc = -(-rows // chunk)
    pad = nc * chunk - rows
    cnt = np.full(nc, chunk, np.float64)
    cnt[-1] = chunk - pad
    if pad:
        d2 = np.pad(d2, ((0, 0), (0, pad)))
        r2 = np.pad(r2, ((0, 0), (0, pad)))
    dc = np.sqrt(d2.reshape(n, nc, chunk).sum(2))
    rc = np.sqrt(r2.reshape(n, nc, chunk).sum(2))
    if floor:
        mean_row = FLOOR_FRAC * np.sqrt(r2).sum(1, keepdims=True) / rows
        rc = np.maximum(rc, np.sqrt(cnt)[None, :] * mean_row)
    e = np.where(dc == 0, 0.0, dc / np.maximum(rc, 1e-300))
    i = int(np.argmax(e))
    return float(e.flat[i]), i // nc, (i % nc) * chunk


def floored_rel(x: np.ndarray, ref: np.ndarray) -> float:
    """Elementwise |x - ref| / (|ref| + mean|ref|), max (reported, not gated)."""
    ref = np.asarray(ref, np.float64)
    return float((np.abs(x - ref) / (np.abs(ref) + np.abs(ref).mean())).max())


def check(name: str, x: np.ndarray, ref: np.ndarray, dtype: str, lead: int = 2, floor: bool = False):
    """Gate x against ref: slice and 16-row-chunk normwise errors both <= TOL[dtype]
    (the chunks when the slices have rows, i.e. ref has two axes after `lead`)."""
    assert np.isfinite(x).all(), f"{name}: non-finite output"
    tol = TOL[dtype]
    e = normwise_rel(x, ref, lead)
    if np.ndim(ref) < lead + 2:   # no row axis below the slices (a slice is one row or a vector)
        print(f"  {name}: normwise rel err {e:.3e} per {'row' if np.ndim(ref) == lead + 1 else 'slice'} "
              f"(tol {tol:.0e}), floored elementwise {floored_rel(x, ref):.3e}", flush=True)
        assert e <= tol, f"{name}: normwise rel err {e:.3e} > {tol:.0e}"
        return e
    ec, sl, row = chunk_rel(x, ref, lead, floor=floor)
    print(f"  {name}: normwise rel err {e:.3e}, worst {CHUNK}-row chunk {ec:.3e} (slice {sl}, row {row})"
          f"{' floored' if floor else ''} (tol {tol:.0e}), floored elementwise {floored_rel(x, ref):.3e}", flush=True)
    assert e <= tol, f"{name}: normwise rel err {e:.3e} > {tol:.0e}"
    assert ec <= tol, f"{name}: rows {row}..{row + CHUNK - 1} of slice {sl}: chunk rel err {ec:.3e} > {tol:.0e}"
    return max(e, ec)
