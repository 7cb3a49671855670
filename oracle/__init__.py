"""fp64 CPU oracle for kernelized causal linear attention.

TEST INFRASTRUCTURE ONLY.  The only code allowed to import this package is
the test suite (``tests/``), the smoke check in ``__graft_entry__.smoke`` and
the CPU-baseline leg of ``bench.py``.  The HIP library and its Python binding
never import, link or call anything here, and this package never imports them.

The arithmetic lives in ``la_oracle.c`` (plain C, double precision, the
literal per-token recurrence, no fast-math, no FMA contraction).  This module
only compiles it with gcc and marshals numpy arrays through ctypes.

Pins: every routine is checked by ``tests/test_oracle_pins.py`` against an
independent quadratic brute force, exact rational arithmetic on tiny inputs,
closed forms, invariants, central finite differences and torch fp64 autograd.
No routine here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c11"]


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the C oracle with gcc into a shared library; returns its path."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *_CFLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def _bind(lib):
    d = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_feature_map.argtypes = [d, d, d, i64]
    lib.orc_forward_causal.argtypes = [d, d, d, d, d, d, d, i64, i64, i64, i64, i64]
    lib.orc_forward_noncausal.argtypes = [d, d, d, d, i64, i64, i64, i64, i64]
    lib.orc_backward_causal.argtypes = [d, d, d, d, d, d, d, i64, i64, i64, i64, i64]
    lib.orc_backward_noncausal.argtypes = [d, d, d, d, d, d, d, i64, i64, i64, i64, i64]
    lib.orc_decode_step.argtypes = [d, d, d, d, d, d, i64, i64, i64, i64]
    lib.orc_rff_features.argtypes = [d, d, d, d, i64, i64, i64]
    lib.orc_forward_causal_features.argtypes = [d, d, d, d, i64, i64, i64, i64, i64]
    lib.orc_forward_causal_poly2.argtypes = [d, d, d, d, i64, i64, i64, i64, i64]
    lib.orc_forward_noncausal_poly2.argtypes = [d, d, d, d, i64, i64, i64, i64, i64]
    lib.orc_forward_poly2_rows.argtypes = [d, d, d, ctypes.POINTER(i64), d, i64, i64, i64, i64, i64, i64, i64]
    lib.orc_backward_causal_poly2.argtypes = [d, d, d, d, d, d, d, i64, i64, i64, i64, i64]
    lib.orc_backward_causal_poly2_rows.argtypes = [d, d, d, d, ctypes.POINTER(i64), i64, ctypes.POINTER(i64), i64,
                                                   d, d, d, i64, i64, i64, i64, i64]
    for f in ("orc_feature_map", "orc_forward_causal", "orc_forward_noncausal",
              "orc_backward_causal", "orc_backward_noncausal", "orc_decode_step", "orc_rff_features",
              "orc_forward_causal_features", "orc_forward_causal_poly2", "orc_forward_noncausal_poly2", "orc_forward_poly2_rows",
              "orc_backward_causal_poly2", "orc_backward_causal_poly2_rows"):
        getattr(lib, f).restype = None
    return lib


def load(path: str | None = None):
    """Load (building first if needed) the oracle library.  A non-default
    ``path`` loads another build of an oracle source, which the tests use to
    check that planted mistakes are caught by the pins."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads(lib=None) -> int:
    return int((lib or load()).orc_num_threads())


def feature_map(x, lib=None):
    """phi(x) = elu(x)+1 and phi'(x), elementwise, in fp64."""
    lib = lib or load()
    x = _f64(x)
    y = np.empty_like(x)
    dy = np.empty_like(x)
    lib.orc_feature_map(_p(x), _p(y), _p(dy), x.size)
    return y, dy


def forward_causal(q, k, v, S0=None, Z0=None, return_state=False, return_den=False, lib=None):
    """Causal linear attention, literal recurrence.  q,k: [B,H,N,D]; v: [B,H,N,M].

    ``S0`` [B,H,D,M] / ``Z0`` [B,H,D] give an optional starting state.  With
    ``return_state`` the final (S_N, Z_N) are returned too; with ``return_den``
    the per-token denominators [B,H,N]."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    M = v.shape[-1]
    assert k.shape == q.shape and v.shape == (B, H, N, M)
    out = np.empty((B, H, N, M), np.float64)
    want_state = return_state or S0 is not None or Z0 is not None
    S = _f64(S0).copy() if S0 is not None else (np.zeros((B, H, D, M)) if want_state else None)
    Z = _f64(Z0).copy() if Z0 is not None else (np.zeros((B, H, D)) if want_state else None)
    den = np.empty((B, H, N), np.float64) if return_den else None
    lib.orc_forward_causal(_p(q), _p(k), _p(v), _p(out), _p(S), _p(Z), _p(den), B, H, N, D, M)
    res = [out]
    if return_state:
        res += [S, Z]
    if return_den:
        res.append(den)
    return res[0] if len(res) == 1 else tuple(res)


def forward_noncausal(q, k, v, lib=None):
    """Non-causal linear attention through the global (S, Z)."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    M = v.shape[-1]
    out = np.empty((B, H, N, M), np.float64)
    lib.orc_forward_noncausal(_p(q), _p(k), _p(v), _p(out), B, H, N, D, M)
    return out


def backward_causal(q, k, v, dout, lib=None):
    """Gradients (dQ, dK, dV) of sum(dout * forward_causal(q,k,v)) w.r.t. raw q,k,v."""
    lib = lib or load()
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, D = q.shape
    M = v.shape[-1]
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    lib.orc_backward_causal(_p(q), _p(k), _p(v), _p(g), _p(dq), _p(dk), _p(dv), B, H, N, D, M)
    return dq, dk, dv


def backward_noncausal(q, k, v, dout, lib=None):
    """Gradients (dQ, dK, dV) of sum(dout * forward_noncausal(q,k,v)) w.r.t. raw q,k,v."""
    lib = lib or load()
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, D = q.shape
    M = v.shape[-1]
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    lib.orc_backward_noncausal(_p(q), _p(k), _p(v), _p(g), _p(dq), _p(dk), _p(dv), B, H, N, D, M)
    return dq, dk, dv


def rff_features(x, omega, b, lib=None):
    """Random Fourier features sqrt(2/R) cos(x omega + b) of the last axis of x
    ([..., D] -> [..., R]); omega [D, R], b [R]."""
    lib = lib or load()
    x, omega, b = _f64(x), _f64(omega), _f64(b)
    D, R = omega.shape
    assert x.shape[-1] == D and b.shape == (R,)
    out = np.empty(x.shape[:-1] + (R,), np.float64)
    lib.orc_rff_features(_p(x), _p(omega), _p(b), _p(out), int(np.prod(x.shape[:-1])), D, R)
    return out


def forward_causal_features(fq, fk, v, lib=None):
    """Causal linear attention on given features fq, fk [B,H,N,F] (no feature map applied)."""
    lib = lib or load()
    fq, fk, v = _f64(fq), _f64(fk), _f64(v)
    B, H, N, F = fq.shape
    M = v.shape[-1]
    assert fk.shape == fq.shape and v.shape == (B, H, N, M)
    out = np.empty((B, H, N, M), np.float64)
    lib.orc_forward_causal_features(_p(fq), _p(fk), _p(v), _p(out), B, H, N, F, M)
    return out


def forward_causal_poly2(q, k, v, lib=None):
    """Causal linear attention with the degree-2 polynomial kernel (q . k)^2,
    through its explicit D^2 feature map.  q,k: [B,H,N,D]; v: [B,H,N,M]."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    M = v.shape[-1]
    assert k.shape == q.shape and v.shape == (B, H, N, M)
    out = np.empty((B, H, N, M), np.float64)
    lib.orc_forward_causal_poly2(_p(q), _p(k), _p(v), _p(out), B, H, N, D, M)
    return out


def backward_causal_poly2(q, k, v, dout, lib=None):
    """Gradients (dQ, dK, dV) of sum(dout * forward_causal_poly2(q,k,v)) w.r.t.
    q, k, v, summed pair by pair (O(N^2) per head)."""
    lib = lib or load()
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, D = q.shape
    M = v.shape[-1]
    assert k.shape == q.shape and v.shape == (B, H, N, M) and g.shape == v.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    lib.orc_backward_causal_poly2(_p(q), _p(k), _p(v), _p(g), _p(dq), _p(dk), _p(dv), B, H, N, D, M)
    return dq, dk, dv


def backward_causal_poly2_rows(q, k, v, dout, rows_q, rows_k, lib=None):
    """Rows of backward_causal_poly2, each summed pair by pair: dq at rows_q,
    dk and dv at rows_k (which should lie near the end: every later token's
    out and d are formed first)."""
    lib = lib or load()
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, D = q.shape
    M = v.shape[-1]
    rq = np.ascontiguousarray(rows_q, np.int64)
    rk = np.ascontiguousarray(rows_k, np.int64)
    assert ((rq >= 0) & (rq < N)).all() and ((rk >= 0) & (rk < N)).all()
    dq = np.empty((B, H, len(rq), D), np.float64)
    dk = np.empty((B, H, len(rk), D), np.float64)
    dv = np.empty((B, H, len(rk), M), np.float64)
    P = ctypes.POINTER(ctypes.c_int64)
    lib.orc_backward_causal_poly2_rows(_p(q), _p(k), _p(v), _p(g), rq.ctypes.data_as(P), len(rq),
                                       rk.ctypes.data_as(P), len(rk), _p(dq), _p(dk), _p(dv), B, H, N, D, M)
    return dq, dk, dv


def forward_noncausal_poly2(q, k, v, lib=None):
    """Non-causal attention with the degree-2 polynomial kernel (q . k)^2, through
    its explicit D^2 feature map.  q,k: [B,H,N,D]; v: [B,H,N,M]."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    M = v.shape[-1]
    assert k.shape == q.shape and v.shape == (B, H, N, M)
    out = np.empty((B, H, N, M), np.float64)
    lib.orc_forward_noncausal_poly2(_p(q), _p(k), _p(v), _p(out), B, H, N, D, M)
    return out


def _poly2_rows(q, k, v, rows, causal, lib):
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    M = v.shape[-1]
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    assert k.shape == q.shape and v.shape == (B, H, N, M) and r.ndim == 1
    assert r.size == 0 or (r.min() >= 0 and r.max() < N)
    out = np.empty((B, H, r.size, M), np.float64)
    lib.orc_forward_poly2_rows(_p(q), _p(k), _p(v), r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                               _p(out), B, H, N, D, M, r.size, 1 if causal else 0)
    return out


def forward_causal_poly2_rows(q, k, v, rows, lib=None):
    """Rows ``rows`` of the degree-2 polynomial causal forward, each summed
    directly from the kernel (q_i . k_j)^2 over j <= i.  Returns [B,H,len(rows),M]."""
    return _poly2_rows(q, k, v, rows, True, lib)


def forward_noncausal_poly2_rows(q, k, v, rows, lib=None):
    """Rows of the non-causal polynomial forward, summed directly over all j."""
    return _poly2_rows(q, k, v, rows, False, lib)


def decode_step(q, k, v, S, Z, lib=None):
    """One decode step for all streams.  q,k: [B,H,D]; v: [B,H,M].  ``S`` [B,H,D,M]
    and ``Z`` [B,H,D] must be contiguous float64 arrays; they are updated in place.
    Returns out [B,H,M]."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    assert S.dtype == np.float64 and S.flags.c_contiguous and Z.dtype == np.float64 and Z.flags.c_contiguous
    B, H, D = q.shape
    M = v.shape[-1]
    out = np.empty((B, H, M), np.float64)
    lib.orc_decode_step(_p(q), _p(k), _p(v), _p(S), _p(Z), _p(out), B, H, D, M)
    return out
