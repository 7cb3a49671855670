"""Independent quadratic (N x N) definitions used to pin the fp64 oracle.

These are the plain definitions of kernelized attention, written as dense
matrix algebra over the full similarity matrix, with no recurrence and no
prefix state:

  a_ij = phi(Q_i) . phi(K_j)                    (similarity, [deck] slide 3)
  causal:     out_i = sum_{j<=i} a_ij V_j / sum_{j<=i} a_ij   ([deck] slide 4)
  non-causal: out_i = sum_j a_ij V_j / sum_j a_ij              ([review] "Proposed method")

The gradient is the direct quadratic one (derivative of each a_ij), a
different route from the oracle's forward/reverse prefix sums:
  w_ij = a_ij / d_i,  dL/da_ij = G_i . (V_j - out_i) / d_i,
  dqh_i = sum_{j<=i} dL/da_ij kh_j,  dkh_j = sum_{i>=j} dL/da_ij qh_i,
  dV_j = sum_{i>=j} w_ij G_i,  then times phi'(.) for Q and K.

Sources: [review] nubint.ai "[Paper Review] Transformers are RNNs", section
"Proposed method"; [deck] zhengyuhong.cn "Transformers are RNNs ... 解读",
slides 3-4; [summary] paperlayer.ai summary, appendix "A. Gradient Derivation".
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def phi(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def dphi(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))


def similarity(q, k, causal: bool):
    qh, kh = phi(q), phi(k)
    a = qh @ np.swapaxes(kh, -1, -2)
    if causal:
        n = a.shape[-1]
        a = a * np.tril(np.ones((n, n)))
    return a


def forward(q, k, v, causal: bool = True):
    a = similarity(q, k, causal)
    return (a @ np.asarray(v, np.float64)) / a.sum(-1, keepdims=True)


def backward_causal(q, k, v, g):
    return backward(q, k, v, g, causal=True)


def backward(q, k, v, g, causal: bool = True):
    q, k, v, g = (np.asarray(x, np.float64) for x in (q, k, v, g))
    qh, kh = phi(q), phi(k)
    a = similarity(q, k, causal)
    d = a.sum(-1, keepdims=True)
    o = (a @ v) / d
    # dL/da_ij = G_i . (V_j - O_i) / d_i, masked to j <= i
    gv = g @ np.swapaxes(v, -1, -2)                       # G_i . V_j
    go = (g * o).sum(-1, keepdims=True)                   # G_i . O_i
    n = a.shape[-1]
    mask = np.tril(np.ones((n, n))) if causal else np.ones((n, n))
    da = (gv - go) / d * mask
    dqh = da @ kh
    dkh = np.swapaxes(da, -1, -2) @ qh
    w = a / d
    dv = np.swapaxes(w, -1, -2) @ g
    return dqh * dphi(q), dkh * dphi(k), dv


def forward_causal_exact(q, k, v):
    """Exact rational causal attention for inputs whose phi is rational, i.e.
    every q, k entry > 0 (phi = x + 1).  q,k: [N][D], v: [N][M] of Fractions."""
    N, D, M = len(q), len(q[0]), len(v[0])
    qh = [[x + 1 for x in row] for row in q]
    kh = [[x + 1 for x in row] for row in k]
    out = []
    for i in range(N):
        a = [sum(qh[i][t] * kh[j][t] for t in range(D)) for j in range(i + 1)]
        den = sum(a)
        out.append([sum(a[j] * v[j][m] for j in range(i + 1)) / den for m in range(M)])
    return out


def to_fractions(x):
    return [[Fraction(float(e)) for e in row] for row in np.asarray(x, np.float64)]
