"""Pins of the fp64 oracle against things other than itself.

Each ``check_*`` takes an oracle library handle and raises AssertionError on a
mismatch.  ``tests/test_oracle_pins.py`` runs them on the real oracle; the
mutation tests run them on copies of the oracle source with a planted mistake
and require that at least one check fails.

What pins what:
  * phi against numpy's exp and the closed form x + 1;
  * causal and non-causal forward against the quadratic brute force (an
    independent definition) and against exact rational arithmetic;
  * closed forms: N = 1 gives V; identical keys give the running mean of V;
    constant V gives V; D = 1 makes the output independent of Q;
  * invariants: last causal row equals the non-causal row, Z_N = sum phi(K),
    S_N = sum phi(K_j) V_j^T, positive denominators, convex-hull bounds,
    carrying (S, Z) across a split equals one pass;
  * decode: stacked decode steps equal the causal forward, and the state after
    t steps equals the sum of outer products;
  * backward: central finite differences, the independent quadratic gradient,
    torch fp64 autograd of the brute force, and homogeneity/shift identities.
"""
from __future__ import annotations

import numpy as np

import oracle
from tests import brute_force as bf


def _rel(x, y):
    x, y = np.asarray(x, np.float64), np.asarray(y, np.float64)
    return float(np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300))


def _rand(seed, *shape, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def check_phi(lib):
    x = np.concatenate([np.linspace(-30, 30, 2001), [0.0, -0.0, 1e-300, -1e-300, -700.0, 5e-324]])
    y, dy = oracle.feature_map(x, lib=lib)
    pos = x > 0
    assert np.array_equal(y[pos], x[pos] + 1.0)
    assert np.allclose(y[~pos], np.exp(x[~pos]), rtol=4e-16, atol=0)
    assert np.array_equal(dy[pos], np.ones(pos.sum()))
    assert np.allclose(dy[~pos], np.exp(x[~pos]), rtol=4e-16, atol=0)
    y0, dy0 = oracle.feature_map(np.array([0.0, -0.0]), lib=lib)
    assert y0.tolist() == [1.0, 1.0] and dy0.tolist() == [1.0, 1.0]
    assert (y > 0).all()


def check_forward_vs_brute(lib):
    shapes = [(1, 2, 256, 32, 32), (2, 3, 37, 5, 7), (1, 1, 1, 4, 3), (1, 2, 50, 1, 2), (2, 1, 65, 16, 1),
              (1, 1, 200, 64, 64)]
    for s, (B, H, N, D, M) in enumerate(shapes):
        q = _rand(10 + s, B, H, N, D)
        k = _rand(20 + s, B, H, N, D)
        v = _rand(30 + s, B, H, N, M)
        o = oracle.forward_causal(q, k, v, lib=lib)
        assert _rel(o, bf.forward(q, k, v, True)) < 1e-12, (B, H, N, D, M)
        onc = oracle.forward_noncausal(q, k, v, lib=lib)
        assert _rel(onc, bf.forward(q, k, v, False)) < 1e-12, (B, H, N, D, M)


def check_forward_exact(lib):
    rng = np.random.default_rng(7)
    N, D, M = 6, 3, 2
    # dyadic positive entries: phi = x + 1 is exact and the rational result is exact
    q = rng.integers(1, 9, (N, D)) / 8.0
    k = rng.integers(1, 9, (N, D)) / 4.0
    v = rng.integers(-8, 9, (N, M)) / 2.0
    exact = bf.forward_causal_exact(bf.to_fractions(q), bf.to_fractions(k), bf.to_fractions(v))
    o = oracle.forward_causal(q[None, None], k[None, None], v[None, None], lib=lib)[0, 0]
    for i in range(N):
        for m in range(M):
            e = float(exact[i][m])
            assert abs(o[i, m] - e) <= 4e-16 * max(1.0, abs(e)), (i, m, o[i, m], e)


def check_closed_forms(lib):
    # N = 1: out_1 = V_1
    q, k, v = _rand(1, 2, 2, 1, 8), _rand(2, 2, 2, 1, 8), _rand(3, 2, 2, 1, 5)
    assert np.allclose(oracle.forward_causal(q, k, v, lib=lib), v, rtol=1e-15, atol=1e-15)
    # identical keys: out_i is the running mean of V, whatever Q is
    N = 40
    q = _rand(4, 1, 1, N, 6)
    k = np.repeat(_rand(5, 1, 1, 1, 6), N, axis=2)
    v = _rand(6, 1, 1, N, 3)
    mean = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    assert _rel(oracle.forward_causal(q, k, v, lib=lib), mean) < 1e-13
    # constant V: out = V
    v = np.full((1, 1, N, 3), 2.5)
    assert np.allclose(oracle.forward_causal(q, _rand(7, 1, 1, N, 6), v, lib=lib), 2.5, rtol=1e-14, atol=0)
    # D = 1: phi(q) cancels in the ratio, so out does not depend on Q
    k1, v1 = _rand(8, 1, 2, N, 1), _rand(9, 1, 2, N, 4)
    o1 = oracle.forward_causal(_rand(10, 1, 2, N, 1), k1, v1, lib=lib)
    o2 = oracle.forward_causal(_rand(11, 1, 2, N, 1) * 3.0, k1, v1, lib=lib)
    assert _rel(o1, o2) < 1e-13
    # ... but with D > 1 it does (guards against a readout that ignores Q)
    o3 = oracle.forward_causal(_rand(10, 1, 2, N, 3), _rand(8, 1, 2, N, 3), v1, lib=lib)
    o4 = oracle.forward_causal(_rand(11, 1, 2, N, 3) * 3.0, _rand(8, 1, 2, N, 3), v1, lib=lib)
    assert _rel(o3, o4) > 1e-3


def check_invariants(lib):
    B, H, N, D, M = 2, 3, 97, 8, 5
    q, k, v = _rand(40, B, H, N, D), _rand(41, B, H, N, D), _rand(42, B, H, N, M)
    o, S, Z, den = oracle.forward_causal(q, k, v, return_state=True, return_den=True, lib=lib)
    onc = oracle.forward_noncausal(q, k, v, lib=lib)
    assert _rel(o[:, :, -1], onc[:, :, -1]) < 1e-13
    kh = bf.phi(k)
    assert _rel(Z, kh.sum(2)) < 1e-14
    assert _rel(S, np.einsum("bhnd,bhnm->bhdm", kh, v)) < 1e-13
    assert (den > 0).all()
    assert _rel(den, (bf.phi(q) * np.cumsum(kh, axis=2)).sum(-1)) < 1e-13
    lo = np.minimum.accumulate(v, axis=2)
    hi = np.maximum.accumulate(v, axis=2)
    assert (o >= lo - 1e-12).all() and (o <= hi + 1e-12).all()
    # first row is exactly V_1 up to rounding
    assert np.allclose(o[:, :, 0], v[:, :, 0], rtol=1e-14, atol=1e-14)
    # carrying the state across a split equals one pass
    c = 41
    o_a, S_a, Z_a = oracle.forward_causal(q[:, :, :c], k[:, :, :c], v[:, :, :c], return_state=True, lib=lib)
    o_b, S_b, Z_b = oracle.forward_causal(q[:, :, c:], k[:, :, c:], v[:, :, c:], S0=S_a, Z0=Z_a,
                                          return_state=True, lib=lib)
    assert _rel(np.concatenate([o_a, o_b], axis=2), o) < 1e-14
    assert _rel(S_b, S) < 1e-14 and _rel(Z_b, Z) < 1e-14


def check_initial_state(lib):
    """An arbitrary starting state (S0 of any sign, Z0 > 0, not the state of
    any prefix) enters every readout as one extra, pre-summed key: written out
    by brute force, out_i = (phi(q_i) S0 + sum_{j<=i} a_ij v_j) /
    (phi(q_i) . Z0 + sum_{j<=i} a_ij), and the final state is S0 + sum_j
    phi(k_j) v_j^T, Z0 + sum_j phi(k_j)."""
    B, H, N, D, M = 2, 2, 33, 5, 3
    q, k, v = _rand(60, B, H, N, D), _rand(61, B, H, N, D), _rand(62, B, H, N, M)
    S0 = _rand(63, B, H, D, M) * 4.0
    Z0 = np.abs(_rand(64, B, H, D)) * 5.0 + 0.5
    o, S, Z = oracle.forward_causal(q, k, v, S0=S0, Z0=Z0, return_state=True, lib=lib)
    qh, kh = bf.phi(q), bf.phi(k)
    a = bf.similarity(q, k, True)
    num = np.einsum("bhnd,bhdm->bhnm", qh, S0) + a @ v
    den = np.einsum("bhnd,bhd->bhn", qh, Z0)[..., None] + a.sum(-1, keepdims=True)
    assert _rel(o, num / den) < 1e-13
    assert _rel(S, S0 + np.einsum("bhnd,bhnm->bhdm", kh, v)) < 1e-13
    assert _rel(Z, Z0 + kh.sum(2)) < 1e-14
    # the start state matters (guards against a recurrence that drops it)
    assert _rel(o, bf.forward(q, k, v)) > 1e-2


def check_decode(lib):
    B, H, T, D, M = 3, 2, 60, 6, 4
    qs, ks, vs = _rand(50, T, B, H, D), _rand(51, T, B, H, D), _rand(52, T, B, H, M)
    S = np.zeros((B, H, D, M))
    Z = np.zeros((B, H, D))
    outs = []
    for t in range(T):
        if t == 25:   # save and resume: continue from copies of the state
            S, Z = S.copy(), Z.copy()
        outs.append(oracle.decode_step(qs[t], ks[t], vs[t], S, Z, lib=lib))
    dec = np.stack(outs, axis=2)                   # [B,H,T,M]
    tr = lambda x: np.ascontiguousarray(np.moveaxis(x, 0, 2))
    fwd = bf.forward(tr(qs), tr(ks), tr(vs), True)
    assert _rel(dec, fwd) < 1e-13
    kh = bf.phi(tr(ks))
    assert _rel(S, np.einsum("bhnd,bhnm->bhdm", kh, tr(vs))) < 1e-13
    assert _rel(Z, kh.sum(2)) < 1e-14


def check_backward_vs_quadratic(lib):
    for s, (B, H, N, D, M) in enumerate([(1, 2, 64, 8, 6), (2, 1, 33, 3, 9), (1, 1, 1, 4, 4), (1, 1, 120, 32, 32)]):
        q, k, v, g = (_rand(60 + 4 * s + i, B, H, N, x) for i, x in enumerate((D, D, M, M)))
        dq, dk, dv = oracle.backward_causal(q, k, v, g, lib=lib)
        rq, rk, rv = bf.backward_causal(q, k, v, g)
        if N == 1:
            # out_1 = V_1 whatever Q, K are: dQ = dK = 0 and dV = G
            assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14 and _rel(dv, g) < 1e-15
            continue
        assert _rel(dq, rq) < 1e-11 and _rel(dk, rk) < 1e-11 and _rel(dv, rv) < 1e-11, (B, H, N, D, M)


def check_backward_fd(lib):
    B, H, N, D, M = 1, 1, 7, 3, 2
    q, k, v, g = _rand(70, B, H, N, D), _rand(71, B, H, N, D), _rand(72, B, H, N, M), _rand(73, B, H, N, M)
    dq, dk, dv = oracle.backward_causal(q, k, v, g, lib=lib)

    def loss(q_, k_, v_):
        return float((oracle.forward_causal(q_, k_, v_, lib=lib) * g).sum())

    eps = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        base = [q, k, v]
        num = np.zeros_like(base[which])
        it = np.nditer(num, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            p = [x.copy() for x in base]
            m_ = [x.copy() for x in base]
            p[which][idx] += eps
            m_[which][idx] -= eps
            num[idx] = (loss(*p) - loss(*m_)) / (2 * eps)
        assert np.allclose(grad, num, rtol=1e-6, atol=1e-8), (which, np.abs(grad - num).max())


def check_backward_autograd(lib):
    import torch

    B, H, N, D, M = 2, 2, 45, 6, 5
    arrs = [_rand(80 + i, B, H, N, x) for i, x in enumerate((D, D, M, M))]
    q, k, v, g = (torch.tensor(a, dtype=torch.float64) for a in arrs)
    q.requires_grad_(True); k.requires_grad_(True); v.requires_grad_(True)
    qh = torch.nn.functional.elu(q) + 1.0
    kh = torch.nn.functional.elu(k) + 1.0
    a = torch.tril(qh @ kh.transpose(-1, -2).contiguous())
    o = (a @ v) / a.sum(-1, keepdim=True)
    (o * g).sum().backward()
    dq, dk, dv = oracle.backward_causal(*arrs, lib=lib)
    assert _rel(dq, q.grad.numpy()) < 1e-11
    assert _rel(dk, k.grad.numpy()) < 1e-11
    assert _rel(dv, v.grad.numpy()) < 1e-11


def check_backward_identities(lib):
    B, H, N, D, M = 1, 2, 300, 16, 12
    q, k, v, g = _rand(90, B, H, N, D), _rand(91, B, H, N, D), _rand(92, B, H, N, M), _rand(93, B, H, N, M)
    dq, dk, dv = oracle.backward_causal(q, k, v, g, lib=lib)
    o = oracle.forward_causal(q, k, v, lib=lib)
    # shifting V[:, m] by t shifts out[:, m] by t, so sum_j dV_j = sum_i G_i
    assert _rel(dv.sum(2), g.sum(2)) < 1e-12
    # out is linear in V: sum_j V_j . dV_j = sum_i G_i . out_i
    assert abs((v * dv).sum() - (g * o).sum()) < 1e-10 * max(1.0, abs((g * o).sum()))
    # out_i is 0-homogeneous in phi(Q_i): sum_d dQ_id * phi(Q_id)/phi'(Q_id) = 0 per token
    w = 1.0 + np.maximum(q, 0.0)
    assert np.abs((dq * w).sum(-1)).max() < 1e-11 * np.abs(dq * w).max() * D
    # ... and 0-homogeneous in all phi(K) together: the sum vanishes per (b, h)
    wk = 1.0 + np.maximum(k, 0.0)
    per_bh = (dk * wk).sum(axis=(2, 3))
    assert np.abs(per_bh).max() < 1e-10 * np.abs(dk * wk).sum()
    # the gradient is not trivially zero
    assert np.abs(dq).max() > 1e-3 and np.abs(dk).max() > 1e-3


def check_backward_noncausal(lib):
    """Non-causal backward: the quadratic gradient without a mask, central
    differences of the oracle's own non-causal forward, torch fp64 autograd of
    the brute-force form, and the identities of the causal case, which hold
    with the mask removed too."""
    import torch

    for s, (B, H, N, D, M) in enumerate([(1, 2, 64, 8, 6), (2, 1, 33, 3, 9), (1, 1, 1, 4, 4), (1, 1, 90, 32, 32)]):
        q, k, v, g = (_rand(300 + 4 * s + i, B, H, N, x) for i, x in enumerate((D, D, M, M)))
        dq, dk, dv = oracle.backward_noncausal(q, k, v, g, lib=lib)
        rq, rk, rv = bf.backward(q, k, v, g, causal=False)
        if N == 1:
            assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14 and _rel(dv, g) < 1e-15
            continue
        assert _rel(dq, rq) < 1e-11 and _rel(dk, rk) < 1e-11 and _rel(dv, rv) < 1e-11, (B, H, N, D, M)
        o = oracle.forward_noncausal(q, k, v, lib=lib)
        assert _rel(dv.sum(2), g.sum(2)) < 1e-12                       # shift of V
        assert _rel((v * dv).sum((2, 3)), (g * o).sum((2, 3))) < 1e-11   # linear in V
        wq, wk = 1.0 + np.maximum(q, 0.0), 1.0 + np.maximum(k, 0.0)
        assert np.abs((dq * wq).sum(-1)).max() < 1e-10 * np.abs(dq * wq).sum(-1).max()
        assert np.abs((dk * wk).sum((2, 3))).max() < 1e-10 * np.abs(dk * wk).sum()

    B, H, N, D, M = 1, 1, 6, 3, 2
    q, k, v, g = _rand(320, B, H, N, D), _rand(321, B, H, N, D), _rand(322, B, H, N, M), _rand(323, B, H, N, M)
    dq, dk, dv = oracle.backward_noncausal(q, k, v, g, lib=lib)
    eps = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros_like(grad)
        it = np.nditer(num, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            p = [x.copy() for x in (q, k, v)]
            m_ = [x.copy() for x in (q, k, v)]
            p[which][idx] += eps
            m_[which][idx] -= eps
            num[idx] = ((oracle.forward_noncausal(*p, lib=lib) - oracle.forward_noncausal(*m_, lib=lib)) * g).sum() \
                / (2 * eps)
        assert np.allclose(grad, num, rtol=1e-6, atol=1e-8), (which, np.abs(grad - num).max())

    B, H, N, D, M = 2, 2, 40, 6, 5
    arrs = [_rand(330 + i, B, H, N, x) for i, x in enumerate((D, D, M, M))]
    tq, tk, tv, tg = (torch.tensor(a, dtype=torch.float64) for a in arrs)
    tq.requires_grad_(True); tk.requires_grad_(True); tv.requires_grad_(True)
    a = (torch.nn.functional.elu(tq) + 1.0) @ (torch.nn.functional.elu(tk) + 1.0).transpose(-1, -2).contiguous()
    out = (a @ tv) / a.sum(-1, keepdim=True)
    (out * tg).sum().backward()
    dq, dk, dv = oracle.backward_noncausal(*arrs, lib=lib)
    assert _rel(dq, tq.grad.numpy()) < 1e-11 and _rel(dk, tk.grad.numpy()) < 1e-11 and _rel(dv, tv.grad.numpy()) < 1e-11


def check_rff_worked_example(lib):
    """Random Fourier features on a hand-worked case.  D = 2, R = 4,
    omega = [[0, 1, 0, 2], [1, 0, 0, 0]] (omega[d][r]), b = (0, pi/2, pi, 0),
    x = (pi/3, pi/4).  The angles x . omega[:, r] + b_r are pi/4, pi/3 + pi/2,
    pi and 2 pi/3, whose cosines are sqrt(2)/2, -sqrt(3)/2, -1 and -1/2;
    times sqrt(2/R) = 1/sqrt(2) that is 1/2, -sqrt(6)/4, -1/sqrt(2),
    -1/(2 sqrt(2)).  An omega read transposed, a missing scale, sin for cos or
    a dropped b each change these numbers."""
    omega = np.array([[0.0, 1.0, 0.0, 2.0], [1.0, 0.0, 0.0, 0.0]])
    b = np.array([0.0, np.pi / 2, np.pi, 0.0])
    x = np.array([[np.pi / 3, np.pi / 4]])
    want = np.array([[0.5, -np.sqrt(6.0) / 4, -1.0 / np.sqrt(2.0), -1.0 / (2.0 * np.sqrt(2.0))]])
    got = oracle.rff_features(x, omega, b, lib=lib)
    assert np.abs(got - want).max() < 1e-15, got


def check_rff_estimates_rbf_kernel(lib):
    """With many features, phi(q) . phi(k) converges to the RBF kernel
    exp(-|q - k|^2 / (2 sigma^2)) (standard deviation about 1/sqrt(2R))."""
    D, R, sigma = 6, 40000, 1.7
    rng = np.random.default_rng(77)
    omega = rng.standard_normal((D, R)) / sigma
    b = rng.uniform(0.0, 2.0 * np.pi, R)
    q = rng.standard_normal((12, D)) * 0.8
    k = rng.standard_normal((12, D)) * 0.8
    fq, fk = oracle.rff_features(q, omega, b, lib=lib), oracle.rff_features(k, omega, b, lib=lib)
    est = (fq * fk).sum(-1)
    exact = np.exp(-((q - k) ** 2).sum(-1) / (2.0 * sigma ** 2))
    assert np.abs(est - exact).max() < 0.03, np.abs(est - exact).max()
    assert np.abs((fq * fq).sum(-1) - 1.0).max() < 0.03           # k(q, q) = 1


def check_forward_features(lib):
    """Causal forward on given features: the quadratic form with
    a_ij = fq_i . fk_j (j <= i) for features of either sign, and the elu + 1
    path when the given features are phi(Q), phi(K)."""
    B, H, N, F, M = 2, 2, 57, 7, 5
    fq = _rand(400, B, H, N, F) * 0.6 + 1.0         # mixed signs, positive denominators
    fk = _rand(401, B, H, N, F) * 0.6 + 1.0
    v = _rand(402, B, H, N, M)
    a = np.tril(fq @ np.swapaxes(fk, -1, -2))
    ref = (a @ v) / a.sum(-1, keepdims=True)
    assert (fq < 0).any() and (fk < 0).any() and (a.sum(-1) > 0).all()
    assert _rel(oracle.forward_causal_features(fq, fk, v, lib=lib), ref) < 1e-12
    q, k = _rand(403, B, H, N, F), _rand(404, B, H, N, F)
    assert _rel(oracle.forward_causal_features(bf.phi(q), bf.phi(k), v, lib=lib),
                oracle.forward_causal(q, k, v, lib=lib)) < 1e-14


def check_poly2(lib):
    """Degree-2 polynomial kernel: the oracle's explicit D^2 feature map
    against brute force with the kernel itself, a_ij = (q_i . k_j)^2 for
    j <= i (all j for the non-causal form, also through the feature map); N = 1
    gives V_1; the last causal row equals the non-causal form; sampled rows
    match the full passes."""
    for s, (B, H, N, D, M) in enumerate([(1, 2, 40, 5, 3), (2, 1, 17, 8, 6), (1, 1, 1, 4, 4), (1, 1, 64, 32, 32)]):
        q, k, v = _rand(500 + 3 * s, B, H, N, D), _rand(501 + 3 * s, B, H, N, D), _rand(502 + 3 * s, B, H, N, M)
        a = np.tril((q @ np.swapaxes(k, -1, -2)) ** 2)
        ref = (a @ v) / a.sum(-1, keepdims=True)
        got = oracle.forward_causal_poly2(q, k, v, lib=lib)
        assert _rel(got, ref) < 1e-12, (B, H, N, D, M, _rel(got, ref))
        if N == 1:
            assert _rel(got, v) < 1e-15
        full = (q @ np.swapaxes(k, -1, -2)) ** 2
        assert _rel(got[:, :, -1], ((full @ v) / full.sum(-1, keepdims=True))[:, :, -1]) < 1e-12
        rows = np.unique(np.array([0, N // 3, N // 2, N - 1]))
        sampled = oracle.forward_causal_poly2_rows(q, k, v, rows, lib=lib)
        assert _rel(sampled, ref[:, :, rows]) < 1e-12, (B, H, N, D, M, _rel(sampled, ref[:, :, rows]))
        # the non-causal form: every key attends
        ref_nc = (full @ v) / full.sum(-1, keepdims=True)
        got_nc = oracle.forward_noncausal_poly2(q, k, v, lib=lib)
        assert _rel(got_nc, ref_nc) < 1e-12, (B, H, N, D, M, _rel(got_nc, ref_nc))
        assert _rel(oracle.forward_noncausal_poly2_rows(q, k, v, rows, lib=lib), ref_nc[:, :, rows]) < 1e-12


def check_poly2_backward(lib):
    """Gradients of the polynomial causal forward: central finite differences of
    the (separately pinned) forward; N = 1 gives dV = dout, dQ = dK = 0; the
    outputs do not change when one query row, or all key rows together, are
    scaled (so dq_i . q_i = 0 for every i and sum_j dk_j . k_j = 0); adding a
    constant to V shifts every output by it (so sum_j dv_j = sum_i dout_i)."""
    for s, (B, H, N, D, M) in enumerate([(1, 1, 6, 3, 2), (1, 2, 5, 2, 3)]):
        q, k = _rand(600 + 4 * s, B, H, N, D), _rand(601 + 4 * s, B, H, N, D)
        v, g = _rand(602 + 4 * s, B, H, N, M), _rand(603 + 4 * s, B, H, N, M)
        grads = oracle.backward_causal_poly2(q, k, v, g, lib=lib)

        def loss(q_, k_, v_):
            return float((oracle.forward_causal_poly2(q_, k_, v_, lib=lib) * g).sum())

        eps = 1e-6
        for which, grad in enumerate(grads):
            base = [q, k, v]
            num = np.zeros_like(base[which])
            it = np.nditer(num, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                p_ = [x.copy() for x in base]
                m_ = [x.copy() for x in base]
                p_[which][idx] += eps
                m_[which][idx] -= eps
                num[idx] = (loss(*p_) - loss(*m_)) / (2 * eps)
            assert np.allclose(grad, num, rtol=1e-6, atol=1e-8), (s, which, np.abs(grad - num).max())
    q, k, v, g = _rand(620, 2, 3, 1, 4), _rand(621, 2, 3, 1, 4), _rand(622, 2, 3, 1, 5), _rand(623, 2, 3, 1, 5)
    dq, dk, dv = oracle.backward_causal_poly2(q, k, v, g, lib=lib)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12 and _rel(dv, g) < 1e-15
    q, k, v, g = _rand(630, 1, 2, 33, 8), _rand(631, 1, 2, 33, 8), _rand(632, 1, 2, 33, 6), _rand(633, 1, 2, 33, 6)
    dq, dk, dv = oracle.backward_causal_poly2(q, k, v, g, lib=lib)
    scale = np.abs(dq).max() * np.abs(q).max()
    assert np.abs((dq * q).sum(-1)).max() < 1e-12 * scale * 8
    assert np.abs((dk * k).sum((-1, -2))).max() < 1e-12 * np.abs(dk).max() * np.abs(k).max() * 33 * 8
    assert _rel(dv.sum(-2), g.sum(-2)) < 1e-12
    # selected rows, each summed on its own, equal the full gradient's rows
    rq, rk = np.array([0, 5, 16, 31, 32]), np.array([20, 27, 31, 32])
    sq, sk, sv = oracle.backward_causal_poly2_rows(q, k, v, g, rq, rk, lib=lib)
    assert _rel(sq, dq[:, :, rq]) < 1e-12 and _rel(sk, dk[:, :, rk]) < 1e-12 and _rel(sv, dv[:, :, rk]) < 1e-12


ALL_CHECKS = [check_phi, check_forward_vs_brute, check_forward_exact, check_closed_forms, check_invariants,
              check_initial_state, check_decode, check_backward_vs_quadratic, check_backward_fd, check_backward_autograd,
              check_backward_identities, check_backward_noncausal, check_rff_worked_example,
              check_rff_estimates_rbf_kernel, check_forward_features, check_poly2, check_poly2_backward]
