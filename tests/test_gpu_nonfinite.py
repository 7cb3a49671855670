"""Non-finite inputs on the GPU: they are not errors, they propagate.

A NaN (or an infinity that turns into one) must reach every output that
depends on it, and outputs that do not depend on it must come out exactly as
in a clean run, except within the NaN's own 16-token chunk and 16-feature
group, where the matrix products can carry it further (0 * NaN = NaN).  Each
case compares against the clean run of the same inputs, bit for bit, outside
those chunks.  -inf in a query is not an error either: phi(-inf) = 0, and the
row matches the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_util import check, dev, host

pytestmark = pytest.mark.gpu

la = pytest.importorskip("kernelized_transformer_amd")

J, COL = 1234, 37           # the poisoned token and feature
C0, C1 = J // 16 * 16, J // 16 * 16 + 16   # its 16-token chunk
G0, G1 = COL // 16 * 16, COL // 16 * 16 + 16   # its 16-feature group


def _say(*a):
    print("[gpu]", *a, flush=True)


def _inputs(B, H, N, D, M, dtype, seed):
    w = wl.Workload(seed, "non-finite", B, H, N, D, M, dtype)
    return w, [dev(x, dtype) for x in wl.forward_inputs(w, with_dout=True)]


def _poison(t, value, row=J, col=COL):
    t = t.clone()
    t[0, 0, row, col] = value
    return t


def _rows_equal(a, b, rows):
    return torch.equal(a[0, 0, rows], b[0, 0, rows])


# (name, B, H, N, D, M, dtype): a many-workgroup bf16 head (hand-off between
# 63 workgroups) and an fp32 one
SHAPES = [("bf16_63_workgroups", 1, 2, 40000, 64, 64, "bf16"), ("f32_d32m64", 1, 2, 3000, 32, 64, "f32")]


@pytest.mark.parametrize("name,B,H,N,D,M,dtype", SHAPES, ids=[s[0] for s in SHAPES])
def test_forward_causal_nan(name, B, H, N, D, M, dtype):
    w, (q, k, v, _) = _inputs(B, H, N, D, M, dtype, 301)
    _say(f"NaN propagation, causal forward {name}")
    clean = la.la_forward_causal(q, k, v)
    nan = float("nan")
    # in a query: only that token's row
    oq = la.la_forward_causal(_poison(q, nan, col=COL % D), k, v)
    # in a key: every row from that token on
    ok = la.la_forward_causal(q, _poison(k, nan, col=COL % D), v)
    # in a value: that column of every row from that token on
    ov = la.la_forward_causal(q, k, _poison(v, nan))
    # +inf in a key: phi(+inf) = inf, every later row turns non-finite
    oi = la.la_forward_causal(q, _poison(k, float("inf"), col=COL % D), v)
    torch.cuda.synchronize()
    assert not torch.isfinite(oq[0, 0, J]).any()
    others = torch.ones(N, dtype=torch.bool, device="cuda")
    others[J] = False
    assert torch.equal(oq[0, 0, others], clean[0, 0, others]) and torch.equal(oq[:, 1:], clean[:, 1:])
    for o in (ok, oi):
        assert not torch.isfinite(o[0, 0, J:]).any(), "an output from the key on stayed finite"
        assert _rows_equal(o, clean, slice(0, C0)) and torch.equal(o[:, 1:], clean[:, 1:])
    assert not torch.isfinite(ov[0, 0, J:, COL]).any()
    assert _rows_equal(ov, clean, slice(0, C0)) and torch.equal(ov[:, 1:], clean[:, 1:])
    keep = [c for c in range(M) if not G0 <= c < G1]
    assert torch.equal(ov[0, 0, :, keep], clean[0, 0, :, keep])


@pytest.mark.parametrize("name,B,H,N,D,M,dtype", SHAPES, ids=[s[0] for s in SHAPES])
def test_forward_noncausal_nan(name, B, H, N, D, M, dtype):
    w, (q, k, v, _) = _inputs(B, H, N, D, M, dtype, 302)
    _say(f"NaN propagation, non-causal forward {name}")
    clean = la.la_forward_noncausal(q, k, v)
    oq = la.la_forward_noncausal(_poison(q, float("nan"), col=COL % D), k, v)
    ok = la.la_forward_noncausal(q, _poison(k, float("nan"), col=COL % D), v)
    torch.cuda.synchronize()
    assert not torch.isfinite(oq[0, 0, J]).any()
    others = torch.ones(N, dtype=torch.bool, device="cuda")
    others[J] = False
    assert torch.equal(oq[0, 0, others], clean[0, 0, others])
    assert not torch.isfinite(ok[0, 0]).any(), "an output stayed finite"
    assert torch.equal(ok[:, 1:], clean[:, 1:])


def test_forward_minus_inf_query_is_finite():
    """phi(-inf) = exp(-inf) = 0: a query entry of -inf only drops that
    feature; the row is finite and matches the oracle."""
    w, (q, k, v, _) = _inputs(1, 2, 3000, 64, 64, "bf16", 303)
    _say("-inf in a query")
    qm = _poison(q, float("-inf"), col=5)
    out = la.la_forward_causal(qm, k, v)
    torch.cuda.synchronize()
    ref = oracle.forward_causal(host(qm), host(k), host(v))
    check("out with -inf in a query", host(out), ref, "bf16")


def test_backward_causal_nan_in_dout():
    """NaN in dout_j (one column): dQ_j is non-finite and every other dQ row
    is unchanged; dK of every earlier token (through h_j) and that column of
    dV of every earlier token are non-finite; rows after j's chunk are
    unchanged, and dV's other feature groups everywhere outside the chunk."""
    w, (q, k, v, g) = _inputs(1, 2, 20000, 64, 64, "bf16", 304)
    _say("NaN propagation, causal backward (bf16, D = M = 64)")
    cq, ck, cv = la.la_backward_causal(q, k, v, g)
    dq, dk, dv = la.la_backward_causal(q, k, v, _poison(g, float("nan")))
    torch.cuda.synchronize()
    assert not torch.isfinite(dq[0, 0, J]).any()
    others = torch.ones(w.N, dtype=torch.bool, device="cuda")
    others[J] = False
    assert torch.equal(dq[0, 0, others], cq[0, 0, others]) and torch.equal(dq[:, 1:], cq[:, 1:])
    assert not torch.isfinite(dk[0, 0, :C0]).any(), "an earlier dK entry stayed finite"
    assert not torch.isfinite(dv[0, 0, :C0, COL]).any()
    for got, clean in ((dk, ck), (dv, cv)):
        assert _rows_equal(got, clean, slice(C1, None)) and torch.equal(got[:, 1:], clean[:, 1:])
    keep = [c for c in range(w.M) if not G0 <= c < G1]
    outside = torch.ones(w.N, dtype=torch.bool, device="cuda")
    outside[C0:C1] = False
    assert torch.equal(dv[0, 0][outside][:, keep], cv[0, 0][outside][:, keep])


def test_decode_nan_stays_in_its_stream():
    """NaN in one stream's key at one step: that stream's state and every
    later output turn non-finite; every other stream is unchanged."""
    w = wl.Workload(305, "decode non-finite", 4, 8, 1, 64, 64, "bf16")
    qs, ks, vs = wl.DecodeStream(w).take(40)
    qd, kd, vd = dev(qs, "bf16"), dev(ks, "bf16"), dev(vs, "bf16")
    _say("NaN propagation, decode")

    def run(kk):
        S = torch.zeros((w.B, w.H, w.D, w.M), device="cuda")
        Z = torch.zeros((w.B, w.H, w.D), device="cuda")
        outs = [la.la_decode_step(qd[t], kk[t], vd[t], S, Z) for t in range(40)]
        return torch.stack(outs), S, Z

    clean = run(kd)
    kp = kd.clone()
    kp[17, 2, 5, 9] = float("nan")
    bad = run(kp)
    torch.cuda.synchronize()
    mask = torch.zeros((w.B, w.H), dtype=torch.bool, device="cuda")
    mask[2, 5] = True
    assert torch.equal(bad[0][:17], clean[0][:17])
    assert not torch.isfinite(bad[0][17:, 2, 5]).any()
    assert torch.equal(bad[0][:, ~mask], clean[0][:, ~mask])
    assert not torch.isfinite(bad[2][2, 5, 9]) and torch.equal(bad[2][~mask], clean[2][~mask])
    assert not torch.isfinite(bad[1][2, 5, 9]).any() and torch.equal(bad[1][~mask], clean[1][~mask])
