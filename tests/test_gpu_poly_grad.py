"""GPU parity of the gradient of the causal degree-2 polynomial forward
(la_backward_causal_poly2) against the fp64 oracle's pairwise definition.

Sizes span several 16-row chunks with ragged tails, one to six blocks of
columns m (M + 1 = 33 or 65 columns in blocks of 33 at D = 32 and 11 at
D = 64), one segment per (b, h) and many (down to one chunk per segment),
both I/O types; the gate is the per-slice and per-chunk normwise bound of
tests/gpu_util.py (floored for dq and dk, whose rows can cancel).
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


def _wl(seed, B, H, N, D, M, dtype):
    return wl.Workload(seed, f"poly gradient seed {seed}", B, H, N, D, M, dtype, 1.0)


def _say(*a):
    print("[gpu]", *a, flush=True)


CASES = [
    ("d32m32_n200_f32", _wl(301, 1, 2, 200, 32, 32, "f32")),
    ("d32m32_n1001_ragged_bf16", _wl(302, 2, 2, 1001, 32, 32, "bf16")),
    ("d32m64_n777_f32_two_blocks", _wl(303, 1, 3, 777, 32, 64, "f32")),
    ("d64m32_n500_bf16_three_blocks", _wl(304, 1, 2, 500, 64, 32, "bf16")),
    ("d64m64_n1500_ragged_f32_six_blocks", _wl(305, 1, 2, 1500, 64, 64, "f32")),
    ("d32m32_b1h1n3000_f32_one_chunk_segments", _wl(306, 1, 1, 3000, 32, 32, "f32")),
    ("d64m64_b1h8n4096_bf16_segments", _wl(307, 1, 8, 4096, 64, 64, "bf16")),
    ("d32m32_b1h8n4096_bf16_segments", _wl(308, 1, 8, 4096, 32, 32, "bf16")),
]


def _run(w):
    q, k, v, g = wl.forward_inputs(w, with_dout=True)
    dq, dk, dv = la.la_backward_causal_poly2(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), dev(g, w.dtype))
    torch.cuda.synchronize()
    return (q, k, v, g), (dq, dk, dv)


@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
def test_backward_causal_poly2(name, w):
    _say(f"polynomial backward {name}: B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}")
    (q, k, v, g), (dq, dk, dv) = _run(w)
    rq, rk, rv = oracle.backward_causal_poly2(q, k, v, g)
    check(f"dq[{name}]", host(dq), rq, w.dtype, floor=True)
    check(f"dk[{name}]", host(dk), rk, w.dtype, floor=True)
    check(f"dv[{name}]", host(dv), rv, w.dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_causal_poly2_single_token(dtype):
    """One token: out_1 = v_1 whatever q and k are, so dv = dout and dq = dk = 0
    up to the rounding residue of e = (g . v - g . out) / d, whose two terms
    are equal in exact arithmetic (out comes back from the forward rounded to
    the I/O type): |dq_a| <= 16 u |k_a| sum_m |g_m v_m| / |q . k| and the same
    for dk with q and k swapped, u = 2^-8 (bf16) or 2^-16 (fp32)."""
    w = _wl(311 if dtype == "bf16" else 312, 2, 3, 1, 32, 64, dtype)
    _say(f"polynomial backward, one token: {dtype}")
    (q, k, v, g), (dq, dk, dv) = _run(w)
    check("dv[single token]", host(dv), g.astype(np.float64), dtype)
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -16
    qk = np.abs((q.astype(np.float64) * k).sum(-1, keepdims=True))
    gv = np.abs(g.astype(np.float64) * v).sum(-1, keepdims=True)
    bq = 16 * u * np.abs(k) * gv / qk
    bk = 16 * u * np.abs(q) * gv / qk
    print(f"  max |dq| / bound {np.max(np.abs(host(dq)) / bq):.3f}, max |dk| / bound {np.max(np.abs(host(dk)) / bk):.3f}",
          flush=True)
    assert (np.abs(host(dq)) <= bq).all() and (np.abs(host(dk)) <= bk).all()


def test_backward_causal_poly2_is_deterministic():
    """The partial sums meet in a fixed order (wavefronts, then column
    blocks): two calls give identical bits."""
    w = _wl(321, 1, 4, 2500, 64, 64, "bf16")
    _say("polynomial backward, repeated call")
    _, a = _run(w)
    _, b = _run(w)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_causal_poly2_long_sampled():
    """The shape the bench times, B1 H8 N65536 D = M = 32 bf16 (32 segments of
    2048 tokens per head on 256 compute units): dq at sampled rows (both ends,
    both sides of every multiple of 2048, random rows) and dk, dv at the last
    40 rows (three 16-row chunks), each summed pair by pair by the oracle."""
    w = _wl(331, 1, 8, 65536, 32, 32, "bf16")
    _say("polynomial backward B1 H8 N65536 D32 M32 bf16, sampled rows")
    (q, k, v, g), (dq, dk, dv) = _run(w)
    N = w.N
    rng = np.random.default_rng(331)
    rows = {0, 1, 15, 16, N - 2, N - 1}
    for b in range(2048, N, 2048):
        rows.update({b - 1, b, b + 1})
    rows.update(int(x) for x in rng.integers(0, N, 32))
    rq = np.array(sorted(rows))
    rk = np.arange(N - 40, N)
    sq, sk, sv = oracle.backward_causal_poly2_rows(q, k, v, g, rq, rk)
    check("dq[long] rows", host(dq)[:, :, rq], sq, w.dtype, floor=True)
    check("dk[long] last rows", host(dk)[:, :, rk], sk, w.dtype, floor=True)
    check("dv[long] last rows", host(dv)[:, :, rk], sv, w.dtype)
