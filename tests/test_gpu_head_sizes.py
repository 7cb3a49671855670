"""GPU parity for head sizes outside {32, 64}: every multiple of 16 up to 128.

The forwards (causal, non-causal, from a start state, on given features, the
no-allocation entry point) and the backwards run the generic path for these
sizes, decode its general kernel; each case is gated against the fp64 oracle
like the rest of the parity suite (normwise per slice and per 16-token chunk;
dQ and dK with the gradient floor).  The polynomial and random-feature
kernels keep D, M in {32, 64} and must say so.
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


def _w(seed, B, H, N, D, M, dtype):
    return wl.Workload(seed, f"head sizes {D}x{M}", B, H, N, D, M, dtype)


def _say(*a):
    print("[gpu]", *a, flush=True)


CASES = [
    ("d128m128_bf16", _w(501, 1, 4, 5000, 128, 128, "bf16")),
    ("d16m16_f32_ragged", _w(502, 2, 3, 1001, 16, 16, "f32")),
    ("d48m80_bf16", _w(503, 1, 2, 3000, 48, 80, "bf16")),
    ("d96m32_f32", _w(504, 1, 3, 2500, 96, 32, "f32")),
    ("d112m64_bf16", _w(505, 2, 2, 1500, 112, 64, "bf16")),
    ("d128m16_f32", _w(506, 1, 2, 777, 128, 16, "f32")),
    ("d32m128_bf16_many_segments", _w(507, 1, 2, 40000, 32, 128, "bf16")),
    ("d80m112_f32_one_token", _w(508, 1, 2, 1, 80, 112, "f32")),
    ("d64m96_bf16", _w(509, 1, 8, 4096, 64, 96, "bf16")),
    ("d128m128_f32", _w(510, 1, 2, 2000, 128, 128, "f32")),
    # fewer column groups than wavefront loads of the shared Q, K rows: each
    # lane moves several pieces (D=128, M=16: four; D=96, M=32: three)
    ("d128m16_bf16", _w(511, 1, 2, 1500, 128, 16, "bf16")),
    ("d96m32_bf16_ragged", _w(512, 2, 2, 1777, 96, 32, "bf16")),
]


@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
def test_forward_causal_head_sizes(name, w):
    q, k, v = wl.forward_inputs(w)
    _say(f"forward causal {name}: B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}")
    out = la.la_forward_causal(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype))
    torch.cuda.synchronize()
    check(f"out[{name}]", host(out), oracle.forward_causal(q, k, v), w.dtype)


@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
def test_forward_noncausal_head_sizes(name, w):
    q, k, v = wl.forward_inputs(w)
    _say(f"forward non-causal {name}: B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}")
    out = la.la_forward_noncausal(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype))
    torch.cuda.synchronize()
    check(f"out[{name}]", host(out), oracle.forward_noncausal(q, k, v), w.dtype)


@pytest.mark.parametrize("name,w,cuts", [
    ("d128m128_bf16", _w(511, 2, 2, 3000, 128, 128, "bf16"), [0, 1234, 3000]),
    ("d48m16_f32", _w(512, 1, 3, 900, 48, 16, "f32"), [0, 1, 450, 900]),
], ids=["d128m128_bf16", "d48m16_f32"])
def test_forward_state_chain_head_sizes(name, w, cuts):
    """Pieces chained through the state (start state in place), against one
    oracle pass; then decode continues from the final state."""
    q, k, v = wl.forward_inputs(w)
    _say(f"state chain {name}: B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}, cuts {cuts}")
    keep, outs = [], []
    S = Z = None
    for a, b in zip(cuts[:-1], cuts[1:]):
        qd, kd, vd = (dev(np.ascontiguousarray(x[:, :, a:b]), w.dtype) for x in (q, k, v))
        keep += [qd, kd, vd]
        if S is None:
            out, S, Z = la.la_forward_causal_state(qd, kd, vd)
        else:
            out, _, _ = la.la_forward_causal_state(qd, kd, vd, s0=S, z0=Z, s_final=S, z_final=Z)
        outs.append(out)
    torch.cuda.synchronize()
    ref, S_ref, Z_ref = oracle.forward_causal(q, k, v, return_state=True)
    check(f"out[{name}]", np.concatenate([host(o) for o in outs], axis=2), ref, w.dtype)
    check(f"S_N[{name}]", host(S), S_ref, w.dtype)
    check(f"Z_N[{name}]", host(Z), Z_ref, w.dtype)


def test_forward_features_and_noalloc_head_sizes():
    """Given features (no feature map) at F = 96, M = 48, and the no-allocation
    entry point at D = M = 16, bit-identical to the workspace call."""
    w = _w(513, 1, 3, 2000, 96, 48, "bf16")
    fq, fk, v = wl.forward_inputs(w)
    fq = wl.round_to(np.float32(1.0) + np.float32(0.5) * fq, w.dtype)
    fk = wl.round_to(np.float32(1.0) + np.float32(0.5) * fk, w.dtype)
    _say("forward on given features, F96 M48 bf16; noalloc D16 M16")
    out = la.la_forward_causal_features(dev(fq, w.dtype), dev(fk, w.dtype), dev(v, w.dtype))
    w2 = _w(514, 2, 2, 1500, 16, 16, "f32")
    q2, k2, v2 = (dev(x, w2.dtype) for x in wl.forward_inputs(w2))
    a = la.la_forward_causal_noalloc(q2, k2, v2)
    b = la.la_forward_causal(q2, k2, v2)
    torch.cuda.synchronize()
    check("out on features", host(out), oracle.forward_causal_features(fq, fk, v), w.dtype)
    assert torch.equal(a, b)


@pytest.mark.parametrize("D,M,dtype", [(128, 128, "bf16"), (16, 16, "f32"), (48, 112, "bf16"), (96, 80, "f32"),
                                       (128, 48, "bf16")],
                         ids=["d128m128_bf16", "d16m16_f32", "d48m112_bf16", "d96m80_f32", "d128m48_bf16"])
def test_decode_head_sizes(D, M, dtype):
    w = _w(515, 3, 5, 1, D, M, dtype)
    steps = 50
    qs, ks, vs = wl.DecodeStream(w).take(steps)
    _say(f"decode D{D} M{M} {dtype}: B3 H5, {steps} steps")
    S = torch.zeros((w.B, w.H, D, M), device="cuda")
    Z = torch.zeros((w.B, w.H, D), device="cuda")
    qd, kd, vd = dev(qs, dtype), dev(ks, dtype), dev(vs, dtype)
    outs = torch.stack([la.la_decode_step(qd[t], kd[t], vd[t], S, Z) for t in range(steps)])
    torch.cuda.synchronize()
    tr = lambda x: np.ascontiguousarray(np.moveaxis(x, 0, 2))
    ref, S_ref, Z_ref = oracle.forward_causal(tr(qs), tr(ks), tr(vs), return_state=True)
    check("decode out (per row)", host(outs), np.moveaxis(ref, 2, 0), dtype, lead=3)
    check("decode S", host(S), S_ref, "f32")
    check("decode Z", host(Z), Z_ref, "f32")


BWD_CASES = [
    ("d128m128_bf16", _w(521, 1, 2, 2000, 128, 128, "bf16")),
    ("d16m16_f32_ragged", _w(522, 2, 3, 1001, 16, 16, "f32")),
    ("d48m80_bf16", _w(523, 1, 2, 3000, 48, 80, "bf16")),
    ("d96m32_f32", _w(524, 1, 3, 1500, 96, 32, "f32")),
    ("d112m64_bf16", _w(525, 2, 2, 1000, 112, 64, "bf16")),
    ("d128m16_f32", _w(526, 1, 2, 777, 128, 16, "f32")),
    ("d32m128_bf16_many_segments", _w(527, 1, 2, 40000, 32, 128, "bf16")),
    ("d80m112_f32_one_token", _w(528, 1, 2, 1, 80, 112, "f32")),
    ("d64m48_bf16", _w(529, 1, 4, 2048, 64, 48, "bf16")),
    ("d128m128_f32", _w(530, 1, 2, 1200, 128, 128, "f32")),
    ("d128m16_bf16", _w(532, 1, 2, 1200, 128, 16, "bf16")),   # several pieces per lane, as above
    ("d96m32_bf16_ragged", _w(533, 2, 2, 1333, 96, 32, "bf16")),
    # fp32 at D <= 64 on split operands: a ragged multi-segment case and one token
    ("d48m48_f32_ragged", _w(534, 2, 2, 3001, 48, 48, "f32")),
    ("d48m16_f32_one_token", _w(535, 1, 3, 1, 48, 16, "f32")),
]


def _check_grads(name, w, got, ref):
    dq, dk, dv = (host(x) for x in got)
    if w.N == 1:   # out_1 = V_1: dQ = dK = 0 up to the rounding residue of two equal terms
        from tests.test_gpu_parity import _check_single_token_grads
        q, k, v, g = wl.forward_inputs(w, with_dout=True)
        _check_single_token_grads(q, k, v, g, dq, dk, w.dtype)
        check(f"dv[{name}]", dv, ref[2], w.dtype)
        return
    check(f"dq[{name}]", dq, ref[0], w.dtype, floor=True)
    check(f"dk[{name}]", dk, ref[1], w.dtype, floor=True)
    check(f"dv[{name}]", dv, ref[2], w.dtype)


@pytest.mark.parametrize("name,w", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_backward_causal_head_sizes(name, w):
    q, k, v, g = wl.forward_inputs(w, with_dout=True)
    _say(f"backward causal {name}: B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}")
    got = la.la_backward_causal(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), dev(g, w.dtype))
    torch.cuda.synchronize()
    _check_grads(name, w, got, oracle.backward_causal(q, k, v, g))


@pytest.mark.parametrize("name,w", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_backward_noncausal_head_sizes(name, w):
    q, k, v, g = wl.forward_inputs(w, with_dout=True)
    _say(f"backward non-causal {name}: B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}")
    got = la.la_backward_noncausal(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), dev(g, w.dtype))
    torch.cuda.synchronize()
    _check_grads(name, w, got, oracle.backward_noncausal(q, k, v, g))


def test_backward_head_sizes_deterministic():
    """The groups' partial sums are added in a fixed order: two calls give
    bit-identical gradients."""
    w = _w(531, 1, 2, 3000, 80, 112, "bf16")
    q, k, v, g = (dev(x, w.dtype) for x in wl.forward_inputs(w, with_dout=True))
    _say("backward determinism D80 M112 bf16")
    a = la.la_backward_causal(q, k, v, g)
    b = la.la_backward_causal(q, k, v, g)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_other_kernels_keep_their_head_sizes():
    q = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(la.LAError) as e:
        la.la_forward_causal_poly2(q, q, q)
    assert e.value.status == 2
    with pytest.raises(la.LAError) as e:
        la.la_forward_causal(q[..., :40].contiguous(), q[..., :40].contiguous(), q)
    assert e.value.status == 2
