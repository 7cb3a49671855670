"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every case draws seeded inputs from ``workloads``, runs the library on the GPU
and compares, per (b, h) slice and per output tensor, the normwise relative
error ||gpu - oracle|| / ||oracle|| against 1e-4 (fp32 I/O) or 2e-2 (bf16 I/O).
The five workloads run at their full sizes; extra cases cover ragged tails,
single tokens, mixed head sizes, many segments and stressed inputs.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_util import TOL, check, dev, host

pytestmark = pytest.mark.gpu

la = pytest.importorskip("kernelized_transformer_amd")


def _wl(seed, B, H, N, D, M, dtype, scale=1.0):
    return wl.Workload(seed, f"edge seed {seed}", B, H, N, D, M, dtype, scale)


def _say(*a):
    print("[gpu]", *a, flush=True)


FWD_CASES = [
    ("w1", wl.WORKLOADS[1]),
    ("w2", wl.WORKLOADS[2]),
    ("w3", wl.WORKLOADS[3]),
    ("w4_n4096", wl.WORKLOADS[4].with_n(4096)),
    ("w4_full", wl.WORKLOADS[4]),
    ("n1_f32", _wl(101, 1, 1, 1, 32, 32, "f32")),
    ("n1_bf16", _wl(102, 2, 1, 1, 64, 64, "bf16")),
    ("n17_d32m64", _wl(103, 2, 3, 17, 32, 64, "f32")),
    ("n33_d64m32", _wl(104, 1, 2, 33, 64, 32, "bf16")),
    ("n100_d64m64_f32", _wl(105, 3, 1, 100, 64, 64, "f32")),
    ("n1000_bf16", _wl(106, 1, 1, 1000, 32, 32, "bf16")),
    ("n4097_ragged", _wl(107, 2, 2, 4097, 64, 64, "bf16")),
    ("n200000_many_segments", _wl(108, 1, 1, 200000, 32, 32, "bf16")),
    ("stress_sigma3_f32", _wl(109, 1, 2, 700, 32, 32, "f32", 3.0)),
    ("stress_sigma3_bf16", _wl(110, 1, 2, 700, 64, 64, "bf16", 3.0)),
]


@pytest.mark.parametrize("name,w", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_forward_causal(name, w):
    q, k, v = wl.forward_inputs(w)
    _say(f"forward causal {name}: B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}")
    out = la.la_forward_causal(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype))
    torch.cuda.synchronize()
    ref = oracle.forward_causal(q, k, v)
    check(f"out[{name}]", host(out), ref, w.dtype)


# Plans of the single-launch causal forward (workgroups per (b, h), nb) that
# exercise its cross-workgroup hand-off: nb = 1 (no hand-off, more workgroups
# than CUs), 2, 3 (ragged last workgroup), 7 and 8 (the single exchange at its
# largest), 36, 63 (fp32, D = M = 64) and 64 (the largest; some workgroups own
# an empty slice of the state record).
PLAN_CASES = [
    ("nb64_empty_slices", _wl(181, 1, 1, 262144, 64, 64, "bf16"), 64),
    ("nb63_f32_d64m64", _wl(182, 1, 2, 40000, 64, 64, "f32"), 63),
    ("nb2_128_heads", _wl(183, 8, 16, 4096, 64, 64, "bf16"), 2),
    ("nb3_ragged_96_heads", _wl(184, 6, 16, 3000, 32, 32, "bf16"), 3),
    ("nb1_1024_heads", _wl(185, 64, 16, 512, 32, 64, "bf16"), 1),
    ("nb36_d32m64", _wl(186, 1, 3, 9000, 32, 64, "bf16"), 36),
    # single-exchange hand-off at its largest: 16 workgroups per head halved to 8
    # (a short problem), and 7 with a ragged last workgroup
    ("nb8_halved_b1h8", _wl(187, 1, 8, 2048, 64, 64, "bf16"), 8),
    ("nb7_direct_ragged", _wl(188, 4, 8, 1700, 64, 64, "bf16"), 7),
    ("nb6_halved_f32_d32m64_ragged", _wl(189, 1, 4, 1500, 32, 64, "f32"), 6),
]


def _fused_nb(BH, N, chunk=16, waves=8, cus=256, direct=8):
    """Workgroups per (b, h) the library plans for the causal forward on a
    device with `cus` compute units."""
    assert torch.cuda.get_device_properties(0).multi_processor_count == cus
    max_blk = min(64, cus)
    nch = -(-N // chunk)
    cpw = max(1, -(-BH * nch // (cus * waves)), -(-nch // (waves * max_blk)))
    nb = -(-N // (waves * cpw * chunk))
    if direct < nb <= 2 * direct and BH * nb <= cus // 2:
        cpw = -(-nch // (waves * direct))
        nb = -(-N // (waves * cpw * chunk))
    return nb


@pytest.mark.parametrize("name,w,nb", PLAN_CASES, ids=[c[0] for c in PLAN_CASES])
def test_forward_causal_plans(name, w, nb):
    assert _fused_nb(w.B * w.H, w.N) == nb
    q, k, v = wl.forward_inputs(w)
    _say(f"forward causal plan {name}: B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}, {nb} workgroups per head")
    out = la.la_forward_causal(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype))
    torch.cuda.synchronize()
    ref = oracle.forward_causal(q, k, v)
    check(f"out[{name}]", host(out), ref, w.dtype)


@pytest.mark.parametrize("name,w,nb", PLAN_CASES, ids=[c[0] for c in PLAN_CASES])
def test_forward_noncausal_plans(name, w, nb):
    """The non-causal forward runs the same single-launch plan: every block
    publishes its total and the slice owners sum all of them."""
    assert _fused_nb(w.B * w.H, w.N) == nb
    q, k, v = wl.forward_inputs(w)
    _say(f"forward non-causal plan {name}: B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}, {nb} workgroups per head")
    out = la.la_forward_noncausal(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype))
    torch.cuda.synchronize()
    check(f"out[{name}]", host(out), oracle.forward_noncausal(q, k, v), w.dtype)


NC_CASES = [("w1", wl.WORKLOADS[1]), ("w2_noncausal", wl.WORKLOADS[2]), ("w3_noncausal", wl.WORKLOADS[3]),
            ("w4_full_noncausal", wl.WORKLOADS[4]),
            ("n1", _wl(111, 1, 1, 1, 32, 32, "f32")), ("n77_d64m32", _wl(112, 2, 2, 77, 64, 32, "bf16")),
            ("n5000_f32", _wl(113, 1, 3, 5000, 64, 64, "f32"))]


@pytest.mark.parametrize("name,w", NC_CASES, ids=[c[0] for c in NC_CASES])
def test_forward_noncausal(name, w):
    q, k, v = wl.forward_inputs(w)
    _say(f"forward non-causal {name}: B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}")
    out = la.la_forward_noncausal(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype))
    torch.cuda.synchronize()
    ref = oracle.forward_noncausal(q, k, v)
    check(f"out[{name}]", host(out), ref, w.dtype)


def test_causal_last_row_equals_noncausal():
    w = _wl(114, 2, 2, 999, 64, 64, "f32")
    q, k, v = (dev(x, w.dtype) for x in wl.forward_inputs(w))
    _say("causal last row == non-causal last row")
    oc = host(la.la_forward_causal(q, k, v))
    onc = host(la.la_forward_noncausal(q, k, v))
    assert np.abs(oc[:, :, -1] - onc[:, :, -1]).max() <= 1e-5 * np.abs(onc[:, :, -1]).max()


BWD_CASES = [
    ("w1_shape", wl.WORKLOADS[1]),
    ("w2_shape", wl.WORKLOADS[2]),
    ("w3_shape_b2h2", wl.WORKLOADS[3].with_shape(B=2, H=2)),
    ("w4_n4096", wl.WORKLOADS[4].with_n(4096)),
    ("w4_full", wl.WORKLOADS[4]),
    ("n1", _wl(121, 1, 2, 1, 32, 32, "f32")),
    ("n17_d32m64", _wl(122, 2, 1, 17, 32, 64, "f32")),
    ("n50_d64m32_bf16", _wl(123, 1, 3, 50, 64, 32, "bf16")),
    ("n3001_ragged_f32", _wl(124, 1, 2, 3001, 64, 64, "f32")),
    ("n100000_many_segments", _wl(125, 1, 1, 100000, 32, 32, "bf16")),
    # bf16 at D = 64 runs two wavefronts per segment: one token, a partial
    # chunk, ragged multi-segment and the M = 32 variant
    ("n1_d64_bf16", _wl(126, 1, 2, 1, 64, 64, "bf16")),
    ("n17_d64m64_bf16", _wl(127, 2, 3, 17, 64, 64, "bf16")),
    ("n3001_ragged_bf16", _wl(128, 1, 2, 3001, 64, 64, "bf16")),
    ("n20000_d64m32_bf16", _wl(129, 2, 2, 20000, 64, 32, "bf16")),
    # many heads: one segment per head (the segment plan's other extreme)
    ("h256_n300_d64_bf16", _wl(141, 4, 64, 300, 64, 64, "bf16")),
    ("h512_n40_d32m64_f32", _wl(142, 8, 64, 40, 32, 64, "f32")),
]


@pytest.mark.parametrize("name,w", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_backward_causal(name, w):
    q, k, v, g = wl.forward_inputs(w, with_dout=True)
    _say(f"backward causal {name}: B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}")
    dq, dk, dv = la.la_backward_causal(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), dev(g, w.dtype))
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward_causal(q, k, v, g)
    if w.N == 1:   # out_1 = V_1: dQ = dK = 0, dV = dout
        _check_single_token_grads(q, k, v, g, host(dq), host(dk), w.dtype)
        check(f"dv[{name}]", host(dv), rv, w.dtype)
        return
    check(f"dq[{name}]", host(dq), rq, w.dtype, floor=True)
    check(f"dk[{name}]", host(dk), rk, w.dtype, floor=True)
    check(f"dv[{name}]", host(dv), rv, w.dtype)


def _check_single_token_grads(q, k, v, g, dq, dk, dtype):
    """One token: out_1 = V_1 whatever q and k are, so dQ = dK = 0 exactly.
    The kernels form them as the difference of two equal terms,
    dphi(q) = phi(k) (g.v - g.out) / d and dphi(k) = phi(q) (g.v - g.out) / d
    with d = phi(q).phi(k), from operands rounded to the I/O type, so what
    remains is a rounding residue of those terms: per element at most
    8 u phi(k)_d phi'(q)_d sum_m |g_m v_m| / d (and the same with q and k
    swapped), u = 2^-8 for bf16 and 2^-16 for fp32, whose operands enter the
    matrix products split into bf16 hi + lo parts within 2^-16 of each value
    (a few roundings of each term, with room to spare)."""
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -16
    pq, dpq = oracle.feature_map(q)
    pk, dpk = oracle.feature_map(k)
    d = (pq * pk).sum(-1, keepdims=True)
    gv = np.abs(g.astype(np.float64) * v.astype(np.float64)).sum(-1, keepdims=True)
    bq = 8 * u * pk * dpq * gv / d
    bk = 8 * u * pq * dpk * gv / d
    print(f"  single token: max |dQ| / bound {np.max(np.abs(dq) / bq):.3f}, "
          f"max |dK| / bound {np.max(np.abs(dk) / bk):.3f}", flush=True)
    assert (np.abs(dq) <= bq).all() and (np.abs(dk) <= bk).all()


BWD_NC_CASES = [
    ("w1", wl.WORKLOADS[1]),
    ("w3", wl.WORKLOADS[3]),
    ("w4_full", wl.WORKLOADS[4]),
    ("n1_bf16", _wl(201, 2, 2, 1, 64, 64, "bf16")),
    ("n17_d32m64_f32", _wl(202, 2, 3, 17, 32, 64, "f32")),
    ("n50_d64m32_bf16", _wl(203, 1, 3, 50, 64, 32, "bf16")),
    ("n3001_ragged_f32", _wl(204, 1, 2, 3001, 64, 64, "f32")),
    ("n100000_many_segments", _wl(205, 1, 1, 100000, 32, 32, "bf16")),
    # bf16 at D = 64: two wavefronts per segment
    ("n3001_ragged_bf16", _wl(206, 1, 2, 3001, 64, 64, "bf16")),
    ("n20000_d64m32_bf16", _wl(207, 2, 2, 20000, 64, 32, "bf16")),
    ("h256_n300_d64_bf16", _wl(143, 4, 64, 300, 64, 64, "bf16")),
]


@pytest.mark.parametrize("name,w", BWD_NC_CASES, ids=[c[0] for c in BWD_NC_CASES])
def test_backward_noncausal(name, w):
    q, k, v, g = wl.forward_inputs(w, with_dout=True)
    _say(f"backward non-causal {name}: B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}")
    dq, dk, dv = la.la_backward_noncausal(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), dev(g, w.dtype))
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward_noncausal(q, k, v, g)
    if w.N == 1:
        _check_single_token_grads(q, k, v, g, host(dq), host(dk), w.dtype)
        check(f"dv[{name}]", host(dv), rv, w.dtype)
        return
    check(f"dq[{name}]", host(dq), rq, w.dtype, floor=True)
    check(f"dk[{name}]", host(dk), rk, w.dtype, floor=True)
    check(f"dv[{name}]", host(dv), rv, w.dtype)


def _decode_run(w, steps, sample=None):
    stream = wl.DecodeStream(w)
    qs, ks, vs = stream.take(steps)
    S = torch.zeros((w.B, w.H, w.D, w.M), dtype=torch.float32, device="cuda")
    Z = torch.zeros((w.B, w.H, w.D), dtype=torch.float32, device="cuda")
    dq_, dk_, dv_ = dev(qs, w.dtype), dev(ks, w.dtype), dev(vs, w.dtype)
    outs = torch.empty((steps, w.B, w.H, w.M), dtype=dq_.dtype, device="cuda")
    for t in range(steps):
        la.la_decode_step(dq_[t], dk_[t], dv_[t], S, Z, out=outs[t])
    torch.cuda.synchronize()
    return qs, ks, vs, host(outs), host(S), host(Z)


def test_decode_small_f32():
    w = _wl(131, 2, 3, 1, 32, 64, "f32")
    _say("decode small f32: B2 H3 D32 M64, 80 steps")
    qs, ks, vs, outs, S, Z = _decode_run(w, 80)
    So = np.zeros((w.B, w.H, w.D, w.M))
    Zo = np.zeros((w.B, w.H, w.D))
    ref = np.stack([oracle.decode_step(qs[t], ks[t], vs[t], So, Zo) for t in range(80)])
    check("decode out", outs, ref, "f32", lead=3)
    check("decode S", S, So, "f32")
    check("decode Z", Z, Zo, "f32")


@pytest.mark.parametrize("D,M", [(64, 32), (32, 64)])
def test_decode_small_bf16_mixed_head_sizes(D, M):
    w = _wl(144, 3, 2, 1, D, M, "bf16")
    _say(f"decode small bf16: B3 H2 D{D} M{M}, 60 steps")
    qs, ks, vs, outs, S, Z = _decode_run(w, 60)
    So = np.zeros((w.B, w.H, w.D, w.M))
    Zo = np.zeros((w.B, w.H, w.D))
    ref = np.stack([oracle.decode_step(qs[t], ks[t], vs[t], So, Zo) for t in range(60)])
    check("decode out", outs, ref, "bf16", lead=3)
    check("decode S", S, So, "f32")
    check("decode Z", Z, Zo, "f32")


def test_decode_full_workload_all_streams():
    """All 3072 steps of all 2048 streams (B256 H8 D=M=64 bf16 I/O, fp32
    state): every step's output row against the oracle's causal forward over
    the stream's stacked steps (the oracle's decode step equals its forward,
    a pinned invariant), each row gated on its own, and the final S and Z of
    every stream."""
    w = wl.WORKLOADS[5]
    _say(f"decode full workload: B{w.B} H{w.H} D{w.D} M{w.M} {w.dtype}, {w.steps} steps")
    qs, ks, vs, outs, S, Z = _decode_run(w, w.steps)
    tr = lambda x: np.ascontiguousarray(np.moveaxis(x, 0, 2))   # [T, B, H, F] -> [B, H, T, F]
    ref, S_ref, Z_ref = oracle.forward_causal(tr(qs), tr(ks), tr(vs), return_state=True)
    del qs, ks, vs
    check("decode out (every stream, every step, per row)", outs, np.moveaxis(ref, 2, 0), w.dtype, lead=3)
    del outs, ref
    check("decode S (every stream)", S, S_ref, "f32")
    check("decode Z (every stream)", Z, Z_ref, "f32")


def test_decode_equals_forward_on_gpu():
    w = _wl(132, 1, 4, 1, 64, 64, "f32")
    T = 300
    _say("decode == causal forward on the stacked sequence")
    qs, ks, vs, outs, _, _ = _decode_run(w, T)
    tr = lambda x: np.ascontiguousarray(np.moveaxis(x, 0, 2))
    fwd = host(la.la_forward_causal(dev(tr(qs), "f32"), dev(tr(ks), "f32"), dev(tr(vs), "f32")))
    np.testing.assert_allclose(np.moveaxis(outs, 0, 2), fwd, rtol=0, atol=2e-5 * np.abs(fwd).max())


# Causal forward carrying the recurrent state across calls: the sequence is
# cut into consecutive pieces; the first call starts from zero and returns
# its final state, each later one continues from it in place.  The joined
# outputs and the last state must match one oracle pass over the whole
# sequence.
STATE_CHAIN_CASES = [
    ("two_pieces_f32_nb1", _wl(191, 2, 3, 300, 32, 64, "f32"), [0, 97, 300]),
    ("two_pieces_bf16_many_blocks", _wl(192, 1, 2, 40000, 64, 64, "bf16"), [0, 12345, 40000]),
    ("four_pieces_bf16_single_token", _wl(193, 4, 4, 5000, 32, 32, "bf16"), [0, 1, 2049, 2050, 5000]),
    ("three_pieces_f32_d64m32", _wl(194, 2, 2, 9000, 64, 32, "f32"), [0, 4500, 4517, 9000]),
]


@pytest.mark.parametrize("name,w,cuts", STATE_CHAIN_CASES, ids=[c[0] for c in STATE_CHAIN_CASES])
def test_forward_state_chain(name, w, cuts):
    q, k, v = wl.forward_inputs(w)
    _say(f"forward state chain {name}: B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}, cuts {cuts}")
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


@pytest.mark.parametrize("name,w", [("bf16_24_blocks", _wl(195, 2, 2, 3000, 64, 64, "bf16")),
                                    ("f32_one_block", _wl(196, 1, 3, 100, 32, 32, "f32"))],
                         ids=["bf16_24_blocks", "f32_one_block"])
def test_forward_state_arbitrary_start(name, w):
    """A start state that no prefix produced (S0 of any sign): outputs and
    final state against the oracle started from the same state; with a null
    final state the outputs are bit-identical."""
    q, k, v = wl.forward_inputs(w)
    S0, Z0 = wl.start_state(w, seed=w.wid + 1000)
    _say(f"forward from an arbitrary state {name}: B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}")
    qd, kd, vd = (dev(x, w.dtype) for x in (q, k, v))
    s0, z0 = dev(S0, "f32"), dev(Z0, "f32")
    out, S1, Z1 = la.la_forward_causal_state(qd, kd, vd, s0=s0, z0=z0)
    out2 = torch.empty_like(out)
    nws = la.la_workspace_size(la.LA_OP_FWD_CAUSAL, w.B, w.H, w.N, w.D, w.M, qd.dtype)
    ws = torch.empty((nws,), dtype=torch.uint8, device="cuda")
    st = la.load().la_forward_causal_state(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out2.data_ptr(),
                                           s0.data_ptr(), z0.data_ptr(), None, None, w.B, w.H, w.N, w.D, w.M,
                                           1 if w.dtype == "bf16" else 0, ws.data_ptr(), nws,
                                           torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    ref, S_ref, Z_ref = oracle.forward_causal(q, k, v, S0=S0, Z0=Z0, return_state=True)
    check(f"out[{name}]", host(out), ref, w.dtype)
    check(f"S_N[{name}]", host(S1), S_ref, w.dtype)
    check(f"Z_N[{name}]", host(Z1), Z_ref, w.dtype)
    assert torch.equal(out, out2)
    assert torch.equal(s0, dev(S0, "f32")) and torch.equal(z0, dev(Z0, "f32"))   # inputs untouched


def test_forward_state_null_and_zero_start_equal_plain_forward():
    w = _wl(197, 2, 4, 6000, 64, 64, "bf16")
    q, k, v = (dev(x, w.dtype) for x in wl.forward_inputs(w))
    _say("state entry point with no / zero start state == la_forward_causal (bitwise)")
    plain = la.la_forward_causal(q, k, v)
    a, _, _ = la.la_forward_causal_state(q, k, v)
    zs = torch.zeros((w.B, w.H, w.D, w.M), device="cuda")
    zz = torch.zeros((w.B, w.H, w.D), device="cuda")
    b, _, _ = la.la_forward_causal_state(q, k, v, s0=zs, z0=zz)
    torch.cuda.synchronize()
    assert torch.equal(plain, a) and torch.equal(plain, b)


def test_forward_state_then_decode():
    """A prompt's forward hands its final state to decode: the decoded
    outputs continue the forward over the whole sequence."""
    w = _wl(198, 2, 4, 1050, 64, 64, "bf16")
    P = 1000
    q, k, v = wl.forward_inputs(w)
    _say(f"prompt forward (N={P}) then {w.N - P} decode steps, bf16")
    qd, kd, vd = (dev(np.ascontiguousarray(x[:, :, :P]), w.dtype) for x in (q, k, v))
    out_p, S, Z = la.la_forward_causal_state(qd, kd, vd)
    steps = []
    for t in range(P, w.N):
        qt, kt, vt = (dev(np.ascontiguousarray(x[:, :, t]), w.dtype) for x in (q, k, v))
        steps.append((qt, kt, vt, la.la_decode_step(qt, kt, vt, S, Z)))
    torch.cuda.synchronize()
    ref = oracle.forward_causal(q, k, v)
    check("prompt out", host(out_p), ref[:, :, :P], w.dtype)
    check("decoded out", np.stack([host(s[3]) for s in steps], axis=2), ref[:, :, P:], w.dtype)


def test_forward_state_full_long_sequence():
    """Final state of the long-sequence workload (B1 H8 N65536 D=M=64 bf16)."""
    w = wl.WORKLOADS[4]
    q, k, v = wl.forward_inputs(w)
    _say(f"final state, full long-sequence workload B{w.B} H{w.H} N{w.N}")
    out, S, Z = la.la_forward_causal_state(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype))
    torch.cuda.synchronize()
    ref, S_ref, Z_ref = oracle.forward_causal(q, k, v, return_state=True)
    check("out", host(out), ref, w.dtype)
    check("S_N", host(S), S_ref, w.dtype)
    check("Z_N", host(Z), Z_ref, w.dtype)


# Random Fourier features and the causal forward on given features.
RFF_CASES = [
    ("w1_r32_f32", wl.WORKLOADS[1], 32),
    ("d32_r64_f32_ragged", _wl(211, 2, 3, 100, 32, 32, "f32"), 64),
    ("d64_r32_bf16_ragged", _wl(212, 1, 3, 1001, 64, 64, "bf16"), 32),
    ("w4_full_r64", wl.WORKLOADS[4], 64),
    # bf16 rows staged through LDS: D = 32 rows (one 16-byte piece per lane), fewer
    # rows than one 16-row tile, and a last wavefront with a partial tile
    ("d32_r64_bf16_ragged", _wl(214, 2, 2, 777, 32, 32, "bf16"), 64),
    ("d32_r32_bf16_5_rows", _wl(215, 1, 1, 5, 32, 32, "bf16"), 32),
    ("d64_r64_f32_ragged", _wl(216, 1, 2, 333, 64, 64, "f32"), 64),
]


@pytest.mark.parametrize("name,w,R", RFF_CASES, ids=[c[0] for c in RFF_CASES])
def test_rff_features(name, w, R):
    x, _, _ = wl.forward_inputs(w)
    om, b = wl.rff_params(w.D, R, seed=w.wid + 2000)
    _say(f"rff features {name}: B{w.B} H{w.H} N{w.N} D{w.D} R{R} {w.dtype}")
    got = la.la_rff_features(dev(x, w.dtype), dev(om, "f32"), dev(b, "f32"))
    torch.cuda.synchronize()
    check(f"features[{name}]", host(got), oracle.rff_features(x, om, b), w.dtype)


@pytest.mark.parametrize("name,w,R", RFF_CASES, ids=[c[0] for c in RFF_CASES])
def test_rff_attention(name, w, R):
    """The causal forward on random Fourier features: given the oracle's
    features (rounded to the I/O type) the GPU forward matches the oracle's
    forward on the same features; and the whole GPU path (features, then
    forward) matches the oracle's whole path from the same q, k, v, omega, b."""
    q, k, v = wl.forward_inputs(w)
    om, b = wl.rff_params(w.D, R, seed=w.wid + 2000)
    _say(f"rff attention {name}: B{w.B} H{w.H} N{w.N} D{w.D} R{R} M{w.M} {w.dtype}")
    fq_o, fk_o = oracle.rff_features(q, om, b), oracle.rff_features(k, om, b)
    fq_r, fk_r = wl.round_to(fq_o, w.dtype), wl.round_to(fk_o, w.dtype)
    vd = dev(v, w.dtype)
    out_given = la.la_forward_causal_features(dev(fq_r, w.dtype), dev(fk_r, w.dtype), vd)
    omd, bd = dev(om, "f32"), dev(b, "f32")
    fq_g = la.la_rff_features(dev(q, w.dtype), omd, bd)
    fk_g = la.la_rff_features(dev(k, w.dtype), omd, bd)
    out_path = la.la_forward_causal_features(fq_g, fk_g, vd)
    torch.cuda.synchronize()
    check(f"out on given features[{name}]", host(out_given), oracle.forward_causal_features(fq_r, fk_r, v), w.dtype)
    check(f"out, whole path[{name}]", host(out_path), oracle.forward_causal_features(fq_o, fk_o, v), w.dtype)


@pytest.mark.parametrize("name,w", [("mixed_sign_bf16_many_blocks", _wl(213, 1, 2, 40000, 64, 64, "bf16")),
                                    ("mixed_sign_f32_d32m64", _wl(214, 2, 2, 777, 32, 64, "f32"))],
                         ids=["mixed_sign_bf16_many_blocks", "mixed_sign_f32_d32m64"])
def test_forward_features_mixed_sign(name, w):
    """Given features of either sign (1 + 0.6 N(0, 1), about 5% negative) with
    positive denominators: no feature map may be applied to them."""
    fq, fk, v = wl.forward_inputs(w)
    fq = wl.round_to(np.float32(1.0) + np.float32(0.6) * fq, w.dtype)
    fk = wl.round_to(np.float32(1.0) + np.float32(0.6) * fk, w.dtype)
    assert (fq < 0).any() and (fk < 0).any()
    _say(f"forward on mixed-sign features {name}: B{w.B} H{w.H} N{w.N} F{w.D} M{w.M} {w.dtype}")
    out = la.la_forward_causal_features(dev(fq, w.dtype), dev(fk, w.dtype), dev(v, w.dtype))
    torch.cuda.synchronize()
    check(f"out[{name}]", host(out), oracle.forward_causal_features(fq, fk, v), w.dtype)


# Degree-2 polynomial kernel (q . k)^2, D, M in {32, 64}.
POLY_CASES = [
    ("w1_f32", wl.WORKLOADS[1]),
    ("w2_f32", wl.WORKLOADS[2]),
    ("w3_bf16", wl.WORKLOADS[3]),
    ("n1_bf16_m64", _wl(221, 2, 2, 1, 32, 64, "bf16")),
    ("n17_f32_m64", _wl(222, 1, 3, 17, 32, 64, "f32")),
    ("n1001_ragged_bf16_m64", _wl(223, 2, 3, 1001, 32, 64, "bf16")),
    ("n100000_many_segments", _wl(224, 1, 1, 100000, 32, 32, "bf16")),
    ("long_b1h8n65536_d32", _wl(225, 1, 8, 65536, 32, 32, "bf16")),
    ("d64_n1_bf16", _wl(226, 2, 2, 1, 64, 64, "bf16")),
    ("d64_n33_f32_m32", _wl(227, 1, 2, 33, 64, 32, "f32")),
    ("d64_n700_ragged_f32", _wl(228, 2, 2, 700, 64, 64, "f32")),
    ("d64_n1500_bf16_m32", _wl(229, 1, 3, 1500, 64, 32, "bf16")),
    ("d64_b8h8n512_single_segment_bf16", _wl(230, 8, 8, 512, 64, 64, "bf16")),
]


@pytest.mark.parametrize("name,w", POLY_CASES, ids=[c[0] for c in POLY_CASES])
def test_forward_causal_poly2(name, w):
    q, k, v = wl.forward_inputs(w)
    _say(f"polynomial forward {name}: B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}")
    out = la.la_forward_causal_poly2(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype))
    torch.cuda.synchronize()
    check(f"out[{name}]", host(out), oracle.forward_causal_poly2(q, k, v), w.dtype)


def _poly_rows(N, seg, n_random, seed):
    """Rows to check on a long sequence: both ends, the chunk edges of the
    first tokens, both sides of every multiple of seg, and random rows."""
    rng = np.random.default_rng(seed)
    rows = {0, 1, 15, 16, 31, 32, 33, N - 2, N - 1}
    for b in range(seg, N, seg):
        rows.update({b - 1, b, b + 1})
    rows.update(int(x) for x in rng.integers(0, N, n_random))
    return np.array(sorted(r for r in rows if 0 <= r < N))


@pytest.mark.parametrize("name,w,seg", [
    ("b1h8n65536_d64m64_bf16", _wl(231, 1, 8, 65536, 64, 64, "bf16"), 4096),
    ("b1h1n20000_d64m64_f32_many_segments", _wl(232, 1, 1, 20000, 64, 64, "f32"), 160),
    ("b1h2n30011_d64m32_bf16", _wl(233, 1, 2, 30011, 64, 32, "bf16"), 256),
], ids=["b1h8n65536_d64m64_bf16", "b1h1n20000_d64m64_f32_many_segments", "b1h2n30011_d64m32_bf16"])
def test_forward_causal_poly2_long_sampled(name, w, seg):
    """Long sequences at D = 64, where the oracle's D^2 feature recurrence
    would take minutes: every output row of the kernel is computed, and
    sampled rows (both ends, both sides of multiples of the segment length,
    random rows) are checked one by one against the kernel summed directly,
    each row under the same relative tolerance."""
    q, k, v = wl.forward_inputs(w)
    _say(f"polynomial forward {name}: B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}, sampled rows")
    out = la.la_forward_causal_poly2(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype))
    torch.cuda.synchronize()
    got = host(out)
    assert np.isfinite(got).all()
    rows = _poly_rows(w.N, seg, 48, w.wid)
    ref = oracle.forward_causal_poly2_rows(q, k, v, rows)
    check(f"out[{name}] rows", got[:, :, rows], ref, w.dtype, lead=3)


NONCAUSAL_POLY_CASES = [
    ("w1_f32", wl.WORKLOADS[1]),
    ("d32m64_n1001_ragged_bf16", _wl(241, 2, 3, 1001, 32, 64, "bf16")),
    ("d64m32_n700_f32", _wl(242, 1, 2, 700, 64, 32, "f32")),
    ("d64m64_b8h8n512_single_segment_bf16", _wl(243, 8, 8, 512, 64, 64, "bf16")),
    ("d32_n1_bf16", _wl(244, 2, 2, 1, 32, 32, "bf16")),
]


@pytest.mark.parametrize("name,w", NONCAUSAL_POLY_CASES, ids=[c[0] for c in NONCAUSAL_POLY_CASES])
def test_forward_noncausal_poly2(name, w):
    q, k, v = wl.forward_inputs(w)
    _say(f"polynomial non-causal forward {name}: B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}")
    out = la.la_forward_noncausal_poly2(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype))
    torch.cuda.synchronize()
    check(f"out[{name}]", host(out), oracle.forward_noncausal_poly2(q, k, v), w.dtype)


def test_forward_noncausal_poly2_long_sampled():
    """B1 H8 N65536 D = M = 32 (several segments, their totals summed by the
    scan): every row computed, sampled rows checked against the kernel summed
    over all keys."""
    w = _wl(245, 1, 8, 65536, 32, 32, "bf16")
    q, k, v = wl.forward_inputs(w)
    _say("polynomial non-causal forward B1 H8 N65536 D32 M32 bf16, sampled rows")
    out = la.la_forward_noncausal_poly2(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype))
    torch.cuda.synchronize()
    got = host(out)
    assert np.isfinite(got).all()
    rows = _poly_rows(w.N, 2048, 32, w.wid)
    check("out rows", got[:, :, rows], oracle.forward_noncausal_poly2_rows(q, k, v, rows), w.dtype, lead=3)


@pytest.mark.parametrize("D,M,dtype,n0,steps", [(32, 32, "bf16", 3000, 40), (64, 64, "f32", 777, 20),
                                                (32, 64, "bf16", 0, 30), (64, 32, "bf16", 1, 25)],
                         ids=["d32m32_bf16", "d64m64_f32", "d32m64_bf16_from_zero", "d64m32_bf16_one_token"])
def test_poly2_state_then_decode(D, M, dtype, n0, steps):
    """A prompt of n0 tokens through la_forward_causal_poly2_state, then
    `steps` decode steps from its final state: the outputs of both equal the
    causal forward over the whole sequence (n0 = 0: decode from a zero
    state)."""
    w = _wl(250 + D + M + n0 % 7, 2, 3, n0 + steps, D, M, dtype)
    q, k, v = wl.forward_inputs(w)
    _say(f"polynomial state + decode D{D} M{M} {dtype}: B2 H3 prompt {n0}, {steps} steps")
    ref = oracle.forward_causal_poly2(q, k, v)
    nst = la.la_poly2_state_floats(D, M)
    if n0 > 0:
        out0, state = la.la_forward_causal_poly2_state(*(dev(np.ascontiguousarray(x[:, :, :n0]), dtype)
                                                          for x in (q, k, v)))
    else:
        state = torch.zeros((w.B, w.H, nst), dtype=torch.float32, device="cuda")
    qd, kd, vd = (dev(np.ascontiguousarray(np.moveaxis(x[:, :, n0:], 2, 0)), dtype) for x in (q, k, v))
    outs = torch.stack([la.la_decode_step_poly2(qd[t], kd[t], vd[t], state) for t in range(steps)])
    torch.cuda.synchronize()
    if n0 > 0:
        check("prompt out", host(out0), ref[:, :, :n0], dtype)
    check("decode out (per row)", host(outs), np.moveaxis(ref[:, :, n0:], 2, 0), dtype, lead=3)
    assert nst > 0 and np.isfinite(host(state)).all()


def test_forward_causal_longest_sequence():
    """One head of 2^20 tokens (64 workgroups of 8 wavefronts, 2048 tokens
    each), checked element by element, with its final state."""
    w = _wl(231, 1, 1, 1 << 20, 32, 32, "bf16")
    q, k, v = wl.forward_inputs(w)
    _say(f"longest sequence: B1 H1 N{w.N} D32 M32 bf16")
    out, S, Z = la.la_forward_causal_state(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype))
    torch.cuda.synchronize()
    ref, S_ref, Z_ref = oracle.forward_causal(q, k, v, return_state=True)
    check("out", host(out), ref, w.dtype)
    check("S_N", host(S), S_ref, w.dtype)
    check("Z_N", host(Z), Z_ref, w.dtype)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
def test_backward_longest_head_identities(causal):
    """The backward on one head of the longest length its two-wavefront
    kernels take (N * 64 < 2^31 elements: byte offsets into the head pass 2^31),
    checked through identities that hold at any length (the oracle would need
    hours): out_i is 0-homogeneous in phi(q_i) and in all phi(k) together, so
    s_i = sum_d dQ_id (1 + max(Q_id, 0)) = 0 for every token and the same sum over
    dK is 0 for the head; out is an average of the V rows, so sum_j dV_j =
    sum_i G_i and sum_j V_j . dV_j = sum_i G_i . out_i.  Each bound is 2^-5 of the
    summed magnitudes of the terms: eight bf16 roundings, since several roundings
    act systematically here (the reverse state, rounded to bf16 once per chunk,
    changes slowly along the sequence, so its rounding error repeats over many
    tokens); random rows of the right scale exceed it about fourfold.  The dQ
    identity is checked per block of 4096 tokens (sum of |s_i| against the summed
    magnitudes): a single token's s_i is a rounding residue of two cancelling terms
    (token 1's whole dQ is one), but any block of wrong rows breaks it.  Every
    output starts as NaN, so rows a kernel failed to write cannot pass as zeros.
    Inputs are seeded N(0, 1) draws made on the device.  The non-causal form
    satisfies the same identities with every sum over the whole sequence, but
    there every token's dV is read from one reverse state rounded to bf16 once,
    and each column's dV keeps one sign along the sequence, so the sum over
    tokens keeps that rounding undiluted (3-5% of sum |dV| at every length from
    2^20 tokens up, measured): the sum of dV is checked for the causal form only."""
    N = (2 ** 31 - 1) // 64
    _say(f"longest backward head ({'causal' if causal else 'non-causal'}): B1 H1 N{N} D=M=64 bf16")
    gen = torch.Generator(device="cuda").manual_seed(241)

    def draw():
        return torch.randn((1, 1, N, 64), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)

    q, k, v, g = draw(), draw(), draw(), draw()
    dq, dk, dv, out = (torch.full_like(q, float("nan")) for _ in range(4))
    (la.la_backward_causal if causal else la.la_backward_noncausal)(q, k, v, g, dq=dq, dk=dk, dv=dv)
    (la.la_forward_causal if causal else la.la_forward_noncausal)(q, k, v, out=out)
    torch.cuda.synchronize()
    for name, x in (("dQ", dq), ("dK", dk), ("dV", dv), ("out", out)):
        assert bool(torch.isfinite(x).all()), f"{name}: rows left unwritten or non-finite"
    tol = 2.0 ** -5
    sum_dv = torch.zeros(64, dtype=torch.float64, device="cuda")
    abs_dv = torch.zeros(64, dtype=torch.float64, device="cuda")
    sum_g = torch.zeros(64, dtype=torch.float64, device="cuda")
    vdv = gout = abs_vdv = abs_gout = dkr = abs_dkr = 0.0
    worst_q = 0.0
    step = 1 << 22
    for t0 in range(0, N, step):
        sl = slice(t0, min(N, t0 + step))
        f = lambda x: x[0, 0, sl].double()
        Q, K, V, G, DQ, DK, DV, O = (f(x) for x in (q, k, v, g, dq, dk, dv, out))
        tq = DQ * (1 + Q.clamp(min=0))
        si, ai = tq.sum(1).abs(), tq.abs().sum(1)
        nb = (si.numel() + 4095) // 4096
        pad = nb * 4096 - si.numel()
        si = torch.nn.functional.pad(si, (0, pad)).view(nb, 4096).sum(1)
        ai = torch.nn.functional.pad(ai, (0, pad)).view(nb, 4096).sum(1)
        worst_q = max(worst_q, float((si / (tol * ai + 1e-30)).max()))
        tk = DK * (1 + K.clamp(min=0))
        dkr += float(tk.sum()); abs_dkr += float(tk.abs().sum())
        sum_dv += DV.sum(0); abs_dv += DV.abs().sum(0); sum_g += G.sum(0)
        vdv += float((V * DV).sum()); abs_vdv += float((V * DV).abs().sum())
        gout += float((G * O).sum()); abs_gout += float((G * O).abs().sum())
    print(f"  dQ identity per 4096 tokens: worst sum |s_i| / bound {worst_q:.3f}", flush=True)
    assert worst_q <= 1.0
    print(f"  dK identity: |sum| / bound {abs(dkr) / (tol * abs_dkr):.3e}", flush=True)
    assert abs(dkr) <= tol * abs_dkr
    ratio = (sum_dv - sum_g).abs() / (tol * abs_dv)
    print(f"  sum dV - sum G per column: worst |difference| / bound {float(ratio.max()):.3f}", flush=True)
    if causal:
        assert float(ratio.max()) <= 1.0
    print(f"  V.dV - G.out: |difference| / bound {abs(vdv - gout) / (tol * (abs_vdv + abs_gout)):.3e}", flush=True)
    assert abs(vdv - gout) <= tol * (abs_vdv + abs_gout)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_causal_closed_forms(dtype):
    """Constant V gives V back; identical keys give the running mean of V
    whatever Q is (closed forms of the method, no oracle involved)."""
    w = _wl(232, 2, 3, 5000, 64, 64, dtype)
    q, k, v = wl.forward_inputs(w)
    _say(f"closed forms on the GPU, {dtype}")
    vc = np.broadcast_to(v[:, :, :1], v.shape).copy()
    out_c = host(la.la_forward_causal(dev(q, dtype), dev(k, dtype), dev(vc, dtype)))
    ks = np.broadcast_to(k[:, :, :1], k.shape).copy()
    out_k = host(la.la_forward_causal(dev(q, dtype), dev(ks, dtype), dev(v, dtype)))
    torch.cuda.synchronize()
    check("constant V", out_c, vc.astype(np.float64), dtype)
    mean = np.cumsum(v.astype(np.float64), axis=2) / np.arange(1, w.N + 1)[None, None, :, None]
    check("identical keys", out_k, mean, dtype)


def test_forward_deterministic_and_guarded():
    w = _wl(141, 2, 3, 1500, 64, 64, "bf16")
    q, k, v = (dev(x, w.dtype) for x in wl.forward_inputs(w))
    _say("determinism + guard bands, forward and backward")
    n = w.B * w.H * w.N * w.M
    pad = 4096
    buf = torch.full((n + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = buf[pad:pad + n].view(w.B, w.H, w.N, w.M)
    la.la_forward_causal(q, k, v, out=out)
    a = out.clone()
    la.la_forward_causal(q, k, v, out=out)
    torch.cuda.synchronize()
    assert torch.equal(a, out)
    assert (buf[:pad] == 7.0).all() and (buf[pad + n:] == 7.0).all()
    g = dev(wl.forward_inputs(w, with_dout=True)[3], w.dtype)
    r1 = la.la_backward_causal(q, k, v, g)
    r2 = la.la_backward_causal(q, k, v, g)
    torch.cuda.synchronize()
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)


def test_fused_forward_error_word_clear():
    """The causal forward's cross-workgroup waits report a time-out by or-ing
    1 into word 1 of the workspace; after a normal call it stays clear."""
    w = _wl(171, 1, 4, 100000, 64, 64, "bf16")
    q, k, v = (dev(x, w.dtype) for x in wl.forward_inputs(w))
    _say("fused forward error word")
    n = la.la_workspace_size(la.LA_OP_FWD_CAUSAL, w.B, w.H, w.N, w.D, w.M, torch.bfloat16)
    ws = torch.zeros((n,), dtype=torch.uint8, device="cuda")
    la.la_forward_causal(q, k, v, workspace=ws)
    torch.cuda.synchronize()
    words = ws[:8].view(torch.int32).cpu().tolist()
    assert words[1] == 0, words


def test_fused_forward_workspace_needs_no_clearing():
    """Garbage in the workspace (including words left by an earlier call with
    another shape, or a backward call) never reads as a published flag:
    results are bit-identical to those with a fresh zeroed workspace."""
    w = _wl(172, 1, 8, 20000, 64, 64, "bf16")
    q, k, v = (dev(x, w.dtype) for x in wl.forward_inputs(w))
    _say("fused forward garbage workspace")
    n = la.la_workspace_size(la.LA_OP_FWD_CAUSAL, w.B, w.H, w.N, w.D, w.M, torch.bfloat16)
    ref = la.la_forward_causal(q, k, v, workspace=torch.zeros((n,), dtype=torch.uint8, device="cuda"))
    ws = torch.full((n,), 0x55, dtype=torch.uint8, device="cuda")
    out1 = la.la_forward_causal(q, k, v, workspace=ws)              # garbage flags
    out2 = la.la_forward_causal(q, k, v, workspace=ws)              # flags of the previous call
    w2 = _wl(173, 1, 2, 30000, 64, 64, "bf16")                      # another plan in the same bytes
    q2, k2, v2 = (dev(x, w2.dtype) for x in wl.forward_inputs(w2))
    la.la_forward_causal(q2, k2, v2, workspace=ws[:la.la_workspace_size(la.LA_OP_FWD_CAUSAL, 1, 2, 30000, 64, 64,
                                                                           torch.bfloat16)])
    out3 = la.la_forward_causal(q, k, v, workspace=ws)
    # the non-causal forward uses the same flags: alternate with the causal one in the same bytes
    nc_ref = la.la_forward_noncausal(q, k, v, workspace=torch.zeros((n,), dtype=torch.uint8, device="cuda"))
    nc1 = la.la_forward_noncausal(q, k, v, workspace=ws)
    out4 = la.la_forward_causal(q, k, v, workspace=ws)
    torch.cuda.synchronize()
    for o in (out1, out2, out3, out4):
        assert torch.equal(o, ref)
    assert torch.equal(nc1, nc_ref)


def test_segment_plan_independence():
    """A head computed alone and inside a large batch (different segment cuts)
    gives the same result up to fp32 rounding."""
    w = _wl(151, 8, 8, 2048, 32, 32, "f32")
    q, k, v = (dev(x, w.dtype) for x in wl.forward_inputs(w))
    _say("segment plan independence")
    full = host(la.la_forward_causal(q, k, v))
    one = host(la.la_forward_causal(q[3:4, 5:6].contiguous(), k[3:4, 5:6].contiguous(), v[3:4, 5:6].contiguous()))
    assert np.abs(full[3:4, 5:6] - one).max() <= 1e-5 * np.abs(one).max()


def test_invalid_arguments_leave_outputs_untouched():
    w = _wl(161, 1, 2, 64, 32, 32, "f32")
    q, k, v = (dev(x, w.dtype) for x in wl.forward_inputs(w))
    _say("error paths on the GPU")
    out = torch.full((1, 2, 64, 32), 3.0, device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(la.LAError) as e:
        la.la_forward_causal(q, k, v, out=out, workspace=small)
    assert e.value.status == 3
    with pytest.raises(la.LAError) as e:
        la.la_forward_causal(q, k, v, out=q)   # output aliases an input
    assert e.value.status == 1
    torch.cuda.synchronize()
    assert (out == 3.0).all()


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
def test_forward_graph_replays(causal):
    """A forward captured into a HIP graph, replayed with new inputs copied
    into the captured tensors: every replay equals an eager call on the same
    inputs (bitwise), with eager calls on the same workspace in between.  The
    captured call clears its hand-off flags first, so a replay never reads its
    predecessor's flags (which hold the same tag)."""
    w = _wl(175, 1, 8, 20000, 64, 64, "bf16")   # 32 workgroups per head: the sliced hand-off
    _say(f"graph replays ({'causal' if causal else 'non-causal'}): B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}")
    sets = [tuple(dev(x, w.dtype) for x in wl.forward_inputs(w, seed=s)) for s in (175, 176, 177)]
    q, k, v = (torch.empty_like(t) for t in sets[0])
    out = torch.empty((w.B, w.H, w.N, w.M), dtype=q.dtype, device="cuda")
    op = la.LA_OP_FWD_CAUSAL if causal else la.LA_OP_FWD_NONCAUSAL
    ws = torch.empty((la.la_workspace_size(op, w.B, w.H, w.N, w.D, w.M, q.dtype),), dtype=torch.uint8, device="cuda")
    f = la.la_forward_causal if causal else la.la_forward_noncausal
    for dst, src in zip((q, k, v), sets[0]):
        dst.copy_(src)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        f(q, k, v, out=out, workspace=ws)
    for rep in (0, 1, 2, 1):
        for dst, src in zip((q, k, v), sets[rep]):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = f(*sets[rep], workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"replay with input set {rep} differs from the eager call"
    del g


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("D", [64, 128], ids=["d64", "d128"])
def test_backward_graph_replays(causal, D):
    """A backward captured into a HIP graph and replayed with new inputs
    copied into the captured tensors gives, on every replay, exactly the
    gradients of an eager call on the same inputs and workspace (eager calls
    in between), for the two-wavefront kernels (D = 64) and the column-group
    kernels (D = 128).  The backward keeps no state between calls: every
    workspace word it reads it wrote earlier in the same call."""
    w = _wl(178, 1, 4, 6000, D, D, "bf16")
    _say(f"backward graph replays ({'causal' if causal else 'non-causal'}): B{w.B} H{w.H} N{w.N} D{w.D} M{w.M}")
    sets = [tuple(dev(x, w.dtype) for x in wl.forward_inputs(w, with_dout=True, seed=s)) for s in (178, 179, 180)]
    q, k, v, g = (torch.empty_like(t) for t in sets[0])
    grads = tuple(torch.empty_like(t) for t in (q, k, v))
    op = la.LA_OP_BWD_CAUSAL if causal else la.LA_OP_BWD_NONCAUSAL
    ws = torch.empty((la.la_workspace_size(op, w.B, w.H, w.N, w.D, w.M, q.dtype),), dtype=torch.uint8, device="cuda")
    f = la.la_backward_causal if causal else la.la_backward_noncausal
    for dst, src in zip((q, k, v, g), sets[0]):
        dst.copy_(src)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        f(q, k, v, g, *grads, workspace=ws)
    for rep in (0, 1, 2, 1):
        for dst, src in zip((q, k, v, g), sets[rep]):
            dst.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        got = tuple(x.clone() for x in grads)
        ref = f(*sets[rep], workspace=ws)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), f"{name}: replay with input set {rep} differs from the eager call"
    del graph


def test_forward_graph_replays_head_size_128():
    """The column-group forward (head size 128) captured into a graph: every
    replay equals an eager call on the same inputs (its records are written
    before they are read in each call)."""
    w = _wl(181, 1, 4, 6000, 128, 128, "bf16")
    _say(f"graph replays (head size 128): B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}")
    sets = [tuple(dev(x, w.dtype) for x in wl.forward_inputs(w, seed=s)) for s in (181, 182, 183)]
    q, k, v = (torch.empty_like(t) for t in sets[0])
    out = torch.empty((w.B, w.H, w.N, w.M), dtype=q.dtype, device="cuda")
    ws = torch.empty((la.la_workspace_size(la.LA_OP_FWD_CAUSAL, w.B, w.H, w.N, w.D, w.M, q.dtype),),
                     dtype=torch.uint8, device="cuda")
    for dst, src in zip((q, k, v), sets[0]):
        dst.copy_(src)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        la.la_forward_causal(q, k, v, out=out, workspace=ws)
    for rep in (0, 1, 2, 1):
        for dst, src in zip((q, k, v), sets[rep]):
            dst.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = la.la_forward_causal(*sets[rep], workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"replay with input set {rep} differs from the eager call"
    del graph


def test_forward_wait_give_up_is_reported():
    """With the wait limit at 0 every hand-off wait gives up at once: the
    kernels still exit, the call returns LA_OK, and la_workspace_check reports
    LA_ERR_TIMEOUT (the binding's checked mode raises it); with the default
    limit restored the same workspace gives the normal result and a clear
    word."""
    w = _wl(176, 1, 8, 20000, 64, 64, "bf16")
    q, k, v = (dev(x, w.dtype) for x in wl.forward_inputs(w))
    _say("forced wait give-up reported through la_workspace_check")
    n = la.la_workspace_size(la.LA_OP_FWD_CAUSAL, w.B, w.H, w.N, w.D, w.M, q.dtype)
    ws = torch.empty((n,), dtype=torch.uint8, device="cuda")
    ref = la.la_forward_causal(q, k, v)
    out = torch.empty_like(ref)
    lib = la.load()
    la.la_workspace_check(ws, clear=True)
    prev = la.la_set_wait_limit(0)
    try:
        for fn in (lib.la_forward_causal, lib.la_forward_noncausal):
            st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), w.B, w.H, w.N, w.D, w.M, 1,
                    ws.data_ptr(), n, torch.cuda.current_stream().cuda_stream)
            assert st == 0
            torch.cuda.synchronize()
            assert la.la_workspace_check(ws, clear=True) == la.LA_ERR_TIMEOUT
        if la.CHECK_WAITS:
            with pytest.raises(la.LAError) as e:
                la.la_forward_causal(q, k, v, out=out, workspace=ws)
            assert e.value.status == la.LA_ERR_TIMEOUT
    finally:
        la.la_set_wait_limit(prev)
    la.la_workspace_check(ws, clear=True)
    la.la_forward_causal(q, k, v, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert la.la_workspace_check(ws) == 0
    assert torch.equal(out, ref)
