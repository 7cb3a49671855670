"""The GPU parity gate itself, on the CPU: errors planted in the oracle's own
outputs must fail it wherever along the sequence they sit.

The outputs of causal linear attention shrink like 1/sqrt(i) along the
sequence, so a normwise error over a whole (b, h) slice barely sees the late
rows: on the long-sequence workload (B1 H8 N65536 D=M=64 bf16) a 5% error in
the last 2048 rows of a head (the rows the last workgroup's cross-workgroup
hand-off feeds) stays far below the bf16 tolerance of 2e-2 in that metric.
The per-16-row-chunk gate of ``gpu_util.check`` catches it, and a single
wrong 16-row chunk anywhere, and a planted error in the last rows of dQ with
the floor used for gradients.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import TOL, check, chunk_rel, normwise_rel


@pytest.fixture(scope="module")
def long_out():
    w = wl.WORKLOADS[4]
    q, k, v = wl.forward_inputs(w)
    return oracle.forward_causal(q, k, v)


def _planted(ref, rows, factor=1.05, head=3):
    x = ref.copy()
    x[0, head, rows] *= factor
    return x


def test_gate_passes_the_oracle_itself(long_out):
    check("oracle vs itself", long_out, long_out, "bf16")


def test_gate_catches_late_rows(long_out):
    x = _planted(long_out, slice(-2048, None))
    # the slice metric alone would pass it
    assert normwise_rel(x, long_out) < 0.25 * TOL["bf16"]
    e, sl, row = chunk_rel(x, long_out)
    assert e == pytest.approx(0.05, rel=1e-9) and sl == 3 and row >= 65536 - 2048
    with pytest.raises(AssertionError, match="chunk rel err"):
        check("planted: last 2048 rows +5%", x, long_out, "bf16")


def test_gate_catches_one_chunk(long_out):
    x = _planted(long_out, slice(40000, 40016), factor=1.03)
    assert normwise_rel(x, long_out) < 0.01 * TOL["bf16"]
    with pytest.raises(AssertionError, match="rows 40000..40015 of slice 3"):
        check("planted: one chunk +3%", x, long_out, "bf16")


def test_gate_catches_ragged_tail():
    w = wl.Workload(3, "ragged", 1, 2, 1000, 32, 32, "f32")
    q, k, v = wl.forward_inputs(w)
    ref = oracle.forward_causal(q, k, v)
    x = ref.copy()
    x[0, 1, 992:] += 3e-4 * np.abs(ref[0, 1, 992:]).max()   # the 8-row partial chunk
    assert normwise_rel(x, ref) < TOL["f32"]
    with pytest.raises(AssertionError, match="rows 992..1007 of slice 1"):
        check("planted: ragged tail", x, ref, "f32")


def test_gate_floor_for_gradients():
    """dQ, dK with the floor: errors in the late rows (whose norms are far
    below the slice's mean) and in one chunk still fail."""
    w = wl.WORKLOADS[4].with_n(16384)
    q, k, v, g = wl.forward_inputs(w, with_dout=True)
    dq, dk, _ = oracle.backward_causal(q, k, v, g)
    for name, ref in (("dq", dq), ("dk", dk)):
        check(f"{name} vs itself", ref, ref, "bf16", floor=True)
        for rows in (slice(-2048, None), slice(16384 - 2048, 16384 - 2032)):
            x = _planted(ref, rows)
            with pytest.raises(AssertionError, match="chunk rel err"):
                check(f"planted {name}", x, ref, "bf16", floor=True)
