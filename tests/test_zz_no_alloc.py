"""la_forward_causal_noalloc, the causal forward on the library's own static
scratch (for callers that cannot allocate), against la_forward_causal with a
caller workspace: bit-identical outputs (same kernels, same plan), on calls in
a row whose second is smaller than the first (the scratch keeps the first
call's contents) and a third that is larger again; the small case is also
gated against the oracle."""
from __future__ import annotations

import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_util import check, dev, host

pytestmark = pytest.mark.gpu

la = pytest.importorskip("kernelized_transformer_amd")


def test_noalloc_equals_workspace_forward():
    cases = [(wl.WORKLOADS[4], 401),                                          # B1 H8 N65536 D=M=64 bf16
             (wl.Workload(402, "smaller", 2, 3, 3001, 32, 64, "f32"), 402),   # second call: smaller
             (wl.Workload(403, "larger", 1, 4, 40000, 64, 32, "bf16"), 403)]
    for w, seed in cases:
        print(f"[gpu] noalloc forward: B{w.B} H{w.H} N{w.N} D{w.D} M{w.M} {w.dtype}", flush=True)
        q, k, v = wl.forward_inputs(w, seed=seed)
        qd, kd, vd = dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype)
        got = la.la_forward_causal_noalloc(qd, kd, vd)
        ref = la.la_forward_causal(qd, kd, vd)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        if w.N <= 4000:
            check("noalloc out", host(got), oracle.forward_causal(q, k, v), w.dtype)


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    q = torch.empty((1, 255, 32768, 64), dtype=torch.bfloat16, device="cuda")
    need = la.la_workspace_size(la.LA_OP_FWD_CAUSAL, 1, 255, 32768, 64, 64, torch.bfloat16)
    assert need > 16 * 2 ** 20
    with pytest.raises(la.LAError) as e:
        la.la_forward_causal_noalloc(q, q, q, out=torch.empty_like(q))
    assert e.value.status == 3
