"""Benchmark of the kernelized linear-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-sweep]

Headline (``value``): causal forward throughput in tokens*heads/s on the long
sequence workload B=1, H=8, N=65536, D=M=64, bf16 I/O, fp32 state.  One step
is one la_forward_causal call over the whole batch, inputs already resident
in HBM; two input sets alternate so that consecutive steps do not re-read the
same 268 MB from the 256 MB Infinity Cache.  Per-call medians over at least 20
calls are reported beside it: alternating inputs, cold (512 MB of scratch
written before each call, which evicts the Infinity Cache) and warm (the same
input again).

In the same run, each timed with HIP events on the stream the library launches
on, and reported next to the headline:
  * decode: 3072 sequential la_decode_step calls for B=256 streams x H=8 heads,
    D=M=64 (steps/s), eager launches and a replayed HIP graph of the same calls;
  * backward: la_backward_causal and la_backward_noncausal on the long-sequence
    workload;
  * non-causal forward on the long-sequence workload;
  * random Fourier features (R = 64) of q and k and the causal forward on them;
  * the degree-2 polynomial kernel: causal and non-causal at D = M = 32,
    causal at D = M = 64;
  * the causal forward from a start state, returning the final state, on the
    long-sequence workload;
  * a head size outside {32, 64}: causal forward and backward at B=1, H=8,
    N=16384, D=M=128 bf16 (the 16-column-group path);
  * the causal forward of the three smaller workloads, and the causal backward
    of the 784-token fp32 one;
  * the causal forward at B=1, H=8, D=M=64 bf16 for N = 512 .. 65536 (the
    sweep; --no-sweep leaves it out).
``roofline`` relates the forward's algorithmic HBM bytes (Q, K, V read once,
out written once: 512 B per token*head) to its measured time against the
MI355X HBM peak of 8 TB/s.  ``cpu_baseline`` times the fp64 oracle on the host
cores over the full long-sequence workload, as a reference point only.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-passes", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--only", choices=["all", "forward", "decode", "backward", "rff", "poly", "noncausal", "sweep", "small",
                                       "headsize"],
                    default="all",
                    help="restrict the timed work (for profiling runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB device to device three times (a plain copy kernel of known size, "
                         "to scale the FETCH_SIZE / WRITE_SIZE counters of a profiling run)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn the counter CSVs of two profiling runs made with --copy-calibration "
                         "into per-launch HBM bytes of the causal forward kernel, and print them")
    return ap.parse_args()


# Sources of the causal forward kernel: a stored traffic figure is used only
# while these are unchanged.
KERNEL_SOURCES = ["kernelized_transformer_amd/csrc/" + f for f in
                  ("la_forward.hip", "la_chunk.h", "la_device.h", "la_internal.h")]
TRAFFIC_FILE = "profiles/forward_causal_B1H8N65536_D64M64_bf16.md"


def kernel_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic():
    """Per-launch HBM bytes of k_fwd_fused from the committed counter summary,
    or None when the kernel sources have changed since it was taken."""
    try:
        text = open(os.path.join(ROOT, TRAFFIC_FILE)).read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if line.startswith("traffic_bytes_per_launch:") or line.startswith("source_sha256:"):
            k_, v_ = line.split(":", 1)
            vals[k_.strip()] = v_.strip().strip("`")
    if vals.get("source_sha256") != kernel_sources_sha256():
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def traffic_from(fetch_csv: str, write_csv: str, copy_mib: int = 1024) -> dict:
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the forward kernel, each
    scaled by bytes / counter of the plain copy kernel in the same run."""
    import csv

    def per_kernel(path, counter):
        out = {}
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return out

    res = {}
    for name, path, counter in (("read", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        rows = per_kernel(path, counter)
        copy = [v for k_, vs in rows.items() if "copyBuffer" in k_ for v in vs]   # the runtime's device copy
        fused = [v for k_, vs in rows.items() if "k_fwd_fused" in k_ for v in vs]
        copy_bytes = copy_mib * 2 ** 20
        big = [v for v in copy if v > 0.25 * copy_bytes]      # the calibration copies, not small copies
        factor = copy_bytes / (sum(big) / len(big))
        res[name] = dict(counter_bytes=sum(fused) / len(fused), copy_counter_bytes=sum(big) / len(big),
                         factor=factor, bytes=sum(fused) / len(fused) * factor)
    res["traffic_bytes_per_launch"] = int(round(res["read"]["bytes"] + res["write"]["bytes"]))
    res["source_sha256"] = kernel_sources_sha256()
    return res


def main():
    a = _args()
    if a.traffic_from:
        print(json.dumps(traffic_from(*a.traffic_from, copy_mib=a.copy_calibration or 1024), indent=1))
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build targets one GPU; the path shards by (batch, head) with no communication, "
              "but only --gpus 1 is measured.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kernelized_transformer_amd as la
    import workloads as wl

    lib = la.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    def to_dev(x, dtype):
        t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)
        return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32).contiguous()

    def log(*m):
        print("[bench]", *m, file=sys.stderr, flush=True)

    if a.copy_calibration:
        src = torch.empty(a.copy_calibration * 2 ** 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"calibration: copied {a.copy_calibration} MiB three times")

    def time_events(fn, iters):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(iters):
            fn(i)
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / 1e3

    def time_each(fn, iters, between=None):
        """Per-call durations (s): one event pair around each call; ``between``
        runs outside the pairs (e.g. a cache flush)."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        torch.cuda.synchronize()
        for i in range(iters):
            if between is not None:
                between()
            ev[i][0].record(stream)
            fn(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) / 1e3 for e0, e1 in ev]

    def med(xs):
        xs = sorted(xs)
        n = len(xs)
        return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])

    # Writing 512 MB of scratch evicts the 256 MB Infinity Cache (and every L2).
    flush_buf = [None]

    def flush():
        if flush_buf[0] is None:
            flush_buf[0] = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device=dev)
        flush_buf[0].fill_(7)

    # ---- forward on the long-sequence workload ----------------------------------
    w4 = wl.WORKLOADS[4]
    BH = w4.B * w4.H
    tok_heads = BH * w4.N
    fwd_bytes = tok_heads * (2 * w4.D + w4.M) * 2 + tok_heads * w4.M * 2      # 512 B / token*head
    fwd_flops = tok_heads * (4 * w4.D * w4.M + 4 * w4.D)                      # recurrence form
    results = {}
    log("generating long-sequence inputs")
    sets = []
    for seed in (4, 40):
        q, k, v, g = wl.forward_inputs(w4, with_dout=True, seed=seed)
        sets.append(tuple(to_dev(x, "bf16") for x in (q, k, v, g)))
    out = torch.empty((w4.B, w4.H, w4.N, w4.M), dtype=torch.bfloat16, device=dev)
    ws_f = torch.empty(max(la.la_workspace_size(op, w4.B, w4.H, w4.N, w4.D, w4.M, torch.bfloat16)
                           for op in (la.LA_OP_FWD_CAUSAL, la.LA_OP_FWD_NONCAUSAL)), dtype=torch.uint8, device=dev)

    def fwd(i, causal=True):
        q, k, v, _ = sets[i % 2]
        f = lib.la_forward_causal if causal else lib.la_forward_noncausal
        st = f(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), w4.B, w4.H, w4.N, w4.D, w4.M,
               la.LA_DTYPE_BF16, ws_f.data_ptr(), ws_f.numel(), sptr)
        if st != 0:
            raise la.LAError("forward", st)

    if a.only in ("all", "forward"):
        for i in range(a.warmup):
            fwd(i)
        t = time_events(fwd, a.steps)
        ms = t / a.steps * 1e3
        results["forward"] = dict(seconds=t, ms_per_step=ms, tok_heads_per_s=tok_heads * a.steps / t)
        log(f"causal forward: {ms:.4f} ms/step, {tok_heads * a.steps / t:.4e} tokens*heads/s")
        # same input every step (Infinity Cache may hold part of it): reported, not the headline
        t_same = time_events(lambda i: fwd(0), a.steps)
        results["forward_same_input"] = dict(ms_per_step=t_same / a.steps * 1e3,
                                             tok_heads_per_s=tok_heads * a.steps / t_same)
        # medians over per-call event pairs: alternating inputs, cold (caches
        # flushed before each call), warm (the same input again)
        reps = max(20, a.steps)
        t_alt = med(time_each(fwd, reps))
        t_cold = med(time_each(fwd, reps, between=flush))
        t_warm = med(time_each(lambda i: fwd(0), reps))
        results["forward_median"] = {
            k_: dict(ms=t_ * 1e3, tok_heads_per_s=tok_heads / t_, hbm_frac=fwd_bytes / t_ / 1e9 / HBM_PEAK_GBS)
            for k_, t_ in (("alternating", t_alt), ("cold", t_cold), ("warm", t_warm))}
        results["forward_median"]["reps"] = reps
        log(f"causal forward medians over {reps}: alternating {t_alt * 1e3:.4f}, cold {t_cold * 1e3:.4f}, "
            f"warm {t_warm * 1e3:.4f} ms")
        # the same forward from a start state, returning the final state (a
        # prompt handed to decode, or one piece of a cut sequence): the states
        # are read and written in fp32 beside Q, K, V and out
        gen = torch.Generator(device=dev).manual_seed(44)
        s0 = torch.randn((w4.B, w4.H, w4.D, w4.M), generator=gen, device=dev)
        z0 = torch.rand((w4.B, w4.H, w4.D), generator=gen, device=dev) + 0.5
        s1, z1 = torch.empty_like(s0), torch.empty_like(z0)

        def fwd_state(i):
            q, k, v, _ = sets[i % 2]
            st = lib.la_forward_causal_state(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), s0.data_ptr(),
                                             z0.data_ptr(), s1.data_ptr(), z1.data_ptr(), w4.B, w4.H, w4.N, w4.D,
                                             w4.M, la.LA_DTYPE_BF16, ws_f.data_ptr(), ws_f.numel(), sptr)
            if st != 0:
                raise la.LAError("forward_state", st)

        for i in range(2):
            fwd_state(i)
        t = time_events(fwd_state, a.steps)
        state_bytes = 2 * BH * (w4.D * w4.M + w4.D) * 4
        results["forward_state"] = dict(ms_per_call=t / a.steps * 1e3, tok_heads_per_s=tok_heads * a.steps / t,
                                        algorithmic_bytes=fwd_bytes + state_bytes,
                                        hbm_frac=(fwd_bytes + state_bytes) / (t / a.steps) / 1e9 / HBM_PEAK_GBS)
        log(f"causal forward from a start state, final state out: {t / a.steps * 1e3:.4f} ms/call")
        del s0, z0, s1, z1

    # ---- backward / non-causal on the long-sequence workload --------------------------
    if a.only in ("all", "backward"):
        dq, dk, dv = (torch.empty_like(sets[0][0]), torch.empty_like(sets[0][1]), torch.empty_like(sets[0][2]))
        ws_b = torch.empty(la.la_workspace_size(la.LA_OP_BWD_CAUSAL, w4.B, w4.H, w4.N, w4.D, w4.M, torch.bfloat16),
                           dtype=torch.uint8, device=dev)

        def bwd(i):
            q, k, v, g = sets[i % 2]
            st = lib.la_backward_causal(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), dq.data_ptr(),
                                        dk.data_ptr(), dv.data_ptr(), w4.B, w4.H, w4.N, w4.D, w4.M, la.LA_DTYPE_BF16,
                                        ws_b.data_ptr(), ws_b.numel(), sptr)
            if st != 0:
                raise la.LAError("backward", st)

        for i in range(2):
            bwd(i)
        nb = max(5, a.steps // 4)
        t = time_events(bwd, nb)
        bwd_bytes = tok_heads * (2 * w4.D + 2 * w4.M) * 2 + tok_heads * (2 * w4.D + w4.M) * 2   # 896 B
        results["backward"] = dict(ms_per_call=t / nb * 1e3, tok_heads_per_s=tok_heads * nb / t,
                                   algorithmic_bytes=bwd_bytes,
                                   hbm_frac=bwd_bytes / (t / nb) / 1e9 / HBM_PEAK_GBS)
        reps = max(20, nb)
        t_alt = med(time_each(bwd, reps))
        t_cold = med(time_each(bwd, reps, between=flush))
        results["backward"]["median"] = {"reps": reps, "alternating_ms": t_alt * 1e3, "cold_ms": t_cold * 1e3}
        log(f"causal backward: {t / nb * 1e3:.4f} ms/call; medians over {reps}: alternating "
            f"{t_alt * 1e3:.4f}, cold {t_cold * 1e3:.4f} ms")
        ws_nb = torch.empty(la.la_workspace_size(la.LA_OP_BWD_NONCAUSAL, w4.B, w4.H, w4.N, w4.D, w4.M,
                                                 torch.bfloat16), dtype=torch.uint8, device=dev)

        def bwd_nc(i):
            q, k, v, g = sets[i % 2]
            st = lib.la_backward_noncausal(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), dq.data_ptr(),
                                           dk.data_ptr(), dv.data_ptr(), w4.B, w4.H, w4.N, w4.D, w4.M,
                                           la.LA_DTYPE_BF16, ws_nb.data_ptr(), ws_nb.numel(), sptr)
            if st != 0:
                raise la.LAError("backward_noncausal", st)

        for i in range(2):
            bwd_nc(i)
        t = time_events(bwd_nc, nb)
        results["backward_noncausal"] = dict(ms_per_call=t / nb * 1e3, tok_heads_per_s=tok_heads * nb / t,
                                             hbm_frac=bwd_bytes / (t / nb) / 1e9 / HBM_PEAK_GBS)
        log(f"non-causal backward: {t / nb * 1e3:.4f} ms/call")
        del dq, dk, dv, ws_b, ws_nb
    if a.only in ("all", "rff"):
        # random Fourier features (R = 64) of q and k, then the causal forward on them
        om, bias = wl.rff_params(w4.D, 64, seed=4004)
        omd, bd = to_dev(om, "f32"), to_dev(bias, "f32")
        fq = torch.empty((w4.B, w4.H, w4.N, 64), dtype=torch.bfloat16, device=dev)
        fk = torch.empty_like(fq)

        def feats(i):
            q, k, _, _ = sets[i % 2]
            for x, f in ((q, fq), (k, fk)):
                st = lib.la_rff_features(x.data_ptr(), omd.data_ptr(), bd.data_ptr(), f.data_ptr(), w4.B, w4.H, w4.N,
                                         w4.D, 64, la.LA_DTYPE_BF16, sptr)
                if st != 0:
                    raise la.LAError("rff_features", st)

        def rff_fwd(i):
            feats(i)
            v = sets[i % 2][2]
            st = lib.la_forward_causal_features(fq.data_ptr(), fk.data_ptr(), v.data_ptr(), out.data_ptr(), w4.B,
                                                w4.H, w4.N, 64, w4.M, la.LA_DTYPE_BF16, ws_f.data_ptr(), ws_f.numel(),
                                                sptr)
            if st != 0:
                raise la.LAError("forward_causal_features", st)

        for i in range(2):
            rff_fwd(i)
        nr = max(5, a.steps // 2)
        t_all = time_events(rff_fwd, nr)
        t_feat = time_events(feats, nr)
        feat_bytes = 2 * tok_heads * (w4.D + 64) * 2        # read q (k), write its features, bf16
        results["rff_forward"] = dict(
            ms_per_call=t_all / nr * 1e3, tok_heads_per_s=tok_heads * nr / t_all,
            features_ms_per_call=t_feat / nr * 1e3,
            features_hbm_frac=feat_bytes / (t_feat / nr) / 1e9 / HBM_PEAK_GBS,
            note="R = 64 random Fourier features of q and k (two la_rff_features calls), then "
                 "la_forward_causal_features on them; features materialized in HBM")
        log(f"rff forward: {t_all / nr * 1e3:.4f} ms/call (features {t_feat / nr * 1e3:.4f} ms)")
        del fq, fk

    if a.only in ("all", "poly"):
        # degree-2 polynomial kernel (q . k)^2 on the long-sequence length, D = M = 32 (the causal and the
        # non-causal form) and D = M = 64.  Algorithmic flops per token*head: the recurrence on the pages'
        # map vec(x x^T) (D^2 features): 4 D^2 (M + 1) (update and readout, numerator and normalizer);
        # the kernels run it on the D (D + 1) / 2 distinct products, 4 D (D + 1) / 2 (M + 1) flops, which
        # is reported beside it (executed_mfma_frac).
        def poly_case(D, M, causal, reps):
            wp = wl.Workload(4, f"polynomial kernel, B1 H8 N65536 D={D} M={M} bf16", 1, 8, w4.N, D, M, "bf16")
            qp, kp, vp = (to_dev(x, "bf16") for x in wl.forward_inputs(wp))
            op = torch.empty_like(vp)
            opc = la.LA_OP_FWD_CAUSAL_POLY2 if causal else la.LA_OP_FWD_NONCAUSAL_POLY2
            wsp = torch.empty(la.la_workspace_size(opc, wp.B, wp.H, wp.N, D, M, torch.bfloat16),
                              dtype=torch.uint8, device=dev)
            fn = lib.la_forward_causal_poly2 if causal else lib.la_forward_noncausal_poly2

            def call(i):
                st = fn(qp.data_ptr(), kp.data_ptr(), vp.data_ptr(), op.data_ptr(), wp.B, wp.H, wp.N, D, M,
                        la.LA_DTYPE_BF16, wsp.data_ptr(), wsp.numel(), sptr)
                if st != 0:
                    raise la.LAError("forward_causal_poly2" if causal else "forward_noncausal_poly2", st)

            for i in range(2):
                call(i)
            t = time_events(call, reps)
            th = wp.B * wp.H * wp.N
            # non-causal: the totals (update) and the readout each once per token, as in the causal form
            flops = th * 4 * D * D * (M + 1)
            flops_exec = th * 4 * (D * (D + 1) // 2) * (M + 1)
            ms = t / reps * 1e3
            del qp, kp, vp, op, wsp
            return dict(workload=wp.name, causal=causal, ms_per_call=ms, tok_heads_per_s=th * reps / t,
                        algorithmic_flops=flops, mfma_frac=flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                        executed_flops=flops_exec,
                        executed_mfma_frac=flops_exec / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS)

        npl = max(5, a.steps // 2)
        results["poly2_forward"] = poly_case(32, 32, True, npl)
        results["poly2_forward"]["note"] = (
            "mfma_frac counts the recurrence on the D^2 features of vec(x x^T); the kernels use the "
            "D(D+1)/2 distinct products (executed_mfma_frac)")
        log(f"polynomial forward D=M=32: {results['poly2_forward']['ms_per_call']:.4f} ms/call")
        results["poly2_forward_noncausal"] = poly_case(32, 32, False, npl)
        log(f"polynomial non-causal forward D=M=32: {results['poly2_forward_noncausal']['ms_per_call']:.4f} ms/call")
        results["poly2_forward_d64"] = poly_case(64, 64, True, max(3, npl // 4))
        log(f"polynomial forward D=M=64: {results['poly2_forward_d64']['ms_per_call']:.4f} ms/call")

        # its gradient at D = M = 32: the forward again (out, d), then two passes over D x D sums per
        # column m, each with a readout and an update: 4 D^2 (M + 1) flops for the forward and
        # 8 D^2 (M + 1) for the passes per token*head on the D^2 count
        def poly_bwd_case(D, M, reps):
            wp = wl.Workload(4, f"polynomial kernel gradient, B1 H8 N65536 D={D} M={M} bf16", 1, 8, w4.N, D, M,
                             "bf16")
            qp, kp, vp, gp = (to_dev(x, "bf16") for x in wl.forward_inputs(wp, with_dout=True))
            dqp, dkp, dvp = torch.empty_like(qp), torch.empty_like(kp), torch.empty_like(vp)
            wsp = torch.empty(la.la_workspace_size(la.LA_OP_BWD_CAUSAL_POLY2, wp.B, wp.H, wp.N, D, M,
                                                   torch.bfloat16), dtype=torch.uint8, device=dev)

            def call(i):
                st = lib.la_backward_causal_poly2(qp.data_ptr(), kp.data_ptr(), vp.data_ptr(), gp.data_ptr(),
                                                  dqp.data_ptr(), dkp.data_ptr(), dvp.data_ptr(), wp.B, wp.H, wp.N,
                                                  D, M, la.LA_DTYPE_BF16, wsp.data_ptr(), wsp.numel(), sptr)
                if st != 0:
                    raise la.LAError("backward_causal_poly2", st)

            for i in range(2):
                call(i)
            t = time_events(call, reps)
            th = wp.B * wp.H * wp.N
            flops = th * 12 * D * D * (M + 1)
            ms = t / reps * 1e3
            del qp, kp, vp, gp, dqp, dkp, dvp, wsp
            return dict(workload=wp.name, ms_per_call=ms, tok_heads_per_s=th * reps / t, algorithmic_flops=flops,
                        mfma_frac=flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                        note="flops: 12 D^2 (M + 1) per token*head (forward again, then the two passes)")

        results["poly2_backward"] = poly_bwd_case(32, 32, max(3, npl // 4))
        log(f"polynomial backward D=M=32: {results['poly2_backward']['ms_per_call']:.4f} ms/call")

    if a.only in ("all", "noncausal"):
        for i in range(2):
            fwd(i, causal=False)
        t = time_events(lambda i: fwd(i, causal=False), a.steps)
        results["noncausal"] = dict(ms_per_call=t / a.steps * 1e3, tok_heads_per_s=tok_heads * a.steps / t,
                                    algorithmic_bytes=fwd_bytes,
                                    hbm_frac=fwd_bytes / (t / a.steps) / 1e9 / HBM_PEAK_GBS)
        log(f"non-causal forward: {t / a.steps * 1e3:.4f} ms/call")

    # ---- smaller forward workloads and the N sweep --------------------------------------
    def fwd_rate(w, seed=None, iters=20):
        q, k, v = (to_dev(x, w.dtype) for x in wl.forward_inputs(w, seed=seed))
        o = torch.empty((w.B, w.H, w.N, w.M), dtype=q.dtype, device=dev)
        dtc = la.LA_DTYPE_BF16 if w.dtype == "bf16" else la.LA_DTYPE_F32
        ws = torch.empty(max(1, la.la_workspace_size(0, w.B, w.H, w.N, w.D, w.M, dtc)), dtype=torch.uint8, device=dev)

        def f(i):
            st = lib.la_forward_causal(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), w.B, w.H, w.N, w.D,
                                       w.M, dtc, ws.data_ptr(), ws.numel(), sptr)
            if st != 0:
                raise la.LAError("forward", st)

        for i in range(3):
            f(i)
        t = time_events(f, iters)
        th = w.B * w.H * w.N
        by = th * ((2 * w.D + w.M) + w.M) * (2 if w.dtype == "bf16" else 4)
        return dict(us_per_call=t / iters * 1e6, tok_heads_per_s=th * iters / t,
                    hbm_frac=by / (t / iters) / 1e9 / HBM_PEAK_GBS)

    if a.only in ("all", "headsize"):
        # a head size outside {32, 64}: the column-group path, forward and backward
        wg = wl.Workload(12, "head size 128, B1 H8 N16384 D=M=128 bf16", 1, 8, 16384, 128, 128, "bf16")
        qg, kg, vg, gg = (to_dev(x, "bf16") for x in wl.forward_inputs(wg, with_dout=True))
        og = torch.empty_like(vg)
        dqg, dkg, dvg = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(vg)
        wsf = torch.empty(la.la_workspace_size(la.LA_OP_FWD_CAUSAL, 1, 8, wg.N, 128, 128, torch.bfloat16),
                          dtype=torch.uint8, device=dev)
        wsb = torch.empty(la.la_workspace_size(la.LA_OP_BWD_CAUSAL, 1, 8, wg.N, 128, 128, torch.bfloat16),
                          dtype=torch.uint8, device=dev)

        def gfwd(i):
            st = lib.la_forward_causal(qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), og.data_ptr(), 1, 8, wg.N, 128,
                                       128, la.LA_DTYPE_BF16, wsf.data_ptr(), wsf.numel(), sptr)
            if st != 0:
                raise la.LAError("forward", st)

        def gbwd(i):
            st = lib.la_backward_causal(qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), gg.data_ptr(), dqg.data_ptr(),
                                        dkg.data_ptr(), dvg.data_ptr(), 1, 8, wg.N, 128, 128, la.LA_DTYPE_BF16,
                                        wsb.data_ptr(), wsb.numel(), sptr)
            if st != 0:
                raise la.LAError("backward", st)

        th = 8 * wg.N
        res = {"workload": wg.name}
        for name, fn, per_tok in (("forward", gfwd, 4 * 128 * 2), ("backward", gbwd, 7 * 128 * 2)):
            for i in range(2):
                fn(i)
            t = time_events(fn, 10)
            res[name] = dict(ms_per_call=t / 10 * 1e3, tok_heads_per_s=th * 10 / t,
                             hbm_frac=th * per_tok / (t / 10) / 1e9 / HBM_PEAK_GBS)
        results["head_size_128"] = res
        log(f"head size 128: forward {res['forward']['ms_per_call']:.4f} ms, "
            f"backward {res['backward']['ms_per_call']:.4f} ms")
        del qg, kg, vg, gg, og, dqg, dkg, dvg, wsf, wsb
    def bwd_rate(w, iters=20):
        q, k, v, g = (to_dev(x, w.dtype) for x in wl.forward_inputs(w, with_dout=True))
        grads = [torch.empty_like(x) for x in (q, k, v)]
        dtc = la.LA_DTYPE_BF16 if w.dtype == "bf16" else la.LA_DTYPE_F32
        ws = torch.empty(max(1, la.la_workspace_size(la.LA_OP_BWD_CAUSAL, w.B, w.H, w.N, w.D, w.M, dtc)),
                         dtype=torch.uint8, device=dev)

        def f(i):
            st = lib.la_backward_causal(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), grads[0].data_ptr(),
                                        grads[1].data_ptr(), grads[2].data_ptr(), w.B, w.H, w.N, w.D, w.M, dtc,
                                        ws.data_ptr(), ws.numel(), sptr)
            if st != 0:
                raise la.LAError("backward", st)

        for i in range(3):
            f(i)
        t = time_events(f, iters)
        th = w.B * w.H * w.N
        by = th * ((2 * w.D + 2 * w.M) + (2 * w.D + w.M)) * (2 if w.dtype == "bf16" else 4)
        return dict(us_per_call=t / iters * 1e6, tok_heads_per_s=th * iters / t,
                    hbm_frac=by / (t / iters) / 1e9 / HBM_PEAK_GBS)

    if a.only in ("all", "small"):
        results["small_workloads"] = {wl.WORKLOADS[i].name: fwd_rate(wl.WORKLOADS[i]) for i in (1, 2, 3)}
        # the causal backward on the 784-token fp32 workload (split fp32 operands)
        results["small_workloads"]["backward, " + wl.WORKLOADS[2].name] = bwd_rate(wl.WORKLOADS[2])
        for name_, r_ in results["small_workloads"].items():
            log(f"{name_}: {r_['us_per_call']:.1f} us/call, {r_['hbm_frac']:.3f} of HBM")
    if (a.only == "all" and not a.no_sweep) or a.only == "sweep":
        results["sweep"] = {str(n): fwd_rate(w4.with_n(n)) for n in wl.SWEEP_N}

    # ---- decode ------------------------------------------------------------------------------
    # A separate workload: the long-sequence tensors are released first, so that
    # the decode state is a fresh allocation as in a serving process (carved out
    # of the caching allocator's older segments it was measured 25% slower).
    del sets, out, ws_f
    flush_buf[0] = None
    torch.cuda.empty_cache()
    if a.only in ("all", "decode"):
        w5 = wl.WORKLOADS[5]
        log("generating decode inputs")
        qs, ks, vs = wl.DecodeStream(w5).take(w5.steps)
        dq5, dk5, dv5 = to_dev(qs, "bf16"), to_dev(ks, "bf16"), to_dev(vs, "bf16")
        del qs, ks, vs
        S = torch.zeros((w5.B, w5.H, w5.D, w5.M), dtype=torch.float32, device=dev)
        Z = torch.zeros((w5.B, w5.H, w5.D), dtype=torch.float32, device=dev)
        o5 = torch.empty((w5.steps, w5.B, w5.H, w5.M), dtype=torch.bfloat16, device=dev)
        BH5 = w5.B * w5.H
        qb, kb, vb, ob = dq5.data_ptr(), dk5.data_ptr(), dv5.data_ptr(), o5.data_ptr()
        sq, so = BH5 * w5.D * 2, BH5 * w5.M * 2
        dec = lib.la_decode_step
        Sp, Zp = S.data_ptr(), Z.data_ptr()

        def one_pass(_):
            for t in range(w5.steps):
                dec(qb + t * sq, kb + t * sq, vb + t * so, Sp, Zp, ob + t * so, w5.B, w5.H, w5.D, w5.M,
                    la.LA_DTYPE_BF16, sptr)

        S.zero_(); Z.zero_()
        one_pass(0)
        passes = []
        for p in range(a.decode_passes):
            S.zero_(); Z.zero_()
            passes.append(time_events(one_pass, 1))
        t_eager = min(passes)
        # the same 3072 calls captured once into a HIP graph and replayed
        g = torch.cuda.CUDAGraph()
        S.zero_(); Z.zero_()
        cap = torch.cuda.Stream(dev)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            cs = torch.cuda.current_stream(dev).cuda_stream
            for t in range(w5.steps):
                dec(qb + t * sq, kb + t * sq, vb + t * so, Sp, Zp, ob + t * so, w5.B, w5.H, w5.D, w5.M,
                    la.LA_DTYPE_BF16, cs)
        gpasses = []
        for p in range(a.decode_passes):
            S.zero_(); Z.zero_()
            torch.cuda.synchronize()
            gpasses.append(time_events(lambda i: g.replay(), 1))
        t_graph = min(gpasses)
        bytes_call = BH5 * (2 * w5.D * w5.M * 4 + 2 * w5.D * 4) + BH5 * (2 * w5.D + 2 * w5.M) * 2
        results["decode"] = dict(
            steps_per_s_eager=w5.steps / t_eager, steps_per_s_graph=w5.steps / t_graph,
            us_per_call_eager=t_eager / w5.steps * 1e6, us_per_call_graph=t_graph / w5.steps * 1e6,
            algorithmic_bytes_per_call=bytes_call,
            effective_gbs_graph=bytes_call * w5.steps / t_graph / 1e9,
            effective_gbs_eager=bytes_call * w5.steps / t_eager / 1e9,
            hbm_frac_graph=bytes_call * w5.steps / t_graph / 1e9 / HBM_PEAK_GBS,
            hbm_frac_eager=bytes_call * w5.steps / t_eager / 1e9 / HBM_PEAK_GBS,
            note="effective bandwidth: algorithmic bytes (S, Z read and written in fp32; q, k, v, out) per call "
                 "over the call's time, against the 8 TB/s HBM peak. The 34.6 MB state is rewritten every call "
                 "and stays largely in the 256 MB memory-side cache (Infinity Cache), so this is not DRAM "
                 "bandwidth: counters show the algorithmic bytes leaving L2, not reaching DRAM")
        log(f"decode: eager {w5.steps / t_eager:.4e} steps/s, graph {w5.steps / t_graph:.4e} steps/s")
        del g

    # ---- CPU baseline: the fp64 oracle on the host cores ---------------------------------------
    cpu = None
    if not a.no_cpu_baseline and a.only == "all":
        import oracle
        lo = oracle.load()
        q, k, v, _ = wl.forward_inputs(w4, with_dout=True)
        threads = min(oracle.num_threads(lo), BH)
        try:
            host_cores = len(os.sched_getaffinity(0))
        except AttributeError:
            host_cores = os.cpu_count()
        t0 = time.time()
        reps = 0
        while True:
            oracle.forward_causal(q, k, v, lib=lo)
            reps += 1
            if time.time() - t0 >= 10.0:
                break
        dt = time.time() - t0
        cpu = {"value": tok_heads * reps / dt, "unit": "tokens*heads/s", "cores": host_cores,
               "threads_used": threads, "os_cpu_count": os.cpu_count(), "kind": "oracle",
               "sample": f"full long-sequence workload (B1 H8 N65536 D=M=64, bf16 values in fp64), "
                         f"{reps} causal forward pass(es) in {dt:.1f} s, OpenMP over the 8 (b,h) recurrences "
                         f"({threads} threads on {host_cores} available cores)"}
        log(f"oracle: {cpu['value']:.4e} tokens*heads/s on {threads} threads")

    f = results.get("forward")
    roof = None
    if f:
        ach = fwd_bytes / (f["ms_per_step"] / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": stored_traffic(),
                "kernel": "k_fwd_fused (the single launch of each la_forward_causal call)",
                "algorithmic_bytes_per_launch": fwd_bytes}
    line = {
        "metric": "causal lin-attn fwd tokens·heads/s (N=65536,D=M=64); decode steps/s",
        "value": f["tok_heads_per_s"] if f else None,
        "unit": "tokens*heads/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": f["ms_per_step"] if f else None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "accumulate": "fp32",
        "data": "synthetic (seeded N(0,1) Q, K, V; no dataset or weights)",
        "config": {"workload": "causal forward B1 H8 N65536 D=M=64 bf16", "B": w4.B, "H": w4.H, "N": w4.N,
                   "D": w4.D, "M": w4.M},
        "roofline": roof,
        "cpu_baseline": cpu,
        "decode": results.get("decode"),
        "extra": {k_: v_ for k_, v_ in results.items() if k_ not in ("decode",)},
        "flops_per_step": fwd_flops,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
