"""Python binding of the gfx950 kernelized linear-attention library (libla.so).

Thin ctypes wrapper over the C ABI in ``include/la.h``: it only checks that
arguments are device tensors of the right dtype and layout, allocates outputs
and workspace with torch (device memory plumbing), and passes raw pointers and
the current HIP stream.  Every step of the computation runs in the HIP
kernels; there is no CPU or PyTorch fallback.  If ``libla.so`` has not been
built, every call raises.

Functions carry the C names:
  la_forward_causal(q, k, v, out=None, workspace=None)
  la_forward_causal_noalloc(q, k, v, out=None)
  la_forward_causal_state(q, k, v, s0=None, z0=None, s_final=None, z_final=None, out=None, workspace=None)
  la_forward_causal_features(fq, fk, v, out=None, workspace=None)
  la_rff_features(x, omega, bias, out=None)
  la_forward_causal_poly2(q, k, v, out=None, workspace=None)
  la_forward_causal_poly2_state(q, k, v, state_final=None, out=None, workspace=None)
  la_forward_noncausal_poly2(q, k, v, out=None, workspace=None)
  la_decode_step_poly2(q, k, v, state, out=None)
  la_poly2_state_floats(D, M)
  la_forward_noncausal(q, k, v, out=None, workspace=None)
  la_backward_causal(q, k, v, dout, dq=None, dk=None, dv=None, workspace=None)
  la_backward_noncausal(q, k, v, dout, dq=None, dk=None, dv=None, workspace=None)
  la_backward_causal_poly2(q, k, v, dout, dq=None, dk=None, dv=None, workspace=None)
  la_decode_step(q, k, v, S, Z, out=None)
  la_workspace_size(op, B, H, N, D, M, dtype)
  la_workspace_check(workspace, clear=False)
  la_set_wait_limit(polls)
  la_status_string(status), la_abi_version()

With the environment variable LA_CHECK_WAITS=1 (the test suite sets it) every
forward call made through this module clears its workspace's error word first
and checks it afterwards (la_workspace_check, which synchronizes the stream),
raising LAError(LA_ERR_TIMEOUT) if a cross-workgroup wait gave up; calls being
captured into a graph are not checked.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["la_forward_causal", "la_forward_causal_noalloc", "la_forward_causal_state", "la_forward_causal_features", "la_rff_features",
           "la_forward_causal_poly2", "la_forward_causal_poly2_state", "la_forward_noncausal_poly2",
           "la_decode_step_poly2", "la_poly2_state_floats",
           "la_forward_noncausal", "la_backward_causal", "la_backward_noncausal", "la_backward_causal_poly2",
           "la_decode_step",
           "la_workspace_size", "la_workspace_check", "la_set_wait_limit", "la_status_string", "la_abi_version",
           "LAError", "lib_path", "load", "LA_ERR_TIMEOUT",
           "LA_OP_FWD_CAUSAL", "LA_OP_FWD_NONCAUSAL", "LA_OP_BWD_CAUSAL", "LA_OP_BWD_NONCAUSAL",
           "LA_OP_FWD_CAUSAL_POLY2", "LA_OP_FWD_NONCAUSAL_POLY2", "LA_OP_BWD_CAUSAL_POLY2", "LA_DTYPE_F32",
           "LA_DTYPE_BF16"]

LA_DTYPE_F32, LA_DTYPE_BF16 = 0, 1
LA_OP_FWD_CAUSAL, LA_OP_FWD_NONCAUSAL, LA_OP_BWD_CAUSAL, LA_OP_BWD_NONCAUSAL, LA_OP_FWD_CAUSAL_POLY2 = 0, 1, 2, 3, 4
LA_OP_FWD_NONCAUSAL_POLY2 = 5
LA_OP_BWD_CAUSAL_POLY2 = 6
_DT = {torch.float32: LA_DTYPE_F32, torch.bfloat16: LA_DTYPE_BF16}

LA_ERR_TIMEOUT = 5
CHECK_WAITS = os.environ.get("LA_CHECK_WAITS", "0") not in ("", "0")

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libla.so")
_lib = None


class LAError(RuntimeError):
    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} failed: {la_status_string(status)} ({status})")


def load():
    """Load libla.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise RuntimeError(f"HIP library not built: {lib_path} is missing "
                           "(run `python -m kernelized_transformer_amd.build`)")
    lib = ctypes.CDLL(lib_path)
    vp, i64, sz, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    fwd = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp, sz, vp]
    lib.la_forward_causal.argtypes = fwd
    lib.la_forward_noncausal.argtypes = fwd
    lib.la_backward_causal.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp, sz, vp]
    lib.la_backward_noncausal.argtypes = lib.la_backward_causal.argtypes
    lib.la_backward_causal_poly2.argtypes = lib.la_backward_causal.argtypes
    lib.la_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, vp]
    lib.la_forward_causal_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
    lib.la_forward_causal_state.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp, sz, vp]
    lib.la_forward_causal_features.argtypes = fwd
    lib.la_forward_causal_poly2.argtypes = fwd
    lib.la_forward_noncausal_poly2.argtypes = fwd
    lib.la_forward_causal_poly2_state.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp, sz, vp]
    lib.la_decode_step_poly2.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, vp]
    lib.la_poly2_state_floats.argtypes = [i64, i64]
    lib.la_poly2_state_floats.restype = i64
    lib.la_rff_features.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
    for f in ("la_forward_causal", "la_forward_causal_noalloc", "la_forward_causal_state", "la_forward_causal_features", "la_rff_features",
              "la_forward_causal_poly2", "la_forward_causal_poly2_state", "la_forward_noncausal_poly2",
              "la_decode_step_poly2",
              "la_forward_noncausal", "la_backward_causal", "la_backward_noncausal", "la_backward_causal_poly2",
              "la_decode_step"):
        getattr(lib, f).restype = i32
    lib.la_workspace_size.argtypes = [i32, i64, i64, i64, i64, i64, i32]
    lib.la_workspace_size.restype = sz
    lib.la_status_string.argtypes = [i32]
    lib.la_status_string.restype = ctypes.c_char_p
    lib.la_abi_version.argtypes = []
    lib.la_abi_version.restype = i32
    lib.la_workspace_check.argtypes = [vp, sz, i32, vp]
    lib.la_workspace_check.restype = i32
    lib.la_set_wait_limit.argtypes = [i64]
    lib.la_set_wait_limit.restype = i64
    _lib = lib
    return lib


def la_status_string(status: int) -> str:
    return load().la_status_string(int(status)).decode()


def la_abi_version() -> int:
    return int(load().la_abi_version())


def la_workspace_size(op: int, B: int, H: int, N: int, D: int, M: int, dtype) -> int:
    dt = _DT[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(load().la_workspace_size(int(op), B, H, N, D, M, dt))


def la_workspace_check(workspace: torch.Tensor, clear: bool = False) -> int:
    """Status of a forward workspace's error word (0 = LA_OK, 5 = LA_ERR_TIMEOUT);
    synchronizes the current stream; ``clear`` zeroes the word afterwards."""
    st = load().la_workspace_check(workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                   1 if clear else 0, _stream(workspace.device))
    if st not in (0, LA_ERR_TIMEOUT):
        raise LAError("la_workspace_check", st)
    return int(st)


def la_set_wait_limit(polls: int) -> int:
    """Polls a forward's hand-off wait makes before giving up (process-wide;
    negative restores the default); returns the previous limit."""
    return int(load().la_set_wait_limit(int(polls)))


def _checking(dev) -> bool:
    return CHECK_WAITS and not torch.cuda.is_current_stream_capturing()


def _checked_call(func: str, call, ws):
    """Runs a forward call; in LA_CHECK_WAITS mode its error word is cleared
    before and checked after."""
    check = _checking(ws.device) and ws.numel() * ws.element_size() >= 256   # else the call rejects it itself
    if check:
        la_workspace_check(ws, clear=True)
    _check(func, call())
    if check and la_workspace_check(ws) != 0:
        raise LAError(func, LA_ERR_TIMEOUT)


def _dev(*ts: torch.Tensor):
    dev = ts[0].device
    for t in ts:
        if not (t.is_cuda and t.device == dev and t.is_contiguous()):
            raise ValueError("expected contiguous tensors on the same GPU")
    return dev


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _ws(op, B, H, N, D, M, dtype, workspace, dev):
    need = la_workspace_size(op, B, H, N, D, M, dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    return workspace, workspace.numel() * workspace.element_size()


def _check(func: str, status: int):
    if status != 0:
        raise LAError(func, status)


def _forward(func: str, op: int, q, k, v, out, workspace):
    dev = _dev(q, k, v)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k: [B,H,N,D]; v: [B,H,N,M]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DT:
        raise ValueError("q, k, v must share dtype float32 or bfloat16")
    B, H, N, D = q.shape
    M = v.shape[-1]
    if out is None:
        out = torch.empty((B, H, N, M), dtype=q.dtype, device=dev)
    _dev(q, out)
    ws, wsb = _ws(op, B, H, N, D, M, q.dtype, workspace, dev)
    if op in (LA_OP_FWD_CAUSAL_POLY2, LA_OP_FWD_NONCAUSAL_POLY2):
        _check(func, getattr(load(), func)(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, D, M,
                                           _DT[q.dtype], ws.data_ptr(), wsb, _stream(dev)))
        return out
    _checked_call(func, lambda: getattr(load(), func)(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H,
                                                      N, D, M, _DT[q.dtype], ws.data_ptr(), wsb, _stream(dev)), ws)
    return out


def la_forward_causal(q, k, v, out=None, workspace=None):
    """Causal linear attention forward; returns out [B,H,N,M]."""
    return _forward("la_forward_causal", LA_OP_FWD_CAUSAL, q, k, v, out, workspace)


def la_forward_causal_noalloc(q, k, v, out=None):
    """la_forward_causal on the library's own scratch (no workspace, no
    allocation in the library; ``out`` is allocated here unless given)."""
    dev = _dev(q, k, v)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k: [B,H,N,D]; v: [B,H,N,M]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DT:
        raise ValueError("q, k, v must share dtype float32 or bfloat16")
    B, H, N, D = q.shape
    M = v.shape[-1]
    if out is None:
        out = torch.empty((B, H, N, M), dtype=q.dtype, device=dev)
    _dev(q, out)
    _check("la_forward_causal_noalloc", load().la_forward_causal_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, D, M, _DT[q.dtype], _stream(dev)))
    return out


def la_forward_causal_state(q, k, v, s0=None, z0=None, s_final=None, z_final=None, out=None, workspace=None):
    """Causal forward from the fp32 state (s0 [B,H,D,M], z0 [B,H,D]; None: zero);
    returns (out, s_final, z_final), the state after the last token (allocated
    unless given; pass s_final=s0, z_final=z0 to update in place)."""
    dev = _dev(q, k, v)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k: [B,H,N,D]; v: [B,H,N,M]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DT:
        raise ValueError("q, k, v must share dtype float32 or bfloat16")
    B, H, N, D = q.shape
    M = v.shape[-1]
    if (s0 is None) != (z0 is None):
        raise ValueError("give both s0 and z0, or neither")
    if s_final is None:
        s_final = torch.empty((B, H, D, M), dtype=torch.float32, device=dev)
    if z_final is None:
        z_final = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    states = [s_final, z_final] + ([s0, z0] if s0 is not None else [])
    for t, shape in zip(states, [(B, H, D, M), (B, H, D)] * 2):
        if t.dtype != torch.float32 or tuple(t.shape) != shape:
            raise ValueError("states: float32 s [B,H,D,M] and z [B,H,D]")
    _dev(q, *states)
    if out is None:
        out = torch.empty((B, H, N, M), dtype=q.dtype, device=dev)
    _dev(q, out)
    ws, wsb = _ws(LA_OP_FWD_CAUSAL, B, H, N, D, M, q.dtype, workspace, dev)
    _checked_call("la_forward_causal_state", lambda: load().la_forward_causal_state(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), s0.data_ptr() if s0 is not None else None,
        z0.data_ptr() if z0 is not None else None, s_final.data_ptr(), z_final.data_ptr(), B, H, N, D, M,
        _DT[q.dtype], ws.data_ptr(), wsb, _stream(dev)), ws)
    return out, s_final, z_final


def la_forward_causal_features(fq, fk, v, out=None, workspace=None):
    """Causal linear attention on given features fq, fk [B,H,N,F] (no feature map applied); returns out."""
    return _forward("la_forward_causal_features", LA_OP_FWD_CAUSAL, fq, fk, v, out, workspace)


def la_forward_causal_poly2(q, k, v, out=None, workspace=None):
    """Causal attention with the degree-2 polynomial kernel (q . k)^2 (D, M in {32, 64}); returns out [B,H,N,M]."""
    return _forward("la_forward_causal_poly2", LA_OP_FWD_CAUSAL_POLY2, q, k, v, out, workspace)


def la_forward_noncausal_poly2(q, k, v, out=None, workspace=None):
    """Non-causal attention with the degree-2 polynomial kernel; returns out [B,H,N,M]."""
    return _forward("la_forward_noncausal_poly2", LA_OP_FWD_NONCAUSAL_POLY2, q, k, v, out, workspace)


def la_poly2_state_floats(D: int, M: int) -> int:
    """Floats of one (b, h)'s polynomial-kernel state (0 if D, M are not supported)."""
    return int(load().la_poly2_state_floats(int(D), int(M)))


def la_forward_causal_poly2_state(q, k, v, state_final=None, out=None, workspace=None):
    """la_forward_causal_poly2 that also returns each (b, h)'s state after its last
    token ([B,H,la_poly2_state_floats(D,M)] float32, opaque), for la_decode_step_poly2."""
    dev = _dev(q, k, v)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k: [B,H,N,D]; v: [B,H,N,M]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DT:
        raise ValueError("q, k, v must share dtype float32 or bfloat16")
    B, H, N, D = q.shape
    M = v.shape[-1]
    nst = la_poly2_state_floats(D, M)
    if out is None:
        out = torch.empty((B, H, N, M), dtype=q.dtype, device=dev)
    if state_final is None:
        state_final = torch.empty((B, H, max(nst, 1)), dtype=torch.float32, device=dev)
    if state_final.dtype != torch.float32 or tuple(state_final.shape) != (B, H, nst) or \
            not state_final.is_contiguous():
        raise ValueError(f"state_final: contiguous float32 [B,H,{nst}]")
    _dev(q, out, state_final)
    ws, wsb = _ws(LA_OP_FWD_CAUSAL_POLY2, B, H, N, D, M, q.dtype, workspace, dev)
    _check("la_forward_causal_poly2_state",
           load().la_forward_causal_poly2_state(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                                state_final.data_ptr(), B, H, N, D, M, _DT[q.dtype], ws.data_ptr(),
                                                wsb, _stream(dev)))
    return out, state_final


def la_decode_step_poly2(q, k, v, state, out=None):
    """One polynomial-kernel decode step: q,k [B,H,D]; v [B,H,M]; state [B,H,la_poly2_state_floats(D,M)]
    float32 updated in place (zeros: empty prefix); returns out [B,H,M]."""
    dev = _dev(q, k, v, state)
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("q, k: [B,H,D]; v: [B,H,M]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DT or state.dtype != torch.float32:
        raise ValueError("q, k, v float32 or bfloat16; state float32")
    B, H, D = q.shape
    M = v.shape[-1]
    nst = la_poly2_state_floats(D, M)
    if tuple(state.shape) != (B, H, nst) or not state.is_contiguous():
        raise ValueError(f"state: contiguous float32 [B,H,{nst}]")
    if out is None:
        out = torch.empty((B, H, M), dtype=q.dtype, device=dev)
    _check("la_decode_step_poly2", load().la_decode_step_poly2(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                               state.data_ptr(), out.data_ptr(), B, H, D, M,
                                                               _DT[q.dtype], _stream(dev)))
    return out


def la_rff_features(x, omega, bias, out=None):
    """Random Fourier features sqrt(2/R) cos(x omega + bias) of x [B,H,N,D]; omega [D,R] and bias [R]
    float32; returns [B,H,N,R] in x's dtype."""
    dev = _dev(x, omega, bias)
    if x.dim() != 4 or x.dtype not in _DT:
        raise ValueError("x: [B,H,N,D] float32 or bfloat16")
    if omega.dtype != torch.float32 or bias.dtype != torch.float32 or omega.dim() != 2 or \
            omega.shape[0] != x.shape[-1] or tuple(bias.shape) != (omega.shape[1],):
        raise ValueError("omega: float32 [D,R]; bias: float32 [R]")
    B, H, N, D = x.shape
    R = omega.shape[1]
    if out is None:
        out = torch.empty((B, H, N, R), dtype=x.dtype, device=dev)
    _dev(x, out)
    st = load().la_rff_features(x.data_ptr(), omega.data_ptr(), bias.data_ptr(), out.data_ptr(), B, H, N, D, R,
                                _DT[x.dtype], _stream(dev))
    _check("la_rff_features", st)
    return out


def la_forward_noncausal(q, k, v, out=None, workspace=None):
    """Non-causal linear attention forward; returns out [B,H,N,M]."""
    return _forward("la_forward_noncausal", LA_OP_FWD_NONCAUSAL, q, k, v, out, workspace)


def la_backward_causal(q, k, v, dout, dq=None, dk=None, dv=None, workspace=None):
    """Gradients of sum(dout * la_forward_causal(q, k, v)); returns (dq, dk, dv)."""
    return _backward("la_backward_causal", LA_OP_BWD_CAUSAL, q, k, v, dout, dq, dk, dv, workspace)


def la_backward_noncausal(q, k, v, dout, dq=None, dk=None, dv=None, workspace=None):
    """Gradients of sum(dout * la_forward_noncausal(q, k, v)); returns (dq, dk, dv)."""
    return _backward("la_backward_noncausal", LA_OP_BWD_NONCAUSAL, q, k, v, dout, dq, dk, dv, workspace)


def la_backward_causal_poly2(q, k, v, dout, dq=None, dk=None, dv=None, workspace=None):
    """Gradients of sum(dout * la_forward_causal_poly2(q, k, v)); returns (dq, dk, dv)."""
    return _backward("la_backward_causal_poly2", LA_OP_BWD_CAUSAL_POLY2, q, k, v, dout, dq, dk, dv, workspace)


def _backward(func, op, q, k, v, dout, dq, dk, dv, workspace):
    dev = _dev(q, k, v, dout)
    if not (q.dtype == k.dtype == v.dtype == dout.dtype) or q.dtype not in _DT:
        raise ValueError("q, k, v, dout must share dtype float32 or bfloat16")
    B, H, N, D = q.shape
    M = v.shape[-1]
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _dev(q, dq, dk, dv)
    ws, wsb = _ws(op, B, H, N, D, M, q.dtype, workspace, dev)
    st = getattr(load(), func)(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                               dk.data_ptr(), dv.data_ptr(), B, H, N, D, M, _DT[q.dtype], ws.data_ptr(), wsb,
                               _stream(dev))
    _check(func, st)
    return dq, dk, dv


def la_decode_step(q, k, v, S, Z, out=None):
    """One decode step; q,k: [B,H,D], v: [B,H,M]; S [B,H,D,M] and Z [B,H,D] fp32 are updated in place."""
    dev = _dev(q, k, v, S, Z)
    if S.dtype != torch.float32 or Z.dtype != torch.float32:
        raise ValueError("S and Z must be float32")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DT:
        raise ValueError("q, k, v must share dtype float32 or bfloat16")
    B, H, D = q.shape
    M = v.shape[-1]
    if out is None:
        out = torch.empty((B, H, M), dtype=q.dtype, device=dev)
    st = load().la_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), S.data_ptr(), Z.data_ptr(),
                               out.data_ptr(), B, H, D, M, _DT[q.dtype], _stream(dev))
    _check("la_decode_step", st)
    return out
