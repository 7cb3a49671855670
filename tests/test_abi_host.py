"""Host-only checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function ``include/la.h`` declares, and
reject bad arguments with the documented status codes before touching any
pointer.  Only argument combinations that fail validation are passed here, so
no call reaches a kernel launch.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import kernelized_transformer_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "la.h")


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z0-9_]+)\s*\(", txt)))


def test_header_declares_the_boundary():
    fns = declared_functions()
    for f in ("la_forward_causal", "la_forward_causal_state", "la_forward_causal_features", "la_rff_features",
              "la_forward_causal_poly2", "la_forward_noncausal", "la_backward_causal", "la_backward_noncausal", "la_decode_step",
              "la_workspace_size", "la_workspace_check", "la_set_wait_limit", "la_status_string", "la_abi_version",
              "la_forward_causal_noalloc", "la_forward_causal_poly2_state", "la_forward_noncausal_poly2",
              "la_decode_step_poly2", "la_poly2_state_floats", "la_backward_causal_poly2"):
        assert f in fns


def test_library_exports_every_declared_symbol():
    lib = la.load()
    for f in declared_functions():
        assert hasattr(lib, f), f"libla.so does not export {f}"


def test_abi_version_and_status_strings():
    assert la.la_abi_version() == 10
    names = [la.la_status_string(s) for s in range(6)]
    assert names == ["LA_OK", "LA_ERR_INVALID_ARGUMENT", "LA_ERR_UNSUPPORTED", "LA_ERR_WORKSPACE", "LA_ERR_HIP",
                     "LA_ERR_TIMEOUT"]
    assert la.la_status_string(99) == "LA_ERR_UNKNOWN"


def test_workspace_size():
    import torch
    f = la.la_workspace_size
    # one fp32 record (D*M + D floats) per segment, 256-byte aligned
    n = f(la.LA_OP_FWD_NONCAUSAL, 1, 2, 256, 32, 32, torch.float32)
    assert n > 0 and n % 256 == 0 and n >= 2 * (32 * 32 + 32) * 4
    c = f(la.LA_OP_FWD_CAUSAL, 1, 2, 256, 32, 32, torch.float32)
    assert c > 0 and c % 256 == 0 and c >= 2 * (32 * 32 + 32) * 4
    assert f(la.LA_OP_BWD_CAUSAL, 1, 2, 256, 32, 32, torch.float32) > 2 * n
    # polynomial gradient: per token the weights [g, h] and one partial dq / dk per column block, at least
    pb = f(la.LA_OP_BWD_CAUSAL_POLY2, 1, 2, 256, 32, 32, torch.float32)
    assert pb % 256 == 0 and pb >= 2 * 256 * (33 + 32) * 4
    assert f(la.LA_OP_BWD_CAUSAL_POLY2, 1, 2, 256, 48, 32, torch.float32) == 0
    # non-causal backward: two record arrays, no per-token buffers
    nb = f(la.LA_OP_BWD_NONCAUSAL, 1, 2, 256, 32, 32, torch.float32)
    assert nb > 0 and nb % 256 == 0 and nb < f(la.LA_OP_BWD_CAUSAL, 1, 2, 256, 32, 32, torch.float32)
    assert f(la.LA_OP_BWD_NONCAUSAL, 1, 8, 65536, 64, 64, torch.bfloat16) < 64 * 2 ** 20
    assert f(7, 1, 2, 256, 32, 32, torch.float32) == 0                        # unknown op
    # polynomial kernel: per segment one fp32 record of 33 (D = 32) or 130
    # (D = 64) feature tiles per 16 columns and the D x D normalizer, in
    # 16 x 16 tiles; a (b, h) that is one segment needs no records
    rec = lambda D, M: ((D // 16) * (D // 16 + 1) // 2 + 15 * (D // 16) ** 2 // 2) * (M // 16) * 1024 + (D // 16) ** 2 * 1024
    pw = f(la.LA_OP_FWD_CAUSAL_POLY2, 1, 2, 256, 32, 64, torch.bfloat16)
    assert pw > 0 and pw % 256 == 0 and pw >= 2 * 2 * rec(32, 64)
    p64 = f(la.LA_OP_FWD_CAUSAL_POLY2, 1, 2, 256, 64, 64, torch.bfloat16)
    assert p64 % 256 == 0 and p64 >= 2 * 2 * rec(64, 64)
    assert f(la.LA_OP_FWD_CAUSAL_POLY2, 64, 8, 256, 32, 32, torch.bfloat16) == 256
    assert f(la.LA_OP_FWD_CAUSAL_POLY2, 1, 2, 256, 48, 64, torch.bfloat16) == 0
    assert f(la.LA_OP_FWD_CAUSAL_POLY2, 1, 2, 256, 32, 16, torch.bfloat16) == 0
    # the non-causal polynomial form keeps the (b, h) total even with one segment
    assert f(la.LA_OP_FWD_NONCAUSAL_POLY2, 64, 8, 256, 32, 32, torch.bfloat16) >= 64 * 8 * rec(32, 32)
    assert f(la.LA_OP_FWD_NONCAUSAL_POLY2, 1, 2, 256, 64, 64, torch.bfloat16) >= 2 * rec(64, 64)
    assert f(la.LA_OP_FWD_NONCAUSAL_POLY2, 1, 2, 256, 48, 64, torch.bfloat16) == 0
    assert la.la_poly2_state_floats(32, 32) * 4 == rec(32, 32)
    assert la.la_poly2_state_floats(64, 64) * 4 == rec(64, 64)
    assert la.la_poly2_state_floats(48, 32) == 0 and la.la_poly2_state_floats(32, 128) == 0
    assert f(la.LA_OP_FWD_CAUSAL, 0, 2, 256, 32, 32, torch.float32) == 0     # invalid shape
    assert f(la.LA_OP_FWD_CAUSAL, 1, 2, 256, 40, 32, torch.float32) == 0     # unsupported D
    assert f(la.LA_OP_FWD_CAUSAL, 1, 2, 256, 48, 128, torch.float32) > 0     # the generic path
    assert f(la.LA_OP_BWD_CAUSAL, 1, 2, 256, 48, 32, torch.float32) > 0      # backward: the generic path too
    assert f(la.LA_OP_BWD_NONCAUSAL, 1, 2, 256, 128, 16, torch.bfloat16) > 0
    assert f(la.LA_OP_BWD_CAUSAL, 1, 2, 256, 40, 32, torch.float32) == 0     # not a multiple of 16
    # grows linearly in N at fixed segment count ceiling
    a = f(la.LA_OP_FWD_CAUSAL, 1, 8, 65536, 64, 64, torch.bfloat16)
    assert a <= 8 * 64 * 2 * (64 * 64 + 64) * 4 + 4096


FAKE = 1 << 32   # 16-byte aligned, never dereferenced: every call below fails validation first


def _fwd(lib, fn, q=FAKE, k=FAKE + (1 << 24), v=FAKE + (2 << 24), out=FAKE + (3 << 24), B=1, H=1, N=8, D=32, M=32,
         dt=0, ws=FAKE + (4 << 24), wsb=0):
    return getattr(lib, fn)(q, k, v, out, B, H, N, D, M, dt, ws, wsb, None)


@pytest.mark.parametrize("fn", ["la_forward_causal", "la_forward_noncausal", "la_forward_causal_features"])
def test_forward_argument_errors(fn):
    lib = la.load()
    assert _fwd(lib, fn, q=0) == 1                      # null input
    assert _fwd(lib, fn, out=0) == 1                    # null output
    assert _fwd(lib, fn, q=FAKE + 8) == 1               # misaligned
    assert _fwd(lib, fn, N=0) == 1                      # empty
    assert _fwd(lib, fn, B=-1) == 1
    assert _fwd(lib, fn, D=40) == 2                     # not a multiple of 16
    assert _fwd(lib, fn, M=144) == 2                    # beyond 128
    assert _fwd(lib, fn, dt=7) == 2                     # unknown dtype
    assert _fwd(lib, fn, out=FAKE + 64) == 1            # output overlaps q
    assert _fwd(lib, fn, ws=0, wsb=1 << 20) == 3        # missing workspace
    assert _fwd(lib, fn, wsb=16) == 3                   # too small
    assert _fwd(lib, fn, ws=FAKE + (4 << 24) + 16, wsb=1 << 20) == 3   # misaligned workspace
    assert _fwd(lib, fn, ws=FAKE, wsb=1 << 20) == 3     # workspace overlaps an input


def test_forward_state_argument_errors():
    lib = la.load()
    b = [FAKE + (i << 24) for i in range(10)]   # q k v out s0 z0 s1 z1 ws

    def fs(q=b[0], k=b[1], v=b[2], out=b[3], s0=b[4], z0=b[5], s1=b[6], z1=b[7], B=1, H=2, N=8, D=32, M=32, dt=1,
           ws=b[8], wsb=0):
        return lib.la_forward_causal_state(q, k, v, out, s0, z0, s1, z1, B, H, N, D, M, dt, ws, wsb, None)

    assert fs() == 3                                # all buffers valid: only the workspace is missing
    assert fs(s0=0, z0=0, s1=0, z1=0) == 3          # no state at all is valid too
    assert fs(s1=b[4], z1=b[5]) == 3                # in place is valid
    assert fs(s0=0) == 1                            # s0 without z0
    assert fs(z1=0) == 1                            # s_final without z_final
    assert fs(s0=b[4] + 4) == 1                     # misaligned start state
    assert fs(z1=b[7] + 8) == 1                     # misaligned final state
    assert fs(s1=b[4] + 16, z1=b[7]) == 1           # final state partly overlaps the start state
    assert fs(s1=b[6], z1=b[6] + 256) == 1          # z_final overlaps s_final
    assert fs(s1=b[4], z1=b[4] + 16) == 1           # in place S, z_final inside it
    assert fs(s1=b[0]) == 1                         # final state over q
    assert fs(D=40) == 2
    assert fs(ws=b[6], wsb=1 << 20) == 3            # workspace overlaps the final state


def test_poly2_argument_errors():
    lib = la.load()
    assert _fwd(lib, "la_forward_causal_poly2", D=48) == 2           # D, M in {32, 64}
    assert _fwd(lib, "la_forward_causal_poly2", M=16) == 2
    assert _fwd(lib, "la_forward_causal_poly2", D=128) == 2
    assert _fwd(lib, "la_forward_causal_poly2", q=0) == 1
    assert _fwd(lib, "la_forward_causal_poly2", out=FAKE + 64) == 1
    assert _fwd(lib, "la_forward_causal_poly2", wsb=16) == 3
    assert _fwd(lib, "la_forward_noncausal_poly2", D=48) == 2
    assert _fwd(lib, "la_forward_noncausal_poly2", q=FAKE + 8) == 1
    assert _fwd(lib, "la_forward_noncausal_poly2", wsb=16) == 3          # the total needs a record
    b = [FAKE + (i << 30) for i in range(6)]   # q k v out state ws

    def fs(q=b[0], k=b[1], v=b[2], out=b[3], st=b[4], D=32, M=32, ws=b[5], wsb=1 << 30):
        return lib.la_forward_causal_poly2_state(q, k, v, out, st, 1, 2, 64, D, M, 1, ws, wsb, None)
    assert fs(st=0) == 1                            # the state is required
    assert fs(st=b[4] + 8) == 1                     # misaligned
    assert fs(st=b[0]) == 1                         # overlaps q
    assert fs(st=b[3]) == 1                         # overlaps out
    assert fs(D=16) == 2
    assert fs(ws=b[4], wsb=1 << 30) == 3            # workspace overlaps the state

    def dec(q=b[0], k=b[1], v=b[2], st=b[4], out=b[3], B=2, H=3, D=32, M=32, dt=1):
        return lib.la_decode_step_poly2(q, k, v, st, out, B, H, D, M, dt, None)
    assert dec(st=0) == 1
    assert dec(st=b[3]) == 1                        # state overlaps out
    assert dec(D=48) == 2
    assert dec(M=128) == 2
    assert dec(B=0) == 1
    assert dec(dt=9) == 2


def test_rff_argument_errors():
    lib = la.load()
    b = [FAKE + (i << 24) for i in range(4)]   # x omega bias out

    def rff(x=b[0], om=b[1], bias=b[2], out=b[3], B=1, H=2, N=8, D=64, R=32, dt=1):
        return lib.la_rff_features(x, om, bias, out, B, H, N, D, R, dt, None)

    assert rff(x=0) == 1
    assert rff(om=0) == 1
    assert rff(bias=b[2] + 4) == 1                  # misaligned
    assert rff(out=b[1]) == 1                       # output over omega
    assert rff(out=b[0] + 16) == 1                  # output overlaps x
    assert rff(R=48) == 2 and rff(D=16) == 2        # unsupported sizes
    assert rff(N=0) == 1
    assert rff(dt=5) == 2


def test_backward_and_decode_argument_errors():
    lib = la.load()
    base = [FAKE + (i << 24) for i in range(8)]
    ok = dict(B=1, H=1, N=8, D=32, M=32, dt=1)

    for fn in ("la_backward_causal", "la_backward_noncausal"):
        def bwd(ptrs, B=1, H=1, N=8, D=32, M=32, dt=1, ws=base[7], wsb=0):
            return getattr(lib, fn)(*ptrs, B, H, N, D, M, dt, ws, wsb, None)

        assert bwd(base[:7]) == 3                                   # no workspace bytes
        assert bwd([0] + base[1:7]) == 1
        assert bwd(base[:4] + [base[0], base[5], base[6]]) == 1     # dq aliases q
        assert bwd(base[:4] + [base[4], base[4], base[6]]) == 1     # dq aliases dk
        assert bwd(base[:3] + [base[6]] + base[4:7]) == 1           # dv aliases dout
        assert bwd(base[:7], D=144) == 2                             # beyond 128
        assert bwd(base[:7], M=40) == 2                              # not a multiple of 16
        assert bwd(base[:7], D=128) == 3                             # supported: then the missing workspace
        assert bwd(base[:7], N=0) == 1
        assert bwd(base[:7], ws=base[2], wsb=1 << 20) == 3          # workspace overlaps v
    assert ok

    def dec(q=base[0], k=base[1], v=base[2], S=base[3], Z=base[4], out=base[5], B=2, H=2, D=64, M=64, dt=1):
        return lib.la_decode_step(q, k, v, S, Z, out, B, H, D, M, dt, None)

    assert dec(S=0) == 1
    assert dec(Z=base[3] + 16) == 1                             # Z overlaps S
    assert dec(out=base[0]) == 1                                # out aliases q
    assert dec(D=100) == 2
    assert dec(B=0) == 1


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(la, "lib_path", str(tmp_path / "missing.so"))
    monkeypatch.setattr(la, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        la.load()


def test_workspace_check_argument_errors():
    """la_workspace_check validates the workspace before touching it."""
    lib = la.load()
    assert lib.la_workspace_check(None, 1 << 20, 0, None) == 3          # missing
    assert lib.la_workspace_check(FAKE + 16, 1 << 20, 0, None) == 3     # misaligned
    assert lib.la_workspace_check(FAKE, 128, 1, None) == 3              # smaller than the header


def test_wait_limit_round_trip():
    lib = la.load()
    default = lib.la_set_wait_limit(5)
    assert default == 1 << 20
    assert lib.la_set_wait_limit(0) == 5
    assert lib.la_set_wait_limit(-1) == 0          # back to the default
    assert lib.la_set_wait_limit(-1) == default


def test_noalloc_argument_errors():
    """The no-allocation forward validates like la_forward_causal and rejects a
    shape whose workspace exceeds its 16 MiB scratch, before any launch."""
    lib = la.load()
    b = [FAKE + (i << 34) for i in range(4)]   # far enough apart for a 1 GB tensor each

    def na(q=b[0], k=b[1], v=b[2], out=b[3], B=1, H=8, N=65536, D=64, M=64, dt=1):
        return lib.la_forward_causal_noalloc(q, k, v, out, B, H, N, D, M, dt, None)

    big = dict(H=255, N=32768)               # 510 blocks of 2 records of 16.6 KB: about 17 MB
    assert la.la_workspace_size(la.LA_OP_FWD_CAUSAL, 1, 255, 32768, 64, 64, 1) > 16 * 2 ** 20
    assert na(**big) == 3
    assert na(q=0, **big) == 1               # argument errors come first
    assert na(D=40) == 2
    assert na(out=b[0]) == 1                 # output aliases q
