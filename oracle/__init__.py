"""fp64 CPU oracle for the Mamba-2 SSD layer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU product path never imports it.

Thin ctypes wrapper over ``ssd_oracle.c`` (see that file for the
definition, citations and layouts).  Every array is converted to contiguous
float64 before the call; bf16 inputs must be passed as their exact values
(bf16 -> fp32 -> fp64 is exact).
"""
import ctypes
import os

import numpy as np

from .build import LIB, build

_lib = None


def _load(path: str = LIB):
    global _lib
    if _lib is None or path != LIB:
        if not os.path.exists(path):
            build()
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int)
        i = ctypes.c_int
        lib.oracle_conv1d_silu.argtypes = [i, i, i, i, dp, dp, dp, ip, i, dp, dp, dp]
        lib.oracle_ssd_scan.argtypes = [i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp,
                                        ip, i, dp, dp, dp]
        lib.oracle_decode_step.argtypes = [i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp,
                                           dp, dp, dp]
        lib.oracle_gated_rmsnorm.argtypes = [i, i, i, i, ctypes.c_double, dp, dp, dp, dp]
        lib.oracle_ssd_scan_bwd.argtypes = [i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                            dp, dp, dp, dp, dp, dp, dp, dp]
        lib.oracle_ssd_scan_bwd.restype = ctypes.c_int
        lib.oracle_decode_step_mimo.argtypes = [i, i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp,
                                                dp, dp, dp, dp]
        lib.oracle_linear.argtypes = [i, i, i, dp, dp, dp]
        for f in (lib.oracle_conv1d_silu, lib.oracle_ssd_scan, lib.oracle_decode_step,
                  lib.oracle_gated_rmsnorm, lib.oracle_decode_step_mimo, lib.oracle_linear):
            f.restype = ctypes.c_int
        if path != LIB:
            return lib
        _lib = lib
    return _lib


def _d(a):
    """Contiguous float64 copy (or None) and its ctypes pointer."""
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _i(a):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int))


def conv1d_silu(x, w, bias=None, seq_idx=None, conv_state_in=None,
                want_state_out=False, num_seqs=None, lib=None):
    """x (batch, L, CH), w (CH, K) -> out (batch, L, CH)[, conv_state_out]."""
    lib = lib or _load()
    x_, xp = _d(x)
    w_, wp = _d(w)
    b_, bp = _d(bias)
    s_, sp = _i(seq_idx)
    ci_, cip = _d(conv_state_in)
    batch, L, CH = x_.shape
    K = w_.shape[1]
    if seq_idx is not None and num_seqs is None:
        num_seqs = int(np.max(s_)) + 1 if L else 1
    rows = num_seqs if seq_idx is not None else batch
    out = np.zeros((batch, L, CH), np.float64)
    co = np.zeros((rows, K - 1, CH), np.float64) if want_state_out else None
    cop = co.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if want_state_out else None
    rc = lib.oracle_conv1d_silu(batch, L, CH, K, xp, wp, bp, sp, int(num_seqs or 0),
                                cip, cop, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc:
        raise ValueError("oracle_conv1d_silu: invalid argument")
    return (out, co) if want_state_out else out


def ssd_scan(x, dt_raw, dt_bias, A, B, C, D=None, seq_idx=None, initial_state=None,
             want_final_state=False, num_seqs=None, lib=None):
    """Sequential recurrence.  x (batch,L,H,P), dt_raw (batch,L,H), B/C (batch,L,G,N).

    Returns y (batch,L,H,P)[, final_state (rows,H,P,N)] in float64.
    """
    lib = lib or _load()
    x_, xp = _d(x)
    dt_, dtp = _d(dt_raw)
    db_, dbp = _d(dt_bias)
    A_, Ap = _d(A)
    B_, Bp = _d(B)
    C_, Cp = _d(C)
    D_, Dp = _d(D)
    s_, sp = _i(seq_idx)
    h0_, h0p = _d(initial_state)
    batch, L, H, P = x_.shape
    G, N = B_.shape[2], B_.shape[3]
    if seq_idx is not None and num_seqs is None:
        num_seqs = int(np.max(s_)) + 1 if L else 1
    rows = num_seqs if seq_idx is not None else batch
    y = np.zeros((batch, L, H, P), np.float64)
    fs = np.zeros((rows, H, P, N), np.float64) if want_final_state else None
    fsp = fs.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if want_final_state else None
    rc = lib.oracle_ssd_scan(batch, L, H, P, N, G, xp, dtp, dbp, Ap, Bp, Cp, Dp, sp,
                             int(num_seqs or 0), h0p, fsp,
                             y.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc:
        raise ValueError("oracle_ssd_scan: invalid argument")
    return (y, fs) if want_final_state else y


def decode_step(xBC, dt_raw, dt_bias, A, D, ssm_state, H, P, N, G, conv_w=None,
                conv_bias=None, conv_state=None, lib=None):
    """One decode token.  Returns (y (batch,H,P), new ssm_state, new conv_state|None).

    Inputs are not modified (the oracle works on float64 copies).
    """
    lib = lib or _load()
    x_, xp = _d(xBC)
    dt_, dtp = _d(dt_raw)
    db_, dbp = _d(dt_bias)
    A_, Ap = _d(A)
    D_, Dp = _d(D)
    w_, wp = _d(conv_w)
    cb_, cbp = _d(conv_bias)
    cs = None if conv_state is None else np.array(conv_state, dtype=np.float64, copy=True, order="C")
    csp = None if cs is None else cs.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    ss = np.array(ssm_state, dtype=np.float64, copy=True, order="C")
    batch = x_.shape[0]
    K = w_.shape[1] if w_ is not None else 0
    y = np.zeros((batch, H, P), np.float64)
    rc = lib.oracle_decode_step(batch, H, P, N, G, K, xp, dtp, dbp, Ap, Dp, wp, cbp, csp,
                                ss.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                y.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc:
        raise ValueError("oracle_decode_step: invalid argument")
    return y, ss, cs


def gated_rmsnorm(y, z, w, group_size, norm_before_gate=False, eps=1e-5, lib=None):
    """y, z (..., CH) (z may be None), w (CH) -> out (..., CH) in float64."""
    lib = lib or _load()
    y_, yp = _d(y)
    z_, zp = _d(z)
    w_, wp = _d(w)
    CH = y_.shape[-1]
    T = int(y_.size // CH) if CH else 0
    out = np.zeros(y_.shape, np.float64)
    rc = lib.oracle_gated_rmsnorm(T, CH, int(group_size), int(bool(norm_before_gate)), float(eps),
                                  yp, zp, wp, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc:
        raise ValueError("oracle_gated_rmsnorm: invalid argument")
    return out


def decode_step_mimo(x, B, C, dt_raw, dt_bias, A, D, ssm_state, trapezoid=False, lam=None,
                     prev_x=None, prev_B=None, lib=None):
    """MIMO decode step.  x (batch,H,P,R), B/C (batch,G,N,R), dt_raw (batch,H),
    state (batch,H,P,N).  Returns (y (batch,H,P,R), new state, new prev_x,
    new prev_B) as float64 copies (prev ones None without the trapezoid)."""
    lib = lib or _load()
    x_, xp = _d(x)
    B_, Bp = _d(B)
    C_, Cp = _d(C)
    dt_, dtp = _d(dt_raw)
    l_, lp = _d(lam)
    db_, dbp = _d(dt_bias)
    A_, Ap = _d(A)
    D_, Dp = _d(D)
    batch, H, P, R = x_.shape
    G, N = B_.shape[1], B_.shape[2]
    ss = np.array(ssm_state, dtype=np.float64, copy=True, order="C")
    px = pb = None
    pxp = pbp = None
    if trapezoid:
        px = np.array(prev_x, dtype=np.float64, copy=True, order="C")
        pb = np.array(prev_B, dtype=np.float64, copy=True, order="C")
        pxp = px.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
        pbp = pb.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    y = np.zeros((batch, H, P, R), np.float64)
    rc = lib.oracle_decode_step_mimo(batch, H, P, N, G, R, int(bool(trapezoid)), xp, Bp, Cp, dtp, lp, dbp,
                                     Ap, Dp, ss.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), pxp, pbp,
                                     y.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc:
        raise ValueError("oracle_decode_step_mimo: invalid argument")
    return y, ss, px, pb


def ssd_scan_bwd(x, dt_raw, dt_bias, A, B, C, D, dy, initial_state=None, d_final_state=None, lib=None):
    """Gradients of the selective scan (batch rows, no seq_idx) for the loss
    L = <dy, y> + <d_final_state, final_state>.  Returns a dict with dx,
    ddt_raw, dB, dC, ddt_bias, dA, dD and dh0 (float64)."""
    lib = lib or _load()
    x_, xp = _d(x)
    dt_, dtp = _d(dt_raw)
    db_, dbp = _d(dt_bias)
    A_, Ap = _d(A)
    B_, Bp = _d(B)
    C_, Cp = _d(C)
    D_, Dp = _d(D)
    h0_, h0p = _d(initial_state)
    dy_, dyp = _d(dy)
    df_, dfp = _d(d_final_state)
    batch, L, H, P = x_.shape
    G, N = B_.shape[2], B_.shape[3]
    out = {"dx": np.zeros((batch, L, H, P)), "ddt_raw": np.zeros((batch, L, H)),
           "dB": np.zeros((batch, L, G, N)), "dC": np.zeros((batch, L, G, N)),
           "ddt_bias": np.zeros(H), "dA": np.zeros(H), "dD": np.zeros(H), "dh0": np.zeros((batch, H, P, N))}
    ptr = {k: v.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) for k, v in out.items()}
    rc = lib.oracle_ssd_scan_bwd(batch, L, H, P, N, G, xp, dtp, dbp, Ap, Bp, Cp, Dp, h0p, dyp, dfp,
                                 ptr["dx"], ptr["ddt_raw"], ptr["dB"], ptr["dC"], ptr["ddt_bias"], ptr["dA"],
                                 ptr["dD"], ptr["dh0"])
    if rc:
        raise ValueError("oracle_ssd_scan_bwd: invalid argument")
    return out


def linear(x, w, lib=None):
    """y (M, N) = x (M, K) . w (N, K)^T in float64 (a projection of the mixer)."""
    lib = lib or _load()
    x_, xp = _d(x)
    w_, wp = _d(w)
    if x_.ndim != 2 or w_.ndim != 2 or x_.shape[1] != w_.shape[1]:
        raise ValueError("x (M, K) and w (N, K) expected")
    M, K = x_.shape
    N = w_.shape[0]
    y = np.zeros((M, N), np.float64)
    rc = lib.oracle_linear(M, N, K, xp, wp, y.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc != 0:
        raise ValueError("oracle_linear: invalid arguments")
    return y
