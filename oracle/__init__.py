"""fp64 CPU oracle of the Mesa layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never touches it, and the two share no code: the only common
module is the seeded input generator, which holds none of the method's
arithmetic.

The arithmetic lives in ``mesa_oracle.c`` (plain C99, fp64, OpenMP over
heads); this file only compiles it with gcc and marshals numpy arrays.  See
the header of ``mesa_oracle.c`` for what is computed and which passage of the
MesaNet summary page (gist.science, paper 2506.05233, section "A Camada
Mesa") each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mesa_oracle.c")
_LIB = os.path.join(_HERE, "libmesa_oracle.so")

STOP_CAP, STOP_TOL, STOP_RR_ZERO, STOP_BREAKDOWN, STOP_Q_ZERO = 0, 1, 2, 3, 4

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        lib.oracle_cg_solve.argtypes = [I, P, P, P, I, D, P, P, P, P, P]
        lib.oracle_cg_solve.restype = I
        lib.oracle_cg_solve_from.argtypes = [I, P, P, P, P, I, D, P, P, P, P, P]
        lib.oracle_cg_solve_from.restype = I
        lib.oracle_forward.argtypes = [P, P, P, P, P, I, I, I, I, I, I, D,
                                       P, P, P, P, P, P, P, P]
        lib.oracle_forward.restype = I
        lib.oracle_decode_step.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, D,
                                           P, P, P, P, P]
        lib.oracle_decode_step.restype = I
        lib.oracle_decode_step_warm.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, D, I,
                                                P, P, P, P, P]
        lib.oracle_decode_step_warm.restype = I
        lib.oracle_qk_preprocess.argtypes = [P, P, I, P, P, I, I, I, I, P]
        lib.oracle_qk_preprocess.restype = I
        lib.oracle_backward.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, D, P, P, P, P, P, P, P, P, P, P]
        lib.oracle_backward.restype = I
        lib.oracle_hawk_scan.argtypes = [P, P, P, P, D, P, I, I, I, P, P]
        lib.oracle_hawk_scan.restype = I
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = I
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    """OpenMP threads the oracle's parallel loops use (one head per thread)."""
    return int(_load().oracle_max_threads())


def cg_solve(Hm, lam, b, max_iters, tol=0.0, x0=None):
    """CG on (Hm + diag(lam)) x = b from x = 0, or from x = x0 when given.

    Returns (x, iters, reason, rho_stop, rho_min_prev).
    """
    lib = _load()
    Hm, lam, b = _f64(Hm), _f64(lam), _f64(b)
    n = b.shape[0]
    assert Hm.shape == (n, n) and lam.shape == (n,)
    x = np.zeros(n)
    scratch = np.zeros(3 * n)
    reason = ctypes.c_int(0)
    rs = ctypes.c_double(0)
    rm = ctypes.c_double(0)
    if x0 is None:
        it = lib.oracle_cg_solve(n, _ptr(Hm), _ptr(lam), _ptr(b), int(max_iters), float(tol),
                                 _ptr(x), _ptr(scratch), ctypes.byref(reason),
                                 ctypes.byref(rs), ctypes.byref(rm))
    else:
        x0 = _f64(x0)
        assert x0.shape == (n,)
        it = lib.oracle_cg_solve_from(n, _ptr(Hm), _ptr(lam), _ptr(b), _ptr(x0), int(max_iters),
                                      float(tol), _ptr(x), _ptr(scratch), ctypes.byref(reason),
                                      ctypes.byref(rs), ctypes.byref(rm))
    return x, it, reason.value, rs.value, rm.value


def forward(q, k, v, gamma, lam, max_iters, tol=0.0, want=None, final_state=False):
    """Mesa-layer forward over [B, H, T] in fp64.

    q, k: [B,H,T,dk]; v: [B,H,T,dv]; gamma: [B,H,T]; lam: [H,dk] -- any real
    dtype, widened exactly to float64.  ``want`` ([B,H,T] bool) selects the
    tokens to solve (all others keep NaN outputs and -1 counts).
    Returns dict(out, iters, reason, rho_stop, rho_min_prev[, final_H, final_G]).
    """
    lib = _load()
    q, k, v, gamma, lam = _f64(q), _f64(k), _f64(v), _f64(gamma), _f64(lam)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, H, T)
    assert gamma.shape == (B, H, T) and lam.shape == (H, dk)
    out = np.full((B, H, T, dv), np.nan)
    iters = np.full((B, H, T), -1, dtype=np.int32)
    reason = np.full((B, H, T), -1, dtype=np.int32)
    rho_stop = np.full((B, H, T), np.nan)
    rho_min_prev = np.full((B, H, T), np.nan)
    w = None if want is None else np.ascontiguousarray(want, dtype=np.uint8)
    fH = np.zeros((B, H, dk, dk)) if final_state else None
    fG = np.zeros((B, H, dv, dk)) if final_state else None
    rc = lib.oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(lam),
                            B, H, T, dk, dv, int(max_iters), float(tol), _ptr(w),
                            _ptr(out), _ptr(iters), _ptr(rho_stop), _ptr(rho_min_prev),
                            _ptr(reason), _ptr(fH), _ptr(fG))
    if rc != 0:
        raise ValueError("oracle_forward rejected its arguments")
    res = dict(out=out, iters=iters, reason=reason, rho_stop=rho_stop, rho_min_prev=rho_min_prev)
    if final_state:
        res["final_H"], res["final_G"] = fH, fG
    return res


def decode_step(q, k, v, gamma, lam, state_H, state_G, max_iters, tol=0.0):
    """One decode step for [N, H] heads; state_H/state_G (float64) are updated in place."""
    lib = _load()
    q, k, v, gamma, lam = _f64(q), _f64(k), _f64(v), _f64(gamma), _f64(lam)
    N, H, dk = q.shape
    dv = v.shape[-1]
    assert state_H.dtype == np.float64 and state_H.flags.c_contiguous
    assert state_G.dtype == np.float64 and state_G.flags.c_contiguous
    assert state_H.shape == (N, H, dk, dk) and state_G.shape == (N, H, dv, dk)
    out = np.zeros((N, H, dv))
    iters = np.zeros((N, H), dtype=np.int32)
    reason = np.zeros((N, H), dtype=np.int32)
    rho_stop = np.zeros((N, H))
    rho_min_prev = np.zeros((N, H))
    rc = lib.oracle_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(lam),
                                _ptr(state_H), _ptr(state_G), N, H, dk, dv,
                                int(max_iters), float(tol), _ptr(out), _ptr(iters),
                                _ptr(rho_stop), _ptr(rho_min_prev), _ptr(reason))
    if rc != 0:
        raise ValueError("oracle_decode_step rejected its arguments")
    return dict(out=out, iters=iters, reason=reason, rho_stop=rho_stop, rho_min_prev=rho_min_prev)


WARM_COLD, WARM_PREVIOUS, WARM_PROJECTED = 0, 1, 2


def decode_step_warm(q, k, v, gamma, lam, state_H, state_G, state_x, max_iters, tol=0.0,
                     mode=WARM_PROJECTED):
    """One decode step with a warm-started solve; state_H/G/x (float64) are updated in place.

    state_x [N, H, dk] holds the previous step's solution on entry and this
    step's on exit.  mode: WARM_COLD (x0 = 0), WARM_PREVIOUS (x0 = x_prev) or
    WARM_PROJECTED (x0 = c x_prev, c minimising the A-norm error).
    """
    lib = _load()
    q, k, v, gamma, lam = _f64(q), _f64(k), _f64(v), _f64(gamma), _f64(lam)
    N, H, dk = q.shape
    dv = v.shape[-1]
    for a in (state_H, state_G, state_x):
        assert a.dtype == np.float64 and a.flags.c_contiguous
    assert state_H.shape == (N, H, dk, dk) and state_G.shape == (N, H, dv, dk)
    assert state_x.shape == (N, H, dk)
    out = np.zeros((N, H, dv))
    iters = np.zeros((N, H), dtype=np.int32)
    reason = np.zeros((N, H), dtype=np.int32)
    rho_stop = np.zeros((N, H))
    rho_min_prev = np.zeros((N, H))
    rc = lib.oracle_decode_step_warm(_ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(lam),
                                     _ptr(state_H), _ptr(state_G), _ptr(state_x), N, H, dk, dv,
                                     int(max_iters), float(tol), int(mode), _ptr(out), _ptr(iters),
                                     _ptr(rho_stop), _ptr(rho_min_prev), _ptr(reason))
    if rc != 0:
        raise ValueError("oracle_decode_step_warm rejected its arguments")
    return dict(out=out, iters=iters, reason=reason, rho_stop=rho_stop, rho_min_prev=rho_min_prev)


def qk_preprocess(x, w, hist=None, want_hist=False):
    """Causal depthwise convolution of width W over tokens, then L2 normalisation per token.

    x: [B,H,T,d]; w: [H,W,d]; hist: [B,H,W-1,d] rows before t = 0 (None = zeros).
    Returns y [B,H,T,d] (float64), and with want_hist also the last W-1 input rows.
    """
    lib = _load()
    x, w = _f64(x), _f64(w)
    B, H, T, d = x.shape
    W = w.shape[1]
    assert w.shape == (H, W, d)
    if hist is not None:
        hist = _f64(hist)
        assert hist.shape == (B, H, W - 1, d)
    y = np.zeros((B, H, T, d))
    ho = np.zeros((B, H, W - 1, d)) if want_hist else None
    rc = lib.oracle_qk_preprocess(_ptr(x), _ptr(w), W, _ptr(hist), _ptr(ho), B, H, T, d, _ptr(y))
    if rc != 0:
        raise ValueError("oracle_qk_preprocess rejected its arguments")
    return (y, ho) if want_hist else y


def backward(q, k, v, gamma, lam, gout, max_iters, tol=0.0):
    """Gradients of a loss with dL/d(out) = gout through the layer (implicit
    differentiation with a k-step adjoint CG; see oracle_backward in the C file).

    Returns dict(dq, dk, dv, dgamma, dlam, x, z_iters, z_rho_stop, z_rho_min_prev, z_reason).
    """
    lib = _load()
    q, k, v, gamma, lam, gout = _f64(q), _f64(k), _f64(v), _f64(gamma), _f64(lam), _f64(gout)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, H, T) and gout.shape == v.shape
    x = np.zeros((B, H, T, dk))
    dq = np.zeros((B, H, T, dk))
    dkk = np.zeros((B, H, T, dk))
    dvv = np.zeros((B, H, T, dv))
    dg = np.zeros((B, H, T))
    dl = np.zeros((H, dk))
    zi = np.zeros((B, H, T), dtype=np.int32)
    zs = np.zeros((B, H, T))
    zm = np.zeros((B, H, T))
    zr = np.zeros((B, H, T), dtype=np.int32)
    rc = lib.oracle_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(lam), _ptr(gout), B, H, T, dk, dv,
                             int(max_iters), float(tol), _ptr(x), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dg),
                             _ptr(dl), _ptr(zi), _ptr(zs), _ptr(zm), _ptr(zr))
    if rc != 0:
        raise ValueError("oracle_backward rejected its arguments")
    return dict(dq=dq, dk=dkk, dv=dvv, dgamma=dg, dlam=dl, x=x, z_iters=zi, z_rho_stop=zs,
                z_rho_min_prev=zm, z_reason=zr)


def hawk_scan(x, ga, gx, lam, c=8.0, h0=None):
    """The Hawk layer's gated linear recurrence over [B, T, D] (see
    oracle_hawk_scan).  Returns (y [B,T,D], h_final [B,D]) in float64."""
    lib = _load()
    x, ga, gx, lam = _f64(x), _f64(ga), _f64(gx), _f64(lam)
    B, T, D = x.shape
    assert ga.shape == x.shape and gx.shape == x.shape and lam.shape == (D,)
    if h0 is not None:
        h0 = _f64(h0)
        assert h0.shape == (B, D)
    y = np.zeros((B, T, D))
    hf = np.zeros((B, D))
    rc = lib.oracle_hawk_scan(_ptr(x), _ptr(ga), _ptr(gx), _ptr(lam), float(c), _ptr(h0), B, T, D, _ptr(y), _ptr(hf))
    if rc != 0:
        raise ValueError("oracle_hawk_scan rejected its arguments")
    return y, hf
