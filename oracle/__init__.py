"""fp64 CPU oracle for the gated delta rule forward -- TEST INFRASTRUCTURE.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The product (the HIP library
and its Python binding in ``gated_delta_rule_34_amd``) never imports, links
or calls anything here, and this package imports nothing from the product.

Two independent formulations live here:

* ``gdn_fwd`` / ``gdn2_fwd`` / ``gdn_step`` -- the per-token recurrence in
  plain C (``gdn_oracle.c``), fp64, one head per OpenMP iteration.  This is
  the definition the device results are compared against.
* ``oracle.chunked`` -- a numpy fp64 evaluation of the same map in chunks
  through the WY form (derived from the recurrence; the pages state that the
  chunked form exists but print no equations).  It is a second, structurally
  different formulation used to pin the recurrence and to expose per-chunk
  intermediates (cumulative gates, A, T, U, W, new values, chunk states).

Pins (``tests/test_oracle_pins.py``) check both against closed forms and
invariants the pages fix.  Absolute values are otherwise parity unpinned:
the pages print no worked numeric example.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (portable flags: no -march=native, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = configure(ctypes.CDLL(_LIB_PATH))
    return _lib


def configure(lib):
    """Argument types of the oracle's C functions on a loaded library."""
    i = ctypes.c_int
    d = ctypes.c_double
    lib.gdn_oracle_fwd.argtypes = [_dp] * 8 + [i] * 5 + [d, i]
    lib.gdn2_oracle_fwd.argtypes = [_dp] * 9 + [i] * 5 + [d, i]
    lib.gdn_oracle_step.argtypes = [_dp] * 7 + [i] * 4 + [d, i]
    lib.gdn2_oracle_step.argtypes = [_dp] * 8 + [i] * 4 + [d, i]
    lib.gdn_oracle_bwd.argtypes = [_dp] * 14 + [i] * 5 + [d, i]
    lib.gdn2_oracle_bwd.argtypes = [_dp] * 16 + [i] * 5 + [d, i]
    lib.gdn_oracle_max_threads.restype = i
    return lib


def _c(x):
    if x is None:
        return None, None
    a = np.ascontiguousarray(x, dtype=np.float64)
    return a, a.ctypes.data_as(_dp)


def max_threads() -> int:
    return int(_load().gdn_oracle_max_threads())


def gdn_fwd(q, k, v, g, beta, h0=None, scale=None, nthreads=0):
    """Per-token GDN recurrence.  q,k [B,T,H,Dk], v [B,T,H,Dv], g,beta [B,T,H],
    h0 [B,H,Dk,Dv] or None.  Returns (o [B,T,H,Dv], S_final [B,H,Dk,Dv]) in fp64."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if scale is None:
        scale = Dk ** -0.5
    keep = [_c(x) for x in (q, k, v, g, beta, h0)]
    o = np.zeros((B, T, H, Dv))
    S = np.zeros((B, H, Dk, Dv))
    _load().gdn_oracle_fwd(*[p for _, p in keep], o.ctypes.data_as(_dp), S.ctypes.data_as(_dp),
                           B, T, H, Dk, Dv, float(scale), int(nthreads))
    return o, S


def gdn2_fwd(q, k, v, log_alpha, b, w, h0=None, scale=None, nthreads=0):
    """Per-token GDN-2 recurrence.  log_alpha, b [B,T,H,Dk]; w [B,T,H,Dv]."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if scale is None:
        scale = Dk ** -0.5
    keep = [_c(x) for x in (q, k, v, log_alpha, b, w, h0)]
    o = np.zeros((B, T, H, Dv))
    S = np.zeros((B, H, Dk, Dv))
    _load().gdn2_oracle_fwd(*[p for _, p in keep], o.ctypes.data_as(_dp), S.ctypes.data_as(_dp),
                            B, T, H, Dk, Dv, float(scale), int(nthreads))
    return o, S


def gdn_step(q, k, v, g, beta, S, scale=None, nthreads=0):
    """One decode step.  q,k [B,H,Dk], v [B,H,Dv], g,beta [B,H], S [B,H,Dk,Dv].
    Returns (o [B,H,Dv], S_new); the input S is not modified."""
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    if scale is None:
        scale = Dk ** -0.5
    keep = [_c(x) for x in (q, k, v, g, beta)]
    S_new = np.array(S, dtype=np.float64, copy=True, order="C")
    o = np.zeros((B, H, Dv))
    _load().gdn_oracle_step(*[p for _, p in keep], S_new.ctypes.data_as(_dp), o.ctypes.data_as(_dp),
                            B, H, Dk, Dv, float(scale), int(nthreads))
    return o, S_new


def gdn2_step(q, k, v, log_alpha, b, w, S, scale=None, nthreads=0):
    """One GDN-2 decode step.  q, k, log_alpha, b [B,H,Dk]; v, w [B,H,Dv];
    S [B,H,Dk,Dv].  Returns (o [B,H,Dv], S_new); the input S is not modified."""
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    if scale is None:
        scale = Dk ** -0.5
    keep = [_c(x) for x in (q, k, v, log_alpha, b, w)]
    S_new = np.array(S, dtype=np.float64, copy=True, order="C")
    o = np.zeros((B, H, Dv))
    _load().gdn2_oracle_step(*[p for _, p in keep], S_new.ctypes.data_as(_dp), o.ctypes.data_as(_dp),
                             B, H, Dk, Dv, float(scale), int(nthreads))
    return o, S_new


def gdn_bwd(q, k, v, g, beta, h0, dO, dST=None, scale=None, nthreads=0):
    """Gradients of L = sum(dO * o) + sum(dST * S_T) for the per-token GDN
    recurrence: returns dq, dk, dv, dg, dbeta, dh0 (dh0 is None when h0 is None)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if scale is None:
        scale = Dk ** -0.5
    keep = [_c(x) for x in (q, k, v, g, beta, h0, dO, dST)]
    dq = np.zeros((B, T, H, Dk))
    dk = np.zeros((B, T, H, Dk))
    dv = np.zeros((B, T, H, Dv))
    dg = np.zeros((B, T, H))
    db = np.zeros((B, T, H))
    dh0 = np.zeros((B, H, Dk, Dv)) if h0 is not None else None
    outs = [a.ctypes.data_as(_dp) for a in (dq, dk, dv, dg, db)] + [dh0.ctypes.data_as(_dp) if dh0 is not None else None]
    _load().gdn_oracle_bwd(*[p for _, p in keep], *outs, B, T, H, Dk, Dv, float(scale), int(nthreads))
    return dq, dk, dv, dg, db, dh0


def gdn2_bwd(q, k, v, log_alpha, b, w, h0, dO, dST=None, scale=None, nthreads=0):
    """Gradients of L = sum(dO * o) + sum(dST * S_T) for the per-token GDN-2
    recurrence: returns dq, dk, dv, dlog_alpha, db, dw, dh0 (dh0 is None when
    h0 is None)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if scale is None:
        scale = Dk ** -0.5
    keep = [_c(x) for x in (q, k, v, log_alpha, b, w, h0, dO, dST)]
    dq = np.zeros((B, T, H, Dk))
    dk = np.zeros((B, T, H, Dk))
    dv = np.zeros((B, T, H, Dv))
    dla = np.zeros((B, T, H, Dk))
    db = np.zeros((B, T, H, Dk))
    dw = np.zeros((B, T, H, Dv))
    dh0 = np.zeros((B, H, Dk, Dv)) if h0 is not None else None
    outs = [a.ctypes.data_as(_dp) for a in (dq, dk, dv, dla, db, dw)] + \
        [dh0.ctypes.data_as(_dp) if dh0 is not None else None]
    _load().gdn2_oracle_bwd(*[p for _, p in keep], *outs, B, T, H, Dk, Dv, float(scale), int(nthreads))
    return dq, dk, dv, dla, db, dw, dh0
