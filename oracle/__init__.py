"""CPU oracle for the KDA / CKDA recurrence — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never imports, links or
falls back to it, and this package imports nothing from the HIP library.

The arithmetic lives in ``kda_oracle.c`` (plain C, fp64 state and sums), which
follows "Semidirect Fourier Delta Attention" (arXiv 2607.11897) §1 eq. (1) for
the state update and §3 eq. (14) for the read-out, with the Complex-KDA ranges
of "Complex KDA: Understanding and Enhancing the Expressivity of Kimi Delta
Attention" (the abstract).  This module only marshals numpy arrays.

Pins: tests/test_oracle_pins.py fixes this oracle against the pages' worked
numbers, closed forms (Householder, rotation, beta = 0), invariants
(non-expansiveness, linearity in the initial state, chunked = sequential) and a
dense brute-force product of per-token affine maps on tiny inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True, cwd=_HERE)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        fp = ctypes.POINTER(ctypes.c_float)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        lib.kda_oracle_forward.argtypes = [fp, fp, fp, fp, fp, fp, dp, dp, dp, i,
                                           i, i, i, i, i, i]
        lib.kda_oracle_forward.restype = i
        d = ctypes.c_double
        lib.kda_oracle_forward_prologue.argtypes = [fp, fp, fp, fp, fp, fp, d, d, d, d, i,
                                                    dp, dp, i, i, i, i, i, i]
        lib.kda_oracle_forward_prologue.restype = i
        lib.kda_oracle_forward_phase.argtypes = [fp, fp, fp, fp, fp, fp, fp, dp, dp,
                                                 i, i, i, i, i, i]
        lib.kda_oracle_forward_phase.restype = i
        lib.kda_oracle_backward.argtypes = [fp, fp, fp, fp, fp, fp, fp, fp, dp, dp, dp, dp, dp,
                                            dp, i, i, i, i, i, i]
        lib.kda_oracle_backward.restype = i
        lib.kda_oracle_backward_phase.argtypes = [fp, fp, fp, fp, fp, fp, fp, fp, fp, dp, dp, dp,
                                                  dp, dp, dp, dp, i, i, i, i, i, i]
        lib.kda_oracle_backward_phase.restype = i
        lib.kda_oracle_backward_prologue.argtypes = [fp, fp, fp, fp, fp, fp, fp, fp, d, d, d, d, i,
                                                     dp, dp, dp, dp, dp, dp, i, i, i, i, i, i]
        lib.kda_oracle_backward_prologue.restype = i
        lib.kda_oracle_decode.argtypes = [fp, fp, fp, fp, fp, dp, dp,
                                          i, i, i, i, i, i]
        lib.kda_oracle_decode.restype = i
        lib.kda_oracle_gate_prep.argtypes = [
            fp, dp, ctypes.POINTER(ctypes.c_ubyte), ctypes.POINTER(ctypes.c_int),
            dp, i, i, i, i, i]
        lib.kda_oracle_gate_prep.restype = i
        _lib = lib
    return _lib


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype)) if a is not None else None


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def forward(q, k, v, alpha, beta, S0=None, nthreads: int | None = None, chunk: int | None = None):
    """Token-by-token forward.  q, k, alpha: [B,T,H,Dk]; v: [B,T,H,Dv];
    beta: [B,T,H]; S0: [B,H,Dk,Dv] or None (zero).  Inputs are taken as float32
    (exact for bf16 and fp32 values).  Returns (out [B,T,H,Dv], ST [B,H,Dk,Dv])
    in float64; with chunk given, also CS [B,H,ceil(T/chunk),Dk,Dv], the state
    before token n*chunk for every n."""
    lib = _load()
    q, k, v, alpha, beta = (_f32(x) for x in (q, k, v, alpha, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, T, H, Dk) and alpha.shape == (B, T, H, Dk)
    assert v.shape == (B, T, H, Dv) and beta.shape == (B, T, H)
    s0 = None if S0 is None else _f32(S0)
    if s0 is not None:
        assert s0.shape == (B, H, Dk, Dv)
    out = np.empty((B, T, H, Dv), dtype=np.float64)
    ST = np.empty((B, H, Dk, Dv), dtype=np.float64)
    CS = None
    if chunk is not None:
        assert chunk > 0
        CS = np.empty((B, H, (T + chunk - 1) // chunk, Dk, Dv), dtype=np.float64)
    rc = lib.kda_oracle_forward(
        _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
        _ptr(alpha, ctypes.c_float), _ptr(beta, ctypes.c_float),
        _ptr(s0, ctypes.c_float), _ptr(out, ctypes.c_double), _ptr(ST, ctypes.c_double),
        _ptr(CS, ctypes.c_double), chunk or 0,
        B, T, H, Dk, Dv, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("kda_oracle_forward failed")
    return (out, ST) if chunk is None else (out, ST, CS)


def forward_prologue(q_raw, k_raw, v, gate, beta_logit, S0=None, *, alpha_min: float,
                     alpha_max: float, beta_max: float, eps: float, normalize_q: bool,
                     nthreads: int | None = None):
    """Forward from raw inputs through the stable parameterisation ("Semidirect
    Fourier Delta Attention" §3, eqs. (15), (17), (18)), in float64:
    alpha = alpha_min + (alpha_max - alpha_min) sigmoid(gate), beta = beta_max
    sigmoid(beta_logit), k = k_raw / (|k_raw| + eps) and q likewise when
    normalize_q.  Layouts as forward(); returns (out, ST) in float64."""
    lib = _load()
    q, k, v, g, c = (_f32(x) for x in (q_raw, k_raw, v, gate, beta_logit))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, T, H, Dk) and g.shape == (B, T, H, Dk)
    assert v.shape == (B, T, H, Dv) and c.shape == (B, T, H)
    s0 = None if S0 is None else _f32(S0)
    out = np.empty((B, T, H, Dv), dtype=np.float64)
    ST = np.empty((B, H, Dk, Dv), dtype=np.float64)
    rc = lib.kda_oracle_forward_prologue(
        _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
        _ptr(g, ctypes.c_float), _ptr(c, ctypes.c_float), _ptr(s0, ctypes.c_float),
        float(alpha_min), float(alpha_max), float(beta_max), float(eps), int(bool(normalize_q)),
        _ptr(out, ctypes.c_double), _ptr(ST, ctypes.c_double),
        B, T, H, Dk, Dv, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("kda_oracle_forward_prologue failed")
    return out, ST


def forward_phase(q, k, v, alpha, theta, beta, S0=None, nthreads: int | None = None):
    """Phase-variant forward ("Semidirect Fourier Delta Attention" §3 eq. (13)):
    channel pairs (2p, 2p+1) decay by alpha_p R(theta_p).  q, k [B,T,H,Dk];
    v [B,T,H,Dv]; alpha, theta [B,T,H,Dk/2]; beta [B,T,H]; S0 [B,H,Dk,Dv] or
    None.  Returns (out, ST) in float64."""
    lib = _load()
    q, k, v, a, th, b = (_f32(x) for x in (q, k, v, alpha, theta, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert Dk % 2 == 0 and a.shape == (B, T, H, Dk // 2) and th.shape == a.shape
    s0 = None if S0 is None else _f32(S0)
    out = np.empty((B, T, H, Dv), dtype=np.float64)
    ST = np.empty((B, H, Dk, Dv), dtype=np.float64)
    rc = lib.kda_oracle_forward_phase(
        _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
        _ptr(a, ctypes.c_float), _ptr(th, ctypes.c_float), _ptr(b, ctypes.c_float),
        _ptr(s0, ctypes.c_float), _ptr(out, ctypes.c_double), _ptr(ST, ctypes.c_double),
        B, T, H, Dk, Dv, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("kda_oracle_forward_phase failed")
    return out, ST


def backward(q, k, v, alpha, beta, dO, S0=None, dST=None, nthreads: int | None = None):
    """Gradients of L = sum <out, dO> + <ST, dST> (dST None = zero) with respect
    to q, k, v, alpha, beta and S0, by the chain rule through each token of
    the recurrence, last token first.  Layouts as forward(); dO like out.
    Returns a dict of float64 arrays dq, dk, dv, dalpha, dbeta, dS0."""
    lib = _load()
    q, k, v, alpha, beta, dO = (_f32(x) for x in (q, k, v, alpha, beta, dO))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, T, H, Dk) and alpha.shape == (B, T, H, Dk)
    assert v.shape == (B, T, H, Dv) and beta.shape == (B, T, H) and dO.shape == v.shape
    s0 = None if S0 is None else _f32(S0)
    ds = None if dST is None else _f32(dST)
    for x in (s0, ds):
        if x is not None:
            assert x.shape == (B, H, Dk, Dv)
    r = {"dq": np.empty((B, T, H, Dk)), "dk": np.empty((B, T, H, Dk)),
         "dv": np.empty((B, T, H, Dv)), "dalpha": np.empty((B, T, H, Dk)),
         "dbeta": np.empty((B, T, H)), "dS0": np.empty((B, H, Dk, Dv))}
    dp = ctypes.c_double
    rc = lib.kda_oracle_backward(
        _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
        _ptr(alpha, ctypes.c_float), _ptr(beta, ctypes.c_float), _ptr(s0, ctypes.c_float),
        _ptr(dO, ctypes.c_float), _ptr(ds, ctypes.c_float),
        _ptr(r["dq"], dp), _ptr(r["dk"], dp), _ptr(r["dv"], dp), _ptr(r["dalpha"], dp),
        _ptr(r["dbeta"], dp), _ptr(r["dS0"], dp), B, T, H, Dk, Dv, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("kda_oracle_backward failed")
    return r


def backward_phase(q, k, v, alpha, theta, beta, dO, S0=None, dST=None,
                   nthreads: int | None = None):
    """Gradients of L = sum <out, dO> + <ST, dST> for the phase-variant forward
    (forward_phase) with respect to q, k, v, alpha, theta, beta and S0; alpha,
    theta and their gradients are [B,T,H,Dk/2].  Returns a dict of float64
    arrays dq, dk, dv, dalpha, dtheta, dbeta, dS0."""
    lib = _load()
    q, k, v, a, th, beta, dO = (_f32(x) for x in (q, k, v, alpha, theta, beta, dO))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert Dk % 2 == 0 and k.shape == q.shape
    assert a.shape == (B, T, H, Dk // 2) and th.shape == a.shape
    assert v.shape == (B, T, H, Dv) and beta.shape == (B, T, H) and dO.shape == v.shape
    s0 = None if S0 is None else _f32(S0)
    ds = None if dST is None else _f32(dST)
    for x in (s0, ds):
        if x is not None:
            assert x.shape == (B, H, Dk, Dv)
    r = {"dq": np.empty((B, T, H, Dk)), "dk": np.empty((B, T, H, Dk)),
         "dv": np.empty((B, T, H, Dv)), "dalpha": np.empty((B, T, H, Dk // 2)),
         "dtheta": np.empty((B, T, H, Dk // 2)), "dbeta": np.empty((B, T, H)),
         "dS0": np.empty((B, H, Dk, Dv))}
    dp = ctypes.c_double
    rc = lib.kda_oracle_backward_phase(
        _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
        _ptr(a, ctypes.c_float), _ptr(th, ctypes.c_float), _ptr(beta, ctypes.c_float),
        _ptr(s0, ctypes.c_float), _ptr(dO, ctypes.c_float), _ptr(ds, ctypes.c_float),
        _ptr(r["dq"], dp), _ptr(r["dk"], dp), _ptr(r["dv"], dp), _ptr(r["dalpha"], dp),
        _ptr(r["dtheta"], dp), _ptr(r["dbeta"], dp), _ptr(r["dS0"], dp), B, T, H, Dk, Dv,
        nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("kda_oracle_backward_phase failed")
    return r


def backward_prologue(q_raw, k_raw, v, gate, beta_logit, dO, S0=None, dST=None, *,
                      alpha_min: float, alpha_max: float, beta_max: float, eps: float,
                      normalize_q: bool, nthreads: int | None = None):
    """Gradients of L = sum <out, dO> + <ST, dST> for the forward from raw
    inputs (forward_prologue) with respect to q_raw, k_raw, v, the gate logits,
    the beta logits and S0.  Returns a dict of float64 arrays dq, dk, dv,
    dgate, dbeta_logit, dS0."""
    lib = _load()
    q, k, v, g, c, dO = (_f32(x) for x in (q_raw, k_raw, v, gate, beta_logit, dO))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, T, H, Dk) and g.shape == (B, T, H, Dk) and c.shape == (B, T, H)
    assert v.shape == (B, T, H, Dv) and dO.shape == v.shape
    s0 = None if S0 is None else _f32(S0)
    ds = None if dST is None else _f32(dST)
    r = {"dq": np.empty((B, T, H, Dk)), "dk": np.empty((B, T, H, Dk)),
         "dv": np.empty((B, T, H, Dv)), "dgate": np.empty((B, T, H, Dk)),
         "dbeta_logit": np.empty((B, T, H)), "dS0": np.empty((B, H, Dk, Dv))}
    dp = ctypes.c_double
    rc = lib.kda_oracle_backward_prologue(
        _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
        _ptr(g, ctypes.c_float), _ptr(c, ctypes.c_float), _ptr(s0, ctypes.c_float),
        _ptr(dO, ctypes.c_float), _ptr(ds, ctypes.c_float),
        float(alpha_min), float(alpha_max), float(beta_max), float(eps), int(bool(normalize_q)),
        _ptr(r["dq"], dp), _ptr(r["dk"], dp), _ptr(r["dv"], dp), _ptr(r["dgate"], dp),
        _ptr(r["dbeta_logit"], dp), _ptr(r["dS0"], dp), B, T, H, Dk, Dv,
        nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("kda_oracle_backward_prologue failed")
    return r


def decode(q, k, v, alpha, beta, S, nthreads: int | None = None):
    """nsteps single-token updates.  q, k, alpha: [N,B,H,Dk]; v: [N,B,H,Dv];
    beta: [N,B,H]; S: [B,H,Dk,Dv] initial state (not modified).
    Returns (out [N,B,H,Dv], S_final [B,H,Dk,Dv]) in float64."""
    lib = _load()
    q, k, v, alpha, beta = (_f32(x) for x in (q, k, v, alpha, beta))
    N, B, H, Dk = q.shape
    Dv = v.shape[-1]
    assert v.shape == (N, B, H, Dv) and beta.shape == (N, B, H)
    Sd = np.array(S, dtype=np.float64, copy=True, order="C")
    assert Sd.shape == (B, H, Dk, Dv)
    out = np.empty((N, B, H, Dv), dtype=np.float64)
    rc = lib.kda_oracle_decode(
        _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
        _ptr(alpha, ctypes.c_float), _ptr(beta, ctypes.c_float),
        _ptr(Sd, ctypes.c_double), _ptr(out, ctypes.c_double),
        N, B, H, Dk, Dv, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("kda_oracle_decode failed")
    return out, Sd


def gate_prep(alpha, chunk: int):
    """Chunk-local gate summary (see kda_oracle.h).  alpha: [B,T,H,Dk].
    Returns dict with L (float64), parity (uint8), zpos (int32) of shape
    [B,H,NC,C,Dk] and gend (float64) [B,H,NC,Dk]."""
    lib = _load()
    a = _f32(alpha)
    B, T, H, Dk = a.shape
    NC = (T + chunk - 1) // chunk
    L = np.zeros((B, H, NC, chunk, Dk), dtype=np.float64)
    par = np.zeros((B, H, NC, chunk, Dk), dtype=np.uint8)
    zp = np.zeros((B, H, NC, chunk, Dk), dtype=np.int32)
    ge = np.zeros((B, H, NC, Dk), dtype=np.float64)
    rc = lib.kda_oracle_gate_prep(
        _ptr(a, ctypes.c_float), _ptr(L, ctypes.c_double), _ptr(par, ctypes.c_ubyte),
        _ptr(zp, ctypes.c_int), _ptr(ge, ctypes.c_double), B, T, H, Dk, chunk)
    if rc != 0:
        raise RuntimeError("kda_oracle_gate_prep failed")
    return {"L": L, "parity": par, "zpos": zp, "gend": ge}
