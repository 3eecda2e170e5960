"""fp64 CPU oracle for the Kalman Linear Attention forward and backward passes.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may import this package; the product path (``scan_amd``) never
does, and nothing here imports ``scan_amd``.

The arithmetic lives in ``kla_oracle.c`` (plain sequential recurrence in fp64,
see its header for the recurrence and its sources; ``bwd`` is the
reverse-mode adjoint of that recurrence, one reverse sweep over a stored
forward trajectory).  This module only builds
that file with gcc, marshals arrays to contiguous fp64 and calls it.

Sources: "Kalman Linear Attention: Parallel Bayesian Filtering For Efficient
Language Modelling and State Tracking" (gist.science explainer, technical
summary > method §1-§3) and "Kalman Delta Networks: Uncertainty-aware
Associative Memory" (abstract; diagonal and isotropic variants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kla_oracle.c")
_LIB = os.path.join(_HERE, "libkla_oracle.so")

DIAG = 0
ISO = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile kla_oracle.c into libkla_oracle.so with gcc (-O2, OpenMP).

    No fast-math: the oracle keeps IEEE fp64 semantics and evaluation order.
    """
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                        "-o", tmp, _SRC], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load(path: str | None = None):
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.kla_oracle_fwd.restype = ctypes.c_int
    lib.kla_oracle_fwd.argtypes = [i, i, i, i, i, i] + [dp] * 12 + [i]
    lib.kla_oracle_step.restype = ctypes.c_int
    lib.kla_oracle_step.argtypes = [i, i, i, i, i] + [dp] * 9 + [i]
    lib.kla_oracle_fwd_residual.restype = ctypes.c_int
    lib.kla_oracle_fwd_residual.argtypes = [i, i, i, i, i, i] + [dp] * 11 + [i]
    if hasattr(lib, "kla_oracle_bwd"):
        lib.kla_oracle_bwd.restype = ctypes.c_int
        lib.kla_oracle_bwd.argtypes = [i, i, i, i, i, i] + [dp] * 19 + [i]
    return lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: upcast the stored values
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def fwd(q, k, v, a, qn, r, l0=None, eta0=None, cov: int = DIAG,
        want_l_all: bool = False, nthreads: int | None = None, lib_path: str | None = None):
    """Run the sequential fp64 recurrence.

    Shapes: q,k [B,H,T,dk]; v [B,H,T,dv]; r [B,H,T];
    diag: a [B,H,T,dk], qn [H,dk], l0 [B,H,dk];  iso: a, qn [B,H,T], l0 [B,H];
    eta0 [B,H,dk,dv].  Returns dict(o, lT, etaT[, l_all]) of fp64 arrays.
    """
    lib = _load(lib_path)
    q, k, v, a, qn, r = (_f64(x) for x in (q, k, v, a, qn, r))
    l0, eta0 = _f64(l0), _f64(eta0)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    nl = dk if cov == DIAG else 1
    o = np.empty((B, H, T, dv))
    lT = np.empty((B, H, nl) if cov == DIAG else (B, H))
    etaT = np.empty((B, H, dk, dv))
    l_all = np.empty((B, H, T, nl) if cov == DIAG else (B, H, T)) if want_l_all else None
    rc = lib.kla_oracle_fwd(B, H, T, dk, dv, cov, _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                            _ptr(qn), _ptr(r), _ptr(l0), _ptr(eta0), _ptr(o), _ptr(lT),
                            _ptr(etaT), _ptr(l_all), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"kla_oracle_fwd failed with code {rc}")
    out = {"o": o, "lT": lT, "etaT": etaT}
    if want_l_all:
        out["l_all"] = l_all
    return out


def step(q, k, v, a, qn, r, l, eta, cov: int = DIAG, nthreads: int | None = None,
         lib_path: str | None = None):
    """One decode step; returns dict(o, l, eta) (inputs are not modified).

    Shapes: q,k [B,H,dk]; v [B,H,dv]; r [B,H]; diag: a [B,H,dk], qn [H,dk],
    l [B,H,dk]; iso: a, qn, l [B,H]; eta [B,H,dk,dv].
    """
    lib = _load(lib_path)
    q, k, v, a, qn, r = (_f64(x) for x in (q, k, v, a, qn, r))
    l = _f64(l).copy()
    eta = _f64(eta).copy()
    B, H, dk = q.shape
    dv = v.shape[-1]
    o = np.empty((B, H, dv))
    rc = lib.kla_oracle_step(B, H, dk, dv, cov, _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                             _ptr(qn), _ptr(r), _ptr(l), _ptr(eta), _ptr(o),
                             nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"kla_oracle_step failed with code {rc}")
    return {"o": o, "l": l, "eta": eta}


def fwd_residual(q, k, v, a, qn, r, l0=None, m0=None, cov: int = DIAG,
                 nthreads: int | None = None, lib_path: str | None = None):
    """Residual-write forward (Kalman-gain-weighted residual write), fp64.

    Same shapes as ``fwd``; the state is the posterior mean m (m0, mT
    [B,H,dk,dv]) with the precision l.  Returns dict(o, lT, mT).
    """
    lib = _load(lib_path)
    q, k, v, a, qn, r = (_f64(x) for x in (q, k, v, a, qn, r))
    l0, m0 = _f64(l0), _f64(m0)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    nl = dk if cov == DIAG else 1
    o = np.empty((B, H, T, dv))
    lT = np.empty((B, H, nl) if cov == DIAG else (B, H))
    mT = np.empty((B, H, dk, dv))
    rc = lib.kla_oracle_fwd_residual(B, H, T, dk, dv, cov, _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                     _ptr(qn), _ptr(r), _ptr(l0), _ptr(m0), _ptr(o), _ptr(lT),
                                     _ptr(mT), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"kla_oracle_fwd_residual failed with code {rc}")
    return {"o": o, "lT": lT, "mT": mT}


def bwd(q, k, v, a, qn, r, l0=None, eta0=None, do=None, dlT=None, detaT=None, cov: int = DIAG,
        nthreads: int | None = None, lib_path: str | None = None):
    """Backward pass of ``fwd`` in fp64 (reverse-mode adjoint of the
    sequential recurrence).

    do [B,H,T,dv] is dL/do; dlT, detaT (shapes of lT, etaT) are the gradients
    of the final state and may be None (zero).  Returns dict(dq, dk, dv, da,
    dqn, dr, dl0, deta0) in the shapes of the inputs q, k, v, a, qn, r, l0
    (diag [B,H,dk], iso [B,H]) and eta0; the diagonal dqn [H,dk] is summed
    over the batch.
    """
    lib = _load(lib_path)
    q, k, v, a, qn, r = (_f64(x) for x in (q, k, v, a, qn, r))
    l0, eta0, do, dlT, detaT = (_f64(x) for x in (l0, eta0, do, dlT, detaT))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    nl = dk if cov == DIAG else 1
    out = {"dq": np.empty((B, H, T, dk)), "dk": np.empty((B, H, T, dk)), "dv": np.empty((B, H, T, dv)),
           "da": np.empty(a.shape), "dqn": np.empty(qn.shape), "dr": np.empty((B, H, T)),
           "dl0": np.empty((B, H, nl) if cov == DIAG else (B, H)), "deta0": np.empty((B, H, dk, dv))}
    rc = lib.kla_oracle_bwd(B, H, T, dk, dv, cov, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(qn),
                            _ptr(r), _ptr(l0), _ptr(eta0), _ptr(do), _ptr(dlT), _ptr(detaT),
                            *(_ptr(out[n]) for n in ("dq", "dk", "dv", "da", "dqn", "dr", "dl0",
                                                     "deta0")),
                            nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"kla_oracle_bwd failed with code {rc}")
    return out
