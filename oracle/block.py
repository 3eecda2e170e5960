"""fp64 oracle of the fused KLA block prologue.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may import this module; the product path (``scan_amd``) never
does, and nothing here imports ``scan_amd``.

The layer around the scan is described as a Mamba-like fused block with a
one-dimensional causal convolution and a SiLU activation ("Kalman Linear
Attention: Parallel Bayesian Filtering For Efficient Language Modelling and
State Tracking", gist.science explainer, technical summary > method §4,
architecture).  The pages print neither the convolution's placement nor the
parametrisation of the filter coefficients, so this module takes the plainest
reading, in which every step is an elementwise map or a short sum:

* q, k and v each pass through their own depthwise causal convolution of W
  taps (W <= 4) along the sequence, plus a per-channel bias, then SiLU:
      x~_t[c] = bias[c] + sum_{j=0}^{W-1} w[c, W-1-j] * x_{t-j}[c]
      q_t = silu(x~_t) = x~_t / (1 + exp(-x~_t))
  Tap W-1 multiplies the current token; rows before token 0 come from a
  convolution state (the W-1 preceding rows, oldest first) or are zero.
* The OU decay is a logistic of its pre-activation, a = sigmoid(za), so that
  0 < a < 1 (a stable transition); the process noise qn = softplus(zqn) >= 0
  and the observation noise r = softplus(zr) + r_eps > 0 are softplus maps,
  the plainest positive parametrisations of a variance.

The Kalman forward itself is the fp64 sequential recurrence of ``kla_oracle.c``
(``oracle.fwd``), fed with the prologue's outputs.
"""
from __future__ import annotations

import numpy as np

from . import DIAG, fwd as _fwd

MAX_WIDTH = 4


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def sigmoid(x):
    """1 / (1 + exp(-x)), evaluated without overflow for either sign."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def softplus(x):
    """log(1 + exp(x)) = max(x, 0) + log1p(exp(-|x|))."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def silu(x):
    """x * sigmoid(x)."""
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def causal_conv(x, w, bias=None, state=None):
    """Depthwise causal convolution along the sequence.

    x [B,H,T,d]; w [H,d,W] (tap W-1 on the current token, tap W-1-j on the
    token j steps back); bias [H,d] or None; state [B,H,W-1,d] (the W-1 rows
    before token 0, oldest first) or None for zeros.  Returns [B,H,T,d] fp64.
    """
    x, w = _f64(x), _f64(w)
    B, H, T, d = x.shape
    W = w.shape[-1]
    if not 1 <= W <= MAX_WIDTH:
        raise ValueError("width must be 1..4")
    prev = np.zeros((B, H, W - 1, d)) if state is None else _f64(state).reshape(B, H, W - 1, d)
    xe = np.concatenate([prev, x], axis=2)          # row W-1+t holds token t
    y = np.zeros((B, H, T, d))
    if bias is not None:
        y += _f64(bias)[None, :, None, :]
    for j in range(W):                              # lag j: token t-j, tap W-1-j
        y += w[None, :, None, :, W - 1 - j] * xe[:, :, W - 1 - j:W - 1 - j + T, :]
    return y


def prologue(xq, xk, xv, za, zqn, zr, wq, wk, wv, bq=None, bk=None, bv=None,
             sq=None, sk=None, sv=None, r_eps=1e-3):
    """The block prologue (diagonal covariance): returns fp64 q, k, v [B,H,T,d],
    a [B,H,T,dk], qn [H,dk] and r [B,H,T]."""
    return {
        "q": silu(causal_conv(xq, wq, bq, sq)),
        "k": silu(causal_conv(xk, wk, bk, sk)),
        "v": silu(causal_conv(xv, wv, bv, sv)),
        "a": sigmoid(_f64(za)),
        "qn": softplus(_f64(zqn)),
        "r": softplus(_f64(zr)) + float(r_eps),
    }


def block_fwd(xq, xk, xv, za, zqn, zr, wq, wk, wv, bq=None, bk=None, bv=None,
              sq=None, sk=None, sv=None, r_eps=1e-3, l0=None, eta0=None,
              nthreads=None, lib_path=None):
    """Prologue, then the fp64 diagonal forward.  Returns dict(o, lT, etaT) as
    the forward oracle does."""
    p = prologue(xq, xk, xv, za, zqn, zr, wq, wk, wv, bq, bk, bv, sq, sk, sv, r_eps)
    return _fwd(p["q"], p["k"], p["v"], p["a"], p["qn"], p["r"], l0, eta0, cov=DIAG,
                nthreads=nthreads, lib_path=lib_path)
