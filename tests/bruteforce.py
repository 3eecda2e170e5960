"""Brute-force joint-Gaussian filtering posteriors in fp64 (numpy), for pins.

Independent of the oracle's recursion: every filtered posterior is obtained
by writing out the joint precision matrix of a scalar chain (prior on
x_{-1}, OU transitions x_u = a_u x_{u-1} + N(0, qn_u), Gaussian evidence
potentials on each x_u) and inverting it with numpy.linalg.  This is the
linear-Gaussian model of "Kalman Linear Attention: Parallel Bayesian
Filtering For Efficient Language Modelling and State Tracking"
(gist.science explainer, method §1), whose filter the method claims to
compute exactly (method §2, main contributions).

Diagonal model (one chain per key dim i and value dim j): evidence precision
k_u[i]^2 / r_u and information k_u[i] v_u[j] / r_u (likelihood of
v = k x + N(0, r)).  Isotropic model ("Kalman Delta Networks" abstract: one
uncertainty scalar per head): the chains share the precision increment
b_u = sum_i k_u[i]^2 / (dk r_u) while the information increment stays
k_u[i] v_u[j] / r_u.
"""
from __future__ import annotations

import numpy as np


def chain_filter(l0, eta0, a, qn, P, h):
    """Batched filtering over independent chains.

    l0, eta0: [N]; a, qn, P, h: [N, T].  Returns (prec [N,T], info [N,T]) of
    the filtering posterior of x_t given evidence up to t.
    """
    N, T = a.shape
    prec = np.empty((N, T))
    info = np.empty((N, T))
    for t in range(T):
        n = t + 2
        J = np.zeros((N, n, n))
        hv = np.zeros((N, n))
        J[:, 0, 0] += l0
        hv[:, 0] += eta0
        for u in range(t + 1):
            p, c = u, u + 1
            J[:, p, p] += a[:, u] ** 2 / qn[:, u]
            J[:, c, c] += 1.0 / qn[:, u]
            J[:, p, c] -= a[:, u] / qn[:, u]
            J[:, c, p] -= a[:, u] / qn[:, u]
            J[:, c, c] += P[:, u]
            hv[:, c] += h[:, u]
        sigma = np.linalg.inv(J)
        mu = np.einsum("nij,nj->ni", sigma, hv)
        var = sigma[:, n - 1, n - 1]
        prec[:, t] = 1.0 / var
        info[:, t] = mu[:, n - 1] / var
    return prec, info


def forward(q, k, v, a, qn, r, l0=None, eta0=None, cov="diag"):
    """Filtering outputs of the whole model for every (b,h), fp64.

    Shapes as the oracle: q,k [B,H,T,dk]; v [B,H,T,dv]; r [B,H,T];
    diag: a [B,H,T,dk], qn [H,dk], l0 [B,H,dk]; iso: a, qn [B,H,T], l0 [B,H];
    eta0 [B,H,dk,dv].  Returns dict(o [B,H,T,dv], l_all, etaT).
    """
    q, k, v, a, qn, r = (np.asarray(x, dtype=np.float64) for x in (q, k, v, a, qn, r))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if eta0 is None:
        eta0 = np.zeros((B, H, dk, dv))
    eta0 = np.asarray(eta0, dtype=np.float64)
    if cov == "diag":
        if l0 is None:
            l0 = np.ones((B, H, dk))
        l0 = np.asarray(l0, dtype=np.float64)
        a_c = np.broadcast_to(np.transpose(a, (0, 1, 3, 2))[:, :, :, None, :], (B, H, dk, dv, T))
        qn_c = np.broadcast_to(qn[None, :, :, None, None], (B, H, dk, dv, T))
        P = (np.transpose(k, (0, 1, 3, 2)) ** 2 / r[:, :, None, :])[:, :, :, None, :]
        P = np.broadcast_to(P, (B, H, dk, dv, T))
        l0_c = np.broadcast_to(l0[:, :, :, None], (B, H, dk, dv))
    else:
        if l0 is None:
            l0 = np.ones((B, H))
        l0 = np.asarray(l0, dtype=np.float64)
        a_c = np.broadcast_to(a[:, :, None, None, :], (B, H, dk, dv, T))
        qn_c = np.broadcast_to(qn[:, :, None, None, :], (B, H, dk, dv, T))
        b = (k ** 2).sum(-1) / (dk * r)                                # [B,H,T]
        P = np.broadcast_to(b[:, :, None, None, :], (B, H, dk, dv, T))
        l0_c = np.broadcast_to(l0[:, :, None, None], (B, H, dk, dv))
    # information increment k_u[i] v_u[j] / r_u  -> [B,H,dk,dv,T]
    hh = np.einsum("bhti,bhtj->bhijt", k, v) / r[:, :, None, None, :]
    N = B * H * dk * dv
    prec, info = chain_filter(l0_c.reshape(N), eta0.reshape(N), a_c.reshape(N, T),
                              qn_c.reshape(N, T), P.reshape(N, T), hh.reshape(N, T))
    prec = prec.reshape(B, H, dk, dv, T)
    info = info.reshape(B, H, dk, dv, T)
    mean = info / prec
    o = np.einsum("bhti,bhijt->bhtj", q, mean)
    if cov == "diag":
        l_all = np.transpose(prec[:, :, :, 0, :], (0, 1, 3, 2))         # [B,H,T,dk]
    else:
        l_all = prec[:, :, 0, 0, :]                                     # [B,H,T]
    return {"o": o, "l_all": l_all, "etaT": info[..., -1], "prec_full": prec}
