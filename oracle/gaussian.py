"""Exact-rational joint-Gaussian filtering posteriors (TEST INFRASTRUCTURE ONLY).

An independent definition of what the KLA recurrence must produce: the
filtering posterior of each scalar chain of the linear-Gaussian model of
"Kalman Linear Attention: Parallel Bayesian Filtering For Efficient Language
Modelling and State Tracking" (gist.science explainer, method §1: OU prior
with process noise, noisy observation through the key, readout of the
posterior mean through the query), obtained by writing out the joint density
of the chain and marginalising it with exact Gauss-Jordan elimination over
``fractions.Fraction``.  No recursion of any kind is used, so agreement with
the sequential oracle pins the oracle's predict/update/readout algebra.

Chain (i, j), variables x_{-1}, x_0 .. x_t:
  prior      exp(-l0/2 x_{-1}^2 + eta0 x_{-1})
  transition x_u | x_{u-1} ~ N(a_u x_{u-1}, qn_u)            (qn_u > 0)
  evidence   exp(-P_u/2 x_u^2 + h_u x_u) with, for the diagonal model,
             P_u = k_u^2 / r_u and h_u = k_u v_u / r_u (the likelihood of
             v_u = k_u x_u + N(0, r_u)).
The filtered precision at t is 1/Cov[x_t, x_t], the information is
E[x_t] / Cov[x_t, x_t].
"""
from __future__ import annotations

from fractions import Fraction as Fr


def _solve_exact(J, h):
    """Return (Sigma, mu) = (J^-1, J^-1 h) by Gauss-Jordan elimination on Fractions."""
    n = len(J)
    aug = [list(J[r]) + [h[r]] + [Fr(int(r == c)) for c in range(n)] for r in range(n)]
    for col in range(n):
        piv = next(r for r in range(col, n) if aug[r][col] != 0)
        aug[col], aug[piv] = aug[piv], aug[col]
        p = aug[col][col]
        aug[col] = [x / p for x in aug[col]]
        for r in range(n):
            if r != col and aug[r][col] != 0:
                f = aug[r][col]
                aug[r] = [x - f * y for x, y in zip(aug[r], aug[col])]
    mu = [aug[r][n] for r in range(n)]
    sigma = [[aug[r][n + 1 + c] for c in range(n)] for r in range(n)]
    return sigma, mu


def chain_posteriors(l0, eta0, a, qn, P, h):
    """Filtering posteriors (precision, information) after every step of one chain.

    All arguments are Fractions (lists of length T for a, qn, P, h).
    Returns two lists of length T.
    """
    T = len(a)
    precs, infos = [], []
    for t in range(T):
        n = t + 2                        # x_{-1} .. x_t
        J = [[Fr(0)] * n for _ in range(n)]
        hv = [Fr(0)] * n
        J[0][0] += l0
        hv[0] += eta0
        for u in range(t + 1):
            p, c = u, u + 1
            J[p][p] += a[u] * a[u] / qn[u]
            J[c][c] += 1 / qn[u]
            J[p][c] -= a[u] / qn[u]
            J[c][p] -= a[u] / qn[u]
            J[c][c] += P[u]
            hv[c] += h[u]
        sigma, mu = _solve_exact(J, hv)
        var = sigma[n - 1][n - 1]
        precs.append(1 / var)
        infos.append(mu[n - 1] / var)
    return precs, infos


def diag_forward_exact(q, k, v, a, qn, r, l0, eta0):
    """Exact outputs of the diagonal model for ONE (b,h) sequence.

    q,k: T x dk; v: T x dv; a: T x dk; qn: dk; r: T; l0: dk; eta0: dk x dv
    (nested lists of Fractions).  Returns (o [T][dv], l [T][dk], eta_T [dk][dv]).
    """
    T, dk, dv = len(q), len(q[0]), len(v[0])
    l_hist = [[None] * dk for _ in range(T)]
    means = [[[None] * dv for _ in range(dk)] for _ in range(T)]
    etaT = [[None] * dv for _ in range(dk)]
    for i in range(dk):
        for j in range(dv):
            P = [k[u][i] * k[u][i] / r[u] for u in range(T)]
            hh = [k[u][i] * v[u][j] / r[u] for u in range(T)]
            precs, infos = chain_posteriors(l0[i], eta0[i][j], [a[u][i] for u in range(T)],
                                            [qn[i]] * T, P, hh)
            for t in range(T):
                l_hist[t][i] = precs[t]
                means[t][i][j] = infos[t] / precs[t]
            etaT[i][j] = infos[T - 1]
    o = [[sum(q[t][i] * means[t][i][j] for i in range(dk)) for j in range(dv)]
         for t in range(T)]
    return o, l_hist, etaT
