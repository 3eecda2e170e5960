"""The chunked form of the backward pass, step by step in fp64 numpy, against
the sequential backward oracle (oracle.bwd).  This checks the algebra the
chunked backward kernels are built on, not the kernels (tests/test_gpu_bwd.py
compares those with the oracle on the GPU).

Per (b,h), diagonal precision, chunks of C tokens; within a chunk
G_t = g_1 ... g_t per key dim (prefix decays from the chunk start),
E_t = g_{t+1} ... g_C (suffix), qh = q / l, w = k / r, A = G (.) qh.
Forward sweep, from the state eta_in at the chunk start:
  S   = G (.) (dO eta_in^T) + G (.) (lower(dO V^T) (W / G))     dq = S / l
  eta_out = G_C (.) (eta_in + (W / G)^T V)
Reverse sweep, from the adjoint eps_out entering the chunk from its end:
  U   = (1 / G) (.) (G_C (.) (V eps_out^T) + upper(V dO^T) A)
  dV  = (W / G) (G_C (.) eps_out) + upper((W / G) A^T) dO
  eps_in = G_C (.) eps_out + A^T dO
The adjoint of log g telescopes into a reverse cumulative sum of per-token
terms, dlog g_t = <detaT, eta_T> + sum_{s >= t} (qh_s S_s - w_s U_s), and the
precision adjoint is one scalar reverse recursion per key dim.  A dropped
term, a wrong triangle or a shifted sum breaks the comparison.
"""
import numpy as np
import pytest

import oracle
from scan_amd import inputs as gen

C = 16


def _chunked_bwd(q, k, v, a, qn, r, l0, eta0, dO, dlT, detaT, mutant=None):
    T, D = q.shape
    nch = (T + C - 1) // C

    def chain(c, l):
        """Precision recursion over chunk c from l (the precision before it)."""
        c0, n = c * C, min(C, T - c * C)
        lprev, lt, g, Dn = (np.zeros((n, D)) for _ in range(4))
        for u in range(n):
            lprev[u] = l
            Dn[u] = a[c0 + u] ** 2 + qn * l
            g[u] = a[c0 + u] / Dn[u]
            l = l / Dn[u] + k[c0 + u] ** 2 / r[c0 + u]
            lt[u] = l
        return c0, n, lprev, lt, g, Dn, np.cumprod(g, axis=0)

    # forward sweep: dq, the per-token terms qh S, the precision at chunk starts
    l, eta = l0.copy(), eta0.copy()
    lstart, Qs, dq = np.zeros((nch, D)), np.zeros((T, D)), np.zeros((T, D))
    for c in range(nch):
        lstart[c] = l
        c0, n, _, lt, g, _, G = chain(c, l)
        l = lt[-1]
        qh, W = q[c0:c0 + n] / lt, k[c0:c0 + n] / r[c0:c0 + n, None]
        V, dOc = v[c0:c0 + n], dO[c0:c0 + n]
        low = np.tril(dOc @ V.T, -1 if mutant == "strict lower in S" else 0)
        S = G * (dOc @ eta.T) + G * (low @ (W / G))
        dq[c0:c0 + n] = S / lt
        Qs[c0:c0 + n] = qh * S
        eta = G[-1][:, None] * (eta + (W / G).T @ V)
    cum = (detaT * eta).sum(1)
    # reverse sweep
    eps, lbar = detaT.copy(), dlT.copy()
    dk, dv, da = np.zeros((T, D)), np.zeros((T, D)), np.zeros((T, D))
    dr, dqn = np.zeros(T), np.zeros(D)
    for c in range(nch - 1, -1, -1):
        c0, n, lprev, lt, g, Dn, G = chain(c, lstart[c])
        gC = G[-1]
        qh, W = q[c0:c0 + n] / lt, k[c0:c0 + n] / r[c0:c0 + n, None]
        V, dOc = v[c0:c0 + n], dO[c0:c0 + n]
        A = G * qh
        up = np.triu(V @ dOc.T, 1 if mutant == "strict upper in U" else 0)
        U = (gC * (V @ eps.T) + up @ A) / G
        dV = (W / G) @ (gC[:, None] * eps) + np.triu((W / G) @ A.T) @ dOc
        eps = (1.0 if mutant == "no decay of the adjoint" else gC[:, None]) * eps + A.T @ dOc
        dv[c0:c0 + n] = dV
        for u in range(n - 1, -1, -1):
            t = c0 + u
            if mutant == "cumulative sum one token late":
                dl = cum.copy()
                cum = cum + Qs[t] - W[u] * U[u]
            else:
                cum = cum + Qs[t] - W[u] * U[u]
                dl = cum
            lbar = lbar - Qs[t] / lt[u]
            rd = 1.0 / Dn[u]
            dk[t] = U[u] / r[t] + 2 * lbar * k[t] / r[t]
            dr[t] = -np.sum(k[t] * U[u] + lbar * k[t] ** 2) / r[t] ** 2
            da[t] = -2 * lbar * a[t] * lprev[u] * rd ** 2 + dl * (qn * lprev[u] - a[t] ** 2) * rd / a[t]
            dqn += -lbar * lprev[u] ** 2 * rd ** 2 - dl * lprev[u] * rd
            lbar = lbar * a[t] ** 2 * rd ** 2 - dl * qn * rd
    return dict(dq=dq, dk=dk, dv=dv, da=da, dr=dr, dqn=dqn, dl0=lbar, deta0=eps)


def _chunked_bwd_iso(q, k, v, a, qn, r, l0, eta0, dO, dlT, detaT):
    """Isotropic: the precision, decay and process noise are scalars per
    token (l_t = l_{t-1} / D_t + |k_t|^2 / (dk r_t)), so G is one scalar per
    token and key dim alike; dlog g and lbar are the head's scalars, the
    per-token terms summed over the key dims."""
    T, D = q.shape
    nch = (T + C - 1) // C

    def chain(c, l):
        c0, n = c * C, min(C, T - c * C)
        lprev, lt, g, Dn = (np.zeros(n) for _ in range(4))
        for u in range(n):
            lprev[u] = l
            Dn[u] = a[c0 + u] ** 2 + qn[c0 + u] * l
            g[u] = a[c0 + u] / Dn[u]
            l = l / Dn[u] + np.sum(k[c0 + u] ** 2) / (D * r[c0 + u])
            lt[u] = l
        return c0, n, lprev, lt, g, Dn, np.cumprod(g)[:, None] * np.ones((1, D))

    l, eta = float(l0), eta0.copy()
    lstart, Qs, dq = np.zeros(nch), np.zeros((T, D)), np.zeros((T, D))
    for c in range(nch):
        lstart[c] = l
        c0, n, _, lt, g, _, G = chain(c, l)
        l = lt[-1]
        qh, W = q[c0:c0 + n] / lt[:, None], k[c0:c0 + n] / r[c0:c0 + n, None]
        V, dOc = v[c0:c0 + n], dO[c0:c0 + n]
        S = G * (dOc @ eta.T) + G * (np.tril(dOc @ V.T) @ (W / G))
        dq[c0:c0 + n] = S / lt[:, None]
        Qs[c0:c0 + n] = qh * S
        eta = G[-1][:, None] * (eta + (W / G).T @ V)
    cum = float((detaT * eta).sum())
    eps, lbar = detaT.copy(), float(dlT)
    dk, dv = np.zeros((T, D)), np.zeros((T, D))
    da, dr, dqn = np.zeros(T), np.zeros(T), np.zeros(T)
    for c in range(nch - 1, -1, -1):
        c0, n, lprev, lt, g, Dn, G = chain(c, lstart[c])
        gC = G[-1]
        qh, W = q[c0:c0 + n] / lt[:, None], k[c0:c0 + n] / r[c0:c0 + n, None]
        V, dOc = v[c0:c0 + n], dO[c0:c0 + n]
        A = G * qh
        U = (gC * (V @ eps.T) + np.triu(V @ dOc.T) @ A) / G
        dv[c0:c0 + n] = (W / G) @ (gC[:, None] * eps) + np.triu((W / G) @ A.T) @ dOc
        eps = gC[:, None] * eps + A.T @ dOc
        for u in range(n - 1, -1, -1):
            t = c0 + u
            cum = cum + np.sum(Qs[t] - W[u] * U[u])
            lbar = lbar - np.sum(Qs[t]) / lt[u]
            rd = 1.0 / Dn[u]
            dk[t] = U[u] / r[t] + 2 * lbar * k[t] / (D * r[t])
            dr[t] = -(np.sum(k[t] * U[u]) + lbar * np.sum(k[t] ** 2) / D) / r[t] ** 2
            da[t] = -2 * lbar * a[t] * lprev[u] * rd ** 2 + cum * (qn[t] * lprev[u] - a[t] ** 2) * rd / a[t]
            dqn[t] = -lbar * lprev[u] ** 2 * rd ** 2 - cum * lprev[u] * rd
            lbar = lbar * a[t] ** 2 * rd ** 2 - cum * qn[t] * rd
    return dict(dq=dq, dk=dk, dv=dv, da=da, dr=dr, dqn=dqn, dl0=lbar, deta0=eps)


def _check(inp, up, st=None, tol=1e-11, mutant=None):
    f = lambda x: x.double().numpy()  # noqa: E731
    q, k, v, a, qn, r = (f(inp[n]) for n in ("q", "k", "v", "a", "qn", "r"))
    B, H, T, D = q.shape
    dO, dlT, detaT = f(up["do"]), f(up["dlT"]), f(up["detaT"])
    l0 = f(st["l0"]) if st else np.ones((B, H, D))
    e0 = f(st["eta0"]) if st else np.zeros((B, H, D, D))
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["qn"], inp["r"],
                     st["l0"] if st else None, st["eta0"] if st else None, do=up["do"],
                     dlT=up["dlT"], detaT=up["detaT"], cov=oracle.DIAG)
    dqn = np.zeros((H, D))
    for b in range(B):
        for h in range(H):
            got = _chunked_bwd(q[b, h], k[b, h], v[b, h], a[b, h], qn[h], r[b, h], l0[b, h], e0[b, h],
                               dO[b, h], dlT[b, h], detaT[b, h], mutant)
            dqn[h] += got["dqn"]
            for n in ("dq", "dk", "dv", "da", "dr", "dl0", "deta0"):
                x, y = got[n], ref[n][b, h]
                assert np.abs(x - y).max() <= tol * np.abs(y).max(), (n, b, h)
    assert np.abs(dqn - ref["dqn"]).max() <= tol * np.abs(ref["dqn"]).max()


@pytest.mark.parametrize("T", [1, 16, 17, 45])
def test_bwd_chunk_algebra_matches_oracle(T):
    inp = gen.make_inputs("small_diag", seed=60 + T, B=2, H=2, T=T, dk=16, dv=16, dtype="f32")
    w = inp["workload"]
    _check(inp, gen.make_upstream(w, seed=61), gen.make_state(w, seed=62))


def test_bwd_chunk_algebra_lm_distribution():
    """The LM layer's value laws (bf16 inputs), default state."""
    inp = gen.make_inputs("lm_diag", seed=63, B=1, H=1, T=70, dk=32, dv=32)
    _check(inp, gen.make_upstream(inp["workload"], seed=64))


@pytest.mark.parametrize("mutant", ["strict lower in S", "strict upper in U", "no decay of the adjoint",
                                    "cumulative sum one token late"])
def test_bwd_chunk_algebra_catches_planted_mistakes(mutant):
    inp = gen.make_inputs("small_diag", seed=65, B=1, H=1, T=40, dk=16, dv=16, dtype="f32")
    w = inp["workload"]
    with pytest.raises(AssertionError):
        _check(inp, gen.make_upstream(w, seed=66), gen.make_state(w, seed=67), mutant=mutant)


@pytest.mark.parametrize("T", [1, 17, 45])
def test_bwd_chunk_algebra_isotropic(T):
    """The isotropic chunk algebra (scalar precision and decay per token, the
    gate adjoint and lbar summed over the key dims) against the oracle."""
    inp = gen.make_inputs("iso", seed=70 + T, B=1, H=2, T=T, dk=16, dv=16, dtype="f32")
    w = inp["workload"]
    up = gen.make_upstream(w, seed=71)
    st = gen.make_state(w, seed=72)
    f = lambda x: x.double().numpy()  # noqa: E731
    q, k, v, a, qn, r = (f(inp[n]) for n in ("q", "k", "v", "a", "qn", "r"))
    dO, dlT, detaT = f(up["do"]), f(up["dlT"]), f(up["detaT"])
    l0, e0 = f(st["l0"]), f(st["eta0"])
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["qn"], inp["r"], st["l0"], st["eta0"],
                     do=up["do"], dlT=up["dlT"], detaT=up["detaT"], cov=oracle.ISO)
    for h in range(2):
        got = _chunked_bwd_iso(q[0, h], k[0, h], v[0, h], a[0, h], qn[0, h], r[0, h], l0[0, h], e0[0, h],
                               dO[0, h], dlT[0, h], detaT[0, h])
        for n in ("dq", "dk", "dv", "da", "dr", "dqn", "dl0", "deta0"):
            x, y = np.asarray(got[n]), np.asarray(ref[n][0, h])
            assert np.abs(x - y).max() <= 1e-11 * np.abs(y).max(), (n, h)
