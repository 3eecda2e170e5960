"""The chunked form of the residual-write forward, step by step in fp64 numpy,
against the sequential oracle (oracle.fwd_residual).  This checks the algebra
the chunked kernel is built on, not the kernel (which tests/test_gpu_residual.py
compares with the oracle on the GPU).

Per (b,h) and chunk of C tokens from the state M0 at its start, with
G_t = a_1 ... a_t per key dim, Kt = G (.) K, Qt = G (.) Q, c = k / lp,
den = k.c + r, Ch = C / G and u'_s = u_s / den_s:
  (diag(den) + strictlower(Kt Ch^T)) U' = V - Kt M0
  O   = Qt M0 + lower(Qt Ch^T) U'
  M_C = G_C (.) M0 + E^T U',   E_s = (a_{s+1} ... a_C) (.) c_s
Key dims whose G leaves [2^-64, 2^64] within a chunk (per group of 64, as a
wave of the kernel) take the exact pair sums D(s,t) k_t c_s instead of the
quotient Ch.  Both paths, a ragged last chunk and a handed-over state are
covered; a dropped term or a transposed operand in the algebra breaks them.
"""
import numpy as np
import pytest
import torch

import oracle
from scan_amd import inputs as gen

C = 16
LO, HI = 2.0 ** -64, 2.0 ** 64


def _chunked(q, k, v, a, qn, r, l0, m0, exact=False, mutant=None):
    B, H, T, D = q.shape
    o = np.zeros((B, H, T, D))
    lT = np.zeros((B, H, D))
    mT = np.zeros((B, H, D, D))
    for b in range(B):
        for h in range(H):
            l, M = l0[b, h].copy(), m0[b, h].copy()
            for c0 in range(0, T, C):
                n = min(C, T - c0)
                K, Q, V = np.zeros((C, D)), np.zeros((C, D)), np.zeros((C, D))
                A, R = np.ones((C, D)), np.ones(C)
                K[:n], Q[:n], V[:n] = k[b, h, c0:c0 + n], q[b, h, c0:c0 + n], v[b, h, c0:c0 + n]
                A[:n], R[:n] = a[b, h, c0:c0 + n], r[b, h, c0:c0 + n]
                cv, gm, g = np.zeros((C, D)), np.zeros((C, D)), np.ones(D)
                for u in range(C):
                    lp = l / (qn[h] * l + A[u] ** 2)
                    cv[u] = K[u] / lp
                    if u < n:
                        l = K[u] ** 2 / R[u] + lp
                    g = g * A[u]
                    gm[u] = g
                den = (K * cv).sum(1) + R
                inr = np.all((gm >= LO) & (gm <= HI), axis=0)
                grp = np.array([inr[w:w + 64].all() for w in range(0, D, 64)])
                fac = np.repeat(grp, 64)[:D] if D >= 64 else np.full(D, grp[0])
                if exact:
                    fac[:] = False
                Kt, Qt = gm * K, gm * Q
                Ch = np.where(fac[None, :], cv / gm, 0.0)
                GK, GQ = Kt @ Ch.T, Qt @ Ch.T
                for t in range(C):
                    for s in range(t + 1):
                        dst = np.prod(A[s + 1:t + 1], axis=0) if s < t else np.ones(D)
                        GK[t, s] += np.sum((dst * K[t] * cv[s])[~fac])
                        GQ[t, s] += np.sum((dst * Q[t] * cv[s])[~fac])
                low = np.zeros_like(GK) if mutant == "no coupling" else np.tril(GK, -1)
                Tp = np.linalg.inv(np.diag(den) + low)
                E, sfx = np.zeros((C, D)), np.ones(D)
                for u in range(C - 1, -1, -1):
                    E[u] = sfx * cv[u]
                    sfx = sfx * (1.0 if mutant == "no decay in E" else A[u])
                U = Tp @ (V - Kt @ M)
                CQ = np.tril(GQ, -1) if mutant == "strict readout" else np.tril(GQ)
                O = Qt @ M + CQ @ U
                gC = gm[0] if mutant == "first decay carried" else gm[-1]
                M = gC[:, None] * M + E.T @ U
                o[b, h, c0:c0 + n] = O[:n]
            lT[b, h], mT[b, h] = l, M
    return o, lT, mT


def _check(inp, st=None, exact=False, tol=1e-12, mutant=None):
    f = lambda x: x.double().numpy()  # noqa: E731
    q, k, v, a, r, qn = (f(inp[n]) for n in ("q", "k", "v", "a", "r", "qn"))
    B, H, T, D = q.shape
    l0 = f(st["l0"]) if st else np.ones((B, H, D))
    m0 = f(st["eta0"]) if st else np.zeros((B, H, D, D))
    o, lT, mT = _chunked(q, k, v, a, qn, r, l0, m0, exact, mutant)
    ref = oracle.fwd_residual(inp["q"], inp["k"], inp["v"], inp["a"], inp["qn"], inp["r"],
                              st["l0"] if st else None, st["eta0"] if st else None, cov=oracle.DIAG)
    assert np.abs(o - ref["o"]).max() <= tol * np.abs(ref["o"]).max()
    assert np.abs(mT - ref["mT"]).max() <= tol * np.abs(ref["mT"]).max()
    assert (np.abs(lT - ref["lT"]) / ref["lT"]).max() <= tol


@pytest.mark.parametrize("T", [1, 16, 17, 40])
@pytest.mark.parametrize("exact", [False, True])
def test_chunk_algebra_matches_oracle(T, exact):
    inp = gen.make_inputs("small_diag", seed=90 + T, B=1, H=2, T=T, dk=64, dv=64, dtype="f32")
    _check(inp, gen.make_state(inp["workload"], seed=17), exact=exact)


def test_chunk_algebra_fast_decay_takes_exact_sums():
    """a = 0.01 (every 7th token 0.9): G falls below 2^-64 within a chunk."""
    T = 45
    inp = gen.make_inputs("small_diag", seed=24, B=1, H=2, T=T, dk=64, dv=64, dtype="f32")
    a = torch.full(inp["a"].shape, 0.01)
    a[:, :, ::7] = 0.9
    inp["a"] = a
    inp["r"] = torch.full((1, 2, T), 1e-3)
    g = torch.Generator().manual_seed(25)
    inp["k"] = 5 * (2 * torch.rand(1, 2, T, 64, generator=g) - 1)
    _check(inp)


def test_chunk_algebra_half_the_key_dims_off():
    """d 128: key dims 0..63 leave the factorisation range, 64..127 do not."""
    inp = gen.make_inputs("small_diag", seed=5, B=1, H=1, T=40, dk=128, dv=128, dtype="f32")
    a = inp["a"].clone()
    a[..., :64] = 0.02
    inp["a"] = a
    _check(inp)


@pytest.mark.parametrize("mutant", ["no coupling", "no decay in E", "strict readout",
                                    "first decay carried"])
def test_chunk_algebra_catches_planted_mistakes(mutant):
    """The comparison is sharp: each planted mistake in the chunk steps fails it."""
    inp = gen.make_inputs("small_diag", seed=7, B=1, H=1, T=40, dk=64, dv=64, dtype="f32")
    with pytest.raises(AssertionError):
        _check(inp, gen.make_state(inp["workload"], seed=8), mutant=mutant)
