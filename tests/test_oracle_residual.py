"""Pins of the residual-write oracle (oracle.fwd_residual) against facts fixed
independently of its code:

* one step equals the exact Gaussian posterior computed by dense linear
  algebra (numpy.linalg.solve on the information form) from a diagonal or
  isotropic prior, with the projected precision (diagonal of the posterior
  precision; its trace average for the isotropic family);
* after every step the residual shrinks by the closed-form factor
  r / (k^T P k + r) (P the predicted covariance);
* with d_k = 1, and with one-hot keys, the recurrence reduces to the
  per-key-dim Kalman filter of the KLA oracle (pinned in test_oracle_pins);
* T = 0 passes the state through.

Source: "Kalman Delta Networks: Uncertainty-aware Associative Memory"
(abstract: the Kalman gain weights each residual write; diagonal and
isotropic approximations by online mean-field variational inference).
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")


def _draw(rng, B, H, T, dk, dv, cov):
    q = rng.standard_normal((B, H, T, dk)) / np.sqrt(dk)
    k = rng.standard_normal((B, H, T, dk)) / np.sqrt(dk)
    v = rng.standard_normal((B, H, T, dv))
    if cov == "diag":
        a = 1 / (1 + np.exp(-(1.5 + rng.standard_normal((B, H, T, dk)))))
        qn = 0.05 + 0.2 * rng.random((H, dk))
        l0 = 0.5 + rng.random((B, H, dk))
    else:
        a = 1 / (1 + np.exp(-(1.5 + rng.standard_normal((B, H, T)))))
        qn = 0.05 + 0.2 * rng.random((B, H, T))
        l0 = 0.5 + rng.random((B, H))
    r = 0.2 + rng.random((B, H, T))
    m0 = rng.standard_normal((B, H, dk, dv))
    return q, k, v, a, qn, r, l0, m0


@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_one_step_is_the_dense_gaussian_posterior(cov):
    rng = np.random.default_rng(1)
    dk, dv = 5, 3
    q, k, v, a, qn, r, l0, m0 = _draw(rng, 1, 1, 1, dk, dv, cov)
    c = oracle.DIAG if cov == "diag" else oracle.ISO
    res = oracle.fwd_residual(q, k, v, a, qn, r, l0, m0, cov=c)
    kt, vt, qt, rt = k[0, 0, 0], v[0, 0, 0], q[0, 0, 0], r[0, 0, 0]
    # predicted covariance in variance form: a^2 * (1/l) + qn, mean a * m
    if cov == "diag":
        at, qnt, l = a[0, 0, 0], qn[0], l0[0, 0]
    else:
        at, qnt, l = np.full(dk, a[0, 0, 0]), np.full(dk, qn[0, 0, 0]), np.full(dk, l0[0, 0])
    var_pred = at ** 2 / l + qnt
    m_pred = at[:, None] * m0[0, 0]
    prec = np.diag(1 / var_pred) + np.outer(kt, kt) / rt
    rhs = np.diag(1 / var_pred) @ m_pred + np.outer(kt, vt) / rt
    mean = np.linalg.solve(prec, rhs)
    np.testing.assert_allclose(res["mT"][0, 0], mean, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(res["o"][0, 0, 0], mean.T @ qt, rtol=1e-12, atol=1e-12)
    if cov == "diag":
        np.testing.assert_allclose(res["lT"][0, 0], np.diag(prec), rtol=1e-13)
    else:
        np.testing.assert_allclose(res["lT"][0, 0], np.trace(prec) / dk, rtol=1e-13)


@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_residual_shrinks_by_the_closed_form_factor(cov):
    rng = np.random.default_rng(2)
    dk, dv, T = 6, 4, 8
    q, k, v, a, qn, r, l0, m0 = _draw(rng, 1, 1, T, dk, dv, cov)
    c = oracle.DIAG if cov == "diag" else oracle.ISO
    l, m = l0, m0
    for t in range(T):
        sl = slice(t, t + 1)
        one = oracle.fwd_residual(q[:, :, sl], k[:, :, sl], v[:, :, sl], a[:, :, sl],
                                  qn if cov == "diag" else qn[:, :, sl], r[:, :, sl], l, m, cov=c)
        kt, vt, rt = k[0, 0, t], v[0, 0, t], r[0, 0, t]
        if cov == "diag":
            at, var_pred = a[0, 0, t], a[0, 0, t] ** 2 / l[0, 0] + qn[0]
        else:
            at = np.full(dk, a[0, 0, t])
            var_pred = np.full(dk, a[0, 0, t] ** 2 / l[0, 0] + qn[0, 0, t])
        before = kt @ (at[:, None] * m[0, 0]) - vt
        after = kt @ one["mT"][0, 0] - vt
        factor = rt / (kt @ (var_pred * kt) + rt)
        np.testing.assert_allclose(after, factor * before, rtol=1e-10, atol=1e-12)
        l, m = one["lT"], one["mT"]


@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_single_key_dim_is_the_kla_filter(cov):
    rng = np.random.default_rng(3)
    q, k, v, a, qn, r, l0, m0 = _draw(rng, 2, 3, 40, 1, 5, cov)
    c = oracle.DIAG if cov == "diag" else oracle.ISO
    res = oracle.fwd_residual(q, k, v, a, qn, r, l0, m0, cov=c)
    eta0 = m0 * (l0[..., None] if cov == "diag" else l0[..., None, None])
    ref = oracle.fwd(q, k, v, a, qn, r, l0, eta0, cov=c)
    lT = ref["lT"][..., None] if cov == "diag" else ref["lT"][..., None, None]
    np.testing.assert_allclose(res["o"], ref["o"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(res["lT"], ref["lT"], rtol=1e-13)
    np.testing.assert_allclose(res["mT"], ref["etaT"] / lT, rtol=1e-10, atol=1e-12)


def test_one_hot_keys_are_the_kla_filter():
    """Each token writes one key dim: the residual write touches only that
    row and equals the per-row Kalman update of the KLA recurrence."""
    rng = np.random.default_rng(4)
    B, H, T, dk, dv = 2, 2, 30, 6, 4
    q, k, v, a, qn, r, l0, m0 = _draw(rng, B, H, T, dk, dv, "diag")
    idx = rng.integers(0, dk, size=(B, H, T))
    k = np.zeros((B, H, T, dk))
    np.put_along_axis(k, idx[..., None], (0.5 + rng.random((B, H, T)))[..., None], axis=-1)
    res = oracle.fwd_residual(q, k, v, a, qn, r, l0, m0, cov=oracle.DIAG)
    ref = oracle.fwd(q, k, v, a, qn, r, l0, m0 * l0[..., None], cov=oracle.DIAG)
    np.testing.assert_allclose(res["o"], ref["o"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(res["lT"], ref["lT"], rtol=1e-13)
    np.testing.assert_allclose(res["mT"], ref["etaT"] / ref["lT"][..., None], rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_empty_sequence_passes_the_state_through(cov):
    rng = np.random.default_rng(5)
    q, k, v, a, qn, r, l0, m0 = _draw(rng, 2, 2, 0, 4, 3, cov)
    c = oracle.DIAG if cov == "diag" else oracle.ISO
    res = oracle.fwd_residual(q, k, v, a, qn, r, l0, m0, cov=c)
    np.testing.assert_array_equal(res["lT"], l0)
    np.testing.assert_array_equal(res["mT"], m0)
