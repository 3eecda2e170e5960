"""Pins for the fp64 backward oracle (oracle.bwd, the reverse-mode adjoint of
the sequential recurrence).

The backward is the other half of training the filter as a sequence-model
primitive ("Kalman Linear Attention: Parallel Bayesian Filtering For
Efficient Language Modelling and State Tracking", fugumt abstract page:
efficient parallel training).  Its result is fixed by the forward: it is the
gradient of L = <dO, o> + <dlT, lT> + <detaT, etaT>.  Pinned against
* central finite differences of the fp64 forward oracle (every input);
* automatic differentiation of an independently written plain torch forward;
* closed-form gradients at a = 1, qn = 0, where the forward is normalised
  linear attention (cumulative sums);
* T = 0 (pass-through) and the split-sequence handoff of the adjoint state;
* a mutation test: planted mistakes in a copy of the source each fail a pin.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle_pins import rand_case

DIAG, ISO = oracle.DIAG, oracle.ISO
NAMES = ("q", "k", "v", "a", "qn", "r", "l0", "eta0")


def upstream(c, cov, seed):
    rng = np.random.default_rng(seed)
    B, H, T, dk = c["q"].shape
    dv = c["v"].shape[-1]
    return dict(do=rng.normal(size=(B, H, T, dv)),
                dlT=rng.normal(size=(B, H, dk) if cov == "diag" else (B, H)),
                detaT=rng.normal(size=(B, H, dk, dv)))


def loss(c, u, cov, lib_path=None):
    out = oracle.fwd(*(c[n] for n in NAMES), cov=DIAG if cov == "diag" else ISO, lib_path=lib_path)
    return float((out["o"] * u["do"]).sum() + (out["lT"] * u["dlT"]).sum()
                 + (out["etaT"] * u["detaT"]).sum())


def grads(c, u, cov, lib_path=None):
    return oracle.bwd(*(c[n] for n in NAMES), do=u["do"], dlT=u["dlT"], detaT=u["detaT"],
                      cov=DIAG if cov == "diag" else ISO, lib_path=lib_path)


def fd_check(c, u, cov, g, name, seed, eps=1e-6):
    """Directional derivative along a random direction, central differences."""
    rng = np.random.default_rng(seed)
    x = c[name]
    e = rng.normal(size=x.shape)
    cp = dict(c, **{name: x + eps * e})
    cm = dict(c, **{name: x - eps * e})
    fd = (loss(cp, u, cov) - loss(cm, u, cov)) / (2 * eps)
    an = float((g["d" + name] * e).sum())
    return abs(fd - an) / max(abs(an), 1e-12)


@pytest.mark.parametrize("cov", ["diag", "iso"])
@pytest.mark.parametrize("seed", [1, 2])
def test_finite_differences_every_input(cov, seed):
    c = rand_case(seed, B=2, H=2, T=7, dk=3, dv=2, cov=cov)
    u = upstream(c, cov, seed + 10)
    g = grads(c, u, cov)
    for name in NAMES:
        err = fd_check(c, u, cov, g, name, seed + 20)
        assert err < 1e-6, (name, err)


def test_finite_differences_elementwise_small():
    """Every element of every gradient, one coordinate at a time (tiny case)."""
    c = rand_case(5, B=1, H=1, T=4, dk=2, dv=2, cov="diag")
    u = upstream(c, "diag", 6)
    g = grads(c, u, "diag")
    eps = 1e-6
    for name in NAMES:
        x = c[name]
        for idx in np.ndindex(*x.shape):
            e = np.zeros_like(x)
            e[idx] = 1.0
            fd = (loss(dict(c, **{name: x + eps * e}), u, "diag")
                  - loss(dict(c, **{name: x - eps * e}), u, "diag")) / (2 * eps)
            an = g["d" + name][idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, idx, fd, an)


def torch_forward(c, cov):
    """The recurrence written out again in plain torch fp64 (information form,
    one token at a time), for automatic differentiation."""
    q, k, v, a, qn, r, l0, eta0 = (c[n] for n in NAMES)
    B, H, T, dk = q.shape
    outs = []
    l, eta = l0, eta0
    for t in range(T):
        kt, vt, rt = k[:, :, t], v[:, :, t], r[:, :, t]
        if cov == "diag":
            at = a[:, :, t]
            pred_var = at * at / l + qn[None]           # a^2 / l + qn
            lp = 1.0 / pred_var
            gate = lp * at / l
            l_new = lp + kt * kt / rt[..., None]
            eta = gate[..., None] * eta + kt[..., None] * vt[:, :, None, :] / rt[..., None, None]
            l = l_new
            o = torch.einsum("bhi,bhij->bhj", q[:, :, t] / l, eta)
        else:
            at, qt_ = a[:, :, t], qn[:, :, t]
            lp = 1.0 / (at * at / l + qt_)
            gate = lp * at / l
            l = lp + (kt * kt).sum(-1) / (dk * rt)
            eta = gate[..., None, None] * eta + kt[..., None] * vt[:, :, None, :] / rt[..., None, None]
            o = torch.einsum("bhi,bhij->bhj", q[:, :, t] / l[..., None], eta)
        outs.append(o)
    return torch.stack(outs, dim=2), l, eta


@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_autograd_of_plain_torch_forward(cov):
    c = rand_case(3, B=2, H=2, T=9, dk=4, dv=3, cov=cov)
    u = upstream(c, cov, 4)
    g = grads(c, u, cov)
    tc = {n: torch.tensor(c[n], dtype=torch.float64, requires_grad=True) for n in NAMES}
    o, lT, etaT = torch_forward(tc, cov)
    L = ((o * torch.tensor(u["do"])).sum() + (lT * torch.tensor(u["dlT"])).sum()
         + (etaT * torch.tensor(u["detaT"])).sum())
    L.backward()
    for n in NAMES:
        ref = tc[n].grad.numpy()
        err = np.abs(g["d" + n] - ref).max() / np.abs(ref).max()
        assert err < 1e-12, (n, err)


@pytest.mark.parametrize("state", [True, False])
def test_closed_form_a1_qn0(state):
    """a = 1, qn = 0: L_t = l0 + cumsum k^2/r and E_t = eta0 + cumsum k v^T/r,
    o_t[j] = sum_i q_t[i] E_t[i,j] / L_t[i].  Differentiating these sums by
    hand gives
      dq_t[i]    = S_t[i] / L_t[i],      S_t[i] = sum_j dO_t[j] E_t[i,j]
      dv_s[j]    = sum_i k_s[i]/r_s (sum_{t>=s} q_t[i] dO_t[j] / L_t[i] + detaT[i,j])
      deta0[i,j] = sum_t q_t[i] dO_t[j] / L_t[i] + detaT[i,j]
      dl0[i]     = -sum_t q_t[i] S_t[i] / L_t[i]^2 + dlT[i]."""
    c = rand_case(8, B=1, H=2, T=6, dk=3, dv=2, cov="diag", state=state)
    c["a"] = np.ones_like(c["a"])
    c["qn"] = np.zeros_like(c["qn"])
    u = upstream(c, "diag", 9)
    g = grads(c, u, "diag")
    q, k, v, r = c["q"], c["k"], c["v"], c["r"]
    B, H, T, dk = q.shape
    l0 = c["l0"] if state else np.ones((B, H, dk))
    eta0 = c["eta0"] if state else np.zeros((B, H, dk, v.shape[-1]))
    L = l0[:, :, None] + np.cumsum(k * k / r[..., None], axis=2)
    E = eta0[:, :, None] + np.cumsum(k[..., None] * v[:, :, :, None, :] / r[..., None, None], axis=2)
    dO = u["do"]
    S = np.einsum("bhtj,bhtij->bhti", dO, E)
    np.testing.assert_allclose(g["dq"], S / L, rtol=1e-12, atol=1e-13)
    W = q[..., None] * dO[:, :, :, None, :] / L[..., None]            # [b,h,t,i,j]
    tail = np.cumsum(W[:, :, ::-1], axis=2)[:, :, ::-1] + u["detaT"][:, :, None]
    dv = np.einsum("bhsi,bhsij->bhsj", k / r[..., None], tail)
    np.testing.assert_allclose(g["dv"], dv, rtol=1e-12, atol=1e-13)
    if state:
        np.testing.assert_allclose(g["deta0"], W.sum(axis=2) + u["detaT"], rtol=1e-12, atol=1e-13)
        dl0 = -(q * S / L ** 2).sum(axis=2) + u["dlT"]
        np.testing.assert_allclose(g["dl0"], dl0, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_empty_sequence_passes_state_gradient(cov):
    c = rand_case(11, B=2, H=2, T=0, dk=3, dv=2, cov=cov)
    u = upstream(c, cov, 12)
    g = grads(c, u, cov)
    np.testing.assert_array_equal(g["dl0"], u["dlT"])
    np.testing.assert_array_equal(g["deta0"], u["detaT"])


@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_split_handoff_of_the_adjoint(cov):
    """Backward over [0, T) equals the backward over [T1, T) from the forward
    state at T1, followed by the backward over [0, T1) with the adjoint of that
    state as its final-state gradient."""
    T, T1 = 9, 4
    c = rand_case(13, B=1, H=2, T=T, dk=3, dv=2, cov=cov)
    u = upstream(c, cov, 14)
    g = grads(c, u, cov)
    tok = ("q", "k", "v", "a", "r") + (("qn",) if cov == "iso" else ())
    first = dict(c, **{n: c[n][:, :, :T1] for n in tok})
    second = dict(c, **{n: c[n][:, :, T1:] for n in tok})
    mid = oracle.fwd(*(first[n] for n in NAMES), cov=DIAG if cov == "diag" else ISO)
    second["l0"], second["eta0"] = mid["lT"], mid["etaT"]
    u2 = dict(u, do=u["do"][:, :, T1:])
    g2 = grads(second, u2, cov)
    u1 = dict(do=u["do"][:, :, :T1], dlT=g2["dl0"], detaT=g2["deta0"])
    g1 = grads(first, u1, cov)
    for n in ("dq", "dk", "dv", "da", "dr"):
        np.testing.assert_allclose(np.concatenate([g1[n], g2[n]], axis=2), g[n], rtol=1e-10, atol=1e-12)
    for n in ("dl0", "deta0"):
        np.testing.assert_allclose(g1[n], g[n], rtol=1e-10, atol=1e-12)
    dqn = g1["dqn"] + g2["dqn"] if cov == "diag" else np.concatenate([g1["dqn"], g2["dqn"]], axis=2)
    np.testing.assert_allclose(dqn, g["dqn"], rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- mutation test

_SRC = os.path.join(os.path.dirname(oracle.__file__), "kla_oracle.c")

MUTANTS = {
    "readout_adjoint_drops_l": ("ebar[(size_t)i * dv + j] += qt[i] * dOt[j] / li;",
                                "ebar[(size_t)i * dv + j] += qt[i] * dOt[j];"),
    "lbar_readout_sign": ("lbar[(cov == KLA_ORACLE_DIAG) ? i : 0] -= qt[i] * (s / li) / li;",
                          "lbar[(cov == KLA_ORACLE_DIAG) ? i : 0] += qt[i] * (s / li) / li;"),
    "gbar_uses_new_state": ("gb += ebar[(size_t)i * dv + j] * ep_[(size_t)i * dv + j];",
                            "gb += ebar[(size_t)i * dv + j] * et_[(size_t)i * dv + j];"),
    "dv_drops_r": ("dvv[(size_t)t * dv + j] += ebar[(size_t)i * dv + j] * kt[i] / rt;",
                   "dvv[(size_t)t * dv + j] += ebar[(size_t)i * dv + j] * kt[i];"),
    "dk_precision_factor": ("dkk[(size_t)t * dk + i] += lb * 2.0 * kt[i] / rt;",
                            "dkk[(size_t)t * dk + i] += lb * kt[i] / rt;"),
    "da_gate_term": ("gb * (qni * lprev - ai * ai) / den2;", "gb * (qni * lprev + ai * ai) / den2;"),
    "dqn_drops_gate": ("dqn_acc[i] += -lb * lprev * lprev / den2 - gb * ai * lprev / den2;",
                       "dqn_acc[i] += -lb * lprev * lprev / den2;"),
    "lbar_carry_drops_gate": ("lbar[i] = lb * ai * ai / den2 - gb * ai * qni / den2;",
                              "lbar[i] = lb * ai * ai / den2;"),
    "ebar_not_decayed": ("for (int j = 0; j < dv; ++j) ebar[(size_t)i * dv + j] *= ai / den;",
                         "for (int j = 0; j < dv; ++j) ebar[(size_t)i * dv + j] *= ai;"),
    "iso_dk_not_normalised": ("dkk[(size_t)t * dk + i] += lb * 2.0 * kt[i] / ((double)dk * rt);",
                              "dkk[(size_t)t * dk + i] += lb * 2.0 * kt[i] / rt;"),
    "iso_dr_sign": ("drt -= lb * ksq / ((double)dk * rt * rt);", "drt += lb * ksq / ((double)dk * rt * rt);"),
}


def _pins_pass(lib_path):
    for cov in ("diag", "iso"):
        c = rand_case(31, B=2, H=2, T=6, dk=3, dv=2, cov=cov)
        u = upstream(c, cov, 32)
        g = grads(c, u, cov, lib_path=lib_path)
        for name in NAMES:
            if not np.all(np.isfinite(g["d" + name])) or fd_check(c, u, cov, g, name, 33) > 1e-6:
                return False
    return True


def test_bwd_pins_accept_the_oracle():
    assert _pins_pass(None)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bwd_pins_reject_mutant(name, tmp_path):
    src = open(_SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", str(lib),
                    str(mpath)], check=True)
    assert not _pins_pass(str(lib)), f"pins did not catch mutant {name}"
