"""Pins for the fp64 oracle: it is checked against things other than itself.

Each pin below comes from the mathematics of the method as the pages state it
("Kalman Linear Attention: Parallel Bayesian Filtering For Efficient Language
Modelling and State Tracking", gist.science explainer, method §1-§3 and main
contributions; "Kalman Delta Networks: Uncertainty-aware Associative Memory",
abstract):

* exact Bayesian filtering  -> brute-force joint-Gaussian posteriors (numpy)
  and an exact-rational worked example (tests/golden);
* Mobius precision map whose maps compose associatively -> 2x2 matrix
  products under arbitrary bracketing;
* a = 1, qn = 0 -> precision and information are plain cumulative sums
  (normalised linear attention);
* k = 0 -> pure prediction: variance recursion and decaying mean;
* OU prior keeps the precision bounded -> fixed point and bounds;
* diagonal vs isotropic variants -> equal where the projections coincide.

A mutation test at the end plants plausible mistakes in a copy of the oracle
source and checks that the pins catch every one of them.
"""
import os
import shutil
import subprocess
import json
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import bruteforce
from scan_amd import inputs as gen

DIAG, ISO = oracle.DIAG, oracle.ISO


def rand_case(seed, B=1, H=2, T=6, dk=3, dv=2, cov="diag", state=True):
    rng = np.random.default_rng(seed)
    sig = lambda x: 1 / (1 + np.exp(-x))
    sp = lambda x: np.log1p(np.exp(x))
    q = rng.normal(size=(B, H, T, dk))
    k = rng.normal(size=(B, H, T, dk))
    v = rng.normal(size=(B, H, T, dv))
    if cov == "diag":
        a = sig(1 + rng.normal(size=(B, H, T, dk)))
        qn = sp(-1 + rng.normal(size=(H, dk)))
        l0 = sp(rng.normal(size=(B, H, dk))) + 0.3
    else:
        a = sig(1 + rng.normal(size=(B, H, T)))
        qn = sp(-1 + rng.normal(size=(B, H, T)))
        l0 = sp(rng.normal(size=(B, H))) + 0.3
    r = sp(rng.normal(size=(B, H, T))) + 0.05
    eta0 = rng.normal(size=(B, H, dk, dv))
    if not state:
        l0 = eta0 = None
    return dict(q=q, k=k, v=v, a=a, qn=qn, r=r, l0=l0, eta0=eta0)


def run(c, cov="diag", **kw):
    return oracle.fwd(c["q"], c["k"], c["v"], c["a"], c["qn"], c["r"], c["l0"], c["eta0"],
                      cov=DIAG if cov == "diag" else ISO, want_l_all=True, **kw)


def relerr(x, ref):
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("cov", ["diag", "iso"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bruteforce_gaussian(cov, seed):
    c = rand_case(seed, cov=cov)
    out = run(c, cov)
    bf = bruteforce.forward(c["q"], c["k"], c["v"], c["a"], c["qn"], c["r"], c["l0"], c["eta0"],
                            cov=cov)
    assert relerr(out["l_all"], bf["l_all"]) < 1e-11
    assert relerr(out["etaT"], bf["etaT"]) < 1e-11
    assert relerr(out["o"], bf["o"]) < 1e-11


def test_bruteforce_default_state():
    c = rand_case(5, state=False)
    out = run(c)
    bf = bruteforce.forward(c["q"], c["k"], c["v"], c["a"], c["qn"], c["r"], cov="diag")
    assert relerr(out["o"], bf["o"]) < 1e-11
    assert relerr(out["lT"], bf["l_all"][:, :, -1]) < 1e-11


def test_golden_worked_example():
    path = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")
    doc = json.load(open(path))
    f = lambda x: np.array(x, dtype=object)
    val = lambda x: np.vectorize(lambda s: float(Fraction(s)))(f(x)).astype(np.float64)
    I = doc["inputs"]
    q, k, v, a = (val(I[n])[None, None] for n in ("q", "k", "v", "a"))
    qn = val(I["qn"])[None]
    r = val(I["r"])[None, None]
    l0 = val(I["l0"])[None, None]
    eta0 = val(I["eta0"])[None, None]
    out = oracle.fwd(q, k, v, a, qn, r, l0, eta0, want_l_all=True)
    O = doc["outputs"]
    assert relerr(out["o"][0, 0], val(O["o"])) < 1e-14
    assert relerr(out["l_all"][0, 0], val(O["l_all"])) < 1e-14
    assert relerr(out["etaT"][0, 0], val(O["etaT"])) < 1e-14


# ---------------------------------------------------------------- Mobius

def _mobius_mats(a, qn, b):
    """Per-step 2x2 maps l -> ((1+b qn) l + b a^2) / (qn l + a^2)."""
    M = np.empty(a.shape + (2, 2))
    M[..., 0, 0] = 1 + b * qn
    M[..., 0, 1] = b * a * a
    M[..., 1, 0] = qn
    M[..., 1, 1] = a * a
    return M


def _tree_product(Ms):
    """Product M_{n-1} ... M_0 with a balanced (non-sequential) bracketing."""
    if len(Ms) == 1:
        return Ms[0]
    mid = len(Ms) // 2
    P = _tree_product(Ms[mid:]) @ _tree_product(Ms[:mid])
    return P / np.abs(P).max(axis=(-2, -1), keepdims=True)  # projective rescale


@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_mobius_associativity(cov):
    c = rand_case(11, T=13, dk=4, cov=cov)
    out = run(c, cov)
    T = c["q"].shape[2]
    if cov == "diag":
        b = c["k"] ** 2 / c["r"][..., None]
        qn = np.broadcast_to(c["qn"][None, :, None, :], b.shape)
        M = _mobius_mats(c["a"], qn, b)                     # [B,H,T,dk,2,2]
        l0 = c["l0"]
    else:
        b = (c["k"] ** 2).sum(-1) / (c["k"].shape[-1] * c["r"])
        M = _mobius_mats(c["a"], c["qn"], b)                 # [B,H,T,2,2]
        l0 = c["l0"]
    for t in range(T):
        P = _tree_product([M[:, :, s] for s in range(t + 1)])
        lt = (P[..., 0, 0] * l0 + P[..., 0, 1]) / (P[..., 1, 0] * l0 + P[..., 1, 1])
        assert relerr(lt, out["l_all"][:, :, t]) < 1e-13


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_closed_form_a1_qn0(cov):
    """a = 1, qn = 0: l_t = l0 + sum b_s, eta_t = eta0 + sum k v^T / r."""
    c = rand_case(3, T=9, dk=4, dv=3, cov=cov)
    c["a"] = np.ones_like(c["a"])
    c["qn"] = np.zeros_like(c["qn"])
    out = run(c, cov)
    k, v, r, q = c["k"], c["v"], c["r"], c["q"]
    dk = k.shape[-1]
    if cov == "diag":
        l = c["l0"][:, :, None, :] + np.cumsum(k ** 2 / r[..., None], axis=2)
    else:
        l = c["l0"][:, :, None] + np.cumsum((k ** 2).sum(-1) / (dk * r), axis=2)
    eta = c["eta0"][:, :, None] + np.cumsum(np.einsum("bhti,bhtj->bhtij", k, v)
                                            / r[..., None, None], axis=2)
    lb = l[..., None] if cov == "diag" else l[..., None, None]
    o = np.einsum("bhti,bhtij->bhtj", q, eta / lb)
    assert relerr(out["l_all"], l) < 1e-14
    assert relerr(out["etaT"], eta[:, :, -1]) < 1e-14
    assert relerr(out["o"], o) < 1e-13


def test_prediction_only_k0():
    """k = 0: variance follows 1/l_t = a^2/l_{t-1} + qn, mean decays by a."""
    c = rand_case(4, T=10, dk=3, dv=2)
    c["k"] = np.zeros_like(c["k"])
    out = run(c)
    var = 1.0 / c["l0"]
    for t in range(10):
        var = c["a"][:, :, t] ** 2 * var + c["qn"][None]
        assert relerr(out["l_all"][:, :, t], 1.0 / var) < 1e-14
    m0 = c["eta0"] / c["l0"][..., None]
    decay = np.cumprod(c["a"], axis=2)                               # [B,H,T,dk]
    o = np.einsum("bhti,bhti,bhij->bhtj", c["q"], decay, m0)
    assert relerr(out["o"], o) < 1e-13


def test_fixed_point_constant_parameters():
    """Constant a, qn, b: l converges to the positive root of
    qn l^2 + (a^2 - 1 - b qn) l - b a^2 = 0 (the Mobius map's fixed point)."""
    B, H, T, dk, dv = 1, 1, 3000, 3, 1
    a_val = np.array([0.9, 0.5, 0.99])
    qn_val = np.array([0.1, 0.3, 0.001])
    k_val = np.array([0.3, 1.0, 0.05])
    r_val = 0.7
    q = np.zeros((B, H, T, dk))
    k = np.broadcast_to(k_val, (B, H, T, dk)).copy()
    v = np.zeros((B, H, T, dv))
    a = np.broadcast_to(a_val, (B, H, T, dk)).copy()
    r = np.full((B, H, T), r_val)
    out = oracle.fwd(q, k, v, a, qn_val[None], r)
    b = k_val ** 2 / r_val
    A, Bq, C = qn_val, a_val ** 2 - 1 - b * qn_val, -b * a_val ** 2
    root = (-Bq + np.sqrt(Bq ** 2 - 4 * A * C)) / (2 * A)
    assert relerr(out["lT"][0, 0], root) < 1e-12


# ---------------------------------------------------------------- variants

def test_iso_equals_diag_when_abs_k_constant():
    c = rand_case(6, T=8, dk=5, dv=3, cov="iso")
    rng = np.random.default_rng(60)
    mag = np.abs(rng.normal(size=c["k"].shape[:3]))[..., None]
    c["k"] = mag * rng.choice([-1.0, 1.0], size=c["k"].shape)
    c["qn"] = np.broadcast_to(c["qn"][:, :, :1], c["qn"].shape).copy()  # time-constant
    iso = run(c, "iso")
    d = dict(c)
    dk = c["k"].shape[-1]
    d["a"] = np.broadcast_to(c["a"][..., None], c["k"].shape).copy()
    d["qn"] = np.broadcast_to(c["qn"][0, :, :1], (c["qn"].shape[1], dk)).copy()
    d["l0"] = np.broadcast_to(c["l0"][..., None], c["k"].shape[:2] + (dk,)).copy()
    # diag qn is per head; use B=1 so the per-(b,h) iso noise maps onto it
    diag = run(d, "diag")
    assert relerr(diag["o"], iso["o"]) < 1e-13
    assert relerr(diag["l_all"][..., 0], iso["l_all"]) < 1e-13
    assert relerr(diag["etaT"], iso["etaT"]) < 1e-13


def test_iso_equals_diag_at_dk1():
    c = rand_case(7, T=8, dk=1, dv=3, cov="iso")
    c["qn"] = np.broadcast_to(c["qn"][:, :, :1], c["qn"].shape).copy()
    iso = run(c, "iso")
    d = dict(c, a=c["a"][..., None], qn=c["qn"][0, :, :1].copy(), l0=c["l0"][..., None])
    diag = run(d, "diag")
    assert relerr(diag["o"], iso["o"]) < 1e-14
    assert relerr(diag["lT"][..., 0], iso["lT"]) < 1e-14


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_linearity(cov):
    c1 = rand_case(8, T=12, cov=cov)
    c2 = rand_case(9, T=12, cov=cov)
    c2.update({n: c1[n] for n in ("q", "k", "a", "qn", "r", "l0")})
    s = dict(c1, v=c1["v"] + 2 * c2["v"], eta0=c1["eta0"] + 2 * c2["eta0"])
    o1, o2, os_ = run(c1, cov)["o"], run(c2, cov)["o"], run(s, cov)["o"]
    assert relerr(os_, o1 + 2 * o2) < 1e-12
    sq = dict(c1, q=3 * c1["q"] - c2["q"])
    c1q = dict(c1, q=c2["q"])
    assert relerr(run(sq, cov)["o"], 3 * o1 - run(c1q, cov)["o"]) < 1e-12


@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_split_handoff(cov):
    c = rand_case(10, T=20, cov=cov)
    full = run(c, cov)
    T1 = 7
    first = {n: (x[:, :, :T1] if n in ("q", "k", "v", "r") or (n == "a") or (cov == "iso" and n == "qn")
                 else x) for n, x in c.items()}
    second = {n: (x[:, :, T1:] if n in ("q", "k", "v", "r") or (n == "a") or (cov == "iso" and n == "qn")
                  else x) for n, x in c.items()}
    o1 = run(first, cov)
    second["l0"], second["eta0"] = o1["lT"], o1["etaT"]
    o2 = run(second, cov)
    assert relerr(np.concatenate([o1["o"], o2["o"]], axis=2), full["o"]) < 1e-13
    assert relerr(o2["lT"], full["lT"]) < 1e-14
    assert relerr(o2["etaT"], full["etaT"]) < 1e-13


@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_steps_equal_forward(cov):
    c = rand_case(12, T=9, cov=cov)
    full = run(c, cov)
    l, eta = c["l0"], c["eta0"]
    for t in range(9):
        sl = lambda x: x[:, :, t]
        s = oracle.step(sl(c["q"]), sl(c["k"]), sl(c["v"]), sl(c["a"]),
                        c["qn"] if cov == "diag" else sl(c["qn"]), sl(c["r"]), l, eta,
                        cov=DIAG if cov == "diag" else ISO)
        assert relerr(s["o"], full["o"][:, :, t]) < 1e-14
        l, eta = s["l"], s["eta"]
    assert relerr(l, full["lT"]) < 1e-15
    assert relerr(eta, full["etaT"]) < 1e-15


def test_batch_permutation():
    c = rand_case(13, B=4, H=2, T=7)
    out = run(c)
    perm = np.array([2, 0, 3, 1])
    p = {n: (x[perm] if (x is not None and n != "qn") else x) for n, x in c.items()}
    outp = run(p)
    for n in ("o", "lT", "etaT"):
        assert np.array_equal(outp[n], out[n][perm])


def test_precision_bounds_on_workload_inputs():
    """OU prior keeps precision bounded: b_t <= l_t < 1/qn + b_t."""
    x = gen.make_inputs("small_diag", seed=0)
    out = oracle.fwd(x["q"], x["k"], x["v"], x["a"], x["qn"], x["r"], want_l_all=True)
    k = x["k"].double().numpy()
    b = k ** 2 / x["r"].double().numpy()[..., None]
    l = out["l_all"]
    qn = x["qn"].double().numpy()[None, :, None, :]
    assert np.all(l >= b) and np.all(l > 0)
    assert np.all(l < 1.0 / qn + b)


def test_empty_sequence_returns_state():
    c = rand_case(14, T=6)
    e = {n: (x[:, :, :0] if n in ("q", "k", "v", "a", "r") else x) for n, x in c.items()}
    out = run(e)
    assert out["o"].shape[2] == 0
    assert np.array_equal(out["lT"], c["l0"]) and np.array_equal(out["etaT"], c["eta0"])


# ---------------------------------------------------------------- mutation test

_SRC = os.path.join(os.path.dirname(oracle.__file__), "kla_oracle.c")

MUTANTS = {
    "a_not_squared": ("at[i] * at[i] + qn[i] * lprev", "at[i] + qn[i] * lprev"),
    "gate_drops_a": ("const double g = lp * at[i] / lprev;", "const double g = lp / lprev;"),
    "precision_drops_r": ("lnew[i] = lp + kt[i] * kt[i] / rt;", "lnew[i] = lp + kt[i] * kt[i];"),
    "write_drops_r": ("row[j] = g * row[j] + kt[i] * vt[j] / rt;\n            }\n            for (int i = 0; i < dk; ++i) l[i] = lnew[i];",
                      "row[j] = g * row[j] + kt[i] * vt[j];\n            }\n            for (int i = 0; i < dk; ++i) l[i] = lnew[i];"),
    "readout_of_eta": ("ot[j] += qt[i] * row[j] / li;", "ot[j] += qt[i] * row[j];"),
    "noise_sign": ("lprev / (at[i] * at[i] + qn[i] * lprev)", "lprev / (at[i] * at[i] - qn[i] * lprev)"),
    "iso_b_not_normalised": ("l[0] = lp + ksq / ((double)dk * rt);", "l[0] = lp + ksq / rt;"),
    "iso_gate_transposed": ("const double g = lp * at / lprev;", "const double g = lprev * at / lp;"),
    "readout_uses_prior": ("for (int i = 0; i < dk; ++i) l[i] = lnew[i];\n            if (l_all)",
                           "if (l_all)"),
    "query_index": ("ot[j] += qt[i] * row[j] / li;", "ot[j] += qt[dk - 1 - i] * row[j] / li;"),
}


def _pins_pass(lib_path):
    ok = True
    for cov in ("diag", "iso"):
        c = rand_case(21, T=5, dk=3, dv=2, cov=cov)
        out = oracle.fwd(c["q"], c["k"], c["v"], c["a"], c["qn"], c["r"], c["l0"], c["eta0"],
                         cov=DIAG if cov == "diag" else ISO, want_l_all=True, lib_path=lib_path)
        bf = bruteforce.forward(c["q"], c["k"], c["v"], c["a"], c["qn"], c["r"], c["l0"],
                                c["eta0"], cov=cov)
        for n in ("o", "l_all", "etaT"):
            if not np.all(np.isfinite(out[n])) or relerr(out[n], bf[n]) > 1e-9:
                ok = False
    return ok


def test_pins_accept_the_oracle():
    assert _pins_pass(None)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    src = open(_SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", str(lib),
                    str(mpath)], check=True)
    assert not _pins_pass(str(lib)), f"pins did not catch mutant {name}"
