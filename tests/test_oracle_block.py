"""Pins of the fp64 block-prologue oracle (oracle/block.py) against what does
not depend on it:

* the causal convolution against numpy's own ``np.convolve``, channel by
  channel, with the state rows prepended;
* one-hot taps, which turn the convolution into an exact shift;
* the sequence handoff: two calls, the second with the last W-1 rows of the
  first as its convolution state (and the first call's lT, etaT as its
  filter state), equal one call;
* the activations' closed forms and identities (sigmoid(0) = 1/2,
  softplus(0) = ln 2, sigmoid(x) + sigmoid(-x) = 1, softplus(x) -
  softplus(-x) = x, silu(x) = x sigmoid(x), no overflow at |x| = 1000);
* the whole block at W = 1 with unit taps against torch's own SiLU,
  sigmoid and softplus feeding the (separately pinned) forward oracle;
* planted mistakes in the oracle's source, each caught by these pins.
"""
import math
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import block
from scan_amd import inputs as gen

NAMES = ("xq", "xk", "xv", "za", "zqn", "zr", "wq", "wk", "wv", "bq", "bk", "bv", "sq", "sk", "sv")


def _np(x):
    return None if x is None else x.double().numpy()


def check_conv_vs_numpy(mod):
    b = gen.make_block_inputs("small_diag", seed=3, B=2, H=2, T=23, width=4, state=True)
    x, w, bias, st = _np(b["xk"]), _np(b["wk"]), _np(b["bk"]), _np(b["sk"])
    y = mod.causal_conv(b["xk"], b["wk"], b["bk"], b["sk"])
    B, H, T, d = x.shape
    W = w.shape[-1]
    for bb in range(B):
        for h in range(H):
            for c in range(d):
                seq = np.concatenate([st[bb, h, :, c], x[bb, h, :, c]])
                # np.convolve flips its second operand: kernel[j] multiplies lag j
                ref = np.convolve(seq, w[h, c, ::-1])[W - 1:W - 1 + T] + bias[h, c]
                np.testing.assert_allclose(y[bb, h, :, c], ref, rtol=0, atol=1e-12)


def check_one_hot_shift(mod):
    b = gen.make_block_inputs("small_diag", seed=4, B=1, H=2, T=17, width=4, state=True)
    x, st = _np(b["xq"]), _np(b["sq"])
    xe = np.concatenate([st, x], axis=2)
    for lag in range(4):
        w = np.zeros((2, 16, 4))
        w[:, :, 3 - lag] = 1.0
        y = mod.causal_conv(b["xq"], w, None, b["sq"])
        np.testing.assert_array_equal(y, xe[:, :, 3 - lag:3 - lag + 17, :])
    # without a state the rows before token 0 are zero
    w = np.zeros((2, 16, 4))
    w[:, :, 0] = 1.0                                  # lag 3
    y = mod.causal_conv(b["xq"], w)
    np.testing.assert_array_equal(y[:, :, :3], 0.0)
    np.testing.assert_array_equal(y[:, :, 3:], x[:, :, :14])


def check_activations(mod):
    assert mod.sigmoid(0.0) == 0.5
    assert abs(mod.softplus(0.0) - math.log(2.0)) < 1e-15
    assert mod.silu(0.0) == 0.0
    xs = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(mod.sigmoid(xs) + mod.sigmoid(-xs), 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(mod.softplus(xs) - mod.softplus(-xs), xs, rtol=0, atol=1e-13)
    np.testing.assert_allclose(mod.silu(xs), xs / (1.0 + np.exp(-xs)), rtol=1e-14, atol=1e-300)
    assert mod.softplus(1000.0) == 1000.0 and mod.softplus(-1000.0) == 0.0
    assert mod.sigmoid(1000.0) == 1.0 and mod.sigmoid(-1000.0) == 0.0
    t = torch.tensor(xs)
    np.testing.assert_allclose(mod.sigmoid(xs), torch.sigmoid(t).numpy(), rtol=1e-14, atol=1e-300)
    # (torch returns x itself above its threshold, 20 by default)
    np.testing.assert_allclose(mod.softplus(xs), torch.nn.functional.softplus(t, threshold=50).numpy(),
                               rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(mod.silu(xs), torch.nn.functional.silu(t).numpy(),
                               rtol=1e-14, atol=1e-300)


def check_width1_against_torch(mod):
    b = gen.make_block_inputs("small_diag", seed=5, B=2, H=2, T=31, width=1, bias=False)
    one = torch.ones(2, 16, 1)
    got = mod.block_fwd(b["xq"], b["xk"], b["xv"], b["za"], b["zqn"], b["zr"], one, one, one,
                        r_eps=1e-3)
    F = torch.nn.functional
    d = lambda x: x.double()
    ref = oracle.fwd(F.silu(d(b["xq"])), F.silu(d(b["xk"])), F.silu(d(b["xv"])),
                     torch.sigmoid(d(b["za"])), F.softplus(d(b["zqn"])),
                     F.softplus(d(b["zr"])) + 1e-3)
    for key in ("o", "lT", "etaT"):
        np.testing.assert_allclose(got[key], ref[key], rtol=1e-12, atol=1e-12)


def check_handoff(mod):
    W, T1, T = 4, 13, 30
    b = gen.make_block_inputs("small_diag", seed=6, B=1, H=2, T=T, width=W, state=True)
    full = mod.block_fwd(*(b[n] for n in NAMES), r_eps=b["r_eps"])
    first = {n: b[n] for n in NAMES}
    second = {n: b[n] for n in NAMES}
    for n in ("xq", "xk", "xv", "za"):
        first[n], second[n] = b[n][:, :, :T1], b[n][:, :, T1:]
    first["zr"], second["zr"] = b["zr"][:, :, :T1], b["zr"][:, :, T1:]
    for x, s in (("xq", "sq"), ("xk", "sk"), ("xv", "sv")):
        second[s] = b[x][:, :, T1 - (W - 1):T1]
    o1 = mod.block_fwd(*(first[n] for n in NAMES), r_eps=b["r_eps"])
    o2 = mod.block_fwd(*(second[n] for n in NAMES), r_eps=b["r_eps"], l0=o1["lT"], eta0=o1["etaT"])
    np.testing.assert_allclose(np.concatenate([o1["o"], o2["o"]], axis=2), full["o"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o2["lT"], full["lT"], rtol=1e-12)
    np.testing.assert_allclose(o2["etaT"], full["etaT"], rtol=1e-12, atol=1e-12)


def check_prologue_pieces(mod):
    b = gen.make_block_inputs("small_diag", seed=7, B=1, H=2, T=9, width=3, state=True)
    p = mod.prologue(*(b[n] for n in NAMES), r_eps=0.25)
    F = torch.nn.functional
    np.testing.assert_allclose(p["a"], torch.sigmoid(b["za"].double()).numpy(), rtol=1e-14)
    np.testing.assert_allclose(p["qn"], F.softplus(b["zqn"].double()).numpy(), rtol=1e-14)
    np.testing.assert_allclose(p["r"], F.softplus(b["zr"].double()).numpy() + 0.25, rtol=1e-14)
    # v's convolution uses v's own taps, bias and state
    yv = torch.tensor(block.causal_conv(b["xv"], b["wv"], b["bv"], b["sv"]))
    np.testing.assert_allclose(p["v"], F.silu(yv).numpy(), rtol=1e-14, atol=1e-300)


PINS = [check_conv_vs_numpy, check_one_hot_shift, check_activations, check_width1_against_torch,
        check_handoff, check_prologue_pieces]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(block)


def test_rejects_wide_convolution():
    with pytest.raises(ValueError):
        block.causal_conv(np.zeros((1, 1, 4, 2)), np.zeros((1, 2, 5)))


# A planted mistake in each step; every one must break at least one pin.
MUTANTS = {
    "taps reversed": ("w[None, :, None, :, W - 1 - j]", "w[None, :, None, :, j]"),
    "state ignored": ("prev = np.zeros((B, H, W - 1, d)) if state is None else "
                      "_f64(state).reshape(B, H, W - 1, d)", "prev = np.zeros((B, H, W - 1, d))"),
    "bias subtracted": ("y += _f64(bias)[None, :, None, :]", "y -= _f64(bias)[None, :, None, :]"),
    "silu is sigmoid": ("return x * sigmoid(x)", "return sigmoid(x)"),
    "softplus drops log1p": ("np.log1p(np.exp(-np.abs(x)))", "np.exp(-np.abs(x))"),
    "r_eps dropped": ('"r": softplus(_f64(zr)) + float(r_eps)', '"r": softplus(_f64(zr))'),
    "qn through sigmoid": ('"qn": softplus(_f64(zqn))', '"qn": sigmoid(_f64(zqn))'),
    "a through softplus": ('"a": sigmoid(_f64(za))', '"a": softplus(_f64(za))'),
    "v with q's taps": ("silu(causal_conv(xv, wv, bv, sv))", "silu(causal_conv(xv, wq, bv, sv))"),
    "one token late": ("xe[:, :, W - 1 - j:W - 1 - j + T, :]", "xe[:, :, W - 2 - j:W - 2 - j + T, :]"),
}


def _mutant(src, old, new):
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle.block_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "block_mutant.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name):
    src = open(block.__file__).read()
    mod = _mutant(src, *MUTANTS[name])
    caught = False
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError):
            caught = True
            break
    assert caught, f"mutant '{name}' passes every pin"
