"""GPU parity of klaFwdBlock (the forward with the fused block prologue)
against the fp64 block oracle (oracle/block.py feeding oracle.fwd).

Parity metric and bars as in tests/gpu_util.py (1e-4 fp32, 2e-2 bf16 inputs).
Cases: every built (dtype, d) with convolution widths 1..4, with and without
biases, convolution states and a filter state, sequence lengths that stop
inside the first chunk, at a chunk boundary and past several chunks with a
ragged tail; the chunked-prefill handoff on the device; every sequence of
the LM-layer shape; bitwise determinism.
"""
import numpy as np
import pytest
import torch

import scan_amd
from oracle import block as oblock
from scan_amd import inputs as gen
from tests.gpu_util import assert_parity, compare, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("xq", "xk", "xv", "za", "zqn", "zr", "wq", "wk", "wv", "bq", "bk", "bv", "sq", "sk", "sv")


def _print_case(*args):
    print("case:", *args, flush=True)


def run_hip(b, l0=None, eta0=None):
    args = [to_dev(b[n]) for n in NAMES]
    o, lT, etaT = scan_amd.fwd_block(*args, r_eps=b["r_eps"], l0=to_dev(l0), eta0=to_dev(eta0))
    torch.cuda.synchronize()
    return {"o": o.double().cpu().numpy(), "lT": lT.double().cpu().numpy(),
            "etaT": etaT.double().cpu().numpy()}


def run_ref(b, l0=None, eta0=None):
    return oblock.block_fwd(*(b[n] for n in NAMES), r_eps=b["r_eps"], l0=l0, eta0=eta0)


SHAPES = [("bf16", 128), ("bf16", 64), ("f32", 64)]


@pytest.mark.parametrize("dtype,d", SHAPES)
@pytest.mark.parametrize("width", [1, 2, 3, 4])
@pytest.mark.parametrize("T", [1, 5, 32, 77])
def test_block_matrix(dtype, d, width, T):
    _print_case("block", dtype, d, width, T)
    b = gen.make_block_inputs("small_diag", seed=100 + T + width, B=2, H=3, T=T, dk=d, dv=d,
                              dtype=dtype, width=width, bias=width % 2 == 0, state=width > 1)
    st = gen.make_state(b["workload"], seed=7) if T % 2 else {"l0": None, "eta0": None}
    hip = run_hip(b, st["l0"], st["eta0"])
    ref = run_ref(b, st["l0"], st["eta0"])
    assert_parity(compare(hip, ref), dtype, f"block {dtype} d{d} W{width} T{T}")


@pytest.mark.parametrize("dtype,d", SHAPES)
def test_block_workload_distributions(dtype, d):
    """The LM-layer draws (a from sigmoid(N(2,1)), long sequences of chunks)."""
    _print_case("block workload", dtype, d)
    b = gen.make_block_inputs("block_lm_diag", seed=3, B=2, H=2, T=300, dk=d, dv=d, dtype=dtype,
                              state=True)
    hip = run_hip(b)
    ref = run_ref(b)
    assert_parity(compare(hip, ref), dtype, f"block workload {dtype} d{d}")


@pytest.mark.parametrize("dtype,d", SHAPES)
def test_block_prefill_handoff(dtype, d):
    """Two calls, the second with the first's last W-1 rows as convolution
    states and its lT, etaT as the filter state, match one call (and the
    oracle).  The cut is not a multiple of the chunk."""
    _print_case("block handoff", dtype, d)
    W, T1, T = 4, 45, 110
    b = gen.make_block_inputs("small_diag", seed=11, B=2, H=2, T=T, dk=d, dv=d, dtype=dtype,
                              width=W, state=True)
    full = run_hip(b)
    first, second = dict(b), dict(b)
    for n in ("xq", "xk", "xv", "za", "zr"):
        first[n] = b[n][:, :, :T1].contiguous()
        second[n] = b[n][:, :, T1:].contiguous()
    for x, s in (("xq", "sq"), ("xk", "sk"), ("xv", "sv")):
        second[s] = b[x][:, :, T1 - (W - 1):T1].contiguous()
    h1 = run_hip(first)
    h2 = run_hip(second, torch.tensor(h1["lT"], dtype=torch.float32),
                 torch.tensor(h1["etaT"], dtype=torch.float32))
    joined = {"o": np.concatenate([h1["o"], h2["o"]], axis=2), "lT": h2["lT"], "etaT": h2["etaT"]}
    assert_parity(compare(joined, full), dtype, f"block handoff vs one call {dtype} d{d}")
    assert_parity(compare(joined, run_ref(b)), dtype, f"block handoff vs oracle {dtype} d{d}")


def test_block_full_lm_shape_every_sequence():
    """B8 H16 T2048 d128 bf16, width 4 with biases: every (b,h) against the
    oracle."""
    _print_case("block full lm shape")
    b = gen.make_block_inputs("block_lm_diag", seed=0)
    hip = run_hip(b)
    ref = run_ref(b)
    assert_parity(compare(hip, ref), "bf16", "block full lm shape")


def test_block_empty_sequence_passes_state():
    _print_case("block T=0")
    b = gen.make_block_inputs("small_diag", seed=1, B=2, H=3, T=0, dk=64, dv=64, dtype="bf16")
    st = gen.make_state(b["workload"], seed=2)
    hip = run_hip(b, st["l0"], st["eta0"])
    assert hip["o"].shape == (2, 3, 0, 64)
    np.testing.assert_array_equal(hip["lT"], st["l0"].double().numpy())
    np.testing.assert_array_equal(hip["etaT"], st["eta0"].double().numpy())


def test_block_deterministic():
    _print_case("block determinism")
    b = gen.make_block_inputs("small_diag", seed=5, B=2, H=4, T=200, dk=128, dv=128, dtype="bf16",
                              state=True)
    r1, r2 = run_hip(b), run_hip(b)
    for key in r1:
        np.testing.assert_array_equal(r1[key], r2[key])


@pytest.mark.parametrize("dtype,d,over,nseg,state", [
    ("bf16", 128, dict(B=1, H=2, T=3000), "3", True),     # ragged last segment, states
    ("bf16", 128, dict(B=1, H=2, T=4096), "", False),     # split chosen by the library
    ("f32", 64, dict(B=1, H=2, T=2300), "2", True),
])
def test_block_sequence_split(monkeypatch, dtype, d, over, nseg, state):
    """klaFwdBlock on few, long sequences: the precision warm-up and the
    segment forwards run the prologue too (k and x rows from before a
    segment's start, the convolution state before the sequence's)."""
    _print_case("block split", dtype, d, over, nseg)
    if nseg:
        monkeypatch.setenv("KLA_FWD_NSEG", nseg)
    b = gen.make_block_inputs("long_diag", seed=60, dk=d, dv=d, dtype=dtype, state=state, **over)
    w = b["workload"]
    dims = scan_amd.KlaDims(w.B, w.H, w.T, d, d, 1 if dtype == "bf16" else 0, 0)
    assert scan_amd.klaFwdWorkspaceBytes(dims) > 0
    st = gen.make_state(w, seed=61) if state else {"l0": None, "eta0": None}
    hip = run_hip(b, st["l0"], st["eta0"])
    ref = run_ref(b, st["l0"], st["eta0"])
    assert_parity(compare(hip, ref), dtype, f"block split {dtype} d{d} {over}")


def test_block_split_warmup_fallback(monkeypatch):
    """One head whose precision cannot settle within the warm-up window (a
    near 1, a tiny process noise): it takes the exact block-product carry,
    computed through the prologue as well."""
    _print_case("block split fallback")
    monkeypatch.setenv("KLA_FWD_NSEG", "3")
    b = gen.make_block_inputs("long_diag", seed=62, B=1, H=2, T=3000, state=True)
    za, zqn = b["za"].clone(), b["zqn"].clone()
    za[:, 0] = 10.0            # a = sigmoid(10) ~ 0.99995
    zqn[0] = -14.0             # qn = softplus(-14) ~ 8e-7
    b["za"], b["zqn"] = za, zqn
    st = gen.make_state(b["workload"], seed=63)
    hip = run_hip(b, st["l0"], st["eta0"])
    ref = run_ref(b, st["l0"], st["eta0"])
    assert_parity(compare(hip, ref), "bf16", "block split fallback")


def test_block_full_long_shape_every_sequence():
    """B1 H16 T32768 d128 bf16 (split by the library), every head against the
    oracle."""
    _print_case("block full long shape")
    b = gen.make_block_inputs("block_long_diag", seed=0)
    hip = run_hip(b)
    ref = run_ref(b)
    assert_parity(compare(hip, ref), "bf16", "block full long shape")
