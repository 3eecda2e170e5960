"""GPU parity, second matrix: every exported klaStep shape against the oracle,
every (b,h) sequence of the full-size workloads, the isotropic/diagonal
equivalence on the device, adversarial gates on the isotropic pipelined
kernel, and bitwise determinism of every forward kernel family.

All inputs come from scan_amd.inputs (seeded).  The oracle sees the stored
values upcast to fp64; for the decode steps it continues from the very state
the HIP prefix forward produced, so each step is checked on its own.
"""
import numpy as np
import pytest
import torch

import oracle
import scan_amd
from scan_amd import inputs as gen
from tests.gpu_util import TOL, assert_parity, compare, run_hip, run_oracle, slab_err, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "a", "qn", "r")


def _print_case(*args):
    print("CASE", *args, flush=True)


def _dev(inp):
    return {k: to_dev(v) for k, v in inp.items() if isinstance(v, torch.Tensor)}


# ------------------------------------------------------------------ klaStep, every shape

@pytest.mark.parametrize("cov", ["diag", "iso"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_step_every_shape_against_oracle(cov, dtype, d):
    """A 40-token klaFwd prefix from a non-trivial state builds the cached
    (l, eta); then 6 klaStep tokens.  The oracle continues from the same
    cached state: every step's output and the final (l, eta) are compared."""
    _print_case("step", cov, dtype, d)
    B, H, TP, NS = 3, 2, 40, 6
    base = "small_diag" if cov == "diag" else "iso"
    pre = gen.make_inputs(base, seed=100 + d, B=B, H=H, T=TP, dk=d, dv=d, dtype=dtype)
    stp = gen.make_inputs(base, seed=200 + d, B=B, H=H, T=NS, dk=d, dv=d, dtype=dtype)
    if cov == "diag":
        stp["qn"] = pre["qn"]               # qn is per (head, key dim) and time-invariant
    st = gen.make_state(pre["workload"], seed=300 + d)
    dp, ds = _dev(pre), _dev(stp)
    _, l, eta = scan_amd.fwd(*(dp[n] for n in NAMES), to_dev(st["l0"]), to_dev(st["eta0"]), cov=cov)
    torch.cuda.synchronize()
    l_start = l.double().cpu().numpy()
    eta_start = eta.double().cpu().numpy()
    outs = []
    for t in range(NS):
        sl = lambda x: x[:, :, t].contiguous()
        qn_t = ds["qn"] if cov == "diag" else sl(ds["qn"])
        outs.append(scan_amd.step(sl(ds["q"]), sl(ds["k"]), sl(ds["v"]), sl(ds["a"]), qn_t,
                                  sl(ds["r"]), l, eta, cov=cov))
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=2).double().cpu().numpy()
    ref = oracle.fwd(*(stp[n] for n in NAMES), l_start, eta_start,
                     cov=oracle.DIAG if cov == "diag" else oracle.ISO)
    hip = {"o": o, "lT": l.double().cpu().numpy(), "etaT": eta.double().cpu().numpy()}
    errs = compare(hip, ref)
    print(cov, dtype, d, errs)
    assert_parity(errs, dtype, f"klaStep {cov} {dtype} d={d}")
    # each step on its own, too (the first step reads the prefix state only)
    for t in range(NS):
        e = slab_err(o[:, :, t], ref["o"][:, :, t], 2)
        assert e <= TOL[dtype], (t, e)


# ------------------------------------------------------------------ full size, every sequence

@pytest.mark.parametrize("name", ["lm_diag", "long_diag", "iso"])
def test_parity_full_size_every_sequence(name):
    """The full workload in the benchmark's launch configuration, every (b,h)
    sequence compared with the oracle (a mis-indexed workgroup slot, value
    tile or segment anywhere in the grid would fail)."""
    _print_case("full every", name)
    inp = gen.make_inputs(name, seed=0)
    w = inp["workload"]
    hip = run_hip(inp, w.cov)
    for k in hip:
        assert np.all(np.isfinite(hip[k])), k
    ref = run_oracle(inp, w.cov)
    errs = compare(hip, ref)
    print(name, errs, flush=True)
    assert_parity(errs, w.dtype, name)


# ------------------------------------------------------------------ iso == diag on the device

@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "bf16"), (64, "f32")])
def test_iso_equals_diag_on_device(d, dtype):
    """With |k_t[i]| the same for every key dim, a_t and qn shared by every
    key dim, and l0 shared too, the isotropic precision increment equals every
    diagonal one, so the two variants compute the same filter.  Both HIP
    forwards are compared with the oracle and with each other."""
    _print_case("iso==diag", d, dtype)
    B, H, T = 2, 3, 300
    base = gen.make_inputs("iso", seed=31, B=B, H=H, T=T, dk=d, dv=d, dtype=dtype)
    g = torch.Generator().manual_seed(32)
    mag = (0.5 + torch.rand(B, H, T, 1, generator=g, dtype=torch.float64)) / d ** 0.5
    sign = torch.where(torch.rand(B, H, T, d, generator=g) < 0.5, -1.0, 1.0).double()
    k = (mag * sign).to(gen.torch_dtype(dtype))
    assert torch.all(k.abs() == k.abs()[..., :1])          # |k| constant over key dims
    qn_h = torch.nn.functional.softplus(-2.0 + 0.7 * torch.randn(H, generator=g, dtype=torch.float64))
    l0_iso = (torch.nn.functional.softplus(torch.randn(B, H, generator=g, dtype=torch.float64)) + 0.2)
    eta0 = torch.randn(B, H, d, d, generator=g, dtype=torch.float64).float()
    iso = dict(base, k=k, qn=qn_h[None, :, None].expand(B, H, T).float().contiguous())
    diag = dict(base, k=k,
                a=base["a"][..., None].expand(B, H, T, d).contiguous(),
                qn=qn_h[:, None].expand(H, d).float().contiguous())
    l0_diag = l0_iso[..., None].expand(B, H, d).float().contiguous()
    hi = run_hip(iso, "iso", l0_iso.float(), eta0)
    hd = run_hip(diag, "diag", l0_diag, eta0)
    ri = run_oracle(iso, "iso", l0_iso.float(), eta0)
    rd = run_oracle(diag, "diag", l0_diag, eta0)
    # the two oracles agree to fp64 rounding (the reduction the pins fix)
    assert slab_err(ri["o"], rd["o"], 2) < 1e-12
    assert_parity(compare(hi, ri), dtype, "iso")
    assert_parity(compare(hd, rd), dtype, "diag")
    hd_iso = dict(hd, lT=hd["lT"][..., 0])
    assert np.allclose(hd["lT"], hd["lT"][..., :1], rtol=1e-6)
    errs = compare(hi, hd_iso)
    print("iso vs diag (HIP)", errs)
    assert_parity(errs, dtype, "iso vs diag")


# ------------------------------------------------------------------ adversarial gates, iso pipe

@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_iso_pipe_adversarial_gates(dtype, d):
    """a -> 0.01 (every 7th token 0.9), r = 1e-3 and |k| up to 5 on the
    isotropic pipelined kernel: chunk gate products far below any fixed
    floor; finite and at parity with the oracle."""
    _print_case("iso adversarial", dtype, d)
    B, H, T = 1, 4, 300
    inp = gen.make_inputs("iso", seed=41, B=B, H=H, T=T, dk=d, dv=d, dtype=dtype)
    assert scan_amd.fwd_kernel_name(B, H, T, d, d, cov="iso", dtype=dtype).startswith(
        "kla_fwd_iso_pipe_kernel")
    g = torch.Generator().manual_seed(42)
    a = torch.full((B, H, T), 0.01)
    a[:, :, ::7] = 0.9
    inp["a"] = a
    inp["r"] = torch.full((B, H, T), 1e-3)
    inp["k"] = (5 * (2 * torch.rand(B, H, T, d, generator=g) - 1)).to(inp["k"].dtype)
    st = gen.make_state(inp["workload"], seed=43)
    hip = run_hip(inp, "iso", st["l0"], st["eta0"])
    for k in hip:
        assert np.all(np.isfinite(hip[k])), k
    ref = run_oracle(inp, "iso", st["l0"], st["eta0"])
    assert_parity(compare(hip, ref), dtype, f"iso adversarial {dtype} d={d}")


# ------------------------------------------------------------------ determinism, every family

@pytest.mark.parametrize("case", [
    ("iso", dict(B=1, H=4, T=700), "kla_fwd_iso_pipe_kernel"),
    ("iso", dict(B=1, H=4, T=700, dk=32, dv=32), "kla_fwd_iso_kernel"),
    ("long_diag", dict(B=1, H=2, T=4096), "kla_fwd_diag_pipe_kernel"),   # sequence split
    ("symbols_diag", dict(B=8, H=4), "kla_fwd_diag_kernel"),
    ("iso", dict(B=16, H=8, T=16), "kla_fwd_short_kernel"),
    ("lm_diag", dict(B=8, H=4, T=9), "kla_fwd_short_kernel"),
])
def test_bitwise_deterministic_every_family(case):
    """Repeated calls on the same inputs give the same bits, for every kernel
    family (no atomics or order-dependent reductions anywhere)."""
    name, over, kname = case
    _print_case("determinism", name, over)
    inp = gen.make_inputs(name, seed=51, **over)
    w = inp["workload"]
    assert scan_amd.fwd_kernel_name(w.B, w.H, w.T, w.dk, w.dv, cov=w.cov,
                                    dtype=w.dtype).startswith(kname)
    if name == "long_diag":
        dims = scan_amd.KlaDims(w.B, w.H, w.T, w.dk, w.dv, 1, 0)
        assert scan_amd.klaFwdWorkspaceBytes(dims) > 0      # the split path
    st = gen.make_state(w, seed=52)
    a = run_hip(inp, w.cov, st["l0"], st["eta0"])
    for _ in range(3):
        b = run_hip(inp, w.cov, st["l0"], st["eta0"])
        for k in a:
            assert np.array_equal(a[k], b[k]), (k, name, over)


# ------------------------------------------------------------------ wavefront-level scan chain

@pytest.mark.parametrize("name,over,nseg,state", [
    ("lm_diag", dict(B=2, H=2, T=333), "", True),             # bf16 d128, ragged last chunk
    ("lm_diag", dict(B=1, H=3, T=150, dk=64, dv=64), "", True),  # bf16 d64 (one chain wave)
    ("long_diag", dict(B=1, H=2, T=3000), "3", True),         # sequence split
    ("lm_diag", dict(B=8, H=16, T=2048), "", False),          # the LM-layer launch
])
def test_scan_chain_parity(monkeypatch, name, over, nseg, state):
    """KLA_DIAG_CHAIN=scan: the diagonal precision of the wave-specialised
    kernel as a wavefront-level Mobius scan (lanes own 4 key dims x 8 tokens,
    group maps composed and scanned across lanes), at parity with the
    oracle."""
    _print_case("scan chain", name, over, nseg)
    monkeypatch.setenv("KLA_DIAG_CHAIN", "scan")
    if nseg:
        monkeypatch.setenv("KLA_FWD_NSEG", nseg)
    inp = gen.make_inputs(name, seed=71, **over)
    w = inp["workload"]
    assert scan_amd.fwd_kernel_name(w.B, w.H, w.T, w.dk, w.dv, cov="diag",
                                    dtype=w.dtype).startswith("kla_fwd_diag_pipe_kernel")
    l0 = eta0 = None
    if state:
        st = gen.make_state(w, seed=72)
        l0, eta0 = st["l0"], st["eta0"]
    hip = run_hip(inp, "diag", l0, eta0)
    ref = run_oracle(inp, "diag", l0, eta0)
    assert_parity(compare(hip, ref), w.dtype, f"scan chain {name} {over}")


def test_scan_chain_adversarial(monkeypatch):
    """The scan chain with a -> 0.01 (every 7th token 0.9), r = 1e-3, |k| up
    to 5: group maps spanning many orders of magnitude (renormalised), gate
    products below the floor (exact chunks)."""
    _print_case("scan chain adversarial")
    monkeypatch.setenv("KLA_DIAG_CHAIN", "scan")
    inp = gen.make_inputs("small_diag", seed=73, B=1, H=2, T=200, dk=128, dv=128, dtype="bf16")
    g = torch.Generator().manual_seed(74)
    a = torch.full((1, 2, 200, 128), 0.01)
    a[:, :, ::7] = 0.9
    inp["a"] = a
    inp["r"] = torch.full((1, 2, 200), 1e-3)
    inp["k"] = (5 * (2 * torch.rand(1, 2, 200, 128, generator=g) - 1)).to(torch.bfloat16)
    hip = run_hip(inp, "diag")
    for k in hip:
        assert np.all(np.isfinite(hip[k])), k
    ref = run_oracle(inp, "diag")
    assert_parity(compare(hip, ref), "bf16", "scan chain adversarial")
