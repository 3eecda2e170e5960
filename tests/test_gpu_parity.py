"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every input comes from scan_amd.inputs (seeded); the oracle sees the stored
values upcast to fp64.  Every case compares every output element (the
full-size workloads, every sequence, are in test_gpu_coverage.py).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import scan_amd
from scan_amd import inputs as gen
from tests.gpu_util import assert_parity, compare, run_hip, run_oracle, to_dev

pytestmark = pytest.mark.gpu


def _print_case(*args):
    print("CASE", *args, flush=True)


# ------------------------------------------------------------------ small, full compare

@pytest.mark.parametrize("name,over", [
    ("small_diag", {}),
    ("lm_diag", dict(B=1, H=2, T=300)),
    ("long_diag", dict(B=1, H=2, T=1100)),
    ("symbols_diag", dict(B=16, H=4)),
    ("iso", dict(B=1, H=3, T=700)),
])
def test_parity_small(name, over):
    _print_case(name, over)
    inp = gen.make_inputs(name, seed=0, **over)
    w = inp["workload"]
    hip = run_hip(inp, w.cov)
    ref = run_oracle(inp, w.cov)
    errs = compare(hip, ref)
    print(name, errs)
    assert_parity(errs, w.dtype, name)


@pytest.mark.parametrize("cov", ["diag", "iso"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("T", [1, 15, 17, 33, 100])
def test_parity_edges_with_state(cov, dtype, d, T):
    """Ragged lengths, every head dim, both dtypes, non-trivial l0/eta0."""
    _print_case(cov, dtype, d, T)
    base = "small_diag" if cov == "diag" else "iso"
    inp = gen.make_inputs(base, seed=T + d, B=2, H=2, T=T, dk=d, dv=d, dtype=dtype)
    st = gen.make_state(inp["workload"], seed=7)
    hip = run_hip(inp, cov, st["l0"], st["eta0"])
    ref = run_oracle(inp, cov, st["l0"], st["eta0"])
    assert_parity(compare(hip, ref), dtype, f"{cov} {dtype} d={d} T={T}")


@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_empty_sequence_returns_state(cov):
    _print_case("empty", cov)
    inp = gen.make_inputs("small_diag" if cov == "diag" else "iso", seed=1, B=2, H=2, T=0,
                          dk=32, dv=32)
    st = gen.make_state(inp["workload"], seed=3)
    hip = run_hip(inp, cov, st["l0"], st["eta0"])
    assert hip["o"].shape[2] == 0
    assert np.array_equal(hip["lT"], st["l0"].double().numpy())
    assert np.array_equal(hip["etaT"], st["eta0"].double().numpy())


# ------------------------------------------------------------------ full size

def test_parity_symbols_full():
    _print_case("full symbols_diag")
    inp = gen.make_inputs("symbols_diag", seed=0)
    hip = run_hip(inp, "diag")
    ref = run_oracle(inp, "diag")
    errs = compare(hip, ref)
    print("symbols_diag", errs)
    assert_parity(errs, "f32", "symbols_diag")


# ------------------------------------------------------------------ properties

@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_split_handoff_on_device(cov):
    _print_case("handoff", cov)
    name = "lm_diag" if cov == "diag" else "iso"
    inp = gen.make_inputs(name, seed=5, B=2, H=2, T=257)
    dev = {k: to_dev(v) for k, v in inp.items() if isinstance(v, torch.Tensor)}
    o, lT, etaT = scan_amd.fwd(dev["q"], dev["k"], dev["v"], dev["a"], dev["qn"], dev["r"], cov=cov)
    T1 = 100
    tsl = lambda x, a, b: x[:, :, a:b].contiguous()
    qn1 = tsl(dev["qn"], 0, T1) if cov == "iso" else dev["qn"]
    qn2 = tsl(dev["qn"], T1, 257) if cov == "iso" else dev["qn"]
    o1, l1, e1 = scan_amd.fwd(*(tsl(dev[n], 0, T1) for n in ("q", "k", "v", "a")), qn1,
                              tsl(dev["r"], 0, T1), cov=cov)
    o2, l2, e2 = scan_amd.fwd(*(tsl(dev[n], T1, 257) for n in ("q", "k", "v", "a")), qn2,
                              tsl(dev["r"], T1, 257), l1, e1, cov=cov)
    torch.cuda.synchronize()
    tol = 2e-2
    full = o.float()
    cat = torch.cat([o1, o2], dim=2).float()
    assert float((cat - full).abs().max() / full.abs().max()) < tol
    assert float(((l2 - lT).abs() / lT).max()) < 1e-5
    assert float((e2 - etaT).abs().max() / etaT.abs().max()) < tol


@pytest.mark.parametrize("cov", ["diag", "iso"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("T", [2, 4, 5, 31, 32])
def test_parity_short_sequences(cov, dtype, d, T):
    """T <= 32 runs on the short-sequence kernel (state in registers, tokens
    in blocks of four): block boundaries, a ragged last block, cached states."""
    _print_case("short", cov, dtype, d, T)
    base = "small_diag" if cov == "diag" else "iso"
    inp = gen.make_inputs(base, seed=40 + T + d, B=3, H=2, T=T, dk=d, dv=d, dtype=dtype)
    assert scan_amd.fwd_kernel_name(3, 2, T, d, d, cov=cov, dtype=dtype) == "kla_fwd_short_kernel"
    st = gen.make_state(inp["workload"], seed=11)
    hip = run_hip(inp, cov, st["l0"], st["eta0"])
    ref = run_oracle(inp, cov, st["l0"], st["eta0"])
    assert_parity(compare(hip, ref), dtype, f"short {cov} {dtype} d={d} T={T}")


@pytest.mark.parametrize("cov", ["diag", "iso"])
@pytest.mark.parametrize("d", [16, 32])
def test_parity_short_packed_heads(cov, d):
    """Small heads share a workgroup (16 of d 16, 4 of d 32): 35 (b,h) leave
    the last workgroup partly filled, and its spare groups store nothing."""
    _print_case("short packed", cov, d)
    base = "small_diag" if cov == "diag" else "iso"
    inp = gen.make_inputs(base, seed=70 + d, B=5, H=7, T=9, dk=d, dv=d, dtype="bf16")
    assert scan_amd.fwd_kernel_name(5, 7, 9, d, d, cov=cov, dtype="bf16") == "kla_fwd_short_kernel"
    st = gen.make_state(inp["workload"], seed=13)
    hip = run_hip(inp, cov, st["l0"], st["eta0"])
    ref = run_oracle(inp, cov, st["l0"], st["eta0"])
    assert_parity(compare(hip, ref), "bf16", f"short packed {cov} d={d}")


@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_short_path_matches_chunked_kernels(cov, monkeypatch):
    """The short-sequence kernel and the chunked kernels (KLA_FWD_SHORT=0)
    give the same results within the fp32 tolerance."""
    _print_case("short vs chunked", cov)
    base = "small_diag" if cov == "diag" else "iso"
    inp = gen.make_inputs(base, seed=21, B=4, H=3, T=27, dk=64, dv=64, dtype="f32")
    st = gen.make_state(inp["workload"], seed=12)
    a = run_hip(inp, cov, st["l0"], st["eta0"])
    monkeypatch.setenv("KLA_FWD_SHORT", "0")
    assert scan_amd.fwd_kernel_name(4, 3, 27, 64, 64, cov=cov, dtype="f32") != "kla_fwd_short_kernel"
    b = run_hip(inp, cov, st["l0"], st["eta0"])
    for key in ("o", "lT", "etaT"):
        assert float(np.abs(a[key] - b[key]).max() / np.abs(b[key]).max()) < 1e-4, key


@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_steps_match_forward(cov):
    _print_case("steps", cov)
    name = "lm_diag" if cov == "diag" else "iso"
    inp = gen.make_inputs(name, seed=9, B=2, H=3, T=20, dk=64, dv=64, dtype="f32")
    dev = {k: to_dev(v) for k, v in inp.items() if isinstance(v, torch.Tensor)}
    o, lT, etaT = scan_amd.fwd(dev["q"], dev["k"], dev["v"], dev["a"], dev["qn"], dev["r"], cov=cov)
    B, H = 2, 3
    l = torch.ones((B, H, 64) if cov == "diag" else (B, H), device="cuda")
    eta = torch.zeros(B, H, 64, 64, device="cuda")
    for t in range(20):
        sl = lambda x: x[:, :, t].contiguous()
        ot = scan_amd.step(sl(dev["q"]), sl(dev["k"]), sl(dev["v"]), sl(dev["a"]),
                           dev["qn"] if cov == "diag" else sl(dev["qn"]), sl(dev["r"]), l, eta,
                           cov=cov)
        assert float((ot - o[:, :, t]).abs().max() / o[:, :, t].abs().max()) < 1e-4
    assert float(((l - lT).abs() / lT).max()) < 1e-5
    assert float((eta - etaT).abs().max() / etaT.abs().max()) < 1e-4


def test_decode_full_batch():
    """iso decode at B=256, H=32: 128-token prefix via klaFwd, 64 klaStep
    tokens; every (b,h) compared with the oracle continuing from its own
    prefix state."""
    _print_case("decode")
    w = gen.DECODE
    pre = gen.make_inputs(w, seed=1)
    stp = gen.make_inputs(w, seed=2, T=gen.DECODE_STEPS)
    dp = {k: to_dev(v) for k, v in pre.items() if isinstance(v, torch.Tensor)}
    ds = {k: to_dev(v) for k, v in stp.items() if isinstance(v, torch.Tensor)}
    _, l, eta = scan_amd.fwd(dp["q"], dp["k"], dp["v"], dp["a"], dp["qn"], dp["r"], cov="iso")
    outs = []
    for t in range(gen.DECODE_STEPS):
        sl = lambda x: x[:, :, t].contiguous()
        outs.append(scan_amd.step(sl(ds["q"]), sl(ds["k"]), sl(ds["v"]), sl(ds["a"]), sl(ds["qn"]),
                                  sl(ds["r"]), l, eta, cov="iso"))
    torch.cuda.synchronize()
    hip = {"o": torch.stack(outs, dim=2).double().cpu().numpy(),
           "lT": l.double().cpu().numpy(), "etaT": eta.double().cpu().numpy()}
    ref_pre = run_oracle(pre, "iso")
    ref = oracle.fwd(stp["q"], stp["k"], stp["v"], stp["a"], stp["qn"], stp["r"],
                     ref_pre["lT"], ref_pre["etaT"], cov=oracle.ISO)
    errs = compare(hip, ref)
    print("decode", errs)
    assert_parity(errs, w.dtype, "decode")


def test_prefill_full_batch():
    """Serving chunk at B=256, H=32 (the bench's iso_prefill16 launch): a
    128-token prefix via klaFwd, then one 16-token klaFwd from the cached
    states (the short-sequence kernel) into a second state buffer; every
    (b,h) compared with the oracle continuing from the same cached states."""
    _print_case("prefill")
    w = gen.PREFILL
    pre = gen.make_inputs(gen.DECODE, seed=1)
    chk = gen.make_inputs(w, seed=2)
    dp = {k: to_dev(v) for k, v in pre.items() if isinstance(v, torch.Tensor)}
    _, l0, eta0 = scan_amd.fwd(dp["q"], dp["k"], dp["v"], dp["a"], dp["qn"], dp["r"], cov="iso")
    assert scan_amd.fwd_kernel_name(w.B, w.H, w.T, w.dk, w.dv, cov="iso",
                                    dtype=w.dtype) == "kla_fwd_short_kernel"
    hip = run_hip(chk, "iso", l0, eta0)
    ref = run_oracle(chk, "iso", l0.cpu(), eta0.cpu())
    errs = compare(hip, ref)
    print("prefill", errs)
    assert_parity(errs, w.dtype, "prefill")


def test_bitwise_deterministic():
    _print_case("determinism")
    inp = gen.make_inputs("lm_diag", seed=3, B=2, H=4, T=500)
    a = run_hip(inp, "diag")
    for _ in range(5):
        b = run_hip(inp, "diag")
        for k in a:
            assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_adversarial_gates_finite_and_exact(dtype):
    """a -> 0.01, r = 1e-3, |k| up to 5: gate products underflow inside a chunk,
    which forces the sub-chunk split; results stay finite and match the oracle."""
    _print_case("adversarial", dtype)
    inp = gen.make_inputs("small_diag", seed=4, B=1, H=2, T=200, dk=64, dv=64, dtype=dtype)
    g = torch.Generator().manual_seed(11)
    T = 200
    a = torch.full((1, 2, T, 64), 0.01)
    a[:, :, ::7] = 0.9
    inp["a"] = a
    inp["r"] = torch.full((1, 2, T), 1e-3)
    inp["k"] = (5 * (2 * torch.rand(1, 2, T, 64, generator=g) - 1)).to(inp["k"].dtype)
    hip = run_hip(inp, "diag")
    for k in hip:
        assert np.all(np.isfinite(hip[k])), k
    ref = run_oracle(inp, "diag")
    assert_parity(compare(hip, ref), dtype, "adversarial")


@pytest.mark.parametrize("vtiles", ["", "2"])
def test_split_adversarial_gates(monkeypatch, vtiles):
    """Gate products that underflow inside chunks in the middle of a split
    sequence (a -> 0.01 on most tokens, r = 1e-3, |k| up to 5 there): those
    chunks take the exact token-by-token path, the others the factorised
    one, across segment boundaries; on the library's 128-column tiles (the
    chain waves form the gates) and on 64-column tiles."""
    _print_case("split adversarial", vtiles)
    if vtiles:
        monkeypatch.setenv("KLA_FWD_VTILES", vtiles)
    inp = gen.make_inputs("long_diag", seed=31, B=1, H=2, T=4096)
    w = inp["workload"]
    dims = scan_amd.KlaDims(w.B, w.H, w.T, w.dk, w.dv, 1, 0)
    assert scan_amd.klaFwdWorkspaceBytes(dims) > 0
    g = torch.Generator().manual_seed(12)
    lo, hi = 1000, 2600
    a = inp["a"].clone()
    a[:, :, lo:hi] = 0.01
    a[:, :, lo:hi:7] = 0.9
    inp["a"] = a
    r = inp["r"].clone()
    r[:, :, lo:hi] = 1e-3
    inp["r"] = r
    k = inp["k"].float().clone()
    k[:, :, lo:hi] = 5 * (2 * torch.rand(1, 2, hi - lo, w.dk, generator=g) - 1)
    inp["k"] = k.to(inp["k"].dtype)
    hip = run_hip(inp, "diag")
    for x in hip:
        assert np.all(np.isfinite(hip[x])), x
    ref = run_oracle(inp, "diag")
    assert_parity(compare(hip, ref), w.dtype, f"split adversarial {vtiles}")


def test_vtile_split_invariance(monkeypatch):
    """Splitting the value columns over workgroups changes no bit (the
    single-role kernel, which builds both one and two tiles at dk = 128)."""
    _print_case("vtiles")
    inp = gen.make_inputs("lm_diag", seed=6, B=1, H=2, T=150)
    monkeypatch.setenv("KLA_FWD_DIAG_IMPL", "chunk")
    monkeypatch.setenv("KLA_FWD_VTILES", "1")
    a = run_hip(inp, "diag")
    monkeypatch.setenv("KLA_FWD_VTILES", "2")
    b = run_hip(inp, "diag")
    for k in a:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "f32")])
def test_parity_rescale_and_exact_mix(d, dtype):
    """Decay regimes in sequence: strong decay (the deferred state scale is
    folded back every chunk), near-zero gates (exact token-by-token chunks),
    then ordinary decay, with a non-trivial initial state."""
    _print_case("rescale-mix", d, dtype)
    T = 520
    inp = gen.make_inputs("small_diag", seed=12, B=1, H=2, T=T, dk=d, dv=d, dtype=dtype)
    g = torch.Generator().manual_seed(13)
    a = torch.sigmoid(2.0 + torch.randn(1, 2, T, d, generator=g, dtype=torch.float64))
    a[:, :, :200] = 0.35 + 0.1 * torch.rand(1, 2, 200, d, generator=g, dtype=torch.float64)
    a[:, :, 260:330] = 0.01
    inp["a"] = a.float()
    st = gen.make_state(inp["workload"], seed=14)
    hip = run_hip(inp, "diag", st["l0"], st["eta0"])
    for k in hip:
        assert np.all(np.isfinite(hip[k])), k
    ref = run_oracle(inp, "diag", st["l0"], st["eta0"])
    assert_parity(compare(hip, ref), dtype, "rescale-mix")


@pytest.mark.parametrize("name,over,nseg,state,vtiles", [
    ("long_diag", dict(B=1, H=2, T=3000), "3", True, "1"),   # bf16 d128, 128-column tiles, ragged last segment
    ("long_diag", dict(B=1, H=2, T=3000), "3", True, "2"),   # the same with 64-column tiles
    ("small_diag", dict(B=1, H=2, T=700, dk=64, dv=64), "4", True, "1"),  # fp32 d64 (64-column tiles)
    ("long_diag", dict(B=1, H=2, T=4096), "", False, ""),    # split and tiles chosen by the library
    ("long_diag", dict(B=1, H=2, T=4096), "", False, "2"),   # library split, 64-column tiles
])
def test_parity_sequence_split(monkeypatch, name, over, nseg, state, vtiles):
    """Sequence split: segment precision products, carries and the output
    correction reproduce the unsplit recurrence, with and without a state,
    on 128-column tiles (the chain waves form the gates, two gate waves)
    and on 64-column tiles."""
    _print_case("split", name, over, nseg, vtiles)
    if nseg:
        monkeypatch.setenv("KLA_FWD_NSEG", nseg)
    if vtiles:
        monkeypatch.setenv("KLA_FWD_VTILES", vtiles)
    inp = gen.make_inputs(name, seed=21, **over)
    w = inp["workload"]
    dims = scan_amd.KlaDims(w.B, w.H, w.T, w.dk, w.dv, 1 if w.dtype == "bf16" else 0, 0)
    assert scan_amd.klaFwdWorkspaceBytes(dims) > 0
    l0 = eta0 = None
    if state:
        st = gen.make_state(w, seed=22)
        l0, eta0 = st["l0"], st["eta0"]
    hip = run_hip(inp, "diag", l0, eta0)
    ref = run_oracle(inp, "diag", l0, eta0)
    assert_parity(compare(hip, ref), w.dtype, f"split {name} {over}")


def _warm_gap(a, k, r, qn, t0, t1):
    """Relative gap after walking tokens [t0, t1) of one head from the
    precisions 0 and +inf (fp64, on the CPU): the quantity the split's
    precision warm-up tests before it trusts its walk."""
    lo = np.zeros(a.shape[-1])
    hi = None
    for t in range(t0, t1):
        b = k[t] ** 2 / r[t]
        hi = 1.0 / qn + b if hi is None else hi / (a[t] ** 2 + qn * hi) + b
        lo = lo / (a[t] ** 2 + qn * lo) + b
    with np.errstate(invalid="ignore", divide="ignore"):
        return (hi - lo) / lo


@pytest.mark.parametrize("case", ["slow_decay", "zero_noise"])
def test_split_warmup_fallback(monkeypatch, case):
    """Sequence split where the precision warm-up cannot settle one head (a
    near 1 with a tiny process noise, or a = 1 and qn = 0 on some key dims,
    where the precision grows without bound): that head takes the exact
    block-product carry, the other head the warm-up, and both match the
    oracle."""
    _print_case("split warm-up fallback", case)
    monkeypatch.setenv("KLA_FWD_NSEG", "3")
    inp = gen.make_inputs("long_diag", seed=21, B=1, H=2, T=3000)
    a, qn = inp["a"].clone(), inp["qn"].clone()
    if case == "slow_decay":
        a[:, 0] = 0.9999
        qn[0] = 1e-6
    else:
        a[:, 0, :, ::5] = 1.0
        qn[0, ::5] = 0.0
    inp["a"], inp["qn"] = a, qn
    w = inp["workload"]
    # the premise: head 0 has not settled 512 tokens before the first
    # segment start (1024), head 1 has
    k = inp["k"][0].float().double().numpy()
    r = inp["r"][0].double().numpy()
    an, qnn = a[0].double().numpy(), qn.double().numpy()
    gap0 = _warm_gap(an[0], k[0], r[0], qnn[0], 512, 1024)
    gap1 = _warm_gap(an[1], k[1], r[1], qnn[1], 512, 1024)
    assert not np.all(gap0 <= 2.0 ** -20)
    assert np.all(gap1 <= 2.0 ** -22)
    st = gen.make_state(w, seed=22)
    hip = run_hip(inp, "diag", st["l0"], st["eta0"])
    ref = run_oracle(inp, "diag", st["l0"], st["eta0"])
    assert_parity(compare(hip, ref), w.dtype, f"split warm-up fallback {case}")


@pytest.mark.parametrize("cov", ["diag", "iso"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_short_adversarial_gates(cov, dtype):
    """The short-sequence kernel with a -> 0.01 (every 7th token 0.9),
    r = 1e-3 and |k| up to 5, from a cached state: finite and at parity."""
    _print_case("short adversarial", cov, dtype)
    T = 31
    base = "small_diag" if cov == "diag" else "iso"
    inp = gen.make_inputs(base, seed=14, B=2, H=3, T=T, dk=64, dv=64, dtype=dtype)
    assert scan_amd.fwd_kernel_name(2, 3, T, 64, 64, cov=cov, dtype=dtype) == "kla_fwd_short_kernel"
    g = torch.Generator().manual_seed(15)
    a = torch.full(inp["a"].shape, 0.01)
    a[:, :, ::7] = 0.9
    inp["a"] = a
    inp["r"] = torch.full((2, 3, T), 1e-3)
    inp["k"] = (5 * (2 * torch.rand(2, 3, T, 64, generator=g) - 1)).to(inp["k"].dtype)
    st = gen.make_state(inp["workload"], seed=16)
    hip = run_hip(inp, cov, st["l0"], st["eta0"])
    for k in hip:
        assert np.all(np.isfinite(hip[k])), k
    ref = run_oracle(inp, cov, st["l0"], st["eta0"])
    assert_parity(compare(hip, ref), dtype, f"short adversarial {cov}")
