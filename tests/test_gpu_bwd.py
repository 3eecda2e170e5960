"""GPU parity of the backward pass (klaBwd through the C ABI) against the fp64
backward oracle (oracle.bwd), on seeded inputs from scan_amd.inputs.

Every gradient is compared element by element with the forward's parity
metric: max |x - ref| / max |ref| per (b,h) slab (per head for the diagonal
qn gradient, which sums over the batch); bars 1e-4 for fp32 inputs, 2e-2 for
bf16 inputs (where dq, dk, dv are rounded to bf16).
"""
import numpy as np
import pytest
import torch

import oracle
import scan_amd
from scan_amd import inputs as gen
from tests.gpu_util import TOL, slab_err, to_dev

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "da", "dqn", "dr", "dl0", "deta0")


def _print_case(*args):
    print("CASE", *args, flush=True)


def run_bwd(inp, up, cov, st=None):
    l0 = eta0 = None
    if st is not None:
        l0, eta0 = st["l0"], st["eta0"]
    g = scan_amd.bwd(*(to_dev(inp[n]) for n in ("q", "k", "v", "a", "qn", "r")), to_dev(l0),
                     to_dev(eta0), to_dev(up["do"]), to_dev(up["dlT"]), to_dev(up["detaT"]), cov=cov)
    torch.cuda.synchronize()
    return {n: x.double().cpu().numpy() for n, x in g.items()}


def run_ref(inp, up, cov, st=None):
    l0 = eta0 = None
    if st is not None:
        l0, eta0 = st["l0"], st["eta0"]
    return oracle.bwd(*(inp[n] for n in ("q", "k", "v", "a", "qn", "r")), l0, eta0, do=up["do"],
                      dlT=up["dlT"], detaT=up["detaT"], cov=oracle.DIAG if cov == "diag" else oracle.ISO)


def bwd_errors(hip, ref, cov):
    errs = {}
    for n in GRADS:
        lead = 1 if (n == "dqn" and cov == "diag") else 2
        errs[n] = slab_err(hip[n], ref[n], lead)
    return errs


def check(hip, ref, cov, dtype, what):
    for n in GRADS:
        assert np.all(np.isfinite(hip[n])), (what, n)
    errs = bwd_errors(hip, ref, cov)
    print(what, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL[dtype]}
    assert not bad, f"{what}: {bad} exceed {TOL[dtype]}"


@pytest.mark.parametrize("cov", ["diag", "iso"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("T", [1, 6, 37])
def test_bwd_matrix_with_state(cov, dtype, d, T):
    """Every head dim, both dtypes and covariances, ragged token blocks,
    non-trivial l0/eta0 and final-state gradients; B = 2 so the diagonal qn
    gradient sums over the batch."""
    _print_case("bwd", cov, dtype, d, T)
    base = "small_diag" if cov == "diag" else "iso"
    inp = gen.make_inputs(base, seed=300 + T + d, B=2, H=3, T=T, dk=d, dv=d, dtype=dtype)
    w = inp["workload"]
    st = gen.make_state(w, seed=301)
    up = gen.make_upstream(w, seed=302)
    check(run_bwd(inp, up, cov, st), run_ref(inp, up, cov, st), cov, dtype, f"bwd {cov} {dtype} d={d} T={T}")


@pytest.mark.parametrize("name,over", [
    ("lm_diag", dict(B=1, H=2, T=300)),
    ("long_diag", dict(B=1, H=2, T=600)),
    ("symbols_diag", dict(B=4, H=4)),
    ("iso", dict(B=1, H=3, T=500)),
    ("small_diag", {}),
])
def test_bwd_workload_distributions(name, over):
    """The benchmark workloads' value distributions, default state."""
    _print_case("bwd workload", name, over)
    inp = gen.make_inputs(name, seed=310, **over)
    w = inp["workload"]
    up = gen.make_upstream(w, seed=311)
    check(run_bwd(inp, up, w.cov), run_ref(inp, up, w.cov), w.cov, w.dtype, f"bwd {name}")


@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_bwd_empty_sequence(cov):
    _print_case("bwd empty", cov)
    inp = gen.make_inputs("small_diag" if cov == "diag" else "iso", seed=320, B=2, H=2, T=0,
                          dk=32, dv=32)
    w = inp["workload"]
    st = gen.make_state(w, seed=321)
    up = gen.make_upstream(w, seed=322)
    hip = run_bwd(inp, up, cov, st)
    assert np.array_equal(hip["dl0"], up["dlT"].double().numpy())
    assert np.array_equal(hip["deta0"], up["detaT"].double().numpy())
    if cov == "diag":
        assert np.all(hip["dqn"] == 0)


@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_bwd_adversarial_gates(cov):
    """a -> 0.01 (every 7th token 0.9), r = 1e-3, |k| up to 5: gates and
    precisions spanning many orders of magnitude; finite and at parity."""
    _print_case("bwd adversarial", cov)
    T = 60
    inp = gen.make_inputs("small_diag" if cov == "diag" else "iso", seed=330, B=1, H=2, T=T,
                          dk=32, dv=32, dtype="f32")
    g = torch.Generator().manual_seed(331)
    a = torch.full(inp["a"].shape, 0.01)
    a[:, :, ::7] = 0.9
    inp["a"] = a
    inp["r"] = torch.full((1, 2, T), 1e-3)
    inp["k"] = 5 * (2 * torch.rand(1, 2, T, 32, generator=g) - 1)
    w = inp["workload"]
    st = gen.make_state(w, seed=332)
    up = gen.make_upstream(w, seed=333)
    check(run_bwd(inp, up, cov, st), run_ref(inp, up, cov, st), cov, "f32", f"bwd adversarial {cov}")


def test_bwd_deterministic():
    _print_case("bwd determinism")
    inp = gen.make_inputs("lm_diag", seed=340, B=2, H=2, T=200)
    w = inp["workload"]
    up = gen.make_upstream(w, seed=341)
    a = run_bwd(inp, up, "diag")
    b = run_bwd(inp, up, "diag")
    for n in GRADS:
        assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("nrg", ["1", "2", "4"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_row_groups(monkeypatch, nrg, dtype):
    """Token-serial kernels: dk = 128 with its key dims on 1, 2 or 4 workgroups per (b,h) (the
    row-group partials of dv and dr summed by the combine pass), ragged token
    blocks, a state and final-state gradients; and the row split equals the
    whole-row kernel to the fp32 bar."""
    _print_case("bwd row groups", nrg, dtype)
    monkeypatch.setenv("KLA_BWD_IMPL", "rows")  # the token-serial kernels, not the chunked ones
    monkeypatch.setenv("KLA_BWD_NRG", nrg)
    inp = gen.make_inputs("small_diag", seed=350, B=2, H=3, T=77, dk=128, dv=128, dtype=dtype)
    w = inp["workload"]
    up = gen.make_upstream(w, seed=351)
    st = gen.make_state(w, seed=352)
    hip = run_bwd(inp, up, "diag", st)
    check(hip, run_ref(inp, up, "diag", st), "diag", dtype, f"bwd row groups {nrg} {dtype}")
    monkeypatch.setenv("KLA_BWD_NRG", "1")
    whole = run_bwd(inp, up, "diag", st)
    errs = bwd_errors(hip, whole, "diag")
    assert all(v <= 1e-5 for v in errs.values()), errs


def test_bwd_full_lm_shape_every_sequence():
    """The LM-layer shape (B8 H16 T2048 d128 bf16, row-split by default),
    every gradient of every (b,h) against the oracle."""
    _print_case("bwd full lm shape")
    inp = gen.make_inputs("lm_diag", seed=0)
    w = inp["workload"]
    up = gen.make_upstream(w, seed=1)
    check(run_bwd(inp, up, "diag"), run_ref(inp, up, "diag"), "diag", "bf16", "bwd full lm shape")


# ------------------------------------------------ chunked kernels (bf16, diag, d 64 / 128)

@pytest.mark.parametrize("cov,d", [("diag", 64), ("diag", 128), ("iso", 64)])
@pytest.mark.parametrize("T", [1, 16, 45, 300])
def test_bwd_chunk_with_state(cov, d, T):
    """The chunked backward: ragged last chunks, a state, final-state
    gradients, B*H = 10 (a grid padded to the XCD pattern at d 128)."""
    _print_case("bwd chunk", cov, d, T)
    inp = gen.make_inputs("lm_diag" if cov == "diag" else "iso", seed=360 + T + d, B=2, H=5, T=T, dk=d, dv=d)
    w = inp["workload"]
    st = gen.make_state(w, seed=361)
    up = gen.make_upstream(w, seed=362)
    check(run_bwd(inp, up, cov, st), run_ref(inp, up, cov, st), cov, "bf16", f"bwd chunk {cov} d={d} T={T}")


@pytest.mark.parametrize("cov,d", [("diag", 64), ("diag", 128), ("iso", 64)])
def test_bwd_chunk_hands_back_out_of_range(cov, d):
    """a = 0.01 on one head: its decay products leave [2^-64, 2^64] within a
    chunk, so the token-serial kernel redoes that (b,h) (and, at d 64, the
    one sharing its workgroup); the rest stay on the chunked path."""
    _print_case("bwd chunk hand-back", cov, d)
    inp = gen.make_inputs("lm_diag" if cov == "diag" else "iso", seed=370, B=2, H=3, T=50, dk=d, dv=d)
    a = inp["a"].clone()
    a[0, 1] = 0.01
    inp["a"] = a
    w = inp["workload"]
    st = gen.make_state(w, seed=371)
    up = gen.make_upstream(w, seed=372)
    check(run_bwd(inp, up, cov, st), run_ref(inp, up, cov, st), cov, "bf16", f"bwd hand-back {cov} d={d}")


@pytest.mark.parametrize("name", ["long_diag", "iso"])
def test_bwd_chunk_matches_token_serial(monkeypatch, name):
    """Chunked and token-serial kernels on the same inputs (long-context and
    isotropic laws): every gradient within the bf16 bar of each other."""
    _print_case("bwd chunk vs token-serial", name)
    inp = gen.make_inputs(name, seed=380, B=1, H=4, T=400)
    w = inp["workload"]
    up = gen.make_upstream(w, seed=381)
    chunk = run_bwd(inp, up, w.cov)
    monkeypatch.setenv("KLA_BWD_IMPL", "rows")
    serial = run_bwd(inp, up, w.cov)
    errs = bwd_errors(chunk, serial, w.cov)
    print("chunk vs serial", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert all(v <= TOL["bf16"] for v in errs.values()), errs


@pytest.mark.parametrize("cov,d", [("diag", 64), ("diag", 128), ("iso", 64)])
def test_bwd_chunk_wait_timeout_hands_back(monkeypatch, cov, d):
    """The reverse sweep's in-workgroup wait, forced to give up at once from
    the host (KLA_BWD_SPIN=0): every (b,h) is flagged and redone by the
    token-serial kernel, and the gradients still match the oracle."""
    _print_case("bwd chunk forced hand-back", cov, d)
    monkeypatch.setenv("KLA_BWD_SPIN", "0")
    inp = gen.make_inputs("lm_diag" if cov == "diag" else "iso", seed=390, B=2, H=3, T=70, dk=d, dv=d)
    w = inp["workload"]
    st = gen.make_state(w, seed=391)
    up = gen.make_upstream(w, seed=392)
    got = run_bwd(inp, up, cov, st)
    check(got, run_ref(inp, up, cov, st), cov, "bf16", f"bwd forced hand-back {cov} d={d}")
    # the same kernel run directly (one row group) gives the same bits
    monkeypatch.setenv("KLA_BWD_IMPL", "rows")
    monkeypatch.setenv("KLA_BWD_NRG", "1")
    serial = run_bwd(inp, up, cov, st)
    for n in GRADS:
        assert np.array_equal(got[n], serial[n]), n
