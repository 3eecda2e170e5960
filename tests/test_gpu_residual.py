"""GPU parity of the residual-write forward (klaFwdResidual through the C
ABI) against the fp64 oracle (oracle.fwd_residual), on seeded inputs from
scan_amd.inputs.  Small cases compare every element; the LM-layer shape
compares sampled (b,h) sequences.  Parity metric and bars as the KLA
forward (tests.gpu_util).  Diagonal dk 64 / 128 run the chunked matrix-core
kernel (exact sums where the decay products leave its range), and so do
isotropic dk 64 / 128; the rest, and those shapes under KLA_RES_IMPL=block,
the block kernel."""
import numpy as np
import pytest
import torch

import oracle
import scan_amd
from scan_amd import inputs as gen
from tests.gpu_util import assert_parity, compare, to_dev

pytestmark = pytest.mark.gpu


def _print_case(*args):
    print("CASE residual", *args, flush=True)


def run_hip_res(inp, cov, l0=None, m0=None):
    o, lT, mT = scan_amd.fwd_residual(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]),
                                      to_dev(inp["a"]), to_dev(inp["qn"]), to_dev(inp["r"]),
                                      to_dev(l0), to_dev(m0), cov=cov)
    torch.cuda.synchronize()
    return {"o": o.double().cpu().numpy(), "lT": lT.double().cpu().numpy(),
            "etaT": mT.double().cpu().numpy()}


def run_oracle_res(inp, cov, l0=None, m0=None):
    res = oracle.fwd_residual(inp["q"], inp["k"], inp["v"], inp["a"], inp["qn"], inp["r"], l0, m0,
                              cov=oracle.DIAG if cov == "diag" else oracle.ISO)
    return {"o": res["o"], "lT": res["lT"], "etaT": res["mT"]}


@pytest.mark.parametrize("cov", ["diag", "iso"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("T", [1, 3, 4, 8, 9, 16, 17, 70])
def test_residual_parity(cov, dtype, d, T):
    """Blocks of four tokens (eight on the matrix-core layout at d 128), whole
    or with a ragged last block, from a cached state."""
    _print_case(cov, dtype, d, T)
    base = "small_diag" if cov == "diag" else "iso"
    inp = gen.make_inputs(base, seed=90 + T + d, B=3, H=2, T=T, dk=d, dv=d, dtype=dtype)
    st = gen.make_state(inp["workload"], seed=17)
    hip = run_hip_res(inp, cov, st["l0"], st["eta0"])
    ref = run_oracle_res(inp, cov, st["l0"], st["eta0"])
    assert_parity(compare(hip, ref), dtype, f"residual {cov} {dtype} d={d} T={T}")


@pytest.mark.parametrize("cov", ["diag", "iso"])
@pytest.mark.parametrize("d", [16, 32, 64])
def test_residual_packed_heads_and_default_state(cov, d):
    """35 (b,h) leave the last workgroup partly filled (16 heads of d 16, 8 of
    d 32, 2 of d 64 per workgroup); l0 = 1, m0 = 0 by NULL pointers."""
    _print_case("packed", cov, d)
    base = "small_diag" if cov == "diag" else "iso"
    inp = gen.make_inputs(base, seed=60 + d, B=5, H=7, T=13, dk=d, dv=d, dtype="bf16")
    hip = run_hip_res(inp, cov)
    ref = run_oracle_res(inp, cov)
    assert_parity(compare(hip, ref), "bf16", f"residual packed {cov} d={d}")


@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_residual_empty_sequence_passes_state(cov):
    _print_case("T=0", cov)
    base = "small_diag" if cov == "diag" else "iso"
    inp = gen.make_inputs(base, seed=3, B=2, H=3, T=0, dk=64, dv=64, dtype="f32")
    st = gen.make_state(inp["workload"], seed=5)
    hip = run_hip_res(inp, cov, st["l0"], st["eta0"])
    assert np.array_equal(hip["lT"], st["l0"].double().numpy())
    assert np.array_equal(hip["etaT"], st["eta0"].double().numpy())


def test_residual_split_handoff():
    """Two calls, the second continuing from the first's state, equal one call
    within the fp32 parity bar (the matrix-core layout rounds its split bf16
    products differently when the block boundaries move)."""
    _print_case("handoff")
    inp = gen.make_inputs("small_diag", seed=8, B=2, H=2, T=50, dk=64, dv=64, dtype="f32")
    full = run_hip_res(inp, "diag")
    a = {k: (v[:, :, :21] if isinstance(v, torch.Tensor) and k != "qn" else v) for k, v in inp.items()}
    b = {k: (v[:, :, 21:] if isinstance(v, torch.Tensor) and k != "qn" else v) for k, v in inp.items()}
    first = run_hip_res(a, "diag")
    second = run_hip_res(b, "diag", torch.from_numpy(first["lT"]).float(),
                         torch.from_numpy(first["etaT"]).float())
    cat = np.concatenate([first["o"], second["o"]], axis=2)
    eo = float(np.abs(cat - full["o"]).max() / np.abs(full["o"]).max())
    em = float(np.abs(second["etaT"] - full["etaT"]).max() / np.abs(full["etaT"]).max())
    print("handoff differences", eo, em)
    assert eo < 1e-4 and em < 1e-4, (eo, em)


RES_SAMPLES = [(0, 0), (3, 7), (7, 15)]


def test_residual_lm_layer_sampled():
    """The LM-layer shape (B8 H16 T2048 d128 bf16, diag) in the benchmark's
    launch configuration; three sampled (b,h) against the oracle."""
    _print_case("lm layer")
    w = gen.RESIDUAL
    inp = gen.make_inputs(w, seed=0)
    hip = run_hip_res(inp, w.cov)
    sub_in = {k: (v[[b for b, _ in RES_SAMPLES], [h for _, h in RES_SAMPLES]][None]
                  if isinstance(v, torch.Tensor) and k != "qn" else v) for k, v in inp.items()}
    # the oracle runs each sampled sequence with its own head's qn
    outs = {"o": [], "lT": [], "etaT": []}
    for n, (b, h) in enumerate(RES_SAMPLES):
        one = {k: (v[:, n:n + 1] if isinstance(v, torch.Tensor) and k != "qn" else v)
               for k, v in sub_in.items()}
        one["qn"] = inp["qn"][h:h + 1]
        r = run_oracle_res(one, w.cov)
        for k in outs:
            outs[k].append(r[k][0, 0])
    ref = {k: np.stack(v) for k, v in outs.items()}
    sub = {k: np.stack([hip[k][b, h] for b, h in RES_SAMPLES]) for k in hip}
    errs = compare(sub, ref, nlead=1)
    print("residual lm layer", errs)
    assert_parity(errs, w.dtype, "residual lm layer")
    for k in hip:
        assert np.all(np.isfinite(hip[k])), k


@pytest.mark.parametrize("cov", ["diag", "iso"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nvt", ["1", "2"])
def test_residual_value_tiles(cov, d, nvt, monkeypatch):
    """Each (b,h) whole in one workgroup, or split into two value tiles."""
    _print_case("tiles", cov, d, nvt)
    monkeypatch.setenv("KLA_RES_VTILES", nvt)
    base = "small_diag" if cov == "diag" else "iso"
    inp = gen.make_inputs(base, seed=120 + d, B=2, H=3, T=23, dk=d, dv=d, dtype="f32")
    st = gen.make_state(inp["workload"], seed=19)
    hip = run_hip_res(inp, cov, st["l0"], st["eta0"])
    ref = run_oracle_res(inp, cov, st["l0"], st["eta0"])
    assert_parity(compare(hip, ref), "f32", f"residual tiles {cov} d={d} nvt={nvt}")


@pytest.mark.parametrize("cov", ["diag", "iso"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_residual_adversarial_gates(cov, dtype):
    """a -> 0.01 (every 7th token 0.9), r = 1e-3, |k| up to 5: near-exact
    interpolating writes and fast decay; finite and at parity."""
    _print_case("adversarial", cov, dtype)
    T = 200
    base = "small_diag" if cov == "diag" else "iso"
    inp = gen.make_inputs(base, seed=24, B=1, H=3, T=T, dk=64, dv=64, dtype=dtype)
    g = torch.Generator().manual_seed(25)
    a = torch.full(inp["a"].shape, 0.01)
    a[:, :, ::7] = 0.9
    inp["a"] = a
    inp["r"] = torch.full((1, 3, T), 1e-3)
    inp["k"] = (5 * (2 * torch.rand(1, 3, T, 64, generator=g) - 1)).to(inp["k"].dtype)
    hip = run_hip_res(inp, cov)
    for k in hip:
        assert np.all(np.isfinite(hip[k])), k
    ref = run_oracle_res(inp, cov)
    assert_parity(compare(hip, ref), dtype, f"residual adversarial {cov}")


@pytest.mark.parametrize("cov", ["diag", "iso"])
@pytest.mark.parametrize("d", [64, 128])
def test_residual_thread_row_layout(cov, d, monkeypatch):
    """KLA_RES_MM=0: 64-column tiles on the thread-row layout instead of the
    matrix cores (the layout d 16 / 32 always use)."""
    _print_case("thread rows", cov, d)
    monkeypatch.setenv("KLA_RES_MM", "0")
    base = "small_diag" if cov == "diag" else "iso"
    inp = gen.make_inputs(base, seed=130 + d, B=2, H=3, T=22, dk=d, dv=d, dtype="f32")
    st = gen.make_state(inp["workload"], seed=21)
    hip = run_hip_res(inp, cov, st["l0"], st["eta0"])
    ref = run_oracle_res(inp, cov, st["l0"], st["eta0"])
    assert_parity(compare(hip, ref), "f32", f"residual thread rows {cov} d={d}")


@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_residual_many_heads_d128(cov):
    """512 (b,h) at d 128: one whole-head tile per workgroup (thread rows)."""
    _print_case("many heads", cov)
    base = "small_diag" if cov == "diag" else "iso"
    inp = gen.make_inputs(base, seed=140, B=32, H=16, T=9, dk=128, dv=128, dtype="bf16")
    hip = run_hip_res(inp, cov)
    sel = [(0, 0), (13, 7), (31, 15)]
    per_head = "qn" if cov == "diag" else None  # diag qn is [H, dk]; iso qn is per (b,h,t)
    sub = {k: (v[[b for b, _ in sel], [h for _, h in sel]][None]
               if isinstance(v, torch.Tensor) and k != per_head else v) for k, v in inp.items()}
    outs = {"o": [], "lT": [], "etaT": []}
    for n, (b, h) in enumerate(sel):
        one = {k: (v[:, n:n + 1] if isinstance(v, torch.Tensor) and k != per_head else v)
               for k, v in sub.items()}
        if cov == "diag":
            one["qn"] = inp["qn"][h:h + 1]
        r = run_oracle_res(one, cov)
        for k in outs:
            outs[k].append(r[k][0, 0])
    ref = {k: np.stack(v) for k, v in outs.items()}
    got = {k: np.stack([hip[k][b, h] for b, h in sel]) for k in hip}
    assert_parity(compare(got, ref, nlead=1), "bf16", f"residual many heads {cov}")


@pytest.mark.parametrize("cov", ["diag", "iso"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_residual_chunk_ragged_grid_every_sequence(cov, dtype, d):
    """19 (b,h), so the 8-apart value tiles leave padding workgroups; chunks of
    16 with a ragged last one; every sequence against the oracle."""
    _print_case("chunk grid", cov, dtype, d)
    base = "small_diag" if cov == "diag" else "iso"
    inp = gen.make_inputs(base, seed=150 + d, B=1, H=19, T=41, dk=d, dv=d, dtype=dtype)
    st = gen.make_state(inp["workload"], seed=23)
    hip = run_hip_res(inp, cov, st["l0"], st["eta0"])
    ref = run_oracle_res(inp, cov, st["l0"], st["eta0"])
    assert_parity(compare(hip, ref), dtype, f"residual chunk grid {cov} {dtype} d={d}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_residual_chunk_partial_fallback(dtype):
    """d 128: key dims 0..63 decay fast enough (a = 0.02) that their decay
    products leave the factorisation range within a chunk, dims 64..127 do
    not; the first half is summed exactly, the second on the matrix cores."""
    _print_case("chunk partial fallback", dtype)
    inp = gen.make_inputs("small_diag", seed=160, B=2, H=2, T=70, dk=128, dv=128, dtype=dtype)
    a = inp["a"].clone()
    a[..., :64] = 0.02
    a[:, 1, 33:, 64:] = 0.03          # head 1: the second half leaves it too, from token 33
    inp["a"] = a
    st = gen.make_state(inp["workload"], seed=29)
    hip = run_hip_res(inp, "diag", st["l0"], st["eta0"])
    for k in hip:
        assert np.all(np.isfinite(hip[k])), k
    ref = run_oracle_res(inp, "diag", st["l0"], st["eta0"])
    assert_parity(compare(hip, ref), dtype, f"residual chunk partial fallback {dtype}")


@pytest.mark.parametrize("cov", ["diag", "iso"])
def test_residual_chunk_matches_block_kernel(cov, monkeypatch):
    """The chunked kernel and the block kernel (KLA_RES_IMPL=block) agree on
    the LM-layer draws within the bf16 bar (both also meet the oracle)."""
    _print_case("chunk vs block", cov)
    inp = gen.make_inputs(gen.RESIDUAL if cov == "diag" else "iso", seed=3, B=2, H=4, T=300,
                          dk=128, dv=128, dtype="bf16")
    chunk = run_hip_res(inp, cov)
    monkeypatch.setenv("KLA_RES_IMPL", "block")
    block = run_hip_res(inp, cov)
    ref = run_oracle_res(inp, cov)
    assert_parity(compare(chunk, ref), "bf16", "residual chunk vs oracle")
    assert_parity(compare(block, ref), "bf16", "residual block vs oracle")
    assert_parity(compare(chunk, block), "bf16", "residual chunk vs block")
