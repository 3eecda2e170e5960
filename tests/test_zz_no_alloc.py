"""klaFwdNoAlloc (the forward for callers that cannot allocate) against klaFwd
through the C ABI: two calls in a row on sequence-split shapes, the second
with a smaller input, each bit-identical to klaFwd with a caller workspace;
plus a shape that needs no workspace and one that needs more than the
library's device scratch (rejected before any work)."""
import pytest
import torch

import scan_amd
from scan_amd import KlaDims
from scan_amd import inputs as gen

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "a", "qn", "r")


def _case(name, **over):
    inp = gen.make_inputs(name, seed=61, device="cuda", **over)
    w = inp["workload"]
    st = gen.make_state(w, seed=62, device="cuda")
    dims = KlaDims(w.B, w.H, w.T, w.dk, w.dv, 1 if w.dtype == "bf16" else 0, 0 if w.cov == "diag" else 1)
    return inp, st, dims, w


def _outs(w, dtype):
    o = torch.empty(w.B, w.H, w.T, w.dv, dtype=dtype, device="cuda")
    lT = torch.empty((w.B, w.H, w.dk) if w.cov == "diag" else (w.B, w.H), device="cuda")
    eT = torch.empty(w.B, w.H, w.dk, w.dv, device="cuda")
    return o, lT, eT


def _ptrs(inp, st):
    return [inp[n].data_ptr() for n in NAMES] + [st["l0"].data_ptr(), st["eta0"].data_ptr()]


def _fwd_ref(inp, st, dims, w):
    o, lT, eT = _outs(w, inp["v"].dtype)
    nb = scan_amd.klaFwdWorkspaceBytes(dims)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    rc = scan_amd.klaFwd(dims, *_ptrs(inp, st), o.data_ptr(), lT.data_ptr(), eT.data_ptr(),
                         ws.data_ptr() if nb else None, nb, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, scan_amd.klaStatusString(rc)
    return o, lT, eT


def _fwd_noalloc(inp, st, dims, w):
    o, lT, eT = _outs(w, inp["v"].dtype)
    rc = scan_amd.klaFwdNoAlloc(dims, *_ptrs(inp, st), o.data_ptr(), lT.data_ptr(), eT.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    assert rc == 0, scan_amd.klaStatusString(rc)
    return o, lT, eT


def test_no_alloc_matches_klafwd_two_calls():
    # a sequence-split shape, then a smaller one (fewer heads, shorter), both
    # needing a workspace that the device scratch provides
    for name, over in (("long_diag", dict(B=1, H=4, T=6144)), ("long_diag", dict(B=1, H=2, T=3500))):
        print("CASE no-alloc", name, over, flush=True)
        inp, st, dims, w = _case(name, **over)
        need = scan_amd.klaFwdWorkspaceBytes(dims)
        assert 0 < need <= 64 << 20
        got = _fwd_noalloc(inp, st, dims, w)
        ref = _fwd_ref(inp, st, dims, w)
        torch.cuda.synchronize()
        for x, y in zip(got, ref):
            assert torch.equal(x, y)


def test_no_alloc_without_workspace_and_too_large():
    print("CASE no-alloc small / too large", flush=True)
    inp, st, dims, w = _case("lm_diag", B=2, H=2, T=100)
    assert scan_amd.klaFwdWorkspaceBytes(dims) == 0
    got = _fwd_noalloc(inp, st, dims, w)
    ref = _fwd_ref(inp, st, dims, w)
    torch.cuda.synchronize()
    for x, y in zip(got, ref):
        assert torch.equal(x, y)
    big = KlaDims(1, 16, 32768, 128, 128, 1, 0)      # the long-context workload: about 147 MB
    assert scan_amd.klaFwdWorkspaceBytes(big) > 64 << 20
    rc = scan_amd.klaFwdNoAlloc(big, *([16] * 9), 16, 16, None)   # rejected before any pointer is used
    assert rc == 5  # KLA_ERR_WORKSPACE
