"""Helpers shared by the GPU parity tests: run the HIP path and the oracle on
the same seeded inputs and compare them with the parity metric.

Parity metric: for o and etaT, max |x - ref| / max |ref| over each (b,h)
slab, worst slab reported; for lT (always positive), elementwise |x-ref|/ref.
Bars: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import scan_amd

TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_dev(x):
    return None if x is None else x.to("cuda").contiguous()


def run_hip(inp, cov, l0=None, eta0=None):
    o, lT, etaT = scan_amd.fwd(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]),
                               to_dev(inp["a"]), to_dev(inp["qn"]), to_dev(inp["r"]),
                               to_dev(l0), to_dev(eta0), cov=cov)
    torch.cuda.synchronize()
    return {"o": o.double().cpu().numpy(), "lT": lT.double().cpu().numpy(),
            "etaT": etaT.double().cpu().numpy()}


def run_oracle(inp, cov, l0=None, eta0=None, sel=None):
    """Oracle on all sequences, or on the (b,h) pairs listed in sel."""
    q, k, v, a, qn, r = (inp[n] for n in ("q", "k", "v", "a", "qn", "r"))
    if sel is not None:
        bs = torch.tensor([s[0] for s in sel])
        hs = torch.tensor([s[1] for s in sel])

        def pick(x):
            return None if x is None else x[bs, hs][None]
        q, k, v, a, r = pick(q), pick(k), pick(v), pick(a), pick(r)
        if cov == "iso":
            qn = pick(qn)
            l0 = pick(l0)
        else:
            qn_sel = qn[hs]                        # [n, dk] per selected head
            l0 = pick(l0)
            eta0 = pick(eta0)
            out = {"o": [], "lT": [], "etaT": []}
            for n in range(len(sel)):
                res = oracle.fwd(q[:, n:n + 1], k[:, n:n + 1], v[:, n:n + 1], a[:, n:n + 1],
                                 qn_sel[n:n + 1], r[:, n:n + 1],
                                 None if l0 is None else l0[:, n:n + 1],
                                 None if eta0 is None else eta0[:, n:n + 1], cov=oracle.DIAG)
                for key in out:
                    out[key].append(res[key][0, 0])
            return {key: np.stack(vals) for key, vals in out.items()}
        eta0 = pick(eta0)
        res = oracle.fwd(q, k, v, a, qn, r, l0, eta0, cov=oracle.ISO)
        return {key: val[0] for key, val in res.items()}
    return oracle.fwd(q, k, v, a, qn, r, l0, eta0, cov=oracle.DIAG if cov == "diag" else oracle.ISO)


def slab_err(x, ref, nlead):
    """Worst over leading slabs of max|x-ref| / max|ref|."""
    x = x.reshape(int(np.prod(x.shape[:nlead])), -1)
    ref = ref.reshape(x.shape)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((np.abs(x - ref).max(axis=1) / den).max())


def rel_err(x, ref):
    return float((np.abs(x - ref) / np.abs(ref)).max())


def compare(hip, ref, nlead=2):
    return {"o": slab_err(hip["o"], ref["o"], nlead),
            "etaT": slab_err(hip["etaT"], ref["etaT"], nlead),
            "lT": rel_err(hip["lT"], ref["lT"])}


def assert_parity(errs, dtype, what=""):
    tol = TOL[dtype]
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    assert not bad, f"{what}: parity errors {errs} exceed {tol}"
