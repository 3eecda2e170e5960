"""Seeded synthetic inputs for the KLA forward workloads.

This module holds no arithmetic of the method: it only draws the inputs
(queries, keys, values, OU decay, process noise, observation noise) with the
distributions of the workloads and casts them to their storage dtypes.  Both
the HIP path and the fp64 oracle are fed from here.

Workloads (all draws in fp64 on the CPU from a seeded torch.Generator, in a
fixed order, then cast; N(mu, s2) below has VARIANCE s2):

  small_diag   B1 H2 T256 dk=dv=16, fp32.  q,k ~ N(0, 1/dk); v ~ N(0,1);
               a = sigmoid(N(2,1)) per token and key; qn = softplus(N(-2,0.5))
               per key; r = softplus(N(0,0.5)) + 1e-3 per token; l0=1, eta0=0.
  lm_diag      B8 H16 T2048 dk=dv=128, bf16 q/k/v/o, fp32 everything else;
               distributions as small_diag (q,k ~ N(0,1/dk)).
  long_diag    B1 H16 T32768 dk=dv=128, bf16; a = sigmoid(N(4,1)) (slow decay).
  symbols_diag B512 H4 T128 dk=dv=32, fp32.  A seeded N(0,1) table E[60,32];
               symbols ~ U{0..59} per (b,t), shared by all heads; k = v = E[sym];
               q ~ N(0,1/dk); a, qn as small_diag; r = softplus(N(0,1)) + 1e-3.
  iso          B4 H32 T8192 dk=dv=64, bf16 q/k/v/o, isotropic: a, qn, r are
               per (b,h,t) scalars with the small_diag distributions.
  iso_decode   B256 H32 dk=dv=64, iso: a 128-token prefix (seed 1) builds the
               cached states, then 64 decode tokens (seed 2).

Any of B, H, T may be overridden to get a smaller case with the same
distributions (used for parity tests the oracle finishes in seconds).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    cov: str          # "diag" or "iso"
    dtype: str        # storage dtype of q, k, v, o: "f32" or "bf16"
    a_mu: float = 2.0
    r_var: float = 0.5
    symbols: bool = False

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "small_diag": Workload("small_diag", 1, 2, 256, 16, 16, "diag", "f32"),
    "lm_diag": Workload("lm_diag", 8, 16, 2048, 128, 128, "diag", "bf16"),
    "long_diag": Workload("long_diag", 1, 16, 32768, 128, 128, "diag", "bf16", a_mu=4.0),
    "symbols_diag": Workload("symbols_diag", 512, 4, 128, 32, 32, "diag", "f32", r_var=1.0,
                             symbols=True),
    "iso": Workload("iso", 4, 32, 8192, 64, 64, "iso", "bf16"),
}

DECODE = Workload("iso_decode", 256, 32, 128, 64, 64, "iso", "bf16")
DECODE_STEPS = 64
# serving: a 16-token chunk (prefill piece or multi-token decode) continuing
# the cached states of the decode batch (T is the chunk length; the states
# come from a DECODE.T-token prefix forward)
PREFILL = Workload("iso_prefill16", 256, 32, 16, 64, 64, "iso", "bf16")
# the residual-write forward at the LM-layer shape (same draws as lm_diag)
RESIDUAL = Workload("residual_lm_diag", 8, 16, 2048, 128, 128, "diag", "bf16")

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPE[name]


def _softplus(x: torch.Tensor) -> torch.Tensor:
    return torch.nn.functional.softplus(x)


def make_inputs(w: Workload | str, seed: int = 0, device: str | torch.device = "cpu",
                **override) -> dict:
    """Draw one workload's inputs.  Returns a dict of tensors on ``device``:
    q, k, v (storage dtype), a, qn, r (fp32); l0/eta0 are None (l0 = 1, eta0 = 0).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    if override:
        w = w.with_(**override)
    g = torch.Generator(device="cpu").manual_seed(seed)
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    f64 = torch.float64

    def randn(*shape):
        return torch.randn(*shape, generator=g, dtype=f64)

    if w.symbols:
        table = randn(60, dk)
        sym = torch.randint(0, 60, (B, T), generator=g)
        kv = table[sym]                                   # [B,T,dk]
        k = kv[:, None].expand(B, H, T, dk).contiguous()
        v = kv[:, None].expand(B, H, T, dv).contiguous() if dv == dk else randn(B, H, T, dv)
        q = randn(B, H, T, dk) / math.sqrt(dk)
    else:
        q = randn(B, H, T, dk) / math.sqrt(dk)
        k = randn(B, H, T, dk) / math.sqrt(dk)
        v = randn(B, H, T, dv)
    if w.cov == "diag":
        a = torch.sigmoid(w.a_mu + randn(B, H, T, dk))
        qn = _softplus(-2.0 + math.sqrt(0.5) * randn(H, dk))
    else:
        a = torch.sigmoid(w.a_mu + randn(B, H, T))
        qn = _softplus(-2.0 + math.sqrt(0.5) * randn(B, H, T))
    r = _softplus(math.sqrt(w.r_var) * randn(B, H, T)) + 1e-3

    st = _TORCH_DTYPE[w.dtype]
    out = {
        "q": q.to(st), "k": k.to(st), "v": v.to(st),
        "a": a.to(torch.float32), "qn": qn.to(torch.float32), "r": r.to(torch.float32),
        "l0": None, "eta0": None, "workload": w,
    }
    for key in ("q", "k", "v", "a", "qn", "r"):
        out[key] = out[key].to(device)
    return out


# the fused block prologue at the LM-layer shape: pre-activations drawn so
# that the prologue's a, qn and r have the lm_diag distributions
BLOCK = Workload("block_lm_diag", 8, 16, 2048, 128, 128, "diag", "bf16")
# and at the long-context shape (same draws as long_diag's laws)
BLOCK_LONG = Workload("block_long_diag", 1, 16, 32768, 128, 128, "diag", "bf16", a_mu=4.0)
BLOCK_WIDTH = 4


def make_block_inputs(w: Workload | str, seed: int = 0, device="cpu", width: int = BLOCK_WIDTH,
                      bias: bool = True, state: bool = False, **override) -> dict:
    """Inputs of the fused block prologue (diagonal covariance).

    xq, xk, xv ~ N(0,1) (storage dtype): the projections before the causal
    convolution; za ~ N(a_mu, 1) (storage dtype), so that sigmoid(za) has the
    workload's distribution of a; zqn ~ N(-2, 0.5) [H,dk] and
    zr ~ N(0, r_var) [B,H,T] (fp32), so that softplus(zqn) and
    softplus(zr) + 1e-3 have the workload's qn and r; convolution taps
    wq, wk, wv [H,d,width] ~ U(-1/sqrt(width), 1/sqrt(width)) and, with bias,
    biases [H,d] from the same law (fp32); with state, convolution states
    [B,H,width-1,d] ~ N(0,1) (storage dtype), else None.  r_eps = 1e-3.
    """
    if isinstance(w, str):
        w = {BLOCK.name: BLOCK, BLOCK_LONG.name: BLOCK_LONG}.get(w) or WORKLOADS[w]
    if override:
        w = w.with_(**override)
    g = torch.Generator(device="cpu").manual_seed(seed)
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    f64 = torch.float64

    def randn(*shape):
        return torch.randn(*shape, generator=g, dtype=f64)

    def unif(*shape):
        return (2.0 * torch.rand(*shape, generator=g, dtype=f64) - 1.0) / math.sqrt(width)

    st = _TORCH_DTYPE[w.dtype]
    out = {
        "xq": randn(B, H, T, dk).to(st), "xk": randn(B, H, T, dk).to(st),
        "xv": randn(B, H, T, dv).to(st),
        "za": (w.a_mu + randn(B, H, T, dk)).to(st),
        "zqn": (-2.0 + math.sqrt(0.5) * randn(H, dk)).to(torch.float32),
        "zr": (math.sqrt(w.r_var) * randn(B, H, T)).to(torch.float32),
        "wq": unif(H, dk, width).to(torch.float32), "wk": unif(H, dk, width).to(torch.float32),
        "wv": unif(H, dv, width).to(torch.float32),
        "bq": None, "bk": None, "bv": None, "sq": None, "sk": None, "sv": None,
        "r_eps": 1e-3, "width": width, "workload": w,
    }
    if bias:
        out["bq"] = unif(H, dk).to(torch.float32)
        out["bk"] = unif(H, dk).to(torch.float32)
        out["bv"] = unif(H, dv).to(torch.float32)
    if state:
        out["sq"] = randn(B, H, width - 1, dk).to(st)
        out["sk"] = randn(B, H, width - 1, dk).to(st)
        out["sv"] = randn(B, H, width - 1, dv).to(st)
    for key, val in out.items():
        if isinstance(val, torch.Tensor):
            out[key] = val.to(device)
    return out


def make_state(w: Workload, seed: int, device="cpu") -> dict:
    """A non-trivial starting state for handoff tests: l0 = softplus(N(0,1)) + 0.2
    (positive), eta0 ~ N(0,1) (any real information vector is valid)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    nl = (w.B, w.H, w.dk) if w.cov == "diag" else (w.B, w.H)
    l0 = _softplus(torch.randn(*nl, generator=g, dtype=torch.float64)) + 0.2
    eta0 = torch.randn(w.B, w.H, w.dk, w.dv, generator=g, dtype=torch.float64)
    return {"l0": l0.to(torch.float32).to(device), "eta0": eta0.to(torch.float32).to(device)}


def make_upstream(w: Workload, seed: int, device="cpu") -> dict:
    """Upstream gradients for a backward pass of workload w: do ~ N(0,1) in the
    storage dtype [B,H,T,dv]; dlT ~ N(0,1) (shape of lT) and detaT ~ N(0,1)
    [B,H,dk,dv] in fp32."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    nl = (w.B, w.H, w.dk) if w.cov == "diag" else (w.B, w.H)
    do = torch.randn(w.B, w.H, w.T, w.dv, generator=g, dtype=torch.float64)
    dlT = torch.randn(*nl, generator=g, dtype=torch.float64)
    detaT = torch.randn(w.B, w.H, w.dk, w.dv, generator=g, dtype=torch.float64)
    return {"do": do.to(_TORCH_DTYPE[w.dtype]).to(device), "dlT": dlT.to(torch.float32).to(device),
            "detaT": detaT.to(torch.float32).to(device)}
