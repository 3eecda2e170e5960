"""Thin Python binding of the gfx950 KLA forward library (include/kla.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libkla.so.  PyTorch provides device memory and the current HIP stream.  There
is no CPU fallback: if the library is missing or no GPU is present the calls
raise.

Low level (same names and arguments as the C ABI, raw device pointers):
    klaFwd, klaStep, klaFwdResidual, klaBwd, klaFwdWorkspaceBytes, klaBwdWorkspaceBytes,
    klaIsSupported, klaStatusString
Convenience (torch tensors in, torch tensors out):
    fwd(q, k, v, a, qn, r, l0=None, eta0=None, cov="diag") -> (o, lT, etaT)
    step(q, k, v, a, qn, r, l, eta, cov="diag") -> o      (l, eta updated in place)
    fwd_residual(q, k, v, a, qn, r, l0=None, m0=None, cov="diag") -> (o, lT, mT)
    bwd(q, k, v, a, qn, r, l0, eta0, do, dlT=None, detaT=None, cov="diag") -> dict of gradients
    fwd_block(xq, xk, xv, za, zqn, zr, wq, wk, wv, ...) -> (o, lT, etaT)  (fused block prologue)
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["klaFwd", "klaFwdNoAlloc", "klaFwdBlock", "klaStep", "klaFwdResidual", "klaBwd",
           "klaFwdWorkspaceBytes", "klaBwdWorkspaceBytes", "klaIsSupported", "klaStatusString",
           "KlaDims", "KlaBlock", "KlaError", "fwd", "fwd_block", "step", "fwd_residual", "bwd",
           "lib_path", "load"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkla.so")

KLA_OK = 0
KLA_F32, KLA_BF16 = 0, 1
KLA_DIAG, KLA_ISO = 0, 1
STATUS_NAMES = {0: "KLA_OK", 1: "KLA_ERR_NULL", 2: "KLA_ERR_SHAPE", 3: "KLA_ERR_UNSUPPORTED",
                4: "KLA_ERR_ALIGN", 5: "KLA_ERR_WORKSPACE", 6: "KLA_ERR_HIP",
                7: "KLA_ERR_INTERNAL", 8: "KLA_ERR_ALIAS"}


class KlaDims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("T", ctypes.c_int),
                ("dk", ctypes.c_int), ("dv", ctypes.c_int),
                ("dtype", ctypes.c_int), ("cov", ctypes.c_int)]


class KlaBlock(ctypes.Structure):
    """klaBlock of include/kla.h: convolution width, taps, biases, states, r_eps."""
    _fields_ = [("width", ctypes.c_int),
                ("wq", ctypes.c_void_p), ("wk", ctypes.c_void_p), ("wv", ctypes.c_void_p),
                ("bq", ctypes.c_void_p), ("bk", ctypes.c_void_p), ("bv", ctypes.c_void_p),
                ("sq", ctypes.c_void_p), ("sk", ctypes.c_void_p), ("sv", ctypes.c_void_p),
                ("r_eps", ctypes.c_float)]


class KlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {klaStatusString(status)}")


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libkla.so (built in-tree by scan_amd.build / __graft_entry__.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"HIP library {_LIB_PATH} is not built; run __graft_entry__.build()")
    try:  # share torch's HIP runtime (same soname) when torch is present
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(_LIB_PATH)
    vp, fp, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t
    dp = ctypes.POINTER(KlaDims)
    lib.klaIsSupported.argtypes = [dp]
    lib.klaIsSupported.restype = ctypes.c_int
    lib.klaFwdWorkspaceBytes.argtypes = [dp]
    lib.klaFwdWorkspaceBytes.restype = sz
    lib.klaFwd.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, fp, vp, fp, fp, vp, sz, vp]
    lib.klaFwd.restype = ctypes.c_int
    lib.klaStep.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, fp, vp, vp]
    lib.klaStep.restype = ctypes.c_int
    lib.klaFwdResidual.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, fp, vp, fp, fp, vp]
    lib.klaFwdResidual.restype = ctypes.c_int
    lib.klaStatusString.argtypes = [ctypes.c_int]
    lib.klaStatusString.restype = ctypes.c_char_p
    lib.klaFwdKernelName.argtypes = [dp]
    lib.klaFwdKernelName.restype = ctypes.c_char_p
    lib.klaFwdNoAlloc.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, fp, vp, fp, fp, vp]
    lib.klaFwdNoAlloc.restype = ctypes.c_int
    lib.klaBwdWorkspaceBytes.argtypes = [dp]
    lib.klaBwdWorkspaceBytes.restype = sz
    lib.klaBwd.argtypes = [dp] + [vp] * 19 + [vp, sz, vp]
    lib.klaBwd.restype = ctypes.c_int
    lib.klaFwdBlock.argtypes = [dp, ctypes.POINTER(KlaBlock)] + [vp] * 11 + [vp, sz, vp]
    lib.klaFwdBlock.restype = ctypes.c_int
    _lib = lib
    return lib


# ------------------------------------------------------------------ C ABI

def klaIsSupported(dims: KlaDims) -> bool:
    return bool(load().klaIsSupported(ctypes.byref(dims)))


def klaFwdWorkspaceBytes(dims: KlaDims) -> int:
    return int(load().klaFwdWorkspaceBytes(ctypes.byref(dims)))


def klaFwd(dims, q, k, v, a, qnoise, r, l0, eta0, o, lT, etaT, workspace, workspaceBytes,
           stream) -> int:
    """Raw call: pointer arguments are ints (device addresses) or None."""
    return int(load().klaFwd(ctypes.byref(dims), q, k, v, a, qnoise, r, l0, eta0, o, lT, etaT,
                             workspace, workspaceBytes, stream))


def klaFwdNoAlloc(dims, q, k, v, a, qnoise, r, l0, eta0, o, lT, etaT, stream) -> int:
    """Raw call of the forward that takes no workspace (pointers as ints or None)."""
    return int(load().klaFwdNoAlloc(ctypes.byref(dims), q, k, v, a, qnoise, r, l0, eta0, o, lT, etaT,
                                    stream))


def klaFwdBlock(dims, blk, xq, xk, xv, za, zqn, zr, l0, eta0, o, lT, etaT, workspace, workspaceBytes,
                stream) -> int:
    """Raw call of the forward with the fused block prologue (blk: KlaBlock or
    None; pointers as ints or None; the workspace as for klaFwd)."""
    return int(load().klaFwdBlock(ctypes.byref(dims), ctypes.byref(blk) if blk is not None else None,
                                  xq, xk, xv, za, zqn, zr, l0, eta0, o, lT, etaT, workspace,
                                  workspaceBytes, stream))


def klaStep(dims, q, k, v, a, qnoise, r, l, eta, o, stream) -> int:
    return int(load().klaStep(ctypes.byref(dims), q, k, v, a, qnoise, r, l, eta, o, stream))


def klaFwdResidual(dims, q, k, v, a, qnoise, r, l0, m0, o, lT, mT, stream) -> int:
    """Raw call of the residual-write forward (pointers as ints or None)."""
    return int(load().klaFwdResidual(ctypes.byref(dims), q, k, v, a, qnoise, r, l0, m0, o, lT, mT,
                                     stream))


def klaBwdWorkspaceBytes(dims: KlaDims) -> int:
    return int(load().klaBwdWorkspaceBytes(ctypes.byref(dims)))


def klaBwd(dims, q, k, v, a, qnoise, r, l0, eta0, dO, dlT, detaT, dq, dk, dv, da, dqnoise, dr, dl0,
           deta0, workspace, workspaceBytes, stream) -> int:
    """Raw call of the backward pass (pointers as ints or None)."""
    return int(load().klaBwd(ctypes.byref(dims), q, k, v, a, qnoise, r, l0, eta0, dO, dlT, detaT,
                             dq, dk, dv, da, dqnoise, dr, dl0, deta0, workspace, workspaceBytes,
                             stream))


def klaStatusString(status: int) -> str:
    try:
        return load().klaStatusString(int(status)).decode()
    except RuntimeError:
        return STATUS_NAMES.get(int(status), f"status {status}")


def klaFwdKernelName(dims: KlaDims) -> str:
    return load().klaFwdKernelName(ctypes.byref(dims)).decode()


def fwd_kernel_name(B, H, T, dk, dv, cov="diag", dtype="bf16") -> str:
    """Kernel family klaFwd launches for these sizes (for profiles and reports)."""
    dims = KlaDims(B, H, T, dk, dv, KLA_BF16 if dtype == "bf16" else KLA_F32,
                   KLA_DIAG if cov == "diag" else KLA_ISO)
    return klaFwdKernelName(dims)


# ------------------------------------------------------------------ torch helpers

def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return KLA_BF16
    if t.dtype == torch.float32:
        return KLA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _check_device(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("all tensors must be contiguous device tensors")


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def fwd(q, k, v, a, qn, r, l0=None, eta0=None, cov: str = "diag", o=None, lT=None, etaT=None,
        want_state: bool = True):
    """KLA forward on the current stream.  Returns (o, lT, etaT) as device tensors.

    q,k [B,H,T,dk], v [B,H,T,dv] (bf16 or fp32); a, qn, r, l0, eta0 fp32 in the
    layouts of include/kla.h.  Outputs are allocated unless passed in.
    """
    import torch
    _check_device(q, k, v, a, qn, r, l0, eta0)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    c = KLA_DIAG if cov == "diag" else KLA_ISO
    dims = KlaDims(B, H, T, dk, dv, _dtype_code(q), c)
    dev = q.device
    if o is None:
        o = torch.empty(B, H, T, dv, dtype=v.dtype, device=dev)
    if want_state:
        if lT is None:
            lT = torch.empty((B, H, dk) if c == KLA_DIAG else (B, H), dtype=torch.float32, device=dev)
        if etaT is None:
            etaT = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev)
    ws_bytes = klaFwdWorkspaceBytes(dims)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    st = klaFwd(dims, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(qn), _ptr(r), _ptr(l0), _ptr(eta0),
                _ptr(o), _ptr(lT), _ptr(etaT), _ptr(ws), ws_bytes, _stream())
    if st != KLA_OK:
        raise KlaError(st, "klaFwd")
    return o, lT, etaT


def fwd_block(xq, xk, xv, za, zqn, zr, wq, wk, wv, bq=None, bk=None, bv=None, sq=None, sk=None,
              sv=None, r_eps: float = 1e-3, l0=None, eta0=None, o=None, lT=None, etaT=None,
              want_state: bool = True):
    """KLA forward with the fused block prologue (diagonal covariance) on the
    current stream.  xq, xk, xv, za in the storage dtype, zqn [H,dk] and zr
    [B,H,T] fp32, taps [H,d,W] and biases [H,d] fp32, states [B,H,W-1,d] in the
    storage dtype.  Returns (o, lT, etaT); outputs are allocated unless passed
    in."""
    import torch
    _check_device(xq, xk, xv, za, zqn, zr, wq, wk, wv, bq, bk, bv, sq, sk, sv, l0, eta0)
    B, H, T, dk = xq.shape
    dv = xv.shape[-1]
    dims = KlaDims(B, H, T, dk, dv, _dtype_code(xq), KLA_DIAG)
    blk = KlaBlock(int(wq.shape[-1]), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(bq), _ptr(bk), _ptr(bv),
                   _ptr(sq), _ptr(sk), _ptr(sv), float(r_eps))
    dev = xq.device
    if o is None:
        o = torch.empty(B, H, T, dv, dtype=xv.dtype, device=dev)
    if want_state:
        if lT is None:
            lT = torch.empty(B, H, dk, dtype=torch.float32, device=dev)
        if etaT is None:
            etaT = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev)
    ws_bytes = klaFwdWorkspaceBytes(dims)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    st = klaFwdBlock(dims, blk, _ptr(xq), _ptr(xk), _ptr(xv), _ptr(za), _ptr(zqn), _ptr(zr),
                     _ptr(l0), _ptr(eta0), _ptr(o), _ptr(lT), _ptr(etaT), _ptr(ws), ws_bytes, _stream())
    if st != KLA_OK:
        raise KlaError(st, "klaFwdBlock")
    return o, lT, etaT


def step(q, k, v, a, qn, r, l, eta, cov: str = "diag", o=None):
    """One decode step on the current stream; l and eta are updated in place."""
    import torch
    _check_device(q, k, v, a, qn, r, l, eta)
    B, H, dk = q.shape
    dv = v.shape[-1]
    c = KLA_DIAG if cov == "diag" else KLA_ISO
    dims = KlaDims(B, H, 1, dk, dv, _dtype_code(q), c)
    if o is None:
        o = torch.empty(B, H, dv, dtype=v.dtype, device=q.device)
    st = klaStep(dims, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(qn), _ptr(r), _ptr(l), _ptr(eta),
                 _ptr(o), _stream())
    if st != KLA_OK:
        raise KlaError(st, "klaStep")
    return o


def fwd_residual(q, k, v, a, qn, r, l0=None, m0=None, cov: str = "diag", o=None, lT=None,
                 mT=None):
    """Residual-write forward on the current stream.  Returns (o, lT, mT), mT
    the posterior mean [B,H,dk,dv].  Layouts as ``fwd``; outputs are
    allocated unless passed in."""
    import torch
    _check_device(q, k, v, a, qn, r, l0, m0)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    c = KLA_DIAG if cov == "diag" else KLA_ISO
    dims = KlaDims(B, H, T, dk, dv, _dtype_code(q), c)
    dev = q.device
    if o is None:
        o = torch.empty(B, H, T, dv, dtype=v.dtype, device=dev)
    if lT is None:
        lT = torch.empty((B, H, dk) if c == KLA_DIAG else (B, H), dtype=torch.float32, device=dev)
    if mT is None:
        mT = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev)
    st = klaFwdResidual(dims, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(qn), _ptr(r), _ptr(l0),
                        _ptr(m0), _ptr(o), _ptr(lT), _ptr(mT), _stream())
    if st != KLA_OK:
        raise KlaError(st, "klaFwdResidual")
    return o, lT, mT


def bwd(q, k, v, a, qn, r, l0=None, eta0=None, do=None, dlT=None, detaT=None, cov: str = "diag",
        want_state: bool = True):
    """Backward pass of ``fwd`` on the current stream: the gradients of
    L = <do, o> + <dlT, lT> + <detaT, etaT>.  Returns a dict of device tensors
    dq, dk, dv (input dtype), da, dqn, dr, dl0, deta0 (fp32) in the shapes of
    the corresponding inputs (the diagonal dqn [H,dk] sums over the batch)."""
    import torch
    _check_device(q, k, v, a, qn, r, l0, eta0, do, dlT, detaT)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    c = KLA_DIAG if cov == "diag" else KLA_ISO
    dims = KlaDims(B, H, T, dk, dv, _dtype_code(q), c)
    dev = q.device
    out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
           "da": torch.empty_like(a), "dqn": torch.empty_like(qn), "dr": torch.empty_like(r)}
    out["dl0"] = (torch.empty((B, H, dk) if c == KLA_DIAG else (B, H), dtype=torch.float32, device=dev)
                  if want_state else None)
    out["deta0"] = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev) if want_state else None
    ws_bytes = klaBwdWorkspaceBytes(dims)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    st = klaBwd(dims, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(qn), _ptr(r), _ptr(l0), _ptr(eta0),
                _ptr(do), _ptr(dlT), _ptr(detaT), *(_ptr(out[n]) for n in
                                                     ("dq", "dk", "dv", "da", "dqn", "dr", "dl0", "deta0")),
                _ptr(ws), ws_bytes, _stream())
    if st != KLA_OK:
        raise KlaError(st, "klaBwd")
    return out
