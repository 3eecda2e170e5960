"""CPU-side contract of the C ABI (no GPU needed, no compute call).

Checks that libkla.so loads, exports every function include/kla.h declares,
and that every host-detectable argument error is returned before any HIP
call.  Pointer arguments here are fake (never dereferenced): validation
rejects the call before anything touches them.
"""
import ctypes
import os
import re
import subprocess

import pytest

import scan_amd
from scan_amd import KlaDims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kla.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS, HIP, INTERNAL, ALIAS = range(9)
F32, BF16 = 0, 1
DIAG, ISO = 0, 1

# fake, well separated, 256-byte aligned "device" addresses
BASE = 1 << 40


def addr(i):
    return BASE + i * (1 << 32)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S[^\n(]*?\b(kla[A-Z]\w*)\s*\(", text, re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = scan_amd.load()
    names = declared_functions()
    assert {"klaFwd", "klaStep", "klaFwdWorkspaceBytes", "klaStatusString",
            "klaIsSupported"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", scan_amd.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (kla\w+)$", out, re.M))
    assert set(names) <= exported


def test_status_strings_cover_every_code():
    seen = set()
    for s in range(9):
        txt = scan_amd.klaStatusString(s)
        assert txt.startswith(scan_amd.STATUS_NAMES[s])
        seen.add(txt)
    assert len(seen) == 9
    assert "unknown" in scan_amd.klaStatusString(99)


@pytest.mark.parametrize("dk", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("cov", [DIAG, ISO])
def test_supported_shapes(dk, dtype, cov):
    assert scan_amd.klaIsSupported(KlaDims(2, 3, 100, dk, dk, dtype, cov))
    assert scan_amd.klaFwdWorkspaceBytes(KlaDims(2, 3, 100, dk, dk, dtype, cov)) == 0


@pytest.mark.parametrize("dims", [(1, 1, 8, 48, 48), (1, 1, 8, 256, 256), (1, 1, 8, 64, 32),
                                  (1, 1, 8, 8, 8)])
def test_unsupported_shapes(dims):
    d = KlaDims(*dims, F32, DIAG)
    assert not scan_amd.klaIsSupported(d)
    assert fwd_call(d) == UNSUP


def fwd_call(d, **over):
    args = dict(q=addr(1), k=addr(2), v=addr(3), a=addr(4), qnoise=addr(5), r=addr(6),
                l0=addr(7), eta0=addr(8), o=addr(9), lT=addr(10), etaT=addr(11), workspace=None,
                workspaceBytes=0, stream=None)
    args.update(over)
    return scan_amd.klaFwd(d, **args)


def step_call(d, **over):
    args = dict(q=addr(1), k=addr(2), v=addr(3), a=addr(4), qnoise=addr(5), r=addr(6),
                l=addr(7), eta=addr(8), o=addr(9), stream=None)
    args.update(over)
    return scan_amd.klaStep(d, **args)


def test_null_dims():
    lib = scan_amd.load()
    assert lib.klaFwd(None, *([None] * 12), 0, None) == NULL
    assert lib.klaStep(None, *([None] * 10)) == NULL
    assert lib.klaIsSupported(None) == 0


@pytest.mark.parametrize("field", ["B", "H", "T", "dk", "dv"])
def test_negative_dims(field):
    d = KlaDims(1, 2, 16, 16, 16, F32, DIAG)
    setattr(d, field, -1)
    assert fwd_call(d) == SHAPE


def test_bad_enums():
    assert fwd_call(KlaDims(1, 2, 16, 16, 16, 7, DIAG)) == UNSUP
    assert fwd_call(KlaDims(1, 2, 16, 16, 16, F32, 5)) == UNSUP
    assert step_call(KlaDims(1, 2, 1, 16, 16, F32, 5)) == UNSUP


@pytest.mark.parametrize("name", ["q", "k", "v", "a", "qnoise", "r", "o"])
def test_required_pointers(name):
    d = KlaDims(1, 2, 16, 16, 16, F32, DIAG)
    assert fwd_call(d, **{name: None}) == NULL


@pytest.mark.parametrize("name", ["q", "k", "v", "a", "qnoise", "r", "l", "eta", "o"])
def test_step_required_pointers(name):
    d = KlaDims(4, 2, 1, 64, 64, BF16, ISO)
    assert step_call(d, **{name: None}) == NULL


@pytest.mark.parametrize("name", ["q", "k", "v", "a", "o", "eta0", "etaT", "l0", "lT", "r"])
def test_misaligned(name):
    d = KlaDims(1, 2, 16, 16, 16, F32, DIAG)
    assert fwd_call(d, **{name: addr(20) + 4}) == ALIGN


def test_empty_batch_is_a_no_op():
    # B*H == 0: nothing to do, nothing is dereferenced, no HIP call
    assert fwd_call(KlaDims(0, 4, 16, 16, 16, F32, DIAG)) == OK
    assert step_call(KlaDims(3, 0, 1, 16, 16, F32, DIAG)) == OK


def test_output_aliasing_rejected():
    d = KlaDims(1, 2, 16, 16, 16, F32, DIAG)
    assert fwd_call(d, o=addr(1)) == ALIAS            # o over q
    assert fwd_call(d, lT=addr(7)) == ALIAS           # lT over l0
    assert fwd_call(d, etaT=addr(8) + 16) == ALIAS    # etaT inside eta0
    assert fwd_call(d, lT=addr(9)) == ALIAS           # lT over o
    ds = KlaDims(1, 2, 1, 16, 16, F32, DIAG)
    assert step_call(ds, o=addr(8)) == ALIAS          # o over eta
    assert step_call(ds, l=addr(8)) == ALIAS          # l over eta


def test_header_documents_every_entry_point():
    text = open(HEADER).read()
    for n in declared_functions():
        # every declaration is preceded by a comment block
        idx = text.index(n + "(")
        assert "*/" in text[max(0, idx - 600):idx], n


def test_kernel_name_reports_the_dispatch():
    lm = KlaDims(8, 16, 2048, 128, 128, BF16, DIAG)
    assert scan_amd.klaFwdKernelName(lm) == "kla_fwd_diag_pipe_kernel (value tiles)"
    # dv = 128 always runs as two 64-column tiles; dk = dv = 64 as one
    assert scan_amd.klaFwdKernelName(KlaDims(64, 16, 2048, 128, 128, BF16, DIAG)) == \
        "kla_fwd_diag_pipe_kernel (value tiles)"
    assert scan_amd.klaFwdKernelName(KlaDims(8, 16, 2048, 64, 64, BF16, DIAG)) == "kla_fwd_diag_pipe_kernel"
    # few long sequences: the sequence split on whole 128-column rows
    assert scan_amd.klaFwdKernelName(KlaDims(1, 16, 32768, 128, 128, BF16, DIAG)) == "kla_fwd_diag_pipe_kernel"
    assert scan_amd.klaFwdKernelName(KlaDims(8, 16, 2048, 64, 64, F32, DIAG)) == "kla_fwd_diag_pipe_kernel"
    assert scan_amd.klaFwdKernelName(KlaDims(2, 3, 100, 32, 32, F32, DIAG)) == "kla_fwd_diag_kernel"
    assert scan_amd.klaFwdKernelName(KlaDims(2, 3, 100, 64, 64, F32, ISO)) == \
        "kla_fwd_iso_pipe_kernel (value tiles)"
    assert scan_amd.klaFwdKernelName(KlaDims(64, 8, 100, 64, 64, F32, ISO)) == "kla_fwd_iso_pipe_kernel"
    assert scan_amd.klaFwdKernelName(KlaDims(4, 32, 8192, 128, 128, BF16, ISO)) == \
        "kla_fwd_iso_pipe_kernel (value tiles)"
    assert scan_amd.klaFwdKernelName(KlaDims(2, 3, 100, 32, 32, F32, ISO)).startswith(
        "kla_fwd_iso_kernel")
    assert scan_amd.klaFwdKernelName(KlaDims(2, 3, 0, 64, 64, BF16, DIAG)) == "kla_fwd_empty_kernel"
    # short sequences (prefill into cached states, multi-token decode)
    for T, cov in ((1, DIAG), (32, DIAG), (7, ISO), (32, ISO)):
        assert scan_amd.klaFwdKernelName(KlaDims(256, 32, T, 64, 64, BF16, cov)) == "kla_fwd_short_kernel"
    assert scan_amd.klaFwdKernelName(KlaDims(256, 32, 33, 64, 64, BF16, DIAG)) != "kla_fwd_short_kernel"
    assert scan_amd.klaFwdKernelName(KlaDims(1, 1, 8, 48, 48, BF16, DIAG)) == ""
    assert scan_amd.klaFwdKernelName(KlaDims(-1, 1, 8, 64, 64, BF16, DIAG)) == ""
    lib = scan_amd.load()
    assert lib.klaFwdKernelName(None) == b""


def test_short_path_switch(monkeypatch):
    short = KlaDims(256, 32, 8, 64, 64, BF16, ISO)
    assert scan_amd.klaFwdKernelName(short) == "kla_fwd_short_kernel"
    assert scan_amd.klaFwdWorkspaceBytes(short) == 0
    monkeypatch.setenv("KLA_FWD_SHORT", "0")
    assert scan_amd.klaFwdKernelName(short) == "kla_fwd_iso_pipe_kernel"


def test_split_workspace_contract(monkeypatch):
    long = KlaDims(1, 16, 32768, 128, 128, BF16, DIAG)
    ws = scan_amd.klaFwdWorkspaceBytes(long)
    assert ws > 0
    assert scan_amd.klaFwdWorkspaceBytes(KlaDims(8, 16, 2048, 128, 128, BF16, DIAG)) == 0
    # a split pays only when each workgroup saves enough tokens
    assert scan_amd.klaFwdWorkspaceBytes(KlaDims(2, 16, 2048, 64, 64, BF16, DIAG)) == 0
    assert scan_amd.klaFwdWorkspaceBytes(KlaDims(2, 16, 8192, 64, 64, BF16, DIAG)) > 0
    assert scan_amd.klaFwdWorkspaceBytes(KlaDims(1, 16, 32768, 32, 32, F32, DIAG)) == 0
    # a split forward without (or with too small) a workspace is rejected
    assert fwd_call(long) == WS
    assert fwd_call(long, workspace=addr(12), workspaceBytes=ws - 1) == WS
    assert fwd_call(long, workspace=addr(12) + 8, workspaceBytes=ws) == ALIGN
    # the workspace may not overlap an input or output
    assert fwd_call(long, workspace=addr(3) - 4096, workspaceBytes=ws) == ALIAS
    assert fwd_call(long, workspace=addr(9) + 4096, workspaceBytes=ws) == ALIAS
    monkeypatch.setenv("KLA_FWD_NSEG", "1")
    assert scan_amd.klaFwdWorkspaceBytes(long) == 0


# ------------------------------------------------------------------ klaFwdResidual

def res_call(d, **over):
    args = dict(q=addr(1), k=addr(2), v=addr(3), a=addr(4), qnoise=addr(5), r=addr(6),
                l0=addr(7), m0=addr(8), o=addr(9), lT=addr(10), mT=addr(11), stream=None)
    args.update(over)
    return scan_amd.klaFwdResidual(d, **args)


def test_residual_argument_errors():
    lib = scan_amd.load()
    assert lib.klaFwdResidual(None, *([None] * 11), None) == NULL
    d = KlaDims(1, 2, 16, 16, 16, F32, DIAG)
    for field in ("B", "H", "T", "dk", "dv"):
        bad = KlaDims(1, 2, 16, 16, 16, F32, DIAG)
        setattr(bad, field, -1)
        assert res_call(bad) == SHAPE, field
    for dims in [(1, 1, 8, 48, 48), (1, 1, 8, 64, 32), (1, 1, 8, 256, 256)]:
        assert res_call(KlaDims(*dims, F32, ISO)) == UNSUP, dims
    assert res_call(KlaDims(1, 2, 16, 16, 16, 7, DIAG)) == UNSUP
    for name in ("q", "k", "v", "a", "qnoise", "r", "o"):
        assert res_call(d, **{name: None}) == NULL, name
    for name in ("q", "k", "v", "a", "o", "m0", "mT", "l0", "lT", "r"):
        assert res_call(d, **{name: addr(20) + 4}) == ALIGN, name
    assert res_call(d, o=addr(2)) == ALIAS           # o over k
    assert res_call(d, lT=addr(7)) == ALIAS          # lT over l0
    assert res_call(d, mT=addr(8) + 16) == ALIAS     # mT inside m0
    assert res_call(KlaDims(0, 4, 16, 16, 16, F32, DIAG)) == OK


# ------------------------------------------------------------------ klaBwd

def bwd_call(d, **over):
    names = ("q", "k", "v", "a", "qnoise", "r", "l0", "eta0", "dO", "dlT", "detaT",
             "dq", "dk", "dv", "da", "dqnoise", "dr", "dl0", "deta0")
    args = {n: addr(i + 1) for i, n in enumerate(names)}
    args.update(workspace=addr(40), workspaceBytes=scan_amd.klaBwdWorkspaceBytes(d), stream=None)
    args.update(over)
    return scan_amd.klaBwd(d, **args)


def test_backward_argument_errors():
    lib = scan_amd.load()
    assert lib.klaBwd(None, *([None] * 19), None, 0, None) == NULL
    d = KlaDims(2, 3, 16, 32, 32, BF16, DIAG)
    # per (b,h): l_t and q dq fp64 [T][dk], qn partial fp32 [dk]
    per = 16 * 32 * 4 + 32
    assert scan_amd.klaBwdWorkspaceBytes(d) == 2 * 3 * 4 * ((per + 63) // 64 * 64)
    # the chunked path (diagonal bf16, dk 64 / 128): the token-serial block
    # (handed-back sequences), the row tiles' flags, then q.dq [T][dk], the
    # partials of dv [NT][T][dk] and dr [NT][T4], the chunk-start precisions
    # [nch][dk] and <detaT, eta_T> [dk]
    for T, dk in [(40, 64), (77, 128), (1, 128)]:
        nt, nch, t4 = dk // 64, (T + 15) // 16, (T + 3) // 4 * 4
        q0 = (4 * T * dk + dk + 4 + 63) // 64 * 64
        end = q0 + T * dk + nt * T * dk + nt * t4 + nch * dk + dk
        assert scan_amd.klaBwdWorkspaceBytes(KlaDims(2, 3, T, dk, dk, BF16, DIAG)) == \
            2 * 3 * 4 * ((end + 63) // 64 * 64), (T, dk)
    for field in ("B", "H", "T", "dk", "dv"):
        bad = KlaDims(2, 3, 16, 32, 32, BF16, DIAG)
        setattr(bad, field, -1)
        assert bwd_call(bad) == SHAPE, field
    for dims in [(1, 1, 8, 48, 48), (1, 1, 8, 64, 32), (1, 1, 8, 256, 256)]:
        assert bwd_call(KlaDims(*dims, F32, DIAG)) == UNSUP, dims
        assert scan_amd.klaBwdWorkspaceBytes(KlaDims(*dims, F32, DIAG)) == 0
    assert bwd_call(KlaDims(1, 2, 16, 16, 16, 7, DIAG)) == UNSUP
    for name in ("q", "k", "v", "a", "qnoise", "r", "dO", "dq", "dk", "dv", "da", "dqnoise", "dr"):
        assert bwd_call(d, **{name: None}) == NULL, name
    for name in ("q", "dO", "dq", "dqnoise", "dl0", "deta0", "detaT", "workspace"):
        assert bwd_call(d, **{name: addr(50) + 4}) == ALIGN, name
    assert bwd_call(d, workspace=None) == WS
    assert bwd_call(d, workspaceBytes=16) == WS
    assert bwd_call(d, dq=addr(2)) == ALIAS             # dq over k
    assert bwd_call(d, dk=addr(12) + 16) == ALIAS       # dk inside dq
    assert bwd_call(d, workspace=addr(14)) == ALIAS     # workspace over da
    assert bwd_call(KlaDims(0, 4, 16, 16, 16, F32, ISO)) == OK


def block_call(dims, blk=None, **over):
    args = dict(xq=addr(1), xk=addr(2), xv=addr(3), za=addr(4), zqn=addr(5), zr=addr(6), l0=None,
                eta0=None, o=addr(7), lT=addr(8), etaT=addr(9), workspace=None, workspaceBytes=0,
                stream=None)
    args.update(over)
    if blk is None:
        blk = scan_amd.KlaBlock(4, addr(10), addr(11), addr(12), None, None, None, None, None, None,
                                1e-3)
    return scan_amd.klaFwdBlock(dims, blk, **args)


def test_block_argument_errors():
    d = KlaDims(2, 3, 40, 128, 128, BF16, DIAG)
    assert scan_amd.klaFwdBlock(d, None, *([None] * 11), None, 0, None) == NULL
    for w in (0, 5, -1):
        blk = scan_amd.KlaBlock(w, addr(10), addr(11), addr(12), None, None, None, None, None, None, 1e-3)
        assert block_call(d, blk) == SHAPE, w
    blk = scan_amd.KlaBlock(4, addr(10), addr(11), addr(12), None, None, None, None, None, None, -1.0)
    assert block_call(d, blk) == SHAPE
    blk = scan_amd.KlaBlock(4, addr(10), addr(11), addr(12), None, None, None, None, None, None,
                            float("nan"))
    assert block_call(d, blk) == SHAPE
    # only the diagonal wave-specialised shapes
    assert block_call(KlaDims(2, 3, 40, 128, 128, BF16, ISO)) == UNSUP
    assert block_call(KlaDims(2, 3, 40, 32, 32, F32, DIAG)) == UNSUP
    assert block_call(KlaDims(2, 3, 40, 128, 128, F32, DIAG)) == UNSUP
    assert block_call(KlaDims(2, 3, 40, 128, 64, BF16, DIAG)) == UNSUP
    for name in ("xq", "xk", "xv", "za", "zqn", "zr", "o"):
        assert block_call(d, **{name: None}) == NULL, name
    blk = scan_amd.KlaBlock(4, None, addr(11), addr(12), None, None, None, None, None, None, 1e-3)
    assert block_call(d, blk) == NULL
    assert block_call(d, xq=addr(1) + 8) == ALIGN
    blk = scan_amd.KlaBlock(4, addr(10) + 2, addr(11), addr(12), None, None, None, None, None, None, 1e-3)
    assert block_call(d, blk) == ALIGN
    blk = scan_amd.KlaBlock(4, addr(10) + 4, addr(11), addr(12), None, None, None, addr(13) + 4, None,
                            None, 1e-3)
    assert block_call(d, blk) == ALIGN                   # states must be 16-byte aligned
    assert block_call(d, o=addr(1)) == ALIAS             # o over xq
    assert block_call(d, lT=addr(5)) == ALIAS            # lT over zqn
    blk = scan_amd.KlaBlock(4, addr(7), addr(11), addr(12), None, None, None, None, None, None, 1e-3)
    assert block_call(d, blk) == ALIAS                   # taps under o
    assert block_call(KlaDims(0, 3, 40, 128, 128, BF16, DIAG)) == OK
    # a split shape needs the forward's workspace
    long = KlaDims(1, 16, 32768, 128, 128, BF16, DIAG)
    need = scan_amd.klaFwdWorkspaceBytes(long)
    assert need > 0
    assert block_call(long) == WS
    assert block_call(long, workspace=addr(20), workspaceBytes=need - 1) == WS
    assert block_call(long, workspace=addr(20) + 8, workspaceBytes=need) == ALIGN
    assert block_call(long, workspace=addr(1), workspaceBytes=need) == ALIAS
