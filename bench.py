#!/usr/bin/env python3
"""KLA forward benchmark on one MI355X.

One step = one klaFwd over the whole batch of the workload (all heads, all
tokens), inputs resident in HBM.  Default workload: the largest single-GPU
configuration, long context B=1 H=16 T=32768 dk=dv=128, bf16 q/k/v/o, fp32
state, slow decay.

Prints ONE JSON line with tokens/s, the roofline of the forward (algorithmic
HBM bytes / measured GPU time against 8 TB/s, and against a device copy of
the same byte count measured in the same process), the algorithmic matrix
flops against the MFMA peak of the input dtype, and the fp64 oracle timed on
the host cores over a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload long_diag] [--no-cpu]
  (workloads: the names in scan_amd.inputs, iso_decode, iso_prefill16,
   residual_lm_diag, block_lm_diag, block_long_diag, bwd_lm_diag, bwd_iso)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# dense matrix-core peaks of MI355X (TFLOP/s), by the dtype of q, k, v
MFMA_PEAK_TFS = {"bf16": 2500.0, "f32": 157.3}
# the last-level cache (MALL) the timed steps must not reuse between steps
MALL_BYTES = 256 << 20

# Kernel sources whose hash keys the stored HBM-traffic counters: the counters
# are reported only while the kernel they were taken on is unchanged.
# Every family also hashes the dispatch (kla_api.cpp: kernel choice, tiles,
# segments), the shared headers and the build flags.
_COMMON_SOURCES = ["scan_amd/csrc/kla_api.cpp", "scan_amd/csrc/kla_common.h",
                   "scan_amd/csrc/kla_internal.h", "scan_amd/build.py"]
KERNEL_SOURCES = {
    "diag": ["scan_amd/csrc/kla_fwd_diag_pipe.hip", "scan_amd/csrc/kla_fwd_diag.hip",
             "scan_amd/csrc/kla_fwd_seg.hip"] + _COMMON_SOURCES,
    "iso": ["scan_amd/csrc/kla_fwd_iso_pipe.hip", "scan_amd/csrc/kla_fwd_iso.hip"] + _COMMON_SOURCES,
    "short": ["scan_amd/csrc/kla_fwd_short.hip", "scan_amd/csrc/kla_short.h"] + _COMMON_SOURCES,
    "residual": ["scan_amd/csrc/kla_fwd_residual.hip", "scan_amd/csrc/kla_fwd_residual_chunk.hip",
                 "scan_amd/csrc/kla_residual.h"] + _COMMON_SOURCES,
    "step": ["scan_amd/csrc/kla_step.hip"] + _COMMON_SOURCES,
    "bwd": ["scan_amd/csrc/kla_bwd.hip", "scan_amd/csrc/kla_bwd_chunk.hip", "scan_amd/csrc/kla_bwd.h"] + _COMMON_SOURCES,
}


def kernel_hash(cov: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[cov]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _stored_record(kind: str, workload: str, cov: str):
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        m = re.search(r"^%s_json: (\{.*\})$" % kind, f.read(), re.M)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_hash") != kernel_hash(cov):
        return None
    return rec


def stored_traffic(workload: str, cov: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary of this
    workload (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size),
    or None when there is none or the kernel sources changed since."""
    return _stored_record("traffic", workload, cov)


def stored_counters(workload: str, cov: str):
    """Matrix-core and VALU counters of the forward from the committed
    rocprofv3 --pmc summary of this workload (MFMA busy cycles over the
    shader busy cycles of the CUs), or None when there is none or the kernel
    sources changed since."""
    return _stored_record("counters", workload, cov)


def alg_flops(w) -> float:
    """Algorithmic matrix flops of one forward: 5 dk dv per token-head (decay
    and rank-1 write 3 dk dv, readout 2 dk dv), independent of chunking."""
    return float(w.B * w.H * w.T * 5 * w.dk * w.dv)


def measure_copy(torch, nbytes: float, reps: int = 10, settle_s: float = 0.0) -> float:
    """GB/s of a plain device-to-device copy that moves nbytes in total (half
    read, half written), timed with HIP events on the current stream.

    With settle_s > 0 the copy first runs for about that many seconds of GPU
    time, untimed: an idle GPU starts below its sustained clock and takes a
    few tens of milliseconds of load to reach it (measured: the long-context
    forward ran 0.45 ms per step after 5 warm-up steps, 0.37 ms after 100).
    Called before a workload's warm-up, this brings the GPU to the clock the
    timed steps then run at, and the copy rate is taken at that same clock."""
    half = int(nbytes // 2) // 16 * 16
    src = torch.empty(half, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    if settle_s > 0:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < settle_s:
            for _ in range(8):
                dst.copy_(src)
            torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2 * half / (ms / 1e3) / 1e9


def alg_bytes(w) -> float:
    """Algorithmic HBM bytes of one forward: each input read once, each output
    written once (l0 = 1, eta0 = 0 are not read), no intermediate state."""
    es = 2 if w.dtype == "bf16" else 4
    ntok = w.B * w.H * w.T
    if w.cov == "diag":
        per_tok = (2 * w.dk + w.dv) * es + 4 * w.dk + 4 + w.dv * es
        per_seq = 4 * w.dk + 4 * w.dk * w.dv
    else:
        per_tok = (2 * w.dk + w.dv) * es + 12 + w.dv * es
        per_seq = 4 + 4 * w.dk * w.dv
    return float(ntok * per_tok + w.B * w.H * per_seq)


def block_alg_bytes(w, width: int) -> float:
    """Algorithmic HBM bytes of one forward with the fused block prologue: the
    projections xq, xk, xv and za read once (storage dtype), zr read once, o
    written once, lT and etaT written once per (b,h), and per head the
    convolution taps and biases of q, k, v and zqn read once."""
    es = 2 if w.dtype == "bf16" else 4
    per_tok = (3 * w.dk + w.dv) * es + 4 + w.dv * es
    per_seq = 4 * w.dk + 4 * w.dk * w.dv
    per_head = (2 * w.dk + w.dv) * (width + 1) * 4 + 4 * w.dk
    return float(w.B * w.H * w.T * per_tok + w.B * w.H * per_seq + w.H * per_head)


def decode_alg_bytes(w) -> float:
    """Algorithmic HBM bytes of one decode step (one token for every (b,h)):
    the fp32 state (l, eta) read and written in place, the token's inputs read
    and its output written."""
    es = 2 if w.dtype == "bf16" else 4
    nl = 1 if w.cov == "iso" else w.dk
    state = 4 * nl + 4 * w.dk * w.dv
    tok = (2 * w.dk + w.dv) * es + 4 * (1 if w.cov == "iso" else w.dk) \
        + 4 * (1 if w.cov == "iso" else 0) + 4 + w.dv * es
    return float(w.B * w.H * (2 * state + tok))


def run_decode(args, torch, np, scan_amd, gen) -> dict:
    """One step = one klaStep for every (b,h) of the decode batch, from states
    produced by a prefix forward (readings: 128-token prefix, seed 1; decode
    tokens seed 2)."""
    w = gen.DECODE
    pre = gen.make_inputs(w, seed=1, device="cuda")
    names = ("q", "k", "v", "a", "qn", "r")
    _, l, eta = scan_amd.fwd(*(pre[n] for n in names), cov=w.cov)
    n = gen.DECODE_STEPS
    host = gen.make_inputs(w, seed=2, T=n)
    toks = []
    for t in range(n):
        toks.append([host[x][:, :, t].contiguous().to("cuda") for x in names])
    o = torch.empty(w.B, w.H, w.dv, dtype=toks[0][2].dtype, device="cuda")
    measure_copy(torch, decode_alg_bytes(w), settle_s=args.settle_s)  # sustained clock
    for i in range(args.warmup):
        scan_amd.step(*toks[i % n], l, eta, cov=w.cov, o=o)
    torch.cuda.synchronize()
    # events around the whole timed region only (see the forward timing in main)
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        scan_amd.step(*toks[i % n], l, eta, cov=w.cov, o=o)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    kern_ms = ms_per_step
    nbytes = decode_alg_bytes(w)
    achieved = nbytes / (kern_ms / 1e3) / 1e9
    print(f"bench: decode {ms_per_step:.4f} ms/step (kernel {kern_ms:.4f} ms), {achieved:.1f} GB/s",
          file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu:
        import oracle
        threads = oracle.default_threads()
        lh = l.cpu().numpy()
        eh = eta.cpu().numpy()
        hx = [[x.cpu() for x in tk] for tk in toks]
        reps, t_cpu = 0, 0.0
        while reps == 0 or (t_cpu < 0.5 * args.cpu_seconds and reps < 1000):
            tk = hx[reps % n]
            t0 = time.perf_counter()
            res = oracle.step(*tk, lh, eh, cov=oracle.ISO if w.cov == "iso" else oracle.DIAG,
                              nthreads=threads)
            t_cpu += time.perf_counter() - t0
            lh, eh = res["l"], res["eta"]
            reps += 1
        cpu = {"value": w.B * reps / t_cpu, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{reps} full decode steps (B={w.B}, H={w.H}), fp64, {t_cpu:.1f}s"}
    return {
        "metric": "KLA decode tokens/s (klaStep, constant-memory state)",
        "value": w.B / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "dk": w.dk, "dv": w.dv, "cov": w.cov,
                   "global_batch": w.B, "seq_len": 1, "parallelism": "none"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "kla_step_kernel", "alg_bytes": nbytes, "kernel_ms": kern_ms},
        "cpu_baseline": cpu,
    }


# backward workloads: the forward workload whose shape and value laws they use
BWD_WORKLOADS = {"bwd_lm_diag": "lm_diag", "bwd_iso": "iso"}


def bwd_alg_bytes(w) -> float:
    """Algorithmic HBM bytes of one backward pass (klaBwd) with upstream
    gradients for o, lT and etaT: the forward's inputs and do read once, the
    input gradients written once (per (b,h) dlT, detaT read and dl0, deta0
    written; the diagonal qn per head read and dqn written, the isotropic
    a, qn per token).  Workspace traffic is not counted."""
    es = 2 if w.dtype == "bf16" else 4
    if w.cov == "iso":
        per_tok = 2 * ((2 * w.dk + w.dv) * es + 12) + w.dv * es
        per_seq = 2 * (4 + 4 * w.dk * w.dv)
        return float(w.B * w.H * w.T * per_tok + w.B * w.H * per_seq)
    per_tok = 2 * ((2 * w.dk + w.dv) * es + 4 * w.dk + 4) + w.dv * es
    per_seq = 2 * (4 * w.dk + 4 * w.dk * w.dv)
    return float(w.B * w.H * w.T * per_tok + w.B * w.H * per_seq + w.H * 8 * w.dk)


def run_bwd(args, torch, np, scan_amd, gen) -> dict:
    """One step = one klaBwd over the whole batch of the LM layer (bwd_lm_diag)
    or of the isotropic workload (bwd_iso): gradients of <do, o> + <dlT, lT> +
    <detaT, etaT> for every input, inputs and upstream gradients resident in
    HBM, rotated like the forward's."""
    name = args.workload
    w = gen.WORKLOADS[BWD_WORKLOADS[name]]
    iso = w.cov == "iso"
    print(f"bench: backward of {w}", file=sys.stderr, flush=True)
    host = gen.make_inputs(w, seed=0)
    up = gen.make_upstream(w, seed=1)
    names = ("q", "k", "v", "a", "qn", "r")
    nbytes = bwd_alg_bytes(w)
    ncopies = max(2, -(-3 * MALL_BYTES // int(nbytes)))
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    dims = scan_amd.KlaDims(B, H, T, dk, dv, scan_amd.KLA_BF16 if w.dtype == "bf16" else scan_amd.KLA_F32,
                            scan_amd.KLA_ISO if iso else scan_amd.KLA_DIAG)
    ws_bytes = scan_amd.klaBwdWorkspaceBytes(dims)
    sets = []
    for _ in range(ncopies):
        ins = {n: host[n].to("cuda") for n in names}
        ins.update({n: up[n].to("cuda") for n in ("do", "dlT", "detaT")})
        outs = {"dq": torch.empty_like(ins["q"]), "dk": torch.empty_like(ins["k"]),
                "dv": torch.empty_like(ins["v"]), "da": torch.empty_like(ins["a"]),
                "dqn": torch.empty_like(ins["qn"]), "dr": torch.empty_like(ins["r"]),
                "dl0": torch.empty((B, H) if iso else (B, H, dk), device="cuda"),
                "deta0": torch.empty(B, H, dk, dv, device="cuda")}
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
        sets.append((ins, outs, ws))
    stream = torch.cuda.current_stream()

    def step(i):
        ins, outs, ws = sets[i % ncopies]
        rc = scan_amd.klaBwd(dims, *(ins[n].data_ptr() for n in names), None, None,
                             ins["do"].data_ptr(), ins["dlT"].data_ptr(), ins["detaT"].data_ptr(),
                             *(outs[n].data_ptr() for n in ("dq", "dk", "dv", "da", "dqn", "dr", "dl0", "deta0")),
                             ws.data_ptr(), ws_bytes, stream.cuda_stream)
        if rc != 0:
            raise scan_amd.KlaError(rc, "klaBwd")

    # the copy reference, taken after it has brought the GPU to its sustained clock
    copy_gbs = measure_copy(torch, nbytes, settle_s=args.settle_s)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    achieved = nbytes / (ms_per_step / 1e3) / 1e9
    print(f"bench: backward {ms_per_step:.4f} ms/step, {achieved:.1f} GB/s algorithmic, "
          f"copy {copy_gbs:.1f} GB/s", file=sys.stderr, flush=True)
    calibration_copy(args, torch)
    cpu = None
    if not args.no_cpu:
        import oracle
        threads = oracle.default_threads()
        cov = oracle.ISO if iso else oracle.DIAG
        one = {n: host[n][:1, :1] for n in names}
        if not iso:
            one["qn"] = host["qn"][:1]
        uo = {n: up[n][:1, :1] for n in ("do", "dlT", "detaT")}
        t0 = time.perf_counter()
        oracle.bwd(*(one[n] for n in names), do=uo["do"], dlT=uo["dlT"], detaT=uo["detaT"], cov=cov, nthreads=1)
        t_one = time.perf_counter() - t0
        nseq = int(max(threads, min(B * H, args.cpu_seconds * threads / max(t_one, 1e-6))))
        nh = H if nseq >= H else max(1, nseq)
        nb = max(1, min(B, nseq // H)) if nseq >= H else 1
        sub = {n: host[n][:nb, :nh] for n in names}
        if not iso:
            sub["qn"] = host["qn"][:nh]
        us = {n: up[n][:nb, :nh] for n in ("do", "dlT", "detaT")}
        reps, t_cpu = 0, 0.0
        while reps == 0 or (t_cpu < 0.5 * args.cpu_seconds and reps < 100):
            t0 = time.perf_counter()
            oracle.bwd(*(sub[n] for n in names), do=us["do"], dlT=us["dlT"], detaT=us["detaT"], cov=cov,
                       nthreads=threads)
            t_cpu += time.perf_counter() - t0
            reps += 1
        seqs = nb * nh
        cpu = {"value": seqs * T * reps / H / t_cpu, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{seqs} of {B * H} (b,h) sequences at full T={T} ({nb}x{nh}), fp64 reverse-mode "
                         f"adjoint, {reps} pass(es) in {t_cpu:.1f}s"}
    traffic = stored_traffic(name, "bwd")
    return {
        "metric": "KLA layer bwd tokens/s at B·T, H×d; % of HBM roofline",
        "value": B * T / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": name, "B": B, "H": H, "T": T, "dk": dk, "dv": dv, "cov": w.cov,
                   "global_batch": B, "seq_len": T, "parallelism": "none"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic["bytes_per_launch"] if traffic else None,
                     "kernel": "kla_bwd_chunk_fwd + kla_bwd_chunk_rev (chunked sweeps)", "alg_bytes": nbytes,
                     "kernel_ms": ms_per_step,
                     "copy_gbs": copy_gbs, "frac_of_copy": achieved / copy_gbs},
        "cpu_baseline": cpu,
    }


def calibration_copy(args, torch) -> None:
    """With --calib-copy-mb, one device copy of known size after the timed
    steps: the reference that scales the HBM traffic counters."""
    if args.calib_copy_mb > 0:
        nb = args.calib_copy_mb << 20
        src = torch.ones(nb, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"bench: calibration copy of {nb} bytes done", file=sys.stderr, flush=True)
        del src, dst


def prefill_alg_bytes(w) -> float:
    """Algorithmic HBM bytes of one forward over a chunk that continues cached
    states: the token inputs and outputs of alg_bytes, plus the fp32 state
    (l, eta) read once and written once."""
    nl = 1 if w.cov == "iso" else w.dk
    per_seq_in = 4 * nl + 4 * w.dk * w.dv
    return alg_bytes(w) + float(w.B * w.H * per_seq_in)


def run_prefill(args, torch, np, scan_amd, gen) -> dict:
    """One step = one klaFwd over a T-token chunk for every (b,h) of the
    decode batch, from cached states (a DECODE.T-token prefix forward, seed 1)
    into a second state buffer; chunk tokens seed 2, two resident copies
    alternated."""
    w = gen.PREFILL
    names = ("q", "k", "v", "a", "qn", "r")
    pre = gen.make_inputs(gen.DECODE, seed=1, device="cuda")
    _, l0, eta0 = scan_amd.fwd(*(pre[n] for n in names), cov=w.cov)
    del pre
    host = gen.make_inputs(w, seed=2)
    sets = [[host[n].to("cuda") for n in names]]
    sets.append([t.clone() for t in sets[0]])
    o = torch.empty(w.B, w.H, w.T, w.dv, dtype=sets[0][2].dtype, device="cuda")
    lT = torch.empty_like(l0)
    etaT = torch.empty_like(eta0)
    kname = scan_amd.fwd_kernel_name(w.B, w.H, w.T, w.dk, w.dv, cov=w.cov, dtype=w.dtype)

    def step(i):
        scan_amd.fwd(*sets[i % 2], l0, eta0, cov=w.cov, o=o, lT=lT, etaT=etaT)
    measure_copy(torch, prefill_alg_bytes(w), settle_s=args.settle_s)  # sustained clock
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    nbytes = prefill_alg_bytes(w)
    achieved = nbytes / (ms_per_step / 1e3) / 1e9
    traffic = stored_traffic(w.name, "short")
    calibration_copy(args, torch)
    print(f"bench: prefill {ms_per_step:.4f} ms/step ({kname}), {achieved:.1f} GB/s",
          file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu:
        import oracle
        threads = oracle.default_threads()
        hx = [host[n].double().numpy() for n in names]
        lh, eh = l0.double().cpu().numpy(), eta0.double().cpu().numpy()
        reps, t_cpu = 0, 0.0
        while reps == 0 or (t_cpu < 0.5 * args.cpu_seconds and reps < 1000):
            t0 = time.perf_counter()
            oracle.fwd(*hx, lh, eh, cov=oracle.ISO if w.cov == "iso" else oracle.DIAG,
                       nthreads=threads)
            t_cpu += time.perf_counter() - t0
            reps += 1
        cpu = {"value": w.B * w.T * reps / t_cpu, "unit": "tokens/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{reps} full chunk forward(s) (B={w.B}, H={w.H}, T={w.T}) from the "
                         f"cached states, fp64, {t_cpu:.1f}s"}
    return {
        "metric": "KLA chunk tokens/s from cached states (klaFwd, T-token prefill / multi-token decode)",
        "value": w.B * w.T / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv,
                   "cov": w.cov, "global_batch": w.B, "seq_len": w.T, "parallelism": "none"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic["bytes_per_launch"] if traffic else None,
                     "kernel": kname, "alg_bytes": nbytes, "kernel_ms": ms_per_step},
        "cpu_baseline": cpu,
    }


def block_cpu_baseline(args, host, w) -> dict:
    """The block oracle (fp64 prologue, then the sequential recurrence) timed
    on a sample of whole sequences of the workload, about --cpu-seconds."""
    import oracle
    from oracle import block as oblock
    threads = oracle.default_threads()
    names = ("xq", "xk", "xv", "za", "zqn", "zr", "wq", "wk", "wv", "bq", "bk", "bv")
    B, H, T = w.B, w.H, w.T

    def sub(nb, nh):
        out = {}
        for n in names:
            x = host[n]
            if n in ("zqn", "wq", "wk", "wv", "bq", "bk", "bv"):
                out[n] = x[:nh]
            else:
                out[n] = x[:nb, :nh]
        return out

    one = sub(1, 1)
    t0 = time.perf_counter()
    oblock.block_fwd(*(one[n] for n in names), r_eps=host["r_eps"], nthreads=1)
    t_one = time.perf_counter() - t0
    nseq = int(max(threads, min(B * H, args.cpu_seconds * threads / max(t_one, 1e-6))))
    nh = H if nseq >= H else max(1, nseq)
    nb = max(1, min(B, nseq // H)) if nseq >= H else 1
    s = sub(nb, nh)
    reps, t_cpu = 0, 0.0
    while reps == 0 or (t_cpu < 0.5 * args.cpu_seconds and reps < 100):
        t0 = time.perf_counter()
        oblock.block_fwd(*(s[n] for n in names), r_eps=host["r_eps"], nthreads=threads)
        t_cpu += time.perf_counter() - t0
        reps += 1
    seqs = nb * nh
    return {"value": seqs * T * reps / H / t_cpu, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{seqs} of {B * H} (b,h) sequences at full T={T} ({nb}x{nh}), fp64 prologue "
                      f"(numpy) + sequential recurrence, {reps} pass(es) in {t_cpu:.1f}s"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_diag")
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="seconds of untimed device copies before the warm-up, so that the "
                         "timed steps run at the sustained clock (0: none)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after the timed steps, run one device copy of this many MiB "
                         "(a known-size reference for HBM traffic counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the forward shards over (b,h) with no communication, see the design notes.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import scan_amd
    from scan_amd import inputs as gen

    if args.workload == gen.DECODE.name:
        print(json.dumps(run_decode(args, torch, np, scan_amd, gen)), flush=True)
        return 0
    if args.workload in BWD_WORKLOADS:
        print(json.dumps(run_bwd(args, torch, np, scan_amd, gen)), flush=True)
        return 0
    if args.workload == gen.PREFILL.name:
        print(json.dumps(run_prefill(args, torch, np, scan_amd, gen)), flush=True)
        return 0
    # the residual-write forward (klaFwdResidual) at the LM-layer shape, the
    # forward with the fused block prologue (klaFwdBlock) at the LM-layer
    # shape, or the KLA forward (klaFwd) on one of the named workloads
    residual = args.workload == gen.RESIDUAL.name
    blockw = args.workload in (gen.BLOCK.name, gen.BLOCK_LONG.name)
    w = (gen.RESIDUAL if residual else
         {gen.BLOCK.name: gen.BLOCK, gen.BLOCK_LONG.name: gen.BLOCK_LONG}[args.workload] if blockw else
         gen.WORKLOADS[args.workload])
    print(f"bench: workload {w}", file=sys.stderr, flush=True)
    if blockw:
        host = gen.make_block_inputs(w, seed=0)
        names = ("xq", "xk", "xv", "za", "zqn", "zr", "wq", "wk", "wv", "bq", "bk", "bv")
        nbytes = block_alg_bytes(w, host["width"])
    else:
        host = gen.make_inputs(w, seed=0)
        names = ("q", "k", "v", "a", "qn", "r")
        nbytes = alg_bytes(w)
    # resident copies of the inputs and outputs, rotated so that the data one
    # step touches was last touched at least three MALL sizes of traffic ago
    # (consecutive steps never hit the 256 MB last-level cache)
    ncopies = max(2, -(-3 * MALL_BYTES // int(nbytes)))
    sets = [[host[n].to("cuda") for n in names]]
    for _ in range(ncopies - 1):
        sets.append([t.clone() for t in sets[0]])
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    outs = []
    for _ in range(ncopies):
        o = torch.empty(B, H, T, dv, dtype=sets[0][2].dtype, device="cuda")
        lT = torch.empty((B, H, dk) if w.cov == "diag" else (B, H), device="cuda")
        etaT = torch.empty(B, H, dk, dv, device="cuda")
        outs.append((o, lT, etaT))

    def step(i):
        s = sets[i % ncopies]
        o, lT, etaT = outs[i % ncopies]
        if residual:
            scan_amd.fwd_residual(*s, cov=w.cov, o=o, lT=lT, mT=etaT)
        elif blockw:
            scan_amd.fwd_block(*s, r_eps=host["r_eps"], o=o, lT=lT, etaT=etaT)
        else:
            scan_amd.fwd(*s, cov=w.cov, o=o, lT=lT, etaT=etaT)

    # a plain device copy of the same byte count, measured now on this machine,
    # after it has brought the GPU to its sustained clock
    copy_gbs = measure_copy(torch, nbytes, settle_s=args.settle_s)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # HIP events on the stream the kernels run on, around the whole timed
    # region only: events between the steps would add their own command
    # processing to what they measure.  The steps are queued back to back, so
    # the mean step time is the GPU time of one forward (for the single-kernel
    # forwards, that kernel's mean launch duration plus its dispatch).
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    total_ms = ev0.elapsed_time(ev1)
    ms_per_step = total_ms / args.steps
    kern_ms = ms_per_step

    tokens = B * T
    value = tokens / (ms_per_step / 1e3)
    achieved = nbytes / (kern_ms / 1e3) / 1e9
    print(f"bench: {ms_per_step:.4f} ms/step (kernel {kern_ms:.4f} ms), {achieved:.1f} GB/s "
          f"algorithmic, {ncopies} rotating input copies, wall {wall:.3f}s",
          file=sys.stderr, flush=True)
    print(f"bench: device copy of {nbytes / 1e6:.1f} MB: {copy_gbs:.1f} GB/s",
          file=sys.stderr, flush=True)

    calibration_copy(args, torch)

    cpu = None
    if not args.no_cpu and blockw:
        cpu = block_cpu_baseline(args, host, w)
    elif not args.no_cpu:
        import oracle
        threads = oracle.default_threads()
        oracle_fwd = oracle.fwd_residual if residual else oracle.fwd
        # calibrate on one sequence, then size the sample to ~cpu-seconds
        one = {n: host[n][:1, :1] for n in names}
        if w.cov == "diag":
            one["qn"] = host["qn"][:1]
        t0 = time.perf_counter()
        oracle_fwd(*(one[n] for n in names), cov=oracle.DIAG if w.cov == "diag" else oracle.ISO,
                   nthreads=1)
        t_one = time.perf_counter() - t0
        nseq_total = B * H
        nseq = int(max(threads, min(nseq_total, args.cpu_seconds * threads / max(t_one, 1e-6))))
        nseq = max(1, min(nseq_total, nseq // H * H if nseq >= H else nseq))
        nb = max(1, nseq // H) if nseq >= H else 1
        nh = H if nseq >= H else nseq
        sub = {n: host[n][:nb, :nh] for n in names}
        if w.cov == "diag":
            sub["qn"] = host["qn"][:nh]
        cov_code = oracle.DIAG if w.cov == "diag" else oracle.ISO
        # the sample is repeated until about half the target time has passed,
        # so that a sample that covers the whole workload still times stably
        reps, t_cpu = 0, 0.0
        while reps == 0 or (t_cpu < 0.5 * args.cpu_seconds and reps < 100):
            t0 = time.perf_counter()
            oracle_fwd(*(sub[n] for n in names), cov=cov_code, nthreads=threads)
            t_cpu += time.perf_counter() - t0
            reps += 1
        seqs = nb * nh
        cpu_tok_s = seqs * T * reps / H / t_cpu   # token-heads/s over H heads = tokens/s
        cpu = {"value": cpu_tok_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{seqs} of {nseq_total} (b,h) sequences at full T={T} "
                         f"({nb}x{nh}), fp64 sequential recurrence, {reps} pass(es) in {t_cpu:.1f}s"}

    fam = "residual" if residual else w.cov
    traffic = stored_traffic(w.name, fam)
    counters = stored_counters(w.name, fam)
    kernel_name = (("kla_fwd_residual_chunk_kernel (16-token chunks on the matrix cores)"
                    if w.cov == "diag" and w.dk == w.dv and w.dk in (64, 128) else "kla_fwd_residual_kernel")
                   if residual else
                   ("kla_fwd_diag_pipe_kernel (block prologue, value tiles)" +
                    (", sequence split" if w.B * w.H < 192 // 2 else "")) if blockw else
                   scan_amd.fwd_kernel_name(w.B, w.H, w.T, w.dk, w.dv, w.cov, w.dtype))
    flops = alg_flops(w)
    mfma_tfs = flops / (kern_ms / 1e3) / 1e12
    line = {
        "metric": ("KLA residual-write layer fwd tokens/s at B·T, H×d; % of HBM roofline" if residual
                   else "KLA block fwd (fused conv1d+SiLU prologue) tokens/s at B·T, H×d; % of HBM roofline"
                   if blockw else "KLA layer fwd tokens/s at B·T, H×d; % of HBM/MFMA roofline"),
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "T": T, "dk": dk, "dv": dv,
                   "cov": w.cov, "global_batch": B, "seq_len": T, "parallelism": "none"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic["bytes_per_launch"] if traffic else None,
                     "kernel": kernel_name, "alg_bytes": nbytes,
                     "kernel_ms": kern_ms,
                     "copy_gbs": copy_gbs, "frac_of_copy": achieved / copy_gbs},
        # algorithmic matrix flops per forward over the same GPU time, against
        # the dense matrix-core peak of the input dtype; mfma_busy is the
        # counter-measured share of CU busy cycles with the matrix cores busy
        # (stored rocprofv3 record of the same kernels, null once they change)
        "mfma": {"achieved": mfma_tfs, "peak": MFMA_PEAK_TFS[w.dtype], "unit": "TFLOP/s",
                 "frac": mfma_tfs / MFMA_PEAK_TFS[w.dtype], "alg_flops": flops,
                 "mfma_busy": counters["mfma_busy"] if counters else None,
                 "valu_busy": counters["valu_busy"] if counters else None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
