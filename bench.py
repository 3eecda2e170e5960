#!/usr/bin/env python3
"""KLA forward benchmark on one MI355X.

One step = one klaFwd over the whole batch of the workload (all heads, all
tokens), inputs resident in HBM.  Default workload: the LM layer at
1.3B-like width, B=8 H=16 T=2048 dk=dv=128, bf16 q/k/v/o, fp32 state.

Prints ONE JSON line with tokens/s, the roofline of the forward kernel
(algorithmic HBM bytes / measured kernel time against 8 TB/s), and the fp64
oracle timed on the host cores over a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload lm_diag] [--no-cpu]
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

# Kernel sources whose hash keys the stored HBM-traffic counters: the counters
# are reported only while the kernel they were taken on is unchanged.
KERNEL_SOURCES = {
    "diag": ["scan_amd/csrc/kla_fwd_diag_pipe.hip", "scan_amd/csrc/kla_fwd_diag.hip",
             "scan_amd/csrc/kla_fwd_seg.hip", "scan_amd/csrc/kla_common.h",
             "scan_amd/csrc/kla_internal.h"],
    "iso": ["scan_amd/csrc/kla_fwd_iso_pipe.hip", "scan_amd/csrc/kla_fwd_iso.hip",
            "scan_amd/csrc/kla_common.h", "scan_amd/csrc/kla_internal.h"],
    "short": ["scan_amd/csrc/kla_fwd_short.hip", "scan_amd/csrc/kla_short.h",
              "scan_amd/csrc/kla_common.h", "scan_amd/csrc/kla_internal.h"],
    "residual": ["scan_amd/csrc/kla_fwd_residual.hip", "scan_amd/csrc/kla_residual.h",
                 "scan_amd/csrc/kla_common.h", "scan_amd/csrc/kla_internal.h"],
}


def kernel_hash(cov: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[cov]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, cov: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary of this
    workload (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size),
    or None when there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        m = re.search(r"^traffic_json: (\{.*\})$", f.read(), re.M)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_hash") != kernel_hash(cov):
        return None
    return rec


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


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="lm_diag")
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
    if args.workload == gen.PREFILL.name:
        print(json.dumps(run_prefill(args, torch, np, scan_amd, gen)), flush=True)
        return 0
    # the residual-write forward (klaFwdResidual) at the LM-layer shape, or
    # the KLA forward (klaFwd) on one of the named workloads
    residual = args.workload == gen.RESIDUAL.name
    w = gen.RESIDUAL if residual else gen.WORKLOADS[args.workload]
    print(f"bench: workload {w}", file=sys.stderr, flush=True)
    host = gen.make_inputs(w, seed=0)
    names = ("q", "k", "v", "a", "qn", "r")
    # two resident copies, alternated, so consecutive steps do not reuse the
    # 256 MB last-level cache
    sets = [[host[n].to("cuda") for n in names]]
    sets.append([t.clone() for t in sets[0]])
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    outs = []
    for _ in range(2):
        o = torch.empty(B, H, T, dv, dtype=sets[0][2].dtype, device="cuda")
        lT = torch.empty((B, H, dk) if w.cov == "diag" else (B, H), device="cuda")
        etaT = torch.empty(B, H, dk, dv, device="cuda")
        outs.append((o, lT, etaT))

    def step(i):
        s = sets[i % 2]
        o, lT, etaT = outs[i % 2]
        if residual:
            scan_amd.fwd_residual(*s, cov=w.cov, o=o, lT=lT, mT=etaT)
        else:
            scan_amd.fwd(*s, cov=w.cov, o=o, lT=lT, etaT=etaT)

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
    nbytes = alg_bytes(w)
    achieved = nbytes / (kern_ms / 1e3) / 1e9
    print(f"bench: {ms_per_step:.4f} ms/step (kernel {kern_ms:.4f} ms), {achieved:.1f} GB/s "
          f"algorithmic, wall {wall:.3f}s", file=sys.stderr, flush=True)

    calibration_copy(args, torch)

    cpu = None
    if not args.no_cpu:
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

    traffic = stored_traffic(w.name, "residual" if residual else w.cov)
    kernel_name = ("kla_fwd_residual_kernel" if residual else
                   scan_amd.fwd_kernel_name(w.B, w.H, w.T, w.dk, w.dv, w.cov, w.dtype))
    line = {
        "metric": ("KLA residual-write layer fwd tokens/s at B·T, H×d; % of HBM roofline" if residual
                   else "KLA layer fwd tokens/s at B·T, H×d; % of HBM/MFMA roofline"),
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
                     "kernel_ms": kern_ms},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
