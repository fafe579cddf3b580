#!/usr/bin/env python3
"""Throughput of the chunked gated delta-rule forward on one MI355X.

One step = one gdr_chunk_fwd call over one batch of synthetic input (every stage of the
chunked forward runs inside it).  Default workload: scalar-gated delta rule, B4 H16 T4096
Dk = Dv = 128, bf16 inputs, fp32 state, chunk 64.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-s 1.0] [--workload gdn|gdn2|pdn|long|plain|kda|decode]
                    [--neumann N [--residual S]] [--impl auto|generic|mfma] [--no-cpu-baseline]
    python bench.py --bwd [--workload gdn|gdn2|plain|kda|pdn]   # gdr_chunk_bwd instead

With --neumann N (and --residual S) the line also carries `exact_vs_approx`: the rel-L2 between
the exact-T output and the band-limited (residual-corrected) one, from the GPU (every stream, and
stream (0,0)) and from the fp64 oracle (stream (0,0), every token).

Counter helpers (used to produce the committed counter summaries under profiles/):
    python bench.py --copy-probe-mb 256          # calibration copy of known size
    python bench.py --workload gdn --copy-probe-mb 256 --traffic-summary F.csv W.csv CF.csv CW.csv
    python bench.py --workload gdn --mfma-summary PMC.csv   # matrix-core counters of the kernel
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tokens/s chunked gated-delta fwd (B4 H16 T4096 d128 bf16); % MFMA/HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
ENGINE_CLOCK_HZ = 2.4e9         # MI355X peak engine clock (256 CUs x 4 SIMDs)
FP32_VALU_PEAK_TFLOPS = 157.3   # MI355X fp32 vector

KERNEL_SOURCES = {
    "mfma": ["chunked_gated_delta_gdr_amd/csrc/chunk_mfma.hip", "chunked_gated_delta_gdr_amd/csrc/kda_prep.hip"],
    "generic": ["chunked_gated_delta_gdr_amd/csrc/chunk_generic.hip"],
    "step": ["chunked_gated_delta_gdr_amd/csrc/recurrent_step.hip"],
}


def alg_bytes(s) -> int:
    """Bytes the method must move per call: inputs read once, output and final state
    (and preconditioner accumulator) written once; intermediates never reach HBM."""
    esz = 2 if s.dtype == "bf16" else 4
    per_tok = (2 * s.Dk + 2 * s.Dv) * esz
    per_tok += 4 if s.gain == "scalar" else (s.Dk + s.Dv) * esz
    per_tok += {"scalar": 4, "channel": 4 * s.Dk}.get(s.decay, 0)
    per_tok += s.Dk * esz if s.wkey == "explicit" else 0
    per_head = s.Dv * s.Dk * 4 + (s.Dk * 4 if s.wkey == "precond" else 0)
    return s.B * s.T * s.H * per_tok + s.B * s.H * per_head


def alg_flops(s, band=None, residual=0) -> float:
    """Algorithmic FLOPs per call (triangular products counted triangular):
    per token-head MACs = 3 Dk Dv (W S^T, Q S^T, state update) + (C-1)/2 Dk (A)
    + (C+1)/2 (2 Dk + 2 Dv) (W, U, Q R^T, P D) + C^2/6 (forward substitution), the last
    term N (N + 1) / 2 for a band N; a residual correction of S steps adds S + 2 triangular
    C x C x C products per chunk ((A T0, S times E Z, T0 Z): (S + 2) C^2 / 6 per token)."""
    C, Dk, Dv = s.chunk, s.Dk, s.Dv
    tri = C * C / 6.0 if band is None or band >= C - 1 else (band * (band + 1) / 2.0)
    if band is not None and residual > 0:
        tri += (residual + 2) * C * C / 6.0
    macs = 3 * Dk * Dv + (C - 1) / 2 * Dk + (C + 1) / 2 * (2 * Dk + 2 * Dv) + tri
    return 2.0 * macs * s.B * s.T * s.H


def source_sha(impl: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[impl] + ["chunked_gated_delta_gdr_amd/csrc/common.h"]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def mfma_counter_file(workload: str, impl: str, tag: str = "") -> str:
    return f"chunk_fwd_{impl}_{workload}{tag}_mfma_counters.json"


def mfma_counters_from_profile(workload: str, impl: str, tag: str = ""):
    """The committed matrix-core counter summary of the kernel, if it was taken on the current
    source; else None."""
    p = os.path.join(ROOT, "profiles", mfma_counter_file(workload, impl, tag))
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    return rec if rec.get("source_sha") == source_sha(impl) else None


def mfma_summary(args):
    """Writes profiles/chunk_fwd_<impl>_<workload>_mfma_counters.json from a rocprofv3 --pmc CSV
    holding SQ_INSTS_VALU_MFMA_MOPS_BF16 (bf16 matrix operations in units of 512 FLOPs),
    SQ_VALU_MFMA_BUSY_CYCLES (matrix-core busy cycles, summed over SIMDs), SQ_BUSY_CYCLES,
    GRBM_GUI_ACTIVE (GPU active cycles) and SQ_LDS_BANK_CONFLICT."""
    names = ["SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_LDS_BANK_CONFLICT",
             "SQ_BUSY_CYCLES", "SQ_INSTS_LDS", "SQ_WAVES"]
    med = {}
    for n in names:
        try:
            med[n] = _counter_per_call(args.mfma_summary, n, args.impl_name)[0]
        except SystemExit:
            pass
    s = __import__("gdr_synth").spec(args.workload)
    rec = {
        "kernel": f"gdr_chunk_fwd/{args.impl_name}", "workload": args.workload,
        "source_sha": source_sha(args.impl_name),
        "counters_median_per_dispatch": med,
        "mfma_bf16_flop_per_dispatch": med.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512.0,
        "alg_flop_per_dispatch": alg_flops(s),
        "cu": 256, "simd_per_cu": 4,
    }
    if "SQ_VALU_MFMA_BUSY_CYCLES" in med:
        # the busy count is summed over every SIMD (it is the same on every dispatch: a count of
        # issued matrix-core cycles, not a sample); GRBM_GUI_ACTIVE sums the XCDs' clocks over the
        # counter window, which is wider than the kernel, so the bench divides the per-SIMD
        # figure by its own launch time at the peak engine clock instead
        rec["mfma_busy_cycles_per_simd"] = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (256 * 4)
    out = os.path.join(ROOT, "profiles", mfma_counter_file(args.workload, args.impl_name, profile_tag(args)))
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


# gdr_chunk_fwd_ws (T, or the per-channel decay's operands, formed for every chunk first) where
# it applies, except on gdn: there the fused kernel is as fast (171-174 us either way on one
# MI355X) at 1.01x the algorithmic HBM bytes instead of 1.57x (keys read twice, T written and
# read back); on gdn2 and the long prefill the workspace path is 20 % and 7 % faster, and the
# per-channel decay runs on the matrix cores only through it
WS_OFF_BY_DEFAULT = {"gdn"}


def wants_workspace(args) -> bool:
    if args.no_workspace or args.workspace == "off":
        return False
    return args.workspace == "on" or args.workload not in WS_OFF_BY_DEFAULT


def workspace_bytes(args, s) -> int:
    if not wants_workspace(args):
        return 0
    import chunked_gated_delta_gdr_amd as G
    return G.gdr_chunk_fwd_workspace_size(G.make_desc(
        B=s.B, T=s.T, H=s.H, Dk=s.Dk, Dv=s.Dv, chunk=s.chunk,
        io_dtype=G.GDR_BF16 if s.dtype == "bf16" else G.GDR_F32,
        gain=G.GDR_GAIN_SCALAR if s.gain == "scalar" else G.GDR_GAIN_CHANNEL,
        decay={"scalar": G.GDR_DECAY_SCALAR, "channel": G.GDR_DECAY_CHANNEL}.get(s.decay, G.GDR_DECAY_NONE),
        wkey=G.GDR_WKEY_DIAG_PRECOND if s.wkey == "precond" else G.GDR_WKEY_SAME, neumann_order=args.neumann,
        residual_steps=args.residual, impl={"auto": 0, "generic": 1, "mfma": 2}[args.impl]))


def profile_tag(args) -> str:
    """Suffix of the committed counter summaries: '_ws' for a call through the workspace."""
    if args.workload == "decode":
        return ""
    return "_ws" if workspace_bytes(args, __import__("gdr_synth").spec(args.workload)) > 0 else ""


def traffic_file(workload: str, impl: str, tag: str = "") -> str:
    return "step_decode_traffic.json" if impl == "step" else f"chunk_fwd_{impl}_{workload}{tag}_traffic.json"


def traffic_from_profile(workload: str, impl: str, tag: str = ""):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", traffic_file(workload, impl, tag))
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("source_sha") != source_sha(impl):
        return None
    return rec.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample of streams, one stream per worker task
# ------------------------------------------------------------------------------------

def _cpu_worker_init():
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"


def _cpu_task(args):
    stream, precond = args
    import oracle
    t0 = time.perf_counter()
    oracle.recurrent_stream(stream, precond=precond)
    return time.perf_counter() - t0


def host_cpu():
    """(CPU model from /proc/cpuinfo, logical cores this process may run on)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return model, cores


def cpu_baseline(s, x, tokens: int, n_streams: int, min_cpu_s: float = 10.0):
    """The fp64 oracle on every sampled stream, one stream per task, over every core this
    process may use, capped by OMP_NUM_THREADS when the environment sets it (a process's share
    of a shared host), and by the number of streams.  Passes over the sample repeat until at least
    `min_cpu_s` of CPU work has been timed."""
    import multiprocessing as mp
    import numpy as np
    model, cores = host_cpu()
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    workers = max(1, min(cores, n_streams, share if share > 0 else cores))
    streams = [(b, h) for b in range(s.B) for h in range(s.H)][:n_streams]
    pre = None
    if s.wkey == "precond":
        pre = dict(rho=s.pc_rho, eps=s.pc_eps, h_init=np.full(s.Dk, s.pc_h0), t0=0)
    # float32 copies travel to the workers: exact, since every input was rounded to fp32 (or
    # further to bf16) when it was generated, and the oracle widens to fp64 itself
    tasks = [({k: (np.ascontiguousarray(v[b, :tokens, h], dtype=np.float32) if v is not None else None)
               for k, v in x.items()}, pre)
             for (b, h) in streams]
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers, initializer=_cpu_worker_init) as pool:
        pool.map(_cpu_task, [(
            {k: (v[:4] if v is not None else None) for k, v in t[0].items()}, t[1]) for t in tasks[:workers]])
        cpu_s, wall, passes = 0.0, 0.0, 0
        while cpu_s < min_cpu_s and passes < 8:   # (the call above warmed the workers' imports)
            t0 = time.perf_counter()
            cpu_s += sum(pool.map(_cpu_task, tasks, chunksize=1))
            wall += time.perf_counter() - t0
            passes += 1
    token_heads = len(streams) * tokens * passes
    return {
        "value": token_heads / s.H / wall,
        "unit": "tokens/s",
        "cores": workers,
        "host_cores": cores,
        "cpu_model": model,
        "kind": "oracle",
        "sample": f"fp64 token-by-token oracle on {len(streams)} of {s.B * s.H} (batch, head) streams x "
                  f"{tokens} of {s.T} tokens, {passes} pass(es) ({token_heads} token-heads, {wall:.2f} s wall "
                  f"on {workers} processes of the {cores} logical cores available"
                  f"{' (OMP_NUM_THREADS=' + str(share) + ' caps the pool)' if 0 < share < cores else ''}, "
                  f"{cpu_s:.1f} s of CPU work); tokens/s = token-heads / H / wall",
    }


# ------------------------------------------------------------------------------------
# HBM traffic from rocprofv3 counters: the chunk kernel's FETCH_SIZE / WRITE_SIZE (KiB per
# dispatch), each scaled by what the same counter reads for a plain device copy of known size
# ------------------------------------------------------------------------------------

def copy_probe(mb: int):
    """A plain device-to-device copy of `mb` MiB, three times (the calibration kernel)."""
    import torch
    dev = torch.device("cuda:0")
    n = mb * (1 << 20) // 4
    src = torch.empty(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1.0)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] copy probe: {mb} MiB x 3", file=sys.stderr)


def _counter_per_dispatch(csv_path: str, counter: str, name_has: str):
    import csv
    per = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and name_has in r["Kernel_Name"]:
                per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for kernels matching '{name_has}' in {csv_path}")
    return sorted(per.values())


# the kernels one forward call may launch: the sequential pass and, with the workspace, the
# kernels that form T (or the per-channel decay's operands and records) for every chunk first
CALL_KERNELS = {"mfma": ("chunk_mfma_kernel", "chunk_t_kernel", "kda_prep_fast_kernel", "kda_prep_robust_kernel"),
                "generic": ("chunk_generic",), "step": ("step_kernel",)}


def _counter_per_call(csv_path: str, counter: str, impl: str):
    """The counter per forward call: the median per dispatch of each kernel the call launches,
    summed over those kernels (each launches once per call)."""
    import csv
    import statistics
    per = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            for k in CALL_KERNELS[impl]:
                if k in r["Kernel_Name"]:
                    d = per.setdefault(k, {})
                    d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for the kernels of '{impl}' in {csv_path}")
    meds = {k: statistics.median(v.values()) for k, v in per.items()}
    return sum(meds.values()), {k: (m, len(per[k])) for k, m in meds.items()}


def traffic_summary(args):
    """Writes profiles/chunk_fwd_<impl>_<workload>_traffic.json from four counter CSVs."""
    import statistics
    fetch, f_parts = _counter_per_call(args.traffic_summary[0], "FETCH_SIZE", args.impl_name)
    write, w_parts = _counter_per_call(args.traffic_summary[1], "WRITE_SIZE", args.impl_name)
    f_c = _counter_per_dispatch(args.traffic_summary[2], "FETCH_SIZE", "copy")
    w_c = _counter_per_dispatch(args.traffic_summary[3], "WRITE_SIZE", "copy")
    copy_kib = args.copy_probe_mb * 1024.0
    # the last copy of the probe is the representative one (the first may find the source
    # still in the last-level cache from the fill)
    fac_f, fac_w = copy_kib / f_c[-1], copy_kib / w_c[-1]
    if args.workload == "decode":
        sd = __import__("gdr_synth").spec("long")
        ab = decode_alg_bytes(sd.decode_batch, sd.H, sd.Dk, sd.Dv)
    else:
        ab = alg_bytes(__import__("gdr_synth").spec(args.workload))
    rec = {
        "kernel": "gdr_recurrent_step" if args.impl_name == "step" else f"gdr_chunk_fwd/{args.impl_name}",
        "workload": args.workload,
        "source_sha": source_sha(args.impl_name),
        "fetch_kib_per_call": fetch, "write_kib_per_call": write,
        "per_kernel_fetch_kib_median_and_dispatches": f_parts, "per_kernel_write_kib_median_and_dispatches": w_parts,
        "copy_probe_mib": args.copy_probe_mb, "copy_fetch_kib": f_c[-1], "copy_write_kib": w_c[-1],
        "scale_fetch": fac_f, "scale_write": fac_w,
        "hbm_bytes_per_launch": round((fetch * fac_f + write * fac_w) * 1024.0),
        "alg_bytes_per_launch": ab,
    }
    out = os.path.join(ROOT, "profiles", traffic_file(args.workload, args.impl_name, profile_tag(args)))
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


# ------------------------------------------------------------------------------------
# decode: gdr_recurrent_step at the long workload's decode batch (64 sequences x 32 heads)
# ------------------------------------------------------------------------------------

def decode_alg_bytes(Bd, H, Dk, Dv, esz=2) -> int:
    """State read and written once (fp32) + q, k, v, beta, log alpha read + o written."""
    return Bd * H * (2 * Dv * Dk * 4 + (2 * Dk + Dv) * esz + 8 + Dv * esz)


def bench_decode(args):
    import numpy as np
    import torch

    import chunked_gated_delta_gdr_amd as G
    import gdr_synth as gs

    s = gs.spec("long")
    Bd, H, Dk, Dv = s.decode_batch, s.H, s.Dk, s.Dv
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nstage = 8   # distinct step inputs staged on the device, used in turn
    t = lambda a, dt: torch.from_numpy(a).to(dev).to(dt)
    steps_in = []
    for i in range(nstage):
        xi = gs.make_decode_inputs(s, i)
        steps_in.append(dict(q=t(xi["q"], torch.bfloat16), k=t(xi["k"], torch.bfloat16),
                             v=t(xi["v"], torch.bfloat16), beta=t(xi["beta"], torch.float32),
                             log_alpha=t(xi["log_alpha"], torch.float32)))
    rng = np.random.Generator(np.random.PCG64(s.seed + 7777))
    s0 = (0.05 * rng.standard_normal((Bd, H, Dv, Dk))).astype(np.float32)
    state = torch.from_numpy(s0).to(dev)
    outs = [torch.empty((Bd, H, Dv), dtype=torch.bfloat16, device=dev) for _ in range(nstage)]
    stream = torch.cuda.current_stream(dev)

    def step(i):
        a = steps_in[i % nstage]
        G.gdr_recurrent_step(a["q"], a["k"], a["v"], state, beta=a["beta"], log_alpha=a["log_alpha"],
                             out=outs[i % nstage], stream=stream)

    # parity first: one step from the known state, sampled streams vs the oracle
    parity = None
    if not args.no_parity:
        import oracle
        step(0)
        torch.cuda.synchronize()
        x0 = gs.make_decode_inputs(s, 0)
        sub = {k: (None if v is None else v[:4]) for k, v in x0.items()}
        o_ref, s_ref, _ = oracle.decode_step(sub, s0[:4].astype(np.float64))
        parity = {"streams": "4 x 32 heads", "rel_l2_out": oracle.rel_l2(outs[0][:4].double().cpu().numpy(), o_ref),
                  "rel_l2_state": oracle.rel_l2(state[:4].double().cpu().numpy(), s_ref)}
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    n_settle = settle(step, args.settle_s)
    ms_per_step, launch = time_steps(step, args.steps, stream)
    avg_s = sum(launch) / len(launch) / 1e3
    print(f"[bench] decode {args.steps} steps: launch avg {avg_s * 1e6:.2f} us min {min(launch) * 1e3:.2f} us",
          file=sys.stderr, flush=True)
    ab = decode_alg_bytes(Bd, H, Dk, Dv)
    gbs = ab / avg_s / 1e9
    rec = {
        "metric": "tokens/s gated-delta decode step (batch 64 x H32 d128, bf16 in, fp32 state in place)",
        "value": round(Bd / (ms_per_step / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle": {"seconds": args.settle_s, "steps": n_settle}, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded decode inputs of the long workload; random fp32 start state)",
        "config": {"workload": f"decode: batch {Bd} H{H} Dk{Dk} Dv{Dv} bf16 scalar gain+decay, state fp32 in place",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic_from_profile("decode", "step"),
                     "kernel": "gdr_recurrent_step",
                     "alg_bytes_per_launch": ab, "avg_launch_us": round(avg_s * 1e6, 2)},
        "cpu_baseline": None, "parity": parity,
    }
    print(json.dumps(rec), flush=True)


def settle(step, seconds: float) -> int:
    """Keep running the step (after the warmup steps, untimed) until `seconds` of wall time
    have passed: the GPU raises its engine clock only under sustained load (~2.05 GHz for the
    first ~30 ms of back-to-back launches, ~2.38 GHz after), so the timed steps see the clock
    a long-running job sees.  Returns the number of steps run."""
    import torch
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            step(n)
            n += 1
        torch.cuda.synchronize()
    return n


def time_steps(step, steps: int, stream):
    """The timed region: `steps` launches back to back between one pair of HIP events on the
    launch stream (synchronized on both sides); returns ms per step.  Then a second region of
    the same length with an event pair around every launch, for the per-launch durations the
    roofline uses (recording events between launches widens the gaps between them, so the
    first region, which `value` comes from, records none).  Returns (ms_per_step, [ms per
    launch])."""
    import torch
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return ms_per_step, [a.elapsed_time(b) for a, b in ev]


def bwd_alg_bytes(s) -> int:
    """Bytes the backward must move per call: the forward's inputs, dO, the initial state
    and dL/dS_T read once; every gradient (fp32) written once."""
    esz = 2 if s.dtype == "bf16" else 4
    per_tok = (2 * s.Dk + 2 * s.Dv) * esz                       # q, k, v, dO
    per_tok += (2 * s.Dk + s.Dv) * 4                            # dq, dk, dv
    per_tok += 8 if s.gain == "scalar" else (s.Dk + s.Dv) * (esz + 4)   # gains and their grads
    per_tok += {"scalar": 8, "channel": 8 * s.Dk}.get(s.decay, 0)   # log alpha and its grad
    per_head = 3 * s.Dv * s.Dk * 4                              # S_0, dS_T, dS_0
    return s.B * s.T * s.H * per_tok + s.B * s.H * per_head


def bwd_alg_flops(s) -> float:
    """Algorithmic FLOPs of one backward call: the forward recompute (alg_flops) plus, per
    token-head, the reverse sweep (R dS^T, the state-gradient update: 3 Dk Dv; P^T dO and
    T^T dD: 2 (C+1)/2 Dv MACs) and the per-chunk products (dO S, dX S, D dS': 3 Dk Dv;
    dO D^T, dX D^T: 2 (C+1)/2 Dv; dM R, dL' R, dM^T Q, dL'^T E: 4 (C+1)/2 Dk MACs)."""
    C, Dk, Dv = s.chunk, s.Dk, s.Dv
    macs = 6 * Dk * Dv + 2 * (C + 1) * Dv + 2 * (C + 1) * Dk
    return alg_flops(s) + 2.0 * macs * s.B * s.T * s.H


def bench_backward(args):
    """One step = one gdr_chunk_bwd call (forward recompute, reverse sweep, per-chunk pass)."""
    import numpy as np
    import torch

    import chunked_gated_delta_gdr_amd as G
    import gdr_synth as gs

    s = gs.spec(args.workload)
    pc = s.wkey == "precond"
    pre = dict(rho=s.pc_rho, eps=s.pc_eps, h0=s.pc_h0, t0=0) if pc else None
    pcargs = dict(precond=True, pc_rho=s.pc_rho, pc_eps=s.pc_eps, pc_h0=s.pc_h0, pc_t0=0) if pc else {}
    x, cot = gs.make_inputs(s), gs.make_cotangents(s)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    io = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    f32 = torch.float32
    t = lambda a, dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
    a = dict(q=t(x["q"], io), k=t(x["k"], io), v=t(x["v"], io), beta=t(x.get("beta"), f32),
             log_alpha=t(x.get("log_alpha"), f32), erase=t(x.get("erase"), io), write=t(x.get("write"), io),
             write_key=t(x.get("write_key"), io))
    rng = np.random.Generator(np.random.PCG64(s.seed + 31))
    s0 = (0.1 * rng.standard_normal((s.B, s.H, s.Dv, s.Dk))).astype(np.float32)
    S0, dO, dST = t(s0, f32), t(cot["d_out"], io), t(cot["d_state_out"], f32)
    desc = G.make_desc(B=s.B, T=s.T, H=s.H, Dk=s.Dk, Dv=s.Dv, chunk=s.chunk, io_dtype=G.GDR_BF16 if
                       s.dtype == "bf16" else G.GDR_F32,
                       gain=G.GDR_GAIN_SCALAR if s.gain == "scalar" else G.GDR_GAIN_CHANNEL,
                       decay={"scalar": G.GDR_DECAY_SCALAR, "channel": G.GDR_DECAY_CHANNEL}.get(s.decay, G.GDR_DECAY_NONE),
                       wkey=G.GDR_WKEY_DIAG_PRECOND if pc else G.GDR_WKEY_SAME, neumann_order=args.neumann)
    ws = torch.empty(G.gdr_chunk_bwd_workspace_size(desc), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    print(f"[bench] backward {args.workload}: workspace {ws.numel() / 2**20:.1f} MiB, steps {args.steps} "
          f"warmup {args.warmup}", file=sys.stderr, flush=True)

    def step():
        return G.gdr_chunk_bwd(a["q"], a["k"], a["v"], dO, beta=a["beta"], log_alpha=a["log_alpha"],
                               erase=a["erase"], write=a["write"], write_key=a["write_key"], state_in=S0,
                               d_state_out=dST, chunk=s.chunk, neumann_order=args.neumann, workspace=ws,
                               stream=stream, **pcargs)

    for _ in range(args.warmup):
        g = step()
    torch.cuda.synchronize()
    n_settle = settle(lambda i: step(), args.settle_s)
    last = {}

    def step_keep(i):
        last["g"] = step()

    ms_per_step, call_ms = time_steps(step_keep, args.steps, stream)
    g = last["g"]
    avg_s = sum(call_ms) / len(call_ms) / 1e3
    print(f"[bench] backward call avg {avg_s * 1e6:.1f} us min {min(call_ms) * 1e3:.1f} us",
          file=sys.stderr, flush=True)
    af = bwd_alg_flops(s)
    ab = bwd_alg_bytes(s)
    parity = None
    if not args.no_parity:
        import oracle
        if args.neumann >= 0:   # the band-limited T: the chunk form's own gradient
            ref = oracle.chunked_grad(x, cot["d_out"], cot["d_state_out"], chunk=s.chunk, band=args.neumann,
                                      state0=s0, streams=[(0, 0)], precond=pre)
        else:
            ref = oracle.recurrent_grad(x, cot["d_out"], cot["d_state_out"], state0=s0, streams=[(0, 0)],
                                        precond=pre, checkpoint=64)
        parity = {"stream": "(0,0)", "tokens": s.T}
        for name in ("dq", "dk", "dv", "dbeta", "dlog_alpha", "derase", "dwrite"):
            if name in ref:
                parity[f"rel_l2_{name}"] = oracle.rel_l2(g[name][0, :, 0].double().cpu().numpy(),
                                                         ref[name][0, :, 0])
        parity["rel_l2_dstate_in"] = oracle.rel_l2(g["dstate_in"][0, 0].double().cpu().numpy(),
                                                   ref["dS0"][0, 0])
        if pc:
            parity["rel_l2_dpc_h_in"] = oracle.rel_l2(g["dpc_h_in"][0, 0].double().cpu().numpy(),
                                                      ref["dpc_h_init"][0, 0])
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        n = min(s.T, 1024)
        sub = {k: (None if v is None else v[:1, :n, :1]) for k, v in x.items()}
        w0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - w0 < 10.0:
            oracle.recurrent_grad(sub, cot["d_out"][:1, :n, :1], None, precond=pre)
            reps += 1
        wall = time.perf_counter() - w0
        cpu = {"value": round(reps * n / wall / s.H, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"fp64 token-by-token reverse sweep on stream (0,0), {n} tokens, {reps} repetitions "
                         f"in {wall:.1f} s on one core; tokens/s = token-heads / H / wall"}
    rec = {
        "metric": f"tokens/s chunked gated-delta backward ({args.workload}: B{s.B} H{s.H} T{s.T} d{s.Dk} {s.dtype})",
        "value": round(s.B * s.T / (ms_per_step / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle": {"seconds": args.settle_s, "steps": n_settle}, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded inputs of the workload; dO, dL/dS_T ~ N(0,1); random fp32 start state)",
        "config": {"workload": f"{args.workload} backward: B{s.B} H{s.H} T{s.T} Dk{s.Dk} Dv{s.Dv} C{s.chunk} "
                               f"{s.dtype} in, fp32 arithmetic and gradients, gain={s.gain} decay={s.decay} "
                               f"wkey={s.wkey}" + (f" band N={args.neumann}" if args.neumann >= 0 else " exact T"),
                   "parallelism": "single GPU"},
        "roofline": {"bound": "alu", "achieved": round(af / avg_s / 1e12, 2), "peak": FP32_VALU_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(af / avg_s / 1e12 / FP32_VALU_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "gdr_chunk_bwd (forward recompute + reverse sweep + per-chunk pass)",
                     "alg_gflop_per_launch": round(af / 1e9, 3), "avg_launch_us": round(avg_s * 1e6, 2),
                     "alg_bytes_per_launch": ab, "hbm_frac_of_alg_bytes": round(ab / avg_s / 1e9 / HBM_PEAK_GBS, 4)},
        "cpu_baseline": cpu, "parity": parity,
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="after the warmup steps, keep stepping (untimed) for this many seconds so the "
                         "engine clock reaches its sustained-load value")
    ap.add_argument("--workload", default="gdn", choices=["gdn", "gdn2", "pdn", "long", "plain", "kda", "decode"])
    ap.add_argument("--neumann", type=int, default=-1)
    ap.add_argument("--residual", type=int, default=0,
                    help="residual-correction steps on the band-N start (needs --neumann N)")
    ap.add_argument("--impl", default="auto", choices=["auto", "generic", "mfma"])
    ap.add_argument("--workspace", default="auto", choices=["auto", "on", "off"],
                    help="call gdr_chunk_fwd_ws with its workspace (auto: everywhere it applies but gdn)")
    ap.add_argument("--no-workspace", action="store_true", help="same as --workspace off")
    ap.add_argument("--bwd", action="store_true", help="time gdr_chunk_bwd instead of the forward")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="run only the counter-calibration copy of this many MiB")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                           "COPY_WRITE_CSV"),
                    help="write the traffic summary of --workload from rocprofv3 counter CSVs")
    ap.add_argument("--impl-name", default="mfma", choices=["mfma", "generic", "step"])
    ap.add_argument("--mfma-summary", metavar="PMC_CSV",
                    help="write the matrix-core counter summary of --workload from a rocprofv3 counter CSV")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(args)
        return
    if args.mfma_summary:
        mfma_summary(args)
        return
    if args.copy_probe_mb:
        copy_probe(args.copy_probe_mb)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): every "
              "(batch, head) stream is independent, so more GPUs would each run their own share of "
              "streams with no communication; bench.py measures the one-GPU share.", file=sys.stderr)
        sys.exit(2)
    if args.workload == "decode":
        bench_decode(args)
        return
    if args.bwd:
        bench_backward(args)
        return

    import numpy as np
    import torch

    import chunked_gated_delta_gdr_amd as G
    import gdr_synth as gs

    s = gs.spec(args.workload)
    x = gs.make_inputs(s)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    io = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    f32 = torch.float32

    def upload(xx):
        t = lambda a, dt: None if a is None else torch.from_numpy(a).to(dev).to(dt)
        return dict(q=t(xx["q"], io), k=t(xx["k"], io), v=t(xx["v"], io), beta=t(xx.get("beta"), f32),
                    log_alpha=t(xx.get("log_alpha"), f32), erase=t(xx.get("erase"), io),
                    write=t(xx.get("write"), io), write_key=t(xx.get("write_key"), io))

    # two resident input sets, alternated, so the 256 MB last-level cache cannot serve the
    # previous step's inputs
    sets = [upload(x)]
    rolled = {k: (None if v is None else np.ascontiguousarray(np.roll(v, 1, axis=2))) for k, v in x.items()}
    sets.append(upload(rolled))
    outs = [torch.empty((s.B, s.T, s.H, s.Dv), dtype=io, device=dev) for _ in sets]
    states = [torch.empty((s.B, s.H, s.Dv, s.Dk), dtype=f32, device=dev) for _ in sets]
    hs = [torch.empty((s.B, s.H, s.Dk), dtype=f32, device=dev) for _ in sets]
    stream = torch.cuda.current_stream(dev)
    precond = s.wkey == "precond"

    # the workspace of gdr_chunk_fwd_ws (T of every chunk formed first) where it applies
    ws_bytes = workspace_bytes(args, s)
    tag = "_ws" if ws_bytes > 0 else ""
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes > 0 else None

    def step(i):
        j = i % 2
        a = sets[j]
        G.gdr_chunk_fwd(a["q"], a["k"], a["v"], beta=a["beta"], log_alpha=a["log_alpha"], erase=a["erase"],
                        write=a["write"], write_key=a["write_key"], precond=precond,
                        pc_h_out=hs[j] if precond else None, out=outs[j], state_out=states[j],
                        chunk=s.chunk, neumann_order=args.neumann, residual_steps=args.residual,
                        impl=args.impl, workspace=ws, stream=stream)

    def kernel_of(neumann, residual):
        code = G.gdr_chunk_fwd_impl(G.make_desc(
            B=s.B, T=s.T, H=s.H, Dk=s.Dk, Dv=s.Dv, chunk=s.chunk,
            io_dtype=G.GDR_BF16 if s.dtype == "bf16" else G.GDR_F32,
            gain=G.GDR_GAIN_SCALAR if s.gain == "scalar" else G.GDR_GAIN_CHANNEL,
            decay={"scalar": G.GDR_DECAY_SCALAR, "channel": G.GDR_DECAY_CHANNEL}.get(s.decay, G.GDR_DECAY_NONE),
            wkey=G.GDR_WKEY_DIAG_PRECOND if precond else G.GDR_WKEY_SAME, neumann_order=neumann,
            residual_steps=residual, impl={"auto": 0, "generic": 1, "mfma": 2}[args.impl]))
        return {G.GDR_IMPL_MFMA: "mfma", G.GDR_IMPL_GENERIC: "generic"}.get(code, "?")

    impl_name = kernel_of(args.neumann, args.residual)
    if s.decay == "channel" and ws is not None:   # the per-channel decay's matrix-core path needs the workspace
        impl_name = "mfma"
    print(f"[bench] workload {args.workload} impl {impl_name} steps {args.steps} warmup {args.warmup}",
          file=sys.stderr, flush=True)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    n_settle = settle(step, args.settle_s)
    wall0 = time.perf_counter()
    ms_per_step, launch_ms = time_steps(step, args.steps, stream)
    wall = time.perf_counter() - wall0
    avg_launch_s = sum(launch_ms) / len(launch_ms) / 1e3
    print(f"[bench] timed {args.steps} steps: {ms_per_step * args.steps:.3f} ms events (then {args.steps} "
          f"launches with per-launch events), {wall * 1e3:.3f} ms host wall for both; "
          f"launch avg {avg_launch_s * 1e6:.2f} us min {min(launch_ms) * 1e3:.2f} us",
          file=sys.stderr, flush=True)

    tokens = s.B * s.T
    value = tokens / (ms_per_step / 1e3)
    ab = alg_bytes(s)
    af = alg_flops(s, None if args.neumann < 0 else args.neumann, args.residual)
    achieved_gbs = ab / avg_launch_s / 1e9
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved_gbs, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
        # (the counters are taken on the exact-T configuration of the workload)
        "traffic": traffic_from_profile(args.workload, impl_name, tag) if args.neumann < 0 else None,
        "kernel": f"gdr_chunk_fwd/{impl_name}",
        "alg_bytes_per_launch": ab,
        "avg_launch_us": round(avg_launch_s * 1e6, 2),
        "mfma_bf16_frac": round(af / avg_launch_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "alg_gflop_per_launch": round(af / 1e9, 3),
    }
    mc = mfma_counters_from_profile(args.workload, impl_name, tag) if args.neumann < 0 and args.residual == 0 else None
    if mc is not None:
        # the matrix-core work the counters saw per dispatch (dense tiles, padding and the split
        # products included), over this run's launch time
        roofline["mfma_bf16_frac_counters"] = round(mc["mfma_bf16_flop_per_dispatch"] / avg_launch_s / 1e12
                                                    / MFMA_BF16_PEAK_TFLOPS, 4)
        if "mfma_busy_cycles_per_simd" in mc:
            roofline["mfma_busy_frac_counters"] = round(mc["mfma_busy_cycles_per_simd"]
                                                        / (avg_launch_s * ENGINE_CLOCK_HZ), 4)

    parity = None
    if not args.no_parity:
        # stream (0,0) of the last timed input set against the oracle: with the exact T the whole
        # stream (the worst 64-token block and the final state too), with a band limit its first
        # 512 tokens against the oracle's chunk form
        import oracle
        n = s.T if args.neumann < 0 else min(512, s.T)
        j = (args.steps - 1) % 2
        xs = x if j == 0 else rolled
        sub = {k: (None if v is None else v[:1, :n, :1]) for k, v in xs.items()}
        pre = dict(rho=s.pc_rho, eps=s.pc_eps, h0=s.pc_h0, t0=0) if precond else None
        if args.neumann < 0:
            o_ref, s_ref, _ = oracle.recurrent(sub, precond=pre)
        else:
            mode = ("neumann", args.neumann) if args.residual <= 0 else ("residual", args.neumann, args.residual)
            o_ref, _, _ = oracle.chunked(sub, chunk=s.chunk, t_mode=mode, precond=pre)
        got = outs[j][:1, :n, :1].double().cpu().numpy()
        parity = {"stream": "(0,0)", "tokens": n, "rel_l2_out": oracle.rel_l2(got, o_ref)}
        if args.neumann < 0:
            parity["rel_l2_out_worst_64_token_block"] = max(
                oracle.rel_l2(got[:, t:t + 64], o_ref[:, t:t + 64]) for t in range(0, n, 64))
            parity["rel_l2_out_last_512_tokens"] = oracle.rel_l2(got[:, -512:], o_ref[:, -512:])
            parity["rel_l2_state"] = oracle.rel_l2(states[j][:1, :1].double().cpu().numpy(), s_ref)

    exact_vs_approx = None
    if args.neumann >= 0 and not args.no_parity:
        # the error between the exact T and the band-limited (or residual-corrected) T: on the GPU
        # over the whole output of the last timed input set and over stream (0,0), and the same
        # quantity from the oracle on stream (0,0), every token
        import oracle
        j = (args.steps - 1) % 2
        xs = x if j == 0 else rolled
        ex = torch.empty_like(outs[j])
        a = sets[j]
        G.gdr_chunk_fwd(a["q"], a["k"], a["v"], beta=a["beta"], log_alpha=a["log_alpha"], erase=a["erase"],
                        write=a["write"], write_key=a["write_key"], precond=precond, out=ex, chunk=s.chunk,
                        impl=args.impl, stream=stream)
        torch.cuda.synchronize()
        ap = outs[j].double()
        exd = ex.double()
        gpu_all = float(torch.linalg.vector_norm(ap - exd) / torch.linalg.vector_norm(exd))
        gpu_00 = float(torch.linalg.vector_norm(ap[0, :, 0] - exd[0, :, 0]) / torch.linalg.vector_norm(exd[0, :, 0]))
        sub = {k: (None if v is None else v[:1, :, :1]) for k, v in xs.items()}
        pre = dict(rho=s.pc_rho, eps=s.pc_eps, h0=s.pc_h0, t0=0) if precond else None
        o_ex, _, _ = oracle.recurrent(sub, precond=pre)
        mode = ("neumann", args.neumann) if args.residual <= 0 else ("residual", args.neumann, args.residual)
        o_ap, _, _ = oracle.chunked(sub, chunk=s.chunk, t_mode=mode, precond=pre)
        exact_vs_approx = {
            "approx": f"band N={args.neumann}" + (f" + {args.residual} residual steps" if args.residual > 0 else ""),
            "rel_l2_exact_vs_approx_gpu_all_streams": gpu_all,
            "rel_l2_exact_vs_approx_gpu_stream00": gpu_00,
            "rel_l2_exact_vs_approx_oracle_stream00": oracle.rel_l2(o_ap, o_ex),
            "stream": "(0,0)", "tokens": s.T,
        }
        ex_impl = kernel_of(-1, 0)
        if ex_impl != impl_name:
            # the approximation ran on another kernel than the exact T (the residual correction
            # has no bf16 matrix-core path): the gap above then also holds the two kernels'
            # different rounding, so the exact T is run on the approximation's kernel as well
            ex2 = torch.empty_like(outs[j])
            G.gdr_chunk_fwd(a["q"], a["k"], a["v"], beta=a["beta"], log_alpha=a["log_alpha"], erase=a["erase"],
                            write=a["write"], write_key=a["write_key"], precond=precond, out=ex2, chunk=s.chunk,
                            impl=impl_name, stream=stream)
            torch.cuda.synchronize()
            ex2d = ex2.double()
            exact_vs_approx["exact_kernel"] = ex_impl
            exact_vs_approx[f"rel_l2_exact_vs_approx_gpu_all_streams_both_{impl_name}"] = float(
                torch.linalg.vector_norm(ap - ex2d) / torch.linalg.vector_norm(ex2d))

    cpu = None
    if not args.no_cpu_baseline:
        # every (batch, head) stream, capped at 300k token-heads: about 10-15 s of single-core
        # oracle work at ~45 us per token-head (the whole gdn / gdn2 / pdn workload)
        cpu = cpu_baseline(s, x, tokens=min(s.T, max(64, 300_000 // (s.B * s.H))), n_streams=s.B * s.H)

    rec = {
        "metric": METRIC if args.workload == "gdn" else
        f"tokens/s chunked gated-delta fwd ({args.workload}: B{s.B} H{s.H} T{s.T} d{s.Dk} {s.dtype}); % MFMA/HBM peak",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup, "settle": {"seconds": args.settle_s, "steps": n_settle},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), gates as the workload states)",
        "config": {"workload": f"{args.workload}: B{s.B} H{s.H} T{s.T} Dk{s.Dk} Dv{s.Dv} C{s.chunk} "
                               f"{s.dtype} gain={s.gain} decay={s.decay} wkey={s.wkey}"
                               + (f" band N={args.neumann}" if args.neumann >= 0 else " exact T")
                               + (f" + {args.residual} residual steps" if args.neumann >= 0 and args.residual > 0 else ""),
                   "B": s.B, "T": s.T, "H": s.H, "Dk": s.Dk, "Dv": s.Dv, "chunk": s.chunk,
                   "impl": impl_name, "workspace": ws is not None, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    if exact_vs_approx is not None:
        rec["exact_vs_approx"] = exact_vs_approx
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
