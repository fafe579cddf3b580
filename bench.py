#!/usr/bin/env python3
"""Throughput of the chunked gated delta-rule forward on one MI355X.

One step = one gdr_chunk_fwd call over one batch of synthetic input (every stage of the
chunked forward runs inside it).  Default workload: scalar-gated delta rule, B4 H16 T4096
Dk = Dv = 128, bf16 inputs, fp32 state, chunk 64.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gdn|gdn2|pdn|long|plain]
                    [--neumann N] [--impl auto|generic|mfma] [--no-cpu-baseline]
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

KERNEL_SOURCES = {
    "mfma": ["chunked_gated_delta_gdr_amd/csrc/chunk_mfma.hip"],
    "generic": ["chunked_gated_delta_gdr_amd/csrc/chunk_generic.hip"],
}


def alg_bytes(s) -> int:
    """Bytes the method must move per call: inputs read once, output and final state
    (and preconditioner accumulator) written once; intermediates never reach HBM."""
    esz = 2 if s.dtype == "bf16" else 4
    per_tok = (2 * s.Dk + 2 * s.Dv) * esz
    per_tok += 4 if s.gain == "scalar" else (s.Dk + s.Dv) * esz
    per_tok += 4 if s.decay == "scalar" else 0
    per_tok += s.Dk * esz if s.wkey == "explicit" else 0
    per_head = s.Dv * s.Dk * 4 + (s.Dk * 4 if s.wkey == "precond" else 0)
    return s.B * s.T * s.H * per_tok + s.B * s.H * per_head


def alg_flops(s, band=None) -> float:
    """Algorithmic FLOPs per call (triangular products counted triangular):
    per token-head MACs = 3 Dk Dv (W S^T, Q S^T, state update) + (C-1)/2 Dk (A)
    + (C+1)/2 (2 Dk + 2 Dv) (W, U, Q R^T, P D) + C^2/6 (forward substitution)."""
    C, Dk, Dv = s.chunk, s.Dk, s.Dv
    tri = C * C / 6.0 if band is None or band >= C - 1 else (band * (band + 1) / 2.0)
    macs = 3 * Dk * Dv + (C - 1) / 2 * Dk + (C + 1) / 2 * (2 * Dk + 2 * Dv) + tri
    return 2.0 * macs * s.B * s.T * s.H


def source_sha(impl: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[impl] + ["chunked_gated_delta_gdr_amd/csrc/common.h"]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str, impl: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"chunk_fwd_{impl}_{workload}_traffic.json")
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


def cpu_baseline(s, x, tokens: int, n_streams: int):
    import multiprocessing as mp
    import numpy as np
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    workers = max(1, min(16, cores, n_streams))
    streams = [(b, h) for b in range(s.B) for h in range(s.H)][:n_streams]
    pre = None
    if s.wkey == "precond":
        pre = dict(rho=s.pc_rho, eps=s.pc_eps, h_init=np.full(s.Dk, s.pc_h0), t0=0)
    tasks = [({k: (v[b, :tokens, h] if v is not None else None) for k, v in x.items()}, pre)
             for (b, h) in streams]
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers, initializer=_cpu_worker_init) as pool:
        pool.map(_cpu_task, tasks[:workers])   # warm the workers (imports)
        t0 = time.perf_counter()
        pool.map(_cpu_task, tasks)
        wall = time.perf_counter() - t0
    token_heads = len(streams) * tokens
    return {
        "value": token_heads / s.H / wall,
        "unit": "tokens/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"fp64 token-by-token oracle on {len(streams)} of {s.B * s.H} (batch, head) streams x "
                  f"{tokens} of {s.T} tokens ({token_heads} token-heads, {wall:.2f} s wall on {workers} "
                  f"processes); tokens/s = token-heads / H / wall",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gdn", choices=["gdn", "gdn2", "pdn", "long", "plain"])
    ap.add_argument("--neumann", type=int, default=-1)
    ap.add_argument("--impl", default="auto", choices=["auto", "generic", "mfma"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): every "
              "(batch, head) stream is independent, so more GPUs would each run their own share of "
              "streams with no communication; this build measures the one-GPU share.", file=sys.stderr)
        sys.exit(2)

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

    def step(i):
        j = i % 2
        a = sets[j]
        G.gdr_chunk_fwd(a["q"], a["k"], a["v"], beta=a["beta"], log_alpha=a["log_alpha"], erase=a["erase"],
                        write=a["write"], write_key=a["write_key"], precond=precond,
                        pc_h_out=hs[j] if precond else None, out=outs[j], state_out=states[j],
                        chunk=s.chunk, neumann_order=args.neumann, impl=args.impl, stream=stream)

    impl_code = G.gdr_chunk_fwd_impl(G.make_desc(
        B=s.B, T=s.T, H=s.H, Dk=s.Dk, Dv=s.Dv, chunk=s.chunk,
        io_dtype=G.GDR_BF16 if s.dtype == "bf16" else G.GDR_F32,
        gain=G.GDR_GAIN_SCALAR if s.gain == "scalar" else G.GDR_GAIN_CHANNEL,
        decay=G.GDR_DECAY_SCALAR if s.decay == "scalar" else G.GDR_DECAY_NONE,
        wkey=G.GDR_WKEY_DIAG_PRECOND if precond else G.GDR_WKEY_SAME, neumann_order=args.neumann,
        impl={"auto": 0, "generic": 1, "mfma": 2}[args.impl]))
    impl_name = {G.GDR_IMPL_MFMA: "mfma", G.GDR_IMPL_GENERIC: "generic"}.get(impl_code, "?")
    print(f"[bench] workload {args.workload} impl {impl_name} steps {args.steps} warmup {args.warmup}",
          file=sys.stderr, flush=True)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # per-launch events on the launch stream, and one pair around the whole timed region
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / args.steps
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    avg_launch_s = sum(launch_ms) / len(launch_ms) / 1e3
    print(f"[bench] timed {args.steps} steps: {ms_total:.3f} ms events, {wall * 1e3:.3f} ms host wall; "
          f"launch avg {avg_launch_s * 1e6:.2f} us min {min(launch_ms) * 1e3:.2f} us",
          file=sys.stderr, flush=True)

    tokens = s.B * s.T
    value = tokens / (ms_per_step / 1e3)
    ab = alg_bytes(s)
    af = alg_flops(s, None if args.neumann < 0 else args.neumann)
    achieved_gbs = ab / avg_launch_s / 1e9
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved_gbs, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
        "traffic": traffic_from_profile(args.workload, impl_name),
        "kernel": f"gdr_chunk_fwd/{impl_name}",
        "alg_bytes_per_launch": ab,
        "avg_launch_us": round(avg_launch_s * 1e6, 2),
        "mfma_bf16_frac": round(af / avg_launch_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "alg_gflop_per_launch": round(af / 1e9, 3),
    }

    parity = None
    if not args.no_parity:
        import oracle
        n = min(512, s.T)
        j = (args.steps - 1) % 2
        xs = x if j == 0 else rolled
        sub = {k: (None if v is None else v[:1, :n, :1]) for k, v in xs.items()}
        pre = dict(rho=s.pc_rho, eps=s.pc_eps, h0=s.pc_h0, t0=0) if precond else None
        if args.neumann < 0:
            o_ref, _, _ = oracle.recurrent(sub, precond=pre)
        else:
            o_ref, _, _ = oracle.chunked(sub, chunk=s.chunk, t_mode=("neumann", args.neumann), precond=pre)
        got = outs[j][:1, :n, :1].double().cpu().numpy()
        parity = {"stream": "(0,0)", "tokens": n, "rel_l2_out": oracle.rel_l2(got, o_ref)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(s, x, tokens=min(s.T, 2048), n_streams=min(s.B * s.H, 64))

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), gates as the workload states)",
        "config": {"workload": f"{args.workload}: B{s.B} H{s.H} T{s.T} Dk{s.Dk} Dv{s.Dv} C{s.chunk} "
                               f"{s.dtype} gain={s.gain} decay={s.decay} wkey={s.wkey}"
                               + (f" band N={args.neumann}" if args.neumann >= 0 else " exact T"),
                   "B": s.B, "T": s.T, "H": s.H, "Dk": s.Dk, "Dv": s.Dv, "chunk": s.chunk,
                   "impl": impl_name, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
