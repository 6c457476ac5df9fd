"""Benchmark: ring AllReduce over 8 virtual ranks on one MI355X (busbw and HBM fraction).

Workload: the 8-rank fp32 ring AllReduce swept over 32 KiB .. 3 MiB per rank, with
the parallelization factor, threads per workgroup and slice size chosen by the
on-device coordinate-descent tuner. A timed step is one collective (one kernel
launch) at the top of the sweep, 3 MiB per rank; the rest of the sweep, the
32-256 MiB points and the tuned-vs-fixed comparison are reported beside it.
Plan compilation and tuning happen before timing.

Prints one JSON line. Only one GPU: --gpus above 1 exits with a message.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

P = 8
HEADLINE_BYTES = 3 << 20
SWEEP = [32 << 10, 64 << 10, 128 << 10, 256 << 10, 512 << 10, 1 << 20, 2 << 20, 3 << 20]
LARGE = [32 << 20, 64 << 20, 128 << 20, 256 << 20]
HBM_PEAK_GBS = 8000.0
TUNE_FACTORS = [1, 2, 4, 8, 16, 24, 32]
TUNE_THREADS = [256, 512, 1024]
TUNE_SLICES = [16 << 10, 32 << 10, 64 << 10, 128 << 10, 256 << 10, 512 << 10, 1 << 20]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--fixed", type=str, default="",
                    help="k,nthreads,slice_bytes,protocol(0 simple, 1 LL): skip tuning (profiling runs)")
    ap.add_argument("--no-extras", action="store_true", help="headline only (profiling runs)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the oracle baseline")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="also run the plain copy kernel this many times on 256 MiB (counter calibration)")
    return ap.parse_args()


def source_digest() -> str:
    h = hashlib.sha256()
    for f in ("executor.hip", "device_abi.h"):
        with open(os.path.join(ROOT, "chunk_schedule_execution_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); the P ranks are "
              "virtual ranks on that GPU, no multi-GPU run exists", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W
    from chunk_schedule_execution_amd import Plan, PlanConfig, capi, programs

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    prog = programs.ring_allreduce(P)

    def inputs(S):
        N = S // 4
        outs = [torch.empty(N, dtype=torch.float32, device=dev) for _ in range(P)]
        if S >= (32 << 20):  # timing-only points: seeded N(0,1) drawn on the device
            g = torch.Generator(device=dev)
            g.manual_seed(2026 * 1000 + S // (1 << 20))
            return N, [torch.randn(N, generator=g, device=dev) for _ in range(P)], outs
        xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=S)
        return N, [torch.from_numpy(x).to(dev) for x in xs], outs

    def tune(N):
        desc = prog.to_desc()
        base = PlanConfig(dtype="f32", max_count=N).to_c()
        arrs = [(capi.C.c_int32 * len(v))(*v) for v in (TUNE_FACTORS, TUNE_THREADS, TUNE_SLICES)]
        space = capi.ccl_tune_space(capi.C.cast(arrs[0], capi.C.POINTER(capi.C.c_int32)), len(TUNE_FACTORS),
                                    capi.C.cast(arrs[1], capi.C.POINTER(capi.C.c_int32)), len(TUNE_THREADS),
                                    capi.C.cast(arrs[2], capi.C.POINTER(capi.C.c_int32)), len(TUNE_SLICES),
                                    1, 3, 10, 3)
        best, rep = capi.ccl_tune([desc], N, base, space, stream.cuda_stream)
        return (best.parallel_factor, best.nthreads, best.slice_bytes, best.protocol), rep.evaluations

    def make_plan(N, k, nt, sl, proto=0):
        return Plan(prog, k, PlanConfig(dtype="f32", max_count=N, nthreads=nt, slice_bytes=sl,
                                        protocol="ll" if proto else "simple"))

    def time_plan(plan, N, ins, outs, iters, warmup=3):
        for _ in range(warmup):
            plan.execute(ins, outs, N, stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            plan.execute(ins, outs, N, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        plan.status()
        return e0.elapsed_time(e1) * 1e-3 / iters

    def busbw(S, t):
        return S / t * 2 * (P - 1) / P / 1e9

    # ---- headline: tune, then warmup + timed steps ----------------------------------
    S = HEADLINE_BYTES
    N, ins, outs = inputs(S)
    t0 = time.perf_counter()
    if args.fixed:
        cfg = tuple(int(v) for v in args.fixed.split(","))
        cfg = cfg + (0,) * (4 - len(cfg))
        tune_evals = 0
    else:
        cfg, tune_evals = tune(N)
    tune_s = time.perf_counter() - t0
    plan = make_plan(N, *cfg)
    info = plan.info()
    plan_bytes = plan.bytes(N)
    for _ in range(args.warmup):
        plan.execute(ins, outs, N, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        plan.execute(ins, outs, N, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    plan.status()
    t_step = e0.elapsed_time(e1) * 1e-3 / args.steps
    # spot check of the timed output against the chain-order oracle
    from oracle import schedule_order as O2
    xs = [t.cpu().numpy() for t in ins]
    idx = np.random.default_rng(0).integers(0, N, 512)
    ok = bool(np.array_equal(outs[3].cpu().numpy()[idx], O2.ring_allreduce_at(xs, P, idx, "f32")))

    achieved = plan_bytes / t_step / 1e9
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "executor_ring_ar_8r_3mib_traffic.json")
    if os.path.exists(tpath):
        with open(tpath) as fh:
            tj = json.load(fh)
        if tj.get("source_digest") == source_digest() and tuple(tj.get("config", [])) == tuple(cfg):
            traffic = tj.get("bytes_per_launch")

    out = {
        "metric": "AllReduce busbw GB/s (8 virtual ranks, 1 GPU) and % of HBM peak",
        "value": round(busbw(S, t_step), 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: seeded fp32 N(0,1) per virtual rank",
        "config": {"workload": "ring AllReduce, 8 virtual ranks on one MI355X, fp32, 3 MiB per rank "
                               "(top of the 32 KiB-3 MiB sweep), one kernel launch per collective",
                   "ranks": P, "bytes_per_rank": S, "elements_per_rank": N,
                   "parallel_factor": cfg[0], "nthreads": cfg[1], "slice_bytes": cfg[2],
                   "protocol": "ll" if cfg[3] else "simple",
                   "scheduler": "hpds", "wg_alloc": "state", "workgroups": info["num_workgroups"],
                   "tuner_evaluations": tune_evals, "tune_seconds": round(tune_s, 2),
                   "compile_ms": round(sum(info["compile_ms"]), 3), "parallelism": "virtual ranks, 1 GPU"},
        "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
        "plan_bytes_per_launch": plan_bytes,
        "oracle_spot_check": ok,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
    }
    plan.destroy()
    del ins, outs

    if not args.no_extras:
        # ---- rest of the sweep and the large sizes, each tuned ----------------------
        sweep = []
        for Si in SWEEP + LARGE:
            Ni, ii, oo = inputs(Si)
            c, _ = tune(Ni)
            p = make_plan(Ni, *c)
            t = time_plan(p, Ni, ii, oo, 20 if Si >= (32 << 20) else 50)
            sweep.append({"bytes_per_rank": Si, "k": c[0], "nthreads": c[1], "slice_bytes": c[2],
                          "protocol": "ll" if c[3] else "simple",
                          "us": round(t * 1e6, 2), "busbw": round(busbw(Si, t), 2),
                          "hbm_frac": round(p.bytes(Ni) / t / 1e9 / HBM_PEAK_GBS, 4)})
            # tuned vs fixed configurations at the same size
            if Si in (1 << 20, 3 << 20, 32 << 20, 128 << 20):
                for name, (k, nt, sl) in (("fixed_k1_nt256_slice128k", (1, 256, min(128 << 10, Si // P))),
                                          ("fixed_k8_nt512_slice256k", (8, 512, 256 << 10))):
                    pf = make_plan(Ni, k, nt, sl)
                    tf = time_plan(pf, Ni, ii, oo, 10 if Si >= (32 << 20) else 30)
                    sweep[-1][name + "_busbw"] = round(busbw(Si, tf), 2)
                    pf.destroy()
            p.destroy()
            del ii, oo
            torch.cuda.empty_cache()
        out["sweep"] = sweep
        # ---- practical streaming ceiling: a plain copy kernel ------------------------
        nb = 1 << 28
        a = torch.empty(nb, dtype=torch.uint8, device=dev)
        b = torch.empty(nb, dtype=torch.uint8, device=dev)
        for _ in range(3):
            capi.ccl_copy_probe(b.data_ptr(), a.data_ptr(), nb, 1024, 512, stream.cuda_stream)
        e0.record(stream)
        for _ in range(10):
            capi.ccl_copy_probe(b.data_ptr(), a.data_ptr(), nb, 1024, 512, stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        tc = e0.elapsed_time(e1) * 1e-3 / 10
        out["copy_probe_GBs"] = round(2 * nb / tc / 1e9, 1)

    if args.copy_probe:
        nb = 1 << 28
        a = torch.zeros(nb, dtype=torch.uint8, device=dev)
        b = torch.empty(nb, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        for _ in range(args.copy_probe):
            capi.ccl_copy_probe(b.data_ptr(), a.data_ptr(), nb, 1024, 512, stream.cuda_stream)
        torch.cuda.synchronize()
        out["copy_probe_bytes_per_launch"] = 2 * nb

    # ---- CPU baseline: the oracle on the host, same workload, bounded time --------
    out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    out["source_digest"] = source_digest()
    print(json.dumps(out), flush=True)


def cpu_baseline(budget_s: float):
    """The chain-order oracle (numpy, one thread for elementwise adds) on the 3 MiB x 8
    rank input, repeated until the budget is spent."""
    import numpy as np

    import workloads as W
    from oracle import schedule_order as O2

    S = HEADLINE_BYTES
    N = S // 4
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=S)
    reps = 0
    t0 = time.perf_counter()
    while True:
        O2.ring_allreduce(xs, P, "f32")
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    t = (time.perf_counter() - t0) / reps
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"value": round(S / t * 2 * (P - 1) / P / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"schedule-order oracle, ring AllReduce 8 ranks x 3 MiB fp32, {reps} repetitions "
                      f"({t * 1e3:.1f} ms each); numpy elementwise adds run on one thread; host has {cores} cores"}


if __name__ == "__main__":
    main()
