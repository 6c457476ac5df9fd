"""Benchmark: ring AllReduce over 8 virtual ranks on one MI355X (busbw and HBM fraction).

Headline step: one 8-rank fp32 ring AllReduce of 3 MiB per rank (the top of the
32 KiB .. 3 MiB sweep), one kernel launch per collective, inputs resident in HBM,
with the parallelization factor (within the sweep's set 1..24), threads per workgroup,
slice size and protocol / transport chosen by the on-device coordinate-descent tuner.
Plan compilation and tuning happen before timing.

The last stdout line is one compact JSON object: the headline, its roofline against
8 TB/s, the same size at factor 32, a cold run over rotating buffer sets, two fixed
(untuned) configurations, the 32 and 256 MiB points (tuned; hot and cold, for the
>= 70 % target), one point of each of the other four configurations, the collective
beside GEMMs, and the CPU oracle's time. Everything else goes to the extras file
(default bench_results/extras.json); --extras (or --section NAME for one part) adds
the long sections: the sweep and its per-factor grid, 4/16/32 ranks, tree vs ring,
tuning under GEMM interference, kernel forms, the other four workloads over their
sizes, workgroup idle fractions and the plain-copy ceiling.

Only one GPU: --gpus above 1 exits with a message.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

P = 8
HEADLINE_BYTES = 3 << 20
SWEEP = [32 << 10, 64 << 10, 128 << 10, 256 << 10, 512 << 10, 1 << 20, 2 << 20, 3 << 20]
HBM_PEAK_GBS = 8000.0
# parallelization factors of the 8-rank ring sweep, 32 KiB to 3 MiB per rank (8 x factor chunks);
# larger sizes and other workloads also try 32, one workgroup per compute unit at 8 ranks
CONFIG_FACTORS = [1, 2, 4, 8, 16, 24]
TUNE_FACTORS = CONFIG_FACTORS + [32]
TUNE_THREADS = [64, 128, 256, 512, 1024]
TUNE_SLICES = [(4 << 10) << i for i in range(11)]  # 4 KiB ... 4 MiB
# tuner protocol ids: (protocol, transport, non-temporal local traffic)
PROTOCOLS = {0: ("simple", "staged", False), 1: ("ll", "staged", False), 2: ("simple", "direct", False),
             3: ("simple", "direct", True)}
# parts of the long measurements, in the order --extras runs them
EXTRA_SECTIONS = ["sweep", "sweep_k", "ranks", "trees", "interference", "kernels", "int4", "hier", "alltoall", "alltonext", "agrs",
                  "idle", "copy"]
DEVICE_INPUT_BYTES = 32 << 20  # at or above this many bytes per rank, inputs are drawn on the device
# executor kernels: the interpreting kernel, a kernel generated for the plan, and the
# generated kernel in the lazy (slice-outer) loop order
KERNELS = {0: "interpreter", 1: "specialized", 2: "lazy", 3: "specialized_loop"}
KERNEL = 1  # every workload runs kernels generated for its plans (compiled when the plan is created)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--fixed", type=str, default="",
                    help="k,nthreads,slice_bytes,protocol(0 simple, 1 LL, 2 simple+direct, 3 simple+direct+streaming)"
                         "[,kernel(0 interpreter, 1 specialized, 2 lazy; default 1)]: skip tuning (profiling runs)")
    ap.add_argument("--no-extras", action="store_true",
                    help="headline only: no cold, large-size or fixed-configuration rows (profiling runs)")
    ap.add_argument("--extras", action="store_true",
                    help="also run the long sections (the rest of the 8-rank sweep, 4/16/32 ranks, tree vs ring, "
                         "interference, kernel forms, the other four workloads, idle fractions, copy ceiling); "
                         "they go to the extras file only")
    ap.add_argument("--extras-file", type=str, default=os.path.join("bench_results", "extras.json"),
                    help="where the full results go (the last stdout line stays a compact summary)")
    ap.add_argument("--bytes", type=int, default=0,
                    help="per-rank size of the timed ring AllReduce instead of 3 MiB (profiling runs of other "
                         "sizes; implies --no-extras)")
    ap.add_argument("--section", choices=EXTRA_SECTIONS, default="",
                    help="after the headline run only this part of the long sections (--extras runs them all)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the oracle baseline")
    ap.add_argument("--no-interference", action="store_true",
                    help="leave out the summary's row of the 3 MiB collective beside GEMMs (shared GPU vs 64 reserved CUs)")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="also run the plain copy kernel this many times on 256 MiB (counter calibration)")
    ap.add_argument("--workload", choices=["ring_allreduce_8r"] + sorted(PROFILE_WORKLOADS),
                    default="ring_allreduce_8r",
                    help="profiling runs of another collective instead of the headline, in a fixed configuration "
                         "(--fixed, else the workload's default)")
    ap.add_argument("--sched", choices=["hpds", "rr", "program"], default="hpds", help="scheduler (--workload runs)")
    ap.add_argument("--alloc", choices=["state", "connection"], default="state",
                    help="workgroup allocation (--workload runs)")
    ap.add_argument("--trace", action="store_true",
                    help="--workload runs: also one traced launch (workgroup idle and link busy fractions)")
    return ap.parse_args()


def source_digest() -> str:
    h = hashlib.sha256()
    for f in ("executor.hip", "executor_device.h", "device_abi.h", "specialize.cpp", "compiler.cpp"):
        with open(os.path.join(ROOT, "chunk_schedule_execution_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def same_launch(a, b, piece_bytes):
    """Two (k, nthreads, slice_bytes, protocol, kernel) configurations run the same
    kernel work: equal apart from slice sizes that both cover the largest instruction
    piece, piece_bytes (one slice each)."""
    a, b = tuple(a), tuple(b)
    if len(a) != 5 or len(b) != 5 or (a[0], a[1], a[3], a[4]) != (b[0], b[1], b[3], b[4]):
        return False
    return a[2] == b[2] or (a[2] >= piece_bytes and b[2] >= piece_bytes)


def handoff_floor(capi, stream, piece, nthreads, ll, windows=(0,)):
    """Median microseconds of one forwarding and one reducing hand-off of `piece` bytes
    (a multiple of 16) by `nthreads`-thread workgroups, per window (0: lines still in
    the L2; else the hop probe's window, lines recent launches did not touch). Under LL
    the probe's times include the chain's first send and last plain store, so a hand-off
    is the difference of a 15-hop and a 1-hop chain."""
    out = {}
    for window in windows:
        for name, two in (("copy", False), ("reduce", True)):
            def med(hops):
                us, inf = capi.ccl_hop_probe(hops, piece, two, nthreads, 30, window_bytes=window,
                                             stream=stream.cuda_stream, ll=ll)
                if inf[1] or inf[2] or not us:
                    raise RuntimeError(f"hop probe failed: {inf}")
                return statistics.median(us)
            h = (15 * med(15) - med(1)) / 14 if ll else med(15)
            out[name + ("_cold" if window else "")] = round(h, 3)
    return out


def instance_bounds(lo, hi, k, align):
    """Bounds of the k instance pieces of the element range [lo, hi): lo plus floor(i (hi
    - lo) / k) rounded down to a multiple of align, and hi last (the rule the plan
    compiler lowers with)."""
    b = [lo]
    for i in range(1, k):
        f = i * (hi - lo) // k
        b.append(lo + f - f % align)
    return b + [hi]


def largest_piece(N, P, k, align=4):
    """Elements of the largest instruction piece of a ring AllReduce of N elements per
    rank over P ranks at factor k: P program chunks at floor(j N / P), each cut into k
    instance pieces (instance_bounds; align: elements per 16 bytes)."""
    best = 0
    for j in range(P):
        b = instance_bounds(j * N // P, (j + 1) * N // P, k, align)
        best = max(best, max(b[i + 1] - b[i] for i in range(k)))
    return best


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# Profiling workloads (--workload): (program factory, ranks, dtype, elements per rank input,
# output elements per rank, bus-bandwidth factor, default --fixed configuration, what it is)
N_BIG_24 = 24 * ((32 << 20) // 24)  # 33,554,424 fp32: the AllGather output, the ReduceScatter input
PROFILE_WORKLOADS = {
    "allgather_24r": ("ring_allgather", (24,), "f32", N_BIG_24 // 24, N_BIG_24, 23 / 24, "32,512,65536,3",
                      "ring AllGather, 24 virtual ranks, fp32, 128 MiB output per rank"),
    "reducescatter_24r": ("ring_reducescatter", (24,), "f32", N_BIG_24, N_BIG_24 // 24, 23 / 24, "32,512,65536,3",
                          "ring ReduceScatter, 24 virtual ranks, fp32, 128 MiB input per rank"),
    "allgather_2d_24r": ("allgather_2d", (3, 8), "f32", N_BIG_24 // 24, N_BIG_24, 23 / 24, "24,256,65536,3",
                         "2-D AllGather, 3 x 8 virtual ranks, fp32, 128 MiB output per rank"),
    "reducescatter_2d_24r": ("reducescatter_2d", (3, 8), "f32", N_BIG_24, N_BIG_24 // 24, 23 / 24, "24,256,65536,3",
                             "2-D ReduceScatter, 3 x 8 virtual ranks, fp32, 128 MiB input per rank"),
    "alltoall_32r": ("direct_alltoall", (32,), "i32", 1 << 22, 1 << 22, 31 / 32, "2,256,262144,3",
                     "direct AllToAll, 32 virtual ranks, int32, 16 MiB per rank"),
    "alltoall_two_phase_32r": ("two_phase_alltoall", (4, 8), "i32", 1 << 22, 1 << 22, 31 / 32, "1,256,262144,3",
                               "two-phase AllToAll, 4 x 8 virtual ranks, int32, 16 MiB per rank"),
    "alltonext_24r": ("alltonext", (3, 8, False), "f32", 1 << 24, 1 << 24, 1.0, "16,256,131072,3",
                      "AllToNext, 24 virtual ranks, fp32, 64 MiB per rank"),
    "alltonext_split_24r": ("alltonext", (3, 8, True), "f32", 1 << 24, 1 << 24, 1.0, "16,256,131072,3",
                            "split AllToNext, 3 x 8 virtual ranks, fp32, 64 MiB per rank"),
    "hier_ar_16r_bf16": ("hierarchical_allreduce", (2, 8), "bf16", 1 << 25, 1 << 25, 2 * 15 / 16, "32,256,131072,3",
                         "hierarchical AllReduce, 2 x 8 virtual ranks, bf16, 64 MiB per rank"),
    "tree_ar_24r": ("tree_allreduce", (24,), "f32", 1 << 18, 1 << 18, 2 * 23 / 24, "8,128,65536,2",
                    "tree AllReduce, 24 virtual ranks, fp32, 1 MiB per rank"),
}


def profile_collective(args) -> None:
    """One JSON line for one of PROFILE_WORKLOADS in a fixed configuration, timed with HIP
    events on the launch stream (profiling runs); with --trace also one traced launch:
    workgroup idle fractions and per-connection busy fractions from the device trace."""
    import torch

    import workloads as W
    from chunk_schedule_execution_amd import Plan, PlanConfig, capi, programs

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    factory, fargs, dtype, count, nout, busf, default_cfg, what = PROFILE_WORKLOADS[args.workload]
    prog = programs.REGISTRY[factory](*fargs)
    Pn = prog.nranks
    cfg = tuple(int(v) for v in (args.fixed or default_cfg).split(","))[:4]
    k, nt, sl, proto = cfg
    kind = {"f32": "normal_f32", "bf16": "normal_bf16", "i32": "uniform_i32"}[dtype]
    ii = W.device_inputs(kind, count, Pn, 6000 + len(args.workload), device=dev)
    tt = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}[dtype]
    oo = [torch.empty(nout, dtype=tt, device=dev) for _ in range(Pn)]

    def make(trace=False):
        return Plan(prog, k, PlanConfig(dtype=dtype, max_count=count, nthreads=nt, slice_bytes=sl,
                                        protocol=PROTOCOLS[proto][0], transport=PROTOCOLS[proto][1],
                                        streaming=PROTOCOLS[proto][2], kernel=KERNELS[KERNEL], scheduler=args.sched,
                                        wg_alloc=args.alloc, trace=trace))
    plan = make()
    for _ in range(args.warmup):
        plan.execute(ii, oo, count, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        plan.execute(ii, oo, count, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    plan.status()
    t = e0.elapsed_time(e1) * 1e-3 / args.steps
    pb = plan.bytes(count)
    esz = {"f32": 4, "bf16": 2, "i32": 4}[dtype]
    Sb = max(count, nout) * esz
    info = plan.info()
    out = {"workload": what, "config": list(cfg), "scheduler": args.sched, "wg_alloc": args.alloc,
           "workgroups": info["num_workgroups"], "steps": args.steps, "us_per_launch": round(t * 1e6, 2),
           "busbw": round(Sb / t * busf / 1e9, 2), "plan_bytes_per_launch": pb,
           "hbm_frac": round(pb / t / 1e9 / HBM_PEAK_GBS, 4), "dag_width": info["dag_width"],
           "dag_depth": info["dag_depth"], "source_digest": source_digest()}
    plan.destroy()
    if args.trace:
        tp = make(trace=True)
        for _ in range(3):
            tp.execute(ii, oo, count, stream)
        torch.cuda.synchronize()
        recs = [r for r in tp.trace() if r[3] > 0]
        t0 = min(r[0] for r in recs)
        span = max(r[1] for r in recs) - t0
        fr = sorted((r[2] + (r[0] - t0) + (t0 + span - r[1])) / span for r in recs)
        busy = sorted(b[4] for b in tp.link_busy())
        out["trace"] = {"span_us": round(span / 100.0, 2), "wg_idle_mean": round(sum(fr) / len(fr), 4),
                        "wg_idle_max": round(fr[-1], 4), "wg_idle_median": round(fr[len(fr) // 2], 4),
                        "connections": len(busy), "link_busy_mean": round(sum(busy) / max(1, len(busy)), 4),
                        "link_busy_min": round(busy[0], 4) if busy else None,
                        "link_busy_max": round(busy[-1], 4) if busy else None}
        tp.destroy()
    if args.copy_probe:
        nb = 1 << 28
        a = torch.zeros(nb, dtype=torch.uint8, device=dev)
        b = torch.empty(nb, dtype=torch.uint8, device=dev)
        for _ in range(args.copy_probe):
            capi.ccl_copy_probe(b.data_ptr(), a.data_ptr(), nb, 256, 256, stream.cuda_stream)
        torch.cuda.synchronize()
    print(json.dumps(out, separators=(",", ":")), flush=True)


def main():
    args = parse()
    if args.workload != "ring_allreduce_8r":
        if args.gpus != 1:
            print("bench.py runs on one GPU only", file=sys.stderr)
            sys.exit(2)
        profile_collective(args)
        return
    if args.bytes:
        args.no_extras = True
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the P ranks are virtual ranks "
              "sharing that GPU's memory, and there is no multi-GPU run", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W
    from chunk_schedule_execution_amd import Plan, PlanConfig, capi, programs

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}

    def device_inputs(kind, n, ranks, seed):
        return W.device_inputs({"f32": "normal_f32", "bf16": "normal_bf16", "i32": "uniform_i32"}[kind], n, ranks,
                               seed, device=dev)

    def ring_inputs(S, seed_offset=0):
        N = S // 4
        outs = [torch.empty(N, dtype=torch.float32, device=dev) for _ in range(P)]
        if S >= DEVICE_INPUT_BYTES or seed_offset:  # seeded N(0,1) drawn on the device
            return N, device_inputs("f32", N, P, 2026 * 1000 + S // (1 << 20) + 7919 * seed_offset), outs
        xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=S)
        return N, [torch.from_numpy(x).to(dev) for x in xs], outs

    def tune(prog, N, dtype="f32", protocols=15, variants=None, kernel=KERNEL, factors=TUNE_FACTORS, num_cus=0,
             on=None):
        """Tuned (k, nthreads, slice_bytes, protocol, kernel) of prog with the given
        executor kernel, or, given a list of programs as `variants`, the best over those
        algorithm subspaces with (..., variant index) appended. num_cus: a CU budget every
        candidate plan is sized to; on: the stream the candidates are timed on."""
        progs = variants if variants is not None else [prog]
        base = PlanConfig(dtype=dtype, max_count=N, kernel=KERNELS[kernel], num_cus=num_cus).to_c()
        arrs = [(capi.C.c_int32 * len(v))(*v) for v in (factors, TUNE_THREADS, TUNE_SLICES)]
        space = capi.ccl_tune_space(capi.C.cast(arrs[0], capi.C.POINTER(capi.C.c_int32)), len(factors),
                                    capi.C.cast(arrs[1], capi.C.POINTER(capi.C.c_int32)), len(TUNE_THREADS),
                                    capi.C.cast(arrs[2], capi.C.POINTER(capi.C.c_int32)), len(TUNE_SLICES),
                                    len(progs), 3, 10, protocols)
        best, rep = capi.ccl_tune([p.to_desc() for p in progs], N, base, space, (on or stream).cuda_stream)
        c = (best.parallel_factor, best.nthreads, best.slice_bytes, best.protocol, kernel)
        return (c + (best.variant,) if variants is not None else c), rep.evaluations

    def make_plan(prog, N, k, nt, sl, proto=0, kern=KERNEL, dtype="f32", **kw):
        return Plan(prog, k, PlanConfig(dtype=dtype, max_count=N, nthreads=nt, slice_bytes=sl,
                                        protocol=PROTOCOLS[proto][0], transport=PROTOCOLS[proto][1],
                                        streaming=PROTOCOLS[proto][2], kernel=KERNELS[kern], **kw))

    def time_launches(fn, iters, warmup=3):
        """Mean seconds per call of fn() (which enqueues work on `stream`), HIP events on `stream`."""
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / iters

    def busbw_ar(S, t, n=P):
        return S / t * 2 * (n - 1) / n / 1e9

    def frac(plan, N, t):
        return round(plan.bytes(N) / t / 1e9 / HBM_PEAK_GBS, 4)


    def stats(plan, N, t):
        return {"us": round(t * 1e6, 2), "plan_bytes": plan.bytes(N), "hbm_frac": frac(plan, N, t)}

    def release(*objs):
        for o in objs:
            if hasattr(o, "destroy"):
                o.destroy()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    def fitting(makers, ks=(8, 4, 2, 1)):
        """The largest parallelization factor at which every maker(k) builds a plan (all
        workgroups co-resident), with those plans; compared variants share it."""
        for k in ks:
            built = []
            try:
                for m in makers:
                    built.append(m(k))
                return k, built
            except capi.CCLError:
                release(*built)
        raise RuntimeError("no parallelization factor fits")

    def cold_time(plan, S, N, first_set, iters_per_set=4):
        """Mean seconds per launch while rotating over buffer sets whose total exceeds
        512 MiB (twice the Infinity Cache): every launch finds its buffers out of the caches."""
        set_bytes = 2 * P * S
        nsets = max(2, (512 << 20) // set_bytes + 1)
        sets = [first_set] + [ring_inputs(S, seed_offset=j)[1:] for j in range(1, nsets)]
        rot = [0]

        def call():
            i_, o_ = sets[rot[0] % nsets]
            rot[0] += 1
            plan.execute(i_, o_, N, stream)
        t = time_launches(call, iters_per_set * nsets, warmup=nsets)
        return t, nsets

    # ---- headline: tune, then warmup + timed steps ----------------------------------
    prog = programs.ring_allreduce(P)
    S = args.bytes or HEADLINE_BYTES
    N, ins, outs = ring_inputs(S)
    t0 = time.perf_counter()
    if args.fixed:
        cfg = tuple(int(v) for v in args.fixed.split(","))
        cfg = cfg + (0, 0, KERNEL)[len(cfg) - 2:] if len(cfg) < 5 else cfg
        tune_evals = 0
    else:
        cfg, tune_evals = tune(prog, N, kernel=KERNEL, factors=ring_factors(S))
    tune_s = time.perf_counter() - t0
    plan = make_plan(prog, N, *cfg)
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
    # per-launch spread from a separate, shorter pass (an event between launches costs time)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(51)]
    ev[0].record(stream)
    for i in range(50):
        plan.execute(ins, outs, N, stream)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(50))
    # a sample of the timed output, which the CPU baseline leg (the one part of this file
    # that runs the oracle) compares with the chain-order result on the same input
    sample_idx = np.random.default_rng(0).integers(0, N, 512)
    gpu_sample = outs[3].cpu().numpy()[sample_idx]

    achieved = plan_bytes / t_step / 1e9
    traffic = None
    tpath = os.path.join(ROOT, "profiles", f"executor_ring_ar_8r_{S >> 20}mib_traffic.json")
    if S % (1 << 20) == 0 and os.path.exists(tpath):
        with open(tpath) as fh:
            tj = json.load(fh)
        if tj.get("source_digest") == source_digest() and same_launch(tj.get("config", []), cfg, largest_piece(N, P, cfg[0]) * 4):
            traffic = tj.get("bytes_per_launch")
    floor_bytes = 2 * P * S  # every rank reads its input once and writes its output once

    size_txt = size_text(S)
    out = {
        "metric": "AllReduce busbw GB/s (8 virtual ranks, 1 GPU) and % of HBM peak",
        "value": round(busbw_ar(S, t_step), 2),
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
        "config": {"workload": f"ring AllReduce, 8 virtual ranks, fp32, {size_txt} per rank, one launch",
                   "k": cfg[0], "nthreads": cfg[1], "slice_bytes": cfg[2],
                   "transport": PROTOCOLS[cfg[3]][1] + ("+streaming" if PROTOCOLS[cfg[3]][2] else "")
                   + ("+ll" if PROTOCOLS[cfg[3]][0] == "ll" else ""), "kernel": KERNELS[cfg[4]],
                   "workgroups": info["num_workgroups"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
    }
    details = {"headline": {
        "bytes_per_rank": S, "elements_per_rank": N, "config": list(cfg),
        "protocol": PROTOCOLS[cfg[3]][0], "transport": PROTOCOLS[cfg[3]][1], "streaming": PROTOCOLS[cfg[3]][2],
        "xcd_local_stores": bool(info["xcd_local"]), "scheduler": "hpds", "wg_alloc": "state",
        "tuner_evaluations": tune_evals, "tune_seconds": round(tune_s, 2), "compile_ms": round(sum(info["compile_ms"]), 3),
        "plan_bytes_per_launch": plan_bytes, "floor_frac": round(floor_bytes / t_step / 1e9 / HBM_PEAK_GBS, 4),
        "us_per_launch": {"mean": round(t_step * 1e6, 2), "min_event_bracketed": round(per[0], 2),
                          "median_event_bracketed": round(statistics.median(per), 2)},
        }}
    progress(f"headline {t_step * 1e6:.2f} us per launch, config {cfg}")
    if PROTOCOLS[cfg[3]][0] == "simple" and S <= SWEEP[-1]:
        # The latency floor of this launch: a ring AllReduce is a chain of 2(P - 1)
        # dependent hand-offs, P - 1 reducing and P - 1 forwarding, the last of which
        # sets no flag. The hop probe times one hand-off of this launch's instruction
        # piece with the executor's own slice code, once over lines still in the L2
        # and once over lines recent launches did not touch (a 4 MiB window).
        piece = -(-largest_piece(N, P, cfg[0]) * 4 // 16) * 16
        hop = handoff_floor(capi, stream, piece, cfg[1], False, windows=(0, 4 << 20))
        chain = (P - 1) * hop["reduce"] + (P - 2) * hop["copy"]
        chain_cold = (P - 1) * hop["reduce_cold"] + (P - 2) * hop["copy_cold"]
        out["latency_floor"] = {"piece_bytes": piece, "hop_us": hop, "chain_us": round(chain, 2),
                                "chain_cold_us": round(chain_cold, 2), "frac": round(chain / (t_step * 1e6), 4),
                                "frac_cold": round(chain_cold / (t_step * 1e6), 4)}
        progress(f"hand-off floor {hop} us: chain {chain:.1f} / {chain_cold:.1f} us of {t_step * 1e6:.1f}")

    if not args.no_extras:
        # cold headline: rotate over buffer sets larger than the Infinity Cache
        t_cold, nsets = cold_time(plan, S, N, (ins, outs))
        out["cold"] = {"us": round(t_cold * 1e6, 2), "busbw": round(busbw_ar(S, t_cold), 2),
                       "frac": frac(plan, N, t_cold)}
        details["headline"]["cold_buffer_sets"] = nsets
        # tuned versus two fixed configurations (same kernel form) at the headline size
        fixed = {}
        for name, (k, nt, sl) in (("k1_nt256_128k", (1, 256, min(128 << 10, S // P))), ("k8_nt512_256k", (8, 512, 256 << 10))):
            pf = make_plan(prog, N, k, nt, sl, 0, cfg[4])
            fixed[name] = round(busbw_ar(S, time_launches(lambda: pf.execute(ins, outs, N, stream), 30)), 2)
            release(pf)
        out["fixed_busbw"] = fixed
        if S <= SWEEP[-1]:
            # the same size at factor 32 (256 workgroups), outside the sweep's factor set
            c32, _ = tune(prog, N, kernel=KERNEL, factors=[32])
            p32 = make_plan(prog, N, *c32)
            t32 = time_launches(lambda: p32.execute(ins, outs, N, stream), args.steps)
            out["factor_32"] = {"nt": c32[1], "us": round(t32 * 1e6, 2), "busbw": round(busbw_ar(S, t32), 2),
                                "frac": frac(p32, N, t32)}
            release(p32)
    release(plan)
    del ins, outs

    if not args.no_extras:
        # the >= 70 % target sizes: tuned, hot (buffers reused) and cold (rotating sets)
        large = []
        for SL in (32 << 20, 256 << 20):
            NL, ii, oo = ring_inputs(SL)
            c, ev_ = tune(prog, NL, kernel=KERNEL, factors=ring_factors(SL))
            pl = make_plan(prog, NL, *c)
            t_hot = time_launches(lambda: pl.execute(ii, oo, NL, stream), 20)
            t_c, nsets = cold_time(pl, SL, NL, (ii, oo), iters_per_set=4 if SL < (256 << 20) else 5)
            row = {"MiB": SL >> 20, "k": c[0], "nt": c[1], "slice": c[2], "proto": c[3],
                   "hot_frac": frac(pl, NL, t_hot), "cold_frac": frac(pl, NL, t_c),
                   "cold_busbw": round(busbw_ar(SL, t_c), 1)}
            if SL == 32 << 20:
                for name, (k, nt, sl) in (("k1_nt256_128k", (1, 256, 128 << 10)), ("k8_nt512_256k", (8, 512, 256 << 10))):
                    pf = make_plan(prog, NL, k, nt, sl, 0, c[4])
                    row["fixed_" + name + "_busbw"] = round(
                        busbw_ar(SL, time_launches(lambda: pf.execute(ii, oo, NL, stream), 5)), 1)
                    release(pf)
            details.setdefault("large", []).append(dict(row, hot_us=round(t_hot * 1e6, 2), cold_us=round(t_c * 1e6, 2),
                                                        cold_buffer_sets=nsets, tuner_evaluations=ev_,
                                                        plan_bytes=pl.bytes(NL)))
            large.append(row)
            progress(f"ring AR 8 ranks {SL >> 20} MiB: hot {t_hot * 1e6:.1f} us, cold {t_c * 1e6:.1f} us")
            release(pl)
            del ii, oo
            torch.cuda.empty_cache()
        out["large"] = large
        out["target_70pct_cold_at_32mib_and_up"] = all(r["cold_frac"] >= 0.70 for r in large)
        # one point of each of the other configurations
        try:
            out["configs"] = config_rows(torch, W, programs, dev, stream, device_inputs, make_plan, time_launches,
                                         release)
        except Exception as e:  # reported, never fatal to the summary line
            out["configs"] = {"error": str(e)[:160]}
            release()
        progress(f"configurations: {out['configs']}")
        if not args.no_interference:
            # the collective beside GEMMs: shared GPU vs reserved compute units
            try:
                out["beside_gemms"] = interference_row(torch, dev, stream, prog, cfg, ring_inputs, tune, make_plan,
                                                       release)
                progress(f"beside GEMMs: {out['beside_gemms']}")
            except Exception as e:  # reported, never fatal to the summary line
                out["beside_gemms"] = {"error": str(e)[:160]}

    if args.section or args.extras:
        details.update(extras(np, torch, W, Plan, PlanConfig, capi, programs, dev, stream, ring_inputs,
                              device_inputs, tune, make_plan, time_launches, busbw_ar, stats, release, fitting,
                              sections={args.section} if args.section else None))

    if args.copy_probe:
        nb = 1 << 28
        a = torch.zeros(nb, dtype=torch.uint8, device=dev)
        b = torch.empty(nb, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        for _ in range(args.copy_probe):
            capi.ccl_copy_probe(b.data_ptr(), a.data_ptr(), nb, 256, 256, stream.cuda_stream)
        torch.cuda.synchronize()
        details["copy_probe_bytes_per_launch"] = 2 * nb
        del a, b

    # ---- CPU baseline: the oracle on the host, same workload, bounded time --------
    # (above DEVICE_INPUT_BYTES the GPU's inputs are drawn on the device, not the oracle's)
    out["cpu_baseline"], ok = cpu_baseline(args.cpu_seconds, S,
                                           (sample_idx, gpu_sample) if S < DEVICE_INPUT_BYTES else None)
    details["headline"]["oracle_spot_check"] = ok
    progress(f"headline output sample against the chain-order oracle: {ok}")
    out["extras_file"] = args.extras_file
    out["source_digest"] = source_digest()
    torch.cuda.synchronize()
    details["summary"] = out
    try:
        os.makedirs(os.path.dirname(os.path.abspath(args.extras_file)), exist_ok=True)
        with open(args.extras_file, "w") as fh:
            json.dump(details, fh, indent=1)
    except OSError as e:
        progress(f"could not write {args.extras_file}: {e}")
    reap_children()
    print(json.dumps(out, separators=(",", ":")), flush=True)


# Launch configurations of the one-point rows for the other configurations in the summary
# line: (parallel factor, threads, slice bytes, protocol id), each the tuned point of the
# matching --section run (hier, alltoall, alltonext, agrs) and each with a GPU parity test
# at that configuration.
CONFIG_POINTS = {
    "hier_fused": (32, 256, 256 << 10, 3),
    "hier_stages": ((32, 512, 64 << 10, 3), (16, 512, 1 << 20, 2), (32, 256, 128 << 10, 3)),
    "a2a_two_phase": (1, 256, 256 << 10, 3),
    "a2a_direct": (2, 256, 256 << 10, 3),
    "a2next": (16, 256, 128 << 10, 3),
    "agrs_ring": (32, 512, 64 << 10, 3),
}


def config_rows(torch, W, programs, dev, stream, device_inputs, make_plan, time_launches, release):
    """One point of each of the other four configurations, at fixed launch settings
    (CONFIG_POINTS): the 4-rank exact-sum ring, the 16-rank bf16 hierarchical AllReduce
    fused and as three launches, the 32-rank int32 AllToAll two-phase and direct, the
    24-rank AllToNext split (both schedulers) and unsplit, and the 24-rank ring
    AllGather / ReduceScatter at 128 MiB."""
    import numpy as np
    out = {}

    def frac(plan, n, t):
        return round(plan.bytes(n) / t / 1e9 / HBM_PEAK_GBS, 4)

    # 4 ranks, 1 MiB integer-valued fp32, 4 chunks, one channel, one slice
    N = 262144
    xs = W.make_inputs("int_f32", N, 4, W.CFG_RING_AR_4R_INT, size_bytes=N * 4)
    ii = [torch.from_numpy(x).to(dev) for x in xs]
    oo = [torch.empty(N, device=dev) for _ in range(4)]
    p = make_plan(programs.ring_allreduce(4), N, 1, 512, N * 4)
    t = time_launches(lambda: p.execute(ii, oo, N, stream), 50)
    exact = bool(np.array_equal(oo[0].cpu().numpy(), np.sum(np.stack(xs).astype(np.float64), 0).astype(np.float32)))
    out["ring_4r_1mib_int"] = {"us": round(t * 1e6, 1), "exact": exact}
    release(p)
    del ii, oo
    # 16 ranks (2 x 8) bf16, 16 MiB: fused vs three launches
    G, L = 2, 8
    N = (16 << 20) // 2
    sh = N // L
    ii = device_inputs("bf16", N, G * L, 3016)
    oo = [torch.empty(N, dtype=torch.bfloat16, device=dev) for _ in range(G * L)]
    mid1 = [torch.empty(sh, dtype=torch.bfloat16, device=dev) for _ in range(G * L)]
    mid2 = [torch.empty(sh, dtype=torch.bfloat16, device=dev) for _ in range(G * L)]
    pf = make_plan(programs.hierarchical_allreduce(G, L), N, *CONFIG_POINTS["hier_fused"], dtype="bf16")
    c1, c2, c3 = CONFIG_POINTS["hier_stages"]
    s1 = make_plan(programs.hier_stage_reducescatter_intra(G, L), N, *c1, dtype="bf16")
    s2 = make_plan(programs.hier_stage_allreduce_inter(G, L), sh, *c2, dtype="bf16")
    s3 = make_plan(programs.hier_stage_allgather_intra(G, L), sh, *c3, dtype="bf16")
    tf = time_launches(lambda: pf.execute(ii, oo, N, stream), 20)

    def three():
        s1.execute(ii, mid1, N, stream)
        s2.execute(mid1, mid2, sh, stream)
        s3.execute(mid2, oo, sh, stream)
    t3 = time_launches(three, 20)
    out["hier_16r_16mib_bf16"] = {"fused_us": round(tf * 1e6, 1), "three_launch_us": round(t3 * 1e6, 1),
                                  "fused_frac": frac(pf, N, tf)}
    release(pf, s1, s2, s3)
    del ii, oo, mid1, mid2
    # 32 ranks (4 x 8) int32, 16 MiB: two-phase vs direct
    G, L = 4, 8
    N = (16 << 20) // 4
    ii = device_inputs("i32", N, G * L, 4016)
    oo = [torch.empty(N, dtype=torch.int32, device=dev) for _ in range(G * L)]
    row = {}
    for name, prog in (("two_phase", programs.two_phase_alltoall(G, L)), ("direct", programs.direct_alltoall(G * L))):
        p = make_plan(prog, N, *CONFIG_POINTS["a2a_" + name], dtype="i32")
        t = time_launches(lambda: p.execute(ii, oo, N, stream), 20)
        row[name + "_us"], row[name + "_frac"] = round(t * 1e6, 1), frac(p, N, t)
        release(p)
    out["a2a_32r_16mib_i32"] = row
    del ii, oo
    release()
    # 24 ranks (3 x 8): AllToNext at 64 MiB, ring AllGather / ReduceScatter at 128 MiB
    G, L = 3, 8
    Pn = G * L
    N = (64 << 20) // 4
    ii = device_inputs("f32", N, Pn, 5064)
    oo = [torch.empty(N, device=dev) for _ in range(Pn)]
    row = {}
    for name, split, sched, alloc in (("split_hpds_state", True, "hpds", "state"),
                                      ("split_rr_connection", True, "rr", "connection"),
                                      ("unsplit", False, "hpds", "state")):
        p = make_plan(programs.alltonext(G, L, split=split), N, *CONFIG_POINTS["a2next"], scheduler=sched,
                      wg_alloc=alloc)
        t = time_launches(lambda: p.execute(ii, oo, N, stream), 10)
        row[name + "_us"] = round(t * 1e6, 1)
        release(p)
    out["a2next_24r_64mib"] = row
    del ii, oo
    release()
    n_big = Pn * ((32 << 20) // Pn)
    row = {}
    for coll in ("allgather", "reducescatter"):
        if coll == "allgather":
            prog, count, nout = programs.ring_allgather(Pn), n_big // Pn, n_big
        else:
            prog, count, nout = programs.ring_reducescatter(Pn), n_big, n_big // Pn
        ii = device_inputs("f32", count, Pn, 6000 + len(coll))
        oo = [torch.empty(nout, device=dev) for _ in range(Pn)]
        p = make_plan(prog, count, *CONFIG_POINTS["agrs_ring"])
        t = time_launches(lambda: p.execute(ii, oo, count, stream), 5)
        row[("ag" if coll == "allgather" else "rs") + "_frac"] = frac(p, count, t)
        release(p)
        del ii, oo
        release()
    out["agrs_24r_128mib_ring"] = row
    return out


def ring_factors(S):
    """Parallelization factors the 8-rank ring AllReduce is tuned over at S bytes per rank:
    the sweep's set up to 3 MiB; above it also 32, and 48 and 64, which put two
    workgroups on a compute unit so that one streams while the other waits for a flag
    (256 MiB: 73.4 % of 8 TB/s at k = 64 x 512 threads against 72.5 % at k = 32 x 1024)."""
    return CONFIG_FACTORS if S <= SWEEP[-1] else TUNE_FACTORS + [48, 64]


def reap_children():
    """Leave no process behind: name any child this run started (the runtime compiler
    or a library may), then end it."""
    try:
        import psutil
    except ImportError:
        return
    kids = psutil.Process().children(recursive=True)
    for k in kids:
        try:
            progress(f"child process left: pid {k.pid} {' '.join(k.cmdline())[:200]}")
            k.terminate()
        except psutil.Error:
            pass
    psutil.wait_procs(kids, timeout=5)


def extras(np, torch, W, Plan, PlanConfig, capi, programs, dev, stream, ring_inputs, device_inputs, tune, make_plan,
           time_launches, busbw_ar, stats, release, fitting, sections=None):
    """The long measurements, by section (all of them when sections is None)."""
    res = {}

    def section_on(name):
        return sections is None or name in sections

    prog = programs.ring_allreduce(P)

    if section_on("sweep"):
        # ---- the rest of the 8-rank sweep and the large sizes, each tuned ---------------
        sweep = []
        for S in SWEEP + [128 << 20]:
            N, ii, oo = ring_inputs(S)
            c, _ = tune(prog, N, kernel=KERNEL, factors=ring_factors(S))
            p = make_plan(prog, N, *c)
            t = time_launches(lambda: p.execute(ii, oo, N, stream), 20 if S >= DEVICE_INPUT_BYTES else 50)
            row = {"bytes_per_rank": S, "k": c[0], "nthreads": c[1], "slice_bytes": c[2],
                   "protocol": PROTOCOLS[c[3]][0], "transport": PROTOCOLS[c[3]][1], "streaming": PROTOCOLS[c[3]][2],
                   "kernel": KERNELS[c[4]], "busbw": round(busbw_ar(S, t), 2), **stats(p, N, t)}
            if S <= SWEEP[-1]:
                # the hand-off floor of this pick's chain: P - 1 reducing and P - 2 forwarding
                # hand-offs of its largest piece, over lines still in the L2
                hf = handoff_floor(capi, stream, -(-largest_piece(N, P, c[0]) * 4 // 16) * 16, c[1],
                                   PROTOCOLS[c[3]][0] == "ll")
                chain = (P - 1) * hf["reduce"] + (P - 2) * hf["copy"]
                row["handoff_us"] = hf
                row["chain_floor_us"] = round(chain, 2)
                row["chain_floor_frac"] = round(chain / row["us"], 4)
            if S in (1 << 20, 3 << 20, 32 << 20, 128 << 20):  # tuned versus fixed configurations
                for name, (k, nt, sl) in (("fixed_k1_nt256_slice128k", (1, 256, min(128 << 10, S // P))),
                                          ("fixed_k8_nt512_slice256k", (8, 512, 256 << 10))):
                    pf = make_plan(prog, N, k, nt, sl, 0, c[4])  # the tuned point's kernel
                    tf = time_launches(lambda: pf.execute(ii, oo, N, stream), 10 if S >= DEVICE_INPUT_BYTES else 30)
                    row[name + "_busbw"] = round(busbw_ar(S, tf), 2)
                    release(pf)
            sweep.append(row)
            progress(f"ring AR 8 ranks {S >> 10} KiB: {row['us']} us" +
                     (f", hand-off chain floor {row['chain_floor_us']} us" if "chain_floor_us" in row else ""))
            release(p)
            del ii, oo
        res["sweep"] = sweep

    if section_on("sweep_k"):
        # every (size, parallelization factor) pair of the 8-rank ring sweep, with threads,
        # slice size and protocol tuned at that factor
        grid = []
        for S in SWEEP:
            N, ii, oo = ring_inputs(S)
            for k in CONFIG_FACTORS:
                c, _ = tune(prog, N, kernel=KERNEL, factors=[k])
                p = make_plan(prog, N, *c)
                t = time_launches(lambda: p.execute(ii, oo, N, stream), 50)
                grid.append({"bytes_per_rank": S, "k": k, "nthreads": c[1], "slice_bytes": c[2],
                             "protocol": PROTOCOLS[c[3]][0], "transport": PROTOCOLS[c[3]][1],
                             "busbw": round(busbw_ar(S, t), 2), **stats(p, N, t)})
                release(p)
            progress(f"ring AR 8 ranks {S >> 10} KiB by factor: " +
                     ", ".join(f"k={r['k']} {r['us']} us" for r in grid if r["bytes_per_rank"] == S))
            del ii, oo
        res["sweep_by_factor"] = grid

    if section_on("ranks"):
        res["ring_ar_rank_counts"] = rank_counts(np, torch, programs, dev, stream, device_inputs, tune, make_plan,
                                                 time_launches, busbw_ar, stats, release)

    if section_on("trees"):
        # ---- tree versus ring AllReduce at small sizes, and the tuner choosing -----------
        trees = []
        for R, S in ((8, 64 << 10), (8, 256 << 10), (8, 1 << 20), (8, 3 << 20), (24, 1 << 20)):
            N = S // 4
            ii = device_inputs("f32", N, R, 77000 + R * 64 + S // 65536)
            oo = [torch.empty(N, device=dev) for _ in range(R)]
            ring, tree = programs.ring_allreduce(R), programs.tree_allreduce(R)
            row = {"ranks": R, "bytes_per_rank": S}
            for name, pr in (("ring", ring), ("tree", tree)):
                c, _ = tune(pr, N)
                p = make_plan(pr, N, *c)
                t = time_launches(lambda: p.execute(ii, oo, N, stream), 50)
                row[name] = {"k": c[0], "nthreads": c[1], "slice_bytes": c[2], "protocol": PROTOCOLS[c[3]][0],
                             "transport": PROTOCOLS[c[3]][1], "busbw": round(busbw_ar(S, t, R), 2), **stats(p, N, t)}
                release(p)
            c, ev = tune(None, N, variants=[ring, tree])
            row["tuner_picks"] = ("ring", "tree")[c[5]]
            row["tuner_evaluations"] = ev
            trees.append(row)
            progress(f"tree vs ring {R} ranks {S >> 10} KiB: {row['tree']['us']} vs {row['ring']['us']} us")
            del ii, oo
        res["tree_vs_ring"] = trees

    if section_on("interference"):
        # ---- tuning under compute interference: bf16 GEMMs on a second stream ----------
        res["interference"] = interference(torch, dev, stream, prog, ring_inputs, tune, make_plan, busbw_ar, release)
        progress("interference done")

    if section_on("kernels"):
        # ---- interpreting vs generated kernels, and the lazy loop order ------------------
        res["kernels"] = kernels(prog, ring_inputs, make_plan, time_launches, release, stream)
        res["kernels_other"] = kernels_other(programs, device_inputs, make_plan, time_launches, release, stream, torch, dev)

    if section_on("int4"):
        # ---- 4 ranks, 1 MiB integer-valued fp32, 4 chunks, one channel, one slice -------
        N = 262144
        xs = W.make_inputs("int_f32", N, 4, W.CFG_RING_AR_4R_INT, size_bytes=N * 4)
        ii = [torch.from_numpy(x).to(dev) for x in xs]
        oo = [torch.empty(N, device=dev) for _ in range(4)]
        p4 = make_plan(programs.ring_allreduce(4), N, 1, 512, N * 4)
        t = time_launches(lambda: p4.execute(ii, oo, N, stream), 100)
        exact = bool(np.array_equal(oo[0].cpu().numpy(), np.sum(np.stack(xs).astype(np.float64), 0).astype(np.float32)))
        res["ring_ar_4r_1mib_int"] = {"busbw": round(busbw_ar(N * 4, t, 4), 2), "exact": exact, **stats(p4, N, t)}
        release(p4)
        del ii, oo

    if section_on("hier"):
        # ---- 16 ranks (2 x 8) bf16 hierarchical AllReduce: fused vs three launches -----
        G, L = 2, 8
        hier = []
        fused_prog = programs.hierarchical_allreduce(G, L)
        stages = (programs.hier_stage_reducescatter_intra(G, L), programs.hier_stage_allreduce_inter(G, L),
                  programs.hier_stage_allgather_intra(G, L))
        for S in [(1 << 20) << i for i in range(9)]:  # 1 MiB ... 256 MiB
            N = S // 2
            ii = device_inputs("bf16", N, G * L, 3000 + S // (1 << 20))
            oo = [torch.empty(N, dtype=torch.bfloat16, device=dev) for _ in range(G * L)]
            cf, _ = tune(fused_prog, N, "bf16")
            pf = make_plan(fused_prog, N, *cf, dtype="bf16")
            tf = time_launches(lambda: pf.execute(ii, oo, N, stream), 10)
            sh = N // L
            mid1 = [torch.empty(sh, dtype=torch.bfloat16, device=dev) for _ in range(G * L)]
            mid2 = [torch.empty(sh, dtype=torch.bfloat16, device=dev) for _ in range(G * L)]
            c1, _ = tune(stages[0], N, "bf16")
            c2, _ = tune(stages[1], sh, "bf16")
            c3, _ = tune(stages[2], sh, "bf16")
            s1 = make_plan(stages[0], N, *c1, dtype="bf16")
            s2 = make_plan(stages[1], sh, *c2, dtype="bf16")
            s3 = make_plan(stages[2], sh, *c3, dtype="bf16")

            def three():
                s1.execute(ii, mid1, N, stream)
                s2.execute(mid1, mid2, sh, stream)
                s3.execute(mid2, oo, sh, stream)
            t3 = time_launches(three, 10)
            row = {"bytes_per_rank": S, "fused_config": list(cf), "stage_configs": [list(c1), list(c2), list(c3)],
                   "fused_us": round(tf * 1e6, 2), "three_launch_us": round(t3 * 1e6, 2),
                   "fused_busbw": round(busbw_ar(S, tf, G * L), 2), "three_launch_busbw": round(busbw_ar(S, t3, G * L), 2),
                   "speedup": round(t3 / tf, 3), "fused_hbm_frac": stats(pf, N, tf)["hbm_frac"],
                   "fused_workgroups": pf.info()["num_workgroups"]}
            release(pf, s1, s2, s3)
            hier.append(row)
            progress(f"hierarchical AllReduce {S >> 20} MiB: fused {row['fused_us']} us, three launches "
                     f"{row['three_launch_us']} us")
            del ii, oo, mid1, mid2
        res["hier_ar_16r_bf16"] = hier
        progress("hierarchical AllReduce done")

    if section_on("alltoall"):
        # ---- 32 ranks (4 x 8) int32 AllToAll: two-phase vs direct ----------------------
        G, L = 4, 8
        Pa = G * L
        a2a = []
        for S in [(1 << 20) << i for i in range(7)]:  # 1 MiB ... 64 MiB
            N = S // 4
            ii = device_inputs("i32", N, Pa, 4000 + S // (1 << 20))
            oo = [torch.empty(N, dtype=torch.int32, device=dev) for _ in range(Pa)]
            row = {"bytes_per_rank": S}
            for name, pr in (("two_phase", programs.two_phase_alltoall(G, L)), ("direct", programs.direct_alltoall(Pa))):
                best = None
                # direct transport, with and without the streaming variant (whose copies keep
                # eight vectors per thread in flight)
                for k, nt, proto in ((1, 256, 2), (2, 256, 2), (2, 128, 2), (4, 128, 2), (1, 256, 3), (2, 256, 3)):
                    try:
                        pl = make_plan(pr, N, k, nt, 256 << 10, proto, dtype="i32")
                    except capi.CCLError:
                        continue  # more workgroups than fit at once
                    t = time_launches(lambda: pl.execute(ii, oo, N, stream), 10)
                    if best is None or t < best[0]:
                        best = (t, k, nt, PROTOCOLS[proto][2], pl.info()["num_workgroups"], stats(pl, N, t)["hbm_frac"])
                    release(pl)
                if best:
                    t, k, nt, streaming, nwg, hf = best
                    row[name] = {"us": round(t * 1e6, 2), "k": k, "nthreads": nt, "streaming": streaming,
                                 "workgroups": nwg, "hbm_frac": hf, "busbw": round(S / t * (Pa - 1) / Pa / 1e9, 2)}
                    if name == "two_phase":
                        # with k > 1 every operation is split per chunk, so the phase-2 transfer of
                        # a gather region becomes one transfer per block instead of one batch
                        row[name]["phase2_batched"] = k == 1
            a2a.append(row)
            progress(f"AllToAll {S >> 20} MiB: " + ", ".join(f"{m} {row[m]['us']} us" for m in ("two_phase", "direct")
                                                               if m in row))
            del ii, oo
            release()
        res["alltoall_32r_int32"] = a2a
        progress("AllToAll done")

    if section_on("alltonext"):
        # ---- 24 ranks (3 x 8): AllToNext split / unsplit, HPDS+state vs RR+connection ---
        G, L = 3, 8
        Pn = G * L
        a2n = []
        for S in (16 << 20, 32 << 20, 64 << 20, 128 << 20):
            N = S // 4
            ii = device_inputs("f32", N, Pn, 5000 + S // (1 << 20))
            oo = [torch.empty(N, device=dev) for _ in range(Pn)]
            row = {"bytes_per_rank": S}
            for split in (True, False):
                modes = (("hpds", "state"), ("rr", "connection"))
                # one launch configuration for both modes (256 threads, 128 KiB slices, direct
                # transport with streaming hints: the best of a sweep at 64 MiB, where 256
                # threads let the split program's 1120-1248 workgroups of k = 16 fit at once)
                k, pls = fitting([lambda k, sc=sc, al=al: make_plan(programs.alltonext(G, L, split=split), N, k, 256,
                                                                      128 << 10, 3, scheduler=sc, wg_alloc=al)
                                  for sc, al in modes], ks=(16, 8, 4, 2, 1))
                for (sched, alloc), pl in zip(modes, pls):
                    t = time_launches(lambda: pl.execute(ii, oo, N, stream), 10)
                    row[f"{'split' if split else 'unsplit'}_{sched}_{alloc}"] = {
                        "us": round(t * 1e6, 2), "algbw": round(S / t / 1e9, 2), "k": k,
                        "workgroups": pl.info()["num_workgroups"], "hbm_frac": stats(pl, N, t)["hbm_frac"]}
                release(*pls)
            a2n.append(row)
            progress(f"AllToNext {S >> 20} MiB done")
            del ii, oo
            release()
        res["alltonext_24r"] = a2n
        progress("AllToNext done")

    if section_on("agrs"):
        G, L = 3, 8
        Pn = G * L
        # AllGather / ReduceScatter on the same 24 ranks, 128 MiB (the larger buffer)
        n_big = Pn * ((32 << 20) // Pn)  # 33,554,424 fp32
        agrs = {}
        for coll in ("allgather", "reducescatter"):
            for variant in ("ring", "2d"):
                if coll == "allgather":
                    pr = programs.ring_allgather(Pn) if variant == "ring" else programs.allgather_2d(G, L)
                    count, nout = n_big // Pn, n_big
                else:
                    pr = programs.ring_reducescatter(Pn) if variant == "ring" else programs.reducescatter_2d(G, L)
                    count, nout = n_big, n_big // Pn
                ii = device_inputs("f32", count, Pn, 6000 + len(coll))
                oo = [torch.empty(nout, device=dev) for _ in range(Pn)]
                modes = (("hpds", "state"), ("rr", "connection"))
                Sb = n_big * 4
                if variant == "ring":
                    # one launch configuration for both modes (512 threads, 64 KiB slices, direct
                    # transport with streaming hints: the best of a sweep of the ring at this size)
                    k, pls = fitting([lambda k, sc=sc, al=al: make_plan(pr, count, k, 512, 64 << 10, 3, scheduler=sc,
                                                                          wg_alloc=al) for sc, al in modes],
                                     ks=(32, 16, 8, 4, 2, 1))
                    for (sched, alloc), pl in zip(modes, pls):
                        t = time_launches(lambda: pl.execute(ii, oo, count, stream), 5)
                        agrs[f"{coll}_{variant}_{sched}_{alloc}"] = {
                            "us": round(t * 1e6, 2), "busbw": round(Sb / t * (Pn - 1) / Pn / 1e9, 2), "k": k,
                            "workgroups": pl.info()["num_workgroups"], "hbm_frac": stats(pl, count, t)["hbm_frac"]}
                    release(*pls)
                else:
                    # each mode at its best point of one small sweep: state-based allocation needs
                    # half the workgroups, so it reaches channel counts whose connection-based
                    # grid would not fit on the device at once
                    for sched, alloc in modes:
                        best = None
                        for k, nt in ((4, 512), (8, 512), (8, 256), (16, 256), (16, 128), (24, 256), (32, 128)):
                            try:
                                pl = make_plan(pr, count, k, nt, 64 << 10, 3, scheduler=sched, wg_alloc=alloc)
                            except capi.CCLError:
                                continue  # more workgroups than fit at once
                            t = time_launches(lambda: pl.execute(ii, oo, count, stream), 5)
                            if best is None or t < best[0]:
                                best = (t, k, nt, pl.info()["num_workgroups"], stats(pl, count, t)["hbm_frac"])
                            release(pl)
                        t, k, nt, nwg, hf = best
                        agrs[f"{coll}_{variant}_{sched}_{alloc}"] = {
                            "us": round(t * 1e6, 2), "busbw": round(Sb / t * (Pn - 1) / Pn / 1e9, 2), "k": k,
                            "nthreads": nt, "workgroups": nwg, "hbm_frac": hf}
                del ii, oo
                release()
        res["allgather_reducescatter_24r_128mib"] = agrs
        progress("AllGather / ReduceScatter done")

    if section_on("idle"):
        G, L = 3, 8
        Pn = G * L
        # ---- workgroup idle fraction from the device trace (one traced launch) ----------
        def idle(pr, N, dtype, k, nt, sl, proto, kern, ii, oo, **kw):
            k, (pl,) = fitting([lambda kk: make_plan(pr, N, kk, nt, sl, proto, kern, dtype=dtype, trace=True, **kw)],
                               ks=[x for x in (k, 8, 4, 2, 1) if x <= k])
            for _ in range(3):
                pl.execute(ii, oo, N, stream)
            torch.cuda.synchronize()
            recs = [r for r in pl.trace() if r[3] > 0]
            t0 = min(r[0] for r in recs)
            span = max(r[1] for r in recs) - t0
            # waiting on flags, plus the time a workgroup is not yet started or already done
            fr = [(r[2] + (r[0] - t0) + (t0 + span - r[1])) / span for r in recs]
            out = {"workgroups": len(recs), "k": k, "mean": round(float(np.mean(fr)), 4),
                   "max": round(float(np.max(fr)), 4)}
            release(pl)
            return out

        N, ii, oo = ring_inputs(HEADLINE_BYTES)
        c, _ = tune(prog, N, kernel=KERNEL, factors=ring_factors(HEADLINE_BYTES))
        idle_rows = {"ring_ar_8r_3mib_tuned": idle(prog, N, "f32", *c, ii, oo)}
        del ii, oo
        N = (64 << 20) // 4
        ii = device_inputs("f32", N, Pn, 5064)
        oo = [torch.empty(N, device=dev) for _ in range(Pn)]
        for sched, alloc in (("hpds", "state"), ("rr", "connection")):
            idle_rows[f"alltonext_24r_64mib_split_{sched}_{alloc}"] = idle(
                programs.alltonext(G, L, split=True), N, "f32", 8, 512, 256 << 10, 2, KERNEL, ii, oo, scheduler=sched,
                wg_alloc=alloc)
        del ii, oo
        release()
        res["wg_idle_fraction"] = idle_rows

    if section_on("copy"):
        # ---- practical streaming ceiling: a plain copy kernel, 1 GiB (beyond every cache) --
        nb = 1 << 30
        a = torch.empty(nb, dtype=torch.uint8, device=dev)
        b = torch.empty(nb, dtype=torch.uint8, device=dev)
        tc = time_launches(lambda: capi.ccl_copy_probe(b.data_ptr(), a.data_ptr(), nb, 256, 256, stream.cuda_stream), 10)
        res["copy_probe_GBs"] = round(2 * nb / tc / 1e9, 1)
        del a, b
        release()

    return res


def rank_counts(np, torch, programs, dev, stream, device_inputs, tune, make_plan, time_launches, busbw_ar, stats,
                release):
    """Ring AllReduce at 4, 16 and 32 virtual ranks, 1 and 32 MiB per rank, each tuned."""
    ranks = []
    for R in (4, 16, 32):
        pr = programs.ring_allreduce(R)
        for S in (1 << 20, 32 << 20):
            N = S // 4
            ii = device_inputs("f32", N, R, 91000 + R * 64 + S // (1 << 20))
            oo = [torch.empty(N, device=dev) for _ in range(R)]
            # candidates interpreted (no kernel generation per point); where 32 channels leave
            # compute units without a workgroup, larger factors are candidates too
            c, ev = tune(pr, N, kernel=0, factors=TUNE_FACTORS + ([48, 64] if R * 32 < 256 else []))
            p = make_plan(pr, N, *c[:4], KERNEL)  # the chosen point timed on its generated kernel
            t = time_launches(lambda: p.execute(ii, oo, N, stream), 20 if S >= DEVICE_INPUT_BYTES else 50)
            ranks.append({"ranks": R, "bytes_per_rank": S, "k": c[0], "nthreads": c[1], "slice_bytes": c[2],
                          "protocol": PROTOCOLS[c[3]][0], "transport": PROTOCOLS[c[3]][1],
                          "streaming": PROTOCOLS[c[3]][2], "kernel": KERNELS[KERNEL],
                          "workgroups": p.info()["num_workgroups"], "busbw": round(busbw_ar(S, t, R), 2),
                          "tuner_evaluations": ev, **stats(p, N, t)})
            progress(f"ring AR {R} ranks {S >> 10} KiB: {ranks[-1]['us']} us")
            release(p)
            del ii, oo
            release()
    return ranks


class GemmLoad:
    """Keeps `stream` busy with 8192^3 bf16 GEMMs while the `with` block runs: a thread
    enqueues batches of GEMMs, keeping two batches in flight, and stops when the block
    ends; the GEMM rate over the block is measured with events on that stream."""

    def __init__(self, torch, stream, a, b, c, batch=4):
        import threading
        self.torch, self.stream, self.a, self.b, self.c, self.batch = torch, stream, a, b, c, batch
        self.stop = threading.Event()
        self.thread = threading.Thread(target=self._run, daemon=True)
        self.count = 0

    def _run(self):
        torch = self.torch
        pending = []
        with torch.cuda.stream(self.stream):
            while not self.stop.is_set():
                for _ in range(self.batch):
                    torch.matmul(self.a, self.b, out=self.c)
                self.count += self.batch
                e = torch.cuda.Event()
                e.record(self.stream)
                pending.append(e)
                if len(pending) > 2:
                    pending.pop(0).synchronize()

    def __enter__(self):
        torch = self.torch
        self.e0, self.e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(self.stream):
            for _ in range(2):  # running before the measured work starts
                torch.matmul(self.a, self.b, out=self.c)
        self.e0.record(self.stream)
        self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        self.thread.join()
        self.e1.record(self.stream)
        self.torch.cuda.synchronize()
        n = self.a.shape[0]
        t = self.e0.elapsed_time(self.e1) * 1e-3
        self.tflops = 2 * n ** 3 * self.count / t / 1e12 if self.count and t > 0 else 0.0
        return False


def interference(torch, dev, stream, prog, ring_inputs, tune, make_plan, busbw_ar, release):
    """AutoCCL tunes inside the running job, where computation competes for the GPU;
    ReSCCL frees compute for it by taking fewer thread blocks. Here 8192^3 bf16 GEMMs
    (hipBLASLt through torch) run beside the 8-rank ring AllReduce:

    * shared: GEMMs on a second stream over the whole GPU; the collective tuned alone
      and tuned while the GEMMs run, both timed under the GEMMs;
    * reserved: for budgets of B = 32 / 64 / 128 compute units, the collective runs on a
      stream masked to B CUs (mask bits 0..B-1: B/8 CUs on each XCD) with plans sized
      to B CUs, the GEMMs on a stream masked to the other 256 - B; the tuner runs there
      while the GEMMs run, and its pick is compared with the one it makes within the
      same budget alone.
    Candidates are timed on the interpreting kernel (no kernel generation inside the
    tuning); the chosen points are timed on their generated kernels. Reported: chosen
    points, workgroups, collective time alone and under the GEMMs, and the GEMM rate
    (alone on its CUs, and meanwhile). Masked streams each hold a hardware queue of their
    own, so one pair per budget is created and kept for both sizes."""
    from chunk_schedule_execution_amd import capi

    n = 8192
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16).contiguous()
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    side = torch.cuda.Stream(device=dev)

    def gemm_tflops(on, count=20):
        with torch.cuda.stream(on):
            for _ in range(3):
                torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(on)
        with torch.cuda.stream(on):
            for _ in range(count):
                torch.matmul(a, b, out=c)
        e1.record(on)
        torch.cuda.synchronize()
        return round(2 * n ** 3 / (e0.elapsed_time(e1) * 1e-3 / count) / 1e12, 1)

    def launches(fn, iters, comm):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(comm)
        for _ in range(iters):
            fn()
        e1.record(comm)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / iters

    def measure(cfg, N, ii, oo, comm, gstream, iters, **kw):
        p = make_plan(prog, N, *cfg, **kw)
        alone = launches(lambda: p.execute(ii, oo, N, comm), iters, comm)
        with GemmLoad(torch, gstream, a, b, c) as g:
            t = launches(lambda: p.execute(ii, oo, N, comm), iters, comm)
        r = {"k": cfg[0], "nthreads": cfg[1], "slice_bytes": cfg[2], "protocol": cfg[3],
             "workgroups": p.info()["num_workgroups"], "us_alone": round(alone * 1e6, 2),
             "us_under_gemms": round(t * 1e6, 2), "gemm_tflops_meanwhile": round(g.tflops, 1)}
        release(p)
        return r

    out = {"gemm": "bf16 8192x8192x8192, torch.matmul", "gemm_alone_tflops": gemm_tflops(side), "sizes": []}
    budgets = (32, 64, 128)
    masked = {B: (capi.ccl_stream_create_cu_masked(capi.cu_mask_words(range(B))),
                  capi.ccl_stream_create_cu_masked(capi.cu_mask_words(range(B, 256)))) for B in budgets}
    try:
        out["gemm_tflops_on_the_other_cus"] = {B: gemm_tflops(torch.cuda.ExternalStream(masked[B][1]))
                                               for B in budgets}
        progress(f"interference: GEMM alone {out['gemm_alone_tflops']} TFLOP/s, on 256-B CUs "
                 f"{out['gemm_tflops_on_the_other_cus']}")
        for S in (3 << 20, 32 << 20):
            N, ii, oo = ring_inputs(S)
            iters = 50 if S < (32 << 20) else 20
            row = {"bytes_per_rank": S}
            c_pure, _ = tune(prog, N, kernel=0, factors=ring_factors(S))
            with GemmLoad(torch, side, a, b, c):
                c_int, ev = tune(prog, N, kernel=0, factors=ring_factors(S))
            row["shared_tuned_alone"] = measure(c_pure[:4] + (KERNEL,), N, ii, oo, stream, side, iters)
            row["shared_tuned_under_gemms"] = measure(c_int[:4] + (KERNEL,), N, ii, oo, stream, side, iters)
            row["shared_tuner_evaluations_under_gemms"] = ev
            progress(f"interference {S >> 20} MiB shared: tuned alone {row['shared_tuned_alone']['us_under_gemms']} "
                     f"us under GEMMs, tuned under GEMMs {row['shared_tuned_under_gemms']['us_under_gemms']} us")
            for B in budgets:
                comm = torch.cuda.ExternalStream(masked[B][0])
                gst = torch.cuda.ExternalStream(masked[B][1])
                c_alone_b, _ = tune(prog, N, kernel=0, num_cus=B, on=comm, factors=ring_factors(S))
                with GemmLoad(torch, gst, a, b, c):
                    c_b, ev_b = tune(prog, N, kernel=0, num_cus=B, on=comm, factors=ring_factors(S))
                entry = {"tuner_evaluations_under_gemms": ev_b,
                         "tuned_alone": measure(c_alone_b[:4] + (KERNEL,), N, ii, oo, comm, gst, iters, num_cus=B),
                         "tuned_under_gemms": measure(c_b[:4] + (KERNEL,), N, ii, oo, comm, gst, iters, num_cus=B)}
                row[f"reserved_{B}_cus"] = entry
                progress(f"interference {S >> 20} MiB, {B} CUs: alone {entry['tuned_under_gemms']['us_alone']} us, "
                         f"under GEMMs {entry['tuned_under_gemms']['us_under_gemms']} us, GEMMs meanwhile "
                         f"{entry['tuned_under_gemms']['gemm_tflops_meanwhile']} TFLOP/s")
            out["sizes"].append(row)
            del ii, oo
    finally:
        torch.cuda.synchronize()
        for pair in masked.values():
            for s_ in pair:
                capi.ccl_stream_destroy(s_)
    del a, b, c
    release()
    return out


def interference_row(torch, dev, stream, prog, cfg, ring_inputs, tune, make_plan, release, budget=64):
    """Compact form of the interference section for the summary line: the 3 MiB ring
    AllReduce beside 8192^3 bf16 GEMMs on the shared GPU (the headline's configuration)
    and on `budget` reserved CUs (tuned while the GEMMs run on the other CUs)."""
    from chunk_schedule_execution_amd import capi

    n = 8192
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16).contiguous()
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    N, ii, oo = ring_inputs(HEADLINE_BYTES)

    def launches(fn, iters, comm):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(comm)
        for _ in range(iters):
            fn()
        e1.record(comm)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / iters

    row = {"MiB": 3, "reserved_cus": budget}
    side = torch.cuda.Stream(device=dev)
    p = make_plan(prog, N, *cfg)
    with GemmLoad(torch, side, a, b, c) as g:
        t = launches(lambda: p.execute(ii, oo, N, stream), 50, stream)
    row["shared_us"], row["shared_gemm_tflops"] = round(t * 1e6, 1), round(g.tflops, 1)
    release(p)
    comm_h = capi.ccl_stream_create_cu_masked(capi.cu_mask_words(range(budget)))
    rest_h = capi.ccl_stream_create_cu_masked(capi.cu_mask_words(range(budget, 256)))
    try:
        comm, rest = torch.cuda.ExternalStream(comm_h), torch.cuda.ExternalStream(rest_h)
        with GemmLoad(torch, rest, a, b, c):
            cb, _ = tune(prog, N, kernel=0, num_cus=budget, on=comm, factors=CONFIG_FACTORS)
        p = make_plan(prog, N, *cb[:4], KERNEL, num_cus=budget)
        with GemmLoad(torch, rest, a, b, c) as g:
            t = launches(lambda: p.execute(ii, oo, N, comm), 50, comm)
        row["reserved_us"], row["reserved_gemm_tflops"] = round(t * 1e6, 1), round(g.tflops, 1)
        row["reserved_k"] = cb[0]
        release(p)
    finally:
        torch.cuda.synchronize()
        capi.ccl_stream_destroy(comm_h)
        capi.ccl_stream_destroy(rest_h)
    del a, b, c, ii, oo
    release()
    return row


def kernels(prog, ring_inputs, make_plan, time_launches, release, stream):
    """The interpreting kernel against kernels generated for the plan (ReSCCL's
    lightweight kernel generation) and the generated kernel in the lazy loop order
    (slice s of every instruction before slice s + 1 of any), on identical plans of the
    8-rank ring AllReduce; several slices per instruction show the lazy order's bubbles."""
    rows = []
    for S, k, nt, sl, proto in ((32 << 10, 4, 256, 64 << 10, 1), (1 << 20, 32, 256, 128 << 10, 1),
                                (1 << 20, 32, 256, 64 << 10, 2), (3 << 20, 32, 256, 64 << 10, 2),
                                (3 << 20, 8, 256, 16 << 10, 2), (3 << 20, 2, 512, 16 << 10, 2),
                                (32 << 20, 32, 512, 64 << 10, 3), (32 << 20, 32, 512, 16 << 10, 3)):
        N, ii, oo = ring_inputs(S)
        row = {"bytes_per_rank": S, "k": k, "nthreads": nt, "slice_bytes": sl, "protocol": PROTOCOLS[proto][0],
               "transport": PROTOCOLS[proto][1], "streaming": PROTOCOLS[proto][2],
               "slices_per_instruction": -(-(S // P // k) // sl)}
        for kern, name in KERNELS.items():
            t0 = time.perf_counter()
            p = make_plan(prog, N, k, nt, sl, proto, kern)
            create = time.perf_counter() - t0
            t = min(time_launches(lambda: p.execute(ii, oo, N, stream), 30 if S >= DEVICE_INPUT_BYTES else 200)
                    for _ in range(3))
            p.status()
            row[name + "_us"] = round(t * 1e6, 2)
            row[name + "_create_s"] = round(create, 2)
            release(p)
        row["specialized_speedup"] = round(row["interpreter_us"] / row["specialized_us"], 3)
        row["lazy_vs_specialized"] = round(row["lazy_us"] / row["specialized_us"], 3)
        rows.append(row)
        progress(f"kernels {S >> 10} KiB k={k}: {row['interpreter_us']} / {row['specialized_us']} / {row['lazy_us']} us")
        del ii, oo
    return rows


def kernels_other(programs, device_inputs, make_plan, time_launches, release, stream, torch, dev):
    from chunk_schedule_execution_amd import capi
    """Interpreting vs generated kernels (the loop form: these programs are too long for
    straight-line code) on the other collectives, identical plans."""
    TT = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}
    rows = []
    for name, pr, dt, N, k, nt, proto in (
            ("hierarchical AR 2x8, 1 MiB bf16", programs.hierarchical_allreduce(2, 8), "bf16", 1 << 19, 16, 512, 1),
            ("hierarchical AR 2x8, 16 MiB bf16", programs.hierarchical_allreduce(2, 8), "bf16", 1 << 23, 16, 512, 2),
            ("tree AR 8 ranks, 64 KiB", programs.tree_allreduce(8), "f32", 1 << 14, 4, 256, 1),
            ("two-phase AllToAll 4x8, 1 MiB int32", programs.two_phase_alltoall(4, 8), "i32", 1 << 18, 1, 256, 2),
            ("2-D ReduceScatter 3x8, 768 KiB", programs.reducescatter_2d(3, 8), "f32", 24 * 8192, 4, 512, 0)):
        P = pr.nranks
        ii = device_inputs(dt, N, P, 8100 + len(rows))
        oo = [torch.empty(max(1, pr.out_chunks * N // pr.in_chunks), dtype=TT[dt], device=dev) for _ in range(P)]
        row = {"workload": name, "k": k, "nthreads": nt, "protocol": PROTOCOLS[proto][0],
               "transport": PROTOCOLS[proto][1]}
        for kern in (0, 1):
            try:
                p = make_plan(pr, N, k, nt, 256 << 10, proto, kern, dtype=dt)
            except capi.CCLError as e:  # e.g. more workgroups than fit at once
                row[KERNELS[kern] + "_skipped"] = str(e)[:120]
                continue
            t = min(time_launches(lambda: p.execute(ii, oo, N, stream), 50) for _ in range(2))
            p.status()
            row[KERNELS[kern] + "_us"] = round(t * 1e6, 2)
            if kern:
                row["generated_instructions"] = p.info()["specialized_instructions"]
            release(p)
        if "interpreter_us" in row and "specialized_us" in row:
            row["specialized_speedup"] = round(row["interpreter_us"] / row["specialized_us"], 3)
        rows.append(row)
        progress(f"kernels: {name}: {row.get('interpreter_us')} / {row.get('specialized_us')} us")
        del ii, oo
    return rows


def size_text(S: int) -> str:
    return f"{S >> 20} MiB" if S % (1 << 20) == 0 else f"{S >> 10} KiB" if S % 1024 == 0 else f"{S} B"


def cpu_baseline(budget_s: float, S: int = HEADLINE_BYTES, gpu_sample=None):
    """The CPU oracles on the 8-rank input of S bytes per rank (3 MiB by default), each
    repeated until its share of the budget is spent: the chain-order oracle (the one the
    GPU output is compared with bit for bit), reported in the metric's unit (busbw), and
    the definition oracle (float64 sums), reported as algbw in the sample text. Given
    gpu_sample = (indices, values) of the GPU's output on the same input, also returns
    whether the chain-order result has those values (None without a sample)."""
    import numpy as np

    import workloads as W
    from oracle import definitions as O1
    from oracle import schedule_order as O2

    N = S // 4
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=S)

    def timed(fn, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            if time.perf_counter() - t0 >= budget:
                return (time.perf_counter() - t0) / reps, reps
    t2, r2 = timed(lambda: O2.ring_allreduce(xs, P, "f32"), 0.7 * budget_s)
    ok = None
    if gpu_sample is not None:
        idx, vals = gpu_sample
        ok = bool(np.array_equal(O2.ring_allreduce(xs, P, "f32")[0][idx], vals))
    t1, r1 = timed(lambda: O1.allreduce(xs, "f32"), 0.3 * budget_s)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    cpu = ""
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(S / t2 * 2 * (P - 1) / P / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"chain-order oracle, numpy, one thread, ring AllReduce 8 x {size_text(S)} fp32: {r2} runs of "
                      f"{t2 * 1e3:.2f} ms as busbw; float64 definition oracle: {r1} runs of {t1 * 1e3:.2f} ms, algbw "
                      f"{S / t1 / 1e9:.3f} GB/s; {cores} host cores ({cpu[:24]})"}, ok


if __name__ == "__main__":
    main()
