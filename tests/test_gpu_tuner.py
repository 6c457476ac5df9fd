"""The on-device tuner (AutoCCL report, methods 1-2: coordinate descent over channels,
threads and chunk size inside each implementation subspace, every point timed on the
device) through the C ABI: it returns a point of the space whose plan is correct, and
the point it returns scores at least as well as the point it started from."""

import numpy as np
import pytest

import workloads as W
from chunk_schedule_execution_amd import PlanConfig, capi, programs
from oracle import schedule_order as O2

pytestmark = pytest.mark.gpu

PROTOCOLS = {0: dict(protocol="simple", transport="staged"), 1: dict(protocol="ll", transport="staged"),
             2: dict(protocol="simple", transport="direct"),
             3: dict(protocol="simple", transport="direct", streaming=True)}


def case(msg):
    print(f"[case] {msg}", flush=True)


def space_of(factors, threads, slices, nvariants, protocols, warmup=2, iters=5):
    arrs = [(capi.C.c_int32 * len(v))(*v) for v in (factors, threads, slices)]
    sp = capi.ccl_tune_space(capi.C.cast(arrs[0], capi.C.POINTER(capi.C.c_int32)), len(factors),
                             capi.C.cast(arrs[1], capi.C.POINTER(capi.C.c_int32)), len(threads),
                             capi.C.cast(arrs[2], capi.C.POINTER(capi.C.c_int32)), len(slices),
                             nvariants, warmup, iters, protocols)
    sp._keep = arrs  # the arrays must outlive the call
    return sp


@pytest.mark.parametrize("kernel", ["interpreter", "specialized"])
def test_device_tuner_picks_a_correct_point(kernel):
    """Ring and tree AllReduce subspaces on 8 ranks at 1 MiB, slice-flag and direct
    protocols, a small grid of factors, threads and slices: the returned point lies in
    the space, scores at least its start, and its plan gives the oracle's bits for the
    program it names, launch after launch on fresh inputs."""
    import torch

    from gpu_util import run
    P, N = 8, 1 << 18
    factors, threads, slices = [1, 4, 16], [256, 512], [32 << 10, 128 << 10]
    progs = [programs.ring_allreduce(P), programs.tree_allreduce(P)]
    case(f"device tuner, ring + tree, 1 MiB, {kernel}")
    sp = space_of(factors, threads, slices, len(progs), protocols=0b0101)
    base = PlanConfig(dtype="f32", max_count=N, kernel=kernel).to_c()
    stream = torch.cuda.current_stream().cuda_stream
    best, rep = capi.ccl_tune([p.to_desc() for p in progs], N, base, sp, stream)
    assert best.variant in (0, 1) and best.protocol in (0, 2)
    assert best.parallel_factor in factors and best.nthreads in threads and best.slice_bytes in slices
    assert rep.evaluations >= 4  # at least the start and one step of each coordinate per subspace
    assert rep.start_score > 0 and rep.best_score >= rep.start_score
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=N * 4 + 101)
    oracle = O2.ring_allreduce if best.variant == 0 else O2.tree_allreduce
    ys, plan = run(progs[best.variant], xs, "f32", k=best.parallel_factor, nthreads=best.nthreads,
                   slice_bytes=best.slice_bytes, kernel=kernel, repeat=2,
                   check=lambda y, x, _: _all_equal(y, oracle(x, P, "f32")[0]), **PROTOCOLS[best.protocol])
    _all_equal(ys, oracle(xs, P, "f32")[0])
    plan.destroy()


def test_device_tuner_skips_points_that_cannot_be_resident():
    """A factor whose grid cannot be co-resident is an infeasible point (negative score),
    not an error: the tuner returns the best feasible one."""
    import torch
    P, N = 32, 1 << 16
    case("device tuner with an infeasible factor")
    sp = space_of([1, 2, 64], [1024], [64 << 10], 1, protocols=0b0001, warmup=1, iters=2)  # 64: 2048 workgroups
    base = PlanConfig(dtype="f32", max_count=N).to_c()
    best, rep = capi.ccl_tune([programs.ring_allreduce(P).to_desc()], N, base, sp,
                              torch.cuda.current_stream().cuda_stream)
    assert best.parallel_factor in (1, 2) and rep.best_score > 0


def _all_equal(ys, want):
    for r, y in enumerate(ys):
        assert np.array_equal(y, want), r
