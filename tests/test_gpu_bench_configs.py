"""GPU parity in the launch configurations that bench.py times, at the sizes it times.

Every test names the bench row it mirrors. Outputs are compared with the CPU oracle
element by element (the chain-order oracle for float reductions, the definitions for
copy-only collectives), except where a size is marked "sampled" below, where the
oracle's folds run on sampled element indices. Large inputs are drawn on the device by
torch's seeded generator and copied to the host for the oracle, so both sides read the
same bits.
"""

import numpy as np
import pytest

import workloads as W
from chunk_schedule_execution_amd import Plan, PlanConfig, capi, programs
from oracle import definitions as O1
from oracle import numerics as nm
from oracle import schedule_order as O2

pytestmark = pytest.mark.gpu

# bench.py's protocol ids: (protocol, transport, non-temporal local traffic)
PROTOCOLS = {0: ("simple", "staged", False), 1: ("ll", "staged", False), 2: ("simple", "direct", False),
             3: ("simple", "direct", True)}


def case(msg):
    print(f"[case] {msg}", flush=True)


def plan_of(prog, count, k, nt, sl, proto, dtype="f32", kernel="specialized", **kw):
    pr, tr, st = PROTOCOLS[proto]
    return Plan(prog, k, PlanConfig(dtype=dtype, max_count=count, nthreads=nt, slice_bytes=sl, protocol=pr,
                                    transport=tr, streaming=st, kernel=kernel, **kw))


def launch(plan, ins, outs, count):
    import torch
    plan.execute(ins, outs, count)
    torch.cuda.synchronize()
    plan.status()


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def filled(n, value, dtype, ranks):
    import torch
    tt = {"f32": torch.float32, "i32": torch.int32, "bf16": torch.bfloat16}[dtype]
    return [torch.full((n,), value, dtype=tt, device="cuda:0") for _ in range(ranks)]


def assert_ranks_equal(ys, want):
    for r, y in enumerate(ys):
        w = want[r] if isinstance(want, list) else want
        if not np.array_equal(y, w):
            bad = np.nonzero(y != w)[0]
            raise AssertionError(f"rank {r}: {bad.size} elements differ, first at {bad[:5]}")


# ------------------------------------------------------------------ headline and large ring AllReduce

@pytest.mark.parametrize("k", [24, 32])
@pytest.mark.parametrize("proto", [0, 1, 2, 3])
def test_headline_ring_ar_8r_3mib(proto, k):
    """Bench headline (ring AllReduce, 8 ranks, 3 MiB fp32 per rank): the tuner's
    k = 24 (the largest factor of the sweep's set) and the `factor_32` row's k = 32, at
    256 threads x 32 KiB slices on a generated kernel, under each of the four
    protocol / transport subspaces the tuner searches. Element-wise against the chain
    order, two launches on different inputs, and the plain relative error within the
    bound recursive summation implies."""
    from gpu_util import run
    P, N = 8, (3 << 20) // 4
    case(f"headline ring AR 3 MiB k={k} nt=256 slice=32K proto={proto}")
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=3 << 20)
    pr, tr, st = PROTOCOLS[proto]
    ys, plan = run(programs.ring_allreduce(P), xs, "f32", k=k, nthreads=256, slice_bytes=32 << 10, protocol=pr,
                   transport=tr, streaming=st, kernel="specialized", repeat=2,
                   check=lambda y, x, _: assert_ranks_equal(y, O2.ring_allreduce(x, P, "f32")[0]))
    want = O2.ring_allreduce(xs, P, "f32")[0]
    assert_ranks_equal(ys, want)
    ref = O1.allreduce(xs, "f32")
    assert nm.scaled_error(ys[0], ref.exact, ref.abs_sum, "f32") <= 1e-6 * P
    assert nm.elementwise_rel_error(ys[0], ref.exact, ref.abs_sum, "f32") <= (P - 1) * 2.0**-24 * 1e3 * (1 + 1e-6)
    assert plan.info()["num_workgroups"] == P * k
    plan.destroy()


@pytest.mark.parametrize("cfg", [(32, 512, 64 << 10, 3), (32, 1024, 64 << 10, 3), (32, 1024, 128 << 10, 3),
                                 (64, 512, 128 << 10, 3), (48, 512, 128 << 10, 3), (64, 512, 32 << 10, 3),
                                 (64, 1024, 128 << 10, 2),
                                 (1, 256, 128 << 10, 0), (8, 512, 256 << 10, 0)])
def test_ring_ar_8r_32mib(cfg):
    """Bench rows `large` (32 MiB, the tuner's streaming points at 512 / 1024 threads)
    and `tuned_vs_fixed` (the two fixed configurations): element-wise, 8 ranks."""
    P, S = 8, 32 << 20
    N = S // 4
    k, nt, sl, proto = cfg
    case(f"ring AR 32 MiB {cfg}")
    ins = W.device_inputs("normal_f32", N, P, 2026 * 1000 + 32)
    outs = filled(N, -7.0, "f32", P)
    plan = plan_of(programs.ring_allreduce(P), N, k, nt, sl, proto)
    launch(plan, ins, outs, N)
    xs = [host(t) for t in ins]
    want = O2.ring_allreduce(xs, P, "f32")[0]
    assert_ranks_equal([host(t) for t in outs], want)
    plan.destroy()


@pytest.mark.parametrize("k,nt,proto", [(32, 1024, 3), (64, 512, 3), (64, 1024, 2)])
@pytest.mark.parametrize("S", [64 << 20, 256 << 20])
def test_ring_ar_8r_large_cold_rotation_sampled(S, k, nt, proto):
    """Bench row `large` cold runs (64 / 256 MiB, 128 KiB slices, one or two workgroups per
    compute unit, streaming or plain direct transport, the tuner's picks at these sizes):
    three buffer sets launched back to back, as the cold timing rotates them; sampled
    elements of every set against the chain order, all ranks identical."""
    import torch
    P, N = 8, S // 4
    case(f"ring AR {S >> 20} MiB rotating sets, sampled, k={k} nt={nt} proto={proto}")
    plan = plan_of(programs.ring_allreduce(P), N, k, nt, 128 << 10, proto)
    sets = []
    for j in range(3):
        sets.append((W.device_inputs("normal_f32", N, P, 70000 + j), filled(N, -7.0, "f32", P)))
    for ins, outs in sets:
        plan.execute(ins, outs, N)
    torch.cuda.synchronize()
    plan.status()
    rng = np.random.default_rng(S >> 20)
    idx = np.unique(np.concatenate([rng.integers(0, N, 4000), [0, N - 1], np.arange(N // P - 3, N // P + 3)]))
    tidx = torch.from_numpy(idx).to("cuda:0")
    for ins, outs in sets:
        for r in range(1, P):
            assert torch.equal(outs[r], outs[0]), r
        xs = [t[tidx].cpu().numpy() for t in ins]
        got = outs[0][tidx].cpu().numpy()
        assert np.array_equal(got, O2.ring_allreduce_columns(xs, N, P, idx, "f32"))
    plan.destroy()


@pytest.mark.parametrize("R,S,cfg", [
    (4, 1 << 20, (64, 128, 4096, 2)), (16, 1 << 20, (32, 128, 65536, 1)), (32, 1 << 20, (32, 64, 32768, 1)),
    (4, 32 << 20, (64, 1024, 65536, 3)), (16, 32 << 20, (32, 512, 131072, 3)), (32, 32 << 20, (32, 256, 65536, 3))])
def test_ring_ar_rank_counts_bench_points(R, S, cfg):
    """Bench section `ranks` (ring AllReduce at 4, 16 and 32 ranks, 1 and 32 MiB per
    rank) at the points its tuner chose: element-wise at 1 MiB, sampled at 32 MiB (4,000
    elements plus the chunk bounds, all ranks identical over the whole buffer)."""
    import torch
    N = S // 4
    k, nt, sl, proto = cfg
    case(f"ring AR {R} ranks {S >> 20} MiB {cfg}")
    ins = W.device_inputs("normal_f32", N, R, 91000 + R * 64 + S // (1 << 20))
    outs = filled(N, -7.0, "f32", R)
    plan = plan_of(programs.ring_allreduce(R), N, k, nt, sl, proto)
    launch(plan, ins, outs, N)
    plan.destroy()
    if S <= (1 << 20):
        xs = [host(t) for t in ins]
        assert_ranks_equal([host(t) for t in outs], O2.ring_allreduce(xs, R, "f32")[0])
        return
    for r in range(1, R):
        assert torch.equal(outs[r], outs[0]), r
    rng = np.random.default_rng(R)
    bounds = np.concatenate([np.arange(-1, 2) + (N * j) // R for j in range(1, R)])
    idx = np.unique(np.concatenate([rng.integers(0, N, 4000), [0, N - 1], bounds]))
    tidx = torch.from_numpy(idx).to("cuda:0")
    cols = [t[tidx].cpu().numpy() for t in ins]
    want = O2.ring_allreduce_columns(cols, N, R, idx, "f32")
    assert np.array_equal(outs[0][tidx].cpu().numpy(), want)


def test_ring_ar_4r_1mib_bench_config():
    """Bench row `ring_ar_4r_1mib_int` (4 ranks, 1 MiB integer-valued fp32, one channel,
    one 1 MiB slice, 512 threads, staged, generated kernel): exact sum, bit for bit."""
    from gpu_util import run
    P, N = 4, 262144
    case("ring AR 4 ranks 1 MiB int, bench config")
    xs = W.make_inputs("int_f32", N, P, W.CFG_RING_AR_4R_INT, size_bytes=N * 4)
    ys, _ = run(programs.ring_allreduce(P), xs, "f32", k=1, nthreads=512, slice_bytes=N * 4, kernel="specialized")
    assert_ranks_equal(ys, O1.allreduce(xs, "f32").exact.astype(np.float32))


# ------------------------------------------------------------------ AllToAll, 32 ranks int32

A2A_POINTS = [(1, 256, 2), (2, 256, 2), (2, 128, 2), (4, 128, 2), (1, 256, 3), (2, 256, 3)]


@pytest.mark.parametrize("name", ["two_phase", "direct"])
def test_alltoall_32r_16mib_bench_points(name):
    """Bench row `alltoall_32r_int32` at 16 MiB: every launch configuration the bench
    tries (k, threads, direct transport with and without streaming hints, 256 KiB
    slices, generated kernel), each the exact transposed block permutation. Points whose
    grid cannot be co-resident are refused at creation, as in the bench."""
    import torch
    G, L = 4, 8
    P, S = G * L, 16 << 20
    N = S // 4
    ins = W.device_inputs("uniform_i32", N, P, 4000 + 16)
    want = O1.alltoall([host(t) for t in ins])
    prog = programs.two_phase_alltoall(G, L) if name == "two_phase" else programs.direct_alltoall(P)
    ran = 0
    for k, nt, proto in A2A_POINTS:
        case(f"alltoall {name} 16 MiB k={k} nt={nt} proto={proto}")
        try:
            plan = plan_of(prog, N, k, nt, 256 << 10, proto, dtype="i32")
        except capi.CCLError as e:
            assert e.status == capi.CCL_ERR_OUT_OF_RESOURCES, str(e)
            continue
        outs = filled(N, -7, "i32", P)
        launch(plan, ins, outs, N)
        assert_ranks_equal([host(t) for t in outs], want)
        plan.destroy()
        ran += 1
        del outs
        torch.cuda.empty_cache()
    assert ran >= 4


@pytest.mark.parametrize("name", ["two_phase", "direct"])
def test_alltoall_32r_64mib(name):
    """Bench row `alltoall_32r_int32` at 64 MiB (2 GiB of inputs), at the points the bench
    measured fastest (k=2 x 256 threads, streaming) and k=1 x 256 without streaming:
    element-wise."""
    import torch
    G, L = 4, 8
    P, S = G * L, 64 << 20
    N = S // 4
    ins = W.device_inputs("uniform_i32", N, P, 4000 + 64)
    xs = [host(t) for t in ins]
    want = O1.alltoall(xs)
    del xs
    prog = programs.two_phase_alltoall(G, L) if name == "two_phase" else programs.direct_alltoall(P)
    for k, nt, proto in ((2, 256, 3), (1, 256, 2)):
        case(f"alltoall {name} 64 MiB k={k} nt={nt} proto={proto}")
        plan = plan_of(prog, N, k, nt, 256 << 10, proto, dtype="i32")
        outs = filled(N, -7, "i32", P)
        launch(plan, ins, outs, N)
        for r in range(P):
            assert np.array_equal(host(outs[r]), want[r]), r
        plan.destroy()
        del outs
        torch.cuda.empty_cache()


# ------------------------------------------------------------------ AllToNext, 24 ranks

@pytest.mark.parametrize("split", [True, False])
def test_alltonext_24r_16mib_bench_config(split):
    """Bench row `alltonext_24r` at 16 MiB (and the summary line's `a2next_24r_64mib`
    launch configuration): k = 16 (the largest factor at which both modes' grids fit, as
    the bench picks it), 256 threads, 128 KiB slices, direct transport with streaming
    hints, HPDS + state and round robin + connection. Rank r's
    input lands at r+1; rank 0 keeps its prior contents."""
    G, L = 3, 8
    P, N = G * L, (16 << 20) // 4
    ins = W.device_inputs("normal_f32", N, P, 5000 + 16)
    xs = [host(t) for t in ins]
    prior = [np.full(N, -3.0, np.float32) for _ in range(P)]
    want = O1.alltonext(xs, prior)
    for sched, alloc in (("hpds", "state"), ("rr", "connection")):
        plan = None
        for k in (16, 8, 4, 2, 1):
            try:
                plan = plan_of(programs.alltonext(G, L, split=split), N, k, 256, 128 << 10, 3, scheduler=sched,
                               wg_alloc=alloc)
                break
            except capi.CCLError as e:
                assert e.status == capi.CCL_ERR_OUT_OF_RESOURCES, str(e)
        case(f"alltonext split={split} 16 MiB {sched}/{alloc} k={plan.parallel_factor}")
        outs = filled(N, -3.0, "f32", P)
        launch(plan, ins, outs, N)
        assert_ranks_equal([host(t) for t in outs], want)
        plan.destroy()


# ------------------------------------------------------------------ AllGather / ReduceScatter, 24 ranks, 128 MiB

N_BIG = 24 * ((32 << 20) // 24)  # 33,554,424 fp32: the AllGather output, the ReduceScatter input


def _agrs_points(variant):
    if variant == "ring":  # one configuration for both modes: k=32 x 512 threads, 64 KiB slices, streaming
        return [("hpds", "state", 32, 512), ("rr", "connection", 32, 512)]
    return [("hpds", "state", 24, 256), ("hpds", "state", 16, 256), ("hpds", "state", 8, 512),
            ("rr", "connection", 16, 128), ("rr", "connection", 8, 256)]


@pytest.mark.parametrize("variant", ["ring", "2d"])
def test_allgather_24r_128mib(variant):
    """Bench row `allgather_reducescatter_24r_128mib`, AllGather: the ring at the bench's
    (32, 512, 64 KiB, direct + streaming) in both modes, and the 2-D program at points of
    its sweep, on full-range int32 (copies are bit-exact whatever the values): every
    rank's 128 MiB output is the rank-ordered concatenation, element for element."""
    import torch
    G, L = 3, 8
    P = G * L
    count = N_BIG // P
    ins = W.device_inputs("uniform_i32", count, P, 6000 + 9)
    want = np.concatenate([host(t) for t in ins])
    prog = programs.ring_allgather(P) if variant == "ring" else programs.allgather_2d(G, L)
    for sched, alloc, k, nt in _agrs_points(variant):
        try:
            plan = plan_of(prog, count, k, nt, 64 << 10, 3, dtype="i32", scheduler=sched, wg_alloc=alloc)
        except capi.CCLError as e:
            assert e.status == capi.CCL_ERR_OUT_OF_RESOURCES and variant == "2d", str(e)
            continue
        case(f"allgather {variant} 128 MiB {sched}/{alloc} k={k} nt={nt}")
        outs = filled(N_BIG, -7, "i32", P)
        launch(plan, ins, outs, count)
        for r in range(P):
            assert np.array_equal(host(outs[r]), want), r
        plan.destroy()
        del outs
        torch.cuda.empty_cache()


@pytest.mark.parametrize("variant", ["ring", "2d"])
def test_reducescatter_24r_128mib(variant):
    """Bench row `allgather_reducescatter_24r_128mib`, ReduceScatter: 128 MiB fp32 N(0,1)
    per rank (shards of 1,398,101 elements, not 16-byte aligned), element-wise against
    the chain order of the ring or of the 2-D program, fp32 bound of the definition."""
    import torch
    G, L = 3, 8
    P = G * L
    ins = W.device_inputs("normal_f32", N_BIG, P, 6000 + 13)
    xs = [host(t) for t in ins]
    want = O2.ring_reducescatter(xs, P, "f32") if variant == "ring" else O2.reducescatter_2d(xs, G, L, "f32")
    ref = O1.reducescatter(xs, "f32")
    del xs
    prog = programs.ring_reducescatter(P) if variant == "ring" else programs.reducescatter_2d(G, L)
    for sched, alloc, k, nt in _agrs_points(variant):
        try:
            plan = plan_of(prog, N_BIG, k, nt, 64 << 10, 3, scheduler=sched, wg_alloc=alloc)
        except capi.CCLError as e:
            assert e.status == capi.CCL_ERR_OUT_OF_RESOURCES and variant == "2d", str(e)
            continue
        case(f"reducescatter {variant} 128 MiB {sched}/{alloc} k={k} nt={nt}")
        outs = filled(N_BIG // P, -7.0, "f32", P)
        launch(plan, ins, outs, N_BIG)
        for r in range(P):
            y = host(outs[r])
            assert np.array_equal(y, want[r]), r
            assert nm.scaled_error(y, ref[r].exact, ref[r].abs_sum, "f32") <= 1e-6 * P
        plan.destroy()
        torch.cuda.empty_cache()


# ------------------------------------------------------------------ hierarchical AllReduce, 16 ranks bf16

def test_hierarchical_16r_bf16_16mib_summary_points():
    """Summary-line row `hier_16r_16mib_bf16` (bench.py CONFIG_POINTS): the fused plan at
    k=32, 256 threads, 256 KiB slices, direct + streaming, and the three launches at
    their own points, 16 MiB per rank: element-wise against the three-step chain order
    on every rank."""
    import bench
    G, L = 2, 8
    P, N = G * L, (16 << 20) // 2
    sh = N // L
    case("hierarchical bf16 16 MiB, summary-line points")
    ins = W.device_inputs("normal_bf16", N, P, 3016)
    xs = [host(t) for t in ins]
    want = O2.hierarchical_allreduce(xs, G, L, "bf16")[0]
    outs = filled(N, 0.0, "bf16", P)
    plan = plan_of(programs.hierarchical_allreduce(G, L), N, *bench.CONFIG_POINTS["hier_fused"], dtype="bf16")
    launch(plan, ins, outs, N)
    plan.destroy()
    assert_ranks_equal([host(t) for t in outs], want)
    c1, c2, c3 = bench.CONFIG_POINTS["hier_stages"]
    mid1, mid2 = filled(sh, 0.0, "bf16", P), filled(sh, 0.0, "bf16", P)
    outs = filled(N, 0.0, "bf16", P)
    s1 = plan_of(programs.hier_stage_reducescatter_intra(G, L), N, *c1, dtype="bf16")
    s2 = plan_of(programs.hier_stage_allreduce_inter(G, L), sh, *c2, dtype="bf16")
    s3 = plan_of(programs.hier_stage_allgather_intra(G, L), sh, *c3, dtype="bf16")
    import torch
    s1.execute(ins, mid1, N)
    s2.execute(mid1, mid2, sh)
    s3.execute(mid2, outs, sh)
    torch.cuda.synchronize()
    for st in (s1, s2, s3):
        st.status()
        st.destroy()
    assert_ranks_equal([host(t) for t in outs], want)


def test_hierarchical_16r_bf16_256mib_sampled():
    """Bench row `hier_ar_16r_bf16` at 256 MiB per rank (4 GiB of inputs), sampled: the
    fused plan (k=16, 512 threads, 256 KiB slices, direct + streaming, generated kernel)
    and the three-launch composition give the three-step chain order at 4,000 random
    elements plus the shard boundaries; all ranks identical over the whole buffer."""
    import torch
    G, L = 2, 8
    P, N = G * L, (256 << 20) // 2
    case("hierarchical bf16 256 MiB fused + three launches, sampled")
    ins = W.device_inputs("normal_bf16", N, P, 3000 + 256)
    rng = np.random.default_rng(256)
    edges = np.concatenate([np.arange(-2, 3) + (N // (L * G)) * j for j in range(1, L * G)])
    idx = np.unique(np.concatenate([rng.integers(0, N, 4000), [0, N - 1], edges]))
    tidx = torch.from_numpy(idx).to("cuda:0")
    cols = [t[tidx].view(torch.int16).cpu().numpy().view(np.uint16) for t in ins]
    want = O2.hierarchical_allreduce_columns(cols, N, G, L, idx, "bf16")
    outs = filled(N, 0.0, "bf16", P)
    plan = plan_of(programs.hierarchical_allreduce(G, L), N, 16, 512, 256 << 10, 3, dtype="bf16")
    launch(plan, ins, outs, N)
    plan.destroy()
    for r in range(1, P):
        assert torch.equal(outs[r].view(torch.int16), outs[0].view(torch.int16)), r
    assert np.array_equal(outs[0][tidx].view(torch.int16).cpu().numpy().view(np.uint16), want)
    del outs
    torch.cuda.empty_cache()
    sh = N // L
    mid1, mid2 = filled(sh, 0.0, "bf16", P), filled(sh, 0.0, "bf16", P)
    outs = filled(N, 0.0, "bf16", P)
    s1 = plan_of(programs.hier_stage_reducescatter_intra(G, L), N, 16, 512, 256 << 10, 3, dtype="bf16")
    s2 = plan_of(programs.hier_stage_allreduce_inter(G, L), sh, 16, 512, 256 << 10, 3, dtype="bf16")
    s3 = plan_of(programs.hier_stage_allgather_intra(G, L), sh, 16, 512, 256 << 10, 3, dtype="bf16")
    s1.execute(ins, mid1, N)
    s2.execute(mid1, mid2, sh)
    s3.execute(mid2, outs, sh)
    torch.cuda.synchronize()
    for s in (s1, s2, s3):
        s.status()
        s.destroy()
    assert np.array_equal(outs[5][tidx].view(torch.int16).cpu().numpy().view(np.uint16), want)
