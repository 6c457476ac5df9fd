"""Host compiler: fusion, byte accounting, scheduling, workgroup allocation and the
lowered-plan checker, on host-only plans (no GPU).

The programs themselves are checked against the oracle's symbolic postcondition and
its sequential interpreter, which share no code with the compiler."""

import collections

import numpy as np
import pytest

import workloads as W
from chunk_schedule_execution_amd import Plan, PlanConfig, capi, programs
from chunk_schedule_execution_amd.dsl import Buffer, Program
from oracle import program as OP
from oracle import schedule_order as O2

SEND, RRS, RRCS, RCS, RECV, RRC, CS, RS = 8, 11, 15, 13, 5, 7, 12, 9


def host_plan(prog, k=1, **cfg):
    cfg.setdefault("max_count", 1 << 20)
    return Plan(prog, k, PlanConfig(host_only=True, **cfg))


def hist(plan):
    return collections.Counter(e.opcode for e in plan.export())


# ---------------------------------------------------------------- fusion

@pytest.mark.parametrize("P", [2, 3, 4, 8])
def test_ring_allreduce_fuses_to_the_rrcs_family(P):
    """Every chunk chain becomes send, (P-2) x recv-reduce-send, recv-reduce-copy-send,
    (P-2) x recv-copy-send, recv: 2P-1 instructions (MSCCLang report, section 3.1)."""
    plan = host_plan(programs.ring_allreduce(P))
    h = hist(plan)
    want = collections.Counter({SEND: P, RRS: P * (P - 2), RRCS: P, RCS: P * (P - 2), RECV: P})
    assert h == +want
    per_rank = collections.Counter(e.rank for e in plan.export())
    assert all(v == 2 * P - 1 for v in per_rank.values())
    info = plan.info()
    assert info["scratch_bytes"] == 0  # every scratch partial was forwarded in registers


def test_no_fusion_keeps_primitives_and_costs_bytes():
    P, N = 4, 4096
    fused = host_plan(programs.ring_allreduce(P))
    prim = host_plan(programs.ring_allreduce(P), no_fusion=True)
    assert prim.info()["num_instructions"] > fused.info()["num_instructions"]
    assert prim.bytes(N) > fused.bytes(N)
    prim.check(seed=3, nsims=3)


def test_two_phase_alltoall_keeps_batched_transfers():
    G, L = 4, 8
    plan = host_plan(programs.two_phase_alltoall(G, L))
    big = [e for e in plan.export() if e.count == L and (e.opcode & capi.CCL_I_SEND)]
    assert len(big) == G * L * (G - 1)  # one batched send per (rank, remote group)


# ---------------------------------------------------------------- byte accounting

@pytest.mark.parametrize("P", [2, 4, 8, 16])
@pytest.mark.parametrize("k", [1, 3])
def test_ring_bytes_closed_forms(P, k):
    """Ring AllReduce moves S(6P-4) bytes over all ranks, ring ReduceScatter and
    AllGather S(3P-1) (S = the larger per-rank buffer); instances do not change it."""
    N = P * 1000
    S = N * 4
    assert host_plan(programs.ring_allreduce(P), k).bytes(N) == S * (6 * P - 4)
    assert host_plan(programs.ring_reducescatter(P), k).bytes(N) == S * (3 * P - 1)
    assert host_plan(programs.ring_allgather(P), k).bytes(N // P) == S * (3 * P - 1)


def test_direct_alltoall_and_alltonext_bytes():
    P, N = 8, 8 * 64
    S = N * 4
    assert host_plan(programs.direct_alltoall(P)).bytes(N) == S * (4 * P - 2)
    G, L = 3, 8
    P = G * L
    N = L * 100
    S = N * 4
    assert host_plan(programs.alltonext(G, L, split=False)).bytes(N) == 4 * S * (P - 1)
    assert host_plan(programs.alltonext(G, L, split=True)).bytes(N) == 4 * S * (P - G) + (G - 1) * S * (8 * L - 4) // L


def test_hierarchical_bytes_and_phase_fusion():
    """Three phases, unfused: intra-group reduce-scatter G*S(3L-1), cross-group ring
    AllReduce S(7G-6) (its reductions land in the output, so they stay written), intra-group
    all-gather G*S(3L-2): S(6P+4G-6). The program moves every chunk on its own channel
    with one-chunk operations, so the phase boundaries fuse at any parallel factor (the
    reduce-scatter's last receive-reduce feeds the cross-group send, the cross-group
    result feeds the all-gather's first send): 2S less, S(6P+4G-8)."""
    for G, L in ((2, 8), (3, 4), (4, 2), (1, 8)):
        P, N = G * L, G * L * 512
        S = N * 2
        for k in (1, 2):
            assert host_plan(programs.hierarchical_allreduce(G, L), k, dtype="bf16").bytes(N) == S * (6 * P + 4 * G - 8)


@pytest.mark.parametrize("name,args", [("ring_allreduce", (5,)), ("tree_allreduce", (7,)), ("ring_reducescatter", (6,)),
                                       ("hierarchical_allreduce", (2, 4)), ("two_phase_alltoall", (2, 4)),
                                       ("alltonext", (3, 4, True)), ("reducescatter_2d", (2, 3)),
                                       ("hier_stage_reducescatter_intra", (2, 4))])
@pytest.mark.parametrize("kernel", ["interpreter", "lazy"])
def test_direct_landings_survive_random_interleavings(name, args, kernel):
    """Every transfer the direct pass rewrites (copies into the destination, reducing
    receives into their output chunk) keeps the collective's postcondition in random
    interleavings of the lowered plan, in task order and in the lazy slice order, at
    several parallel factors (fused, multi-chunk instructions)."""
    for k in (1, 2, 3):
        try:
            plan = host_plan(programs.REGISTRY[name](*args), k, max_count=1 << 12, transport="direct", nthreads=128,
                             kernel=kernel)
        except capi.CCLError as e:
            assert kernel == "lazy" and e.status == capi.CCL_ERR_UNSUPPORTED  # plans with completion waits
            continue
        plan.check(seed=11 + k, nsims=4)


def test_ll_protocol_doubles_slot_traffic():
    P, N = 8, 8000
    S = N * 4
    simple = host_plan(programs.ring_allreduce(P)).bytes(N)
    ll = host_plan(programs.ring_allreduce(P), protocol="ll").bytes(N)
    # every slot write and read carries 4 flag bytes per 4 data bytes: 4 slot ops per
    # chain hop (send+recv of each of the 2(P-1) transfers per chunk)
    assert ll - simple == 2 * (2 * (P - 1)) * S // P * P


def test_direct_transport_bytes_and_opcodes():
    """Direct transport: the sender writes each transfer into the receiver's own memory.
    A receive that copies lands in its destination; a reducing receive lands in the chunk
    it reduces into and reduces in place. Ring AllReduce then moves S(5P-4) bytes with no
    staging slot: every all-gather hop but the owner's becomes wait-and-forward from the
    output, the last one only waits; direct AllToAll reaches its floor 2PS."""
    for P in (2, 3, 8):
        N = P * 1000
        S = N * 4
        plan = host_plan(programs.ring_allreduce(P), 2, transport="direct")
        assert plan.bytes(N) == S * (5 * P - 4)
        LOCAL = capi.CCL_I_LOCAL_IN
        want = collections.Counter({SEND: 2 * P, RRS | LOCAL: 2 * P * (P - 2), RRCS | LOCAL: 2 * P,
                                    capi.CCL_I_RECV | capi.CCL_I_SEND | LOCAL: 2 * P * (P - 2),
                                    capi.CCL_I_RECV | LOCAL: 2 * P})
        marks = capi.CCL_I_SKIP | capi.CCL_I_NOFLAG
        assert collections.Counter(e.opcode & ~marks for e in plan.export()) == +want
        # the last hop of every chain only waits and nothing follows it: skipped, and its
        # sender (the chain's last forwarding instruction) sets no flag
        ex = plan.export()
        skipped = [e for e in ex if e.opcode & capi.CCL_I_SKIP]
        assert len(skipped) == 2 * P and all(e.opcode & ~marks == capi.CCL_I_RECV | LOCAL for e in skipped)
        assert {e.xout for e in ex if e.opcode & capi.CCL_I_NOFLAG} == {e.xin for e in skipped}
        assert plan.info()["staging_bytes"] == 0
        plan.check(seed=2, nsims=3)
    P, N = 8, 8 * 64
    S = N * 4
    a2a = host_plan(programs.direct_alltoall(P), transport="direct")
    assert a2a.bytes(N) == 2 * P * S and a2a.info()["staging_bytes"] == 0
    # the LL protocol keeps its flag units in slots: direct transport does not apply
    ll = host_plan(programs.ring_allreduce(8), protocol="ll", transport="direct")
    assert ll.bytes(8000) == host_plan(programs.ring_allreduce(8), protocol="ll").bytes(8000)


def test_direct_transport_skips_locations_touched_before_the_receive():
    """Rank 1 writes its output chunk locally before receiving into it: a direct write
    could land before that local copy, so the transfer keeps its slot."""
    IN, OUT = Buffer.input, Buffer.output
    p = Program("custom", 2, 1, 1)
    p.chunk(1, IN, 0).copy(1, OUT, 0)
    p.chunk(0, IN, 0).copy(1, OUT, 0)
    plan = host_plan(p, transport="direct")
    assert not any(e.opcode & capi.CCL_I_LOCAL_IN for e in plan.export())
    assert plan.bytes(100) == host_plan(p).bytes(100)
    plan.check(seed=1, nsims=4)


def test_count_granule():
    assert host_plan(programs.ring_allreduce(8)).info()["count_granule"] == 1
    assert host_plan(programs.two_phase_alltoall(4, 8)).info()["count_granule"] == 32
    assert host_plan(programs.reducescatter_2d(3, 8)).info()["count_granule"] == 24


def _tree_shape(P):
    internal = P // 2              # heap nodes t with 2t+1 < P
    two_kids = (P - 1) // 2        # heap nodes t with 2t+2 < P
    return P - internal, internal, two_kids


@pytest.mark.parametrize("P", [2, 3, 4, 5, 7, 8, 9, 16])
@pytest.mark.parametrize("c", [1, 2])
def test_tree_allreduce_bytes_closed_form(P, c):
    """Per chunk of s elements, counted from the fused instructions: each of the L
    leaves sends its input (read + slot write) and, in the broadcast, receives into
    its output (slot read + write); a two-child node stores its first receive plus its
    own input to scratch (3 accesses) and sends its second child's data once more
    (SEND, 2); every non-root interior node sends up with a reduce-send (3) and
    forwards the broadcast with a receive-copy-send (3); the root's last receive writes
    the output and starts the broadcast (4). That is 4L + 5T + 6I - 2 slices of s,
    I interior and T two-child nodes, and P*c chunks of S/(P*c) make it a multiple of
    S. Direct transport drops the 2 accesses of each leaf's copy-only receive and the
    slot read of every forwarding node: minus 2L + (I - 1)."""
    L, I, T = _tree_shape(P)
    N = P * c * 64
    S = 4 * N
    staged = host_plan(programs.tree_allreduce(P, c)).bytes(N)
    direct = host_plan(programs.tree_allreduce(P, c), transport="direct").bytes(N)
    assert staged == S * (4 * L + 5 * T + 6 * I - 2)
    assert direct == staged - S * (2 * L + I - 1)


@pytest.mark.parametrize("P", [5, 8, 16, 24])
def test_tree_is_shallower_than_the_ring(P):
    """The point of the tree: its dependent chain grows with log P where the ring's is
    2P - 1 instructions (at P = 4 both come to 7 sub-pipelines, the tree's being
    stretched by link conflicts between the trees of different chunks)."""
    tree = host_plan(programs.tree_allreduce(P)).info()["num_subpipelines"]
    ring = host_plan(programs.ring_allreduce(P)).info()["num_subpipelines"]
    assert tree < ring
    depth = P.bit_length() - 1
    assert tree <= 4 * depth + 2


# ---------------------------------------------------------------- scheduling

def _subpipes_by_instr(plan):
    return [e.subpipe for e in plan.export() if e.instance == 0]


@pytest.mark.parametrize("name,args", [("ring_allreduce", (8,)), ("hierarchical_allreduce", (2, 4)),
                                       ("two_phase_alltoall", (2, 4)), ("alltonext", (3, 4)),
                                       ("allgather_2d", (3, 4)), ("reducescatter_2d", (3, 4))])
@pytest.mark.parametrize("sched", ["hpds", "rr", "program"])
def test_every_transfer_crosses_to_a_later_subpipeline(name, args, sched):
    plan = host_plan(programs.REGISTRY[name](*args), scheduler=sched)
    ex = [e for e in plan.export() if e.instance == 0]
    assert all(e.subpipe >= 0 for e in ex)
    sender = {e.xout: e for e in ex if e.xout >= 0}
    for e in ex:
        if e.xin >= 0:
            assert sender[e.xin].subpipe < e.subpipe
    if sched == "program":
        assert plan.info()["num_subpipelines"] == len(ex)


@pytest.mark.parametrize("name,args", [("ring_allreduce", (8,)), ("two_phase_alltoall", (2, 4)),
                                       ("alltonext", (3, 8)), ("reducescatter_2d", (3, 4))])
def test_hpds_subpipelines_have_no_link_conflict(name, args):
    """ReSCCL report, section 2.2: a sub-pipeline holds tasks free of data and link
    conflicts; the link of a task is the connection its send uses."""
    plan = host_plan(programs.REGISTRY[name](*args), scheduler="hpds")
    seen = set()
    for e in plan.export():
        if e.instance != 0 or e.send_peer < 0:
            continue
        key = (e.subpipe, e.rank, e.send_peer, e.channel)
        assert key not in seen
        seen.add(key)


@pytest.mark.parametrize("P", [3, 4, 8, 16])
def test_hpds_meets_the_critical_path_on_rings(P):
    """A chunk's chain is 2P-1 dependent instructions, so no schedule has fewer than
    2P-1 sub-pipelines; HPDS reaches that bound, and every workgroup runs the ring
    step by step (chain of rank r at step t is (r - t))."""
    plan = host_plan(programs.ring_allreduce(P), scheduler="hpds")
    assert plan.info()["num_subpipelines"] == 2 * P - 1
    prog_order = host_plan(programs.ring_allreduce(P), scheduler="program")
    assert prog_order.info()["num_subpipelines"] == P * (2 * P - 1)


def test_state_allocation_uses_fewer_workgroups():
    """ReSCCL report, section 2.2 (state-based allocation): connections of one rank
    that are never active in the same sub-pipeline share a workgroup."""
    G, L = 3, 8
    for prog in (programs.alltonext(G, L, split=True), programs.two_phase_alltoall(4, 8),
                 programs.reducescatter_2d(G, L), programs.allgather_2d(G, L)):
        conn = host_plan(prog, scheduler="hpds", wg_alloc="connection", nthreads=128).info()["num_workgroups"]
        state = host_plan(prog, scheduler="hpds", wg_alloc="state", nthreads=128).info()["num_workgroups"]
        assert state <= conn, prog.name
    conn = host_plan(programs.alltonext(G, L), wg_alloc="connection").info()["num_workgroups"]
    state = host_plan(programs.alltonext(G, L), wg_alloc="state").info()["num_workgroups"]
    assert state < conn


def test_workgroup_order_follows_subpipelines():
    plan = host_plan(programs.allgather_2d(3, 4), scheduler="hpds", wg_alloc="state")
    by_wg = collections.defaultdict(list)
    for e in plan.export():
        by_wg[e.wg].append(e.subpipe)
    for sps in by_wg.values():
        assert sps == sorted(sps)


def test_instances_sit_on_one_xcd():
    """Instance i of every rank gets a workgroup id congruent to i mod 8 (workgroups
    are dispatched to the eight XCDs round robin)."""
    for k in (1, 3, 8, 24):
        plan = host_plan(programs.ring_allreduce(8), k=k)
        for e in plan.export():
            assert e.wg % 8 == e.instance % 8


# ---------------------------------------------------------------- lowered-plan checker

@pytest.mark.parametrize("name,args", [("ring_allreduce", (4,)), ("ring_allreduce", (5,)),
                                       ("ring_reducescatter", (4,)), ("ring_allgather", (4,)),
                                       ("hierarchical_allreduce", (2, 4)), ("direct_alltoall", (4,)),
                                       ("two_phase_alltoall", (2, 4)), ("alltonext", (2, 4)),
                                       ("allgather_2d", (2, 4)), ("reducescatter_2d", (2, 4)),
                                       ("tree_allreduce", (6,)), ("tree_allreduce", (3, 2))])
@pytest.mark.parametrize("knobs", [dict(k=1, scheduler="hpds", wg_alloc="state"),
                                   dict(k=2, scheduler="rr", wg_alloc="connection"),
                                   dict(k=3, scheduler="program", wg_alloc="state", protocol="ll"),
                                   dict(k=2, scheduler="hpds", wg_alloc="state", transport="direct"),
                                   dict(k=1, scheduler="rr", wg_alloc="connection", transport="direct")])
def test_lowered_plans_pass_random_interleavings(name, args, knobs):
    knobs = dict(knobs)
    k = knobs.pop("k")
    plan = host_plan(programs.REGISTRY[name](*args), k=k, **knobs)
    plan.check(seed=11, nsims=3)


def test_hierarchical_stages_pass_the_checker():
    for prog in (programs.hier_stage_reducescatter_intra(2, 4), programs.hier_stage_allreduce_inter(2, 4),
                 programs.hier_stage_allgather_intra(2, 4)):
        host_plan(prog, k=2).check(seed=5, nsims=2)


# ---------------------------------------------------------------- programs vs the oracle

ALL_PROGRAMS = [
    ("allreduce", programs.ring_allreduce(5), None),
    ("reducescatter", programs.ring_reducescatter(4), None),
    ("allgather", programs.ring_allgather(4), None),
    ("allreduce", programs.hierarchical_allreduce(3, 4), None),
    ("alltoall", programs.direct_alltoall(5), None),
    ("alltoall", programs.two_phase_alltoall(3, 4), None),
    ("alltonext", programs.alltonext(3, 4, split=True), None),
    ("alltonext", programs.alltonext(3, 4, split=False), None),
    ("allgather", programs.allgather_2d(3, 4), None),
    ("reducescatter", programs.reducescatter_2d(3, 4), None),
    ("reducescatter_intra", programs.hier_stage_reducescatter_intra(3, 4), 4),
    ("allreduce_inter", programs.hier_stage_allreduce_inter(3, 4), 4),
    ("allgather_intra", programs.hier_stage_allgather_intra(3, 4), 4),
    ("allreduce", programs.tree_allreduce(5), None),
    ("allreduce", programs.tree_allreduce(8, 2), None),
    ("allreduce", programs.tree_allreduce(1), None),
]


@pytest.mark.parametrize("coll,prog,L", ALL_PROGRAMS, ids=[p.name for _, p, _ in ALL_PROGRAMS])
def test_library_programs_meet_the_oracles_postcondition(coll, prog, L):
    assert OP.check_postcondition(prog.as_tuples(), coll, prog.nranks, prog.in_chunks, prog.scratch_chunks, L)


@pytest.mark.parametrize("P", [2, 3, 4, 8])
def test_ring_program_follows_the_documented_chain(P):
    """The package's ring program, run by the oracle's sequential interpreter, gives
    the same bits as the oracle's chain-order fold."""
    N = P * 37 + 3
    xs = W.make_inputs("normal_f32", N, P, 77, size_bytes=N)
    prog = programs.ring_allreduce(P)
    ys = OP.run_program(prog.as_tuples(), xs, "f32", prog.in_chunks, prog.out_chunks, prog.scratch_chunks)
    want = O2.ring_allreduce(xs, P, "f32")
    for r in range(P):
        assert np.array_equal(ys[r], want[r])


def test_hierarchical_and_2d_programs_follow_the_documented_chains():
    G, L = 3, 4
    P, N = G * L, 12 * 41
    xb = W.make_inputs("normal_bf16", N, P, 78, size_bytes=N)
    h = programs.hierarchical_allreduce(G, L)
    ys = OP.run_program(h.as_tuples(), xb, "bf16", h.in_chunks, h.out_chunks, h.scratch_chunks)
    want = O2.hierarchical_allreduce(xb, G, L, "bf16")
    assert all(np.array_equal(ys[r], want[r]) for r in range(P))
    xs = W.make_inputs("normal_f32", N, P, 79, size_bytes=N)
    rs = programs.reducescatter_2d(G, L)
    ys = OP.run_program(rs.as_tuples(), xs, "f32", rs.in_chunks, rs.out_chunks, rs.scratch_chunks)
    want = O2.reducescatter_2d(xs, G, L, "f32")
    assert all(np.array_equal(ys[r], want[r]) for r in range(P))


# ---------------------------------------------------------------- tuner (host logic)

def _space(factors, threads, slices, nvariants=1, protocols=1):
    arrs = [(C * len(v))(*v) for C, v in ((capi.C.c_int32, factors), (capi.C.c_int32, threads),
                                          (capi.C.c_int32, slices))]
    sp = capi.ccl_tune_space(capi.C.cast(arrs[0], capi.C.POINTER(capi.C.c_int32)), len(factors),
                             capi.C.cast(arrs[1], capi.C.POINTER(capi.C.c_int32)), len(threads),
                             capi.C.cast(arrs[2], capi.C.POINTER(capi.C.c_int32)), len(slices),
                             nvariants, 0, 1, protocols)
    sp._keep = arrs
    return sp


def test_coordinate_descent_finds_the_peak_of_a_unimodal_objective():
    """AutoCCL report, methods 1-2: each resource parameter is unimodal, so raising one
    coordinate until the objective stops improving reaches the peak."""
    F, T, S = [1, 2, 4, 8, 16, 24, 32], [64, 128, 256, 512, 1024], [4096 << i for i in range(8)]
    peak = (16, 256, 4096 << 5)

    def f(p):
        return 100 - abs(np.log2(p.parallel_factor) - 4) - abs(np.log2(p.nthreads) - 8) - \
            abs(np.log2(p.slice_bytes) - np.log2(peak[2]))
    best, rep = capi.ccl_tune_coordinate_descent(_space(F, T, S), f)
    assert (best.parallel_factor, best.nthreads, best.slice_bytes) == peak
    assert rep.best_score == pytest.approx(100)
    # one rising pass, then one confirming pass over the neighbours of the peak
    assert rep.evaluations <= 1 + len(F) + len(T) + len(S) + 3 + 12


def test_coordinate_descent_repeats_passes_when_coordinates_interact():
    """Coordinate descent repeats its passes until none moves: here the best thread
    count depends on the slice size (as measured for large ring AllReduces, where
    1024 threads win only with larger slices), so one rising pass stops at 512
    threads and a second pass raises it."""
    F, T, S = [32], [64, 128, 256, 512, 1024], [16384 << i for i in range(6)]

    def f(p):
        big = p.slice_bytes >= 262144
        t = {64: 1, 128: 2, 256: 3, 512: 5, 1024: 7 if big else 4}[p.nthreads]
        c = {16384: 0, 32768: 1, 65536: 2, 131072: 3, 262144: 4, 524288: 2}[p.slice_bytes]
        return 10.0 * t + c
    one_pass = max(f(type("P", (), dict(parallel_factor=32, nthreads=512, slice_bytes=sl))) for sl in S)
    best, rep = capi.ccl_tune_coordinate_descent(_space(F, T, S), f)
    assert (best.nthreads, best.slice_bytes) == (1024, 262144)
    assert rep.best_score == 74 > one_pass
    # an exhaustive search agrees
    pts = [(f(type("P", (), dict(parallel_factor=32, nthreads=t, slice_bytes=sl))), t, sl) for t in T for sl in S]
    assert max(pts)[0] == rep.best_score


def test_coordinate_descent_evaluates_each_point_once():
    seen = []

    def f(p):
        seen.append((p.parallel_factor, p.nthreads, p.slice_bytes, p.protocol, p.variant))
        return float(p.parallel_factor % 7 + p.nthreads // 64 + p.slice_bytes // 4096)
    best, rep = capi.ccl_tune_coordinate_descent(_space([1, 2, 4, 8, 16], [64, 128, 256], [4096, 8192, 16384],
                                                        nvariants=2, protocols=3), f)
    assert len(seen) == len(set(seen)) == rep.evaluations


def test_coordinate_descent_looks_past_one_dip_and_picks_the_subspace():
    F = [1, 2, 4, 8, 16, 24, 32]

    def f(p):
        # factor 24 is worse than 16 and 32 (idle compute units); protocol 1 is better
        base = {1: 1, 2: 2, 4: 4, 8: 8, 16: 16, 24: 12, 32: 20}[p.parallel_factor]
        return base + (5 if p.protocol == 1 else 0) + (3 if p.variant == 1 else 0)
    best, rep = capi.ccl_tune_coordinate_descent(_space(F, [256], [65536], nvariants=2, protocols=3), f)
    assert best.parallel_factor == 32 and best.protocol == 1 and best.variant == 1
    assert rep.best_score == 28


def test_coordinate_descent_also_starts_from_the_middle():
    """Every subspace gets a second descent from the middle of each coordinate: here the
    one from the corner stops behind a dip two candidates wide (past the one-step
    look-ahead), the one from the middle reaches the peak."""
    F = [1, 2, 4, 8, 16, 24, 32]

    def f(p):
        return float({1: 3, 2: 4, 4: 1, 8: 1, 16: 9, 24: 8, 32: 7}[p.parallel_factor])
    best, rep = capi.ccl_tune_coordinate_descent(_space(F, [256], [65536]), f)
    assert best.parallel_factor == 16 and rep.best_score == 9


def test_coordinate_descent_stops_on_infeasible_points():
    def f(p):
        return -1.0 if p.parallel_factor > 4 else float(p.parallel_factor)
    best, rep = capi.ccl_tune_coordinate_descent(_space([1, 2, 4, 8, 16], [256], [4096]), f)
    assert best.parallel_factor == 4


@pytest.mark.parametrize("name,args,k,knobs,all_skipped", [
    ("direct_alltoall", (8,), 1, dict(dtype="i32"), True),
    ("alltonext", (3, 4, False), 2, {}, True),
    ("alltonext", (3, 4, True), 2, {}, False),
    ("two_phase_alltoall", (2, 4), 1, dict(dtype="i32"), False),
    ("ring_allgather", (6,), 2, {}, False),
])
def test_idle_receives_are_skipped_and_their_senders_set_no_flag(name, args, k, knobs, all_skipped):
    """With direct transport a receive whose data the sender places, which stores nothing,
    sets no completion flag and precedes nothing in the dependency graph is skipped, and
    its sender sets no flag (and so never waits for its stores): direct AllToAll and
    unsplit AllToNext consist of such receives only. Random interleavings of the
    lowered plan still end in the postcondition."""
    plan = host_plan(programs.REGISTRY[name](*args), k, transport="direct", **knobs)
    ex = plan.export()
    recv_only = [e for e in ex if e.opcode & ~(capi.CCL_I_SKIP | capi.CCL_I_NOFLAG) == capi.CCL_I_RECV | capi.CCL_I_LOCAL_IN]
    skipped = [e for e in ex if e.opcode & capi.CCL_I_SKIP]
    assert skipped and all(e in recv_only for e in skipped) and all(e.done_flag < 0 for e in skipped)
    assert (len(skipped) == len(recv_only)) if all_skipped else (len(skipped) <= len(recv_only))
    assert {e.xout for e in ex if e.opcode & capi.CCL_I_NOFLAG} == {e.xin for e in skipped}
    plan.check(seed=5, nsims=4)
    # staged transport keeps every receive (it copies from the slot)
    staged = host_plan(programs.REGISTRY[name](*args), k, **knobs)
    assert not any(e.opcode & (capi.CCL_I_SKIP | capi.CCL_I_NOFLAG) for e in staged.export())
