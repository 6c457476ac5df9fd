"""Property tests of the host compiler on random chunk programs (hypothesis).

Random AllReduce programs give every chunk its own reduction chain (a random order of
the ranks, partials through scratch) and its own broadcast tree (each rank receives
the sum from a random rank that already holds it); random AllToAll programs send each
block directly or through a random intermediate rank. The routes, and so the DAGs,
the links and the channel use, are unlike any library program.

For every program and every scheduler / workgroup allocation / transport / parallel
factor drawn (ReSCCL report, section 2.2; MSCCLang report, section 3.1):
- the compiler's symbolic postcondition accepts it, and the oracle's own symbolic
  check (which shares no code with the compiler) agrees;
- every receive sits in a later sub-pipeline than its send;
- an HPDS sub-pipeline holds at most one send per link (rank, peer, channel);
- each workgroup runs its tasks in sub-pipeline order;
- inside one sub-pipeline a workgroup serves one (receive peer, send peer, channel)
  signature, also after state-based merging, which never uses more workgroups than
  connection-based allocation;
- the lowered plan runs to completion in random interleavings on the host, with
  outputs that meet the postcondition (no deadlock, no race).
"""

import collections

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from chunk_schedule_execution_amd import Plan, PlanConfig
from chunk_schedule_execution_amd.dsl import Buffer, Program
from oracle import program as OP

IN, OUT, SCR = Buffer.input, Buffer.output, Buffer.scratch


def host_plan(prog, k=1, **cfg):
    cfg.setdefault("max_count", 1 << 16)
    return Plan(prog, k, PlanConfig(host_only=True, nthreads=128, **cfg))


@st.composite
def random_allreduce(draw):
    P = draw(st.integers(2, 5))
    c = draw(st.integers(1, 2))
    C = P * c
    prog = Program("allreduce", P, C, C, scratch_chunks=C, name="random_allreduce")
    for j in range(C):
        order = draw(st.permutations(list(range(P))))
        ch = draw(st.integers(0, 1))
        cur = prog.chunk(order[0], IN, j)
        for step, r in enumerate(order[1:], start=1):
            dst = cur.copy(r, OUT if step == P - 1 else SCR, j, ch)
            dst.reduce(prog.chunk(r, IN, j), ch)
            cur = dst
        holders = [order[-1]]
        for r in draw(st.permutations(list(order[:-1]))):
            src = draw(st.sampled_from(holders))
            prog.chunk(src, OUT, j).copy(r, OUT, j, ch)
            holders.append(r)
    return prog


@st.composite
def random_alltoall(draw):
    P = draw(st.integers(2, 5))
    prog = Program("alltoall", P, P, P, scratch_chunks=P * P, name="random_alltoall")
    for s in range(P):
        for d in range(P):
            blk = prog.chunk(s, IN, d)  # block d of rank s becomes block s of rank d
            ch = draw(st.integers(0, 1))
            others = [m for m in range(P) if m not in (s, d)]
            if s != d and others and draw(st.booleans()):
                m = draw(st.sampled_from(others))
                blk = blk.copy(m, SCR, s * P + d, ch)
            blk.copy(d, OUT, s, ch)
    return prog


KNOBS = st.fixed_dictionaries({
    "k": st.integers(1, 2),
    "scheduler": st.sampled_from(["hpds", "rr", "program"]),
    "wg_alloc": st.sampled_from(["state", "connection"]),
    "transport": st.sampled_from(["staged", "direct"]),
})


def check_plan_properties(prog, knobs, seed):
    knobs = dict(knobs)
    k = knobs.pop("k")
    plan = host_plan(prog, k, **knobs)
    ex = plan.export()
    sender = {e.xout: e for e in ex if e.xout >= 0}
    for e in ex:
        assert e.subpipe >= 0
        if e.xin >= 0:
            assert sender[e.xin].subpipe < e.subpipe, "a receive must follow its send"
    if knobs["scheduler"] == "hpds":
        links = collections.Counter((e.instance, e.subpipe, e.rank, e.send_peer, e.channel)
                                    for e in ex if e.send_peer >= 0)
        assert max(links.values()) == 1, "two sends on one link in a sub-pipeline"
    by_wg = collections.defaultdict(list)
    for e in ex:
        by_wg[e.wg].append(e)
    for tasks in by_wg.values():
        assert len({t.rank for t in tasks}) == 1
        sps = [t.subpipe for t in tasks]
        assert sps == sorted(sps), "a workgroup runs its tasks in sub-pipeline order"
    # inside one sub-pipeline a workgroup serves one signature (receive peer, send peer,
    # channel); a task without a receive or a send fits any value there
    for tasks in by_wg.values():
        active = collections.defaultdict(lambda: (set(), set(), set()))
        for t in tasks:
            rp, sp, ch = active[t.subpipe]
            if t.recv_peer >= 0:
                rp.add(t.recv_peer)
            if t.send_peer >= 0:
                sp.add(t.send_peer)
            ch.add(t.channel)
        for rp, sp, ch in active.values():
            assert len(rp) <= 1 and len(sp) <= 1 and len(ch) == 1, "two links of one workgroup active together"
    if knobs["wg_alloc"] == "state":
        other = host_plan(prog, k, **dict(knobs, wg_alloc="connection"))
        assert plan.info()["num_workgroups"] <= other.info()["num_workgroups"]
    plan.check(seed=seed, nsims=2)


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(prog=random_allreduce(), knobs=KNOBS, seed=st.integers(0, 2**31))
def test_random_allreduce_programs(prog, knobs, seed):
    assert OP.check_postcondition(prog.as_tuples(), "allreduce", prog.nranks, prog.in_chunks, prog.scratch_chunks)
    check_plan_properties(prog, knobs, seed)


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(prog=random_alltoall(), knobs=KNOBS, seed=st.integers(0, 2**31))
def test_random_alltoall_programs(prog, knobs, seed):
    assert OP.check_postcondition(prog.as_tuples(), "alltoall", prog.nranks, prog.in_chunks, prog.scratch_chunks)
    check_plan_properties(prog, knobs, seed)


@settings(max_examples=60, deadline=None)
@given(prog=random_allreduce())
def test_random_allreduce_rr_and_hpds_agree_on_work(prog):
    """Schedulers and allocations reorder and regroup the same lowered instructions:
    each lowers the program to the same multiset of operations per rank."""
    def ops(plan):
        return sorted((e.rank, e.opcode, e.count, e.recv_peer, e.send_peer, e.chunk_id) for e in plan.export())
    base = ops(host_plan(prog, scheduler="program", wg_alloc="connection"))
    for sched in ("hpds", "rr"):
        for alloc in ("state", "connection"):
            assert ops(host_plan(prog, scheduler=sched, wg_alloc=alloc)) == base


def test_a_program_that_breaks_the_postcondition_is_refused():
    """The compiler's symbolic check rejects a chain that skips a rank (the oracle's
    check agrees), so the property tests above only see valid programs."""
    from chunk_schedule_execution_amd import capi

    P = 3
    prog = Program("allreduce", P, P, P, scratch_chunks=P, name="broken")
    for j in range(P):
        cur = prog.chunk(0, IN, j).copy(1, OUT, j)
        cur.reduce(prog.chunk(1, IN, j))  # rank 2's input never joins
        cur.copy(0, OUT, j)
        cur.copy(2, OUT, j)
    with pytest.raises(AssertionError, match="rank 0 output chunk 0"):
        OP.check_postcondition(prog.as_tuples(), "allreduce", P, P, P)
    with pytest.raises(capi.CCLError) as e:
        host_plan(prog)
    assert e.value.status == capi.CCL_ERR_INVALID_PROGRAM
