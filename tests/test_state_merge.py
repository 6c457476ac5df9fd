"""State-based workgroup allocation against the colouring optimum (ReSCCL report,
section 2.2: connections never active in the same sub-pipeline share a workgroup).

Per rank, the connection-based workgroups of a plan and the sub-pipelines each is
active in form the input of the merge. The most of them active in one sub-pipeline is a
lower bound on any merge. When every activity set is an interval the conflict graph is
an interval graph, the bound is the optimum, and the greedy first-fit by first
activation must reach it; in general the merge must stay between the bound and the
connection count."""

import collections

import numpy as np
import pytest

from chunk_schedule_execution_amd import Plan, PlanConfig, programs
from random_programs import random_allreduce, random_alltoall


def plan(prog, alloc):
    return Plan(prog, 1, PlanConfig(host_only=True, scheduler="hpds", wg_alloc=alloc, nthreads=128))


def per_rank(prog):
    conn, state = plan(prog, "connection").export(), plan(prog, "state").export()
    active = collections.defaultdict(set)
    for e in conn:
        active[(e.rank, e.wg)].add(e.subpipe)
    for r in range(prog.nranks):
        sets = [v for (rr, _), v in active.items() if rr == r]
        bound = max(collections.Counter(sp for s in sets for sp in s).values()) if sets else 0
        intervals = all(max(s) - min(s) + 1 == len(s) for s in sets)
        merged = len({e.wg for e in state if e.rank == r})
        yield r, len(sets), merged, bound, intervals


def programs_under_test():
    progs = [programs.alltonext(3, 4, split=True), programs.two_phase_alltoall(2, 4), programs.reducescatter_2d(3, 4),
             programs.allgather_2d(3, 4), programs.hierarchical_allreduce(2, 4), programs.tree_allreduce(8)]
    for seed in range(80):
        rng = np.random.default_rng([9, seed])
        P = int(rng.integers(2, 6))
        progs.append(random_allreduce(rng, P, 1) if rng.random() < 0.5 else random_alltoall(rng, P))
    return progs


def test_the_bound_on_a_hand_checked_case():
    """Three connections active in {0}, {1} and {0, 1}: two at once at most, and two
    workgroups suffice ({0} with {1}, and {0, 1} alone)."""
    sets = [{0}, {1}, {0, 1}]
    assert max(collections.Counter(sp for s in sets for sp in s).values()) == 2


def test_state_merge_meets_the_colouring_optimum():
    seen = collections.Counter()
    for prog in programs_under_test():
        for r, nconn, merged, bound, intervals in per_rank(prog):
            assert bound <= merged <= nconn, (prog.name, r)
            if intervals:
                assert merged == bound, (prog.name, r, merged, bound)
            seen["interval" if intervals else "general"] += 1
    assert seen["interval"] >= 50 and seen["general"] >= 50, seen


@pytest.mark.parametrize("G,L", [(3, 4), (3, 8)])
def test_split_alltonext_merges_below_connection_count(G, L):
    """The pages' own motivating case: most connections of the split AllToNext are idle
    most of the time, so merging saves workgroups."""
    prog = programs.alltonext(G, L, split=True)
    total_conn = sum(n for _, n, _, _, _ in per_rank(prog))
    total_merged = sum(m for _, _, m, _, _ in per_rank(prog))
    assert total_merged < total_conn
