"""The seeded random programs that the GPU parity test runs, checked on the host first:
the compiler accepts every one, the oracle's symbolic postcondition agrees, and each
lowered plan runs to completion with a correct result in random interleavings of its
workgroups (no deadlock, no race) before any of them reaches a GPU."""

import pytest

from chunk_schedule_execution_amd import Plan, PlanConfig
from oracle import program as OP
from random_programs import case_typed

SEEDS = list(range(96))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_program_case_passes_the_host_checker(seed):
    prog, k, knobs, n, dtype = case_typed(seed)
    OP.check_postcondition(prog.as_tuples(), prog.collective, prog.nranks, prog.in_chunks, prog.scratch_chunks)
    plan = Plan(prog, k, PlanConfig(host_only=True, max_count=n, dtype=dtype, **knobs))
    plan.check(seed=seed, nsims=3)
