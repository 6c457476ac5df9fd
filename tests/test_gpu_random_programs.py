"""GPU parity on seeded random chunk programs: random AllReduce reduction chains and
broadcast trees, random multi-hop AllToAll routes, each under a random scheduler,
workgroup allocation, protocol / transport, parallel factor, workgroup size, slice
size, kernel and (from seed 48 on) element type (the same cases pass the host plan
checker in test_random_programs_host.py). Every output must equal, bit for bit, the
oracle's sequential interpreter of the same program on the same inputs: the
executor may reorder work in time but must keep each chunk's association order."""

import numpy as np
import pytest

import workloads as W
from oracle import program as OP
from random_programs import case_typed

pytestmark = pytest.mark.gpu

SEEDS = list(range(96))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_program_matches_the_program_order_oracle(seed):
    from gpu_util import run

    prog, k, knobs, n, dtype = case_typed(seed)
    print(f"[case] seed {seed}: {prog.name} {dtype} k={k} {knobs} n={n}", flush=True)
    kind = {"f32": "normal_f32", "bf16": "normal_bf16", "i32": "uniform_i32"}[dtype]
    xs = W.make_inputs(kind, n, prog.nranks, 90, size_bytes=n * 4 + seed)
    ys, plan = run(prog, xs, dtype, k=k, **knobs)
    want = OP.run_program(prog.as_tuples(), xs, dtype, prog.in_chunks, prog.out_chunks, prog.scratch_chunks)
    for r in range(prog.nranks):
        assert np.array_equal(ys[r], want[r]), f"rank {r}"
    plan.destroy()
