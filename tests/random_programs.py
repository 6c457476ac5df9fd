"""Seeded random chunk programs for tests (no hypothesis: the same seed gives the same
program on the host and on the GPU).

AllReduce: every chunk gets its own reduction chain (a random order of the ranks,
partials through scratch, the sum landing in the last rank's output) and its own
broadcast tree (each remaining rank receives from a random rank that already holds the
sum). AllToAll: every block goes directly or through a random intermediate rank's
scratch. Channels are drawn per chunk or block."""

import numpy as np

from chunk_schedule_execution_amd.dsl import Buffer, Program

IN, OUT, SCR = Buffer.input, Buffer.output, Buffer.scratch


def random_allreduce(rng: np.random.Generator, P: int, c: int = 1, channels: int = 2) -> Program:
    C = P * c
    prog = Program("allreduce", P, C, C, scratch_chunks=C, name=f"random_allreduce_p{P}")
    for j in range(C):
        order = [int(r) for r in rng.permutation(P)]
        ch = int(rng.integers(channels))
        cur = prog.chunk(order[0], IN, j)
        for step, r in enumerate(order[1:], start=1):
            dst = cur.copy(r, OUT if step == P - 1 else SCR, j, ch)
            dst.reduce(prog.chunk(r, IN, j), ch)
            cur = dst
        holders = [order[-1]]
        for r in [int(x) for x in rng.permutation(order[:-1])]:
            src = holders[int(rng.integers(len(holders)))]
            prog.chunk(src, OUT, j).copy(r, OUT, j, ch)
            holders.append(r)
    return prog


def random_alltoall(rng: np.random.Generator, P: int, channels: int = 2) -> Program:
    prog = Program("alltoall", P, P, P, scratch_chunks=P * P, name=f"random_alltoall_p{P}")
    for s in range(P):
        for d in range(P):
            blk = prog.chunk(s, IN, d)  # block d of rank s becomes block s of rank d
            ch = int(rng.integers(channels))
            others = [m for m in range(P) if m not in (s, d)]
            if s != d and others and rng.random() < 0.5:
                blk = blk.copy(others[int(rng.integers(len(others)))], SCR, s * P + d, ch)
            blk.copy(d, OUT, s, ch)
    return prog


def case(seed: int):
    """(program, parallel factor, plan knobs, elements per rank) of one seeded case."""
    rng = np.random.default_rng([2026, 77, seed])
    P = int(rng.integers(2, 7))
    if rng.random() < 0.7:
        c = int(rng.integers(1, 3))
        prog = random_allreduce(rng, P, c)
    else:
        prog = random_alltoall(rng, P)
    k = int(rng.integers(1, 4))
    knobs = {
        "scheduler": ["hpds", "rr", "program"][int(rng.integers(3))],
        "wg_alloc": ["state", "connection"][int(rng.integers(2))],
        "nthreads": [64, 128, 256][int(rng.integers(3))],
        "slice_bytes": [1024, 4096, 65536][int(rng.integers(3))],
    }
    proto = int(rng.integers(3))
    if proto == 1:
        knobs["protocol"] = "ll"
    elif proto == 2:
        knobs["transport"] = "direct"
    knobs["kernel"] = ["interpreter", "specialized"][int(rng.integers(2))]
    n = prog.in_chunks * int(rng.integers(200, 3000))
    if prog.collective == "allreduce":
        n += int(rng.integers(0, prog.in_chunks))  # ragged chunks; AllToAll moves whole blocks
    return prog, k, knobs, n


def case_typed(seed: int):
    """(program, parallel factor, plan knobs, elements per rank, dtype). Seeds below 48
    are case(seed) in fp32; from 48 on the element type cycles through fp32, bf16 and
    int32 and the parallel factor is drawn from 1..8, so instance pieces meet the 16-byte
    grid of both element sizes and empty pieces."""
    prog, k, knobs, n = case(seed)
    if seed < 48:
        return prog, k, knobs, n, "f32"
    rng = np.random.default_rng([2026, 78, seed])
    return prog, int(rng.integers(1, 9)), knobs, n, ("f32", "bf16", "i32")[seed % 3]

