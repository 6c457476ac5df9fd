"""GPU parity: the HIP executor, called through the C ABI, against the CPU oracle.

Bit-exact where the definitions or the schedule order fix the bits (integer data,
copy-only collectives, fp32/bf16 adds in each chain's order); scaled error bounds
against the float64 definition besides.
"""

import numpy as np
import pytest

import workloads as W
from chunk_schedule_execution_amd import programs
from oracle import definitions as O1
from oracle import numerics as nm
from oracle import schedule_order as O2

pytestmark = pytest.mark.gpu


def _run(*a, **k):
    from gpu_util import run
    return run(*a, **k)


def test_ring_allreduce_4r_1mib_integer_exact():
    """4 ranks, 1 MiB fp32 per rank, integer values in [-8, 8], 4 chunks, one channel,
    one slice: every partial sum is exact, so the result equals the definition bit for bit."""
    P, N = 4, 262144
    print(f"[case] ring AR P={P} N={N} f32 int-valued k=1", flush=True)
    xs = W.make_inputs("int_f32", N, P, W.CFG_RING_AR_4R_INT, size_bytes=N * 4)
    ys, plan = _run(programs.ring_allreduce(P), xs, "f32", k=1, slice_bytes=N // P * 4, nthreads=256)
    exact = O1.allreduce(xs, "f32").exact.astype(np.float32)
    o2 = O2.ring_allreduce(xs, P, "f32")
    for r in range(P):
        assert np.array_equal(ys[r], exact), r
        assert np.array_equal(ys[r], o2[r]), r
    assert plan.info()["num_workgroups"] == P
