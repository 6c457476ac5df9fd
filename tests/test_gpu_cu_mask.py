"""Compute units reserved for the collective (AutoCCL report, method 3 and its
interference results; ReSCCL report, section 1: thread blocks taken from computation):
a CU-masked stream keeps its kernels on its CUs, a plan sized to that budget fits them,
and the collective keeps the oracle's bits while GEMMs run on the complementary CUs.

Masked streams each hold a hardware queue of their own, which the runtime hands out
sparingly (creating a seventh in one process has failed with out-of-memory), so this
module creates two and shares them."""

import numpy as np
import pytest

import workloads as W
from chunk_schedule_execution_amd import Plan, PlanConfig, capi, programs
from oracle import schedule_order as O2

pytestmark = pytest.mark.gpu

COMM_CUS = 32  # mask bits 0..31: four CUs on each of the eight XCDs


def case(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def streams():
    comm = capi.ccl_stream_create_cu_masked(capi.cu_mask_words(range(COMM_CUS)))
    rest = capi.ccl_stream_create_cu_masked(capi.cu_mask_words(range(COMM_CUS, 256)))
    yield comm, rest
    import torch
    torch.cuda.synchronize()
    capi.ccl_stream_destroy(comm)
    capi.ccl_stream_destroy(rest)


def test_masked_streams_keep_to_their_compute_units(streams):
    """Workgroups of the 32-CU stream land on 32 distinct CUs, four per XCD; those of
    the complementary stream on the other 224, never on the first 32."""
    comm, rest = streams
    case("placement of masked streams")
    a = set(capi.ccl_cu_probe(comm, 512, 50))
    b = set(capi.ccl_cu_probe(rest, 2048, 50))
    assert len(a) == COMM_CUS
    per_xcd = {}
    for x, *_ in a:
        per_xcd[x] = per_xcd.get(x, 0) + 1
    assert per_xcd == {x: COMM_CUS // 8 for x in range(8)}
    assert len(b) == 256 - COMM_CUS and not (a & b)


def test_collective_on_reserved_cus_beside_gemms(streams):
    """A ring AllReduce plan sized to the 32-CU budget runs on the masked stream while
    bf16 GEMMs keep the other 224 CUs busy: the bits of the chain order, launch after
    launch on fresh inputs, and no watchdog expiry."""
    import torch

    from gpu_util import run
    comm, rest = streams
    P, N = 8, 3 * 65536 + 24
    case("ring AR on 32 reserved CUs beside GEMMs")
    a = torch.randn(4096, 4096, device="cuda:0").to(torch.bfloat16)
    b = torch.randn(4096, 4096, device="cuda:0").to(torch.bfloat16).contiguous()
    c = torch.empty(4096, 4096, device="cuda:0", dtype=torch.bfloat16)
    torch.cuda.synchronize()
    gemm_stream = torch.cuda.ExternalStream(rest)
    comm_stream = torch.cuda.ExternalStream(comm)
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=N * 4 + 73)
    for knobs in (dict(k=4, nthreads=256, transport="direct", kernel="specialized"), dict(k=8, nthreads=256),
                  dict(k=4, nthreads=512, protocol="ll")):
        case(f"  {knobs}")
        with torch.cuda.stream(gemm_stream):
            for _ in range(30):
                torch.matmul(a, b, out=c)
        with torch.cuda.stream(comm_stream):
            ys, plan = run(programs.ring_allreduce(P), xs, "f32", num_cus=COMM_CUS, repeat=3,
                           check=lambda y, x, _: _all_equal(y, O2.ring_allreduce(x, P, "f32")[0]), **knobs)
        _all_equal(ys, O2.ring_allreduce(xs, P, "f32")[0])
        assert plan.info()["max_resident_wgs"] <= COMM_CUS * 8
        plan.destroy()
    torch.cuda.synchronize()


def test_budget_refuses_a_grid_larger_than_its_cus():
    """k=32 at 1024 threads needs 256 co-resident workgroups of the interpreting kernel:
    more than 32 CUs hold."""
    with pytest.raises(capi.CCLError) as e:
        Plan(programs.ring_allreduce(8), 32, PlanConfig(max_count=1 << 16, nthreads=1024, num_cus=COMM_CUS))
    assert e.value.status == capi.CCL_ERR_OUT_OF_RESOURCES


def _all_equal(ys, want):
    for r, y in enumerate(ys):
        assert np.array_equal(y, want), r
