"""ccl_execute_static, the entry point that allocates nothing, against ccl_execute.

Each case creates the same plan twice: once for ccl_execute (device memory of its own,
generated kernel) and once host-only (no device memory at all) for ccl_execute_static,
which runs on the library's static device scratch. Two calls in a row, the second with
a smaller input, must give the same bits from both entry points and the oracle's bits.
"""

import numpy as np
import pytest

import workloads as W
from chunk_schedule_execution_amd import Plan, PlanConfig, capi, programs
from oracle import definitions as O1
from oracle import schedule_order as O2

pytestmark = pytest.mark.gpu


def case(msg):
    print(f"[case] {msg}", flush=True)


def _both(prog, make_xs, want_of, dtype, k, counts, dev_kernel="specialized", **cfg):
    import torch

    from gpu_util import to_dev, to_host
    fill = {"f32": lambda j: np.float32(-3 - j), "i32": lambda j: np.int32(-3 - j),
            "bf16": lambda j: np.uint16(0xC040 + j)}[dtype]  # bf16 0xC040 = -3.0
    mc = max(counts)
    dev = Plan(prog, k, PlanConfig(dtype=dtype, max_count=mc, kernel=dev_kernel, **cfg))
    host = Plan(prog, k, PlanConfig(dtype=dtype, max_count=mc, host_only=True, **cfg))
    for j, N in enumerate(counts):
        xs = make_xs(N, j)
        ins = [to_dev(x, dtype) for x in xs]
        nout = dev.output_len(N)
        prior = [np.full(nout, fill(j)) for _ in xs]
        out_a = [to_dev(p, dtype) for p in prior]
        out_b = [to_dev(p, dtype) for p in prior]
        dev.execute(ins, out_a, N)
        host.execute_static(ins, out_b, N)
        torch.cuda.synchronize()
        dev.status()
        host.status()
        want = want_of(xs, prior)
        for r in range(len(xs)):
            a, b = to_host(out_a[r], dtype)[:nout], to_host(out_b[r], dtype)[:nout]
            assert np.array_equal(a, b), (prog.name, N, r)
            assert np.array_equal(b, want[r]), (prog.name, N, r)
        del ins, out_a, out_b
    dev.destroy()
    host.destroy()


def _ring_inputs(P, kind="normal_f32"):
    return lambda N, j: W.make_inputs(kind, N, P, W.CFG_RING_AR_8R, size_bytes=N * 4 + 1000 * j + 3)


@pytest.mark.parametrize("knobs", [dict(transport="direct"), dict(transport="staged"), dict(protocol="ll")])
def test_static_ring_allreduce_matches_execute(knobs):
    P = 8
    case(f"static ring AR {knobs}")
    # slots are sized for the largest count: staged 3 MiB per rank takes 42 MiB of the
    # static scratch, LL (twice the slot bytes) is run at 1 MiB
    counts = [262144, 65536 + 24] if knobs.get("protocol") == "ll" else [3 * 262144, 65536 + 24]
    _both(programs.ring_allreduce(P), _ring_inputs(P), lambda xs, _: [O2.ring_allreduce(xs, P, "f32")[0]] * P, "f32",
          32 if knobs.get("transport") == "direct" else 8, counts, nthreads=256, slice_bytes=32 << 10, **knobs)


def test_static_tree_hierarchical_alltoall_match_execute():
    """Scratch partials and completion waits (tree), bf16 (hierarchical), int32 copies
    through staging (two-phase AllToAll): the plans alternate, so the static scratch's
    tables are replaced between calls."""
    P = 8
    case("static tree AR")
    _both(programs.tree_allreduce(P), _ring_inputs(P), lambda xs, _: [O2.tree_allreduce(xs, P, "f32")[0]] * P, "f32",
          4, [8 * 40001, 8 * 999], slice_bytes=16 << 10)
    G, L = 2, 8
    case("static hierarchical bf16")
    _both(programs.hierarchical_allreduce(G, L),
          lambda N, j: W.make_inputs("normal_bf16", N, G * L, W.CFG_HIER_AR_16R_BF16, size_bytes=N * 2 + j),
          lambda xs, _: [O2.hierarchical_allreduce(xs, G, L, "bf16")[0]] * (G * L), "bf16", 2, [8 * 4099, 8 * 77],
          slice_bytes=8192)
    G, L = 4, 8
    case("static two-phase alltoall")
    _both(programs.two_phase_alltoall(G, L),
          lambda N, j: W.make_inputs("uniform_i32", N, G * L, W.CFG_A2A_32R_INT32, size_bytes=N * 4 + j),
          lambda xs, _: O1.alltoall(xs), "i32", 1, [32 * 1031, 32 * 17], nthreads=256)
    case("static alltonext split (rank 0 keeps its prior contents)")
    G, L = 3, 8
    _both(programs.alltonext(G, L, split=True),
          lambda N, j: W.make_inputs("normal_f32", N, G * L, W.CFG_A2NEXT_AGRS_24R, size_bytes=N * 4 + j),
          lambda xs, prior: O1.alltonext(xs, prior), "f32", 2, [8 * 777, 8 * 100])


def test_static_refuses_plans_beyond_the_array_and_reports_timeouts():
    """A staged ring at 256 MiB per rank needs far more slots than the static scratch
    holds: OUT_OF_RESOURCES, nothing launched. A dropped flag (failure injection) makes
    the static launch time out under its watchdog; ccl_plan_status reports it, and a
    healthy static call afterwards is exact."""
    import torch

    from gpu_util import to_dev
    P = 8
    case("static: too large, and a watchdog expiry")
    big = Plan(programs.ring_allreduce(P), 8, PlanConfig(max_count=1 << 26, host_only=True))
    g = big.info()["count_granule"]
    x = [torch.zeros(g, device="cuda:0") for _ in range(P)]
    y = [torch.zeros(g, device="cuda:0") for _ in range(P)]
    with pytest.raises(capi.CCLError) as e:
        big.execute_static(x, y, g)
    assert e.value.status == capi.CCL_ERR_OUT_OF_RESOURCES
    big.destroy()
    N = 4 * 4096
    xs = W.make_inputs("int_f32", N, 4, W.CFG_RING_AR_4R_INT, size_bytes=N * 4)
    ins = [to_dev(v, "f32") for v in xs]
    outs = [torch.empty(N, device="cuda:0") for _ in range(4)]
    bad = Plan(programs.ring_allreduce(4), 2, PlanConfig(max_count=N, nthreads=256, timeout_us=20000,
                                                         debug_drop_flag=True, host_only=True))
    bad.execute_static(ins, outs, N)
    with pytest.raises(capi.CCLError) as e:
        bad.status()
    assert e.value.status == capi.CCL_ERR_TIMEOUT
    bad.destroy()
    good = Plan(programs.ring_allreduce(4), 2, PlanConfig(max_count=N, nthreads=256, host_only=True))
    good.execute_static(ins, outs, N)
    good.status()
    want = O1.allreduce(xs, "f32").exact.astype(np.float32)
    for r in range(4):
        assert np.array_equal(outs[r].cpu().numpy(), want), r
    good.destroy()
