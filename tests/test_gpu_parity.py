"""GPU parity: the HIP executor, called through the C ABI, against the CPU oracle.

Bit-exact where the definitions or the schedule order fix the bits (integer data,
copy-only collectives, fp32 / bf16 adds in each chain's order); besides that the
scaled error against the float64 definition: max |y - s| / sum|x| <= 1e-6 * P for
fp32 and <= 2e-2 for bf16 (fp32 accumulate, bf16 stores).
"""

import numpy as np
import pytest

import workloads as W
from chunk_schedule_execution_amd import programs
from oracle import definitions as O1
from oracle import numerics as nm
from oracle import schedule_order as O2

pytestmark = pytest.mark.gpu

F32_TOL = lambda P: 1e-6 * P  # noqa: E731
BF16_TOL = 2e-2


def _run(*a, **k):
    from gpu_util import run
    return run(*a, **k)


def case(msg):
    print(f"[case] {msg}", flush=True)


def assert_all_equal(ys, want):
    for r, y in enumerate(ys):
        if not np.array_equal(y, want):
            bad = np.nonzero(y != want)[0]
            raise AssertionError(f"rank {r}: {bad.size} elements differ, first at {bad[:5]}: {y[bad[:5]]} vs {want[bad[:5]]}")


def chk_ring(P, dtype="f32"):
    """Check of one launch of a repeated run: the ring's chain order on that launch's inputs."""
    return lambda ys, xs, prior: assert_all_equal(ys, O2.ring_allreduce(xs, P, dtype)[0])


def chk_tree(nchunks, dtype="f32"):
    return lambda ys, xs, prior: assert_all_equal(ys, O2.tree_allreduce(xs, nchunks, dtype)[0])


def chk_hier(G, L, dtype="bf16"):
    return lambda ys, xs, prior: assert_all_equal(ys, O2.hierarchical_allreduce(xs, G, L, dtype)[0])


def chk_per_rank(want_of):
    """want_of(xs, prior) gives every rank's expected output."""
    def check(ys, xs, prior):
        want = want_of(xs, prior)
        for r in range(len(ys)):
            assert np.array_equal(ys[r], want[r]), r
    return check


def chk_alltoall():
    return chk_per_rank(lambda xs, prior: O1.alltoall(xs))


def chk_allgather():
    return chk_per_rank(lambda xs, prior: [O1.allgather(xs)] * len(xs))


# ------------------------------------------------------------------ ring AllReduce

def test_ring_allreduce_4r_1mib_integer_exact():
    """4 ranks, 1 MiB fp32 per rank, integer values in [-8, 8], 4 chunks, one channel,
    one slice: every partial sum is exact, so the result equals the definition bit for bit."""
    P, N = 4, 262144
    case(f"ring AR P={P} N={N} f32 int-valued k=1")
    xs = W.make_inputs("int_f32", N, P, W.CFG_RING_AR_4R_INT, size_bytes=N * 4)
    ys, plan = _run(programs.ring_allreduce(P), xs, "f32", k=1, slice_bytes=N // P * 4, nthreads=256)
    exact = O1.allreduce(xs, "f32").exact.astype(np.float32)
    assert_all_equal(ys, exact)
    assert_all_equal(ys, O2.ring_allreduce(xs, P, "f32")[0])
    assert plan.info()["num_workgroups"] == P


@pytest.mark.parametrize("S", [32 << 10, 1 << 20])
@pytest.mark.parametrize("k", [1, 2, 4, 8, 16, 24])
def test_ring_allreduce_8r_fp32(S, k):
    """8 ranks, fp32 N(0,1), 8 chunks, k parallel instances (k=24 gives ragged,
    unaligned sub-chunks): bit-exact against the chain-order oracle, within the fp32
    bound of the definition, identical on every rank."""
    P, N = 8, S // 4
    case(f"ring AR P={P} S={S} k={k}")
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=S)
    ys, _ = _run(programs.ring_allreduce(P), xs, "f32", k=k, slice_bytes=64 << 10)
    assert_all_equal(ys, O2.ring_allreduce(xs, P, "f32")[0])
    ref = O1.allreduce(xs, "f32")
    assert nm.scaled_error(ys[0], ref.exact, ref.abs_sum, "f32") <= F32_TOL(P)


@pytest.mark.parametrize("knobs", [
    dict(nthreads=64, slice_bytes=4096, scheduler="program", wg_alloc="connection"),
    dict(nthreads=1024, slice_bytes=1 << 20, scheduler="rr", wg_alloc="connection"),
    dict(nthreads=256, slice_bytes=8192, scheduler="hpds", wg_alloc="state"),
])
def test_knob_invariance(knobs):
    """Threads, slice size, scheduler and workgroup allocation change the time order
    only: the bits stay those of the chain order."""
    P, N = 8, 100_000
    case(f"ring AR knobs {knobs}")
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=N * 4)
    ys, _ = _run(programs.ring_allreduce(P), xs, "f32", k=3, **knobs)
    assert_all_equal(ys, O2.ring_allreduce(xs, P, "f32")[0])


@pytest.mark.parametrize("P,N,k", [(1, 1000, 1), (2, 4099, 2), (3, 7, 1), (8, 5, 1), (8, 1001, 24), (5, 123457, 7)])
def test_ring_edge_shapes(P, N, k):
    """One rank (a copy), two ranks (one correctly rounded add), fewer elements than
    chunks (empty chunks), odd lengths with many instances (unaligned pieces)."""
    case(f"ring AR edge P={P} N={N} k={k}")
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=N * 4 + 1)
    ys, _ = _run(programs.ring_allreduce(P), xs, "f32", k=k, slice_bytes=4096)
    assert_all_equal(ys, O2.ring_allreduce(xs, P, "f32")[0])
    if P == 2:
        assert_all_equal(ys, (xs[0].astype(np.float64) + xs[1].astype(np.float64)).astype(np.float32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("knobs", [dict(transport="staged", kernel="interpreter"),
                                   dict(transport="direct", kernel="specialized"),
                                   dict(protocol="ll", kernel="specialized")])
@pytest.mark.parametrize("N", [8 * 10, 8 * 37 + 3])
def test_ring_instances_shorter_than_the_16_byte_grid(dtype, knobs, N):
    """Instance bounds sit on the 16-byte grid of their chunk, so with chunks of a few
    elements and k = 24 most pieces are empty and the rest hold a multiple of 16 bytes'
    worth (the last one the remainder). Chain order, bit for bit, three launches."""
    P = 8
    case(f"ring AR tiny chunks N={N} k=24 {dtype} {knobs}")
    kind = "normal_f32" if dtype == "f32" else "normal_bf16"
    xs = W.make_inputs(kind, N, P, W.CFG_RING_AR_8R, size_bytes=N * 4 + 3)
    chk = chk_ring(P, dtype)
    ys, _ = _run(programs.ring_allreduce(P), xs, dtype, k=24, nthreads=128, slice_bytes=4096, repeat=3, check=chk,
                 **knobs)
    chk(ys, xs, None)


@pytest.mark.parametrize("knobs", [dict(transport="staged", kernel="interpreter"),
                                   dict(transport="direct", kernel="specialized"),
                                   dict(protocol="ll", kernel="specialized")])
def test_bf16_special_values_round_like_the_oracle(knobs):
    """bf16 sums whose fp32 results are NaNs with payloads (signalling and quiet inputs),
    infinities, overflows and subnormals: every stored bf16 is the oracle's, NaNs as the
    quiet NaN 0x7fc0 (the conversion instruction alone would keep part of the payload).
    NaNs are positive and +inf never meets -inf, so which operand's NaN an add returns
    cannot change the bits."""
    P, N = 8, 8 * 4096 + 37
    case(f"bf16 ring AR special values {knobs}")
    xs = [np.asarray(x, np.uint16).copy() for x in W.make_inputs("normal_bf16", N, P, W.CFG_RING_AR_8R)]
    rng = np.random.default_rng(5)
    col = np.arange(N)
    for r in range(P):
        x = xs[r]
        nan1 = col % 7 == 1
        x[nan1 & (rng.integers(0, P, N) == r)] = rng.choice(np.array([0x7F81, 0x7FC1, 0x7FFF, 0x7FA5], np.uint16))
        x[(col % 7 == 2) & (r < 2)] = np.uint16(0x7F95) if r == 0 else np.uint16(0x7FC3)
        x[(col % 7 == 3) & (r == 3)] = np.uint16(0x7F80)                       # +inf among finite values
        x[col % 7 == 4] = np.uint16(0x7F7F)                                      # largest finite: the sum overflows
        x[col % 7 == 5] = rng.integers(1, 0x80, int(np.count_nonzero(col % 7 == 5))).astype(np.uint16)  # subnormal
    want = O2.ring_allreduce(xs, P, "bf16")[0]
    assert np.count_nonzero(want == 0x7FC0) > N // 8 and np.count_nonzero(want == 0x7F80) > N // 8
    ys, _ = _run(programs.ring_allreduce(P), xs, "bf16", k=3, nthreads=256, slice_bytes=8192, **knobs)
    assert_all_equal(ys, want)


def test_ring_subnormals_are_kept():
    P, N = 8, 4096
    case("ring AR subnormal inputs")
    xs = W.make_inputs("normal_f32_denorm", N, P, W.CFG_RING_AR_8R, size_bytes=N * 4)
    ys, _ = _run(programs.ring_allreduce(P), xs, "f32", k=2)
    want = O2.ring_allreduce(xs, P, "f32")[0]
    assert np.count_nonzero(want) > N // 2
    assert_all_equal(ys, want)


@pytest.mark.parametrize("algo", ["ring", "tree"])
@pytest.mark.parametrize("transport,kernel", [("staged", "interpreter"), ("direct", "interpreter"),
                                              ("direct", "specialized")])
def test_repeated_launches_and_counts(algo, transport, kernel):
    """Epoch-valued flags: back-to-back launches need no reset; one plan serves several
    counts up to max_count (direct transport: the landings move with the count)."""
    P = 8
    prog = programs.ring_allreduce(P) if algo == "ring" else programs.tree_allreduce(P)
    oracle = O2.ring_allreduce if algo == "ring" else O2.tree_allreduce
    from chunk_schedule_execution_amd import Plan, PlanConfig
    plan = Plan(prog, 4, PlanConfig(dtype="f32", max_count=50_000, slice_bytes=8192, transport=transport,
                                    kernel=kernel))
    check = chk_ring(P) if algo == "ring" else chk_tree(P)
    for N in (50_000, 777, 50_000, 12_345, 1):
        case(f"{algo} AR {transport} {kernel} repeated N={N}")
        xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=N * 4 + 7)
        ys, _ = _run(prog, xs, "f32", plan=plan, repeat=3, check=check)
        assert_all_equal(ys, oracle(xs, P, "f32")[0])
    plan.destroy()


@pytest.mark.parametrize("S,k,nt,sl,knobs", [
    (3 << 20, 8, 512, 256 << 10, dict(kernel="interpreter")),
    (3 << 20, 32, 256, 64 << 10, dict(transport="direct", kernel="specialized")),  # the factor_32 point
    (3 << 20, 24, 256, 16 << 10, dict(transport="direct", kernel="specialized")),  # the benchmark's headline point
    (32 << 20, 32, 512, 64 << 10, dict(transport="direct", streaming=True, kernel="specialized")),
    (256 << 20, 32, 512, 256 << 10, dict(transport="direct", streaming=True, kernel="specialized"))])
def test_ring_allreduce_8r_full_size_sampled(S, k, nt, sl, knobs):
    """Full sizes in the benchmark's launch configurations: sampled elements against the
    chain-order oracle, the fp32 bound everywhere sampled, and all ranks identical over
    the whole buffer."""
    P, N = 8, S // 4
    case(f"ring AR full size S={S} k={k} nt={nt} {knobs}")
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=S)
    rng = np.random.default_rng(1)
    idx = np.unique(np.concatenate([rng.integers(0, N, 4000), [0, N - 1], np.arange(N // P - 3, N // P + 3)]))

    def sampled(ys, xj, prior):
        for r in range(1, P):
            assert np.array_equal(ys[r], ys[0])
        assert np.array_equal(ys[0][idx], O2.ring_allreduce_at(xj, P, idx, "f32"))
    ys, _ = _run(programs.ring_allreduce(P), xs, "f32", k=k, nthreads=nt, slice_bytes=sl, repeat=2, check=sampled,
                 **knobs)
    for r in range(1, P):
        assert np.array_equal(ys[r], ys[0])
    assert np.array_equal(ys[0][idx], O2.ring_allreduce_at(xs, P, idx, "f32"))
    ref = O1.allreduce_at(xs, idx, "f32")
    assert nm.scaled_error(ys[0][idx], ref.exact, ref.abs_sum, "f32") <= F32_TOL(P)


def test_hierarchical_allreduce_16r_bf16_64mib_sampled():
    """The 2 x 8 bf16 hierarchical AllReduce at 64 MiB per rank in the benchmark's kind
    of launch (generated kernel, direct transport, k=16): sampled elements against the
    oracle's chain order, all ranks identical."""
    G, L = 2, 8
    P, N = G * L, (64 << 20) // 2
    case(f"hierarchical bf16 64 MiB sampled")
    xs = W.make_inputs("normal_bf16", N, P, W.CFG_HIER_AR_16R_BF16, size_bytes=64 << 20)
    ys, _ = _run(programs.hierarchical_allreduce(G, L), xs, "bf16", k=16, nthreads=512, slice_bytes=256 << 10,
                 transport="direct", kernel="specialized")
    for r in range(1, P):
        assert np.array_equal(ys[r], ys[0])
    rng = np.random.default_rng(2)
    idx = np.unique(np.concatenate([rng.integers(0, N, 4000), [0, N - 1]]))
    assert np.array_equal(ys[0][idx], O2.hierarchical_allreduce_at(xs, G, L, idx, "bf16"))


# ------------------------------------------------------------------ hierarchical, bf16

@pytest.mark.parametrize("k", [1, 2])
def test_hierarchical_allreduce_16r_bf16(k):
    """2 groups x 8 ranks, bf16 N(0,1), fp32 accumulate with a bf16 store at every step:
    bit-exact against the three-step chain order, within 2e-2 of the definition."""
    G, L, N = 2, 8, 1 << 19
    case(f"hier AR bf16 G={G} L={L} N={N} k={k}")
    xs = W.make_inputs("normal_bf16", N, G * L, W.CFG_HIER_AR_16R_BF16, size_bytes=N * 2)
    ys, _ = _run(programs.hierarchical_allreduce(G, L), xs, "bf16", k=k)
    assert_all_equal(ys, O2.hierarchical_allreduce(xs, G, L, "bf16")[0])
    ref = O1.allreduce(xs, "bf16")
    assert nm.scaled_error(ys[0], ref.exact, ref.abs_sum, "bf16") <= BF16_TOL


def test_hierarchical_fused_equals_three_launches():
    """The single fused kernel and the three separate collectives (reduce-scatter in the
    group, AllReduce across groups, all-gather in the group) give the same bits."""
    G, L, N = 2, 8, 8 * 4096 + 8 * 3
    case("hier AR fused vs three launches")
    xs = W.make_inputs("normal_bf16", N, G * L, W.CFG_HIER_AR_16R_BF16, size_bytes=N * 2 + 1)
    fused, _ = _run(programs.hierarchical_allreduce(G, L), xs, "bf16", k=2)
    t1, _ = _run(programs.hier_stage_reducescatter_intra(G, L), xs, "bf16", count=N)
    t2, _ = _run(programs.hier_stage_allreduce_inter(G, L), t1, "bf16", count=N // L)
    t3, _ = _run(programs.hier_stage_allgather_intra(G, L), t2, "bf16", count=N // L)
    assert_all_equal(fused, O2.hierarchical_allreduce(xs, G, L, "bf16")[0])
    for r in range(G * L):
        assert np.array_equal(t3[r], fused[r]), r


# ------------------------------------------------------------------ AllToAll, int32

@pytest.mark.parametrize("name", ["two_phase", "direct"])
def test_alltoall_32r_int32(name):
    """4 groups x 8 ranks, int32 uniform over the full range, 1 MiB per rank: the output
    is exactly the transposed block permutation."""
    G, L, N = 4, 8, 1 << 18
    P = G * L
    case(f"alltoall {name} P={P} N={N}")
    xs = W.make_inputs("uniform_i32", N, P, W.CFG_A2A_32R_INT32, size_bytes=N * 4)
    prog = programs.two_phase_alltoall(G, L) if name == "two_phase" else programs.direct_alltoall(P)
    ys, _ = _run(prog, xs, "i32", k=1, nthreads=256)
    want = O1.alltoall(xs)
    for r in range(P):
        assert np.array_equal(ys[r], want[r]), r


def test_alltoall_provenance_decodes():
    G, L = 4, 8
    P, b = G * L, 333
    case("two-phase alltoall provenance")
    xs = [W.provenance_i32(P * b, r) for r in range(P)]
    ys, _ = _run(programs.two_phase_alltoall(G, L), xs, "i32", k=2, nthreads=128)
    for r in range(P):
        y = ys[r].astype(np.int64)
        pos = np.arange(P * b)
        assert np.array_equal(y >> 20, pos // b)
        assert np.array_equal(y & (2**20 - 1), r * b + pos % b)


# ------------------------------------------------------------------ AllToNext, AG, RS (24 ranks)

@pytest.mark.parametrize("split", [True, False])
def test_alltonext_24r(split):
    """rank r's buffer lands at rank r+1; rank 0's output keeps its prior contents."""
    G, L, N = 3, 8, (1 << 18) + 8 * 5
    P = G * L
    case(f"alltonext split={split} N={N}")
    xs = W.make_inputs("normal_f32", N, P, W.CFG_A2NEXT_AGRS_24R, size_bytes=N * 4)
    prior = [np.full(N, -3.0, np.float32) for _ in range(P)]
    ys, _ = _run(programs.alltonext(G, L, split=split), xs, "f32", k=2, prior=prior)
    want = O1.alltonext(xs, prior)
    for r in range(P):
        assert np.array_equal(ys[r], want[r]), r


@pytest.mark.parametrize("variant", ["ring", "2d"])
@pytest.mark.parametrize("sched,alloc", [("hpds", "state"), ("rr", "connection")])
def test_allgather_24r(variant, sched, alloc):
    G, L = 3, 8
    P, n = G * L, 4097
    case(f"allgather {variant} {sched}/{alloc}")
    xs = W.make_inputs("normal_f32", n, P, W.CFG_A2NEXT_AGRS_24R, size_bytes=n * 4)
    prog = programs.ring_allgather(P) if variant == "ring" else programs.allgather_2d(G, L)
    ys, _ = _run(prog, xs, "f32", k=2, scheduler=sched, wg_alloc=alloc)
    want = O1.allgather(xs)
    for r in range(P):
        assert np.array_equal(ys[r], want), r


@pytest.mark.parametrize("variant", ["ring", "2d"])
@pytest.mark.parametrize("sched,alloc", [("hpds", "state"), ("rr", "connection")])
def test_reducescatter_24r(variant, sched, alloc):
    G, L = 3, 8
    P = G * L
    N = P * 4099
    case(f"reducescatter {variant} {sched}/{alloc}")
    xs = W.make_inputs("normal_f32", N, P, W.CFG_A2NEXT_AGRS_24R, size_bytes=N * 4)
    prog = programs.ring_reducescatter(P) if variant == "ring" else programs.reducescatter_2d(G, L)
    ys, _ = _run(prog, xs, "f32", k=2, scheduler=sched, wg_alloc=alloc)
    want = O2.ring_reducescatter(xs, P, "f32") if variant == "ring" else O2.reducescatter_2d(xs, G, L, "f32")
    ref = O1.reducescatter(xs, "f32")
    for r in range(P):
        assert np.array_equal(ys[r], want[r]), r
        assert nm.scaled_error(ys[r], ref[r].exact, ref[r].abs_sum, "f32") <= F32_TOL(P)


@pytest.mark.parametrize("coll", ["allgather", "reducescatter"])
def test_24r_ring_at_three_workgroups_per_cu(coll):
    """k=32 x 512 threads on 24 ranks: 768 workgroups, three per compute unit. Only the
    generated kernel compiled for that occupancy holds them all; the outputs keep the
    bits of the oracle (provenance copies for AllGather, chain order for ReduceScatter)."""
    P = 24
    case(f"{coll} 24 ranks k=32 nt=512 generated, 3 workgroups per CU")
    if coll == "allgather":
        n = 32 * 1001 + 5
        xs = W.make_inputs("prov_i32", n, P, W.CFG_A2NEXT_AGRS_24R, size_bytes=n * 4)
        ys, plan = _run(programs.ring_allgather(P), xs, "i32", k=32, nthreads=512, slice_bytes=4096,
                        transport="direct", streaming=True, kernel="specialized")
        want = O1.allgather(xs)
        for r in range(P):
            assert np.array_equal(ys[r], want), r
    else:
        N = P * (32 * 301 + 3)
        xs = W.make_inputs("normal_f32", N, P, W.CFG_A2NEXT_AGRS_24R, size_bytes=N * 4)
        ys, plan = _run(programs.ring_reducescatter(P), xs, "f32", k=32, nthreads=512, slice_bytes=4096,
                        transport="direct", streaming=True, kernel="specialized")
        want = O2.ring_reducescatter(xs, P, "f32")
        for r in range(P):
            assert np.array_equal(ys[r], want[r]), r
    info = plan.info()
    assert info["num_workgroups"] == 768 and info["max_resident_wgs"] >= 768
    plan.destroy()


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("kernel", ["interpreter", "specialized"])
@pytest.mark.parametrize("transport", ["staged", "direct"])
def test_reducescatter_shards_off_the_16_byte_grid_streaming(dtype, kernel, transport):
    """ReduceScatter whose shards are no multiple of 16 bytes, streaming variant: the
    last hop of every chain reads at the shard's phase (slot or landing, and the input)
    and writes the output at 0, so it goes element by element with eight elements per
    thread in flight, and the last pass of a piece is partial. Chain order, bit for bit,
    two launches on different inputs."""
    P, n = 5, 3 * 2048 + 7
    N = P * n
    case(f"reducescatter off-grid shards {dtype} {kernel} {transport} streaming")
    kind = {"f32": "normal_f32", "bf16": "normal_bf16", "i32": "uniform_i32"}[dtype]
    xs = W.make_inputs(kind, N, P, W.CFG_A2NEXT_AGRS_24R)
    chk = chk_per_rank(lambda x, _: O2.ring_reducescatter(x, P, dtype))
    ys, plan = _run(programs.ring_reducescatter(P), xs, dtype, k=2, nthreads=256, slice_bytes=64 << 10,
                    transport=transport, streaming=True, kernel=kernel, repeat=2, check=chk)
    chk(ys, xs, None)
    plan.destroy()


def test_int32_reduction_wraps():
    P, N = 4, 1000
    case("ring AR int32 wrap")
    xs = [np.full(N, 2**31 - 1, np.int32), np.ones(N, np.int32), np.full(N, -5, np.int32), np.arange(N, dtype=np.int32)]
    ys, _ = _run(programs.ring_allreduce(P), xs, "i32", k=1)
    want = O1.allreduce(xs, "i32").exact
    assert_all_equal(ys, want)


# ------------------------------------------------------------------ low-latency protocol

@pytest.mark.parametrize("P,N,k", [(8, 8192, 1), (8, 786432, 24), (8, 1001, 3), (4, 262144, 1), (2, 5, 1)])
def test_ll_ring_allreduce(P, N, k):
    """Flag-in-data units instead of slice flags: same bits as the chain order."""
    case(f"LL ring AR P={P} N={N} k={k}")
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=N * 4 + 3)
    ys, plan = _run(programs.ring_allreduce(P), xs, "f32", k=k, protocol="ll", nthreads=256)
    assert_all_equal(ys, O2.ring_allreduce(xs, P, "f32")[0])


@pytest.mark.parametrize("N", [(1 << 16) + 16, 8 * 1001 + 8])
def test_ll_hierarchical_bf16_odd_lengths(N):
    """bf16 pairs share a 4-byte unit: odd chunk lengths leave a half-filled last unit."""
    G, L = 2, 8
    case(f"LL hier AR bf16 N={N}")
    xs = W.make_inputs("normal_bf16", N, G * L, W.CFG_HIER_AR_16R_BF16, size_bytes=N * 2 + 5)
    ys, _ = _run(programs.hierarchical_allreduce(G, L), xs, "bf16", k=2, protocol="ll")
    assert_all_equal(ys, O2.hierarchical_allreduce(xs, G, L, "bf16")[0])


def test_ll_alltoall_and_alltonext():
    G, L = 4, 8
    P, b = G * L, 1037
    case("LL two-phase alltoall + alltonext")
    xs = W.make_inputs("uniform_i32", P * b, P, W.CFG_A2A_32R_INT32, size_bytes=P * b * 4 + 9)
    ys, _ = _run(programs.two_phase_alltoall(G, L), xs, "i32", k=1, protocol="ll", nthreads=256)
    want = O1.alltoall(xs)
    for r in range(P):
        assert np.array_equal(ys[r], want[r]), r
    G, L, N = 3, 8, 8 * 777
    xs = W.make_inputs("normal_f32", N, G * L, W.CFG_A2NEXT_AGRS_24R, size_bytes=N * 4 + 9)
    prior = [np.full(N, -3.0, np.float32) for _ in range(G * L)]
    ys, _ = _run(programs.alltonext(G, L, split=True), xs, "f32", k=2, prior=prior, protocol="ll")
    want = O1.alltonext(xs, prior)
    for r in range(G * L):
        assert np.array_equal(ys[r], want[r]), r


def test_ll_repeated_launches():
    """LL flags are the launch's epoch: repeated launches over the same slots stay exact."""
    P, N = 8, 50_000
    case("LL ring AR repeated")
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=N * 4 + 11)
    ys, _ = _run(programs.ring_allreduce(P), xs, "f32", k=4, protocol="ll", repeat=5, check=chk_ring(P))
    assert_all_equal(ys, O2.ring_allreduce(xs, P, "f32")[0])


# ------------------------------------------------------------------ slot store policy

@pytest.mark.parametrize("protocol", ["simple", "ll"])
@pytest.mark.parametrize("k,nt,num_cus", [(8, 256, 0), (3, 512, 0), (32, 1024, 0), (5, 256, 10)])
def test_xcd_local_and_coherent_stores_agree(protocol, k, nt, num_cus):
    """An XCD-aligned layout writes transfers with plain stores and sets each flag with a
    plain store when the receiving workgroup published the sender's own XCD, else with a
    release; under LL the units themselves are plain stores for such a receiver and
    agent-coherent stores for any other. With a budget of 10 CUs the layout estimate rejects the aligned grid: the plan keeps
    coherent stores, or (forced) runs the XCD-local variant with most receivers on other
    XCDs, so both flag kinds occur. Every way the bits are the chain order, launch after
    launch."""
    P, N = 8, 3 * 65536 + 24
    case(f"ring AR store policy {protocol} k={k} nt={nt} num_cus={num_cus}")
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=N * 4 + 13)
    want = O2.ring_allreduce(xs, P, "f32")[0]
    modes = [dict(xcd_local=True), dict(xcd_local=False)]
    if num_cus == 10:
        modes.append(dict(xcd_local=True, force_xcd_local=True))
    for mode in modes:
        ys, plan = _run(programs.ring_allreduce(P), xs, "f32", k=k, protocol=protocol, nthreads=nt,
                        slice_bytes=16 << 10, repeat=4, check=chk_ring(P), num_cus=num_cus, **mode)
        info = plan.info()
        aligned = num_cus != 10
        assert info["xcd_local"] == (1 if mode["xcd_local"] and (aligned or mode.get("force_xcd_local")) else 0)
        if num_cus == 10:
            assert info["grid_workgroups"] == P * k  # no XCD padding
        assert_all_equal(ys, want)


def test_xcd_local_hierarchical_and_alltoall():
    G, L, N = 2, 8, 8 * 4099
    case("store policy: hierarchical bf16, two-phase alltoall")
    xs = W.make_inputs("normal_bf16", N, G * L, W.CFG_HIER_AR_16R_BF16, size_bytes=N * 2 + 17)
    want = O2.hierarchical_allreduce(xs, G, L, "bf16")[0]
    for xcd_local in (True, False):
        ys, _ = _run(programs.hierarchical_allreduce(G, L), xs, "bf16", k=2, xcd_local=xcd_local, repeat=3,
                     check=chk_hier(G, L),
                     slice_bytes=8192)
        assert_all_equal(ys, want)
    G, L, b = 4, 8, 513
    P = G * L
    xs = W.make_inputs("uniform_i32", P * b, P, W.CFG_A2A_32R_INT32, size_bytes=P * b * 4 + 17)
    want = O1.alltoall(xs)
    for xcd_local in (True, False):
        ys, _ = _run(programs.two_phase_alltoall(G, L), xs, "i32", k=1, xcd_local=xcd_local, repeat=3, check=chk_alltoall(),
                     nthreads=256)
        for r in range(P):
            assert np.array_equal(ys[r], want[r]), r


# ------------------------------------------------------------------ tree AllReduce

@pytest.mark.parametrize("P,c,N,k,dtype", [(8, 1, 786432, 8, "f32"), (8, 2, 8 * 1001 + 5, 3, "f32"),
                                           (5, 1, 123457, 7, "f32"), (3, 1, 7, 1, "f32"), (1, 1, 1000, 1, "f32"),
                                           (16, 1, 16 * 4099, 2, "bf16"), (24, 1, 24 * 513, 1, "f32")])
@pytest.mark.parametrize("mode", ["staged", "direct", "ll"])
def test_tree_allreduce(P, c, N, k, dtype, mode):
    """Heap tree per chunk rooted at its owner: the bits of the documented tree order,
    for every transport and protocol, over repeated launches."""
    case(f"tree AR P={P} c={c} N={N} k={k} {dtype} {mode}")
    kind = "normal_bf16" if dtype == "bf16" else "normal_f32"
    xs = W.make_inputs(kind, N, P, W.CFG_TREE_AR, size_bytes=N * 4 + P)
    knobs = dict(protocol="ll") if mode == "ll" else dict(transport=mode)
    ys, _ = _run(programs.tree_allreduce(P, c), xs, dtype, k=k, slice_bytes=8192, repeat=2,
                 check=chk_tree(P * c, dtype), **knobs)
    assert_all_equal(ys, O2.tree_allreduce(xs, P * c, dtype)[0])


def test_tree_allreduce_integer_exact():
    P, N = 8, 1 << 18
    case(f"tree AR P={P} N={N} int-valued")
    xs = W.make_inputs("int_f32", N, P, W.CFG_TREE_AR, size_bytes=N * 4)
    ys, _ = _run(programs.tree_allreduce(P), xs, "f32", k=4)
    assert_all_equal(ys, O1.allreduce(xs, "f32").exact.astype(np.float32))


# ------------------------------------------------------------------ plan-specialized kernels

@pytest.mark.parametrize("kernel", ["specialized", "lazy"])
@pytest.mark.parametrize("P,N,k,sl,knobs", [(8, 3 * 65536 + 24, 8, 8192, dict(transport="direct")),
                                            (5, 123457, 3, 4096, {}),
                                            (8, 8 * 1001, 2, 65536, dict(protocol="ll")),
                                            (8, 1 << 20, 4, 65536, dict(transport="direct", streaming=True))])
def test_specialized_ring_allreduce(kernel, P, N, k, sl, knobs):
    """Generated kernels (task order and the lazy slice-outer order, which here runs up
    to dozens of slices per instruction) give the chain-order bits."""
    case(f"{kernel} ring AR P={P} N={N} k={k} slice={sl} {knobs}")
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=N * 4 + 37)
    ys, plan = _run(programs.ring_allreduce(P), xs, "f32", k=k, slice_bytes=sl, kernel=kernel, repeat=3,
                    check=chk_ring(P), **knobs)
    assert plan.info()["specialized_shapes"] == 1
    assert_all_equal(ys, O2.ring_allreduce(xs, P, "f32")[0])


@pytest.mark.parametrize("kernel", ["specialized", "lazy"])
def test_specialized_other_collectives(kernel):
    """Generated kernels for the other small programs: the three hierarchical stages
    (bf16, chained like the three-launch composition), 24-rank ring AllGather and
    ReduceScatter, direct AllToAll and unsplit AllToNext."""
    G, L, N = 2, 8, 8 * 4099
    P = G * L
    case(f"{kernel} hierarchical stages bf16")
    xs = W.make_inputs("normal_bf16", N, P, W.CFG_HIER_AR_16R_BF16, size_bytes=N * 2 + 41)
    sh = N // L
    mid, _ = _run(programs.hier_stage_reducescatter_intra(G, L), xs, "bf16", k=2, slice_bytes=4096, kernel=kernel)
    mid2, _ = _run(programs.hier_stage_allreduce_inter(G, L), mid, "bf16", k=2, count=sh, kernel=kernel)
    ys, plan = _run(programs.hier_stage_allgather_intra(G, L), mid2, "bf16", k=2, count=sh, slice_bytes=4096,
                    kernel=kernel)
    assert plan.info()["specialized_shapes"] >= 1
    assert_all_equal(ys, O2.hierarchical_allreduce(xs, G, L, "bf16")[0])
    G, L = 3, 8
    P, n = G * L, 24 * 41
    xs = W.make_inputs("prov_i32", n, P, W.CFG_A2NEXT_AGRS_24R, size_bytes=n * 4 + 43)
    case(f"{kernel} ring allgather 24")
    ys, _ = _run(programs.ring_allgather(P), xs, "i32", k=2, transport="direct", kernel=kernel)
    assert_all_equal(ys, O1.allgather(xs))
    xs = W.make_inputs("normal_f32", n * P, P, W.CFG_A2NEXT_AGRS_24R, size_bytes=n * P * 4 + 43)
    case(f"{kernel} ring reducescatter 24")
    ys, _ = _run(programs.ring_reducescatter(P), xs, "f32", k=2, slice_bytes=4096, kernel=kernel)
    want = O2.ring_reducescatter(xs, P, "f32")
    for r in range(P):
        assert np.array_equal(ys[r], want[r]), r
    P, b = 8, 1031
    xs = W.make_inputs("uniform_i32", P * b, P, W.CFG_A2A_32R_INT32, size_bytes=P * b * 4 + 43)
    case(f"{kernel} direct alltoall 8")
    ys, _ = _run(programs.direct_alltoall(P), xs, "i32", k=1, transport="direct", kernel=kernel)
    want = O1.alltoall(xs)
    for r in range(P):
        assert np.array_equal(ys[r], want[r]), r
    N = 8 * 777
    case(f"{kernel} alltonext unsplit")
    xs = W.make_inputs("normal_f32", N, G * L, W.CFG_A2NEXT_AGRS_24R, size_bytes=N * 4 + 43)
    prior = [np.full(N, -3.0, np.float32) for _ in range(G * L)]
    ys, _ = _run(programs.alltonext(G, L, split=False), xs, "f32", k=2, prior=prior, slice_bytes=4096, kernel=kernel)
    want = O1.alltonext(xs, prior)
    for r in range(G * L):
        assert np.array_equal(ys[r], want[r]), r


@pytest.mark.parametrize("kernel", ["specialized_loop", "lazy"])
def test_generated_loop_form_long_programs(kernel):
    """The loop form (one step per distinct operation word) on the long programs: split
    AllToNext, and with the task order also the plans with completion waits: fused
    hierarchical bf16, 2-D ReduceScatter, tree and two-phase AllToAll."""
    G, L, N = 2, 8, 8 * 4099
    if kernel != "lazy":  # the fused hierarchical plan has completion waits
        case(f"{kernel} fused hierarchical bf16")
        xs = W.make_inputs("normal_bf16", N, G * L, W.CFG_HIER_AR_16R_BF16, size_bytes=N * 2 + 53)
        ys, plan = _run(programs.hierarchical_allreduce(G, L), xs, "bf16", k=2, slice_bytes=4096, kernel=kernel,
                        repeat=2, check=chk_hier(G, L))
        assert 0 < plan.info()["specialized_instructions"] <= 12
        assert_all_equal(ys, O2.hierarchical_allreduce(xs, G, L, "bf16")[0])
    G, L, N = 3, 8, 8 * 777
    case(f"{kernel} alltonext split")
    xs = W.make_inputs("normal_f32", N, G * L, W.CFG_A2NEXT_AGRS_24R, size_bytes=N * 4 + 53)
    prior = [np.full(N, -3.0, np.float32) for _ in range(G * L)]
    ys, _ = _run(programs.alltonext(G, L, split=True), xs, "f32", k=2, prior=prior, slice_bytes=4096, kernel=kernel)
    want = O1.alltonext(xs, prior)
    for r in range(G * L):
        assert np.array_equal(ys[r], want[r]), r
    if kernel == "lazy":  # the remaining plans have completion waits
        return
    P, n = G * L, 24 * 41
    xs = W.make_inputs("normal_f32", n * P, P, W.CFG_A2NEXT_AGRS_24R, size_bytes=n * P * 4 + 53)
    case(f"{kernel} reducescatter 2d")
    ys, _ = _run(programs.reducescatter_2d(G, L), xs, "f32", k=2, kernel=kernel)
    want = O2.reducescatter_2d(xs, G, L, "f32")
    for r in range(P):
        assert np.array_equal(ys[r], want[r]), r
    P, N = 8, 8 * 3001
    case(f"{kernel} tree AR")
    xs = W.make_inputs("normal_f32", N, P, W.CFG_TREE_AR, size_bytes=N * 4 + 53)
    ys, _ = _run(programs.tree_allreduce(P), xs, "f32", k=4, kernel=kernel, repeat=2, check=chk_tree(P))
    assert_all_equal(ys, O2.tree_allreduce(xs, P, "f32")[0])
    G, L, b = 4, 8, 257
    P = G * L
    case(f"{kernel} two-phase alltoall")
    xs = W.make_inputs("uniform_i32", P * b, P, W.CFG_A2A_32R_INT32, size_bytes=P * b * 4 + 53)
    ys, _ = _run(programs.two_phase_alltoall(G, L), xs, "i32", k=1, transport="direct", nthreads=256, kernel=kernel)
    want = O1.alltoall(xs)
    for r in range(P):
        assert np.array_equal(ys[r], want[r]), r


def test_specialized_kernel_trace():
    """The generated kernel keeps the per-workgroup and per-instruction trace."""
    P, N = 8, 8 * 4096
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=N * 4 + 47)
    ys, plan = _run(programs.ring_allreduce(P), xs, "f32", k=2, kernel="specialized", trace=True)
    assert_all_equal(ys, O2.ring_allreduce(xs, P, "f32")[0])
    wg, it = plan.trace(instructions=True)
    ran = [w for w in wg if w[3] > 0]
    assert len(ran) == plan.info()["num_workgroups"]
    assert sum(w[3] for w in ran) == plan.info()["num_instructions"]
    assert all(r[2] >= r[0] > 0 for r in it)


# ------------------------------------------------------------------ under compute interference

def test_collectives_under_concurrent_gemms():
    """bf16 GEMMs keep a second stream (default priority) busy while ring and tree
    AllReduce plans run on the main one: the bits stay those of the oracle and no wait
    times out, although the GEMMs hold compute units the executor's workgroups wait for."""
    import torch
    side = torch.cuda.Stream()
    a = torch.randn(4096, 4096, device="cuda:0").to(torch.bfloat16)
    b = torch.randn(4096, 4096, device="cuda:0").to(torch.bfloat16).contiguous()
    c = torch.empty(4096, 4096, device="cuda:0", dtype=torch.bfloat16)
    torch.cuda.synchronize()
    P, N = 8, 3 * 65536 + 24
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=N * 4 + 31)
    for prog, want, chk, knobs in ((programs.ring_allreduce(P), O2.ring_allreduce(xs, P, "f32")[0], chk_ring(P),
                                    dict(k=32, transport="direct")),
                                   (programs.tree_allreduce(P), O2.tree_allreduce(xs, P, "f32")[0], chk_tree(P),
                                    dict(k=8)),
                                   (programs.ring_allreduce(P), O2.ring_allreduce(xs, P, "f32")[0], chk_ring(P),
                                    dict(k=8, protocol="ll"))):
        case(f"{prog.name} {knobs} under GEMMs")
        with torch.cuda.stream(side):
            for _ in range(40):
                torch.matmul(a, b, out=c)
        ys, _ = _run(prog, xs, "f32", repeat=4, check=chk, **knobs)
        assert_all_equal(ys, want)


# ------------------------------------------------------------------ direct transport

@pytest.mark.parametrize("P,N,k", [(2, 4099, 2), (3, 7, 1), (8, 3 * 65536 + 24, 8), (8, 8 * 1001, 24), (5, 123457, 7)])
@pytest.mark.parametrize("xcd_local", [True, False])
def test_direct_ring_allreduce(P, N, k, xcd_local):
    """Senders write the all-gather hops straight into the receivers' outputs; the
    receivers forward from there. Same chain-order bits, repeated launches."""
    case(f"direct ring AR P={P} N={N} k={k} xcd_local={xcd_local}")
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=N * 4 + 19)
    ys, plan = _run(programs.ring_allreduce(P), xs, "f32", k=k, transport="direct", xcd_local=xcd_local,
                    slice_bytes=8192, repeat=3, check=chk_ring(P))
    assert any(e.opcode & 0x10 for e in plan.export())
    assert_all_equal(ys, O2.ring_allreduce(xs, P, "f32")[0])


def test_direct_other_collectives():
    """Hierarchical bf16, two-phase and direct AllToAll, split AllToNext, ring and 2-D
    AllGather / ReduceScatter with direct transport."""
    G, L, N = 2, 8, 8 * 4099
    case("direct hierarchical bf16")
    xs = W.make_inputs("normal_bf16", N, G * L, W.CFG_HIER_AR_16R_BF16, size_bytes=N * 2 + 23)
    ys, _ = _run(programs.hierarchical_allreduce(G, L), xs, "bf16", k=2, transport="direct", repeat=2,
                 check=chk_hier(G, L))
    assert_all_equal(ys, O2.hierarchical_allreduce(xs, G, L, "bf16")[0])
    G, L, b = 4, 8, 257
    P = G * L
    xs = W.make_inputs("uniform_i32", P * b, P, W.CFG_A2A_32R_INT32, size_bytes=P * b * 4 + 23)
    want = O1.alltoall(xs)
    for prog in (programs.two_phase_alltoall(G, L), programs.direct_alltoall(P)):
        case(f"direct {prog.name}")
        ys, _ = _run(prog, xs, "i32", k=1, transport="direct", nthreads=256, repeat=2, check=chk_alltoall())
        for r in range(P):
            assert np.array_equal(ys[r], want[r]), r
    G, L, N = 3, 8, 8 * 777
    case("direct alltonext split")
    xs = W.make_inputs("normal_f32", N, G * L, W.CFG_A2NEXT_AGRS_24R, size_bytes=N * 4 + 23)
    prior = [np.full(N, -3.0, np.float32) for _ in range(G * L)]
    ys, _ = _run(programs.alltonext(G, L, split=True), xs, "f32", k=2, prior=prior, transport="direct")
    want = O1.alltonext(xs, prior)
    for r in range(G * L):
        assert np.array_equal(ys[r], want[r]), r
    P, n = G * L, 24 * 41
    xs = W.make_inputs("prov_i32", n, P, W.CFG_A2NEXT_AGRS_24R, size_bytes=n * 4 + 29)
    for prog in (programs.ring_allgather(P), programs.allgather_2d(G, L)):
        case(f"direct {prog.name}")
        ys, _ = _run(prog, xs, "i32", k=2, transport="direct")
        assert_all_equal(ys, O1.allgather(xs))
    xs = W.make_inputs("normal_f32", n * P, P, W.CFG_A2NEXT_AGRS_24R, size_bytes=n * P * 4 + 29)
    case("direct ring reducescatter")
    ys, _ = _run(programs.ring_reducescatter(P), xs, "f32", k=2, transport="direct")
    want = O2.ring_reducescatter(xs, P, "f32")
    for r in range(P):
        assert np.array_equal(ys[r], want[r]), r


@pytest.mark.parametrize("transport", ["staged", "direct"])
def test_streaming_hints_keep_the_bits(transport):
    """Non-temporal hints on local traffic are cache policy only: same bits."""
    P, N = 8, 3 * 65536 + 40
    case(f"streaming ring AR {transport}")
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=N * 4 + 31)
    ys, _ = _run(programs.ring_allreduce(P), xs, "f32", k=8, transport=transport, streaming=True, repeat=2,
                 check=chk_ring(P),
                 slice_bytes=16 << 10)
    assert_all_equal(ys, O2.ring_allreduce(xs, P, "f32")[0])
    G, L, N = 2, 8, 8 * 2051
    case(f"streaming hierarchical bf16 {transport}")
    xs = W.make_inputs("normal_bf16", N, G * L, W.CFG_HIER_AR_16R_BF16, size_bytes=N * 2 + 31)
    ys, _ = _run(programs.hierarchical_allreduce(G, L), xs, "bf16", k=2, transport=transport, streaming=True)
    assert_all_equal(ys, O2.hierarchical_allreduce(xs, G, L, "bf16")[0])
    # bf16 in the streaming variant moves four vectors per thread per pass: several full
    # passes per instruction, odd chunk lengths (unaligned heads) and ragged tails
    P, N = 8, 3 * 262144 + 40
    case(f"streaming ring AR bf16 {transport}")
    xs = W.make_inputs("normal_bf16", N, P, W.CFG_HIER_AR_16R_BF16, size_bytes=N * 2 + 7)
    ys, _ = _run(programs.ring_allreduce(P), xs, "bf16", k=4, nthreads=256, transport=transport, streaming=True,
                 slice_bytes=64 << 10, repeat=2, check=chk_ring(P, "bf16"))
    assert_all_equal(ys, O2.ring_allreduce(xs, P, "bf16")[0])


@pytest.mark.parametrize("transport", ["staged", "direct"])
def test_streaming_copies_several_passes(transport):
    """Streaming copies and forwards of 32-bit data move eight vectors per thread per
    pass: pieces of several passes and slices, odd lengths (unaligned heads, ragged
    tails), int32 provenance values that must all land in rank order."""
    P, n = 8, 3 * 65536 + 13
    case(f"streaming ring AllGather {transport}")
    xs = W.make_inputs("prov_i32", n, P, W.CFG_A2NEXT_AGRS_24R, size_bytes=n * 4)
    ys, _ = _run(programs.ring_allgather(P), xs, "i32", k=2, nthreads=256, slice_bytes=64 << 10,
                 transport=transport, streaming=True, kernel="specialized", repeat=2,
                 check=chk_allgather())
    want = O1.allgather(xs)
    for r in range(P):
        assert np.array_equal(ys[r], want), r


@pytest.mark.parametrize("kernel", ["interpreter", "specialized"])
def test_watchdog_ends_a_launch_whose_flag_never_comes(kernel):
    """Failure detection: transfer 0's sender never sets its flag (failure injection),
    so its receiver waits out a 20 ms watchdog budget, records CCL_ERR_TIMEOUT and
    aborts the launch; every other waiter leaves, the launch ends, and the status call
    reports the timeout. Later launches of the same plan fail the same way, and a
    healthy plan afterwards still matches the oracle."""
    import time

    import torch

    from chunk_schedule_execution_amd import Plan, PlanConfig, capi
    from gpu_util import to_dev

    P, N = 4, 4 * 4096
    case(f"watchdog, dropped flag, {kernel} kernel")
    xs = W.make_inputs("int_f32", N, P, W.CFG_RING_AR_4R_INT, size_bytes=N * 4)
    ins = [to_dev(x, "f32") for x in xs]
    outs = [torch.empty(N, device="cuda:0") for _ in range(P)]
    bad = Plan(programs.ring_allreduce(P), 2, PlanConfig(dtype="f32", max_count=N, nthreads=256, timeout_us=20000,
                                                         debug_drop_flag=True, kernel=kernel))
    for launch in range(2):
        t0 = time.perf_counter()
        bad.execute(ins, outs, N)
        with pytest.raises(capi.CCLError) as e:
            bad.status()
        assert e.value.status == capi.CCL_ERR_TIMEOUT, str(e.value)
        assert time.perf_counter() - t0 < 5.0
    bad.destroy()
    ys, _ = _run(programs.ring_allreduce(P), xs, "f32", k=2, nthreads=256, kernel=kernel)
    assert_all_equal(ys, O1.allreduce(xs, "f32").exact.astype(np.float32))


def test_execute_refuses_graph_capture():
    """Each launch carries a fresh epoch: a graph would replay a stale one."""
    import torch
    from chunk_schedule_execution_amd import Plan, PlanConfig, capi
    P, N = 4, 1024
    case("graph capture refused")
    plan = Plan(programs.ring_allreduce(P), 1, PlanConfig(max_count=N))
    ins = [torch.zeros(N, device="cuda:0") for _ in range(P)]
    outs = [torch.empty(N, device="cuda:0") for _ in range(P)]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    err = None
    try:
        with torch.cuda.graph(g, stream=s):
            try:
                plan.execute(ins, outs, N, s)
            except capi.CCLError as e:
                err = e
    except RuntimeError:
        pass  # torch may reject the empty capture itself
    assert err is not None and err.status == capi.CCL_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    plan.execute(ins, outs, N)  # the plan still works outside the capture
    torch.cuda.synchronize()
    plan.status()
    plan.destroy()


# ------------------------------------------------------------------ debug poison, link utilisation, CU budget

@pytest.mark.parametrize("what", ["ring_staged", "ring_ll", "ring_direct", "tree_scratch", "hier_bf16", "a2a_two_phase"])
def test_debug_poison_changes_no_bits(what):
    """CCL_FLAG_DEBUG_POISON fills the staging slots and scratch with 0xFA bytes before
    every launch: a read of a slot or a scratch partial before its producer wrote it in
    this launch would carry the sentinel into the outputs. Launch after launch on fresh
    inputs the bits stay the oracle's."""
    P, N = 8, 3 * 65536 + 24
    case(f"debug poison {what}")
    if what.startswith("ring"):
        xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=N * 4 + 61)
        knobs = {"ring_staged": dict(), "ring_ll": dict(protocol="ll"), "ring_direct": dict(transport="direct")}[what]
        ys, plan = _run(programs.ring_allreduce(P), xs, "f32", k=8, slice_bytes=16 << 10, debug_poison=True, repeat=3,
                        check=chk_ring(P), **knobs)
        assert_all_equal(ys, O2.ring_allreduce(xs, P, "f32")[0])
        assert plan.info()["staging_bytes"] > 0 or what == "ring_direct"
    elif what == "tree_scratch":
        xs = W.make_inputs("normal_f32", N, P, W.CFG_TREE_AR, size_bytes=N * 4 + 61)
        ys, plan = _run(programs.tree_allreduce(P), xs, "f32", k=4, slice_bytes=16 << 10, debug_poison=True, repeat=3,
                        check=chk_tree(P), kernel="specialized")
        assert plan.info()["scratch_bytes"] > 0
        assert_all_equal(ys, O2.tree_allreduce(xs, P, "f32")[0])
    elif what == "hier_bf16":
        G, L, N = 2, 8, 8 * 4099
        xs = W.make_inputs("normal_bf16", N, G * L, W.CFG_HIER_AR_16R_BF16, size_bytes=N * 2 + 61)
        ys, _ = _run(programs.hierarchical_allreduce(G, L), xs, "bf16", k=2, slice_bytes=4096, debug_poison=True,
                     repeat=2, check=chk_hier(G, L))
        assert_all_equal(ys, O2.hierarchical_allreduce(xs, G, L, "bf16")[0])
    else:
        G, L, b = 4, 8, 517
        P = G * L
        xs = W.make_inputs("uniform_i32", P * b, P, W.CFG_A2A_32R_INT32, size_bytes=P * b * 4 + 61)
        ys, _ = _run(programs.two_phase_alltoall(G, L), xs, "i32", k=1, nthreads=256, debug_poison=True, repeat=2,
                     check=chk_alltoall())
        want = O1.alltoall(xs)
        for r in range(P):
            assert np.array_equal(ys[r], want[r]), r


def test_link_busy_fractions_of_a_traced_ring():
    """Link utilisation from the device trace: one record per (src, dst, channel,
    instance) connection of the 8-rank ring (P * k of them), every fraction in (0, 1]."""
    P, N, k = 8, 8 * 65536, 4
    case("link busy fractions, ring AR traced")
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=N * 4 + 67)
    ys, plan = _run(programs.ring_allreduce(P), xs, "f32", k=k, slice_bytes=32 << 10, trace=True,
                    kernel="specialized")
    assert_all_equal(ys, O2.ring_allreduce(xs, P, "f32")[0])
    links = plan.link_busy()
    assert len(links) == P * k
    assert {(s, d) for s, d, _, _, _ in links} == {(r, (r + 1) % P) for r in range(P)}
    assert all(0.0 < f <= 1.0 for *_, f in links), links
    plan.destroy()


def test_cu_budget_bounds_the_grid():
    """A plan created for a budget of 16 compute units is checked against 16 CUs'
    occupancy: a grid larger than that is refused, one within it runs and keeps the
    oracle's bits (the budget only shrinks the bound; it reserves nothing)."""
    from chunk_schedule_execution_amd import Plan, PlanConfig, capi
    P, N = 8, 8 * 4096
    case("CU budget 16")
    full = Plan(programs.ring_allreduce(P), 4, PlanConfig(max_count=N, nthreads=1024))
    budget = Plan(programs.ring_allreduce(P), 2, PlanConfig(max_count=N, nthreads=1024, num_cus=16))
    per_cu = full.info()["max_resident_wgs"] // 256
    assert budget.info()["max_resident_wgs"] == per_cu * 16
    full.destroy()
    budget.destroy()
    with pytest.raises(capi.CCLError) as e:
        Plan(programs.ring_allreduce(P), 32, PlanConfig(max_count=N, nthreads=1024, num_cus=16))
    assert e.value.status == capi.CCL_ERR_OUT_OF_RESOURCES
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=N * 4 + 71)
    ys, _ = _run(programs.ring_allreduce(P), xs, "f32", k=2, nthreads=256, num_cus=16, kernel="specialized")
    assert_all_equal(ys, O2.ring_allreduce(xs, P, "f32")[0])


def test_chrome_trace_export_of_a_launch(tmp_path):
    """The device trace of a launch as Chrome / Perfetto trace events: one complete event
    per instruction of the plan, on the thread of its workgroup, inside the launch's span."""
    import json

    from chunk_schedule_execution_amd.trace_export import write_chrome_trace
    P, N = 8, 8 * 8192
    case("chrome trace export")
    xs = W.make_inputs("normal_f32", N, P, W.CFG_RING_AR_8R, size_bytes=N * 4 + 79)
    ys, plan = _run(programs.ring_allreduce(P), xs, "f32", k=2, transport="direct", trace=True, kernel="specialized")
    assert_all_equal(ys, O2.ring_allreduce(xs, P, "f32")[0])
    path = str(tmp_path / "launch.json")
    n = write_chrome_trace(plan, path)
    assert n == plan.info()["num_instructions"]
    tr = json.load(open(path))
    xev = [e for e in tr["traceEvents"] if e["ph"] == "X"]
    assert len(xev) == n and all(e["dur"] >= 0 and e["ts"] >= 0 for e in xev)
    assert {e["pid"] for e in xev} == set(range(P))
    assert sum(1 for e in xev if e["name"] == "recv (skipped)") == 2 * P  # the chains' last hops
    plan.destroy()
