"""Plan-specialized kernels (generated per plan, compiled with hiprtc at create) and the
lazy loop order, on the host: generation, compilation for gfx950 (no GPU needed),
refusals, and the plan checker's interleavings in the lazy order."""

import pytest

from chunk_schedule_execution_amd import Plan, PlanConfig, capi, programs


def host_plan(prog, k=1, **cfg):
    cfg.setdefault("max_count", 1 << 16)
    return Plan(prog, k, PlanConfig(host_only=True, **cfg))


@pytest.mark.parametrize("kernel", ["specialized", "lazy"])
def test_ring_allreduce_compiles_to_one_shape(kernel):
    """Every rank's workgroups of a ring run the same operations, so one straight-line
    sequence serves all 8k workgroups."""
    plan = host_plan(programs.ring_allreduce(8), 4, transport="direct", kernel=kernel)
    assert plan.info()["specialized_shapes"] == 1
    assert host_plan(programs.ring_allreduce(8), 4).info()["specialized_shapes"] == 0


def test_small_pieces_read_records_through_the_scalar_cache():
    """Straight-line code whose instruction pieces are all at most 8 KiB (3 KiB under
    the LL protocol) reads each step's record with scalar loads; larger pieces, the loop
    form, the lazy order and the interpreter keep the records the workgroup copies into
    LDS."""
    def rec(S, k, **kw):
        kw.setdefault("kernel", "specialized")
        return host_plan(programs.ring_allreduce(8), k, max_count=S // 4, nthreads=256, slice_bytes=131072,
                         transport="direct", **kw).info()["specialized_scalar_records"]
    assert rec(1 << 20, 24) == 1 and rec(1 << 20, 16) == 1   # 5.3 and 8 KiB pieces
    assert rec(32 << 10, 16, protocol="ll") == 1 and rec(512 << 10, 24, protocol="ll") == 1  # LL: up to 3 KiB
    assert rec(1 << 20, 32, protocol="ll") == 0                                             # 4 KiB LL pieces
    assert rec(3 << 20, 24) == 0 and rec(2 << 20, 24) == 0   # 16 and 10.7 KiB pieces
    assert rec(1 << 20, 16, kernel="specialized_loop") == 0
    assert rec(1 << 20, 16, kernel="lazy") == 0
    assert rec(1 << 20, 16, kernel="interpreter") == 0
    def bf(S):
        return host_plan(programs.ring_allreduce(8), 16, max_count=S // 2, dtype="bf16", nthreads=256,
                         transport="direct", kernel="specialized").info()["specialized_scalar_records"]
    assert bf(1 << 20) == 1 and bf(2 << 20) == 0              # bf16 pieces of 8 and 16 KiB


def test_other_dtypes_and_protocols_compile():
    assert host_plan(programs.hier_stage_reducescatter_intra(2, 8), 2, dtype="bf16", kernel="specialized").info()[
        "specialized_shapes"] == 1
    assert host_plan(programs.ring_allreduce(4), 2, protocol="ll", kernel="lazy").info()["specialized_shapes"] == 1
    assert host_plan(programs.direct_alltoall(4), 1, dtype="i32", kernel="specialized").info()["specialized_shapes"] >= 1


def test_generated_kernel_asks_for_the_occupancy_its_grid_needs():
    """All workgroups of a launch wait on each other's flags, so all must be resident:
    a grid of more than one 4-wave workgroup per compute unit is compiled for that many
    waves per SIMD, one that fits in fewer is compiled without a request."""
    def waves(prog, k, nt, **kw):
        return host_plan(prog, k, nthreads=nt, kernel="specialized", num_cus=256, **kw).info()
    one = waves(programs.ring_allreduce(8), 32, 256, transport="direct")  # 256 x 4 waves: one per CU
    assert one["grid_workgroups"] == 256 and one["specialized_waves_per_simd"] == 1
    assert waves(programs.ring_allreduce(8), 32, 1024)["specialized_waves_per_simd"] == 4  # 16 waves per CU
    ag = waves(programs.ring_allgather(24), 32, 512, transport="direct")  # 768 x 8 waves over 256 CUs
    assert ag["grid_workgroups"] == 768 and ag["specialized_waves_per_simd"] == 6
    assert waves(programs.ring_allreduce(8), 64, 1024)["specialized_waves_per_simd"] == 8  # the most a SIMD holds
    assert host_plan(programs.ring_allreduce(8), 32, nthreads=1024).info()["specialized_waves_per_simd"] == 0


def test_lazy_order_refuses_completion_waits():
    """A completion wait covers a whole instruction; in the lazy order its workgroup may
    still be at an earlier slice of others, so such plans are refused."""
    assert host_plan(programs.tree_allreduce(8), 1).info()["num_waits"] > 0
    with pytest.raises(capi.CCLError) as e:
        host_plan(programs.tree_allreduce(8), 1, kernel="lazy")
    assert e.value.status == capi.CCL_ERR_UNSUPPORTED


@pytest.mark.parametrize("name,args,dtype", [("two_phase_alltoall", (4, 8), "i32"),
                                             ("hierarchical_allreduce", (2, 8), "bf16"), ("tree_allreduce", (8,), "f32")])
def test_long_programs_get_the_loop_form(name, args, dtype):
    """Straight-line code inlines one step per instruction of every distinct workgroup
    program; past 24 instructions it would outgrow the instruction cache, so long plans
    get the loop form: one step per distinct operation word, selected per record."""
    prog = programs.REGISTRY[name](*args)
    loop = host_plan(prog, 2, dtype=dtype, nthreads=256, kernel="specialized").info()
    assert 3 <= loop["specialized_instructions"] <= 12  # distinct operation words
    assert loop["specialized_code_bytes"] < 64 << 10
    short = host_plan(programs.ring_allreduce(8), 2, kernel="specialized").info()
    assert short["specialized_instructions"] == 15  # straight-line: every instruction
    edge = host_plan(programs.ring_allreduce(12), 2, kernel="specialized").info()
    assert edge["specialized_instructions"] == 23  # 2P - 1: still straight-line
    long_ring = host_plan(programs.ring_allreduce(16), 2, kernel="specialized").info()
    assert long_ring["specialized_instructions"] < 31  # 31 would not fit the instruction cache
    forced = host_plan(programs.ring_allreduce(8), 2, kernel="specialized_loop").info()
    assert forced["specialized_instructions"] == len({e.opcode for e in host_plan(programs.ring_allreduce(8), 2).export()})


@pytest.mark.parametrize("name,args,k,knobs", [("ring_allreduce", (5,), 2, dict(transport="direct")),
                                               ("ring_allreduce", (4,), 3, {}),
                                               ("ring_reducescatter", (6,), 2, {}),
                                               ("hier_stage_reducescatter_intra", (2, 4), 2, {}),
                                               ("alltonext", (3, 4, False), 2, {}),
                                               ("ring_allgather", (6,), 2, {})])
def test_lazy_plans_pass_random_interleavings(name, args, k, knobs):
    """The plan checker runs the lazy order too: iteration s takes slice s of every
    instruction of a workgroup; no interleaving deadlocks or reads unwritten data, and
    the postcondition holds."""
    host_plan(programs.REGISTRY[name](*args), k, kernel="lazy", **knobs).check(seed=7, nsims=3)


def test_lazy_order_refuses_overlapping_local_ranges():
    """In the lazy order two instructions of one workgroup are ordered slice by slice
    only, so a workgroup that writes chunks [0, 2) of a buffer and then reads chunk 1 of
    it (an overlapping, different range: slice 0 of the read covers elements written in a
    later slice of the write) is refused; the task order takes the same plan."""
    from chunk_schedule_execution_amd.dsl import Buffer, Program
    pr = Program("custom", 2, 2, 2, name="overlap")
    pr.chunk(0, Buffer.input, 0, count=2).copy(0, Buffer.output, 0)
    pr.chunk(0, Buffer.output, 1).copy(1, Buffer.output, 1)
    pr.chunk(1, Buffer.input, 0).copy(1, Buffer.output, 0)
    ex = host_plan(pr, 1).export()
    assert ex[0].wg == ex[1].wg  # the write and the overlapping read share a workgroup
    with pytest.raises(capi.CCLError) as e:
        host_plan(pr, 1, kernel="lazy")
    assert e.value.status == capi.CCL_ERR_UNSUPPORTED and "identical chunk ranges" in str(e.value)
    assert host_plan(pr, 1, kernel="specialized").info()["specialized_shapes"] >= 1


@pytest.mark.parametrize("name,args,k,knobs", [("ring_allreduce", (8,), 4, dict(transport="direct")),
                                               ("ring_allreduce", (8,), 2, dict(protocol="ll")),
                                               ("ring_reducescatter", (24,), 2, {}),
                                               ("ring_allgather", (24,), 2, dict(transport="direct")),
                                               ("direct_alltoall", (8,), 1, dict(dtype="i32")),
                                               ("alltonext", (3, 8, True), 2, {}),
                                               ("hier_stage_allgather_intra", (2, 8), 2, dict(dtype="bf16"))])
def test_lazy_order_accepts_the_library_programs(name, args, k, knobs):
    """The library's programs without completion waits keep identical ranges inside a
    workgroup, so the range check accepts them."""
    assert host_plan(programs.REGISTRY[name](*args), k, kernel="lazy", **knobs).info()["specialized_shapes"] >= 1
