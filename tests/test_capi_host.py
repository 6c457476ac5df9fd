"""The C-ABI library on the host: it loads, exports every entry point the header
declares, rejects bad arguments with the documented status codes, and needs no GPU
for host-only plans."""

import ctypes as C
import os
import re

import pytest

from chunk_schedule_execution_amd import Plan, PlanConfig, capi, programs
from chunk_schedule_execution_amd.dsl import Buffer, Program

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_entry_points():
    text = open(os.path.join(ROOT, "include", "ccl.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ccl_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_entry_points()
    assert len(names) >= 15
    lib = C.CDLL(capi.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(capi.EXPORTED)


def test_error_strings_and_version():
    assert capi.ccl_version() >= 1
    for code in range(0, -8, -1):
        assert capi.ccl_error_string(code) and capi.ccl_error_string(code) != "unknown status"
    assert capi.ccl_error_string(-99) == "unknown status"


def host_plan(prog, k=1, **cfg):
    cfg.setdefault("max_count", 1 << 20)
    return Plan(prog, k, PlanConfig(host_only=True, **cfg))


def test_host_only_plan_cannot_execute():
    p = host_plan(programs.ring_allreduce(4))
    with pytest.raises(capi.CCLError) as e:
        capi.ccl_execute(p.handle, [1, 2, 3, 4], [5, 6, 7, 8], 16)
    assert e.value.status == capi.CCL_ERR_INVALID_ARGUMENT


def test_destroy_null_is_noop():
    assert capi.lib().ccl_plan_destroy(None) == capi.CCL_OK


@pytest.mark.parametrize("field,value,status", [
    ("nthreads", 100, capi.CCL_ERR_INVALID_ARGUMENT),
    ("nthreads", 2048, capi.CCL_ERR_INVALID_ARGUMENT),
    ("max_count", 0, capi.CCL_ERR_INVALID_ARGUMENT),
    ("dtype", "f64", None),
])
def test_bad_configs(field, value, status):
    prog = programs.ring_allreduce(4)
    if value == "f64":
        cfg = PlanConfig(host_only=True).to_c()
        cfg.dtype = 7
        with pytest.raises(capi.CCLError) as e:
            capi.ccl_plan_create(prog.to_desc(), 4, 4, 1, cfg)
        assert e.value.status == capi.CCL_ERR_UNSUPPORTED
        return
    with pytest.raises(capi.CCLError) as e:
        host_plan(prog, **{field: value})
    assert e.value.status == status


def test_mismatched_shape_arguments():
    prog = programs.ring_allreduce(4)
    cfg = PlanConfig(host_only=True).to_c()
    for nr, nc, k in ((3, 4, 1), (4, 5, 1), (4, 4, 0)):
        with pytest.raises(capi.CCLError) as e:
            capi.ccl_plan_create(prog.to_desc(), nr, nc, k, cfg)
        assert e.value.status == capi.CCL_ERR_INVALID_ARGUMENT


def _bad_program(kind):
    p = Program("allreduce", 2, 2, 2, scratch_chunks=2)
    IN, OUT, SCR = Buffer.input, Buffer.output, Buffer.scratch
    if kind == "out_of_range":
        p.chunk(0, IN, 0).copy(1, OUT, 2)
    elif kind == "input_write":
        p.chunk(0, OUT, 0).copy(1, IN, 0)
    elif kind == "overlap":
        p.chunk(0, OUT, 0, 2).copy(0, OUT, 1)
    elif kind == "uninitialized_scratch":
        p.chunk(0, SCR, 0).copy(1, OUT, 0)
    elif kind == "skips_a_rank":  # rank 1's chunk 0 never added
        for j in range(2):
            p.chunk(j, IN, j).copy(j, OUT, j)
            p.chunk(j, OUT, j).copy(1 - j, OUT, j)
    elif kind == "double_count":
        for j in range(2):
            o = p.chunk(j, IN, j).copy(j, OUT, j)
            o.reduce(p.chunk(1 - j, IN, j))
            o.reduce(p.chunk(1 - j, IN, j))
            o.copy(1 - j, OUT, j)
    return p


@pytest.mark.parametrize("kind", ["out_of_range", "input_write", "overlap", "uninitialized_scratch",
                                  "skips_a_rank", "double_count"])
def test_verifier_rejects(kind):
    with pytest.raises(capi.CCLError) as e:
        host_plan(_bad_program(kind))
    assert e.value.status == capi.CCL_ERR_INVALID_PROGRAM, str(e.value)


def test_custom_collective_skips_postcondition_but_not_bounds():
    p = _bad_program("skips_a_rank")
    p.collective = "custom"
    host_plan(p)  # accepted: no postcondition for custom programs
    q = _bad_program("out_of_range")
    q.collective = "custom"
    q.out_chunks = 2
    with pytest.raises(capi.CCLError):
        host_plan(q)


def test_too_many_workgroups_for_the_device():
    # 32 ranks x 31 peers of direct AllToAll at 8 instances cannot all be resident
    with pytest.raises(capi.CCLError) as e:
        host_plan(programs.direct_alltoall(32), k=8, nthreads=1024)
    assert e.value.status == capi.CCL_ERR_OUT_OF_RESOURCES


def test_plan_bytes_rejects_bad_counts():
    p = host_plan(programs.ring_allreduce(4), max_count=100)
    with pytest.raises(capi.CCLError):
        p.bytes(101)
    assert p.bytes(0) == 0


def test_build_script_loads_without_the_library():
    # The build entry point must work on a fresh checkout, where libccl.so does not exist
    # yet: loading the build script may not import the package (whose __init__ loads it).
    import subprocess
    import sys

    code = ("import importlib.util, os, sys\n"
            f"spec = importlib.util.spec_from_file_location('b', os.path.join({ROOT!r}, "
            "'chunk_schedule_execution_amd', 'build.py'))\n"
            "m = importlib.util.module_from_spec(spec); spec.loader.exec_module(m)\n"
            "assert callable(m.build)\n"
            "assert 'chunk_schedule_execution_amd.capi' not in sys.modules\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    src = open(os.path.join(ROOT, "__graft_entry__.py")).read()
    assert "from chunk_schedule_execution_amd.build import" not in src


def test_flag_dropping_needs_the_staged_slice_flag_protocol():
    """The watchdog's failure injection (transfer 0's flag is never set) is refused where
    a missing flag would go unnoticed: LL flags travel inside the data, and a direct
    receive that ends its workgroup is not waited for."""
    prog = programs.ring_allreduce(4)
    assert host_plan(prog, debug_drop_flag=True).info()["num_transfers"] > 0
    for knobs in (dict(protocol="ll"), dict(transport="direct")):
        with pytest.raises(capi.CCLError) as e:
            host_plan(prog, debug_drop_flag=True, **knobs)
        assert e.value.status == capi.CCL_ERR_UNSUPPORTED


@pytest.mark.parametrize("P,c", [(4, 1), (8, 1), (8, 2), (3, 2)])
def test_dag_parallelism_of_the_ring(P, c):
    """The fused ring is c*P independent chains of 2P-1 instructions (send, P-2 reducing
    forwards, the final reduce, P-2 forwards, the last receive): depth 2P-1, and the
    largest set of mutually unordered instructions takes one from each chain."""
    info = host_plan(programs.ring_allreduce(P, c) if c > 1 else programs.ring_allreduce(P), 2).info()
    assert info["dag_depth"] == 2 * P - 1
    assert info["dag_width"] == c * P


def test_dag_parallelism_of_the_tree_and_two_phase_alltoall():
    """The tree's chains are shorter than the ring's (depth below 2P-1), and the two-phase
    AllToAll's phase-1 copies into distinct gather slots are all unordered, so its width
    is at least the number of ranks."""
    tree = host_plan(programs.tree_allreduce(8), 1).info()
    assert 0 < tree["dag_depth"] < 15 and tree["dag_width"] >= 8
    a2a = host_plan(programs.two_phase_alltoall(4, 8), 1).info()
    assert a2a["dag_width"] >= 32 and a2a["dag_depth"] >= 3


def test_litmus_rejects_bad_arguments_before_touching_the_gpu():
    """Zero rounds, a word count that is not a multiple of 4, more than 2^20 words."""
    for args in ((False, 0, 64), (False, 10, 6), (False, 10, 1 << 21)):
        with pytest.raises(capi.CCLError) as e:
            capi.ccl_litmus_message_passing(*args)
        assert e.value.status == capi.CCL_ERR_INVALID_ARGUMENT


def test_hop_probe_rejects_bad_arguments_before_touching_the_gpu():
    """No hops, a chain longer than one XCD's compute units, a payload off the 16-byte
    grid or above 4 MiB, a workgroup size that is no multiple of 64, no launches, a
    window smaller than two payloads or above 16 MiB."""
    for args in ((0, 16, False), (32, 16, False), (15, 24, False), (15, (4 << 20) + 16, True),
                 (15, 16384, False, 96), (15, 16384, False, 256, 0), (15, 16384, False, 256, 10, 16384),
                 (15, 16384, False, 256, 10, (16 << 20) + 256)):
        with pytest.raises(capi.CCLError) as e:
            capi.ccl_hop_probe(*args)
        assert e.value.status == capi.CCL_ERR_INVALID_ARGUMENT
    with pytest.raises(capi.CCLError) as e:  # LL regions hold twice the payload: a window of 3 payloads is too small
        capi.ccl_hop_probe(15, 16384, False, 256, 10, 3 * 16384, ll=True)
    assert e.value.status == capi.CCL_ERR_INVALID_ARGUMENT


def test_tuner_cache_answers_a_known_key_without_timing(tmp_path):
    """The persistent tuner cache times a key once: a second request (same programs, rank
    count, dtype, count bucket, device, space and base flags) is answered from the file,
    also after reloading it; another count bucket or base configuration is a new key."""
    from chunk_schedule_execution_amd.tuner_cache import TunerCache, count_bucket

    calls = []

    def fake_tune(descs, count, base, space, stream):
        calls.append(count)
        best = capi.ccl_tune_point(0, 4, 256, 65536, 2, 0)
        rep = capi.ccl_tune_report(7, 0, 123.0, 100.0)
        return best, rep

    arrs = [(C.c_int32 * 3)(1, 4, 16), (C.c_int32 * 2)(256, 512), (C.c_int32 * 2)(32768, 65536)]
    space = capi.ccl_tune_space(C.cast(arrs[0], C.POINTER(C.c_int32)), 3, C.cast(arrs[1], C.POINTER(C.c_int32)), 2,
                                C.cast(arrs[2], C.POINTER(C.c_int32)), 2, 1, 2, 5, 5)
    base = PlanConfig(max_count=1 << 20).to_c()
    path = str(tmp_path / "tune.json")
    cache = TunerCache(path, tune=fake_tune)
    progs = [programs.ring_allreduce(8)]
    p1 = cache.tune(progs, 300000, base, space, device="MI355X")
    p2 = cache.tune(progs, 262145, base, space, device="MI355X")  # same bucket (2^19)
    assert count_bucket(300000) == count_bucket(262145) == 1 << 19
    assert calls == [300000] and (p2.parallel_factor, p2.protocol) == (p1.parallel_factor, p1.protocol) == (4, 2)
    cache.tune(progs, 1 << 20, base, space, device="MI355X")  # another bucket
    cache.tune(progs, 300000, PlanConfig(max_count=1 << 20, num_cus=32).to_c(), space, device="MI355X")
    assert calls == [300000, 1 << 20, 300000]
    again = TunerCache(path, tune=fake_tune)
    again.tune(progs, 300000, base, space, device="MI355X")
    assert again.hits == 1 and len(calls) == 3
    again.tune([programs.tree_allreduce(8)], 300000, base, space, device="MI355X")
    assert len(calls) == 4
