"""ctypes binding of ``include/ccl.h``: the same entry points under the same names.

Argument marshalling only. Nothing here computes any part of a collective; every
step runs in ``libccl.so`` (host compiler and HIP executor). If the library is not
built the import fails loudly -- there is no fallback.
"""

from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libccl.so")

# ---- constants (mirror ccl.h) -------------------------------------------------
CCL_OK = 0
CCL_ERR_INVALID_ARGUMENT = -1
CCL_ERR_INVALID_PROGRAM = -2
CCL_ERR_UNSUPPORTED = -3
CCL_ERR_OUT_OF_RESOURCES = -4
CCL_ERR_HIP = -5
CCL_ERR_TIMEOUT = -6
CCL_ERR_INTERNAL = -7

CCL_OP_COPY, CCL_OP_REDUCE = 0, 1
CCL_BUF_INPUT, CCL_BUF_OUTPUT, CCL_BUF_SCRATCH = 0, 1, 2
CCL_REDOP_SUM = 0
CCL_F32, CCL_BF16, CCL_I32 = 0, 1, 2
(CCL_COLL_ALLREDUCE, CCL_COLL_ALLGATHER, CCL_COLL_REDUCESCATTER, CCL_COLL_ALLTOALL, CCL_COLL_ALLTONEXT,
 CCL_COLL_CUSTOM) = range(6)
CCL_SCOPE_ALL, CCL_SCOPE_INTRA, CCL_SCOPE_INTER = 0, 1, 2
CCL_SCHED_PROGRAM_ORDER, CCL_SCHED_HPDS, CCL_SCHED_RR = 0, 1, 2
CCL_WG_CONNECTION, CCL_WG_STATE = 0, 1
CCL_FLAG_TRACE, CCL_FLAG_HOST_ONLY, CCL_FLAG_NO_FUSION, CCL_FLAG_NO_VERIFY, CCL_FLAG_LL = 0x1, 0x2, 0x4, 0x8, 0x10
CCL_FLAG_COHERENT_ONLY = 0x20
CCL_FLAG_DIRECT = 0x40
CCL_FLAG_STREAMING = 0x80
CCL_FLAG_FORCE_XCD_LOCAL = 0x100
CCL_FLAG_SPECIALIZE = 0x200
CCL_FLAG_LAZY = 0x400
CCL_FLAG_SPECIALIZE_LOOP = 0x800
CCL_FLAG_DEBUG_DROP_FLAG = 0x1000
CCL_FLAG_DEBUG_POISON = 0x2000
CCL_I_RECV, CCL_I_SRCB, CCL_I_DSTA, CCL_I_SEND, CCL_I_LOCAL_IN = 0x1, 0x2, 0x4, 0x8, 0x10
CCL_I_SKIP, CCL_I_NOFLAG = 0x20, 0x40


class ccl_chunk_op(C.Structure):
    _fields_ = [("kind", C.c_uint8), ("redop", C.c_uint8), ("channel", C.c_uint16),
                ("src_rank", C.c_int32), ("src_buf", C.c_int32), ("src_idx", C.c_int32),
                ("dst_rank", C.c_int32), ("dst_buf", C.c_int32), ("dst_idx", C.c_int32),
                ("count", C.c_int32)]


class ccl_program_desc(C.Structure):
    _fields_ = [("collective", C.c_int32), ("nranks", C.c_int32), ("in_chunks", C.c_int32),
                ("out_chunks", C.c_int32), ("scratch_chunks", C.c_int32), ("group_size", C.c_int32),
                ("group_scope", C.c_int32), ("reserved", C.c_int32),
                ("ops", C.POINTER(ccl_chunk_op)), ("nops", C.c_size_t)]


class ccl_plan_config(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("redop", C.c_int32), ("max_count", C.c_int64),
                ("nthreads", C.c_int32), ("slice_bytes", C.c_int32), ("scheduler", C.c_int32),
                ("wg_alloc", C.c_int32), ("flags", C.c_uint32), ("num_cus", C.c_int32),
                ("timeout_us", C.c_int64)]


class ccl_plan_info_t(C.Structure):
    _fields_ = [("nranks", C.c_int32), ("nchunks", C.c_int32), ("parallel_factor", C.c_int32),
                ("dtype", C.c_int32), ("num_workgroups", C.c_int32), ("max_wg_per_rank", C.c_int32),
                ("num_instructions", C.c_int32), ("num_subpipelines", C.c_int32),
                ("num_connections", C.c_int32), ("num_transfers", C.c_int32), ("num_waits", C.c_int32),
                ("count_granule", C.c_int32), ("nthreads", C.c_int32), ("slice_bytes", C.c_int32),
                ("max_resident_wgs", C.c_int32), ("grid_workgroups", C.c_int32),
                ("xcd_local", C.c_int32), ("specialized_shapes", C.c_int32),
                ("staging_bytes", C.c_int64), ("scratch_bytes", C.c_int64), ("flag_bytes", C.c_int64),
                ("table_bytes", C.c_int64), ("compile_ms", C.c_double * 6), ("opcode_hist", C.c_int32 * 16),
                ("specialized_instructions", C.c_int32), ("specialized_waves_per_simd", C.c_int32),
                ("specialized_code_bytes", C.c_int64), ("dag_width", C.c_int32), ("dag_depth", C.c_int32),
                ("specialized_scalar_records", C.c_int32)]


class ccl_instr_info(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "rank", "wg", "subpipe", "channel", "instance", "opcode", "a_buf", "a_idx", "b_buf", "b_idx",
        "d_buf", "d_idx", "count", "recv_peer", "send_peer", "xin", "xout", "nwaits", "chunk_id",
        "done_flag")]


class ccl_link_busy(C.Structure):
    _fields_ = [("src_rank", C.c_int32), ("dst_rank", C.c_int32), ("channel", C.c_int32), ("instance", C.c_int32),
                ("busy_fraction", C.c_double)]


class ccl_tune_point(C.Structure):
    _fields_ = [("variant", C.c_int32), ("parallel_factor", C.c_int32), ("nthreads", C.c_int32),
                ("slice_bytes", C.c_int32), ("protocol", C.c_int32), ("reserved", C.c_int32)]


class ccl_tune_space(C.Structure):
    _fields_ = [("factors", C.POINTER(C.c_int32)), ("nfactors", C.c_int32),
                ("nthreads", C.POINTER(C.c_int32)), ("nnthreads", C.c_int32),
                ("slices", C.POINTER(C.c_int32)), ("nslices", C.c_int32),
                ("nvariants", C.c_int32), ("warmup", C.c_int32), ("iters", C.c_int32),
                ("protocols", C.c_int32)]


class ccl_tune_report(C.Structure):
    _fields_ = [("evaluations", C.c_int32), ("reserved", C.c_int32), ("best_score", C.c_double),
                ("start_score", C.c_double)]


ccl_tune_objective = C.CFUNCTYPE(C.c_double, C.POINTER(ccl_tune_point), C.c_void_p)


class CCLError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {ccl_error_string(status)} ({status}): {detail}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python chunk_schedule_execution_amd/build.py")
    # torch ships its own HIP runtime under the same soname (libamdhip64.so.7). Loading
    # torch first makes libccl.so bind to that copy, so the process holds one HIP runtime
    # and torch's tensors and streams are valid for the library.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = C.CDLL(LIB_PATH)
    P = C.POINTER
    sig = {
        "ccl_version": (C.c_int, []),
        "ccl_error_string": (C.c_char_p, [C.c_int]),
        "ccl_last_error_detail": (C.c_char_p, []),
        "ccl_plan_create": (C.c_int, [P(ccl_program_desc), C.c_int, C.c_int, C.c_int, P(ccl_plan_config),
                                      P(C.c_void_p)]),
        "ccl_execute": (C.c_int, [C.c_void_p, P(C.c_void_p), P(C.c_void_p), C.c_int64, C.c_void_p]),
        "ccl_execute_static": (C.c_int, [C.c_void_p, P(C.c_void_p), P(C.c_void_p), C.c_int64, C.c_void_p]),
        "ccl_plan_destroy": (C.c_int, [C.c_void_p]),
        "ccl_plan_info": (C.c_int, [C.c_void_p, P(ccl_plan_info_t)]),
        "ccl_plan_bytes": (C.c_int64, [C.c_void_p, C.c_int64]),
        "ccl_plan_export": (C.c_int, [C.c_void_p, P(ccl_instr_info), C.c_size_t, P(C.c_size_t)]),
        "ccl_plan_check": (C.c_int, [C.c_void_p, C.c_uint64, C.c_int]),
        "ccl_plan_status": (C.c_int, [C.c_void_p]),
        "ccl_plan_read_trace": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t]),
        "ccl_plan_link_busy": (C.c_int, [C.c_void_p, P(ccl_link_busy), C.c_size_t, P(C.c_size_t)]),
        "ccl_tune_coordinate_descent": (C.c_int, [P(ccl_tune_space), P(ccl_tune_point), ccl_tune_objective,
                                                  C.c_void_p, P(ccl_tune_point), P(ccl_tune_report)]),
        "ccl_tune": (C.c_int, [P(P(ccl_program_desc)), C.c_int, C.c_int64, P(ccl_plan_config),
                               P(ccl_tune_space), C.c_void_p, P(ccl_tune_point), P(ccl_tune_report)]),
        "ccl_copy_probe": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int, C.c_int, C.c_void_p]),
        "ccl_litmus_message_passing": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int64, P(C.c_int64), C.c_void_p]),
        "ccl_hop_probe": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int64, C.c_int64,
                                    P(C.c_double), P(C.c_int64), C.c_void_p]),
        "ccl_stream_create_cu_masked": (C.c_int, [P(C.c_uint32), C.c_int, P(C.c_void_p)]),
        "ccl_stream_destroy": (C.c_int, [C.c_void_p]),
        "ccl_cu_probe": (C.c_int, [C.c_void_p, C.c_int, C.c_int, P(C.c_uint32)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("ccl_version", "ccl_error_string", "ccl_last_error_detail", "ccl_plan_create", "ccl_execute",
            "ccl_execute_static",
            "ccl_plan_destroy", "ccl_plan_info", "ccl_plan_bytes", "ccl_plan_export", "ccl_plan_check",
            "ccl_plan_status", "ccl_plan_read_trace", "ccl_plan_link_busy", "ccl_tune_coordinate_descent", "ccl_tune",
            "ccl_copy_probe", "ccl_litmus_message_passing", "ccl_hop_probe", "ccl_stream_create_cu_masked",
            "ccl_stream_destroy", "ccl_cu_probe")


def lib():
    return _lib


def ccl_error_string(status: int) -> str:
    return _lib.ccl_error_string(status).decode()


def ccl_last_error_detail() -> str:
    return _lib.ccl_last_error_detail().decode()


def _check(status: int, where: str) -> int:
    if status != CCL_OK:
        raise CCLError(status, where, ccl_last_error_detail())
    return status


def ccl_version() -> int:
    return _lib.ccl_version()


def ccl_plan_create(desc: ccl_program_desc, nranks: int, nchunks: int, parallel_factor: int,
                    cfg: ccl_plan_config) -> int:
    """Returns the plan handle (an integer address)."""
    h = C.c_void_p()
    _check(_lib.ccl_plan_create(C.byref(desc), nranks, nchunks, parallel_factor, C.byref(cfg), C.byref(h)),
           "ccl_plan_create")
    return h.value


def ccl_execute(plan: int, sendbufs, recvbufs, count: int, stream: int = 0) -> None:
    """sendbufs / recvbufs: sequences of device addresses (ints), one per rank."""
    n = len(sendbufs)
    sb = (C.c_void_p * n)(*sendbufs)
    rb = (C.c_void_p * n)(*recvbufs)
    _check(_lib.ccl_execute(C.c_void_p(plan), sb, rb, C.c_int64(count), C.c_void_p(stream)), "ccl_execute")


def ccl_execute_static(plan: int, sendbufs, recvbufs, count: int, stream: int = 0) -> None:
    """ccl_execute without any device allocation (the library's static device scratch)."""
    n = len(sendbufs)
    sb = (C.c_void_p * n)(*sendbufs)
    rb = (C.c_void_p * n)(*recvbufs)
    _check(_lib.ccl_execute_static(C.c_void_p(plan), sb, rb, C.c_int64(count), C.c_void_p(stream)),
           "ccl_execute_static")


def ccl_plan_destroy(plan: int) -> None:
    _check(_lib.ccl_plan_destroy(C.c_void_p(plan)), "ccl_plan_destroy")


def ccl_plan_info(plan: int) -> ccl_plan_info_t:
    info = ccl_plan_info_t()
    _check(_lib.ccl_plan_info(C.c_void_p(plan), C.byref(info)), "ccl_plan_info")
    return info


def ccl_plan_bytes(plan: int, count: int) -> int:
    v = _lib.ccl_plan_bytes(C.c_void_p(plan), C.c_int64(count))
    if v < 0:
        _check(int(v), "ccl_plan_bytes")
    return int(v)


def ccl_plan_export(plan: int):
    n = C.c_size_t()
    _check(_lib.ccl_plan_export(C.c_void_p(plan), None, 0, C.byref(n)), "ccl_plan_export")
    arr = (ccl_instr_info * max(1, n.value))()
    _check(_lib.ccl_plan_export(C.c_void_p(plan), arr, n.value, C.byref(n)), "ccl_plan_export")
    return [arr[i] for i in range(n.value)]


def ccl_plan_check(plan: int, seed: int = 1, nsims: int = 4) -> None:
    _check(_lib.ccl_plan_check(C.c_void_p(plan), C.c_uint64(seed), nsims), "ccl_plan_check")


def ccl_plan_status(plan: int) -> None:
    _check(_lib.ccl_plan_status(C.c_void_p(plan)), "ccl_plan_status")


def ccl_plan_read_trace(plan: int, nwg: int, ninstr: int = 0):
    """Per-workgroup records, and per-instruction records when ninstr > 0."""
    n = nwg + ninstr
    buf = (C.c_uint64 * (4 * max(1, n)))()
    _check(_lib.ccl_plan_read_trace(C.c_void_p(plan), buf, C.sizeof(buf)), "ccl_plan_read_trace")
    recs = [tuple(buf[4 * w:4 * w + 4]) for w in range(n)]
    return (recs[:nwg], recs[nwg:]) if ninstr else recs


def ccl_plan_link_busy(plan: int):
    """Per-connection busy fractions of the last traced launch: a list of
    (src_rank, dst_rank, channel, instance, busy_fraction)."""
    n = C.c_size_t()
    _check(_lib.ccl_plan_link_busy(C.c_void_p(plan), None, 0, C.byref(n)), "ccl_plan_link_busy")
    arr = (ccl_link_busy * max(1, n.value))()
    _check(_lib.ccl_plan_link_busy(C.c_void_p(plan), arr, n.value, C.byref(n)), "ccl_plan_link_busy")
    return [(a.src_rank, a.dst_rank, a.channel, a.instance, a.busy_fraction) for a in arr[:n.value]]


def ccl_tune_coordinate_descent(space: ccl_tune_space, objective, start: ccl_tune_point | None = None):
    """objective(point: ccl_tune_point) -> float. Returns (best point, report)."""
    cb = ccl_tune_objective(lambda p, _u: float(objective(p.contents)))
    best = ccl_tune_point()
    rep = ccl_tune_report()
    _check(_lib.ccl_tune_coordinate_descent(C.byref(space), C.byref(start) if start is not None else None, cb,
                                            None, C.byref(best), C.byref(rep)), "ccl_tune_coordinate_descent")
    return best, rep


def ccl_tune(descs, count: int, base: ccl_plan_config, space: ccl_tune_space, stream: int = 0):
    arr = (C.POINTER(ccl_program_desc) * len(descs))(*[C.pointer(d) for d in descs])
    best = ccl_tune_point()
    rep = ccl_tune_report()
    _check(_lib.ccl_tune(arr, len(descs), C.c_int64(count), C.byref(base), C.byref(space), C.c_void_p(stream),
                         C.byref(best), C.byref(rep)), "ccl_tune")
    return best, rep


def ccl_copy_probe(dst: int, src: int, nbytes: int, nblocks: int, nthreads: int, stream: int = 0) -> None:
    _check(_lib.ccl_copy_probe(C.c_void_p(dst), C.c_void_p(src), C.c_size_t(nbytes), nblocks, nthreads,
                               C.c_void_p(stream)), "ccl_copy_probe")


def ccl_litmus_message_passing(cross_xcd: bool, rounds: int, words: int, timeout_us: int = 200000, stream: int = 0):
    """Per pair: (producer XCD, consumer XCD, rounds completed, mismatching words, first bad
    round, its first word index, plain flag stores, expired waits)."""
    res = (C.c_int64 * 64)()
    _check(_lib.ccl_litmus_message_passing(int(bool(cross_xcd)), rounds, words, C.c_int64(timeout_us), res,
                                           C.c_void_p(stream)), "ccl_litmus_message_passing")
    return [tuple(res[8 * p:8 * p + 8]) for p in range(8)]


def ccl_hop_probe(hops: int, nbytes: int, two_operands: bool, nthreads: int = 256, launches: int = 20,
                  window_bytes: int = 0, timeout_us: int = 200000, stream: int = 0, ll: bool = False):
    """(microseconds per hand-off of each launch, (chain workgroups off workgroup 0's XCD,
    launches with an expired wait, launches whose data arrived wrong, launches completed))."""
    us = (C.c_double * launches)()
    info = (C.c_int64 * 4)()
    _check(_lib.ccl_hop_probe(hops, nbytes, int(bool(two_operands)), int(bool(ll)), nthreads, launches,
                              C.c_int64(window_bytes),
                              C.c_int64(timeout_us), us, info, C.c_void_p(stream)), "ccl_hop_probe")
    return list(us[:info[3]]), tuple(info)


def cu_mask_words(cus, nwords: int = 8):
    """32-bit mask words enabling the given compute-unit indices."""
    m = [0] * nwords
    for c in cus:
        m[c // 32] |= 1 << (c % 32)
    return m


def ccl_stream_create_cu_masked(mask_words) -> int:
    """A stream restricted to the CUs whose bits are set; returns its handle (hipStream_t)."""
    n = len(mask_words)
    arr = (C.c_uint32 * n)(*[int(w) & 0xFFFFFFFF for w in mask_words])
    s = C.c_void_p()
    _check(_lib.ccl_stream_create_cu_masked(arr, n, C.byref(s)), "ccl_stream_create_cu_masked")
    return s.value


def ccl_stream_destroy(stream: int) -> None:
    _check(_lib.ccl_stream_destroy(C.c_void_p(stream)), "ccl_stream_destroy")


def ccl_cu_probe(stream: int, nblocks: int, hold_us: int = 50):
    """Per block (XCD, shader engine, shader array, CU id) where it ran."""
    out = (C.c_uint32 * (2 * nblocks))()
    _check(_lib.ccl_cu_probe(C.c_void_p(stream), nblocks, hold_us, out), "ccl_cu_probe")
    res = []
    for b in range(nblocks):
        x, hw = out[2 * b], out[2 * b + 1]
        res.append((x, (hw >> 13) & 7, (hw >> 12) & 1, (hw >> 8) & 15))
    return res
