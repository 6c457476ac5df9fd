"""Convenience wrapper over the C ABI: a ``Plan`` object owning one ``ccl_plan``.

torch supplies device memory (``data_ptr``) and the stream (``cuda_stream``);
everything else -- compilation, the launch, the kernel -- is in ``libccl.so``.
"""

from __future__ import annotations

from dataclasses import dataclass

from . import capi
from .dsl import Program

DTYPES = {"f32": capi.CCL_F32, "bf16": capi.CCL_BF16, "i32": capi.CCL_I32}
ELEM_SIZE = {"f32": 4, "bf16": 2, "i32": 4}
SCHEDULERS = {"program": capi.CCL_SCHED_PROGRAM_ORDER, "hpds": capi.CCL_SCHED_HPDS, "rr": capi.CCL_SCHED_RR}
WG_ALLOC = {"connection": capi.CCL_WG_CONNECTION, "state": capi.CCL_WG_STATE}


@dataclass
class PlanConfig:
    dtype: str = "f32"
    max_count: int = 1 << 20
    nthreads: int = 512
    slice_bytes: int = 256 * 1024
    protocol: str = "simple"  # "simple" (slice flags) or "ll" (flag in every 8-byte unit)
    transport: str = "staged"  # "staged" (every transfer through a slot) or "direct" (copy receives skip it)
    streaming: bool = False  # non-temporal hints on local-buffer traffic (large working sets)
    scheduler: str = "hpds"
    wg_alloc: str = "state"
    trace: bool = False
    host_only: bool = False
    no_fusion: bool = False
    xcd_local: bool = True  # plain transfer stores when the layout keeps transfers on one XCD
    force_xcd_local: bool = False  # that variant even for spread layouts (tests its release path)
    num_cus: int = 0
    timeout_us: int = 0
    # failure injection for watchdog tests: transfer 0's flag is never set
    debug_drop_flag: bool = False
    # debug mode: staging slots and scratch filled with a sentinel before every launch
    debug_poison: bool = False
    # "interpreter" (one kernel for every plan), "specialized" (a kernel generated for
    # this plan: straight-line code for short plans, the loop form for long ones),
    # "specialized_loop" (the loop form always) or "lazy" (a generated kernel in the
    # slice-outer loop order)
    kernel: str = "interpreter"

    def to_c(self) -> capi.ccl_plan_config:
        flags = 0
        if self.trace:
            flags |= capi.CCL_FLAG_TRACE
        if self.host_only:
            flags |= capi.CCL_FLAG_HOST_ONLY
        if self.no_fusion:
            flags |= capi.CCL_FLAG_NO_FUSION
        if self.transport == "direct":
            flags |= capi.CCL_FLAG_DIRECT
        elif self.transport != "staged":
            raise ValueError(f"unknown transport {self.transport!r}")
        if self.streaming:
            flags |= capi.CCL_FLAG_STREAMING
        if self.force_xcd_local:
            flags |= capi.CCL_FLAG_FORCE_XCD_LOCAL
        if not self.xcd_local:
            flags |= capi.CCL_FLAG_COHERENT_ONLY
        if self.kernel == "specialized":
            flags |= capi.CCL_FLAG_SPECIALIZE
        elif self.kernel == "specialized_loop":
            flags |= capi.CCL_FLAG_SPECIALIZE | capi.CCL_FLAG_SPECIALIZE_LOOP
        elif self.kernel == "lazy":
            flags |= capi.CCL_FLAG_SPECIALIZE | capi.CCL_FLAG_LAZY
        elif self.kernel != "interpreter":
            raise ValueError(f"unknown kernel {self.kernel!r}")
        if self.debug_drop_flag:
            flags |= capi.CCL_FLAG_DEBUG_DROP_FLAG
        if self.debug_poison:
            flags |= capi.CCL_FLAG_DEBUG_POISON
        if self.protocol == "ll":
            flags |= capi.CCL_FLAG_LL
        elif self.protocol != "simple":
            raise ValueError(f"unknown protocol {self.protocol!r}")
        return capi.ccl_plan_config(DTYPES[self.dtype], capi.CCL_REDOP_SUM, int(self.max_count), int(self.nthreads),
                                    int(self.slice_bytes), SCHEDULERS[self.scheduler], WG_ALLOC[self.wg_alloc],
                                    flags, int(self.num_cus), int(self.timeout_us))


class Plan:
    def __init__(self, prog: Program, parallel_factor: int = 1, config: PlanConfig | None = None, **kw):
        self.program = prog
        self.config = config if config is not None else PlanConfig(**kw)
        self.parallel_factor = parallel_factor
        self._desc = prog.to_desc()
        self.handle = capi.ccl_plan_create(self._desc, prog.nranks, prog.in_chunks, parallel_factor,
                                           self.config.to_c())

    # ---- queries -------------------------------------------------------------
    def info(self) -> dict:
        i = capi.ccl_plan_info(self.handle)
        d = {name: getattr(i, name) for name, _ in capi.ccl_plan_info_t._fields_
             if name not in ("compile_ms", "opcode_hist", "reserved", "reserved0")}
        d["compile_ms"] = list(i.compile_ms)
        d["opcode_hist"] = list(i.opcode_hist)
        return d

    def bytes(self, count: int) -> int:
        return capi.ccl_plan_bytes(self.handle, count)

    def export(self):
        return capi.ccl_plan_export(self.handle)

    def check(self, seed: int = 1, nsims: int = 4) -> None:
        capi.ccl_plan_check(self.handle, seed, nsims)

    def status(self) -> None:
        capi.ccl_plan_status(self.handle)

    def trace(self, instructions: bool = False):
        """Per-workgroup trace of the last launch (plans built with trace=True), one
        record per launch-grid workgroup (idle padding ids record zeros); with
        ``instructions`` also the per-instruction {start, data ready, end} records."""
        i = self.info()
        if instructions:
            return capi.ccl_plan_read_trace(self.handle, i["grid_workgroups"], i["num_instructions"])
        return capi.ccl_plan_read_trace(self.handle, i["grid_workgroups"])

    def link_busy(self):
        """Per-connection busy fractions of the last launch (plans built with trace=True):
        (src_rank, dst_rank, channel, instance, busy_fraction) per connection."""
        return capi.ccl_plan_link_busy(self.handle)

    def output_len(self, count: int) -> int:
        return (self.program.out_chunks * count) // self.program.in_chunks

    # ---- execution -----------------------------------------------------------
    def execute(self, inputs, outputs, count: int | None = None, stream=None) -> None:
        """inputs / outputs: per-rank torch tensors (or objects with data_ptr())."""
        if count is None:
            count = inputs[0].numel()
        s = 0
        if stream is not None:
            s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        else:
            import torch
            s = torch.cuda.current_stream().cuda_stream
        capi.ccl_execute(self.handle, [t.data_ptr() for t in inputs], [t.data_ptr() for t in outputs], count, s)

    def execute_static(self, inputs, outputs, count: int | None = None, stream=None) -> None:
        """Like execute, allocating nothing: the plan (host-only plans included) runs on the
        library's static device scratch."""
        if count is None:
            count = inputs[0].numel()
        if stream is not None:
            s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        else:
            import torch
            s = torch.cuda.current_stream().cuda_stream
        capi.ccl_execute_static(self.handle, [t.data_ptr() for t in inputs], [t.data_ptr() for t in outputs], count,
                                s)

    def destroy(self) -> None:
        if self.handle:
            capi.ccl_plan_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.destroy()
