"""Chrome / Perfetto trace of one traced launch (plans built with trace=True).

Host-side tooling over ``ccl_plan_read_trace`` and ``ccl_plan_export``: one process per
virtual rank, one thread per launch-grid workgroup, one complete event per executed
instruction (from its start to its end, with the time its first slice waited for data
as an argument), so a launch can be opened in chrome://tracing or ui.perfetto.dev. The
device clock is the 100 MHz wall clock: one tick is 10 ns.
"""

from __future__ import annotations

import json

from . import capi

TICK_US = 0.01  # 100 MHz device wall clock


def opcode_name(op: int) -> str:
    """recv / reduce / copy / send letters of an instruction, e.g. 'rrcs'."""
    if op & capi.CCL_I_SKIP:
        return "recv (skipped)"
    parts = []
    if op & capi.CCL_I_RECV:
        parts.append("r")
    if op & capi.CCL_I_SRCB:
        parts.append("r")
    if op & capi.CCL_I_DSTA:
        parts.append("c")
    if op & capi.CCL_I_SEND:
        parts.append("s")
    name = "".join(parts) or "nop"
    return {"r": "recv", "s": "send", "c": "copy", "rr": "reduce"}.get(name, name)


def chrome_trace(plan) -> dict:
    """The trace-event dictionary of the plan's last launch."""
    info = plan.info()
    wgs, instrs = plan.trace(instructions=True)
    ex = plan.export()
    starts = [r[0] for r in instrs if r[0] > 0] + [w[0] for w in wgs if w[3] > 0]
    if not starts:
        return {"traceEvents": [], "displayTimeUnit": "ns"}
    t0 = min(starts)
    events = []
    for r in range(info["nranks"]):
        events.append({"ph": "M", "name": "process_name", "pid": r, "args": {"name": f"rank {r}"}})
    seen_wg = set()
    for e, (start, ready, end, _) in zip(ex, instrs):
        if start == 0:
            continue
        if e.wg not in seen_wg:
            seen_wg.add(e.wg)
            events.append({"ph": "M", "name": "thread_name", "pid": e.rank, "tid": e.wg,
                           "args": {"name": f"workgroup {e.wg} (channel {e.channel}, instance {e.instance})"}})
        events.append({"ph": "X", "name": opcode_name(e.opcode), "pid": e.rank, "tid": e.wg,
                       "ts": (start - t0) * TICK_US, "dur": max(0, end - start) * TICK_US,
                       "args": {"chunk": e.chunk_id, "subpipeline": e.subpipe, "send_peer": e.send_peer,
                                "recv_peer": e.recv_peer, "first_slice_wait_us": max(0, ready - start) * TICK_US,
                                "chunks": e.count}})
    return {"traceEvents": events, "displayTimeUnit": "ns",
            "otherData": {"workgroups": info["num_workgroups"], "instructions": info["num_instructions"]}}


def write_chrome_trace(plan, path: str) -> int:
    """Writes the trace of the plan's last launch to `path`; returns the number of
    instruction events."""
    tr = chrome_trace(plan)
    with open(path, "w") as fh:
        json.dump(tr, fh)
    return sum(1 for e in tr["traceEvents"] if e["ph"] == "X")
