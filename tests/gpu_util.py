"""Helpers for GPU tests: upload per-rank numpy inputs, run a plan through the C ABI,
download outputs. torch is used for device memory and the stream only."""

import numpy as np
import torch

from chunk_schedule_execution_amd import Plan, PlanConfig

TORCH_OF = {"f32": torch.float32, "bf16": torch.int16, "i32": torch.int32}
NP_OF = {"f32": np.float32, "bf16": np.uint16, "i32": np.int32}


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    a = np.ascontiguousarray(x)
    if dtype == "bf16":
        a = a.view(np.int16)
    return torch.from_numpy(a.copy()).to("cuda:0")


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    a = t.cpu().numpy()
    if dtype == "bf16":
        a = a.view(np.uint16)
    return a


def negate(x: np.ndarray, dtype: str) -> np.ndarray:
    """-x in the storage type (bf16: the sign bit flipped; int32: two's-complement wrap)."""
    if dtype == "bf16":
        return np.asarray(x, np.uint16) ^ np.uint16(0x8000)
    with np.errstate(over="ignore"):
        return (-np.asarray(x)).astype(np.asarray(x).dtype)


def launch_variant(xs, j: int, dtype: str):
    """Inputs of the j-th launch before the last of a repeated run: rank r gets rank
    (r + j) mod P's input, negated for odd j. Every launch thus moves other values than
    the launch before it, and the last launch (j = 0) runs on xs itself."""
    P = len(xs)
    out = [np.asarray(xs[(r + j) % P]).copy() for r in range(P)]
    return [negate(x, dtype) for x in out] if j % 2 else out


def sentinel(dtype: str, j: int) -> int:
    """Output fill of the j-th launch from the end (distinct per launch)."""
    return -7 - j


def run(prog, xs, dtype, k=1, count=None, prior=None, repeat=1, check=None, plan=None, **cfg):
    """Execute ``prog`` on inputs xs; returns (outputs of the launch on xs, plan).

    With ``repeat`` > 1 the plan runs ``repeat`` launches back to back on the stream,
    each with its own inputs (``launch_variant``) and its own output buffers, filled
    beforehand with a launch-specific sentinel (or, given ``prior``, with that launch's
    variant of it); the last launch runs on xs. ``check(ys, xs_j, prior_j)`` is called
    on the outputs of every earlier launch, so a launch that picks up a previous
    launch's slot data, flags or low-latency units gives wrong values and fails.
    """
    P = prog.nranks
    N = len(xs[0]) if count is None else count
    if repeat > 1 and check is None:
        raise ValueError("a repeated run needs a check of every launch")
    own = plan is None
    if own:
        cfg.setdefault("max_count", max(N, 1))
        plan = Plan(prog, k, PlanConfig(dtype=dtype, **cfg))
    nout = plan.output_len(N)
    launches = []
    for j in reversed(range(repeat)):  # j = 0 is the last launch, on xs
        xj = xs if j == 0 else launch_variant(xs, j, dtype)
        pj = None
        if prior is not None:
            pj = prior if j == 0 else launch_variant(prior, j, dtype)
        ins = [to_dev(x, dtype) for x in xj]
        if pj is not None:
            outs = [to_dev(p, dtype) for p in pj]
        else:
            outs = [torch.full((max(nout, 1),), sentinel(dtype, j), dtype=TORCH_OF[dtype], device="cuda:0")
                    for _ in range(P)]
        launches.append((j, xj, pj, ins, outs))
    torch.cuda.synchronize()
    for _, _, _, ins, outs in launches:
        plan.execute(ins, outs, N)
    torch.cuda.synchronize()
    plan.status()
    ys = None
    for j, xj, pj, _, outs in launches:
        yj = [to_host(o, dtype)[:nout] for o in outs]
        if j == 0:
            ys = yj
        else:
            check(yj, xj, pj)
    return ys, plan
