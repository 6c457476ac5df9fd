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


def run(prog, xs, dtype, k=1, count=None, prior=None, repeat=1, **cfg):
    """Execute ``prog`` once (or ``repeat`` times) on inputs xs; returns (outputs, plan)."""
    P = prog.nranks
    N = len(xs[0]) if count is None else count
    cfg.setdefault("max_count", max(N, 1))
    plan = Plan(prog, k, PlanConfig(dtype=dtype, **cfg))
    ins = [to_dev(x, dtype) for x in xs]
    nout = plan.output_len(N)
    if prior is not None:
        outs = [to_dev(p, dtype) for p in prior]
    else:
        outs = [torch.full((max(nout, 1),), -7, dtype=TORCH_OF[dtype], device="cuda:0") for _ in range(P)]
    for _ in range(repeat):
        plan.execute(ins, outs, N)
    torch.cuda.synchronize()
    plan.status()
    ys = [to_host(o, dtype)[:nout] for o in outs]
    return ys, plan
