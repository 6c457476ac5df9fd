"""Seeded synthetic inputs for the collective executor and for the CPU oracle.

This module is the only code shared by the oracle side and the GPU side. It draws
numbers and nothing else: no reduction, no rounding rule of the collectives, no
chunk arithmetic. Every rank's buffer comes from its own numpy generator seeded
with ``[2026, cfg_id, size_bytes, rank]`` so that any rank's input can be
regenerated on its own (the oracle checks sampled elements at full size that way).

The collectives move data without looking at it, so the value distributions only
need to exercise the arithmetic: integer-valued fp32 (exact sums), fp32 N(0,1),
bf16 rounded from fp32 N(0,1), full-range int32, and a provenance encoding whose
values name their own (rank, index).

bf16 data is carried as ``uint16`` bit patterns. The fp32 -> bf16 step of the bf16
generator uses torch's CPU cast, a library routine, so that no rounding code of
this project is involved in making inputs.
"""

from __future__ import annotations

import numpy as np

# Config ids used in seeds. They name workloads by their shape.
CFG_RING_AR_4R_INT = 1        # ring AllReduce, 4 ranks, integer-valued fp32
CFG_RING_AR_8R = 2            # ring AllReduce, 8 ranks, fp32 N(0,1)
CFG_HIER_AR_16R_BF16 = 3      # hierarchical AllReduce, 2x8 ranks, bf16
CFG_A2A_32R_INT32 = 4         # two-phase AllToAll, 4x8 ranks, int32
CFG_A2NEXT_AGRS_24R = 5       # AllToNext / AllGather / ReduceScatter, 3x8 ranks, fp32
CFG_TREE_AR = 6               # tree AllReduce, 1..24 ranks, fp32 / bf16 N(0,1)

DTYPES = ("f32", "bf16", "i32")
ELEM_SIZE = {"f32": 4, "bf16": 2, "i32": 4}
NP_STORAGE = {"f32": np.float32, "bf16": np.uint16, "i32": np.int32}


def rank_rng(cfg_id: int, size_bytes: int, rank: int) -> np.random.Generator:
    """Generator for one rank's buffer of one workload point."""
    return np.random.default_rng([2026, int(cfg_id), int(size_bytes), int(rank)])


def integer_valued_f32(n: int, rng: np.random.Generator, lo: int = -8, hi: int = 8) -> np.ndarray:
    """Uniform integers in [lo, hi] stored as fp32: every partial sum of a few ranks is exact."""
    return rng.integers(lo, hi + 1, size=n, dtype=np.int64).astype(np.float32)


def normal_f32(n: int, rng: np.random.Generator) -> np.ndarray:
    return rng.standard_normal(n, dtype=np.float32)


def normal_bf16_bits(n: int, rng: np.random.Generator) -> np.ndarray:
    """fp32 N(0,1) rounded to bf16 by torch's CPU cast; returned as uint16 bit patterns."""
    import torch

    f = torch.from_numpy(rng.standard_normal(n, dtype=np.float32))
    return f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def uniform_i32(n: int, rng: np.random.Generator) -> np.ndarray:
    return rng.integers(-(2**31), 2**31, size=n, dtype=np.int64).astype(np.int32)


def provenance_i32(n: int, rank: int) -> np.ndarray:
    """Element i of rank r holds r * 2**20 + i: any copy of it names where it came from."""
    if n > 2**20:
        raise ValueError("provenance encoding holds at most 2**20 elements per rank")
    return (np.int64(rank) * 2**20 + np.arange(n, dtype=np.int64)).astype(np.int32)


def provenance_f32(n: int, rank: int) -> np.ndarray:
    """Same encoding as fp32 (exact below 2**24, so at most 15 ranks x 2**20)."""
    v = np.int64(rank) * 2**20 + np.arange(n, dtype=np.int64)
    if v.size and int(v.max()) >= 2**24:
        raise ValueError("provenance values must stay below 2**24 to be exact in fp32")
    return v.astype(np.float32)


def make_rank_input(kind: str, n: int, cfg_id: int, size_bytes: int, rank: int) -> np.ndarray:
    """One rank's input. ``kind`` is one of int_f32, normal_f32, normal_bf16, uniform_i32,
    prov_i32, prov_f32, normal_f32_denorm."""
    if kind == "prov_i32":
        return provenance_i32(n, rank)
    if kind == "prov_f32":
        return provenance_f32(n, rank)
    rng = rank_rng(cfg_id, size_bytes, rank)
    if kind == "int_f32":
        return integer_valued_f32(n, rng)
    if kind == "normal_f32":
        return normal_f32(n, rng)
    if kind == "normal_bf16":
        return normal_bf16_bits(n, rng)
    if kind == "uniform_i32":
        return uniform_i32(n, rng)
    if kind == "normal_f32_denorm":
        # N(0,1) scaled into the fp32 subnormal range (|x| around 1e-39), so that
        # partial sums stay subnormal and a flush-to-zero anywhere shows up.
        return (normal_f32(n, rng) * np.float32(1e-39)).astype(np.float32)
    raise ValueError(f"unknown input kind {kind!r}")


def make_inputs(kind: str, n: int, nranks: int, cfg_id: int, size_bytes: int | None = None):
    """Inputs of all ranks as a list of numpy arrays."""
    if size_bytes is None:
        size_bytes = n * (2 if kind == "normal_bf16" else 4)
    return [make_rank_input(kind, n, cfg_id, size_bytes, r) for r in range(nranks)]


def device_inputs(kind: str, n: int, nranks: int, seed: int, device="cuda:0"):
    """Inputs of all ranks drawn on the GPU by torch's seeded generator (large sizes,
    where drawing on the host would dominate): one generator seeded with ``seed``, ranks
    drawn in order. ``kind``: normal_f32, normal_bf16 (N(0,1) cast by torch; returned as
    torch.bfloat16), uniform_i32 (the whole int32 range). Both sides read the same bits:
    the oracle gets them through a device-to-host copy."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    if kind == "uniform_i32":
        return [torch.randint(-2**31, 2**31 - 1, (n,), generator=g, device=device, dtype=torch.int32)
                for _ in range(nranks)]
    if kind == "normal_f32":
        return [torch.randn(n, generator=g, device=device) for _ in range(nranks)]
    if kind == "normal_bf16":
        return [torch.randn(n, generator=g, device=device).to(torch.bfloat16) for _ in range(nranks)]
    raise ValueError(f"unknown device input kind {kind!r}")
