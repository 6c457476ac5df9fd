"""O1: the collectives by their definitions.

The pages name the collectives that the schedules implement -- AllReduce and
hierarchical AllReduce, AllToAll and the new AllToNext (MSCCLang report, §3.2
"Experimental validation"), AllGather / ReduceScatter / AllReduce (AutoCCL report,
"Experimental design"; ReSCCL report, §2.3 "Evaluation") -- but they do not spell
out what each one computes. These are the standard definitions, for P ranks where
x_r is rank r's input of N elements:

* AllReduce:     y_r = sum over r' of x_r'                    (every rank)
* AllGather:     y_r = concat(x_0, ..., x_{P-1})              (every rank)
* ReduceScatter: y_r = sum over r' of x_r'[r*n : (r+1)*n],   n = N / P
* AllToAll:      y_r[s*b : (s+1)*b] = x_s[r*b : (r+1)*b],     b = N / P
* AllToNext:     y_{r+1} = x_r for r < P-1; y_0 keeps what it held (the transfer
  is not cyclic: it feeds the next pipeline stage).

Sums are exact-ish references: float64 for fp32/bf16 data (values widened
exactly), int64 wrapped to int32 for int32 data. Work is done in blocks of at
most 16 Mi elements so host memory stays bounded.

Grouped forms cover the three stages of a hierarchical AllReduce run as separate
launches, with P = G*L ranks numbered r = g*L + l:
* ``reducescatter_intra``: a ReduceScatter inside every group of L ranks.
* ``allreduce_inter``: an AllReduce among the G ranks that share a lane l.
* ``allgather_intra``: an AllGather inside every group.
"""

from __future__ import annotations

import numpy as np

from .numerics import to_f64, wrap_i32

BLOCK = 16 * 1024 * 1024


def _sum_f64(parts, dtype):
    """float64 sum and float64 sum of magnitudes of same-length arrays."""
    n = len(parts[0])
    s = np.zeros(n, dtype=np.float64)
    a = np.zeros(n, dtype=np.float64)
    for lo in range(0, n, BLOCK):
        hi = min(n, lo + BLOCK)
        for p in parts:
            v = to_f64(p[lo:hi], dtype)
            s[lo:hi] += v
            a[lo:hi] += np.abs(v)
    return s, a


def _sum_i32(parts):
    n = len(parts[0])
    out = np.zeros(n, dtype=np.int32)
    for lo in range(0, n, BLOCK):
        hi = min(n, lo + BLOCK)
        acc = np.zeros(hi - lo, dtype=np.int64)
        for p in parts:
            acc += np.asarray(p[lo:hi], dtype=np.int64)
        out[lo:hi] = wrap_i32(acc)
    return out


class Sum:
    """Reference of a reduction: ``exact`` (float64 or wrapped int32) and, for floats,
    ``abs_sum`` (float64) for the scaled error bound."""

    def __init__(self, exact, abs_sum=None):
        self.exact = exact
        self.abs_sum = abs_sum


def reduce_sum(parts, dtype) -> Sum:
    if dtype == "i32":
        return Sum(_sum_i32(parts))
    s, a = _sum_f64(parts, dtype)
    return Sum(s, a)


def allreduce(xs, dtype) -> Sum:
    """The one reference every rank's output must reach."""
    return reduce_sum(xs, dtype)


def allgather(xs):
    return np.concatenate([np.asarray(x) for x in xs])


def reducescatter(xs, dtype):
    """List of P ``Sum`` objects, one per output shard."""
    P = len(xs)
    N = len(xs[0])
    if N % P:
        raise ValueError("ReduceScatter needs N divisible by P")
    n = N // P
    return [reduce_sum([x[r * n:(r + 1) * n] for x in xs], dtype) for r in range(P)]


def alltoall(xs):
    P = len(xs)
    N = len(xs[0])
    if N % P:
        raise ValueError("AllToAll needs N divisible by P")
    b = N // P
    stacked = np.stack([np.asarray(x).reshape(P, b) for x in xs])  # [src, dst_block, b]
    return [stacked[:, r, :].reshape(-1).copy() for r in range(P)]


def alltonext(xs, prior_outputs):
    """y_{r+1} = x_r; y_0 is rank 0's output as it was before the call."""
    P = len(xs)
    ys = [np.asarray(prior_outputs[0]).copy()]
    for r in range(1, P):
        ys.append(np.asarray(xs[r - 1]).copy())
    return ys


# ---- grouped forms (P = G * L, rank r = g * L + l) --------------------------------

def reducescatter_intra(xs, dtype, L):
    """ReduceScatter inside each group of L consecutive ranks."""
    P = len(xs)
    if P % L:
        raise ValueError("P must be a multiple of L")
    out = []
    for r in range(P):
        g, l = divmod(r, L)
        grp = xs[g * L:(g + 1) * L]
        out.append(reducescatter(grp, dtype)[l])
    return out


def allreduce_inter(xs, dtype, L):
    """AllReduce among the ranks that share a lane l across the G groups."""
    P = len(xs)
    out = []
    for r in range(P):
        l = r % L
        out.append(reduce_sum([xs[h] for h in range(l, P, L)], dtype))
    return out


def allgather_intra(xs, L):
    P = len(xs)
    out = []
    for r in range(P):
        g = r // L
        out.append(allgather(xs[g * L:(g + 1) * L]))
    return out


# ---- sampled evaluation at full sizes ---------------------------------------------

def allreduce_at(xs, idx, dtype) -> Sum:
    """AllReduce reference at element indices ``idx`` only."""
    return reduce_sum([np.asarray(x)[idx] for x in xs], dtype)
