"""O2 by algorithm: the results of the textbook schedules, in their order of addition.

A schedule may run its steps in any time order that keeps the data dependencies
(ReSCCL report, §2.2: sub-pipelines only hold tasks free of data and link
conflicts), and fusing recv/reduce/copy/send into one instruction does not
re-associate anything (MSCCLang report, §3.1: fusion merges neighbouring
operations). So each output chunk is the left fold of its addends in the order the
chunk travels, and that order is fixed by the algorithm alone. This module writes
those folds out, one storage-dtype rounding per addition (see ``numerics``).
Splitting a chunk into instances or slices does not change which chain an element
follows, so the folds run on whole chunks.

Conventions (the pages leave them open; any fixed choice works, this is the one
taken):

* Chunks. With C chunks over N elements, chunk j covers
  [floor(j*N/C), floor((j+1)*N/C)).
* Ring (P ranks, C = P*c chunks). Chunk j belongs to rank o = j // c. Its
  reduce-scatter chain starts at rank o+1 and visits o+2, ..., o+P-1, ending at o
  (indices mod P): acc = x_{o+1}; acc = acc + x_{o+2}; ...; acc = acc + x_o.
  The all-gather then forwards rank o's result to o+1, o+2, ..., o-1.
* Hierarchical AllReduce (P = G*L, rank r = g*L + l, C = L*G chunks). Chunk j lies
  in shard l = j // G and has in-shard index g' = j % G. Step 1: a ring
  reduce-scatter inside each group: shard l's chain starts at local rank l+1 and
  ends at l. Step 2: a ring AllReduce over the G ranks of lane l, where chunk j's
  chain starts at group g'+1 and ends at group g'. Step 3: a ring all-gather of the
  shards inside each group. (MSCCLang report, §4.2 "Hierarchical AllReduce"; the
  same three-step shape as the cluster primitives of the HetCCL page, "Methodology"
  item 3.)
* Tree AllReduce (P ranks, C = P*c chunks, chunk j owned by o = j // c). Position t
  holds rank (o + t) mod P; its children are positions 2t+1 and 2t+2 (a heap). A
  leaf's partial is its input; a node with one child (2t+1) adds that child's
  partial to its input; a node with two adds child 2t+2's partial to its input, then
  child 2t+1's partial (the subtree at 2t+2 is never the deeper one, so its partial
  is ready first). The root's partial is the result, which every rank receives
  unchanged. The pages fix no order inside the tree; this one is the reading taken.
  (The AutoCCL report, "other value", compares tree and ring AllReduce.)
* Two-dimensional ReduceScatter (P = G*L, C = P blocks, block b = h*L + l belongs
  to rank b). Step 1: inside each group, block b's chain runs over the lanes
  l+1, ..., l (so lane l holds the group's partial of every block of lane l).
  Step 2: among the ranks of lane l, block b's chain runs over groups h+1, ..., h.
"""

from __future__ import annotations

import numpy as np

from .numerics import add_stored


def chunk_bounds(N: int, C: int):
    return [((j * N) // C, ((j + 1) * N) // C) for j in range(C)]


def fold(parts, dtype):
    """Left fold with one rounding per addition: ((p0 + p1) + p2) + ..."""
    acc = np.asarray(parts[0]).copy()
    for p in parts[1:]:
        acc = add_stored(acc, p, dtype)
    return acc


def _ring_chunk(xs, lo, hi, owner, dtype):
    P = len(xs)
    order = [(owner + 1 + t) % P for t in range(P)]
    return fold([np.asarray(xs[r][lo:hi]) for r in order], dtype)


def ring_allreduce(xs, nchunks, dtype):
    """Every rank's output of the ring AllReduce (they are all the same array)."""
    P = len(xs)
    N = len(xs[0])
    if nchunks % P:
        raise ValueError("ring programs use a multiple of P chunks")
    c = nchunks // P
    y = np.empty_like(np.asarray(xs[0]))
    for j, (lo, hi) in enumerate(chunk_bounds(N, nchunks)):
        y[lo:hi] = _ring_chunk(xs, lo, hi, j // c, dtype)
    return [y.copy() for _ in range(P)]


def _tree_chunk(xs, lo, hi, owner, dtype):
    P = len(xs)

    def partial(t):
        x = np.asarray(xs[(owner + t) % P][lo:hi])
        kids = [u for u in (2 * t + 2, 2 * t + 1) if u < P]  # shallower subtree first
        if not kids:
            return x.copy()
        acc = add_stored(partial(kids[0]), x, dtype)
        for u in kids[1:]:
            acc = add_stored(acc, partial(u), dtype)
        return acc
    return partial(0)


def tree_allreduce(xs, nchunks, dtype):
    """Every rank's output of the tree AllReduce (they are all the same array)."""
    P = len(xs)
    N = len(xs[0])
    if nchunks % P:
        raise ValueError("tree programs use a multiple of P chunks")
    c = nchunks // P
    y = np.empty_like(np.asarray(xs[0]))
    for j, (lo, hi) in enumerate(chunk_bounds(N, nchunks)):
        y[lo:hi] = _tree_chunk(xs, lo, hi, j // c, dtype)
    return [y.copy() for _ in range(P)]


def ring_reducescatter(xs, nchunks, dtype):
    """Rank r receives the chunks it owns, j in [r*c, (r+1)*c)."""
    P = len(xs)
    N = len(xs[0])
    if nchunks % P or N % P:
        raise ValueError("ring ReduceScatter needs C and N divisible by P")
    c = nchunks // P
    bounds = chunk_bounds(N, nchunks)
    out = []
    for r in range(P):
        pieces = [_ring_chunk(xs, lo, hi, r, dtype) for (lo, hi) in bounds[r * c:(r + 1) * c]]
        out.append(np.concatenate(pieces) if pieces else np.asarray(xs[0])[:0].copy())
    return out


def hierarchical_allreduce(xs, G, L, dtype):
    P = len(xs)
    if P != G * L:
        raise ValueError("P must equal G*L")
    N = len(xs[0])
    C = L * G
    y = np.empty_like(np.asarray(xs[0]))
    for j, (lo, hi) in enumerate(chunk_bounds(N, C)):
        l, gp = divmod(j, G)
        partial = []
        for g in range(G):
            lanes = [(l + 1 + t) % L for t in range(L)]
            partial.append(fold([np.asarray(xs[g * L + ln][lo:hi]) for ln in lanes], dtype))
        groups = [(gp + 1 + t) % G for t in range(G)]
        y[lo:hi] = fold([partial[g] for g in groups], dtype)
    return [y.copy() for _ in range(P)]


def reducescatter_2d(xs, G, L, dtype):
    P = len(xs)
    if P != G * L:
        raise ValueError("P must equal G*L")
    N = len(xs[0])
    if N % P:
        raise ValueError("ReduceScatter needs N divisible by P")
    n = N // P
    out = []
    for b in range(P):
        h, l = divmod(b, L)
        lo, hi = b * n, (b + 1) * n
        partial = []
        for g in range(G):
            lanes = [(l + 1 + t) % L for t in range(L)]
            partial.append(fold([np.asarray(xs[g * L + ln][lo:hi]) for ln in lanes], dtype))
        groups = [(h + 1 + t) % G for t in range(G)]
        out.append(fold([partial[g] for g in groups], dtype))
    return out


# ---- the three stages of a hierarchical AllReduce as separate collectives --------

def ring_reducescatter_intra(xs, L, dtype):
    """Ring ReduceScatter inside each group of L ranks, one chunk per shard."""
    P = len(xs)
    out = [None] * P
    for g in range(P // L):
        part = ring_reducescatter(xs[g * L:(g + 1) * L], L, dtype)
        for l in range(L):
            out[g * L + l] = part[l]
    return out


def ring_allreduce_inter(xs, L, dtype):
    """Ring AllReduce among the G ranks of each lane, G chunks."""
    P = len(xs)
    G = P // L
    out = [None] * P
    for l in range(L):
        ranks = list(range(l, P, L))
        res = ring_allreduce([xs[r] for r in ranks], G, dtype)
        for i, r in enumerate(ranks):
            out[r] = res[i]
    return out


# ---- the same folds at sampled element indices (checks at full sizes) --------------

def chunk_of(idx, N: int, C: int):
    """Chunk that holds each element index: the last chunk whose start is <= index."""
    starts = np.array([(j * N) // C for j in range(C + 1)], dtype=np.int64)
    return np.searchsorted(starts, np.asarray(idx, dtype=np.int64), side="right") - 1


def ring_allreduce_at(xs, nchunks, idx, dtype):
    """Ring AllReduce output at element indices ``idx`` (same for every rank)."""
    idx = np.asarray(idx, dtype=np.int64)
    return ring_allreduce_columns([np.asarray(x)[idx] for x in xs], len(xs[0]), nchunks, idx, dtype)


def ring_allreduce_columns(cols, N, nchunks, idx, dtype):
    """The same, given only each rank's values at ``idx`` (cols[r] = x_r[idx]) and the
    per-rank length N: full-size inputs never need to be on the host."""
    P = len(cols)
    c = nchunks // P
    idx = np.asarray(idx, dtype=np.int64)
    owner = chunk_of(idx, N, nchunks) // c
    out = np.empty(len(idx), dtype=np.asarray(cols[0]).dtype)
    for o in range(P):
        sel = np.nonzero(owner == o)[0]
        if sel.size == 0:
            continue
        order = [(o + 1 + t) % P for t in range(P)]
        out[sel] = fold([np.asarray(cols[r])[sel] for r in order], dtype)
    return out


def hierarchical_allreduce_at(xs, G, L, idx, dtype):
    idx = np.asarray(idx, dtype=np.int64)
    return hierarchical_allreduce_columns([np.asarray(x)[idx] for x in xs], len(xs[0]), G, L, idx, dtype)


def hierarchical_allreduce_columns(cols, N, G, L, idx, dtype):
    """Hierarchical AllReduce at ``idx`` given only each rank's values there."""
    C = L * G
    idx = np.asarray(idx, dtype=np.int64)
    j = chunk_of(idx, N, C)
    out = np.empty(len(idx), dtype=np.asarray(cols[0]).dtype)
    for jj in np.unique(j):
        sel = np.nonzero(j == jj)[0]
        l, gp = divmod(int(jj), G)
        partial = []
        for g in range(G):
            lanes = [(l + 1 + t) % L for t in range(L)]
            partial.append(fold([np.asarray(cols[g * L + ln])[sel] for ln in lanes], dtype))
        groups = [(gp + 1 + t) % G for t in range(G)]
        out[sel] = fold([partial[g] for g in groups], dtype)
    return out
