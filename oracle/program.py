"""O2 by program: run a chunk program one operation at a time, in program order.

A chunk program (MSCCLang report, §3.1 "System design": a Python-embedded,
chunk-oriented language in which the user declares input, output and scratch
buffers and copy/reduce operations on chunks) has sequential semantics. This
module is its plain interpreter. It takes the program as data -- a list of tuples

    (kind, src_rank, src_buf, src_idx, dst_rank, dst_buf, dst_idx, count)

with kind "copy" (dst <- src) or "reduce" (dst <- dst + src), buffers "in", "out",
"scr" and indices/counts in chunks -- and it never imports the library that
compiles such programs.

Chunk j of any buffer covers elements [floor(j*N/C), floor((j+1)*N/C)) where N
is the per-rank input length and C the number of chunks the input is cut into;
the same formula extends past C for longer buffers (an AllGather output holds
P*C chunks). An operation whose source and destination ranges have different
lengths is an error.

The symbolic executor runs the same program on multisets: every input chunk is
the atom (rank, chunk), a copy replaces the destination's multiset, a reduce adds
the source's into it. A collective's postcondition is then a statement about which
atoms every output chunk must hold, once each -- a check on the program with no
floating point at all.
"""

from __future__ import annotations

from collections import Counter

import numpy as np

from .numerics import add_stored, storage_np

BUFS = ("in", "out", "scr")


def _bound(j: int, N: int, C: int) -> int:
    return (j * N) // C


def out_chunks_of(collective: str, P: int, C: int, L: int | None = None) -> int:
    if collective in ("allreduce", "alltoall", "alltonext", "allreduce_inter"):
        return C
    if collective == "allgather":
        return P * C
    if collective == "allgather_intra":
        return L * C
    if collective == "reducescatter":
        return C // P
    if collective == "reducescatter_intra":
        return C // L
    raise ValueError(collective)


def run_program(ops, xs, dtype, nchunks, out_chunks, scr_chunks, prior_outputs=None):
    """Execute ``ops`` sequentially; return the P output buffers."""
    P = len(xs)
    N = len(xs[0])
    npdt = storage_np(dtype)
    bufs = []
    for r in range(P):
        n_out = _bound(out_chunks, N, nchunks)
        out = (np.asarray(prior_outputs[r]).astype(npdt).copy() if prior_outputs is not None
               else np.zeros(n_out, dtype=npdt))
        if len(out) != n_out:
            raise ValueError("prior output has the wrong length")
        bufs.append({"in": np.asarray(xs[r]).astype(npdt).copy(), "out": out,
                     "scr": np.zeros(_bound(scr_chunks, N, nchunks), dtype=npdt)})
    for op in ops:
        kind, sr, sb, si, dr, db, di, cnt = op
        s_lo, s_hi = _bound(si, N, nchunks), _bound(si + cnt, N, nchunks)
        d_lo, d_hi = _bound(di, N, nchunks), _bound(di + cnt, N, nchunks)
        if s_hi - s_lo != d_hi - d_lo:
            raise ValueError(f"operation {op} moves ranges of different lengths")
        src = bufs[sr][sb][s_lo:s_hi].copy()
        if kind == "copy":
            bufs[dr][db][d_lo:d_hi] = src
        elif kind == "reduce":
            bufs[dr][db][d_lo:d_hi] = add_stored(bufs[dr][db][d_lo:d_hi], src, dtype)
        else:
            raise ValueError(kind)
    return [b["out"] for b in bufs]


def run_symbolic(ops, P, nchunks, out_chunks, scr_chunks):
    """Execute ``ops`` on multisets. Output chunk values are Counters of (rank, chunk)
    atoms, or None for chunks the program never wrote."""
    state = []
    for r in range(P):
        state.append({"in": [Counter({(r, j): 1}) for j in range(nchunks)],
                      "out": [None] * out_chunks,
                      "scr": [None] * scr_chunks})
    for op in ops:
        kind, sr, sb, si, dr, db, di, cnt = op
        if sb not in BUFS or db not in BUFS:
            raise ValueError(f"bad buffer in {op}")
        if db == "in":
            raise ValueError("programs may not write their input buffers")
        for t in range(cnt):
            sbuf = state[sr][sb]
            dbuf = state[dr][db]
            if not (0 <= si + t < len(sbuf)) or not (0 <= di + t < len(dbuf)):
                raise IndexError(f"chunk out of range in {op}")
            v = sbuf[si + t]
            if v is None:
                raise ValueError(f"{op} reads a chunk that was never written")
            if kind == "copy":
                dbuf[di + t] = Counter(v)
            elif kind == "reduce":
                if dbuf[di + t] is None:
                    raise ValueError(f"{op} reduces into a chunk that was never written")
                dbuf[di + t] = dbuf[di + t] + v
            else:
                raise ValueError(kind)
    return [s["out"] for s in state]


def expected_symbolic(collective, P, nchunks, L=None):
    """Postcondition: the multiset every output chunk must hold (None = untouched)."""
    C = nchunks
    out = []
    for r in range(P):
        if collective == "allreduce":
            out.append([Counter({(s, j): 1 for s in range(P)}) for j in range(C)])
        elif collective == "allgather":
            out.append([Counter({(s, j): 1}) for s in range(P) for j in range(C)])
        elif collective == "reducescatter":
            c = C // P
            out.append([Counter({(s, r * c + j): 1 for s in range(P)}) for j in range(c)])
        elif collective == "alltoall":
            c = C // P
            out.append([Counter({(s, r * c + j): 1}) for s in range(P) for j in range(c)])
        elif collective == "alltonext":
            out.append([None] * C if r == 0 else [Counter({(r - 1, j): 1}) for j in range(C)])
        elif collective == "reducescatter_intra":
            g, l = divmod(r, L)
            c = C // L
            out.append([Counter({(g * L + s, l * c + j): 1 for s in range(L)}) for j in range(c)])
        elif collective == "allreduce_inter":
            l = r % L
            out.append([Counter({(h, j): 1 for h in range(l, P, L)}) for j in range(C)])
        elif collective == "allgather_intra":
            g = r // L
            out.append([Counter({(g * L + s, j): 1}) for s in range(L) for j in range(C)])
        else:
            raise ValueError(collective)
    return out


def check_postcondition(ops, collective, P, nchunks, scr_chunks, L=None):
    """Raise AssertionError naming the first wrong output chunk."""
    oc = out_chunks_of(collective, P, nchunks, L)
    got = run_symbolic(ops, P, nchunks, oc, scr_chunks)
    want = expected_symbolic(collective, P, nchunks, L)
    for r in range(P):
        for j in range(oc):
            if got[r][j] != want[r][j]:
                raise AssertionError(f"rank {r} output chunk {j}: got {got[r][j]}, want {want[r][j]}")
    return True
