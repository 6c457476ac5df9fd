"""Chunk-oriented program builder (MSCCLang report, section 3.1: a Python-embedded
language where the user declares input/output/scratch buffers and writes copy and
reduce operations on chunks; the compiler traces them in program order).

A ``Program`` records operations; ``ChunkRef.copy`` and ``ChunkRef.reduce`` append
one operation each and return the destination, so chains read like the route a
chunk takes:

    c = prog.chunk(rank, Buffer.input, j)
    c = c.copy(rank + 1, Buffer.scratch, j)
    c.reduce(prog.chunk(rank + 1, Buffer.input, j))     # scratch_j += input_j

Semantics are sequential: ``dst.reduce(src)`` means dst <- dst + src at that point
of the program. The program is serialized into ``ccl_chunk_op`` records for
``ccl_plan_create``; nothing is computed here.
"""

from __future__ import annotations

import ctypes as C
from dataclasses import dataclass, field

from . import capi


class Buffer:
    input = capi.CCL_BUF_INPUT
    output = capi.CCL_BUF_OUTPUT
    scratch = capi.CCL_BUF_SCRATCH
    names = {0: "in", 1: "out", 2: "scr"}


COLLECTIVES = {
    "allreduce": capi.CCL_COLL_ALLREDUCE, "allgather": capi.CCL_COLL_ALLGATHER,
    "reducescatter": capi.CCL_COLL_REDUCESCATTER, "alltoall": capi.CCL_COLL_ALLTOALL,
    "alltonext": capi.CCL_COLL_ALLTONEXT, "custom": capi.CCL_COLL_CUSTOM,
}
SCOPES = {"all": capi.CCL_SCOPE_ALL, "intra": capi.CCL_SCOPE_INTRA, "inter": capi.CCL_SCOPE_INTER}


@dataclass(frozen=True)
class Op:
    kind: int
    src_rank: int
    src_buf: int
    src_idx: int
    dst_rank: int
    dst_buf: int
    dst_idx: int
    count: int
    channel: int = 0


@dataclass
class ChunkRef:
    prog: "Program"
    rank: int
    buf: int
    idx: int
    count: int = 1

    def copy(self, rank: int, buf: int, idx: int, ch: int = 0) -> "ChunkRef":
        """dst <- self; returns dst."""
        dst = ChunkRef(self.prog, rank, buf, idx, self.count)
        self.prog._add(capi.CCL_OP_COPY, self, dst, ch)
        return dst

    def reduce(self, src: "ChunkRef", ch: int = 0) -> "ChunkRef":
        """self <- self + src; returns self."""
        if src.count != self.count:
            raise ValueError("reduce operands cover different chunk counts")
        self.prog._add(capi.CCL_OP_REDUCE, src, self, ch)
        return self


@dataclass
class Program:
    collective: str
    nranks: int
    in_chunks: int
    out_chunks: int
    scratch_chunks: int = 0
    group_size: int = 0
    group_scope: str = "all"
    name: str = ""
    ops: list = field(default_factory=list)

    def chunk(self, rank: int, buf: int, idx: int, count: int = 1) -> ChunkRef:
        return ChunkRef(self, rank, buf, idx, count)

    def _add(self, kind: int, src: ChunkRef, dst: ChunkRef, ch: int) -> None:
        self.ops.append(Op(kind, src.rank, src.buf, src.idx, dst.rank, dst.buf, dst.idx, src.count, ch))

    # ---- serialization ------------------------------------------------------
    def to_desc(self) -> capi.ccl_program_desc:
        arr = (capi.ccl_chunk_op * max(1, len(self.ops)))()
        for i, o in enumerate(self.ops):
            arr[i] = capi.ccl_chunk_op(o.kind, capi.CCL_REDOP_SUM, o.channel, o.src_rank, o.src_buf, o.src_idx,
                                       o.dst_rank, o.dst_buf, o.dst_idx, o.count)
        d = capi.ccl_program_desc(COLLECTIVES[self.collective], self.nranks, self.in_chunks, self.out_chunks,
                                  self.scratch_chunks, self.group_size, SCOPES[self.group_scope], 0,
                                  C.cast(arr, C.POINTER(capi.ccl_chunk_op)), len(self.ops))
        d._keepalive = arr  # the array must outlive the descriptor
        return d

    def as_tuples(self):
        """Plain (kind, src_rank, src_buf, src_idx, dst_rank, dst_buf, dst_idx, count) tuples."""
        kinds = {capi.CCL_OP_COPY: "copy", capi.CCL_OP_REDUCE: "reduce"}
        return [(kinds[o.kind], o.src_rank, Buffer.names[o.src_buf], o.src_idx, o.dst_rank,
                 Buffer.names[o.dst_buf], o.dst_idx, o.count) for o in self.ops]
