"""Library of chunk programs: the schedules the executor runs.

Algorithms named on the pages -- ring and hierarchical AllReduce, the two-phase
aggregated AllToAll and the AllToNext with its cross-group hop split over all ranks
of a group (MSCCLang report, sections 3.2 and 4.1-4.4), AllGather / ReduceScatter
(AutoCCL report, experimental design; ReSCCL report, section 2.3) -- written with
the chunk DSL. The pages give no step lists; the conventions below are the readings
taken, and the compiler's postcondition check verifies each program symbolically.

Conventions: ring direction r -> r+1. In a ring over C = P*c chunks, chunk j belongs
to rank o = j // c; its reduce-scatter chain starts at o+1 and ends at o, then its
all-gather forwards o -> o+1 -> ... -> o-1. Grouped programs number P = G*L ranks
r = g*L + l. Programs are written chain by chain (the order a person writes them in);
scheduling decides the execution order.
"""

from __future__ import annotations

from .dsl import Buffer, Program

IN, OUT, SCR = Buffer.input, Buffer.output, Buffer.scratch


def _ring_reduce_chain(prog: Program, ranks, j: int, cnt: int, final):
    """Reduce chunk range [j, j+cnt) of ranks[0], ranks[1], ..., ranks[-1] in that order;
    partials pass through each rank's scratch, the sum lands in ``final`` (buf, idx) of
    ranks[-1]. Returns the ChunkRef holding the sum."""
    if len(ranks) == 1:
        fb, fi = final
        return prog.chunk(ranks[0], IN, j, cnt).copy(ranks[0], fb, fi)
    cur = prog.chunk(ranks[0], IN, j, cnt)
    for step, r in enumerate(ranks[1:], start=1):
        last = step == len(ranks) - 1
        dst = cur.copy(r, final[0], final[1]) if last else cur.copy(r, SCR, j)
        dst.reduce(prog.chunk(r, IN, j, cnt))
        cur = dst
    return cur


def _ring_forward(cur, ranks, buf: int, idx: int):
    """Copy ``cur`` along ranks (ranks[0] already holds it) into (buf, idx)."""
    for r in ranks[1:]:
        cur = cur.copy(r, buf, idx)
    return cur


def ring_allreduce(P: int, c: int = 1) -> Program:
    C = P * c
    prog = Program("allreduce", P, C, C, scratch_chunks=C, name=f"ring_allreduce_p{P}")
    for j in range(C):
        o = j // c
        chain = [(o + 1 + t) % P for t in range(P)]
        cur = _ring_reduce_chain(prog, chain, j, 1, (OUT, j))
        _ring_forward(cur, [(o + t) % P for t in range(P)], OUT, j)
    return prog


def ring_reducescatter(P: int, c: int = 1) -> Program:
    C = P * c
    prog = Program("reducescatter", P, C, c, scratch_chunks=C, name=f"ring_reducescatter_p{P}")
    for j in range(C):
        o = j // c
        chain = [(o + 1 + t) % P for t in range(P)]
        _ring_reduce_chain(prog, chain, j, 1, (OUT, j - o * c))
    return prog


def ring_allgather(P: int, c: int = 1) -> Program:
    prog = Program("allgather", P, c, P * c, name=f"ring_allgather_p{P}")
    for r in range(P):
        for t in range(c):
            cur = prog.chunk(r, IN, t).copy(r, OUT, r * c + t)
            _ring_forward(cur, [(r + s) % P for s in range(P)], OUT, r * c + t)
    return prog


def _ring_reduce_chain_ch(prog: Program, ranks, j: int, final, ch: int):
    """_ring_reduce_chain of one chunk on channel ``ch``."""
    if len(ranks) == 1:
        return prog.chunk(ranks[0], IN, j).copy(ranks[0], final[0], final[1], ch)
    cur = prog.chunk(ranks[0], IN, j)
    for step, r in enumerate(ranks[1:], start=1):
        last = step == len(ranks) - 1
        dst = cur.copy(r, final[0], final[1], ch) if last else cur.copy(r, SCR, j, ch)
        dst.reduce(prog.chunk(r, IN, j), ch)
        cur = dst
    return cur


def _ring_forward_ch(cur, ranks, buf: int, idx: int, ch: int):
    for r in ranks[1:]:
        cur = cur.copy(r, buf, idx, ch)
    return cur


def hierarchical_allreduce(G: int, L: int) -> Program:
    """Intra-group ring reduce-scatter of shards, cross-group ring AllReduce of every
    shard chunk among the ranks of a lane, intra-group ring all-gather of the shards,
    in one program (one kernel). Shard l is chunks [l*G, (l+1)*G); chunk l*G + g' of it
    travels on channel g' in every phase, so the G chunks of a shard run side by side on
    separate connections (on one channel they would share each connection, and the
    scheduler would serialize them: 31 dependent steps instead of 17 at G=2, L=8). The
    per-element chains, and so the results, are the same either way."""
    P, C = G * L, L * G
    prog = Program("allreduce", P, C, C, scratch_chunks=C, name=f"hier_allreduce_g{G}l{L}")
    for g in range(G):  # step 1: shard l reduced onto lane l
        for l in range(L):
            lanes = [g * L + (l + 1 + t) % L for t in range(L)]
            for gp in range(G):
                _ring_reduce_chain_ch(prog, lanes, l * G + gp, (OUT, l * G + gp), gp)
    for l in range(L):  # step 2: chunk l*G + g' reduced onto group g', then forwarded
        for gp in range(G):
            j = l * G + gp
            if G == 1:
                continue
            groups = [(gp + 1 + t) % G for t in range(G)]
            cur = prog.chunk(groups[0] * L + l, OUT, j)
            for h in groups[1:]:
                dst = prog.chunk(h * L + l, OUT, j)
                dst.reduce(cur, gp)
                cur = dst
            _ring_forward_ch(cur, [((gp + t) % G) * L + l for t in range(G)], OUT, j, gp)
    for g in range(G):  # step 3: shard l forwarded around the group
        for l in range(L):
            for gp in range(G):
                cur = prog.chunk(g * L + l, OUT, l * G + gp)
                _ring_forward_ch(cur, [g * L + (l + t) % L for t in range(L)], OUT, l * G + gp, gp)
    return prog


def hier_stage_reducescatter_intra(G: int, L: int) -> Program:
    """Stage 1 of the three-launch hierarchical AllReduce: ring ReduceScatter inside
    every group (shard l = chunk l lands in lane l's output)."""
    P = G * L
    prog = Program("reducescatter", P, L, 1, scratch_chunks=L, group_size=L, group_scope="intra",
                   name=f"hier_rs_intra_g{G}l{L}")
    for g in range(G):
        for l in range(L):
            lanes = [g * L + (l + 1 + t) % L for t in range(L)]
            _ring_reduce_chain(prog, lanes, l, 1, (OUT, 0))
    return prog


def hier_stage_allreduce_inter(G: int, L: int) -> Program:
    """Stage 2: ring AllReduce among the G ranks of each lane, G chunks."""
    P = G * L
    prog = Program("allreduce", P, G, G, scratch_chunks=G, group_size=L, group_scope="inter",
                   name=f"hier_ar_inter_g{G}l{L}")
    for l in range(L):
        for j in range(G):
            chain = [((j + 1 + t) % G) * L + l for t in range(G)]
            cur = _ring_reduce_chain(prog, chain, j, 1, (OUT, j))
            _ring_forward(cur, [((j + t) % G) * L + l for t in range(G)], OUT, j)
    return prog


def hier_stage_allgather_intra(G: int, L: int) -> Program:
    """Stage 3: ring AllGather inside every group."""
    P = G * L
    prog = Program("allgather", P, 1, L, group_size=L, group_scope="intra", name=f"hier_ag_intra_g{G}l{L}")
    for g in range(G):
        for l in range(L):
            cur = prog.chunk(g * L + l, IN, 0).copy(g * L + l, OUT, l)
            _ring_forward(cur, [g * L + (l + t) % L for t in range(L)], OUT, l)
    return prog


def tree_allreduce(P: int, c: int = 1) -> Program:
    """Binary-tree AllReduce: chunk j (owner o = j // c) is reduced up a heap-ordered
    tree over the ranks o, o+1, ..., o-1 (position t has children 2t+1 and 2t+2; the
    owner is the root), then copied back down it. A node's partial is (child 2t+2's
    partial + its own input) + child 2t+1's partial: the shallower subtree arrives
    first. About 2*log2(P) dependent hops
    per chunk instead of the ring's 2(P-1), for more bytes (two-child nodes keep a
    scratch partial); every rank is the root of c chunks. (The AutoCCL report finds
    tree above ring AllReduce in one setting, "other value" and its Table 5.)"""
    C = P * c
    prog = Program("allreduce", P, C, C, scratch_chunks=C, name=f"tree_allreduce_p{P}")
    for j in range(C):
        o = j // c
        rank = [(o + t) % P for t in range(P)]
        part = {}
        for t in reversed(range(P)):  # children (larger t) before parents
            kids = [u for u in (2 * t + 2, 2 * t + 1) if u < P]
            if not kids:
                part[t] = prog.chunk(rank[t], IN, j)
                continue
            buf = OUT if t == 0 else SCR
            acc = part[kids[0]].copy(rank[t], buf, j)
            acc.reduce(prog.chunk(rank[t], IN, j))
            for u in kids[1:]:
                acc.reduce(part[u])
            part[t] = acc
        if P == 1:
            prog.chunk(rank[0], IN, j).copy(rank[0], OUT, j)
        for t in range(P):  # broadcast, parents before children
            for u in (2 * t + 1, 2 * t + 2):
                if u < P:
                    prog.chunk(rank[t], OUT, j).copy(rank[u], OUT, j)
    return prog


def direct_alltoall(P: int) -> Program:
    """Every block straight to its destination (the single-phase baseline)."""
    prog = Program("alltoall", P, P, P, name=f"direct_alltoall_p{P}")
    for s in range(P):
        for r in range(P):
            prog.chunk(s, IN, r).copy(r, OUT, s)
    return prog


def two_phase_alltoall(G: int, L: int) -> Program:
    """Two-phase aggregated AllToAll (MSCCLang report, section 4.3). Phase 1: inside
    group g, the block that rank (g, l') holds for remote rank (h, l) is gathered at
    (g, l), slot l' of its region for group h. Phase 2: (g, l) sends that L-block
    region to (h, l) in one batched transfer. Phase 3: (h, l) places the L blocks at
    output blocks g*L .. g*L+L-1. Blocks for the own group go directly. A block bound
    for group h travels on channel h, so the G - 1 blocks one rank gathers at another for
    different groups do not queue on one connection."""
    P = G * L
    prog = Program("alltoall", P, P, P, scratch_chunks=2 * P, name=f"two_phase_alltoall_g{G}l{L}")
    # scratch [0, P): gather regions (region h = chunks [h*L, h*L+L)); [P, 2P): landing regions
    for g in range(G):
        for lp in range(L):
            src = g * L + lp
            for h in range(G):
                if h == g:
                    continue
                for l in range(L):
                    prog.chunk(src, IN, h * L + l).copy(g * L + l, SCR, h * L + lp, h)
    for g in range(G):
        for l in range(L):
            for h in range(G):
                if h == g:
                    continue
                landed = prog.chunk(g * L + l, SCR, h * L, L).copy(h * L + l, SCR, P + g * L, g)
                landed.copy(h * L + l, OUT, g * L, g)
    for g in range(G):
        for lp in range(L):
            for l in range(L):
                prog.chunk(g * L + lp, IN, g * L + l).copy(g * L + l, OUT, g * L + lp, g)
    return prog


def alltonext(G: int, L: int, split: bool = True) -> Program:
    """AllToNext: rank r's buffer goes to rank r+1 (not cyclic; rank 0's output is left
    alone). With ``split``, each cross-group hop (g, L-1) -> (g+1, 0) is cut into L parts
    and part j travels (g, L-1) -> (g, j) -> (g+1, j) -> (g+1, 0), so every rank of both
    groups carries a share of the cross-group traffic (MSCCLang report, section 4.4)."""
    P = G * L
    C = L if split else 1
    prog = Program("alltonext", P, C, C, scratch_chunks=2 * C if split else 0,
                   name=f"alltonext_g{G}l{L}{'_split' if split else ''}")
    for r in range(P - 1):
        g, l = divmod(r, L)
        cross = l == L - 1
        if not (split and cross):
            prog.chunk(r, IN, 0, C).copy(r + 1, OUT, 0)
            continue
        nxt = (g + 1) * L
        for j in range(C):
            cur = prog.chunk(r, IN, j)
            if g * L + j != r:
                cur = cur.copy(g * L + j, SCR, j)            # out-relay area [0, C)
            if j == 0:
                cur.copy(nxt, OUT, j)
            else:
                cur = cur.copy(nxt + j, SCR, C + j)          # in-relay area [C, 2C)
                cur.copy(nxt, OUT, j)
    return prog


def allgather_2d(G: int, L: int) -> Program:
    """Cross-group ring AllGather among the ranks of each lane, then an intra-group ring
    AllGather of the G gathered blocks. Block g*L + l travels on channel g in both
    phases: the G blocks that follow the same ring would otherwise share its connections
    and run one after another (23 dependent steps instead of 10 at 3x8)."""
    P = G * L
    prog = Program("allgather", P, 1, P, name=f"allgather_2d_g{G}l{L}")
    for l in range(L):
        for g in range(G):
            b = g * L + l
            cur = prog.chunk(b, IN, 0).copy(b, OUT, b, g)
            _ring_forward_ch(cur, [((g + t) % G) * L + l for t in range(G)], OUT, b, g)
    for h in range(G):
        for l in range(L):
            for g in range(G):
                b = g * L + l
                cur = prog.chunk(h * L + l, OUT, b)
                _ring_forward_ch(cur, [h * L + (l + t) % L for t in range(L)], OUT, b, g)
    return prog


def reducescatter_2d(G: int, L: int) -> Program:
    """Intra-group ring reduce of every block onto the lane that owns it, then a
    cross-group ring reduce among the ranks of that lane ending at the owner. Block
    h*L + l travels on channel h in both phases, so the G blocks that follow the same
    chains do not share connections (24 dependent steps instead of 10 at 3x8)."""
    P = G * L
    prog = Program("reducescatter", P, P, 1, scratch_chunks=P, name=f"reducescatter_2d_g{G}l{L}")
    for g in range(G):
        for b in range(P):
            l = b % L
            lanes = [g * L + (l + 1 + t) % L for t in range(L)]
            _ring_reduce_chain_ch(prog, lanes, b, (SCR, b), b // L)
    for b in range(P):
        h, l = divmod(b, L)
        groups = [(h + 1 + t) % G for t in range(G)]
        cur = prog.chunk(groups[0] * L + l, SCR, b)
        if G == 1:
            cur.copy(b, OUT, 0, h)
            continue
        for step, gg in enumerate(groups[1:], start=1):
            if step == G - 1:
                dst = prog.chunk(gg * L + l, SCR, b).copy(gg * L + l, OUT, 0, h)
            else:
                dst = prog.chunk(gg * L + l, SCR, b)
            dst.reduce(cur, h)
            cur = dst
    return prog


REGISTRY = {
    "ring_allreduce": ring_allreduce,
    "tree_allreduce": tree_allreduce,
    "ring_reducescatter": ring_reducescatter,
    "ring_allgather": ring_allgather,
    "hierarchical_allreduce": hierarchical_allreduce,
    "direct_alltoall": direct_alltoall,
    "two_phase_alltoall": two_phase_alltoall,
    "alltonext": alltonext,
    "allgather_2d": allgather_2d,
    "reducescatter_2d": reducescatter_2d,
    "hier_stage_reducescatter_intra": hier_stage_reducescatter_intra,
    "hier_stage_allreduce_inter": hier_stage_allreduce_inter,
    "hier_stage_allgather_intra": hier_stage_allgather_intra,
}
