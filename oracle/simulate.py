"""Snapshot-per-step execution of a schedule on host buffers (oracle; test
infrastructure only).

For each step: first every row's source slice is copied out (all sends of a
step leave from the state before the step), then the rows are applied in row
order, ``dst = src`` or ``dst = dst (+) src``.  Two reduce rows of one step into
the same destination therefore accumulate in row order; the Double Binary Tree
relies on that for a parent with two children.

Buffers hold ``count`` elements per rank (numpy storage types, bf16 as uint16).
For every collective except AllToAll, an out-of-place call is defined as the
in-place call applied to a copy of the send buffers.
"""

from __future__ import annotations

import numpy as np

from . import numerics
from .schedules import Plan, make_plan, part


def check_hazards(plan: Plan) -> None:
    """Raise if a step is not free of conflicts inside the step.

    Ordinary step: no row may read (from the receive side) a region that
    another row of the step writes, and two rows may write overlapping regions
    only if both are reduce rows (they accumulate in row order).
    Staged step (a permutation done with staging): the written regions must be
    pairwise disjoint; reads are from the snapshot.
    """
    for st, rows in enumerate(plan.steps):
        writes = {}
        reads = {}
        for idx, r in enumerate(rows):
            writes.setdefault(r.dst, []).append((r.dst_off, r.dst_off + r.n, idx, r.reduce))
            if not r.from_send:
                reads.setdefault(r.src, []).append((r.src_off, r.src_off + r.n, idx))
        for rank, ws in writes.items():
            for x in range(len(ws)):
                for y in range(x + 1, len(ws)):
                    a, b = ws[x], ws[y]
                    if a[0] < b[1] and b[0] < a[1] and not (a[3] and b[3] and not plan.staged[st]):
                        raise AssertionError(f"step {st}: rows {a[2]} and {b[2]} both write "
                                             f"rank {rank}")
        if plan.staged[st]:
            continue
        for rank, rs in reads.items():
            ws = sorted(writes.get(rank, []))
            for lo, hi, i in rs:
                for a, b, j, _ in ws:
                    if a < hi and lo < b and i != j:
                        raise AssertionError(f"step {st}: row {i} reads rank {rank} "
                                             f"[{lo}, {hi}) which row {j} writes")


def run_plan(plan: Plan, dtype: str, op: str, send: list, recv: list | None = None,
             trace: bool = False):
    """Execute ``plan`` and return the receive buffers (and the per-row checksums
    when ``trace``).  ``send`` is not modified."""
    N = plan.nranks
    if len(send) != N:
        raise ValueError("one buffer per rank")
    if plan.kind == "alltoall":
        recv = [np.zeros_like(a) for a in send] if recv is None else [r.copy() for r in recv]
    else:
        recv = [a.copy() for a in send]
    sums = []
    for rows in plan.steps:
        snaps = []
        for r in rows:
            space = send if r.from_send else recv
            snaps.append(space[r.src][r.src_off:r.src_off + r.n].copy())
        for r, s in zip(rows, snaps):
            d = recv[r.dst][r.dst_off:r.dst_off + r.n]
            if r.reduce:
                d[...] = numerics.combine(d, s, dtype, op)
            else:
                d[...] = s
            if trace:
                sums.append(numerics.row_checksum(d))
    return (recv, sums) if trace else recv


def defined_regions(kind: str, nranks: int, count: int, root: int = 0):
    """Per rank, the element ranges whose final value the collective defines.

    AllReduce / AllGather / Broadcast / AllToAll: the whole buffer.
    ReduceScatter and Scatter: chunk i of rank i.  Gather and Reduce: all of
    the root.
    """
    N = nranks
    out = []
    for i in range(N):
        if kind in ("allreduce", "allgather", "broadcast", "alltoall"):
            out.append([(0, count)])
        elif kind in ("reducescatter", "scatter"):
            out.append([(part(count, N, i), part(count, N, i + 1))])
        elif kind in ("gather", "reduce"):
            out.append([(0, count)] if i == root else [])
        else:
            raise ValueError(kind)
    return out


def _run(kind, algo, arrays, dtype, op="sum", root=0, chunks=1, trace=False, recv=None):
    plan = make_plan(kind, algo, len(arrays), len(arrays[0]), root, chunks)
    return run_plan(plan, dtype, op, arrays, recv=recv, trace=trace)


def allreduce(arrays, dtype, op="sum", algo="ring", trace=False):
    """Every rank ends with the elementwise reduction over ranks."""
    return _run("allreduce", algo, arrays, dtype, op, trace=trace)


def reducescatter(arrays, dtype, op="sum", algo="ring", trace=False):
    """Rank i ends with chunk i of the reduction."""
    return _run("reducescatter", algo, arrays, dtype, op, trace=trace)


def allgather(arrays, dtype, algo="ring", trace=False):
    """Rank i starts with chunk i; every rank ends with all chunks."""
    return _run("allgather", algo, arrays, dtype, trace=trace)


def broadcast(arrays, dtype, root=0, algo="binomial", chunks=1, trace=False):
    """B_i = A_root (eq:onetoall-bcast-semantic)."""
    return _run("broadcast", algo, arrays, dtype, root=root, chunks=chunks, trace=trace)


def scatter(arrays, dtype, root=0, algo="binomial", trace=False):
    """Rank i receives chunk i of the root (eq:onetoall-scatter-semantic)."""
    return _run("scatter", algo, arrays, dtype, root=root, trace=trace)


def gather(arrays, dtype, root=0, algo="binomial", trace=False):
    """The root collects chunk i of every rank i."""
    return _run("gather", algo, arrays, dtype, root=root, trace=trace)


def reduce(arrays, dtype, op="sum", root=0, algo="binomial", trace=False):
    """The root ends with the elementwise reduction over ranks."""
    return _run("reduce", algo, arrays, dtype, op, root=root, trace=trace)


def alltoall(send, dtype, algo="pairwise", trace=False):
    """recv_j block i = send_i block j (blocks of count/N elements)."""
    return _run("alltoall", algo, send, dtype, trace=trace)


def run_plan_columns(plan: Plan, dtype: str, op: str, cols: np.ndarray, send_cols: list) -> list:
    """The plan restricted to a set of columns (element offsets) of every rank.

    Valid for every schedule whose rows keep their offset (src_off == dst_off),
    i.e. all but AllToAll: output element x of a rank then depends only on
    element x of the ranks, through exactly the rows that cover x.  ``cols`` is
    sorted; ``send_cols[r]`` holds rank r's values at those columns.  Returns the
    receive side at those columns, computed with the same snapshot-per-step rule
    as ``run_plan``.
    """
    if plan.kind == "alltoall":
        raise ValueError("alltoall rows move data between offsets")
    recv = [np.array(a, copy=True) for a in send_cols]
    for rows in plan.steps:
        moves = []
        for r in rows:
            assert r.src_off == r.dst_off
            a = np.searchsorted(cols, r.src_off, side="left")
            b = np.searchsorted(cols, r.src_off + r.n, side="left")
            if a < b:
                moves.append((r, a, b, recv[r.src][a:b].copy()))
        for r, a, b, s in moves:
            d = recv[r.dst][a:b]
            d[...] = numerics.combine(d, s, dtype, op) if r.reduce else s
    return recv
