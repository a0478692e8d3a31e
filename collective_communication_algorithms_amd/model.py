"""The pages' alpha-beta (Hockney) cost formulas and busbw coefficients.

Used to put predictions beside measured times.  Symbols as on the pages: N
ranks, M bytes per rank, alpha start-up latency (seconds), beta link bandwidth
(bytes per second), k pipeline chunks.
"""

from __future__ import annotations

import math


def _L(N: int) -> int:
    return math.ceil(math.log2(N)) if N > 1 else 0


def time(kind: str, algo: str, N: int, M: float, alpha: float, beta: float, k: int = 1) -> float:
    """Predicted time of one call.

    Ring ("集合通信算法延迟公式", eq:model-algo-ring-rs / -ag / -ar), Halving-
    Doubling (eq:model-algo-rhd-*), Double Binary Tree (eq:model-algo-dbt-ar),
    Pairwise / Bruck AllToAll (eq:model-algo-a2a-pairwise / -bruck), Broadcast
    ("一对多通信：Broadcast 与 Scatter", eq:chain-bcast, eq:binomial-bcast,
    eq:pipe-chain-bcast, eq:pipe-tree-bcast, and the bidirectional ring of
    "SCCL 的 Broadcast 实现"), binomial Scatter / Gather
    (eq:binomial-scatter, eq:onetoall-gather-scatter-duality).
    """
    L = _L(N)
    frac = (N - 1) / N
    if kind == "allreduce":
        if algo == "ring":
            return 2 * (N - 1) * alpha + 2 * frac * M / beta
        if algo == "rhd":
            return 2 * L * alpha + 2 * frac * M / beta
        if algo == "dbt":
            return 2 * L * alpha + L * M / beta
    if kind in ("reducescatter", "allgather"):
        if algo == "ring":
            return (N - 1) * alpha + frac * M / beta
        if algo == "rhd":
            return L * alpha + frac * M / beta
    if kind == "broadcast":
        if algo == "chain":
            return (N - 1) * (alpha + M / beta)
        if algo == "binomial":
            return L * (alpha + M / beta)
        if algo == "chain_pipe":
            return (N + k - 2) * (alpha + M / (k * beta))
        if algo == "binomial_pipe":
            return (L + k - 1) * (alpha + M / (k * beta))
        if algo == "bidir_ring":
            # both ring directions from the root (SCCL's 4-chip scheme): the
            # chain is ceil((N-1)/2) hops long, pipelined in k chunks
            return (N // 2 + k - 1) * (alpha + M / (k * beta)) if N > 1 else 0.0
    if kind in ("scatter", "gather") and algo == "binomial":
        return L * alpha + frac * M / beta
    if kind == "scatter" and algo == "linear":
        return (N - 1) * alpha + frac * M / beta          # eq:onetoall-scatter-naive
    if kind == "broadcast" and algo == "scatter_allgather":
        return (time("scatter", "binomial", N, M, alpha, beta) +
                time("allgather", "ring", N, M, alpha, beta))
    if kind == "reduce" and algo == "binomial":
        return L * (alpha + M / beta)                      # eq:model-algo-reduce-tree
    if kind == "alltoall":
        if algo in ("pairwise", "ring"):
            return (N - 1) * alpha + frac * M / beta
        if algo == "bruck":
            return L * alpha + frac * M / beta
    if kind == "reduce" and algo == "tree":
        return L * (alpha + M / beta)
    raise ValueError(f"no formula for {kind}/{algo}")


def latency_steps(kind: str, algo: str, N: int, k: int = 1) -> int:
    """The alpha coefficient of ``time`` (number of start-ups)."""
    return round(time(kind, algo, N, 0.0, 1.0, 1.0, k))


def bandwidth_coef(kind: str, algo: str, N: int, k: int = 1) -> float:
    """The M/beta coefficient of ``time``."""
    return time(kind, algo, N, 1.0, 0.0, 1.0, k)


def busbw_coef(kind: str, N: int) -> float:
    """busbw = algbw * coefficient ("集合通信算法延迟公式", @tbl-model-algo-busbw-coef).

    Scatter and Gather are not in the table; their coefficient follows the same
    rule (the bandwidth lower bound times beta over M: eq:onetoall-scatter-bw-lb).
    """
    if kind == "allreduce":
        return 2 * (N - 1) / N
    if kind in ("allgather", "reducescatter", "alltoall", "scatter", "gather"):
        return (N - 1) / N
    if kind in ("broadcast", "reduce"):
        return 1.0
    raise ValueError(kind)


def ring_dbt_crossover(N: int, alpha: float, beta: float) -> float:
    """Message size where Ring and DBT AllReduce take equal time
    (eq:model-algo-ring-dbt-crossover)."""
    L = math.log2(N)
    return 2 * alpha * beta * ((N - 1) - L) / (L - 2 * (N - 1) / N)


def best_chunks(algo: str, N: int, M: float, alpha: float, beta: float, kmax: int = 4096) -> int:
    """Integer k minimising the pipeline formula (the page prints a closed-form
    k* for the chain that does not minimise its own formula; the argmin is used)."""
    return min(range(1, kmax + 1), key=lambda k: (time("broadcast", algo, N, M, alpha, beta, k), k))


def overlapped_time(compute: float, comm: float) -> float:
    """Wall time of compute and a collective that run concurrently on two
    streams: the longer of the two (the HCCL blog, 延迟掩盖：计算与通信的Overlap,
    Overlap的性能收益: with overlap only the part of the collective that
    outlasts the compute remains visible).  Times in any one unit."""
    return max(compute, comm)


def serial_time(compute: float, comm: float) -> float:
    """Wall time of compute followed by the collective on one stream."""
    return compute + comm


def hidden_fraction(compute: float, comm: float, both: float) -> float:
    """Share of the collective's time that a measured overlapped run hid:
    (compute + comm - both) / comm; 1 means fully hidden, 0 none."""
    return (compute + comm - both) / comm if comm > 0 else 0.0
