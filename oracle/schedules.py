"""Step-by-step schedules of every collective (oracle; test infrastructure only).

A schedule is a list of steps; a step is a list of rows; a row says "rank ``src``
sends ``n`` elements at element offset ``src_off`` to rank ``dst``, which stores
them at ``dst_off``, either overwriting (copy) or as ``dst <- dst (+) src``
(reduce)".  All sends of one step leave from the state before the step: in the
pages' model the sends of one step happen at once ("一对多通信：Broadcast 与
Scatter", 二叉树 Broadcast: every rank that holds the data sends in the same step).

Conventions (readings of points the pages leave open):
  * N equal chunks of one rank buffer use the floor partition
    chunk c = elements [c*count//N, (c+1)*count//N).  The HCCL blog's listing
    computes ``count / size`` and drops the remainder; on the configurations the
    pages discuss N divides count and every reading agrees.
  * After ReduceScatter rank i owns chunk i (the pages do not say which 1/N a
    rank ends with).  The Ring indices are the HCCL blog's shifted by one so
    that Ring AllReduce is literally ReduceScatter followed by AllGather.
  * Recursive halving pairs at distances N/2, N/4, ..., 1 with the lower rank
    keeping the lower half, then doubling at 1, 2, ..., N/2 (the order of the
    source the page cites; the page's "distance 2^k" would leave rank r with
    chunk bitreverse(r)).  Round k still moves M/2^(k+1) and 2^k*M/N bytes.
  * The two Double Binary Tree trees are built as in ``dbt_trees``.
  * Pipeline chunks are the floor partition of count into k parts.
  * Scatter / Gather keep every chunk at its in-place offset (chunk i of each
    rank buffer); a chunk range that wraps past rank N-1 becomes two rows.
  * Pairwise round k sends block (i+k) mod N of rank i to rank (i+k) mod N.
  * Bruck: rotate, then per round k shift every block index with bit k set by
    2^k ranks, then rotate back (the source the page cites).

Zero-length rows are dropped; the step itself still exists, so the step count
is a property of the algorithm and N only.
"""

from __future__ import annotations

from dataclasses import dataclass, field

KINDS = ("allreduce", "reducescatter", "allgather", "broadcast", "scatter",
         "gather", "alltoall", "reduce")
ALGOS = ("ring", "rhd", "dbt", "binomial", "chain_pipe", "binomial_pipe",
         "pairwise", "bruck", "linear", "scatter_allgather", "bidir_ring")


@dataclass(frozen=True)
class Row:
    step: int
    src: int
    dst: int
    src_off: int
    dst_off: int
    n: int
    reduce: bool = False
    from_send: bool = False   # AllToAll: source is the send buffer


@dataclass
class Plan:
    kind: str
    algo: str
    nranks: int
    count: int
    root: int = 0
    chunks: int = 1
    steps: list = field(default_factory=list)   # list[list[Row]]
    local: list = field(default_factory=list)   # per step: a local phase, not a counted step
    staged: list = field(default_factory=list)  # per step: a permutation done with staging

    @property
    def nsteps(self) -> int:
        """Counted communication steps (local rearrangement phases excluded)."""
        return sum(1 for x in self.local if not x)

    @property
    def rows(self) -> list:
        return [r for s in self.steps for r in s]


def ceil_log2(n: int) -> int:
    k = 0
    while (1 << k) < n:
        k += 1
    return k


def is_pow2(n: int) -> bool:
    return n >= 1 and (n & (n - 1)) == 0


def part(count: int, parts: int, c: int) -> int:
    """Start element of part c of the floor partition of ``count`` into ``parts``."""
    return (c * count) // parts


class _Builder:
    def __init__(self, plan: Plan):
        self.plan = plan

    def new_step(self, local=False, staged=False) -> int:
        self.plan.steps.append([])
        self.plan.local.append(local)
        self.plan.staged.append(staged)
        return len(self.plan.steps) - 1

    def row(self, step, src, dst, off, n, reduce=False, dst_off=None, from_send=False):
        if n <= 0:
            return
        self.plan.steps[step].append(Row(step, src, dst, off, off if dst_off is None else dst_off,
                                         n, reduce, from_send))


# ----------------------------------------------------------------------------
# Ring ("集合通信算法延迟公式", Ring AllReduce; eq:model-algo-ring-rs / -ag / -ar;
# Ring AllGather / Ring ReduceScatter sections)
# ----------------------------------------------------------------------------

def _ring_rs(b: _Builder, N: int, count: int):
    """N-1 steps; at step s rank r sends chunk (r-s-1) mod N to r+1, which reduces it."""
    for s in range(N - 1):
        st = b.new_step()
        for r in range(N):
            c = (r - s - 1) % N
            lo, hi = part(count, N, c), part(count, N, c + 1)
            b.row(st, r, (r + 1) % N, lo, hi - lo, reduce=True)


def _ring_ag(b: _Builder, N: int, count: int):
    """N-1 steps; at step s rank r forwards chunk (r-s) mod N to r+1 (copy)."""
    for s in range(N - 1):
        st = b.new_step()
        for r in range(N):
            c = (r - s) % N
            lo, hi = part(count, N, c), part(count, N, c + 1)
            b.row(st, r, (r + 1) % N, lo, hi - lo)


# ----------------------------------------------------------------------------
# Recursive Halving-Doubling (eq:model-algo-rhd-rs / -ag / -ar)
# ----------------------------------------------------------------------------

def _rhd_rs(b: _Builder, N: int, count: int):
    """log2 N halving rounds.  Round k: distance d = N >> (k+1); each rank keeps
    half of its current chunk range (lower rank the lower half) and reduces the
    partner's copy of that half into it."""
    seg = [(0, N)] * N
    k = 0
    while (N >> (k + 1)) >= 1:
        d = N >> (k + 1)
        st = b.new_step()
        new = list(seg)
        for r in range(N):
            lo, hi = seg[r]
            mid = (lo + hi) // 2
            keep = (lo, mid) if (r & d) == 0 else (mid, hi)
            new[r] = keep
            a, z = part(count, N, keep[0]), part(count, N, keep[1])
            b.row(st, r ^ d, r, a, z - a, reduce=True)
        seg = new
        k += 1
    return seg


def _rhd_ar_folded(b: _Builder, N: int, count: int):
    """Recursive halving-doubling AllReduce for N that is not a power of two.

    The page requires N = 2^n; the source it cites folds the surplus first.
    With P the largest power of two below N and r = N - P: rank 2i reduces its
    whole buffer into rank 2i+1 (i < r); the P ranks 2i+1 (i < r) and 2r..N-1
    then run halving and doubling on the P-way partition of the buffer as core
    ranks 0..P-1; finally rank 2i+1 copies the result back to rank 2i.
    2 log2 P + 2 steps."""
    P = 1 << (N.bit_length() - 1)
    r = N - P
    core = [2 * i + 1 for i in range(r)] + list(range(2 * r, N))
    st = b.new_step()
    for i in range(r):
        b.row(st, 2 * i, 2 * i + 1, 0, count, reduce=True)
    seg = [(0, P)] * P
    d = P // 2
    while d >= 1:
        st = b.new_step()
        new = list(seg)
        for j in range(P):
            lo, hi = seg[j]
            mid = (lo + hi) // 2
            keep = (lo, mid) if (j & d) == 0 else (mid, hi)
            new[j] = keep
            a, z = part(count, P, keep[0]), part(count, P, keep[1])
            b.row(st, core[j ^ d], core[j], a, z - a, reduce=True)
        seg = new
        d //= 2
    seg = [(j, j + 1) for j in range(P)]
    d = 1
    while d < P:
        st = b.new_step()
        new = list(seg)
        for j in range(P):
            lo, hi = seg[j ^ d]
            a, z = part(count, P, lo), part(count, P, hi)
            b.row(st, core[j ^ d], core[j], a, z - a)
            new[j] = (min(seg[j][0], lo), max(seg[j][1], hi))
        seg = new
        d <<= 1
    st = b.new_step()
    for i in range(r):
        b.row(st, 2 * i + 1, 2 * i, 0, count)


def _rhd_ag(b: _Builder, N: int, count: int):
    """log2 N doubling rounds.  Round k: distance d = 2^k; each rank copies in its
    partner's current block of 2^k chunks; the block doubles."""
    seg = [(r, r + 1) for r in range(N)]
    d = 1
    while d < N:
        st = b.new_step()
        new = list(seg)
        for r in range(N):
            p = r ^ d
            lo, hi = seg[p]
            a, z = part(count, N, lo), part(count, N, hi)
            b.row(st, p, r, a, z - a)
            new[r] = (min(seg[r][0], lo), max(seg[r][1], hi))
        seg = new
        d <<= 1


# ----------------------------------------------------------------------------
# Double Binary Tree (eq:model-algo-dbt-ar)
# ----------------------------------------------------------------------------

def _tz(x: int) -> int:
    t = 0
    while x % 2 == 0:
        x //= 2
        t += 1
    return t


def dbt_trees(N: int):
    """The two complementary trees, as {node: [children]} with root noted.

    The page asks for two binary trees of height log2 N with different parent /
    child relations, each carrying half the data.  Construction (any N >= 2;
    for N = 2^n the two trees have complementary leaves):
    tree 1 has rank 0 as root whose only child is the root of build(1, N);
    build(lo, hi) takes as node the element of [lo, hi) with the most trailing
    zero bits (unique in a run of consecutive integers), with left subtree
    build(lo, m) and right subtree build(m+1, hi).  Tree 2 is tree 1 with every
    label shifted by +1 mod N; the odd ranks are tree 1's leaves and the even
    ranks tree 2's.
    """
    children = {}

    def build(lo, hi):
        if lo >= hi:
            return None
        m = max(range(lo, hi), key=_tz)
        children[m] = []
        left = build(lo, m)
        right = build(m + 1, hi)
        for c in (left, right):
            if c is not None:
                children[m].append(c)
        return m

    t1 = {0: []}
    top = build(1, N)
    t1.update(children)
    if top is not None:
        t1[0].append(top)
    t2 = {(u + 1) % N: [(c + 1) % N for c in cs] for u, cs in t1.items()}
    return (0, t1), (1 % N, t2)


def _heights_depths(root, tree):
    h, dpt = {}, {root: 0}

    def height(u):
        if u not in h:
            cs = tree.get(u, [])
            h[u] = 0 if not cs else 1 + max(height(c) for c in cs)
        return h[u]

    height(root)
    order = [root]
    for u in order:
        for c in tree.get(u, []):
            dpt[c] = dpt[u] + 1
            order.append(c)
    return h, dpt


def _dbt_ar(b: _Builder, N: int, count: int):
    """Reduce up both trees (level by height, left child before right child,
    tree 1 before tree 2), then broadcast down (level by depth).  Tree 1 carries
    elements [0, count//2), tree 2 [count//2, count).  2*ceil(log2 N) steps.
    When a node's children have different heights (N not a power of two) the
    lower child's value arrives one step earlier and is reduced first."""
    H = ceil_log2(N)
    halves = [(0, count // 2), (count // 2, count)]
    trees = dbt_trees(N)
    info = [_heights_depths(root, t) for root, t in trees]
    for h in range(1, H + 1):
        st = b.new_step()
        for (root, t), (hts, _), (lo, hi) in zip(trees, info, halves):
            for parent in sorted(t):
                for c in t[parent]:
                    if hts[c] == h - 1:
                        b.row(st, c, parent, lo, hi - lo, reduce=True)
    for j in range(1, H + 1):
        st = b.new_step()
        for (root, t), (_, dps), (lo, hi) in zip(trees, info, halves):
            for parent in sorted(t):
                if dps[parent] == j - 1:
                    for c in t[parent]:
                        b.row(st, parent, c, lo, hi - lo)


# ----------------------------------------------------------------------------
# One-to-many ("一对多通信：Broadcast 与 Scatter")
# ----------------------------------------------------------------------------

def _binomial_pairs(N: int, j: int):
    """Sub-step j (1-based) of the binomial tree in relative ranks: distance
    d = 2^(L-j); every v that is a multiple of 2d with v+d < N sends to v+d."""
    L = ceil_log2(N)
    d = 1 << (L - j)
    return [(v, v + d, d) for v in range(0, N, 2 * d) if v + d < N]


def _bcast_binomial(b: _Builder, N, count, root):
    """ceil(log2 N) steps, the whole message each time (eq:binomial-bcast)."""
    for j in range(1, ceil_log2(N) + 1):
        st = b.new_step()
        for v, w, _ in _binomial_pairs(N, j):
            b.row(st, (root + v) % N, (root + w) % N, 0, count)


def _bcast_chain_pipe(b: _Builder, N, count, root, k):
    """Chain 0 -> 1 -> ... -> N-1 (relative), k chunks; chunk c enters at step c
    and crosses hop h at step c+h; N+k-2 steps (eq:pipe-chain-bcast).  k = 1 is the
    chain Broadcast (eq:chain-bcast)."""
    if N < 2:
        return
    for t in range(N + k - 2):
        st = b.new_step()
        for c in range(k):
            h = t - c
            if 0 <= h <= N - 2:
                lo, hi = part(count, k, c), part(count, k, c + 1)
                b.row(st, (root + h) % N, (root + h + 1) % N, lo, hi - lo)


def _bcast_bidir_ring(b: _Builder, N, count, root, k):
    """Bidirectional ring ("一对多通信：Broadcast 与 Scatter", SCCL 的 Broadcast 实现):
    the root sends both ways round the ring at once; the clockwise chain covers
    relative ranks 1..ceil((N-1)/2), the counter-clockwise chain N-1 down to
    ceil((N-1)/2)+1.  With k chunks, chunk c crosses hop h of each chain at step
    c+h: ceil((N-1)/2)+k-1 steps."""
    cw, ccw = N // 2, (N - 1) // 2
    for t in range(cw + k - 1 if N > 1 else 0):
        st = b.new_step()
        for c in range(k):
            h = t - c
            lo, hi = part(count, k, c), part(count, k, c + 1)
            if 0 <= h < cw:
                b.row(st, (root + h) % N, (root + h + 1) % N, lo, hi - lo)
            if 0 <= h < ccw:
                b.row(st, (root - h) % N, (root - h - 1) % N, lo, hi - lo)


def _bcast_binomial_pipe(b: _Builder, N, count, root, k):
    """Binomial tree, k chunks; chunk c takes binomial sub-step j+1 at step c+j;
    ceil(log2 N)+k-1 steps (eq:pipe-tree-bcast).  k = 1 is the binomial tree."""
    L = ceil_log2(N)
    if L == 0:
        return
    for t in range(L + k - 1):
        st = b.new_step()
        for c in range(k):
            j = t - c
            if 0 <= j <= L - 1:
                lo, hi = part(count, k, c), part(count, k, c + 1)
                for v, w, _ in _binomial_pairs(N, j + 1):
                    b.row(st, (root + v) % N, (root + w) % N, lo, hi - lo)


def _reduce_binomial(b: _Builder, N, count, root):
    """Tree Reduce ("集合通信算法延迟公式", Tree Reduce: the mirror of the tree
    Broadcast, log2 N steps of the whole message): at step j (distance
    d = 2^(j-1)) every relative rank v whose lowest set bit is d sends its
    partial result to v-d, which reduces it into its own."""
    L = ceil_log2(N)
    for j in range(1, L + 1):
        d = 1 << (j - 1)
        st = b.new_step()
        for v in range(d, N, 2 * d):
            b.row(st, (root + v) % N, (root + v - d) % N, 0, count, reduce=True)


def _scatter_linear(b: _Builder, N, count, root):
    """Naive Scatter ("一对多通信：Broadcast 与 Scatter", 逐个发送（Naive）):
    the root sends each rank its chunk directly, one rank per step, N-1 steps."""
    for i in range(1, N):
        st = b.new_step()
        a = (root + i) % N
        lo, hi = part(count, N, a), part(count, N, a + 1)
        b.row(st, root, a, lo, hi - lo)


def _chunk_range_rows(b: _Builder, st, N, count, root, src_v, dst_v, rel_lo, rel_hi):
    """Rows moving relative chunks [rel_lo, rel_hi) from relative rank src_v to
    dst_v; absolute chunk = (root + rel) mod N, split where it wraps."""
    a0 = (root + rel_lo) % N
    n = rel_hi - rel_lo
    first = min(n, N - a0)
    for a, m in ((a0, first), (0, n - first)):
        if m > 0:
            lo, hi = part(count, N, a), part(count, N, a + m)
            b.row(st, (root + src_v) % N, (root + dst_v) % N, lo, hi - lo)


def _scatter_binomial(b: _Builder, N, count, root):
    """ceil(log2 N) steps; at sub-step j every holder v sends the chunks of the
    subtree it hands to v+d, i.e. relative chunks [v+d, v+2d) (eq:binomial-scatter)."""
    for j in range(1, ceil_log2(N) + 1):
        st = b.new_step()
        for v, w, d in _binomial_pairs(N, j):
            _chunk_range_rows(b, st, N, count, root, v, w, w, min(w + d, N))


def _gather_binomial(b: _Builder, N, count, root):
    """Scatter with the data flow reversed (eq:onetoall-gather-scatter-duality):
    at step j (distance d = 2^(j-1)) every v whose lowest set bit is d sends the
    relative chunks [v, v+d) it has collected to v-d."""
    L = ceil_log2(N)
    for j in range(1, L + 1):
        d = 1 << (j - 1)
        st = b.new_step()
        for v in range(d, N, 2 * d):
            _chunk_range_rows(b, st, N, count, root, v, v - d, v, min(v + d, N))


# ----------------------------------------------------------------------------
# AllToAll ("集合通信算法延迟公式", AllToAll section; eq:model-algo-a2a-pairwise /
# -bruck)
# ----------------------------------------------------------------------------

def _a2a_pairwise(b: _Builder, N, count):
    """Own block copied locally, then N-1 rounds: in round k rank i sends its
    block (i+k) mod N to rank (i+k) mod N, which stores it as block i."""
    B = count // N
    st = b.new_step(local=True)
    for i in range(N):
        b.row(st, i, i, i * B, B, dst_off=i * B, from_send=True)
    for k in range(1, N):
        st = b.new_step()
        for i in range(N):
            j = (i + k) % N
            b.row(st, i, j, j * B, B, dst_off=i * B, from_send=True)


def _a2a_ring(b: _Builder, N, count):
    """Ring AllToAll ("集合通信算法延迟公式", Ring: each round only between ring
    neighbours), read as store-and-forward: in round t = 1..N-1 every rank passes
    to its successor the N-t blocks that have not yet reached their destination.
    Storage: first tmp_i[j] = send_i[(i+j) mod N] (block j is t hops from home
    after t rounds), round t moves slots t..N-1 one rank on, so slot t arrives;
    last recv_i[(i-j) mod N] = tmp_i[j].  tmp is the receive buffer."""
    B = count // N
    st = b.new_step(local=True)
    for i in range(N):
        for j in range(N):
            b.row(st, i, i, ((i + j) % N) * B, B, dst_off=j * B, from_send=True)
    for t in range(1, N):
        st = b.new_step(staged=True)
        for j in range(t, N):
            for i in range(N):
                b.row(st, i, (i + 1) % N, j * B, B)
    st = b.new_step(local=True, staged=True)
    for i in range(N):
        for j in range(N):
            b.row(st, i, i, j * B, B, dst_off=((i - j) % N) * B)


def _a2a_bruck(b: _Builder, N, count):
    """Phase 1 (local): tmp_i[j] = send_i[(i+j) mod N].  Round k = 0..L-1: every
    block index j with bit k set moves from rank i to rank i+2^k (all at once).
    Phase 3 (local): recv_i[(i-j) mod N] = tmp_i[j].  tmp is the receive buffer."""
    B = count // N
    st = b.new_step(local=True)
    for i in range(N):
        for j in range(N):
            b.row(st, i, i, ((i + j) % N) * B, B, dst_off=j * B, from_send=True)
    for k in range(ceil_log2(N)):
        st = b.new_step(staged=True)
        for j in range(N):
            if (j >> k) & 1:
                for i in range(N):
                    b.row(st, i, (i + (1 << k)) % N, j * B, B)
    st = b.new_step(local=True, staged=True)
    for i in range(N):
        for j in range(N):
            b.row(st, i, i, j * B, B, dst_off=((i - j) % N) * B)


# ----------------------------------------------------------------------------

VALID = {
    "allreduce": ("ring", "rhd", "dbt"),
    "reducescatter": ("ring", "rhd"),
    "allgather": ("ring", "rhd"),
    "broadcast": ("binomial", "chain_pipe", "binomial_pipe"),
    "scatter": ("binomial",),
    "gather": ("binomial",),
    "alltoall": ("pairwise", "bruck"),
    "reduce": ("binomial",),
}
VALID["broadcast"] = VALID["broadcast"] + ("scatter_allgather", "bidir_ring")
VALID["scatter"] = VALID["scatter"] + ("linear",)
VALID["alltoall"] = VALID["alltoall"] + ("ring",)


def make_plan(kind: str, algo: str, nranks: int, count: int, root: int = 0,
              chunks: int = 1) -> Plan:
    """The schedule of one collective call, all rows in step order."""
    N = int(nranks)
    if kind not in VALID or algo not in VALID[kind]:
        raise ValueError(f"{algo} is not an algorithm of {kind}")
    if N < 1:
        raise ValueError("nranks")
    if algo == "rhd" and kind != "allreduce" and not is_pow2(N):
        raise ValueError("recursive halving-doubling ReduceScatter / AllGather need N = 2^n")
    if kind == "alltoall" and count % N:
        raise ValueError("alltoall needs count divisible by N")
    pipelined = algo in ("chain_pipe", "binomial_pipe", "bidir_ring")
    if pipelined and not (1 <= chunks <= max(count, 1)):
        raise ValueError("chunks")
    p = Plan(kind, algo, N, count, root, chunks if pipelined else 1)
    b = _Builder(p)
    if kind == "allreduce":
        if algo == "ring":
            _ring_rs(b, N, count)
            _ring_ag(b, N, count)
        elif algo == "rhd":
            if is_pow2(N):
                _rhd_rs(b, N, count)
                _rhd_ag(b, N, count)
            else:
                _rhd_ar_folded(b, N, count)
        else:
            if N >= 2:
                _dbt_ar(b, N, count)
    elif kind == "reducescatter":
        (_ring_rs if algo == "ring" else _rhd_rs)(b, N, count)
    elif kind == "allgather":
        (_ring_ag if algo == "ring" else _rhd_ag)(b, N, count)
    elif kind == "broadcast":
        if algo == "binomial":
            _bcast_binomial(b, N, count, root)
        elif algo == "chain_pipe":
            _bcast_chain_pipe(b, N, count, root, chunks)
        elif algo == "binomial_pipe":
            _bcast_binomial_pipe(b, N, count, root, chunks)
        elif algo == "bidir_ring":
            _bcast_bidir_ring(b, N, count, root, chunks)
        else:
            # "一对多通信：Broadcast 与 Scatter", Broadcast 与 Scatter 的关系: Scatter
            # then AllGather; the chunks stay at their offsets, so after the
            # binomial Scatter rank i holds chunk i, which the Ring AllGather needs
            _scatter_binomial(b, N, count, root)
            _ring_ag(b, N, count)
    elif kind == "scatter":
        (_scatter_binomial if algo == "binomial" else _scatter_linear)(b, N, count, root)
    elif kind == "reduce":
        _reduce_binomial(b, N, count, root)
    elif kind == "gather":
        _gather_binomial(b, N, count, root)
    else:
        {"pairwise": _a2a_pairwise, "bruck": _a2a_bruck, "ring": _a2a_ring}[algo](b, N, count)
    return p


def counts(plan: Plan, itemsize: int) -> dict:
    """Step count, row count, critical-path bytes and schedule memory bytes.

    critical bytes: per counted step, the largest total carried by one
    (src, dst) edge, summed over steps (the beta term of the pages' model).
    hbm bytes: every row reads its source and writes its destination, a reduce
    row also reads the destination: 2n or 3n elements' bytes.
    """
    crit = 0
    hbm = 0
    for st, rows in enumerate(plan.steps):
        edges = {}
        for r in rows:
            edges[(r.src, r.dst)] = edges.get((r.src, r.dst), 0) + r.n
            hbm += (3 if r.reduce else 2) * r.n * itemsize
        if not plan.local[st] and edges:
            crit += max(edges.values()) * itemsize
    return {"steps": plan.nsteps, "rows": len(plan.rows), "crit_bytes": crit, "hbm_bytes": hbm}
