"""Pins of the oracle's schedules to what the pages fix (CPU only).

Each check compares the oracle with a fact that does not come from the oracle:
a table the pages print (tests/golden/), a closed-form step or byte count the
pages state, or an identity the pages state.
"""

import json
import math
import os

import pytest

from oracle.schedules import Plan, ceil_log2, counts, dbt_trees, make_plan
from oracle.simulate import check_hazards

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NS = list(range(1, 17)) + [32, 64]
POW2 = [1, 2, 4, 8, 16, 32, 64]


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def edges(step_rows):
    return sorted({(r.src, r.dst) for r in step_rows})


# --- printed worked examples -------------------------------------------------

def test_binomial_broadcast_matches_printed_8_node_table():
    g = golden("binomial_bcast_n8.json")
    count = 8 * 1024
    p = make_plan("broadcast", "binomial", g["nranks"], count, g["root"])
    assert p.nsteps == len(g["steps"])
    holders = {g["root"]}
    for st, (rows, want, nh) in enumerate(zip(p.steps, g["steps"], g["holders_after_step"])):
        assert edges(rows) == sorted(tuple(e) for e in want), st
        for r in rows:
            assert r.src in holders and r.n == count          # only holders send, all M
        holders |= {r.dst for r in rows}
        assert len(holders) == nh


def test_binomial_scatter_matches_printed_8_node_table():
    g = golden("binomial_scatter_n8.json")
    N, count = g["nranks"], 8 * 64
    p = make_plan("scatter", "binomial", N, count, g["root"])
    assert p.nsteps == len(g["steps"])
    total = 0.0
    for rows, want, frac in zip(p.steps, g["steps"], g["bytes_per_edge_fraction_of_M"]):
        got = {}
        for r in rows:
            assert r.src_off == r.dst_off                     # chunks stay in place
            assert r.src_off % (count // N) == 0 and r.n % (count // N) == 0
            chunks = list(range(r.src_off // (count // N), (r.src_off + r.n) // (count // N)))
            got.setdefault((r.src, r.dst), []).extend(chunks)
        assert {k: sorted(v) for k, v in got.items()} == {(a, b): c for a, b, c in want}
        for e, ch in got.items():
            assert len(ch) * (count // N) == pytest.approx(frac * count)
        total += frac
    assert total == pytest.approx(g["bandwidth_sum_fraction_of_M"])
    assert total == pytest.approx(1 - 1 / N)                  # eq:onetoall-scatter-binomial-bw-sum


@pytest.mark.parametrize("N", NS)
@pytest.mark.parametrize("root", [0, 1, 5])
def test_gather_is_scatter_reversed(N, root):
    """eq:onetoall-gather-scatter-duality: reverse the data flow of Scatter."""
    if root >= N:
        pytest.skip("root outside the ranks")
    count = 3 * N + 2
    sc = make_plan("scatter", "binomial", N, count, root)
    ga = make_plan("gather", "binomial", N, count, root)
    assert sc.nsteps == ga.nsteps
    for s_rows, g_rows in zip(sc.steps, reversed(ga.steps)):
        fwd = sorted((r.src, r.dst, r.src_off, r.n) for r in s_rows)
        rev = sorted((r.dst, r.src, r.src_off, r.n) for r in g_rows)
        assert fwd == rev


# --- closed-form step counts --------------------------------------------------

def closed_form_steps(kind, algo, N, k=1):
    L = math.ceil(math.log2(N)) if N > 1 else 0
    table = {
        ("allreduce", "ring"): 2 * (N - 1),
        ("reducescatter", "ring"): N - 1,
        ("allgather", "ring"): N - 1,
        ("allreduce", "rhd"): 2 * L,
        ("reducescatter", "rhd"): L,
        ("allgather", "rhd"): L,
        ("allreduce", "dbt"): 2 * L,
        ("broadcast", "binomial"): L,
        ("broadcast", "chain_pipe"): (N + k - 2) if N > 1 else 0,
        ("broadcast", "binomial_pipe"): (L + k - 1) if N > 1 else 0,
        ("scatter", "binomial"): L,
        ("gather", "binomial"): L,
        ("alltoall", "pairwise"): N - 1,
        ("alltoall", "bruck"): L,
    }
    return table[(kind, algo)]


@pytest.mark.parametrize("N", NS)
def test_step_counts_equal_closed_forms(N):
    count = 4 * N * 64
    pow2 = (N & (N - 1)) == 0
    cases = [("allreduce", "ring"), ("reducescatter", "ring"), ("allgather", "ring"),
             ("broadcast", "binomial"), ("scatter", "binomial"), ("gather", "binomial"),
             ("alltoall", "pairwise"), ("alltoall", "bruck")]
    if pow2:
        cases += [("allreduce", "rhd"), ("reducescatter", "rhd"), ("allgather", "rhd"),
                  ("allreduce", "dbt")]
    for kind, algo in cases:
        p = make_plan(kind, algo, N, count)
        assert p.nsteps == closed_form_steps(kind, algo, N), (kind, algo)
    for k in (1, 2, 8, 64):
        for algo in ("chain_pipe", "binomial_pipe"):
            p = make_plan("broadcast", algo, N, count, 0, k)
            assert p.nsteps == closed_form_steps("broadcast", algo, N, k), (algo, k)


# --- closed-form critical-path bytes ------------------------------------------

@pytest.mark.parametrize("N", NS)
def test_critical_bytes_equal_closed_forms(N):
    sz = 4
    count = N * 64 * 8             # divisible by N and by every k below
    M = count * sz
    L = ceil_log2(N)

    def crit(kind, algo, k=1):
        return counts(make_plan(kind, algo, N, count, 0, k), sz)["crit_bytes"]

    assert crit("reducescatter", "ring") == (N - 1) * M // N          # eq:model-algo-ring-reducescatter
    assert crit("allgather", "ring") == (N - 1) * M // N              # eq:model-algo-ring-allgather
    assert crit("allreduce", "ring") == 2 * (N - 1) * M // N          # eq:model-algo-ring-ar
    assert crit("alltoall", "pairwise") == (N - 1) * M // N           # eq:model-algo-a2a-pairwise
    assert crit("scatter", "binomial") == (N - 1) * M // N             # eq:binomial-scatter
    assert crit("broadcast", "binomial") == L * M                      # eq:binomial-bcast
    for k in (1, 2, 8, 64):
        if N > 1:
            assert crit("broadcast", "chain_pipe", k) == (N + k - 2) * M // k     # eq:pipe-chain-bcast
            assert crit("broadcast", "binomial_pipe", k) == (L + k - 1) * M // k  # eq:pipe-tree-bcast
    if (N & (N - 1)) == 0:
        assert crit("allreduce", "rhd") == 2 * (N - 1) * M // N        # eq:model-algo-rhd-ar
        assert crit("reducescatter", "rhd") == (N - 1) * M // N        # eq:model-algo-rhd-rs
        assert crit("allgather", "rhd") == (N - 1) * M // N            # eq:model-algo-rhd-ag
        assert crit("gather", "binomial") == (N - 1) * M // N          # eq:onetoall-gather-scatter-duality
        if N > 1:
            assert crit("allreduce", "dbt") == L * M                   # eq:model-algo-dbt-ar


@pytest.mark.parametrize("N", [2, 4, 8, 16, 32, 64])
def test_rhd_round_bytes(N):
    """Halving round k moves M/2^(k+1); doubling round k moves 2^k * M/N."""
    sz, count = 2, N * 128
    M = count * sz
    rs = make_plan("reducescatter", "rhd", N, count)
    for k, rows in enumerate(rs.steps):
        assert {r.n * sz for r in rows} == {M >> (k + 1)}
        assert {abs(r.src - r.dst) for r in rows} == {N >> (k + 1)}
    ag = make_plan("allgather", "rhd", N, count)
    for k, rows in enumerate(ag.steps):
        assert {r.n * sz for r in rows} == {(1 << k) * M // N}
        assert {abs(r.src - r.dst) for r in rows} == {1 << k}


@pytest.mark.parametrize("N", [2, 4, 8, 16, 32])
def test_bruck_round_bytes_are_popcount_sums(N):
    """Round k packs every block index j with bit k set and sends it 2^k ranks
    on; per-edge bytes are |{j : bit k of j}| * M/N."""
    sz, count = 2, N * 16
    B = count // N
    p = make_plan("alltoall", "bruck", N, count)
    rounds = [rows for rows, loc in zip(p.steps, p.local) if not loc]
    assert len(rounds) == ceil_log2(N)
    for k, rows in enumerate(rounds):
        per_edge = {}
        for r in rows:
            assert (r.dst - r.src) % N == (1 << k) % N
            per_edge[(r.src, r.dst)] = per_edge.get((r.src, r.dst), 0) + r.n
        want = sum(1 for j in range(N) if (j >> k) & 1) * B
        assert set(per_edge.values()) == {want}
    total = counts(p, sz)["crit_bytes"]
    assert total == sum(bin(j).count("1") for j in range(N)) * B * sz


# --- identities ---------------------------------------------------------------

@pytest.mark.parametrize("N", [1, 2, 3, 5, 8, 13, 16])
def test_ring_allreduce_is_reducescatter_then_allgather(N):
    """T_Ring-AR = T_Ring-RS + T_Ring-AG: the rows of AllReduce are the rows of
    ReduceScatter followed by the rows of AllGather."""
    count = 7 * N + 3
    ar = make_plan("allreduce", "ring", N, count)
    rs = make_plan("reducescatter", "ring", N, count)
    ag = make_plan("allgather", "ring", N, count)
    strip = lambda rows: [(r.src, r.dst, r.src_off, r.dst_off, r.n, r.reduce) for r in rows]
    assert [strip(s) for s in ar.steps] == [strip(s) for s in rs.steps + ag.steps]
    for sz in (1, 2, 4):
        a, b, c = counts(ar, sz), counts(rs, sz), counts(ag, sz)
        assert a["steps"] == b["steps"] + c["steps"]
        assert a["crit_bytes"] == b["crit_bytes"] + c["crit_bytes"]
        assert a["hbm_bytes"] == b["hbm_bytes"] + c["hbm_bytes"]


@pytest.mark.parametrize("N", [1, 2, 4, 8, 16])
def test_rhd_allreduce_is_halving_then_doubling(N):
    count = 5 * N
    ar = make_plan("allreduce", "rhd", N, count)
    rs = make_plan("reducescatter", "rhd", N, count)
    ag = make_plan("allgather", "rhd", N, count)
    strip = lambda rows: [(r.src, r.dst, r.src_off, r.n, r.reduce) for r in rows]
    assert [strip(s) for s in ar.steps] == [strip(s) for s in rs.steps + ag.steps]


@pytest.mark.parametrize("N", [2, 3, 5, 8, 11])
def test_pipelines_with_one_chunk_are_chain_and_binomial(N):
    """k = 1 reproduces eq:chain-bcast (N-1 hops of M) and eq:binomial-bcast."""
    count = 40
    chain = make_plan("broadcast", "chain_pipe", N, count, 0, 1)
    assert [edges(s) for s in chain.steps] == [[(h, h + 1)] for h in range(N - 1)]
    assert all(r.n == count for r in chain.rows)
    bp = make_plan("broadcast", "binomial_pipe", N, count, 0, 1)
    bi = make_plan("broadcast", "binomial", N, count, 0)
    assert [edges(s) for s in bp.steps] == [edges(s) for s in bi.steps]


# --- the double binary tree construction ----------------------------------------

@pytest.mark.parametrize("N", [2, 4, 8, 16, 32, 64])
def test_dbt_trees_are_complementary_binary_trees_of_height_log2n(N):
    """Two binary trees over all ranks, height log2 N each, and every rank is a
    leaf in exactly one of them (the property that lets both halves move at once)."""
    H = ceil_log2(N)
    leaves = []
    for root, t in dbt_trees(N):
        nodes = set(t)
        assert nodes == set(range(N))
        kids = [c for cs in t.values() for c in cs]
        assert sorted(kids + [root]) == list(range(N))        # a tree: every non-root has one parent
        assert all(len(cs) <= 2 for u, cs in t.items() if u != root)

        def height(u):
            return 0 if not t[u] else 1 + max(height(c) for c in t[u])
        assert height(root) == H
        leaves.append({u for u, cs in t.items() if not cs})
    if N > 2:
        assert leaves[0].isdisjoint(leaves[1])
        assert leaves[0] | leaves[1] == set(range(N))


def test_dbt_trees_n8_shape():
    (r1, t1), (r2, t2) = dbt_trees(8)
    assert r1 == 0 and {u: c for u, c in t1.items() if c} == {0: [4], 4: [2, 6], 2: [1, 3], 6: [5, 7]}
    assert r2 == 1 and {u: c for u, c in t2.items() if c} == {1: [5], 5: [3, 7], 3: [2, 4], 7: [6, 0]}


# --- every plan is hazard free; the hazard check catches planted conflicts -------

@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 7, 8, 9, 16, 32])
def test_all_plans_are_hazard_free(N):
    count = 6 * N + 5
    pow2 = (N & (N - 1)) == 0
    for kind, algos in [("allreduce", ["ring"] + (["rhd", "dbt"] if pow2 else [])),
                        ("reducescatter", ["ring"] + (["rhd"] if pow2 else [])),
                        ("allgather", ["ring"] + (["rhd"] if pow2 else [])),
                        ("scatter", ["binomial"]), ("gather", ["binomial"])]:
        for algo in algos:
            for root in {0, N - 1}:
                check_hazards(make_plan(kind, algo, N, count, root))
    for algo in ("binomial", "chain_pipe", "binomial_pipe"):
        for k in (1, 3, 8):
            check_hazards(make_plan("broadcast", algo, N, count, N // 2, k))
    for algo in ("pairwise", "bruck"):
        check_hazards(make_plan("alltoall", algo, N, N * 3))


def test_hazard_checker_rejects_planted_conflicts():
    p = make_plan("allreduce", "ring", 4, 64)
    # move a row of step 1 so that it writes what another row of the step reads
    bad = Plan(p.kind, p.algo, p.nranks, p.count, steps=[list(s) for s in p.steps],
               local=list(p.local), staged=list(p.staged))
    r0, r1 = bad.steps[1][0], bad.steps[1][1]
    from dataclasses import replace
    bad.steps[1][1] = replace(r1, dst=r0.src, dst_off=r0.src_off, reduce=False)
    with pytest.raises(AssertionError):
        check_hazards(bad)


# --- Tree Reduce, linear Scatter, Broadcast as Scatter + AllGather ---------------

@pytest.mark.parametrize("N", NS)
def test_reduce_and_linear_scatter_counts(N):
    """Tree Reduce: log2 N steps of the whole message (eq:model-algo-reduce-tree);
    naive Scatter: N-1 steps, (N-1)M/N bytes (eq:onetoall-scatter-naive);
    Scatter + AllGather Broadcast: ceil(log2 N) + N-1 steps, 2(N-1)M/N bytes."""
    sz, count = 4, N * 64 * 8
    M, L = count * sz, ceil_log2(N)
    for root in {0, N - 1}:
        red = make_plan("reduce", "binomial", N, count, root)
        assert red.nsteps == L
        assert counts(red, sz)["crit_bytes"] == L * M
        assert all(r.n == count and r.reduce for r in red.rows)
        lin = make_plan("scatter", "linear", N, count, root)
        assert lin.nsteps == N - 1
        assert counts(lin, sz)["crit_bytes"] == (N - 1) * M // N
        assert all(r.src == root for r in lin.rows)
        sag = make_plan("broadcast", "scatter_allgather", N, count, root)
        assert sag.nsteps == L + N - 1
        assert counts(sag, sz)["crit_bytes"] == 2 * (N - 1) * M // N


@pytest.mark.parametrize("N", NS)
@pytest.mark.parametrize("root", [0, 3])
def test_reduce_is_binomial_broadcast_reversed(N, root):
    """Tree Reduce is the tree Broadcast run backwards ("集合通信算法延迟公式", Tree Reduce)."""
    if root >= N:
        pytest.skip("root outside the ranks")
    bc = make_plan("broadcast", "binomial", N, 10, root)
    red = make_plan("reduce", "binomial", N, 10, root)
    for b_rows, r_rows in zip(bc.steps, reversed(red.steps)):
        assert sorted((r.src, r.dst) for r in b_rows) == sorted((r.dst, r.src) for r in r_rows)


# --- non-power-of-two N: folded halving-doubling, general double binary tree -----

@pytest.mark.parametrize("N", [3, 5, 6, 7, 9, 12, 13, 31, 33])
def test_folded_rhd_and_general_dbt_counts(N):
    """RHD with N != 2^n: the r = N - P surplus ranks fold into a P = 2^floor(log2 N)
    core, the core runs 2 log2 P halving / doubling rounds, the result is copied
    back: 2 log2 P + 2 steps; bytes M + 2(P-1)M/P + M.  DBT: 2 ceil(log2 N) steps."""
    P = 1 << (N.bit_length() - 1)
    lP = P.bit_length() - 1
    sz, count = 4, 64 * P * N
    M = count * sz
    rhd = make_plan("allreduce", "rhd", N, count)
    assert rhd.nsteps == 2 * lP + 2
    assert counts(rhd, sz)["crit_bytes"] == M + 2 * (P - 1) * M // P + M
    assert {(r.src, r.dst) for r in rhd.steps[0]} == {(2 * i, 2 * i + 1) for i in range(N - P)}
    assert {(r.src, r.dst) for r in rhd.steps[-1]} == {(2 * i + 1, 2 * i) for i in range(N - P)}
    dbt = make_plan("allreduce", "dbt", N, count)
    assert dbt.nsteps == 2 * ceil_log2(N)
    for root, t in dbt_trees(N):
        kids = [c for cs in t.values() for c in cs]
        assert sorted(kids + [root]) == list(range(N))
        assert all(len(cs) <= 2 for u, cs in t.items() if u != root)

        def height(u):
            return 0 if not t[u] else 1 + max(height(c) for c in t[u])
        assert height(root) == ceil_log2(N)


# --- bidirectional-ring Broadcast ---------------------------------------------------

def test_bidir_ring_broadcast_matches_printed_4_chip_example():
    g = golden("bidir_ring_bcast_n4.json")
    p = make_plan("broadcast", "bidir_ring", g["nranks"], 4096, g["root"], 1)
    assert p.nsteps == len(g["steps"]) == ceil_log2(g["nranks"])
    for rows, want in zip(p.steps, g["steps"]):
        assert edges(rows) == sorted(tuple(e) for e in want)
        assert all(r.n == 4096 for r in rows)


@pytest.mark.parametrize("N", NS)
@pytest.mark.parametrize("k", [1, 2, 5])
def test_bidir_ring_broadcast_counts_and_neighbour_edges(N, k):
    """Both directions of the ring carry the message at once, so the farther half
    is ceil((N-1)/2) hops away: ceil((N-1)/2) + k - 1 steps of M/k bytes with k
    chunks; every edge joins ring neighbours; every rank but the root receives
    every chunk exactly once, from a rank that already holds it."""
    sz, count = 4, 64 * k * max(N, 1)
    M = count * sz
    for root in {0, N - 1}:
        p = make_plan("broadcast", "bidir_ring", N, count, root, k)
        H = (N - 1 + 1) // 2
        assert p.nsteps == (H + k - 1 if N > 1 else 0)
        assert counts(p, sz)["crit_bytes"] == p.nsteps * M // k
        holds = {(root, c) for c in range(k)}
        got = {}
        for rows in p.steps:
            new = set()
            for r in rows:
                assert (r.dst - r.src) % N in (1, N - 1)
                c = r.src_off * k // count
                assert (r.src, c) in holds and r.src_off == r.dst_off and r.n == count // k
                got[(r.dst, c)] = got.get((r.dst, c), 0) + 1
                new.add((r.dst, c))
            holds |= new
        assert got == {(d, c): 1 for d in range(N) if d != root for c in range(k)}
        check_hazards(p)



# --- Ring AllToAll (store-and-forward between neighbours) -----------------------------

@pytest.mark.parametrize("N", NS)
def test_ring_alltoall_rounds_hops_and_bytes(N):
    """N-1 rounds, the latency term of eq:model-algo-a2a-ring; every round only
    between ring neighbours i -> i+1.  Round t forwards the N-t blocks that are
    still travelling, so the rows carry exactly sum_d d = N(N-1)/2 blocks per
    rank in total: every block crosses the d links to its destination once and
    takes no detour.  Per link that is (N-1)M/2 bytes, not the (N-1)M/N the
    printed formula gives (no neighbour-only schedule can do better)."""
    sz, B = 4, 24
    count = N * B
    M = count * sz
    p = make_plan("alltoall", "ring", N, count)
    assert p.nsteps == N - 1
    rounds = [rows for rows, loc in zip(p.steps, p.local) if not loc]
    assert len(rounds) == N - 1
    hops = 0
    for t, rows in enumerate(rounds, start=1):
        per_edge = {}
        for r in rows:
            assert (r.dst - r.src) % N == 1 % N and r.src_off == r.dst_off
            per_edge[(r.src, r.dst)] = per_edge.get((r.src, r.dst), 0) + r.n
            hops += r.n
        assert per_edge == {(i, (i + 1) % N): (N - t) * B for i in range(N)}
    assert hops == N * (N * (N - 1) // 2) * B
    assert counts(p, sz)["crit_bytes"] == (N - 1) * M // 2
