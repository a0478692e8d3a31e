"""Pins of three oracle functions the full-size GPU checks rest on (CPU only).

* ``run_plan_columns`` (the plan restricted to sampled columns, used for every
  full-size parity check): against ``run_plan`` on the whole buffers, over
  random plans of every collective but AllToAll, every algorithm, ragged
  counts, roots and chunk counts, every dtype and op, on column sets that
  contain every row boundary; every element compared, defined or not.
* ``defined_regions`` (which elements a parity check compares): against the
  buffer contract of the collective calls written out per element with its
  own chunk arithmetic, and against the definitions ("一对多通信：Broadcast 与
  Scatter", Scatter 语义定义 and Broadcast 语义定义; "集合通信算法延迟公式",
  Ring ReduceScatter / AllGather): on random integer inputs every defined
  element holds the value the definition gives, for every algorithm.
* the uint8 branch of ``numerics.combine``: every pair of bytes against
  integer arithmetic (sum modulo 2^8, max, min).

Each pin is shown to fail on a planted mistake: ``searchsorted`` with its side
flipped, an empty region list, a shifted region, bytes compared as int8.
"""

import numpy as np
import pytest

import oracle.simulate as sim
from oracle import numerics
from oracle.schedules import VALID, make_plan
from oracle.simulate import defined_regions, run_plan, run_plan_columns

KINDS = [k for k in VALID if k != "alltoall"]
PIPELINED = ("chain_pipe", "binomial_pipe", "bidir_ring")


def random_values(g, n, dtype):
    if dtype == "int32":
        return g.integers(-(1 << 31), (1 << 31) - 1, n, dtype=np.int64).astype(np.int32)
    if dtype == "uint8":
        return g.integers(0, 256, n).astype(np.uint8)
    if dtype == "float32":
        return g.standard_normal(n).astype(np.float32)
    return numerics.f32_to_bf16_rne(g.standard_normal(n).astype(np.float32))


def draw_case(i):
    g = np.random.default_rng(500 + i)
    kind = KINDS[i % len(KINDS)]
    algo = VALID[kind][(i // len(KINDS)) % len(VALID[kind])]
    if algo == "rhd" and kind in ("reducescatter", "allgather"):
        N = int(2 ** g.integers(0, 5))
    else:
        N = int(g.integers(1, 14))
    count = int(g.integers(0, 9 * N + 40))
    root = int(g.integers(0, N))
    k = int(g.integers(1, max(1, min(count, 9)) + 1)) if algo in PIPELINED else 1
    dtype = ["int32", "uint8", "float32", "bfloat16"][i % 4]
    op = ["sum", "max", "min"][(i // 4) % 3] if kind in ("allreduce", "reducescatter", "reduce") else "sum"
    return g, kind, algo, N, count, root, k, dtype, op


def boundary_columns(plan, g, count):
    """Every row boundary (and its neighbours) plus a random sample."""
    c = set()
    for r in plan.rows:
        for b in (r.dst_off - 1, r.dst_off, r.dst_off + r.n - 1, r.dst_off + r.n):
            if 0 <= b < count:
                c.add(b)
    if count:
        c.update(int(x) for x in g.integers(0, count, min(count, 7)))
    return np.array(sorted(c), dtype=np.int64)


def columns_agree(run_columns, cases=range(240)):
    """True when ``run_columns`` equals run_plan restricted to the columns, on
    every element of every rank, for all the cases."""
    for i in cases:
        g, kind, algo, N, count, root, k, dtype, op = draw_case(i)
        plan = make_plan(kind, algo, N, count, root, k)
        a = [random_values(g, count, dtype) for _ in range(N)]
        full = run_plan(plan, dtype, op, a)
        cols = boundary_columns(plan, g, count)
        got = run_columns(plan, dtype, op, cols, [x[cols] for x in a])
        for r in range(N):
            if not np.array_equal(got[r].view(np.uint8), full[r][cols].view(np.uint8)):
                return False
    return True


def test_run_plan_columns_equals_run_plan_on_whole_buffers():
    assert columns_agree(run_plan_columns)


class _FlippedSearchsorted:
    """numpy with searchsorted's side flipped: a plausible slip in the column
    restriction (a column exactly at a row's start would fall out of it)."""

    def __getattr__(self, name):
        return getattr(np, name)

    @staticmethod
    def searchsorted(a, v, side="left", sorter=None):
        return np.searchsorted(a, v, side="right" if side == "left" else "left", sorter=sorter)


def test_planted_searchsorted_slip_is_caught(monkeypatch):
    monkeypatch.setattr(sim, "np", _FlippedSearchsorted())
    assert not columns_agree(sim.run_plan_columns, cases=range(60))


# --- defined regions ------------------------------------------------------------------

def chunk_of(x, count, N):
    """The chunk holding element x under the floor partition, found by a scan
    (chunk c starts at floor(c * count / N))."""
    c = 0
    while c + 1 < N and (c + 1) * count // N <= x:
        c += 1
    return c


def contract_defined(kind, N, count, root, rank, x):
    """The collective calls' buffer contract, element by element."""
    if kind in ("allreduce", "allgather", "broadcast", "alltoall"):
        return True
    if kind in ("reducescatter", "scatter"):
        return chunk_of(x, count, N) == rank
    if kind in ("gather", "reduce"):
        return rank == root
    raise ValueError(kind)


def region_mask(regions, count):
    m = np.zeros(count, dtype=bool)
    for lo, hi in regions:
        m[lo:hi] = True
    return m


def regions_match_contract(regions_fn):
    for kind in list(VALID):
        for N in range(1, 11):
            for count in sorted({0, 1, N - 1, N, 2 * N + 1, 5 * N + 3, 37}):
                if count < 0:
                    continue
                for root in sorted({0, N // 2, N - 1}):
                    regs = regions_fn(kind, N, count, root)
                    if len(regs) != N:
                        return False
                    for i in range(N):
                        want = np.array([contract_defined(kind, N, count, root, i, x) for x in range(count)],
                                        dtype=bool)
                        if not np.array_equal(region_mask(regs[i], count), want):
                            return False
    return True


def test_defined_regions_match_the_contract():
    assert regions_match_contract(defined_regions)


def definition_holds(regions_fn, trials=3):
    """On random int32 inputs, every element the regions call defined holds what
    the collective's definition gives, for every algorithm of the collective,
    and every rank the contract gives output has a non-empty region."""
    for kind in KINDS:
        for algo in VALID[kind]:
            for N in (1, 2, 3, 4, 5, 8):
                if algo == "rhd" and kind in ("reducescatter", "allgather") and N & (N - 1):
                    continue
                count, root = 4 * N + 3, N - 1
                regs = regions_fn(kind, N, count, root)
                for i in range(N):
                    if any(contract_defined(kind, N, count, root, i, x) for x in range(count)) and \
                            not region_mask(regs[i], count).any():
                        return False
                for t in range(trials):
                    g = np.random.default_rng(1000 * N + t)
                    a = [g.integers(-(1 << 20), 1 << 20, count).astype(np.int32) for _ in range(N)]
                    out = run_plan(make_plan(kind, algo, N, count, root, 3 if algo in PIPELINED else 1),
                                   "int32", "sum", a)
                    total = np.sum(np.stack(a).astype(np.int64), axis=0).astype(np.int32)
                    for i in range(N):
                        for x in np.nonzero(region_mask(regs[i], count))[0]:
                            c = chunk_of(x, count, N)
                            want = {"allreduce": total[x], "reducescatter": total[x], "reduce": total[x],
                                    "broadcast": a[root][x], "scatter": a[root][x],
                                    "allgather": a[c][x], "gather": a[c][x]}[kind]
                            if out[i][x] != want:
                                return False
    return True


def test_defined_elements_hold_the_definitions():
    assert definition_holds(defined_regions)


def test_planted_region_mistakes_are_caught():
    def empty(kind, N, count, root=0):
        return [[] for _ in range(N)]

    def shifted(kind, N, count, root=0):
        return [[(lo + 1, hi + 1) if hi < count else (lo, hi) for lo, hi in regs]
                for regs in defined_regions(kind, N, count, root)]

    def root_everywhere(kind, N, count, root=0):
        regs = defined_regions(kind, N, count, root)
        return [[(0, count)] if kind in ("gather", "reduce") else r for r in regs]

    for bad in (empty, shifted, root_everywhere):
        assert not regions_match_contract(bad)
    assert not definition_holds(empty)
    assert not definition_holds(root_everywhere)


# --- uint8 element rule ------------------------------------------------------------------

def uint8_rule_holds(combine):
    a = np.repeat(np.arange(256, dtype=np.uint8), 256)
    b = np.tile(np.arange(256, dtype=np.uint8), 256)
    ai, bi = a.astype(int), b.astype(int)
    want = {"sum": (ai + bi) % 256, "max": np.maximum(ai, bi), "min": np.minimum(ai, bi)}
    for op in ("sum", "max", "min"):
        got = combine(a.copy(), b.copy(), "uint8", op)
        if got.dtype != np.uint8 or not np.array_equal(got.astype(int), want[op]):
            return False
    return True


def test_uint8_combine_every_pair():
    assert uint8_rule_holds(numerics.combine)


def test_planted_uint8_slips_are_caught():
    def as_int8(d, s, dtype, op):
        r = numerics.combine(d.view(np.int8), s.view(np.int8), "int32", op)
        return r.view(np.uint8)

    def no_wrap(d, s, dtype, op):
        if op == "sum":
            return np.minimum(d.astype(int) + s.astype(int), 255).astype(np.uint8)
        return numerics.combine(d, s, dtype, op)

    def swapped(d, s, dtype, op):
        return numerics.combine(d, s, dtype, {"max": "min", "min": "max"}.get(op, op))

    for bad in (as_int8, no_wrap, swapped):
        assert not uint8_rule_holds(bad)


@pytest.mark.parametrize("N", [2, 5, 8])
def test_uint8_reductions_against_brute_force(N):
    """Whole collectives on uint8 data: the elementwise wrap-around sum, max
    and min over ranks, computed with Python integers."""
    g = np.random.default_rng(N)
    count = 7 * N + 5
    a = [g.integers(0, 256, count).astype(np.uint8) for _ in range(N)]
    ints = np.stack(a).astype(int)
    for op, want in (("sum", ints.sum(axis=0) % 256), ("max", ints.max(axis=0)), ("min", ints.min(axis=0))):
        for algo in VALID["allreduce"]:
            out = run_plan(make_plan("allreduce", algo, N, count), "uint8", op, a)
            for i in range(N):
                assert np.array_equal(out[i].astype(int), want), (op, algo, i)
