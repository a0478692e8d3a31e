"""Property-based checks over random calls (CPU only; hypothesis).

For a random (collective, algorithm, N, count, root, k):
  * the oracle's schedule is hazard-free;
  * the C++ generator behind coll_plan gives the oracle's rows and counts;
  * the oracle's result equals the collective's definition on random int32
    data (sum and max reductions) or uint8 data (copies), written out here
    directly from the definitions.
"""

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle.schedules import VALID, make_plan
from oracle.simulate import check_hazards, defined_regions, run_plan
from tests.test_plan_cpp import compare

PIPELINED = ("chain_pipe", "binomial_pipe", "bidir_ring")
SETTINGS = settings(max_examples=1000, deadline=None, suppress_health_check=[HealthCheck.too_slow],
                    derandomize=True)


@st.composite
def calls(draw):
    kind = draw(st.sampled_from(sorted(VALID)))
    algo = draw(st.sampled_from(VALID[kind]))
    if algo == "rhd" and kind != "allreduce":
        N = 2 ** draw(st.integers(0, 5))
    else:
        N = draw(st.integers(1, 24))
    count = N * draw(st.integers(0, 12)) if kind == "alltoall" else draw(st.integers(0, 400))
    root = draw(st.integers(0, N - 1))
    k = draw(st.integers(1, max(1, min(count, 16)))) if algo in PIPELINED else 1
    return kind, algo, N, count, root, k


def part(count, N, i):
    return i * count // N


def definition(kind, a, root, op):
    """The collective's result from its definition (None where undefined)."""
    N, count = len(a), len(a[0])
    stack = np.stack(a).astype(np.int64)
    if kind in ("allreduce", "reducescatter", "reduce"):
        red = stack.sum(axis=0) if op == "sum" else stack.max(axis=0)
        red = ((red + 2 ** 31) % 2 ** 32 - 2 ** 31).astype(np.int32)
        return [red.copy() for _ in range(N)]
    if kind == "allgather":
        full = np.concatenate([a[i][part(count, N, i):part(count, N, i + 1)] for i in range(N)])
        return [full.copy() for _ in range(N)]
    if kind == "broadcast":
        return [a[root].copy() for _ in range(N)]
    if kind == "scatter":
        return [a[root].copy() for _ in range(N)]          # chunk i of rank i is compared
    if kind == "gather":
        full = np.concatenate([a[i][part(count, N, i):part(count, N, i + 1)] for i in range(N)])
        return [full.copy() for _ in range(N)]             # the root is compared
    if kind == "alltoall":
        B = count // N
        return [np.concatenate([a[i][j * B:(j + 1) * B] for i in range(N)]) for j in range(N)]
    raise ValueError(kind)


@SETTINGS
@given(calls())
def test_plan_is_hazard_free_and_cpp_agrees(call):
    kind, algo, N, count, root, k = call
    check_hazards(make_plan(kind, algo, N, count, root, k))
    compare(kind, algo, N, count, root, k, dtype="int32")


@SETTINGS
@given(calls(), st.integers(0, 2 ** 32 - 1), st.sampled_from(["sum", "max"]))
def test_oracle_equals_definition(call, seed, op):
    kind, algo, N, count, root, k = call
    g = np.random.default_rng(seed)
    reduces = kind in ("allreduce", "reducescatter", "reduce")
    a = [g.integers(-(2 ** 31), 2 ** 31, count, dtype=np.int64).astype(np.int32) for _ in range(N)]
    plan = make_plan(kind, algo, N, count, root, k)
    got = run_plan(plan, "int32", op if reduces else "sum", a)
    want = definition(kind, a, root, op)
    for i, regs in enumerate(defined_regions(kind, N, count, root)):
        for lo, hi in regs:
            assert np.array_equal(got[i][lo:hi], want[i][lo:hi]), (kind, algo, N, count, root, k, i)
