"""Pins of the oracle's results to the collectives' definitions (CPU only).

Integer and copy results are compared with the semantic definitions computed
directly (a sum over ranks with wrap-around, a copy of the root, a transpose of
blocks).  Float results are compared bit for bit with the association order
written out in closed form (a fold along the ring, a butterfly, a fold over
each tree), and against fp64 within a proven error bound.  bf16 rounding is
compared with torch's own conversion.  Planted mistakes in a plan must be caught.
"""

from dataclasses import replace

import numpy as np
import pytest

import oracle
from oracle import numerics
from oracle.schedules import Plan, dbt_trees, make_plan, part
from oracle.simulate import run_plan

NS_SMALL = list(range(1, 13)) + [16, 32]


def rng_ints(N, count, seed, lo=-(1 << 20), hi=1 << 20):
    g = np.random.default_rng(seed)
    return [g.integers(lo, hi, count, endpoint=True, dtype=np.int32) for _ in range(N)]


def wrap_sum(arrs):
    s = np.zeros(len(arrs[0]), dtype=np.int64)
    for a in arrs:
        s = s + a.astype(np.int64)
    return (((s + (1 << 31)) % (1 << 32)) - (1 << 31)).astype(np.int32)


def chunk(count, N, i):
    return slice(part(count, N, i), part(count, N, i + 1))


def counts_for(N):
    return sorted({0, 1, max(N - 1, 0), N, 3 * N + 1, 257})


# --- integer semantics, brute force -----------------------------------------------

@pytest.mark.parametrize("N", NS_SMALL)
def test_allreduce_reducescatter_allgather_int32(N):
    pow2 = (N & (N - 1)) == 0
    for count in counts_for(N):
        # values near the int32 limits make the sums wrap
        a = rng_ints(N, count, 10 * N + count, lo=-(1 << 31), hi=(1 << 31) - 1)
        want = wrap_sum(a) if count else np.zeros(0, np.int32)
        for algo in ["ring"] + (["rhd", "dbt"] if pow2 else []):
            for o in oracle.allreduce(a, "int32", algo=algo):
                assert np.array_equal(o, want), (algo, count)
        for algo in ["ring"] + (["rhd"] if pow2 else []):
            rs = oracle.reducescatter(a, "int32", algo=algo)
            for i in range(N):
                assert np.array_equal(rs[i][chunk(count, N, i)], want[chunk(count, N, i)])
            full = np.concatenate([a[i][chunk(count, N, i)] for i in range(N)])
            for o in oracle.allgather(a, "int32", algo=algo):
                assert np.array_equal(o, full), (algo, count)


@pytest.mark.parametrize("op,fn", [("max", np.max), ("min", np.min)])
@pytest.mark.parametrize("N", [2, 3, 4, 7, 8])
def test_allreduce_max_min_int32(N, op, fn):
    count = 5 * N + 3
    a = rng_ints(N, count, 99 + N)
    want = fn(np.stack(a), axis=0)
    algos = ["ring"] + (["rhd", "dbt"] if (N & (N - 1)) == 0 else [])
    for algo in algos:
        for o in oracle.allreduce(a, "int32", op=op, algo=algo):
            assert np.array_equal(o, want)


@pytest.mark.parametrize("N", NS_SMALL)
def test_broadcast_scatter_gather_uint8(N):
    g = np.random.default_rng(N)
    for count in counts_for(N):
        a = [g.integers(0, 256, count, dtype=np.uint8) for _ in range(N)]
        for root in sorted({0, N // 2, N - 1}):
            for algo, ks in (("binomial", [1]), ("chain_pipe", [1, 2, 7]),
                             ("binomial_pipe", [1, 3, 8]), ("bidir_ring", [1, 2, 7])):
                for k in ks:
                    if k > max(count, 1):
                        continue
                    for o in oracle.broadcast(a, "uint8", root, algo, k):
                        assert np.array_equal(o, a[root]), (algo, k, root, count)
            sc = oracle.scatter(a, "uint8", root)
            for i in range(N):
                assert np.array_equal(sc[i][chunk(count, N, i)], a[root][chunk(count, N, i)])
            ga = oracle.gather(a, "uint8", root)
            full = np.concatenate([a[i][chunk(count, N, i)] for i in range(N)])
            assert np.array_equal(ga[root], full)


@pytest.mark.parametrize("N", list(range(1, 20)) + [32])
def test_alltoall_is_block_transpose(N):
    B = 3
    count = N * B
    a = rng_ints(N, count, 7 * N)
    for algo in ("pairwise", "bruck", "ring"):
        out = oracle.alltoall(a, "int32", algo)
        for j in range(N):
            for i in range(N):
                assert np.array_equal(out[j][i * B:(i + 1) * B], a[i][j * B:(j + 1) * B]), (algo, i, j)


def test_copy_collectives_only_move_bytes():
    """Every output byte of a copy collective is some input byte (AllToAll is a
    permutation: each input block appears exactly once)."""
    N, B = 8, 4
    a = [np.full(N * B, 10 * i, dtype=np.int32) + np.repeat(np.arange(N, dtype=np.int32), B)
         for i in range(N)]
    out = oracle.alltoall(a, "int32", "bruck")
    blocks = sorted(tuple(o[i * B:(i + 1) * B]) for o in out for i in range(N))
    src = sorted(tuple(x[j * B:(j + 1) * B]) for x in a for j in range(N))
    assert blocks == src


# --- float association, written out in closed form ---------------------------------

def f32_rank(N, count, seed):
    g = np.random.default_rng(seed)
    return [g.standard_normal(count).astype(np.float32) for _ in range(N)]


def bf16_rank(N, count, seed, sigma=0.02):
    import torch
    out = []
    for x in f32_rank(N, count, seed):
        t = torch.from_numpy(x * np.float32(sigma)).to(torch.bfloat16)
        out.append(t.view(torch.int16).numpy().view(np.uint16).copy())
    return out


def add(dtype, x, y):
    """dst (+) src for one pair of whole arrays, written without the oracle:
    fp32 via numpy's binary32 add; bf16 via torch (widen, add in binary32, round)."""
    if dtype == "float32":
        return (x + y).astype(np.float32)
    import torch
    tx = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).float()
    ty = torch.from_numpy(y.view(np.int16).copy()).view(torch.bfloat16).float()
    return (tx + ty).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def ring_fold(a, dtype, N, count):
    """Chunk c leaves rank c+1 first and gains one rank per step along the ring:
    ((a_{c+1} + a_{c+2}) + ...) + a_c."""
    out = np.empty_like(a[0])
    for c in range(N):
        sl = chunk(count, N, c)
        acc = a[(c + 1) % N][sl]
        for m in range(2, N + 1):
            acc = add(dtype, a[(c + m) % N][sl], acc)
        out[sl] = acc
    return out


def butterfly(a, dtype, N):
    """Halving at distances N/2, N/4, ..., 1: v_k(r) = v_{k-1}(r) + v_{k-1}(r ^ d)."""
    v = list(a)
    d = N // 2
    while d >= 1:
        v = [add(dtype, v[r], v[r ^ d]) for r in range(N)]
        d //= 2
    count = len(a[0])
    out = np.empty_like(a[0])
    for c in range(N):
        out[chunk(count, N, c)] = v[c][chunk(count, N, c)]
    return out


def tree_fold(a, dtype, N):
    """Each node's value is its own folded with its children's subtree values in
    the order they arrive: by subtree height, then left before right (for
    N = 2^n siblings have equal height: ((own + left) + right)).  Tree 1 on
    the first half of the elements, tree 2 on the second."""
    count = len(a[0])
    out = np.empty_like(a[0])
    for (root, t), sl in zip(dbt_trees(N), (slice(0, count // 2), slice(count // 2, count))):
        def height(u):
            return 0 if not t[u] else 1 + max(height(c) for c in t[u])

        def fold(u):
            acc = a[u][sl]
            for _, _, c in sorted((height(c), i, c) for i, c in enumerate(t[u])):
                acc = add(dtype, acc, fold(c))
            return acc
        out[sl] = fold(root)
    return out


def folded_butterfly(a, dtype, N):
    """RHD for N != 2^n: v(2i+1) = a(2i+1) + a(2i) for i < r = N - P, the P core
    ranks then fold as a butterfly (distance P/2 first) on the P-way partition;
    every rank ends with the core's chunks."""
    P = 1 << (N.bit_length() - 1)
    r = N - P
    core = [2 * i + 1 for i in range(r)] + list(range(2 * r, N))
    v = [add(dtype, a[c], a[c - 1]) if k < r else a[c] for k, c in enumerate(core)]
    d = P // 2
    while d >= 1:
        v = [add(dtype, v[j], v[j ^ d]) for j in range(P)]
        d //= 2
    count = len(a[0])
    out = np.empty_like(a[0])
    for c in range(P):
        sl = slice(part(count, P, c), part(count, P, c + 1))
        out[sl] = v[c][sl]
    return out


@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
@pytest.mark.parametrize("N", [2, 3, 4, 5, 8, 16])
def test_float_association_matches_closed_forms(N, dtype):
    count = 37 * N + 5
    a = f32_rank(N, count, N) if dtype == "float32" else bf16_rank(N, count, N)
    for o in oracle.allreduce(a, dtype, algo="ring"):
        assert np.array_equal(o.view(np.uint8), ring_fold(a, dtype, N, count).view(np.uint8))
    if (N & (N - 1)) == 0:
        want = butterfly(a, dtype, N)
        for o in oracle.allreduce(a, dtype, algo="rhd"):
            assert np.array_equal(o.view(np.uint8), want.view(np.uint8))
        want = tree_fold(a, dtype, N)
        for o in oracle.allreduce(a, dtype, algo="dbt"):
            assert np.array_equal(o.view(np.uint8), want.view(np.uint8))


@pytest.mark.parametrize("algo", ["ring", "rhd", "dbt"])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
@pytest.mark.parametrize("N", [8, 16])
def test_float_error_bounds_against_fp64(N, dtype, algo):
    """|y - y64| <= gamma_D * sum|a_r| elementwise (D rounded adds on the path,
    u = 2^-24, or 2^-8 + 2^-24 for bf16 where each row rounds twice), and the
    normwise error within 1e-5 (fp32) / 1e-2 (bf16)."""
    count = 4096
    a = f32_rank(N, count, 3) if dtype == "float32" else bf16_rank(N, count, 3)
    wide = [x.astype(np.float64) if dtype == "float32" else numerics.bf16_to_f32(x).astype(np.float64)
            for x in a]
    y64 = np.sum(wide, axis=0)
    absum = np.sum(np.abs(wide), axis=0)
    y = oracle.allreduce(a, dtype, algo=algo)[0]
    y = y.astype(np.float64) if dtype == "float32" else numerics.bf16_to_f32(y).astype(np.float64)
    D = {"ring": N - 1, "rhd": int(np.log2(N)), "dbt": int(np.log2(N)) + 1}[algo]
    u = 2.0 ** -24 if dtype == "float32" else 2.0 ** -8 + 2.0 ** -24
    gamma = D * u / (1 - D * u)
    assert np.all(np.abs(y - y64) <= gamma * absum * (1 + 1e-12))
    rel = np.linalg.norm(y - y64) / np.linalg.norm(y64)
    assert rel <= (1e-5 if dtype == "float32" else 1e-2)


# --- element arithmetic ---------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    import torch
    g = np.random.default_rng(5)
    x = g.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    bits = x.view(np.uint32)
    # exact ties (dropped half == 0x8000) with even and odd kept parts
    ties = ((bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38,
                        np.finfo(np.float32).max, 1e-40, -1e-40, 1.0, -1.0], dtype=np.float32)
    allx = np.concatenate([x, ties, special])
    mine = numerics.f32_to_bf16_rne(allx)
    ref = torch.from_numpy(allx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    nan = numerics.f32_to_bf16_rne(np.array([np.nan, -np.nan], dtype=np.float32))
    assert list(nan) == [0x7FC0, 0x7FC0]


def test_bf16_widening_is_exact():
    import torch
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    b = b[(b & 0x7F80) != 0x7F80]                      # finite patterns
    mine = numerics.bf16_to_f32(b)
    ref = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(mine.view(np.uint32), ref.view(np.uint32))


def test_fp32_add_is_correctly_rounded():
    """binary64 carries more than 2*24+2 bits, so rounding the binary64 sum of two
    binary32 values to binary32 is the correctly rounded binary32 sum."""
    g = np.random.default_rng(11)
    x = (g.standard_normal(100000) * 2.0 ** g.integers(-30, 30, 100000)).astype(np.float32)
    y = (g.standard_normal(100000) * 2.0 ** g.integers(-30, 30, 100000)).astype(np.float32)
    y[:100] = np.float32(1e-42)                          # subnormals are kept
    x[:100] = np.float32(1e-42)
    got = numerics.combine(x, y, "float32", "sum")
    want = (x.astype(np.float64) + y.astype(np.float64)).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # a subnormal doubles by doubling its bit pattern; nothing is flushed to zero
    assert got[:1].view(np.uint32)[0] == 2 * x[:1].view(np.uint32)[0] != 0


def test_int32_sum_wraps():
    a = np.array([2 ** 31 - 1, -2 ** 31, -1], dtype=np.int32)
    b = np.array([1, -1, 1], dtype=np.int32)
    assert list(numerics.combine(a, b, "int32", "sum")) == [-2 ** 31, 2 ** 31 - 1, 0]


def test_float_max_min_pick_an_operand():
    g = np.random.default_rng(2)
    x = g.standard_normal(1000).astype(np.float32)
    y = g.standard_normal(1000).astype(np.float32)
    assert np.array_equal(numerics.combine(x, y, "float32", "max"), np.maximum(x, y))
    assert np.array_equal(numerics.combine(x, y, "float32", "min"), np.minimum(x, y))
    bx, by = numerics.f32_to_bf16_rne(x), numerics.f32_to_bf16_rne(y)
    m = numerics.combine(bx, by, "bfloat16", "max")
    assert np.array_equal(numerics.bf16_to_f32(m), np.maximum(numerics.bf16_to_f32(bx),
                                                             numerics.bf16_to_f32(by)))


def test_row_checksum_definition():
    g = np.random.default_rng(4)
    for n in (0, 1, 2, 3, 5, 8, 13):
        for dt in (np.uint8, np.uint16, np.int32):
            a = g.integers(0, 200, n).astype(dt)
            raw = a.tobytes() + b"\0" * ((-len(a.tobytes())) % 4)
            want = sum(int.from_bytes(raw[i:i + 4], "little") for i in range(0, len(raw), 4))
            assert numerics.row_checksum(a) == want % (1 << 64)


def test_copy_row_checksums_equal_the_source():
    N, count = 8, 8 * 33
    a = [np.random.default_rng(i).integers(0, 256, count, dtype=np.uint8) for i in range(N)]
    plan = make_plan("broadcast", "binomial_pipe", N, count, 3, 5)
    _, sums = run_plan(plan, "uint8", "sum", a, trace=True)
    rows = plan.rows
    assert len(sums) == len(rows)
    for r, s in zip(rows, sums):
        assert s == numerics.row_checksum(a[3][r.src_off:r.src_off + r.n])


# --- planted mistakes are caught ----------------------------------------------------

def _mutants(plan):
    """Copies of ``plan`` with one plausible slip each: a dropped row, a row
    sent to the wrong rank, a chunk index off by one, a copy that should reduce."""
    rows = plan.rows
    out = []
    for idx in (0, len(rows) // 2, len(rows) - 1):
        r = rows[idx]
        for bad in (None,
                    replace(r, dst=(r.dst + 1) % plan.nranks) if (r.dst + 1) % plan.nranks != r.src else None,
                    replace(r, src_off=(r.src_off + r.n) % plan.count, dst_off=(r.dst_off + r.n) % plan.count),
                    replace(r, reduce=not r.reduce)):
            if bad == r:
                continue                      # a shift by the whole buffer changes nothing
            steps = [list(s) for s in plan.steps]
            st = steps[r.step]
            pos = st.index(r)
            if bad is None:
                del st[pos]
            else:
                st[pos] = bad
            out.append(Plan(plan.kind, plan.algo, plan.nranks, plan.count, plan.root,
                            plan.chunks, steps, list(plan.local), list(plan.staged)))
    return out


@pytest.mark.parametrize("kind,algo", [("allreduce", "ring"), ("allreduce", "rhd"),
                                       ("allreduce", "dbt"), ("reducescatter", "ring")])
def test_planted_schedule_mistakes_are_caught(kind, algo):
    """Every mutant fails the integer brute-force check or the float closed-form
    association check (a misrouted partial sum can still reach the right integer
    total, but never with the schedule's association)."""
    N, count = 8, 8 * 6
    a = rng_ints(N, count, 1)
    want = wrap_sum(a)
    f = f32_rank(N, count, 2)
    fwant = {"ring": ring_fold, "rhd": lambda x, d, n, c: butterfly(x, d, n),
             "dbt": lambda x, d, n, c: tree_fold(x, d, n)}[algo](f, "float32", N, count)
    plan = make_plan(kind, algo, N, count)
    regions = [slice(0, count) if kind == "allreduce" else chunk(count, N, i) for i in range(N)]
    muts = _mutants(plan)
    caught = 0
    for m in muts:
        out = run_plan(m, "int32", "sum", a)
        fout = run_plan(m, "float32", "sum", f)
        ok = all(np.array_equal(out[i][regions[i]], want[regions[i]]) for i in range(N))
        ok = ok and all(np.array_equal(fout[i][regions[i]].view(np.uint32),
                                       fwant[regions[i]].view(np.uint32)) for i in range(N))
        caught += not ok
    assert caught == len(muts)


# --- Tree Reduce, linear Scatter, Broadcast as Scatter + AllGather ---------------

@pytest.mark.parametrize("N", NS_SMALL)
def test_reduce_linear_scatter_scatter_allgather_brute_force(N):
    g = np.random.default_rng(300 + N)
    for count in counts_for(N):
        a = [g.integers(-(1 << 31), (1 << 31) - 1, count, endpoint=True, dtype=np.int32) for _ in range(N)]
        want = wrap_sum(a) if count else np.zeros(0, np.int32)
        for root in sorted({0, N // 2, N - 1}):
            assert np.array_equal(oracle.reduce(a, "int32", root=root)[root], want)
            for op, fn in (("max", np.max), ("min", np.min)):
                if count:
                    assert np.array_equal(oracle.reduce(a, "int32", op=op, root=root)[root], fn(np.stack(a), axis=0))
            sc = oracle.scatter(a, "int32", root, algo="linear")
            for i in range(N):
                assert np.array_equal(sc[i][chunk(count, N, i)], a[root][chunk(count, N, i)])
            for o in oracle.broadcast(a, "int32", root, algo="scatter_allgather"):
                assert np.array_equal(o, a[root])


def binomial_fold(a, dtype, N, root):
    """Relative rank v's value after step j is its own folded with the subtree
    [v + 2^(j-1), v + 2^j): R(v, j) = R(v, j-1) + R(v + 2^(j-1), j-1)."""
    def R(v, j):
        if j == 0:
            return a[(root + v) % N]
        d = 1 << (j - 1)
        acc = R(v, j - 1)
        return add(dtype, acc, R(v + d, j - 1)) if v + d < N else acc
    L = 0
    while (1 << L) < N:
        L += 1
    return R(0, L)


@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
@pytest.mark.parametrize("N", [2, 3, 5, 8, 13, 16])
def test_reduce_association_matches_binomial_fold(N, dtype):
    count = 21 * N + 2
    a = f32_rank(N, count, 50 + N) if dtype == "float32" else bf16_rank(N, count, 50 + N)
    for root in (0, N - 1):
        got = oracle.reduce(a, dtype, root=root)[root]
        assert np.array_equal(got.view(np.uint8), binomial_fold(a, dtype, N, root).view(np.uint8))


def test_planted_reduce_mistakes_are_caught():
    N, count = 8, 40
    a = rng_ints(N, count, 9)
    f = f32_rank(N, count, 10)
    plan = make_plan("reduce", "binomial", N, count, 2)
    fwant = binomial_fold(f, "float32", N, 2)
    muts = _mutants(plan)
    caught = 0
    for m in muts:
        ok = np.array_equal(run_plan(m, "int32", "sum", a)[2], wrap_sum(a))
        ok = ok and np.array_equal(run_plan(m, "float32", "sum", f)[2].view(np.uint32), fwant.view(np.uint32))
        caught += not ok
    assert caught == len(muts)


@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
@pytest.mark.parametrize("N", [3, 5, 6, 7, 9, 12])
def test_non_power_of_two_association(N, dtype):
    count = 37 * N + 11
    a = f32_rank(N, count, 70 + N) if dtype == "float32" else bf16_rank(N, count, 70 + N)
    want = folded_butterfly(a, dtype, N)
    for o in oracle.allreduce(a, dtype, algo="rhd"):
        assert np.array_equal(o.view(np.uint8), want.view(np.uint8))
    want = tree_fold(a, dtype, N)
    for o in oracle.allreduce(a, dtype, algo="dbt"):
        assert np.array_equal(o.view(np.uint8), want.view(np.uint8))


@pytest.mark.parametrize("N", list(range(1, 20)) + [31, 33])
def test_non_power_of_two_brute_force(N):
    for count in (1, N, 5 * N + 2, 300):
        a = rng_ints(N, count, 90 + N, lo=-(1 << 31), hi=(1 << 31) - 1)
        for algo in ("rhd", "dbt"):
            for o in oracle.allreduce(a, "int32", algo=algo):
                assert np.array_equal(o, wrap_sum(a)), (algo, N, count)


@pytest.mark.parametrize("N", [5, 6])
def test_planted_non_power_of_two_mistakes_are_caught(N):
    count = N * 12
    a = rng_ints(N, count, 4)
    f = f32_rank(N, count, 5)
    for algo, fn in (("rhd", folded_butterfly), ("dbt", tree_fold)):
        plan = make_plan("allreduce", algo, N, count)
        fwant = fn(f, "float32", N)
        muts = _mutants(plan)
        caught = 0
        for m in muts:
            ok = all(np.array_equal(o, wrap_sum(a)) for o in run_plan(m, "int32", "sum", a))
            ok = ok and all(np.array_equal(o.view(np.uint32), fwant.view(np.uint32))
                            for o in run_plan(m, "float32", "sum", f))
            caught += not ok
        assert caught == len(muts), (algo, N)


@pytest.mark.parametrize("N,k", [(4, 1), (7, 3), (8, 2)])
def test_planted_bidir_ring_broadcast_mistakes_are_caught(N, k):
    """A dropped, misrouted, shifted or reducing row of the bidirectional-ring
    Broadcast leaves some rank with something other than the root's bytes."""
    count = N * k * 5
    a = rng_ints(N, count, 7)
    plan = make_plan("broadcast", "bidir_ring", N, count, 1, k)
    muts = _mutants(plan)
    assert muts
    for m in muts:
        out = run_plan(m, "int32", "sum", a)
        assert not all(np.array_equal(o, a[1]) for o in out)


@pytest.mark.parametrize("N", [3, 5, 8])
def test_planted_ring_alltoall_mistakes_are_caught(N):
    """A dropped, misrouted, shifted or reducing row of the Ring AllToAll breaks
    the block transpose."""
    B = 4
    a = rng_ints(N, N * B, 11)
    plan = make_plan("alltoall", "ring", N, N * B)
    muts = _mutants(plan)
    assert muts
    for m in muts:
        out = run_plan(m, "int32", "sum", a, rng_ints(N, N * B, 12))   # receive buffers hold garbage
        ok = all(np.array_equal(out[j][i * B:(i + 1) * B], a[i][j * B:(j + 1) * B])
                 for i in range(N) for j in range(N))
        assert not ok
