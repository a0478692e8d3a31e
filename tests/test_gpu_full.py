"""Parity at the configurations' full sizes, in the default launch configuration
(the one bench.py times), on sampled outputs the oracle computes exactly.

Every schedule except AllToAll keeps each element at its offset, so element x
of every output depends only on element x of the inputs: the oracle restricted
to a sample of columns (``run_plan_columns``) gives the exact expected values
there.  AllToAll keeps the offset inside a block, so the oracle runs on blocks
cut down to a sample of in-block offsets.  Inputs are drawn on the device by
torch's seeded generator (never by the path under test).
"""

import numpy as np
import pytest

import seeded_inputs as si
from oracle.schedules import make_plan
from oracle.simulate import defined_regions, run_plan_columns
from oracle import numerics

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(autouse=True)
def _defaults(gpu_device):
    import collective_communication_algorithms_amd as coll
    for k, v in {"exec": 0, "group_tiles": 0, "max_grid": 0, "nontemporal": -1, "reverse": 1, "col_tiles": 0}.items():
        coll.coll_set_option(k, v)
    yield
    coll.coll_set_option("exec", 0)


def sample_columns(count, N, stride=4097, edge=65536, around=256, extra=()):
    parts = [np.arange(0, count, stride), np.arange(0, min(edge, count)), np.arange(max(0, count - edge), count)]
    for c in extra:
        parts.append(np.arange(max(0, c - around), min(count, c + around)))
    for c in range(1, N):
        b = c * count // N
        parts.append(np.arange(max(0, b - around), min(count, b + around)))
    return np.unique(np.concatenate(parts))


def gather_cols(tensors, cols, dtype):
    import torch
    idx = torch.from_numpy(cols).to(tensors[0].device)
    return [si.tensor_to_host(t.index_select(0, idx), dtype) for t in tensors]


def check_sampled(kind, algo, N, count, dtype, workload, sigma=1.0, root=0, k=1, extra=()):
    import torch
    import collective_communication_algorithms_amd as coll
    dev = torch.device("cuda:0")
    buf = torch.empty((N, count), dtype=si.to_torch_dtype(dtype), device=dev)
    ranks = si.device_rank_tensors(workload, N, count, dtype, dev, sigma=sigma, out=buf)
    cols = sample_columns(count, N, extra=extra)
    before = gather_cols(ranks, cols, dtype)
    coll.COLLECTIVE_FNS[kind](ranks, op="sum", algo=algo, root=root, chunks=k)
    torch.cuda.synchronize()
    after = gather_cols(ranks, cols, dtype)
    want = run_plan_columns(make_plan(kind, algo, N, count, root, k), dtype, "sum", cols, before)
    for i, regs in enumerate(defined_regions(kind, N, count, root)):
        for lo, hi in regs:
            m = (cols >= lo) & (cols < hi)
            assert np.array_equal(after[i][m].view(np.uint8), want[i][m].view(np.uint8)), \
                (kind, algo, dtype, N, count, i, int(np.sum(after[i][m] != want[i][m])))
    del buf, ranks
    torch.cuda.empty_cache()
    return before, after


@pytest.mark.parametrize("algo", ["ring", "rhd", "dbt"])
@pytest.mark.parametrize("dtype,sigma", [("float32", 1.0), ("bfloat16", 0.02)])
def test_allreduce_n8_256MiB(algo, dtype, sigma):
    count = (256 << 20) // si.ITEMSIZE[dtype]
    before, after = check_sampled("allreduce", algo, 8, count, dtype, 3, sigma=sigma)
    wide = [x.astype(np.float64) if dtype == "float32" else numerics.bf16_to_f32(x).astype(np.float64)
            for x in before]
    y64 = np.sum(wide, axis=0)
    y = after[0].astype(np.float64) if dtype == "float32" else numerics.bf16_to_f32(after[0]).astype(np.float64)
    assert np.linalg.norm(y - y64) / np.linalg.norm(y64) <= (1e-5 if dtype == "float32" else 1e-2)


@pytest.mark.parametrize("algo", ["ring", "rhd", "dbt"])
@pytest.mark.parametrize("dtype,sigma", [("float32", 1.0), ("bfloat16", 0.02), ("int32", 1.0)])
def test_allreduce_n8_40MiB_ragged(algo, dtype, sigma):
    """A column space between 32 and 48 MiB with a ragged count: the large-grid
    launch shapes whose Ring grid has 2 work groups per CU (fewer than 6
    column groups per CU), on a capped grid with chunk boundaries that fall
    inside 16-byte units."""
    count = (40 << 20) // si.ITEMSIZE[dtype] + 3
    check_sampled("allreduce", algo, 8, count, dtype, 7, sigma=sigma)


@pytest.mark.parametrize("algo,k", [("binomial", 1), ("chain_pipe", 1), ("chain_pipe", 8), ("chain_pipe", 13),
                                    ("chain_pipe", 64), ("binomial_pipe", 1), ("binomial_pipe", 8),
                                    ("binomial_pipe", 64), ("bidir_ring", 1), ("bidir_ring", 8),
                                    ("bidir_ring", 13)])
def test_broadcast_n8_64MiB(algo, k):
    check_sampled("broadcast", algo, 8, 64 << 20, "uint8", 2, k=k)


@pytest.mark.parametrize("kind,algo", [("scatter", "binomial"), ("scatter", "linear"), ("gather", "binomial"),
                                       ("broadcast", "scatter_allgather")])
def test_scatter_gather_n8_64MiB(kind, algo):
    check_sampled(kind, algo, 8, 64 << 20, "uint8", 2)


@pytest.mark.parametrize("dtype,sigma", [("float32", 1.0), ("bfloat16", 0.02)])
def test_reduce_n8_256MiB(dtype, sigma):
    check_sampled("reduce", "binomial", 8, (256 << 20) // si.ITEMSIZE[dtype], dtype, 3, sigma=sigma, root=3)


@pytest.mark.parametrize("kind", ["reducescatter", "allgather"])
@pytest.mark.parametrize("algo", ["ring", "rhd"])
def test_reducescatter_allgather_n64_256MiB(kind, algo):
    """64 ranks x 256 MiB bf16 N(0, 1e-3): 16 GiB resident."""
    check_sampled(kind, algo, 64, (256 << 20) // 2, "bfloat16", 4, sigma=1e-3)


@pytest.mark.parametrize("algo", ["pairwise", "bruck", "ring"])
def test_alltoall_n32_512x4096(algo):
    """32 ranks; each sends 512 tokens x 4096 bf16 to every peer (128 MiB per rank)."""
    import torch
    import collective_communication_algorithms_amd as coll
    import oracle
    dev = torch.device("cuda:0")
    N, B = 32, 512 * 4096
    count = N * B
    sbuf = torch.empty((N, count), dtype=torch.bfloat16, device=dev)
    send = si.device_rank_tensors(5, N, count, "bfloat16", dev, out=sbuf)
    rbuf = torch.empty_like(sbuf)
    recv = [rbuf[i] for i in range(N)]
    offs = np.unique(np.concatenate([np.arange(0, B, 1021), np.arange(0, 256), np.arange(B - 256, B)]))
    S = len(offs)
    cols = (np.arange(N)[:, None] * B + offs[None, :]).reshape(-1)
    red_in = gather_cols(send, cols, "bfloat16")
    coll.coll_alltoall(send, recv, algo=algo)
    torch.cuda.synchronize()
    got = gather_cols(recv, cols, "bfloat16")
    want = oracle.alltoall(red_in, "bfloat16", algo)
    for j in range(N):
        assert np.array_equal(got[j], want[j]), (algo, j)
    # and against the definition on the sample: recv_j block i = send_i block j
    for j in (0, 17, 31):
        for i in (0, 5, 31):
            assert np.array_equal(got[j][i * S:(i + 1) * S], red_in[i][j * S:(j + 1) * S])
    del sbuf, rbuf, send, recv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("algo,N,checksums", [("ring", 8, False), ("ring", 16, False), ("ring", 16, True),
                                              ("rhd", 32, True)])
def test_allreduce_at_fewer_work_groups_per_cu(algo, N, checksums):
    """The column kernel's variants that run at fewer work groups per CU engage
    from 128 tiles per CU, 32 MiB of columns per rank: the paired one (8 ranks,
    no checksums) and the capped batched ones (16 and 32 ranks, with and
    without checksums).  int32 at exactly that size: whole buffers and every
    row checksum bit for bit against the oracle."""
    from tests.gpu_util import assert_parity
    count = (32 << 20) // 4
    a = si.rank_arrays(40 + N, N, count, "int32")
    assert_parity("allreduce", algo, a, "int32", checksums=checksums)


@pytest.mark.parametrize("algo", ["pairwise", "bruck", "ring"])
def test_alltoall_row_checksums_n32_128MiB(algo):
    """C5 at full size with row checksums, in the default launch (every
    algorithm one direct copy of the blocks): every row's checksum equals the
    oracle's.  An AllToAll row only moves a block, so its checksum is that of
    the send block it carries; which block that is comes from the oracle's own
    plan run on blocks holding their ids (a row's checksum over a one-element
    int32 block is the element), and the block's checksum from the oracle's
    row_checksum over the full-size send block."""
    import torch
    import collective_communication_algorithms_amd as coll
    from oracle.simulate import run_plan
    dev = torch.device("cuda:0")
    N, B = 32, (128 << 20) // 2 // 32
    count = N * B
    ids = [np.arange(i * N, (i + 1) * N, dtype=np.int32) for i in range(N)]
    _, carried = run_plan(make_plan("alltoall", algo, N, N), "int32", "sum", ids, trace=True)
    sbuf = torch.empty((N, count), dtype=torch.bfloat16, device=dev)
    send = si.device_rank_tensors(9, N, count, "bfloat16", dev, out=sbuf)
    rbuf = torch.empty_like(sbuf)
    rows, cnt = coll.coll_plan("alltoall", algo, N, count, "bfloat16")
    assert len(rows) == len(carried)
    sums = torch.full((len(rows),), -1, dtype=torch.int64, device=dev)
    coll.coll_set_checksums(sums)
    try:
        coll.coll_alltoall(send, [rbuf[i] for i in range(N)], algo=algo)
    finally:
        coll.coll_set_checksums(None)
    torch.cuda.synchronize()
    st = coll.coll_get_stats()
    assert st["round_trips"] == 1 and st["moved_bytes"] == 2 * N * count * 2
    host = sbuf.view(torch.int16).cpu().numpy().view(np.uint16)
    block_sum = {}
    for b in sorted({int(c) for c in carried}):
        i, j = divmod(b, N)
        block_sum[b] = numerics.row_checksum(host[i, j * B:(j + 1) * B])
    got = sums.cpu().numpy().view(np.uint64)
    plan = make_plan("alltoall", algo, N, count)
    want_by_key = {}
    for idx, r in enumerate(r for st_rows in plan.steps for r in st_rows):
        want_by_key[(r.step, r.src, r.dst, r.src_off, r.dst_off, r.n)] = block_sum[int(carried[idx])]
    for j, r in enumerate(rows):
        assert int(got[j]) == want_by_key[tuple(r[:6])], (algo, j, r)
    # and the receive buffers: recv_j block i = send_i block j, on sampled blocks
    rhost = rbuf.view(torch.int16)
    for j in (0, 13, 31):
        for i in (0, 7, 31):
            assert torch.equal(rhost[j, i * B:(i + 1) * B].cpu(), sbuf.view(torch.int16)[i, j * B:(j + 1) * B].cpu())
    del sbuf, rbuf, send, sums
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kind,algo,N,count,dtype,k", [
    ("allreduce", "ring", 8, (256 << 20) // 4, "float32", 1),
    ("allgather", "ring", 8, (256 << 20) // 2, "bfloat16", 1),
    ("broadcast", "chain_pipe", 8, 128 << 20, "uint8", 1),
])
def test_row_kernel_long_pieces(kind, algo, N, count, dtype, k):
    """The row kernel (exec 2) at full size without checksums, where one-piece-
    per-step schedules take 4-tile column groups (pieces of 16 MiB and more over
    128 MiB of columns for copies, 8 MiB over 64 MiB for reductions; the host
    check pins that these three shapes get them): bit-exact on sampled columns."""
    import collective_communication_algorithms_amd as coll
    coll.coll_set_option("exec", 2)
    check_sampled(kind, algo, N, count, dtype, 3, k=k)


def test_columns_past_4GiB():
    """Rank buffers of 4.5 GiB and a few bytes: column offsets past 2^32 bytes
    in the schedules, the work lists and the row kernel's addresses.  Chain
    Broadcast of uint8 over 3 ranks and Ring AllReduce of int32 over 2 ranks,
    checked on sampled columns (around byte 2^32 too) against the oracle."""
    nb = (9 << 29) + 77
    check_sampled("broadcast", "chain_pipe", 3, nb, "uint8", 2, root=1, extra=(1 << 32,))
    n4 = (9 << 29) // 4 + 5
    check_sampled("allreduce", "ring", 2, n4, "int32", 3, extra=((1 << 32) // 4,))
