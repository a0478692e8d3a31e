"""Collective calls captured in a HIP graph (through torch.cuda.CUDAGraph) and
replayed: after one eager call has built and cached the schedule, a call only
launches kernels, which capture records.  Every replay, with eager work and
synchronisation between replays, must give the eager result bit for bit."""

import numpy as np
import pytest

import seeded_inputs as si

pytestmark = pytest.mark.gpu


def test_captured_collectives_replay_exactly(gpu_device):
    import torch
    import collective_communication_algorithms_amd as coll
    N, count = 8, 8 * 20000 + 8
    a = si.rank_arrays(15, N, count, "float32")
    u = si.rank_arrays(16, N, 1 << 18, "uint8")
    pristine = torch.stack([si.host_to_tensor(x, "float32", gpu_device) for x in a])
    pu = torch.stack([si.host_to_tensor(x, "uint8", gpu_device) for x in u])
    live, lu = pristine.clone(), pu.clone()
    recv = torch.empty_like(pristine)
    ps = list(pristine[:, :N * 20000])   # 80,000-byte blocks: the direct copy path
    recv2 = torch.empty((N, N * 20000), dtype=torch.float32, device=gpu_device)
    recv3 = torch.empty_like(recv2)   # Bruck: its first rotation as a direct copy

    def work():
        coll.coll_allreduce(list(live), algo="ring")
        coll.coll_allreduce(list(live), algo="dbt", op="max")
        coll.coll_broadcast(list(lu), algo="bidir_ring", root=5, chunks=3)
        coll.coll_alltoall(list(pristine), list(recv), algo="bruck")
        coll.coll_alltoall(ps, list(recv2), algo="pairwise")
        coll.coll_alltoall(ps, list(recv3), algo="bruck")

    # eager reference (also builds and caches every schedule before capture)
    work()
    torch.cuda.synchronize()
    want = (live.clone(), lu.clone(), recv.clone(), recv2.clone(), recv3.clone())
    live.copy_(pristine)
    lu.copy_(pu)
    recv.zero_()
    recv2.zero_()
    recv3.zero_()
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        live.copy_(pristine)          # eager work between replays
        lu.copy_(pu)
        recv.zero_()
        recv2.zero_()
        recv3.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, w, name in ((live, want[0], "allreduce"), (lu, want[1], "broadcast"), (recv, want[2], "alltoall"),
                             (recv2, want[3], "alltoall pairwise"), (recv3, want[4], "alltoall bruck copy")):
            assert torch.equal(got.view(torch.uint8), w.view(torch.uint8)), (rep, name)
    coll.coll_check()


def test_captured_calls_with_checksums_replay_exactly(gpu_device):
    """Row checksums under capture: a captured call clears its partial slots
    itself, so every replay gives the eager checksums, also with checksummed
    eager calls on the same buffers between replays."""
    import torch
    import collective_communication_algorithms_amd as coll
    N, count = 8, 8 * 30000 + 5
    a = si.rank_arrays(17, N, count, "float32")
    pristine = torch.stack([si.host_to_tensor(x, "float32", gpu_device) for x in a])
    live = pristine.clone()
    rows, _ = coll.coll_plan("allreduce", "ring", N, count, "float32")
    sums = torch.full((len(rows),), -1, dtype=torch.int64, device=gpu_device)
    coll.coll_set_checksums(sums)
    try:
        coll.coll_allreduce(list(live), algo="ring")          # eager: builds the schedule and the slots
        torch.cuda.synchronize()
        want, want_sums = live.clone(), sums.clone()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        live.copy_(pristine)
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                coll.coll_allreduce(list(live), algo="ring")
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for rep in range(4):
            live.copy_(pristine)                               # an eager checksummed call between replays
            sums.fill_(-1)
            coll.coll_allreduce(list(live), algo="ring")
            torch.cuda.synchronize()
            assert torch.equal(sums, want_sums) and torch.equal(live.view(torch.int32), want.view(torch.int32)), rep
            live.copy_(pristine)
            sums.fill_(-1)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(sums, want_sums), ("replay", rep)
            assert torch.equal(live.view(torch.int32), want.view(torch.int32)), ("replay", rep)
    finally:
        coll.coll_set_checksums(None)


def test_captured_calls_outlive_eviction_growth_and_new_tables(gpu_device):
    """What a captured call's kernels read stays valid for every replay while
    eager calls change the library's state underneath: the schedule cache
    shrunk to nothing (every unpinned schedule evicted), new column tables for
    the same schedule (another tile count), the checksum slot buffer of the
    same caller buffer grown by a larger schedule, and more than 16 caller
    checksum buffers (slot buffers evicted); a checksummed Pairwise AllToAll
    run as one direct copy beside them.  Replays must still give the
    eager results and checksums bit for bit."""
    import torch
    import collective_communication_algorithms_amd as coll
    dev = gpu_device
    N, count = 8, 8 * 30000 + 5
    a = si.rank_arrays(18, N, count, "float32")
    pristine = torch.stack([si.host_to_tensor(x, "float32", dev) for x in a])
    live = pristine.clone()
    # a row-kernel call captured beside the column-kernel one: AllToAll
    pa = torch.stack([si.host_to_tensor(x, "bfloat16", dev) for x in si.rank_arrays(19, 16, 16 * 999, "bfloat16")])
    recv = torch.empty_like(pa)
    # and a checksummed Pairwise AllToAll that runs as one direct copy (2,000-byte blocks)
    pd = torch.stack([si.host_to_tensor(x, "bfloat16", dev) for x in si.rank_arrays(20, 16, 16 * 1000, "bfloat16")])
    recv_d = torch.empty_like(pd)
    rows_d, _ = coll.coll_plan("alltoall", "pairwise", 16, 16 * 1000, "bfloat16")
    sums_d = torch.full((len(rows_d),), -1, dtype=torch.int64, device=dev)
    # and a checksummed Bruck AllToAll: its first rotation a direct copy, its rounds in the permutation kernel
    recv_b = torch.empty_like(pd)
    rows_b, _ = coll.coll_plan("alltoall", "bruck", 16, 16 * 1000, "bfloat16")
    sums_b = torch.full((len(rows_b),), -1, dtype=torch.int64, device=dev)
    rows8, _ = coll.coll_plan("allreduce", "ring", N, count, "float32")
    rows16, _ = coll.coll_plan("allreduce", "ring", 16, 16 * 30000, "float32")
    cap = max(len(rows8), len(rows16))
    sums = torch.full((cap,), -1, dtype=torch.int64, device=dev)
    old_cache = coll.coll_get_option("cache_bytes")

    def work():
        coll.coll_set_checksums(sums)
        coll.coll_allreduce(list(live), algo="ring")
        coll.coll_set_checksums(None)
        coll.coll_alltoall(list(pa), list(recv), algo="bruck")
        coll.coll_set_checksums(sums_d)
        coll.coll_alltoall(list(pd), list(recv_d), algo="pairwise")
        coll.coll_set_checksums(sums_b)
        coll.coll_alltoall(list(pd), list(recv_b), algo="bruck")
        coll.coll_set_checksums(None)

    try:
        work()
        torch.cuda.synchronize()
        want, want_recv = live.clone(), recv.clone()
        want_sums = sums[:len(rows8)].clone()
        want_d, want_sums_d = recv_d.clone(), sums_d.clone()
        want_b, want_sums_b = recv_b.clone(), sums_b.clone()
        live.copy_(pristine)
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                work()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()

        # eager calls that replace or free what an unpinned call would use
        coll.coll_set_option("cache_bytes", 0)
        other = [torch.randn(N, 4096 * (i + 1) + 3, device=dev) for i in range(4)]
        for t in other:
            coll.coll_allreduce(list(t), algo="dbt")
            coll.coll_alltoall(list(t[:, :4096]), list(torch.empty_like(t[:, :4096])), algo="pairwise")
        coll.coll_set_checksums(sums)
        coll.coll_set_option("col_tiles", 2)
        coll.coll_allreduce(list(live), algo="ring")        # same schedule, new column tables
        coll.coll_set_option("col_tiles", 0)
        big = torch.randn(16, 16 * 30000, device=dev)
        coll.coll_allreduce(list(big), algo="ring")         # same caller buffer, larger slot buffer
        for i in range(17):                                   # more caller buffers than slot buffers kept
            extra = torch.zeros(len(rows8), dtype=torch.int64, device=dev)
            coll.coll_set_checksums(extra)
            coll.coll_allreduce(list(other[0]), algo="ring")
        coll.coll_set_checksums(None)
        torch.cuda.synchronize()

        for rep in range(3):
            live.copy_(pristine)
            recv.zero_()
            recv_d.zero_()
            recv_b.zero_()
            sums.fill_(-1)
            sums_d.fill_(-1)
            sums_b.fill_(-1)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(live.view(torch.int32), want.view(torch.int32)), ("allreduce", rep)
            assert torch.equal(recv.view(torch.int16), want_recv.view(torch.int16)), ("alltoall", rep)
            assert torch.equal(sums[:len(rows8)], want_sums), ("checksums", rep)
            assert torch.equal(recv_d.view(torch.int16), want_d.view(torch.int16)), ("pairwise", rep)
            assert torch.equal(sums_d, want_sums_d), ("pairwise checksums", rep)
            assert torch.equal(recv_b.view(torch.int16), want_b.view(torch.int16)), ("bruck", rep)
            assert torch.equal(sums_b, want_sums_b), ("bruck checksums", rep)
        coll.coll_check()
    finally:
        coll.coll_set_checksums(None)
        coll.coll_set_option("cache_bytes", old_cache)
        coll.coll_set_option("col_tiles", 0)
