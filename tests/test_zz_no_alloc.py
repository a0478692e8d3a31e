"""The allocation-free AllReduce (coll_allreduce_noalloc): through the C ABI,
bit for bit the same results and row checksums as coll_allreduce on the same
inputs, for two calls in a row (the second on a smaller input), in and out of
place, for several algorithms and dtypes; it adds nothing to the library's
device memory; and it refuses what it cannot run with a clear error."""

import ctypes

import numpy as np
import pytest

import seeded_inputs as si

pytestmark = pytest.mark.gpu


def _ptrs(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def _call(fn_name, send, recv, dtype, algo):
    import torch
    from collective_communication_algorithms_amd import _lib
    lib = _lib.load()
    st = getattr(lib, fn_name)(_ptrs(send), _ptrs(recv) if recv is not None else None, len(send), send[0].numel(),
                               _lib.DTYPES[dtype], _lib.OPS["sum"], _lib.ALGOS[algo], 0, 1,
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def _run_both(host, dtype, algo, inplace, checksums):
    """Runs coll_allreduce and coll_allreduce_noalloc on copies of the same
    inputs; returns (outputs, checksums) of each."""
    import torch
    import collective_communication_algorithms_amd as coll
    dev = torch.device("cuda:0")
    res = []
    for fn in ("coll_allreduce", "coll_allreduce_noalloc"):
        send = [si.host_to_tensor(x, dtype, dev) for x in host]
        recv = None if inplace else [torch.empty_like(t) for t in send]
        sums = None
        if checksums:
            nrows = len(coll.coll_plan("allreduce", algo, len(host), len(host[0]), dtype)[0])
            sums = torch.zeros(max(nrows, 1), dtype=torch.int64, device=dev)
            coll.coll_set_checksums(sums)
        try:
            st = _call(fn, send, recv, dtype, algo)
            assert st == 0, (fn, st, coll.coll_get_stats())
            torch.cuda.synchronize()
        finally:
            coll.coll_set_checksums(None)
        out = recv if recv is not None else send
        res.append(([si.tensor_to_host(t, dtype) for t in out], sums.cpu().numpy() if sums is not None else None))
    return res


@pytest.mark.parametrize("dtype,algo,inplace", [("float32", "ring", True), ("bfloat16", "dbt", True),
                                                ("int32", "rhd", False), ("float32", "auto", True)])
def test_noalloc_matches_allreduce(gpu_device, dtype, algo, inplace):
    for call, (N, count) in enumerate(((8, 8 * 70000 + 77), (6, 6 * 1000 + 5))):
        host = si.rank_arrays(40 + call, N, count, dtype, sigma=0.02 if dtype == "bfloat16" else 1.0)
        for cks in (True, False):
            (ref, ref_sums), (got, got_sums) = _run_both(host, dtype, algo, inplace, cks)
            for i in range(N):
                assert np.array_equal(got[i].view(np.uint8), ref[i].view(np.uint8)), (call, i, cks)
            if cks:
                assert np.array_equal(got_sums, ref_sums), (call, cks)


def test_noalloc_allocates_nothing(gpu_device):
    """After a first call has taken the scratch's address, further calls (new
    shapes and algorithms, checksums on and off) leave the device's free
    memory, the library's cache and torch's allocator as they were."""
    import torch
    import collective_communication_algorithms_amd as coll
    dev = torch.device("cuda:0")
    a = [si.host_to_tensor(x, "float32", dev) for x in si.rank_arrays(3, 8, 8 * 4096, "float32")]
    assert _call("coll_allreduce_noalloc", a, None, "float32", "ring") == 0
    torch.cuda.synchronize()
    cache = coll.coll_cache_info()
    alloc = torch.cuda.memory_allocated(dev)
    sums = torch.zeros(4096, dtype=torch.int64, device=dev)
    bufs = [[si.host_to_tensor(x, "float32", dev) for x in si.rank_arrays(4, N, count, "float32")]
            for N, count in ((8, 8 * 4096 + 3), (4, 4 * 50000), (16, 16 * 999))]
    torch.cuda.synchronize()
    alloc = torch.cuda.memory_allocated(dev)
    free0, _ = torch.cuda.mem_get_info(dev)
    for b in bufs:
        for algo in ("ring", "dbt", "rhd"):
            for cks in (False, True):
                coll.coll_set_checksums(sums if cks else None)
                assert _call("coll_allreduce_noalloc", b, None, "float32", algo) == 0
        coll.coll_set_checksums(None)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated(dev) == alloc
    assert coll.coll_cache_info() == cache
    assert torch.cuda.mem_get_info(dev)[0] == free0


@pytest.mark.parametrize("algo", ["ring", "rhd"])
def test_noalloc_matches_allreduce_batched_leaves(gpu_device, algo):
    """More ranks than register slots (leaves brought in batches): 64 ranks
    with and without row checksums (63-op programs: per-tile wave sums), then
    32 and 16."""
    for call, (N, count, cks) in enumerate(((64, 64 * 3000 + 17, False), (64, 64 * 1000 + 3, True),
                                            (32, 32 * 500 + 9, True), (16, 16 * 100 + 1, True))):
        host = si.rank_arrays(60 + call, N, count, "float32")
        (ref, ref_sums), (got, got_sums) = _run_both(host, "float32", algo, True, cks)
        for i in range(N):
            assert np.array_equal(got[i].view(np.uint8), ref[i].view(np.uint8)), (call, i)
        if cks:
            assert np.array_equal(got_sums, ref_sums), call


def test_noalloc_refuses_what_it_cannot_run(gpu_device):
    import torch
    from collective_communication_algorithms_amd import _lib
    dev = torch.device("cuda:0")
    # rank buffers off 16-byte alignment
    buf = torch.zeros((8, 1024 + 1), dtype=torch.float32, device=dev)
    st = _call("coll_allreduce_noalloc", [buf[i, 1:] for i in range(8)], None, "float32", "ring")
    assert st == _lib.COLL_ERR_UNSUPPORTED and b"16-byte" in _lib.load().coll_last_error()
    # more ranks than a program list holds (65)
    b = [torch.zeros(65 * 64, dtype=torch.float32, device=dev) for _ in range(65)]
    st = _call("coll_allreduce_noalloc", b, None, "float32", "ring")
    assert st == _lib.COLL_ERR_UNSUPPORTED and b"column kernel" in _lib.load().coll_last_error()
