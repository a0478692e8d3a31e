"""Collectives on a side stream while a stand-in compute kernel runs on another
(the HCCL blog's overlap of compute and communication): results must still be
the oracle's, bit for bit.  Streams keep the default priority."""

import numpy as np
import pytest

import seeded_inputs as si
from oracle.schedules import make_plan
from oracle.simulate import run_plan

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _defaults(gpu_device):
    import collective_communication_algorithms_amd as coll
    for k, v in {"exec": 0, "group_tiles": 0, "max_grid": 0, "nontemporal": -1, "reverse": 1}.items():
        coll.coll_set_option(k, v)
    yield
    coll.coll_set_option("max_grid", 0)


@pytest.mark.parametrize("max_grid", [0, 1024])
@pytest.mark.parametrize("kind,algo,dtype,N,count", [
    ("allreduce", "ring", "float32", 8, (1 << 20) + 77),
    ("allreduce", "dbt", "bfloat16", 8, 300001),
    ("reducescatter", "rhd", "int32", 16, 16 * 5000 + 9),
    ("broadcast", "bidir_ring", "uint8", 8, 1 << 20),
    ("alltoall", "bruck", "bfloat16", 16, 16 * 4099),
    ("alltoall", "ring", "int32", 8, 8 * 10000),
])
def test_side_stream_collective_beside_compute(kind, algo, dtype, N, count, max_grid):
    import torch
    import collective_communication_algorithms_amd as coll
    dev = torch.device("cuda:0")
    coll.coll_set_option("max_grid", max_grid)
    a = si.rank_arrays(21, N, count, dtype, sigma=0.02 if dtype == "bfloat16" else 1.0)
    send = [si.host_to_tensor(x, dtype, dev) for x in a]
    recv = [torch.empty_like(t) for t in send] if kind == "alltoall" else None
    spin_out = torch.zeros(1024 * 256, dtype=torch.float32, device=dev)
    main_s = torch.cuda.current_stream(dev)
    side_s = torch.cuda.Stream(dev)
    torch.cuda.synchronize()
    start = torch.cuda.Event()
    start.record(main_s)
    side_s.wait_event(start)
    coll.coll_calib_spin(spin_out, 200000, 1024, stream=main_s)
    coll.COLLECTIVE_FNS[kind](send, recv, op="sum", algo=algo, root=3 % N, stream=side_s)
    torch.cuda.synchronize()
    got = [si.tensor_to_host(t, dtype) for t in (recv if recv is not None else send)]
    want = run_plan(make_plan(kind, algo, N, count, 3 % N), dtype, "sum", a)
    from oracle.simulate import defined_regions
    for i, regs in enumerate(defined_regions(kind, N, count, 3 % N)):
        for lo, hi in regs:
            assert np.array_equal(got[i][lo:hi].view(np.uint8), want[i][lo:hi].view(np.uint8)), (kind, algo, i)
    # the compute ran too: every thread stored a finite value, equal for threads
    # that start from the same seed
    s = spin_out.cpu().numpy()
    assert np.isfinite(s).all() and np.array_equal(s[:1024], s[1024:2048])
