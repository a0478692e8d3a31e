"""Seeded random calls at large sizes (column spaces of 8 to 96 MiB, where
the large-grid launch shapes apply: the cache window, the copy-only rule, and
groups split at row boundaries when every group has a work group of its own),
checked on sampled columns the oracle computes exactly (every collective but
AllToAll keeps each element at its column).  Case i draws everything from
numpy's PCG64 seeded with 9000 + i; inputs come from torch's seeded device
generator."""

import numpy as np
import pytest

import seeded_inputs as si
from oracle.schedules import VALID, make_plan
from oracle.simulate import defined_regions, run_plan_columns
from tests.test_gpu_full import gather_cols, sample_columns

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

PIPELINED = ("chain_pipe", "binomial_pipe", "bidir_ring")
KINDS = ["allreduce", "reducescatter", "allgather", "broadcast", "scatter", "gather", "reduce"]


@pytest.fixture(autouse=True)
def _defaults(gpu_device):
    import collective_communication_algorithms_amd as coll
    for k, v in {"exec": 0, "group_tiles": 0, "max_grid": 0, "nontemporal": -1, "reverse": 1}.items():
        coll.coll_set_option(k, v)
    yield


def draw(i):
    rng = np.random.default_rng(9000 + i)
    kind = str(rng.choice(KINDS))
    algo = str(rng.choice(VALID[kind]))
    N = int(2 ** rng.integers(1, 5)) if (algo == "rhd" and kind in ("reducescatter", "allgather")) \
        else int(rng.integers(2, 21))
    dtype = str(rng.choice(["int32", "uint8", "float32", "bfloat16"]))
    sz = si.ITEMSIZE[dtype]
    count = int(rng.integers(8 << 20, 96 << 20)) // sz
    op = str(rng.choice(["sum", "max", "min"]))
    root = int(rng.integers(0, N))
    k = int(rng.integers(1, 18)) if algo in PIPELINED else 1
    inplace = bool(rng.random() < 0.7)
    return dict(kind=kind, algo=algo, N=N, count=count, dtype=dtype, op=op, root=root, k=k, inplace=inplace)


@pytest.mark.parametrize("i", range(32))
def test_random_large_call_matches_the_oracle_on_sampled_columns(i):
    import torch
    import collective_communication_algorithms_amd as coll
    c = draw(i)
    print("case", i, c, flush=True)
    N, count, dtype = c["N"], c["count"], c["dtype"]
    dev = torch.device("cuda:0")
    buf = torch.empty((N, count), dtype=si.to_torch_dtype(dtype), device=dev)
    send = si.device_rank_tensors(9000 + i, N, count, dtype, dev, sigma=0.02 if dtype == "bfloat16" else 1.0,
                                  out=buf)
    recv = None
    if not c["inplace"]:
        rbuf = torch.empty_like(buf)
        rbuf.view(torch.uint8).fill_(0x5A)
        recv = list(rbuf)
    cols = sample_columns(count, N)
    before = gather_cols(send, cols, dtype)
    coll.COLLECTIVE_FNS[c["kind"]](send, recv, op=c["op"], algo=c["algo"], root=c["root"], chunks=c["k"])
    torch.cuda.synchronize()
    after = gather_cols(recv if recv is not None else send, cols, dtype)
    plan = make_plan(c["kind"], c["algo"], N, count, c["root"], c["k"])
    want = run_plan_columns(plan, dtype, c["op"], cols, before)
    for r, regs in enumerate(defined_regions(c["kind"], N, count, c["root"])):
        for lo, hi in regs:
            m = (cols >= lo) & (cols < hi)
            assert np.array_equal(after[r][m].view(np.uint8), want[r][m].view(np.uint8)), (i, r)
    del buf, send, recv
    torch.cuda.empty_cache()
