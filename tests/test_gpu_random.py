"""Seeded random calls through the C-ABI against the oracle: every collective
and algorithm, 1 to 72 ranks, empty and ragged counts, every dtype and op, in
and out of place, buffers off 16-byte alignment, checksums on and off, and
random launch options (column kernel or row kernel, tiles per work group,
group sizes, grid caps, nontemporal masks).  Bit-exact on every defined element and every row
checksum.  Case i draws everything from numpy's PCG64 seeded with 7000 + i."""

import numpy as np
import pytest

import seeded_inputs as si
from oracle.schedules import VALID
from tests.gpu_util import assert_parity

pytestmark = pytest.mark.gpu

DEFAULTS = {"exec": 0, "group_tiles": 0, "max_grid": 0, "nontemporal": -1, "reverse": 1, "col_tiles": 0}
OPTION_CHOICES = {"exec": [0, 0, 0, 1, 2], "group_tiles": [0, 0, 0, 1, 2, 8], "max_grid": [0, 0, 0, 3, 64, 1000],
                  "nontemporal": [-1, -1, 0, 1, 5, 7], "reverse": [0, 1], "col_tiles": [0, 0, 1, 3]}
PIPELINED = ("chain_pipe", "binomial_pipe", "bidir_ring")


@pytest.fixture(autouse=True)
def _options(gpu_device):
    import collective_communication_algorithms_amd as coll
    yield
    for k, v in DEFAULTS.items():
        coll.coll_set_option(k, v)


def draw(i):
    rng = np.random.default_rng(7000 + i)
    kind = str(rng.choice(sorted(VALID)))
    algo = str(rng.choice(VALID[kind]))
    if algo == "rhd" and kind in ("reducescatter", "allgather"):
        N = int(2 ** rng.integers(0, 5))
    else:
        N = int(rng.integers(1, 25)) if rng.random() < 0.9 else int(rng.integers(25, 73))
    u = rng.random()
    count = 0 if u < 0.03 else int(rng.integers(1, 300)) if u < 0.4 else int(rng.integers(300, 20000)) \
        if u < 0.9 else int(rng.integers(20000, 300000))
    if kind == "alltoall":
        count -= count % N
    dtype = str(rng.choice(["int32", "uint8", "float32", "bfloat16"]))
    op = str(rng.choice(["sum", "max", "min"]))
    root = int(rng.integers(0, N))
    k = int(rng.integers(1, min(17, max(count, 1)) + 1)) if algo in PIPELINED else 1
    inplace = kind != "alltoall" and bool(rng.random() < 0.7)
    offset = int(rng.choice([0, 0, 0, 1, 3]))
    checksums = bool(rng.random() < 0.5)
    options = {name: int(rng.choice(vals)) for name, vals in OPTION_CHOICES.items()}
    return dict(kind=kind, algo=algo, N=N, count=count, dtype=dtype, op=op, root=root, k=k, inplace=inplace,
                offset=offset, checksums=checksums, options=options)


@pytest.mark.parametrize("i", range(400))
def test_random_call_matches_the_oracle(i):
    import collective_communication_algorithms_amd as coll
    c = draw(i)
    print("case", i, c, flush=True)
    for name, v in c["options"].items():
        coll.coll_set_option(name, v)
    a = si.rank_arrays(7000 + i, c["N"], c["count"], c["dtype"], sigma=0.02 if c["dtype"] == "bfloat16" else 1.0)
    assert_parity(c["kind"], c["algo"], a, c["dtype"], op=c["op"], root=c["root"], k=c["k"], inplace=c["inplace"],
                  checksums=c["checksums"], offset_elems=c["offset"])
