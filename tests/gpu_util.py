"""Helpers for the GPU parity tests: run a collective through the C-ABI library
and compare it with the oracle on the same seeded inputs."""

from __future__ import annotations

import numpy as np

import seeded_inputs as si
from oracle.schedules import make_plan
from oracle.simulate import defined_regions, run_plan

DEV = "cuda:0"


def _device_copy(a, dtype, offset_elems):
    import torch
    t = si.host_to_tensor(a, dtype, DEV)
    if offset_elems:
        big = torch.zeros(len(a) + offset_elems + 64, dtype=t.dtype, device=DEV)
        big[offset_elems:offset_elems + len(a)] = t
        t = big[offset_elems:offset_elems + len(a)]
    return t


def gpu_run(kind, algo, arrays, dtype, op="sum", root=0, k=1, inplace=True, checksums=False, offset_elems=0):
    """Run one collective on cuda:0; returns (receive buffers on the host, checksums or None)."""
    import torch
    import collective_communication_algorithms_amd as coll
    send = [_device_copy(a, dtype, offset_elems) for a in arrays]
    recv = None
    if not inplace or kind == "alltoall":
        recv = []
        for s in send:
            r = torch.empty(s.numel() + offset_elems + 64, dtype=s.dtype, device=DEV)
            r.view(torch.uint8).fill_(0x5A)          # garbage the collective must overwrite
            recv.append(r[offset_elems:offset_elems + s.numel()])
    sums = None
    if checksums:
        rows, _ = coll.coll_plan(kind, algo, len(arrays), len(arrays[0]), dtype, root, k)
        sums = torch.full((max(len(rows), 1),), -1, dtype=torch.int64, device=DEV)
        coll.coll_set_checksums(sums)
    try:
        coll.COLLECTIVE_FNS[kind](send, recv, op=op, algo=algo, root=root, chunks=k)
    finally:
        if checksums:
            coll.coll_set_checksums(None)
    torch.cuda.synchronize()
    out = recv if recv is not None else send
    host = [si.tensor_to_host(t, dtype) for t in out]
    cks = sums.cpu().numpy().view(np.uint64).copy() if checksums else None
    return host, cks


def assert_parity(kind, algo, arrays, dtype, op="sum", root=0, k=1, inplace=True, checksums=False,
                  offset_elems=0):
    """GPU result == oracle result, bit for bit, on every element the collective
    defines; with ``checksums`` every row's checksum equals the oracle's."""
    import collective_communication_algorithms_amd as coll
    N, count = len(arrays), len(arrays[0])
    got, cks = gpu_run(kind, algo, arrays, dtype, op, root, k, inplace, checksums, offset_elems)
    plan = make_plan(kind, algo, N, count, root, k)
    want, wsums = run_plan(plan, dtype, op, arrays, trace=True)
    for i, regs in enumerate(defined_regions(kind, N, count, root)):
        for lo, hi in regs:
            g = got[i][lo:hi].view(np.uint8)
            w = want[i][lo:hi].view(np.uint8)
            if not np.array_equal(g, w):
                bad = np.nonzero(got[i][lo:hi] != want[i][lo:hi])[0]
                raise AssertionError(f"{kind}/{algo} {dtype} N={N} count={count} root={root} k={k} "
                                     f"inplace={inplace}: rank {i} differs at {len(bad)} elements, "
                                     f"first {lo + bad[:5]}")
    if checksums:
        rows, _ = coll.coll_plan(kind, algo, N, count, dtype, root, k)
        want_by_row = {}
        idx = 0
        for st, srows in enumerate(plan.steps):
            for r in srows:
                want_by_row[(st, r.src, r.dst, r.src_off, r.dst_off, r.n)] = wsums[idx]
                idx += 1
        for j, r in enumerate(rows):
            key = r[:6]
            assert int(cks[j]) == want_by_row[key], (kind, algo, j, r, int(cks[j]), want_by_row[key])
    return got, want
