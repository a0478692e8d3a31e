"""The calibration kernels that give the column kernel its achievable
ceilings compute what they claim, so that their rates are rates of real
work: the copy and add streams, and every access pattern of
coll_calib_pattern (each store buffer ends with the u32 word sum, per 16-byte
unit, of the load buffers; a fill writes every unit), with and without a cap
on the work groups per CU."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def test_copy_and_add_streams(gpu_device):
    import torch
    import collective_communication_algorithms_amd as coll
    g = torch.Generator(device="cpu").manual_seed(5)
    a = torch.randn(1 << 18, generator=g).to(gpu_device)
    b = torch.randn(1 << 18, generator=g).to(gpu_device)
    c = torch.full_like(a, float("nan"))
    coll.coll_calib_copy(c, a)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int32), a.view(torch.int32))
    coll.coll_calib_add(c, a, b)
    torch.cuda.synchronize()
    assert torch.equal(c, a + b)


@pytest.mark.parametrize("nl,ns,groups", [(0, 1, 0), (8, 8, 0), (8, 8, 4), (8, 8, 32), (8, 1, 0), (1, 7, 0),
                                          (64, 1, 3), (1, 63, 0)])
def test_access_patterns(gpu_device, nl, ns, groups):
    import torch
    import collective_communication_algorithms_amd as coll
    nbuf = max(nl, ns + (1 if nl == 1 else 0), 1)
    words = 1024 + 64                                      # 4 KiB + 256 B: not a multiple of 1 KiB
    g = np.random.default_rng(nl * 100 + ns)
    host = g.integers(0, 2 ** 32, size=(nbuf, words), dtype=np.uint64).astype(np.uint32)
    t = torch.from_numpy(host.view(np.int32)).to(gpu_device)
    views = list(t)
    with pytest.raises(coll.CollError):
        coll.coll_calib_pattern(views[:nl], views[:ns])    # 4,352 bytes per buffer
    t = torch.from_numpy(host[:, :1024].copy().view(np.int32)).to(gpu_device)   # 4 KiB per buffer
    views = list(t)
    in_place = nl == ns
    loads = views[:nl]
    stores = views[:ns] if in_place else (views[nbuf - ns:] if nl else views[:ns])
    coll.coll_calib_pattern(loads, stores, groups_per_cu=groups)
    torch.cuda.synchronize()
    got = t.cpu().numpy().view(np.uint32)
    src = host[:, :1024]
    if nl:
        want = src[:nl].astype(np.uint64).sum(axis=0).astype(np.uint32)   # u32 wrap-around sum
        for k in range(ns):
            row = k if in_place else (nbuf - ns + k)
            assert np.array_equal(got[row], want), (nl, ns, k)
        if not in_place:
            for r in range(nbuf - ns):
                assert np.array_equal(got[r], src[r]), (nl, ns, "load buffer changed", r)
    else:
        assert not np.array_equal(got[0], src[0])
        units = got[0].reshape(-1, 4)
        lanes = np.arange(units.shape[0]) % 64
        wgs = np.arange(units.shape[0]) // 64
        assert np.array_equal(units[:, 0], lanes) and np.array_equal(units[:, 1], wgs)
