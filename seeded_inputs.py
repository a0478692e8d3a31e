"""Seeded synthetic rank buffers shared by the tests, the bench and the smoke check.

This module draws random numbers and nothing else: it holds none of the
collectives' arithmetic (no reduction, no rounding rule of the method, no
schedule).  Both the CPU oracle's callers and the GPU path's callers take their
inputs from here, so the two sides see identical bytes.

Recipe: rank r of workload w uses numpy ``Generator(PCG64(1000 * w + r))``.
  int32   uniform integers in [lo, hi] inclusive
  uint8   uniform in [0, 255]
  float32 standard normal scaled by sigma
  bf16    float32 standard normal scaled by sigma, converted to bfloat16 by
          torch's CPU conversion (a library routine), stored as uint16 bits;
          plant_bf16_specials writes NaN / infinity / extreme patterns into
          seeded places of such buffers

Large device-resident workloads use ``device_rank_tensors``: torch's own
seeded generator on the device, same seeds.  Those inputs come from PyTorch's
RNG, never from the HIP path under test.
"""

from __future__ import annotations

import numpy as np

DTYPES = ("int32", "uint8", "float32", "bfloat16")
ITEMSIZE = {"int32": 4, "uint8": 1, "float32": 4, "bfloat16": 2}
# numpy storage type of each dtype (bf16 is held as its raw 16-bit pattern)
STORAGE = {"int32": np.int32, "uint8": np.uint8, "float32": np.float32,
           "bfloat16": np.uint16}


def seed_for(workload: int, rank: int) -> int:
    return 1000 * int(workload) + int(rank)


def _bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def rank_array(workload: int, rank: int, count: int, dtype: str,
               sigma: float = 1.0, lo: int = -(1 << 20), hi: int = 1 << 20) -> np.ndarray:
    """One rank's buffer of ``count`` elements (numpy storage type)."""
    rng = np.random.Generator(np.random.PCG64(seed_for(workload, rank)))
    if dtype == "int32":
        return rng.integers(lo, hi, size=count, endpoint=True, dtype=np.int32)
    if dtype == "uint8":
        return rng.integers(0, 255, size=count, endpoint=True, dtype=np.uint8)
    if dtype == "float32":
        x = rng.standard_normal(count, dtype=np.float32)
        return (x * np.float32(sigma)).astype(np.float32)
    if dtype == "bfloat16":
        x = rng.standard_normal(count, dtype=np.float32) * np.float32(sigma)
        return _bf16_bits_from_f32(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def rank_arrays(workload: int, nranks: int, count: int, dtype: str, **kw) -> list:
    return [rank_array(workload, r, count, dtype, **kw) for r in range(nranks)]


# bfloat16 bit patterns outside the normal range of the other inputs: quiet and
# signalling NaNs of either sign with payloads, the infinities, the largest
# finite values (two of them add past the range), subnormals and signed zeros
BF16_SPECIALS = np.array([0x7FC1, 0xFFC0, 0x7F81, 0xFFFF, 0x7FA5, 0x7F80, 0xFF80, 0x7F7F, 0xFF7F, 0x7F7F,
                          0x0001, 0x8001, 0x007F, 0x8000, 0x0000], dtype=np.uint16)


def plant_bf16_specials(arrays: list, seed: int, nplant: int) -> list:
    """Copies of bfloat16 rank buffers with ``nplant`` entries of BF16_SPECIALS
    written at seeded (rank, position) pairs, so that most of the buffer stays
    ordinary and a few places meet NaN, infinity and overflow."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = [np.array(a, dtype=np.uint16, copy=True) for a in arrays]
    ranks = rng.integers(0, len(out), size=nplant)
    pos = rng.integers(0, len(out[0]), size=nplant)
    vals = rng.choice(BF16_SPECIALS, size=nplant)
    for r, i, v in zip(ranks, pos, vals):
        out[int(r)][int(i)] = v
    return out


def to_torch_dtype(dtype: str):
    import torch
    return {"int32": torch.int32, "uint8": torch.uint8, "float32": torch.float32,
            "bfloat16": torch.bfloat16}[dtype]


def host_to_tensor(a: np.ndarray, dtype: str, device):
    """numpy storage array -> torch tensor of the collective's dtype on ``device``."""
    import torch
    if dtype == "bfloat16":
        t = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def tensor_to_host(t, dtype: str) -> np.ndarray:
    """torch tensor -> numpy storage array (bf16 as uint16 bits)."""
    import torch
    t = t.detach().to("cpu").contiguous()
    if dtype == "bfloat16":
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def device_rank_tensors(workload: int, nranks: int, count: int, dtype: str, device,
                        sigma: float = 1.0, lo: int = -(1 << 20), hi: int = 1 << 20,
                        out=None):
    """Large inputs drawn on the device by torch's seeded generator.

    Returns a list of ``nranks`` 1-D tensors; if ``out`` is a (nranks, count)
    tensor the values are written into its rows.
    """
    import torch
    tdt = to_torch_dtype(dtype)
    res = []
    for r in range(nranks):
        g = torch.Generator(device=device)
        g.manual_seed(seed_for(workload, r))
        if dtype == "int32":
            x = torch.randint(lo, hi + 1, (count,), generator=g, device=device, dtype=torch.int32)
        elif dtype == "uint8":
            x = torch.randint(0, 256, (count,), generator=g, device=device, dtype=torch.uint8)
        else:
            x = torch.randn(count, generator=g, device=device, dtype=torch.float32)
            x.mul_(sigma)
            x = x.to(tdt)
        if out is not None:
            out[r].copy_(x)
            res.append(out[r])
        else:
            res.append(x)
        del g
    return res
