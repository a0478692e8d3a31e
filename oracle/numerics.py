"""Element semantics of the schedule rows (oracle; test infrastructure only).

A copy row moves bits.  A ``recv_and_reduce`` row (the HCCL blog's Ring
AllReduce listing names it; "集合通信算法延迟公式", Ring ReduceScatter phase:
the receiver reduces what it receives into its own chunk) computes
``dst <- dst (+) src`` elementwise, where (+) is:

  int32     sum modulo 2**32 (two's complement wrap); max / min ordinary
  uint8     sum modulo 2**8; max / min ordinary
  float32   IEEE-754 binary32 add, round to nearest even, subnormals kept
  bfloat16  both operands widened exactly to binary32, one binary32 add, then
            binary32 -> bfloat16 round to nearest even (NaN -> 0x7FC0), at every row

max picks src when src > dst, else dst; min picks src when src < dst, else dst.
The pages name SUM / MAX / MIN and the FP32 / BF16 types (HCCL blog,
hccl_allreduce parameter list) but fix no rounding rule; the one above is the
plain reading.

bfloat16 values are held as their uint16 bit patterns.
"""

from __future__ import annotations

import numpy as np

OPS = ("sum", "max", "min")


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening: a bfloat16 is the top 16 bits of a binary32."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """binary32 -> bfloat16, round to nearest, ties to even; NaN -> 0x7FC0.

    Dropping the low 16 bits of the pattern truncates toward zero in magnitude
    (the sign is separate).  Adding 0x7FFF plus the lowest kept bit before the
    shift rounds up exactly when the dropped half exceeds 0x8000, or equals it
    and the kept part is odd: round-half-to-even.  A carry out of the mantissa
    bumps the exponent, which is the correct rounding (up to infinity at the top).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r[nan] = np.uint16(0x7FC0)
    return r


def combine(dst: np.ndarray, src: np.ndarray, dtype: str, op: str) -> np.ndarray:
    """Result of one reduce row, ``dst (+) src``, in the storage type of ``dtype``."""
    if op not in OPS:
        raise ValueError(op)
    if dtype in ("int32", "uint8"):
        if op == "sum":
            ut = np.uint32 if dtype == "int32" else np.uint8
            return (dst.view(ut) + src.view(ut)).view(dst.dtype)   # unsigned add wraps
        if op == "max":
            return np.where(src > dst, src, dst)
        return np.where(src < dst, src, dst)
    if dtype == "float32":
        if op == "sum":
            return np.add(dst, src, dtype=np.float32)
        if op == "max":
            return np.where(src > dst, src, dst)
        return np.where(src < dst, src, dst)
    if dtype == "bfloat16":
        a = bf16_to_f32(dst)
        b = bf16_to_f32(src)
        if op == "sum":
            return f32_to_bf16_rne(np.add(a, b, dtype=np.float32))
        if op == "max":
            return np.where(b > a, src, dst)
        return np.where(b < a, src, dst)
    raise ValueError(dtype)


def row_checksum(region: np.ndarray) -> int:
    """Checksum of a row's destination region after the row.

    The region's bytes are read as little-endian uint32 words counted from the
    region's first byte, the last word zero-padded; the checksum is their sum
    modulo 2**64.
    """
    b = np.ascontiguousarray(region).view(np.uint8)
    pad = (-len(b)) % 4
    if pad:
        b = np.concatenate([b, np.zeros(pad, dtype=np.uint8)])
    w = b.view("<u4").astype(np.uint64)
    return int(w.sum(dtype=np.uint64)) & ((1 << 64) - 1)
