"""Python names for the C ABI of include/coll.h: argument marshalling only.

Rank buffers are torch tensors on one GPU (PyTorch supplies device memory and
the stream).  Every step of every collective runs in libcoll.so's kernels.
"""

from __future__ import annotations

import ctypes

from . import _lib
from ._lib import ALGOS, DTYPES, KINDS, OPS, OPTIONS, CollCounts, CollError, CollRow, check  # noqa: F401

_TORCH_DT = None


def _dtype_name(t) -> str:
    global _TORCH_DT
    import torch
    if _TORCH_DT is None:
        _TORCH_DT = {torch.int32: "int32", torch.uint8: "uint8", torch.float32: "float32",
                     torch.bfloat16: "bfloat16"}
    try:
        return _TORCH_DT[t.dtype]
    except KeyError:
        raise CollError(_lib.COLL_ERR_INVALID_ARG, f"unsupported dtype {t.dtype}") from None


def _code(table, name, what):
    try:
        return table[name]
    except (KeyError, TypeError):
        raise CollError(_lib.COLL_ERR_INVALID_ARG, f"unknown {what} {name!r}") from None


def _ptr_array(tensors):
    arr = (ctypes.c_void_p * len(tensors))()
    for i, t in enumerate(tensors):
        arr[i] = t.data_ptr()
    return arr


def _check_tensors(send, recv):
    """Every rank buffer a contiguous GPU tensor of one device, dtype and size
    (the C ABI trusts `count` elements behind every pointer)."""
    if len(send) == 0:
        raise CollError(_lib.COLL_ERR_INVALID_ARG, "no rank buffers")
    if recv is not None and len(recv) != len(send):
        raise CollError(_lib.COLL_ERR_INVALID_ARG, "one receive buffer per rank")
    t0 = send[0]
    if not t0.is_cuda:
        raise CollError(_lib.COLL_ERR_INVALID_ARG, "rank buffers must be GPU tensors")
    dev, dt, n = t0.get_device(), t0.dtype, t0.numel()
    for group in (send, recv or ()):
        for t in group:
            if t.get_device() != dev or t.dtype != dt or t.numel() != n or not t.is_contiguous():
                raise CollError(_lib.COLL_ERR_INVALID_ARG,
                                "rank buffers must share device, dtype and size, and be contiguous")


def _stream_handle(device, stream):
    import torch
    idx = device.index if isinstance(device, torch.device) else int(device)
    if stream is None:
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)   # skips building a Stream object
        return ctypes.c_void_p(raw(idx) if raw is not None else torch.cuda.current_stream(idx).cuda_stream)
    if getattr(stream, "device_index", idx) != idx:
        raise CollError(_lib.COLL_ERR_INVALID_ARG, "the stream belongs to another device than the rank buffers")
    return ctypes.c_void_p(stream.cuda_stream)


def _collective(name, send, recv, op, algo, root, chunks, stream):
    import torch
    op_code, algo_code = _code(OPS, op, "op"), _code(ALGOS, algo, "algorithm")
    _check_tensors(send, recv)
    fn = getattr(_lib.load(), name)
    idx = send[0].get_device()
    args = (_ptr_array(send), _ptr_array(recv) if recv is not None else None, len(send), send[0].numel(),
            DTYPES[_dtype_name(send[0])], op_code, algo_code, int(root), int(chunks))
    # the library works on the current device: make it the tensors' one
    if torch._C._cuda_getDevice() == idx:
        st = fn(*args, _stream_handle(idx, stream))
    else:
        with torch.cuda.device(idx):
            st = fn(*args, _stream_handle(idx, stream))
    check(st)


def coll_allreduce(send, recv=None, op="sum", algo="default", root=0, chunks=1, stream=None):
    _collective("coll_allreduce", send, recv, op, algo, root, chunks, stream)


def coll_reducescatter(send, recv=None, op="sum", algo="default", root=0, chunks=1, stream=None):
    _collective("coll_reducescatter", send, recv, op, algo, root, chunks, stream)


def coll_allgather(send, recv=None, op="sum", algo="default", root=0, chunks=1, stream=None):
    _collective("coll_allgather", send, recv, op, algo, root, chunks, stream)


def coll_broadcast(send, recv=None, op="sum", algo="default", root=0, chunks=1, stream=None):
    _collective("coll_broadcast", send, recv, op, algo, root, chunks, stream)


def coll_scatter(send, recv=None, op="sum", algo="default", root=0, chunks=1, stream=None):
    _collective("coll_scatter", send, recv, op, algo, root, chunks, stream)


def coll_gather(send, recv=None, op="sum", algo="default", root=0, chunks=1, stream=None):
    _collective("coll_gather", send, recv, op, algo, root, chunks, stream)


def coll_alltoall(send, recv, op="sum", algo="default", root=0, chunks=1, stream=None):
    _collective("coll_alltoall", send, recv, op, algo, root, chunks, stream)


def coll_reduce(send, recv=None, op="sum", algo="default", root=0, chunks=1, stream=None):
    _collective("coll_reduce", send, recv, op, algo, root, chunks, stream)


def coll_allreduce_noalloc(send, recv=None, op="sum", algo="default", root=0, chunks=1, stream=None):
    """coll_allreduce without any device allocation (the library's fixed
    scratch array; the column kernel only)."""
    _collective("coll_allreduce_noalloc", send, recv, op, algo, root, chunks, stream)


COLLECTIVE_FNS = {"allreduce": coll_allreduce, "reducescatter": coll_reducescatter, "allgather": coll_allgather,
                  "broadcast": coll_broadcast, "scatter": coll_scatter, "gather": coll_gather,
                  "alltoall": coll_alltoall, "reduce": coll_reduce}


def coll_plan(kind, algo, nranks, count, dtype, root=0, chunks=1):
    """(rows, counts) of the in-place schedule; rows are tuples
    (step, src, dst, src_off, dst_off, n, reduce, local, from_send, staged)."""
    lib = _lib.load()
    k, a, d = _code(KINDS, kind, "collective"), _code(ALGOS, algo, "algorithm"), _code(DTYPES, dtype, "dtype")
    n = ctypes.c_size_t(0)
    counts = CollCounts()
    check(lib.coll_plan(k, a, nranks, count, d, root, chunks, None, ctypes.byref(n), None))
    rows = (CollRow * max(n.value, 1))()
    check(lib.coll_plan(k, a, nranks, count, d, root, chunks, rows, ctypes.byref(n), ctypes.byref(counts)))
    out = [(r.step, r.src, r.dst, r.src_off, r.dst_off, r.n, r.reduce, r.local, r.from_send, r.staged)
           for r in rows[:n.value]]
    return out, {"steps": counts.steps, "rows": counts.rows, "crit_bytes": counts.crit_bytes,
                 "hbm_bytes": counts.hbm_bytes, "moved_bytes": counts.moved_bytes,
                 "round_trips": counts.round_trips}


def coll_get_stats():
    lib = _lib.load()
    c = CollCounts()
    check(lib.coll_get_stats(ctypes.byref(c)))
    return {"steps": c.steps, "rows": c.rows, "crit_bytes": c.crit_bytes, "hbm_bytes": c.hbm_bytes,
            "moved_bytes": c.moved_bytes, "round_trips": c.round_trips}


def coll_set_checksums(sums=None):
    """``sums``: an int64 GPU tensor (one slot per schedule row), or None to stop."""
    lib = _lib.load()
    if sums is None:
        check(lib.coll_set_checksums(None, 0))
    else:
        check(lib.coll_set_checksums(ctypes.c_void_p(sums.data_ptr()), sums.numel()))


def coll_set_option(name, value):
    check(_lib.load().coll_set_option(_code(OPTIONS, name, "option"), int(value)))


def coll_last_kernel_ms() -> float:
    """Milliseconds between the HIP events around the data-moving kernels of
    this thread's last call made with the "timing" option on (waits for it)."""
    ms = ctypes.c_float()
    check(_lib.load().coll_last_kernel_ms(ctypes.byref(ms)))
    return float(ms.value)


def coll_check(stream=None, device=None):
    """Wait for the stream's work (the current stream of ``device``, default
    the current device, when None) and raise CollError if it failed."""
    import torch
    if stream is None:
        dev = torch.cuda.current_device() if device is None else device
        handle = _stream_handle(dev, None)
    else:
        handle = ctypes.c_void_p(stream.cuda_stream)
    check(_lib.load().coll_check(handle))


def coll_get_option(name):
    v = ctypes.c_int64(0)
    check(_lib.load().coll_get_option(_code(OPTIONS, name, "option"), ctypes.byref(v)))
    return v.value


def coll_cache_info():
    """(schedules cached, device bytes they hold)."""
    n, b = ctypes.c_int64(0), ctypes.c_int64(0)
    check(_lib.load().coll_cache_info(ctypes.byref(n), ctypes.byref(b)))
    return n.value, b.value


def coll_finalize():
    _lib.load().coll_finalize()


def coll_calib_copy(dst, src, stream=None):
    check(_lib.load().coll_calib_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                                      dst.numel() * dst.element_size(), _stream_handle(dst.device, stream)))


def coll_calib_spin(out, iters, grid, stream=None):
    """``out``: a float32 GPU tensor of at least grid * 256 elements."""
    if out.dtype.itemsize != 4 or out.numel() < int(grid) * 256:
        raise CollError(_lib.COLL_ERR_INVALID_ARG, "out needs grid * 256 float32 elements")
    check(_lib.load().coll_calib_spin(ctypes.c_void_p(out.data_ptr()), int(iters), int(grid),
                                      _stream_handle(out.device, stream)))


def coll_calib_pattern(loads, stores, groups_per_cu=0, stream=None):
    """The column kernel's access pattern over GPU tensors: every tile of
    each tensor in ``loads`` summed and stored to each tensor in ``stores``
    (all of one size in bytes; see include/coll.h for the supported counts),
    with at most ``groups_per_cu`` work groups per CU when nonzero."""
    ts = list(loads) + list(stores)
    nbytes = ts[0].numel() * ts[0].element_size()
    if any(t.numel() * t.element_size() != nbytes for t in ts):
        raise CollError(_lib.COLL_ERR_INVALID_ARG, "calibration buffers must all have one size")
    lp = (ctypes.c_void_p * max(len(loads), 1))(*[t.data_ptr() for t in loads])
    sp = (ctypes.c_void_p * len(stores))(*[t.data_ptr() for t in stores])
    check(_lib.load().coll_calib_pattern(lp if loads else None, len(loads), sp, len(stores), nbytes, int(groups_per_cu),
                                         _stream_handle(ts[0].device, stream)))


def coll_calib_add(dst, a, b, stream=None):
    check(_lib.load().coll_calib_add(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(a.data_ptr()),
                                     ctypes.c_void_p(b.data_ptr()), dst.numel() * dst.element_size(),
                                     _stream_handle(dst.device, stream)))
