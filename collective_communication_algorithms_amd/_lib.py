"""ctypes view of libcoll.so (declarations in include/coll.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in this package.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcoll.so")

COLL_OK, COLL_ERR_INVALID_ARG, COLL_ERR_UNSUPPORTED, COLL_ERR_HIP, COLL_ERR_NO_MEMORY = range(5)
STATUS_NAMES = {0: "COLL_OK", 1: "COLL_ERR_INVALID_ARG", 2: "COLL_ERR_UNSUPPORTED", 3: "COLL_ERR_HIP",
                4: "COLL_ERR_NO_MEMORY"}

DTYPES = {"int32": 0, "uint8": 1, "float32": 2, "bfloat16": 3}
OPS = {"sum": 0, "max": 1, "min": 2}
ALGOS = {"default": 0, "ring": 1, "rhd": 2, "dbt": 3, "binomial": 4, "chain_pipe": 5, "binomial_pipe": 6,
         "pairwise": 7, "bruck": 8, "linear": 9, "scatter_allgather": 10, "auto": 11,
         "bidir_ring": 12}
KINDS = {"allreduce": 0, "reducescatter": 1, "allgather": 2, "broadcast": 3, "scatter": 4, "gather": 5,
         "alltoall": 6, "reduce": 7}
OPTIONS = {"exec": 0, "group_tiles": 1, "max_grid": 2, "nontemporal": 3, "reverse": 4, "model_alpha_ns": 5,
           "model_beta_gbps": 6, "cache_bytes": 7, "col_tiles": 8, "timing": 9, "a2a_direct": 10}
MAX_RANKS = 128

COLLECTIVES = ("coll_allreduce", "coll_reducescatter", "coll_allgather", "coll_broadcast", "coll_scatter",
               "coll_gather", "coll_alltoall", "coll_reduce", "coll_allreduce_noalloc")


class CollRow(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int32), ("src", ctypes.c_int32), ("dst", ctypes.c_int32),
                ("reduce", ctypes.c_uint8), ("local", ctypes.c_uint8), ("from_send", ctypes.c_uint8),
                ("staged", ctypes.c_uint8), ("src_off", ctypes.c_int64), ("dst_off", ctypes.c_int64),
                ("n", ctypes.c_int64)]


class CollCounts(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int64), ("rows", ctypes.c_int64), ("crit_bytes", ctypes.c_int64),
                ("hbm_bytes", ctypes.c_int64), ("moved_bytes", ctypes.c_int64), ("round_trips", ctypes.c_int64)]


class CollError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python -m collective_communication_algorithms_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    ptrs = ctypes.POINTER(ctypes.c_void_p)
    for name in COLLECTIVES:
        f = getattr(lib, name)
        f.argtypes = [ptrs, ptrs, ctypes.c_int, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                      ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        f.restype = ctypes.c_int
    lib.coll_plan.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_size_t, ctypes.c_int,
                              ctypes.c_int, ctypes.c_int, ctypes.POINTER(CollRow), ctypes.POINTER(ctypes.c_size_t),
                              ctypes.POINTER(CollCounts)]
    lib.coll_plan.restype = ctypes.c_int
    lib.coll_get_stats.argtypes = [ctypes.POINTER(CollCounts)]
    lib.coll_get_stats.restype = ctypes.c_int
    lib.coll_set_checksums.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.coll_set_checksums.restype = ctypes.c_int
    lib.coll_set_option.argtypes = [ctypes.c_int, ctypes.c_int64]
    lib.coll_set_option.restype = ctypes.c_int
    lib.coll_last_kernel_ms.argtypes = [ctypes.POINTER(ctypes.c_float)]
    lib.coll_last_kernel_ms.restype = ctypes.c_int
    lib.coll_check.argtypes = [ctypes.c_void_p]
    lib.coll_check.restype = ctypes.c_int
    lib.coll_get_option.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int64)]
    lib.coll_get_option.restype = ctypes.c_int
    lib.coll_cache_info.argtypes = [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
    lib.coll_cache_info.restype = ctypes.c_int
    lib.coll_status_string.argtypes = [ctypes.c_int]
    lib.coll_status_string.restype = ctypes.c_char_p
    lib.coll_last_error.argtypes = []
    lib.coll_last_error.restype = ctypes.c_char_p
    lib.coll_finalize.argtypes = []
    lib.coll_finalize.restype = None
    lib.coll_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.coll_calib_copy.restype = ctypes.c_int
    lib.coll_calib_spin.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
    lib.coll_calib_spin.restype = ctypes.c_int
    lib.coll_calib_add.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_void_p]
    lib.coll_calib_add.restype = ctypes.c_int
    lib.coll_calib_pattern.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.POINTER(ctypes.c_void_p),
                                       ctypes.c_int, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    lib.coll_calib_pattern.restype = ctypes.c_int
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != COLL_OK:
        raise CollError(status, load().coll_last_error().decode(errors="replace"))
