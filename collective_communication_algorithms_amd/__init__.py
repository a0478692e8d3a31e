"""Collective-communication schedules over N virtual ranks in one MI355X's HBM.

The work runs in libcoll.so (HIP kernels for gfx950 behind the C ABI of
include/coll.h); this package only marshals arguments to it.
"""

from .api import (COLLECTIVE_FNS, CollError, coll_allgather, coll_allreduce, coll_allreduce_noalloc, coll_alltoall,  # noqa: F401
                  coll_broadcast, coll_cache_info, coll_calib_add, coll_check, coll_calib_copy, coll_calib_pattern, coll_calib_spin,
                  coll_finalize,
                  coll_gather, coll_get_option, coll_get_stats, coll_last_kernel_ms, coll_plan, coll_reduce, coll_reducescatter,
                  coll_scatter, coll_set_checksums, coll_set_option)
from . import model  # noqa: F401
