"""CPU oracle for collective-communication schedules: TEST INFRASTRUCTURE ONLY.

Plain, slow and deliberately obvious.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import anything from here; the
product path (the C-ABI library and its Python binding) never does, and shares no
code, header, table or helper with this package.

What it computes, from the pages it follows:
  * "一对多通信：Broadcast 与 Scatter" (tier6-model.pages.dev): Broadcast and
    Scatter semantics (eq:onetoall-bcast-semantic, eq:onetoall-scatter-semantic),
    chain / binomial / chunked-pipeline Broadcast, binomial Scatter, and Gather as
    Scatter with the data flow reversed (eq:onetoall-gather-scatter-duality).
  * "集合通信算法延迟公式" (t6page.pages.dev): Ring ReduceScatter + AllGather
    AllReduce, Recursive Halving-Doubling, Double Binary Tree, Pairwise and Bruck
    AllToAll, Tree Reduce.
  * The HCCL blog (agent.csdn.net): the Ring AllReduce chunk walk and the
    ``recv_and_reduce`` row, used for chunk indices only.

Modules
  numerics   element semantics of a reduce row per dtype, and the row checksum
  schedules  one step-by-step row generator per (collective, algorithm)
  simulate   the snapshot-per-step executor and one function per collective

Every function here is pinned by a ``-m "not gpu"`` test against something other
than itself: the pages' printed 8-node tables, closed-form step and byte counts,
brute-force semantics on tiny inputs, torch's bfloat16 conversion, and
fp64 error bounds.  ``run_plan_columns`` is pinned to ``run_plan`` on whole
buffers, ``defined_regions`` to the buffer contract written out per element and
to the collectives' definitions, and the uint8 element rule to every pair of
bytes (tests/test_oracle_columns_regions.py, each with a planted mistake it
catches).  No function is left "parity unpinned".
"""

from . import numerics, schedules, simulate  # noqa: F401
from .simulate import (allreduce, reducescatter, allgather, broadcast, scatter,  # noqa: F401
                       gather, alltoall, reduce, run_plan)
from .schedules import make_plan  # noqa: F401
