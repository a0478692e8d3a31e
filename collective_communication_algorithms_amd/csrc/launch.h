// Host entry points of the device kernels (defined in kernels.hip).
#pragma once

#include <hip/hip_runtime_api.h>

#include "coll.h"
#include "device_types.h"

namespace coll {

// fine: the variant for lists of small pieces; fwd: the variant that keeps
// stored units in registers for ITEM_SRC_FWD / ITEM_DSRC_FWD entries
hipError_t launch_rows(const RowsArgs& a, int dtype, int op, bool cks, uint32_t nt, bool fine, bool fwd,
                       uint32_t grid, hipStream_t stream);
// hoist: descriptors read once per group, loads unconditional (groups over 32 rows)
hipError_t launch_perm(const PermArgs& a, int unit, int slots, bool hoist, bool cks, uint32_t grid,
                       hipStream_t stream);

hipError_t launch_fill_u64(uint64_t* p, uint64_t n, uint64_t value, hipStream_t stream);
// nrows rows of a.row_bytes (a multiple of 16), a.wgs_per_row 1 KiB tiles each;
// with cks one partial checksum slot per work group
hipError_t launch_copy_rows(const CopyRowsArgs& a, uint64_t nrows, bool cks, bool nt, hipStream_t stream);
// out[r] = the u64 wrap-sum of partial[r * SUM_LANES .. r * SUM_LANES + SUM_LANES), r < nrows;
// the slots read are set back to zero
hipError_t launch_fold_sums(uint64_t* partial, uint64_t* out, uint64_t nrows, hipStream_t stream);
// (nloads, nstores) in {(0,1), (8,8), (8,1), (1,7), (64,1), (1,63)}; p.send[0 .. nloads)
// the load buffers, p.recv[0 .. nstores) the store buffers; bytes a multiple of 1024;
// lds_bytes of LDS reserved per work group (unused; caps the groups per CU)
hipError_t launch_calib_pattern(const RankPtrs& p, int nloads, int nstores, uint64_t bytes, uint32_t lds_bytes,
                                hipStream_t stream);
hipError_t launch_calib(void* dst, const void* a, const void* b, uint64_t bytes, hipStream_t stream);
// the C ABI's error reporting (the message coll_last_error returns), for entry
// points outside abi.cpp
coll_status_t report_error(coll_status_t st, const char* msg);
coll_status_t report_hip_error(hipError_t e, const char* what);
hipError_t launch_spin(float* out, uint32_t iters, uint32_t grid, hipStream_t stream);
// column kernel: the variant of (unit, leaves, accs) (ColVariant), nontemporal
// loads and stores when `nt`; one work group of COL_THREADS per ColWork; the
// first nranks (1 .. COL_THREADS) addresses of a.p are passed
hipError_t launch_col(const ColArgs& a, int nranks, int dtype, int op, int unit, int leaves, int accs, bool batched,
                      bool capped, bool nt, uint32_t grid, hipStream_t stream);
// out[r] = the sum of the partial slots row r's ColRefs name, r < nrows, by way
// of tmp (nrows * COL_FOLD_SLICES slots)
hipError_t launch_col_fold(const ColRef* refs, const uint32_t* row_off, const uint64_t* partial, uint64_t* tmp,
                           uint64_t* out, uint64_t nrows, hipStream_t stream);
// out[r] = src[idx[r]] for r < n (row checksums copied from others).
hipError_t launch_gather_sums(const uint32_t* idx, const uint64_t* src, uint64_t* out, uint64_t n,
                              hipStream_t stream);
// The address of the current device's allocation-free scratch
// (COLL_NOALLOC_SCRATCH_BYTES, 256-byte aligned), taken once per device.
hipError_t noalloc_scratch(void** out);
int rows_blocks_per_cu(int dtype, int op, bool cks, uint32_t nt);
int perm_blocks_per_cu(int unit, int slots, bool hoist, bool cks, bool nt);

}  // namespace coll
