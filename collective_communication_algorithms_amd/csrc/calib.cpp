// The calibration entry points of the C ABI: plain streams, the column
// kernel's access patterns without programs, and a register-only stand-in
// for compute.  They share nothing with the collectives but error reporting.
#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "coll.h"
#include "device_types.h"
#include "launch.h"

using namespace coll;

namespace {

coll_status_t calib(void* dst, const void* a, const void* b, size_t bytes, void* stream) {
  if (!dst || !a) return report_error(COLL_ERR_INVALID_ARG, "NULL buffer");
  if (bytes % 16 || (reinterpret_cast<uint64_t>(dst) | reinterpret_cast<uint64_t>(a) | reinterpret_cast<uint64_t>(b)) % 16)
    return report_error(COLL_ERR_INVALID_ARG, "calibration needs 16-byte sizes and pointers");
  if (bytes == 0) return COLL_OK;
  const hipError_t he = launch_calib(dst, a, b, bytes, reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return report_hip_error(he, "calibration launch");
  return COLL_OK;
}

}  // namespace

extern "C" {

coll_status_t coll_calib_copy(void* dst, const void* src, size_t bytes, void* stream) {
  return calib(dst, src, nullptr, bytes, stream);
}

coll_status_t coll_calib_add(void* dst, const void* a, const void* b, size_t bytes, void* stream) {
  if (!b) return report_error(COLL_ERR_INVALID_ARG, "NULL buffer");
  return calib(dst, a, b, bytes, stream);
}

coll_status_t coll_calib_pattern(void* const* loads, int nloads, void* const* stores, int nstores, size_t bytes,
                                 int groups_per_cu, void* stream) {
  const bool known = (nloads == 0 && nstores == 1) || (nloads == 8 && nstores == 8) || (nloads == 8 && nstores == 1) ||
                     (nloads == 1 && nstores == 7) || (nloads == 64 && nstores == 1) || (nloads == 1 && nstores == 63);
  if (!known) return report_error(COLL_ERR_UNSUPPORTED, "no calibration pattern with these load and store counts");
  if ((nloads > 0 && !loads) || !stores) return report_error(COLL_ERR_INVALID_ARG, "NULL buffer list");
  if (bytes % 1024) return report_error(COLL_ERR_INVALID_ARG, "pattern calibration needs a multiple of 1024 bytes");
  if (groups_per_cu != 0 && (groups_per_cu < COLL_CALIB_MIN_GROUPS || groups_per_cu > COLL_CALIB_MAX_GROUPS))
    return report_error(COLL_ERR_INVALID_ARG, "groups_per_cu outside 0 or [COLL_CALIB_MIN_GROUPS, COLL_CALIB_MAX_GROUPS]");
  // the largest multiple of 512 bytes (the LDS allocation granule) of which
  // groups_per_cu fit in a CU's 160 KiB
  const uint32_t lds = groups_per_cu ? (uint32_t(160u * 1024u) / uint32_t(groups_per_cu)) & ~511u : 0u;
  RankPtrs p;
  for (int i = 0; i < COLL_MAX_RANKS; ++i) p.send[i] = p.recv[i] = 0;
  for (int i = 0; i < nloads; ++i) p.send[i] = reinterpret_cast<uint64_t>(loads[i]);
  for (int i = 0; i < nstores; ++i) p.recv[i] = reinterpret_cast<uint64_t>(stores[i]);
  for (int i = 0; i < COLL_MAX_RANKS; ++i) {
    if ((i < nloads && !p.send[i]) || (i < nstores && !p.recv[i])) return report_error(COLL_ERR_INVALID_ARG, "NULL buffer");
    if ((p.send[i] | p.recv[i]) % 16) return report_error(COLL_ERR_INVALID_ARG, "calibration needs 16-byte aligned buffers");
  }
  if (bytes == 0) return COLL_OK;
  const hipError_t he = launch_calib_pattern(p, nloads, nstores, bytes, lds, reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return report_hip_error(he, "calibration launch");
  return COLL_OK;
}

coll_status_t coll_calib_spin(float* out, uint32_t iters, uint32_t grid, void* stream) {
  if (!out) return report_error(COLL_ERR_INVALID_ARG, "NULL buffer");
  if (reinterpret_cast<uint64_t>(out) % 4) return report_error(COLL_ERR_INVALID_ARG, "out must be 4-byte aligned");
  if (grid < 1 || grid > COLL_SPIN_MAX_GRID) return report_error(COLL_ERR_INVALID_ARG, "grid outside [1, COLL_SPIN_MAX_GRID]");
  if (iters > COLL_SPIN_MAX_ITERS) return report_error(COLL_ERR_INVALID_ARG, "iters above COLL_SPIN_MAX_ITERS");
  const hipError_t he = launch_spin(out, iters, grid, reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return report_hip_error(he, "spin launch");
  return COLL_OK;
}

}  // extern "C"
