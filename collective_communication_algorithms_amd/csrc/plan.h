// Schedules of the collectives as step-ordered row tables, their counts and
// their hazard check.  Host-only C++; no HIP dependency.
#pragma once

#include <cstdint>
#include <functional>
#include <string>
#include <vector>

#include "coll.h"

namespace coll {

struct Row {
  int32_t step, src, dst;
  uint8_t reduce, local, from_send, staged;
  int64_t src_off, dst_off, n;  // elements
};

struct Step {
  int64_t first = 0, nrows = 0;  // rows [first, first + nrows) of Schedule::rows
  bool local = false;            // rank-internal rearrangement, not a counted step
  bool staged = false;           // in-place permutation: every read precedes every write
};

struct Schedule {
  coll_kind_t kind{};
  coll_algo_t algo{};
  int N = 0;
  int64_t count = 0;
  int root = 0;
  int chunks = 1;
  std::vector<Row> rows;    // step-major
  std::vector<Step> steps;
  int64_t counted_steps() const;
};

// The algorithm a COLL_ALGO_DEFAULT request stands for.
coll_algo_t resolve_algo(coll_kind_t kind, coll_algo_t algo);

// Algorithms that take the `chunks` pipeline count.
inline bool algo_pipelined(coll_algo_t a) {
  return a == COLL_ALGO_CHAIN_PIPE || a == COLL_ALGO_BINOMIAL_PIPE || a == COLL_ALGO_BIDIR_RING;
}

// alpha-beta constants for COLL_ALGO_AUTO: seconds per step, schedule bytes per second.
struct CostModel {
  double alpha_s = 1.18e-6;
  double beta_Bps = 7.0e12;
};

// What a schedule costs as it would run: the dependent memory round trips
// (a step each for the row kernel, one for the column kernel) and the bytes
// its kernels move.
struct PlannedCost {
  int64_t round_trips = 0;
  int64_t bytes = 0;
};

// COLL_ALGO_AUTO: among the collective's candidate algorithms valid for N, the
// one whose schedule minimises round_trips * alpha + bytes / beta (first
// candidate on ties), with the cost `cost(schedule)` if given, else the
// schedule's steps and bytes.  Returns COLL_OK and the algorithm, or an error.
coll_status_t choose_algo(coll_kind_t kind, int N, int64_t count, int elem_size, int root, const CostModel& m,
                          coll_algo_t& out, std::string& err,
                          const std::function<PlannedCost(const Schedule&)>* cost = nullptr);

// Validates (kind, algo, N, count, root, chunks) and builds the in-place
// schedule.  Returns COLL_OK or an error status with a message in `err`.
// The argument checks of build_schedule alone, with no rows built: the same
// status and message build_schedule would give for these arguments.
coll_status_t validate_schedule_args(coll_kind_t kind, coll_algo_t algo, int N, int64_t count, int root,
                                     int chunks, std::string& err);

// COLL_ALGO_AUTO must be resolved with choose_algo first.
coll_status_t build_schedule(coll_kind_t kind, coll_algo_t algo, int N, int64_t count, int root,
                             int chunks, Schedule& out, std::string& err);

coll_counts_t count_schedule(const Schedule& s, int elem_size);

// Empty when every step is free of conflicts inside the step; else a message.
std::string check_schedule(const Schedule& s);

}  // namespace coll
