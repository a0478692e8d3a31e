// Turning a schedule into the item tables the kernels walk.  Host-only C++.
#pragma once

#include <cstdint>
#include <vector>

#include "device_types.h"
#include "plan.h"

namespace coll {

// One kernel launch (or one launch per step in step mode) over a step range.
struct Phase {
  enum Kind { ROWS, PERM } kind = ROWS;
  uint32_t s0 = 0, s1 = 0;     // DevStep range
  uint64_t colspace = 0;       // ROWS: largest column byte; PERM: block bytes
};

struct Bound {
  std::vector<DevItem> items;
  std::vector<DevStep> steps;
  std::vector<Phase> phases;
  coll_counts_t counts{};      // as executed
  int64_t nrows = 0;           // schedule rows (checksum slots)
  int perm_unit = 16;          // PERM: bytes per unit (16, 8, 4, 2 or 1)
};

// In place (`inplace`) or out of place.  Out of place, a row reads from the send
// buffer every region that no earlier row has written on the receive side, and
// each region of a rank's defined output that no row writes is copied from
// send to receive in the first step.
Bound bind_schedule(const Schedule& s, int elem_size, bool inplace);

// The regions of rank i's receive buffer whose final value the collective
// defines (element ranges).
std::vector<std::pair<int64_t, int64_t>> defined_output(const Schedule& s, int rank);

}  // namespace coll
