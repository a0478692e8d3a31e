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
  std::vector<uint64_t> bounds;  // ROWS: columns in (0, colspace) where a row starts or ends, sorted
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

// The row boundaries of a phase that fall inside column groups of `gbytes`
// bytes (sorted).
std::vector<uint64_t> group_cuts(const Phase& ph, uint64_t gbytes);

// Work lists of one row phase on a grid of G work groups, with column groups
// of `group_tiles` 4 KiB tiles, each group that a column of `cuts` (sorted)
// falls inside split there in two; groups are numbered in column order.  With
// the cuts of group_cuts, no group holds two rows that end or start inside it,
// so a group never has two chains of pieces to run one after the other.
// Every item is cut at group boundaries and each piece goes to the list of the
// work group that owns its group.
//  one launch for the phase (per_step false): group g belongs to work group
//    g mod G in every step, so each column is only ever touched by one work
//    group and the steps need no synchronisation between work groups;
//  one launch per step (per_step true): the same, except that with `reverse`
//    odd steps hand group g to work group G-1-(g mod G), which reverses the
//    order groups are dispatched in (the launches order the steps).
// A list keeps step order and row order within each column group; with
// `reverse`, odd steps are listed back to front (items too, unless the step
// accumulates several rows into one destination).  `group_major` lists a work
// group's groups one after the other, each through all its steps (its
// columns' data stays cached from one step to the next); otherwise all its
// groups go step by step.  Launch j gives work group w the pieces
// off[j*(G+1) + w] .. off[j*(G+1) + w + 1] of `list`.  Runs (ITEM_BATCH_NEXT)
// are marked on the final order.
void build_worklist(const Bound& b, const Phase& ph, uint32_t G, uint32_t group_tiles, bool reverse,
                    bool per_step, bool group_major, const std::vector<uint64_t>& cuts, std::vector<uint32_t>& off,
                    std::vector<DevItem>& list);

// The regions of rank i's receive buffer whose final value the collective
// defines (element ranges).
std::vector<std::pair<int64_t, int64_t>> defined_output(const Schedule& s, int rank);

}  // namespace coll
