// Compiling a schedule into column programs (see device_types.h), and the
// tables the column kernel walks.  Host-only C++.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "device_types.h"
#include "plan.h"

namespace coll {

// Register capacities of the column kernel's variants: `unit` bytes per lane
// and column, at most `leaves` leaves and slots, and checksums of up to
// `accs` ops (0: the variant computes no checksums; 16 a per-lane
// accumulator file, 8 slots and unbatched programs only; 8 and 64 wave sums
// merged across lanes; -1 no checksums, the leaves loaded in pairs, at most 16
// work groups per CU); `batched` variants
// also run programs that bring their leaves in batches (RELOAD ops), at the
// cost of the registers that takes.  Every list of a program holds at most
// 64 instructions (one per lane).
constexpr int COL_LIST_MAX_STORES = 64;  // one store per lane

struct ColVariant {
  int unit = 16;
  int leaves = 8;
  int accs = 0;
  bool batched = false;
  int stores = COL_LIST_MAX_STORES;  // the variant is picked for programs of at most this many stores
  int min_stores = 0, min_leaves = 0;  // ... and of at least this many stores and leaves
  bool capped = false;          // batched: launched with reserved LDS, fewer work groups per CU
};

// With checksums: row `row`'s checksum over segment `seg` is the sum of op
// `op`'s values there (several rows may share an op: a copy carries the value
// of the op that made it, with the same rotation).
struct ColRowRef {
  uint32_t row, seg, op;
};

struct ColPlan {
  bool ok = false;
  std::string why;               // when not ok: the first reason
  ColVariant v;
  uint64_t colspace = 0;         // bytes of columns (count * element size)
  std::vector<ColSeg> segs;
  std::vector<ColInstr> code;
  std::vector<ColRowRef> refs;   // checksums only; one per (row, segment it covers)
  uint64_t moved_bytes = 0;      // leaf loads and stores: bytes each segment moves, summed
  uint32_t max_leaves = 0, max_slots = 0, max_ops = 0, max_stores = 0;
  bool batched = false;          // some program loads its leaves in batches
};

constexpr int COL_LIST_MAX = 64;

// Compiles the in-place or out-of-place call of schedule `s` (element size
// `sz`) into one program per segment, and picks the smallest variant that
// holds every program.  Not ok (with a reason) for AllToAll, for schedules
// whose rows change offset, for more than `max_segments` segments, and for
// programs no variant holds; the row kernel runs those.
//
// Semantics of a segment, column by column (the pages' step model: every send
// of a step leaves from the state before the step): each rank starts with its
// input (the send buffer's value; in place that is the receive buffer); per
// step, every covering row's source value is taken first, then the rows are
// applied in row order, a copy setting the destination's value, a reduce row
// replacing it with combine(destination, source).  A rank's final value is
// stored when the collective defines its output there and a row wrote it, or
// (out of place) when no row did; in place, a rank whose final value is its
// own input needs no store (the kernel stores nothing before a program's
// end).  Stores outside the defined output are not made: the contract leaves
// those bytes unspecified.
ColPlan compile_colplan(const Schedule& s, int sz, bool inplace, bool checksums, size_t max_segments = 8192);

// The kernel's tables for work groups of `tiles_per_group` consecutive tiles
// (64 lanes x unit bytes each, on the global tile grid) of one segment.  With
// checksums, work group w of segment k stores its nop partial sums at
// partial[base_k + w * nop ...]; row r's ColRefs are refs[row_off[r] ..
// row_off[r + 1]).
struct ColTables {
  std::vector<ColWork> work;
  std::vector<uint32_t> row_off;  // nrows + 1 (checksums), else empty
  std::vector<ColRef> refs;
  uint64_t partials = 0;          // partial-sum slots the work groups write
};

ColTables col_tables(const ColPlan& p, uint32_t tiles_per_group, size_t nrows);

}  // namespace coll
