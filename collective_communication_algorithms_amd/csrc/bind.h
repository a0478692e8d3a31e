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
  // per rank, the byte ranges of its receive buffer whose final value the
  // collective defines (sorted); the rest is left unspecified
  std::vector<std::vector<std::pair<uint64_t, uint64_t>>> defined;
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
// are marked on the final order, and so are the forwarding variant's marks:
// ITEM_SRC_FWD / ITEM_DSRC_FWD, and ITEM_NO_STORE on a store that a later entry
// over the same columns overwrites before any load, or (group-major lists of
// the call's last phase, one launch) on a store outside its rank's defined
// output that no later entry of its column group loads.
void build_worklist(const Bound& b, const Phase& ph, uint32_t G, uint32_t group_tiles, bool reverse,
                    bool per_step, bool group_major, const std::vector<uint64_t>& cuts, std::vector<uint32_t>& off,
                    std::vector<DevItem>& list);

// The host side of one row phase's launches: the work lists of build_worklist
// on a grid of G = min(column groups (+ row-boundary cuts when they fit), cap)
// work groups, and the row-kernel variant that runs them.
struct RowsList {
  uint32_t G = 1;
  bool fine = false;        // the fine variant (runs, or pieces of under one tile on average)
  bool fwd = false;         // the forwarding variant (group-major, at least 60 % of entries forward)
  uint64_t fwd_saved = 0;   // bytes the forwarding variant neither loads nor stores
  std::vector<uint32_t> off;
  std::vector<DevItem> list;
};

RowsList plan_rows_list(const Bound& b, const Phase& ph, uint64_t cap, uint32_t group_tiles, bool reverse,
                        bool per_step, bool group_major);

// ---- launch shape of a row phase ----------------------------------------------

// Column spaces of at least BLOCKED_MIN_COLSPACE bytes get large grids: one
// column group per work group (BLOCKED_GROUP_TILES_COPY tiles for copy-only
// schedules, BLOCKED_GROUP_TILES_REDUCE with reduce rows), or the cache window
// of rows_shape.  Smaller ones get a grid of the work groups that fit on the
// device at once.  8 MiB: against the earlier 32 MiB, 8 ranks x 8-24 MiB ran
// 9-51 % faster in nearly every collective (Ring AllReduce fp32 16 MiB 78.0 ->
// 52.6 us, Ring AllGather bf16 32 ranks x 16 MiB 187 -> 91 us, chain Broadcast
// 16 MiB 39.9 -> 25.7 us; binomial Gather 16 MiB 11.5 -> 12.2 us); at 2 MiB
// the large grid made Ring AllReduce slower (20 -> 31 us).
constexpr uint32_t BLOCKED_GROUP_TILES_REDUCE = 4;
constexpr uint32_t BLOCKED_GROUP_TILES_COPY = 8;
constexpr uint64_t BLOCKED_MIN_COLSPACE = uint64_t(8) << 20;
// Long pieces (see rows_shape): at least LONG_PIECE_MIN_COLSPACE_* bytes of
// columns, and rows that start or end no more often than every
// LONG_PIECE_REDUCE bytes (reductions) or LONG_PIECE_COPY bytes (copies) on
// average.
constexpr uint64_t LONG_PIECE_MIN_COLSPACE_REDUCE = uint64_t(64) << 20;
constexpr uint64_t LONG_PIECE_MIN_COLSPACE_COPY = uint64_t(128) << 20;
constexpr uint64_t LONG_PIECE_REDUCE = uint64_t(8) << 20;
constexpr uint64_t LONG_PIECE_COPY = uint64_t(16) << 20;

struct RowsShapeInput {
  uint64_t colspace = 0;
  uint64_t segment = 0;             // mean bytes between the phase's row boundaries (phase_segment)
  bool has_reduce = false;
  bool checksums = false;           // the kernels also compute per-row checksums
  int elem_size = 4;
  int nranks = 1;
  uint32_t cus = 1;                 // compute units of the device
  uint64_t resident = 1;            // work groups of the kernel that fit on the device at once
  bool per_step = false;            // one launch per step
  int64_t forced_group_tiles = 0;   // > 0: the caller's group size
  int64_t forced_grid = 0;          // > 0: the caller's grid cap
};

struct RowsShape {
  uint32_t group_tiles = 8;
  uint64_t cap = 1;                 // grid cap: one work group per group up to this many
  bool group_major = false;         // a work group takes its groups one at a time through all steps
};

// Whether the phase's 4-tile column groups average two or more pieces per
// step (halving-doubling, trees, RHD AllGather, binomial Broadcast) or not
// (Ring, chains).
bool several_pieces_per_step(const Bound& b, const Phase& ph);

// The mean length in bytes of the column ranges between a row phase's row
// boundaries: colspace / (boundaries + 1).
uint64_t phase_segment(const Phase& ph);

// Group size for a grid of `max_groups` work groups: enough groups to give
// each of them one, up to 8 tiles per group.
uint32_t resident_group_tiles(uint64_t colspace, uint64_t max_groups);

// The launch shape of a row phase.  `several()` answers several_pieces_per_step
// and is called only when the choice depends on it.
//
// Large column spaces (one launch for all steps) take their groups in
// group-major lists.  fp32 / int32 / bf16 reductions, and copy-only schedules
// over 16 or more ranks, whose groups see several pieces per step (trees,
// halving-doubling) use a resident grid of 2 work groups per CU with 4-tile
// groups, which keeps the data in flight small enough for the caches.
// Measured at 8 x 256 MiB fp32 against one group per work group: DBT 1.158 ->
// 1.040 ms, RHD 1.207 -> 1.066, Reduce 0.683 -> 0.655; bf16: DBT 1.130 ->
// 1.055, RHD 1.182 -> 1.081; bf16 64 x 256 MiB ReduceScatter RHD 7.06 -> 6.81
// ms.  Copy-only: bf16 RHD AllGather 64 x 256 MiB 6.19 -> 5.36 ms, 16 x 128 MiB
// 0.638 -> 0.606; at 8 ranks (RHD AllGather, binomial Broadcast) within 3 %
// either way, so they keep one group per work group.  Grids are whole
// multiples of the CU count (2.5 per CU measured 10 % slower).  Reductions with
// one piece per step (Ring), which the forwarding variant of the row kernel
// runs, take 8-tile groups, one per work group: their operands pass from step
// to step in registers, so a small grid keeps nothing in the caches that
// matters (Ring AllReduce fp32 8 x 32 MiB 97.6 -> 87.0 us against 2 per CU, 8 x
// 256 MiB 0.870 -> 0.851 ms against 3 per CU; 64-rank bf16 ReduceScatter 3.17
// -> 3.10 ms).  Copy schedules with one piece per step and uint8 reductions
// (not measured) keep one group per work group as well.  One group per work
// group itself beat a resident-sized grid at 8 x 256 MiB by 15-22 %
// (AllReduce), 18 % (Tree Reduce), 9-24 % (64-rank ReduceScatter), 3-7 %
// (64-rank AllGather).  One launch per step: 4 resident grids' worth of groups
// per launch.
template <class Several>
RowsShape rows_shape(const RowsShapeInput& in, Several&& several_pieces) {
  int known = -1;  // several_pieces(), asked at most once
  auto several = [&] {
    if (known < 0) known = several_pieces() ? 1 : 0;
    return known != 0;
  };
  RowsShape r;
  const bool blocked = !in.per_step && in.colspace >= BLOCKED_MIN_COLSPACE;
  r.group_major = blocked;
  r.cap = in.per_step ? 4 * in.resident : in.resident;
  r.group_tiles = blocked ? (in.has_reduce ? BLOCKED_GROUP_TILES_REDUCE : BLOCKED_GROUP_TILES_COPY)
                          : resident_group_tiles(in.colspace, in.resident);
  if (blocked) {
    r.cap = uint64_t(1) << 20;
    const bool reduce_rule = in.has_reduce && in.elem_size >= 2;
    const bool copy_rule = !in.has_reduce && in.nranks >= 16;
    if ((reduce_rule || copy_rule) && in.forced_group_tiles <= 0) {
      if (several()) {
        r.group_tiles = BLOCKED_GROUP_TILES_REDUCE;
        r.cap = uint64_t(in.cus) * 2u;
      } else if (reduce_rule) {
        r.group_tiles = 8;
      }
    }
  }
  // fewer 8-tile groups than 2 per CU (8 x 8 MiB: 256): 4-tile groups, twice
  // as many (8 ranks x 8 MiB: Ring AllReduce fp32 31.0 -> 28.4 us, Ring
  // ReduceScatter bf16 26.6 -> 22.6, Ring AllGather 18.4 -> 17.1, chain
  // Broadcast 18.4 -> 17.0; at 16 MiB and up 8 tiles are as fast or faster)
  if (blocked && in.forced_group_tiles <= 0 && r.group_tiles == 8 &&
      (in.colspace + 8 * TILE_BYTES - 1) / (8 * TILE_BYTES) < 2 * uint64_t(in.cus))
    r.group_tiles = 4;
  // Long pieces, one per step: 4-tile groups, one per work group, against 8
  // tiles.  Reductions, pieces of 8 MiB and more: Ring AllReduce fp32 8 x 256
  // MiB 831 -> 808 us, bf16 833 -> 782, fp32 8 x 128 MiB 431 -> 404, bf16 16 x
  // 192 MiB 1290 -> 1215, fp32 32 x 256 MiB 3397 -> 3309, Ring ReduceScatter
  // fp32 8 x 128 MiB 253 -> 244.  Copies, pieces of 16 MiB and more: Ring
  // AllGather bf16 8 x 256 MiB 412 -> 396, 8 x 128 MiB 197.5 -> 192.3, chain
  // Broadcast uint8 8 x 256 MiB 420 -> 400, 8 x 128 MiB in one piece 198 ->
  // 192; but in 64 MiB of columns copies keep 8 tiles (chain Broadcast 8 x 64
  // MiB in one piece 87 against 96 us, Ring AllGather bf16 4 x 64 MiB 48
  // against 51).  Shorter pieces keep 8 tiles: 64 x
  // 256 MiB bf16 (4 MiB pieces) ReduceScatter 3144 against 3534 us, AllGather
  // 3219 against 3350; AllGather bf16 32 x 256 MiB (8 MiB) 1622 against 1663,
  // 8 x 96 MiB (12 MiB) 141 against 144; chain Broadcast 8 x 96 MiB 143
  // against 145.  With row checksums twice as many groups make twice as many
  // checksum atomics, which takes the gain away (Ring AllReduce fp32 8 x 256
  // MiB: row kernel 0.827 ms with 8 tiles, 0.828-0.832 with 4), so calls with
  // checksums keep 8 tiles.
  if (blocked && !in.checksums && in.forced_group_tiles <= 0 && r.group_tiles == 8 && r.cap == (uint64_t(1) << 20) &&
      in.colspace >= (in.has_reduce ? LONG_PIECE_MIN_COLSPACE_REDUCE : LONG_PIECE_MIN_COLSPACE_COPY) &&
      in.segment >= (in.has_reduce ? LONG_PIECE_REDUCE : LONG_PIECE_COPY) && !several())
    r.group_tiles = 4;
  if (in.forced_group_tiles > 0) r.group_tiles = uint32_t(in.forced_group_tiles);
  if (in.forced_grid > 0) r.cap = uint64_t(in.forced_grid);
  return r;
}

// The regions of rank i's receive buffer whose final value the collective
// defines (element ranges).
std::vector<std::pair<int64_t, int64_t>> defined_output(const Schedule& s, int rank);

}  // namespace coll
