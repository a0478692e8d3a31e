// Tables the host builds from a schedule and the kernels walk.
//
// Column space.  Every row of the Ring, Halving-Doubling, Double Binary Tree,
// Broadcast, Scatter and Gather schedules keeps its elements at the same offset
// on both ranks, so a byte offset in a rank buffer ("column") names the same
// data position on every rank.  Each work item is a byte range of columns on
// one (source rank -> destination rank) edge.  A thread of the row kernel owns
// fixed 16-byte column units on every rank for the whole call, so every value a
// thread reads was written by itself in an earlier step (or is input): steps
// need no synchronisation between threads or work groups, only program order.
// Pairwise AllToAll rows read only the send buffers, which no row writes.  The
// permutation kernel (Bruck's and the Ring AllToAll's staged steps) uses the
// offset inside a block as its column instead; every such row keeps that offset.
#pragma once

// Longest run of ITEM_BATCH_NEXT-linked work-list entries the row kernel takes at once.
#define RUN_MAX 4

#include <stdint.h>

#include "coll.h"

namespace coll {

enum : uint32_t {
  ITEM_REDUCE = 1u << 0,     // dst <- dst (+) src, else dst <- src
  ITEM_SRC_SEND = 1u << 1,   // source read from the send buffer of src_rank
  ITEM_DSRC_SEND = 1u << 2,  // old destination value read from the send buffer of dst_rank
  ITEM_VEC = 1u << 3,        // src_delta and dst_delta are multiples of 16
  ITEM_CKS_SHIFT = 4,        // bits 4..5: (-row start byte) mod 4, for the row checksum
  ITEM_BATCH_NEXT = 1u << 6, // work lists only: the next entry of this list joins this one's
                             // run (same step, both inside one tile, no common destination
                             // bytes); a run's loads are all issued before its stores
  ITEM_SRC_FWD = 1u << 7,    // work lists only: the source bytes are the previous entry's
                             // destination bytes (same columns, an earlier step), still held
                             // in the registers of the thread that stored them
  ITEM_DSRC_FWD = 1u << 8,   // work lists only: the old destination value is the previous
                             // entry's result over the same columns, still in registers
  ITEM_NO_STORE = 1u << 9,   // work lists only: a later entry of the list overwrites this
                             // entry's destination bytes (same columns) before any entry
                             // loads them; the forwarding variant does not store them
};


constexpr uint32_t NO_ROW = 0xFFFFFFFFu;

struct DevItem {          // 48 bytes
  uint64_t col0, col1;    // column bytes [col0, col1)
  int64_t src_delta;      // source address = base(src) + column + src_delta
  int64_t dst_delta;      // destination address = base(dst) + column + dst_delta
  uint32_t row;           // schedule row (checksum slot) or NO_ROW
  uint16_t src_rank, dst_rank;
  uint32_t flags;
  uint32_t pad;           // work lists: bit w set if wave w of the work group has bytes in
                          // the piece (wave w handles bytes [1024w, 1024w + 1024) of a tile)
};
static_assert(sizeof(DevItem) == 48, "work-list entries are 12 words");

enum : uint32_t {
  STEP_STAGED = 1u << 0,  // in-place permutation: all reads of a group before its writes
  STEP_ORDERED = 1u << 1, // some items accumulate into the same destination: keep item order
};

struct DevStep {          // 16 bytes
  uint32_t item0, nitems; // items [item0, item0 + nitems)
  uint32_t gsize;         // staged steps: items per staging group (groups are contiguous)
  uint32_t flags;         // STEP_*
};

struct RankPtrs {
  uint64_t send[COLL_MAX_RANKS];
  uint64_t recv[COLL_MAX_RANKS];
};

enum DType : int { DT_I32 = 0, DT_U8 = 1, DT_F32 = 2, DT_BF16 = 3 };
enum Op : int { OP_SUM = 0, OP_MAX = 1, OP_MIN = 2 };

constexpr int TILE_BYTES = 4096;      // 256 threads x 16 bytes
constexpr int BLOCK_THREADS = 256;
constexpr int WAVE_BYTES = TILE_BYTES / (BLOCK_THREADS / 64);  // one wave's bytes of a tile

// Pieces of whole tiles, at most FWD_TILES of them, 16-byte aligned on both
// sides: the forwarding variant of the row kernel keeps the units it stored for
// such a piece in registers, for the next entry of its list to use.
constexpr uint32_t FWD_TILES = 8;
constexpr bool fwd_eligible(uint64_t col0, uint64_t col1, uint32_t flags) {
  return (flags & ITEM_VEC) != 0 && col1 > col0 && col0 % TILE_BYTES == 0 && col1 % TILE_BYTES == 0 &&
         (col1 - col0) / TILE_BYTES <= FWD_TILES;
}

// Row checksums are accumulated in SUM_LANES partial slots per row: a wave adds
// its piece's sum to slot row * SUM_LANES + (work-group index mod SUM_LANES), so
// that the device-scope atomics of one row spread over SUM_LANES addresses (8
// cache lines) instead of meeting on one; a fold kernel then writes each row's
// total.
constexpr uint32_t SUM_LANES = 64;

// Nontemporal hints, per operand of a row.
enum : uint32_t { NT_SRC = 1u << 0, NT_DSRC = 1u << 1, NT_DST = 1u << 2, NT_ALL = 7u };

struct RowsArgs {                     // row kernel (copy / recv_and_reduce)
  const DevItem* list;                // this launch's work list (pieces inside one column group)
  const uint32_t* off;                // G + 1 offsets into `list`, one slice per work group
  uint64_t* sums;                     // partial row checksums (SUM_LANES per row) or nullptr
  uint32_t bases16;                   // all rank base pointers 16-byte aligned
  uint32_t pad;
  RankPtrs p;
};

// ---- column programs --------------------------------------------------------
//
// Every schedule but AllToAll keeps each element at its column, so a column's
// final values depend only on that column's inputs, through the rows that
// cover it.  Between two consecutive row boundaries (a *segment*) the same rows
// cover every column, so the host can run the schedule there once, on
// symbols, and write down what it computes: a *column program*.  The column
// kernel then runs that program on every column of the segment.  It loads each
// input the program needs once (a leaf, into a register slot), combines in the
// rows' exact order (so the float association is the schedule's), adds every
// row's result to that row's checksum, and stores only the defined outputs.
enum : uint32_t {
  CI_COMBINE = 1u << 0,  // op: y = A (+) B (a recv_and_reduce row); else the op's value is A (a copy row)
  CI_A_Y = 1u << 1,      // op: A is y, not slot `a`; store: the value is y, not slot `a`
  CI_B_Y = 1u << 2,      // op: B is y, not slot `b`
  CI_WRITE = 1u << 3,    // op: y also goes to slot `out` (it is needed after y changes)
  CI_CKS = 1u << 4,      // op: the value's words go to the checksum of the op's row
  CI_RELOAD = 1u << 5,   // op: first load the next m = (arg >> 8) & 0xff leaves of the loads list
                         // (1 <= m <= COL_BATCH) into slots 0 .. m-1
};

// Leaves a RELOAD brings in at most.
constexpr uint32_t COL_BATCH = 8;
// Dynamic LDS the column kernel's paired variant without checksums reserves
// (and never touches): 160 KiB per CU hold 16 such work groups, 4 waves per
// SIMD, where its registers alone would allow 8
constexpr uint32_t COL_PAIRED_LDS = 10240;
// The same for batched programs that store 8 or more buffers (AllReduces over
// 9-64 ranks), with or without checksums, on top of their own LDS slots
constexpr uint32_t COL_BATCHED_CAP_LDS = 13312;

struct ColInstr {        // 8 bytes
  uint8_t flags;         // CI_* (ops, stores)
  uint8_t a, b, out;     // slots: A / stored value, B, result
  uint32_t arg;          // load / store: rank; op: bits 0-1 (-row start byte) mod 4 for its
                         // checksum, bits 8-15 RELOAD's leaf count
};

struct ColSeg {          // 40 bytes: one segment's program
  uint64_t s0, s1;       // column bytes [s0, s1)
  uint32_t loads, ops, stores;  // first instruction of each list
  uint16_t nfirst, pad0;  // leaves 0 .. nfirst-1 are loaded into slots 0 .. nfirst-1 before the
                          // ops; ops flagged RELOAD bring in the rest
  uint16_t nload, nop, nstore, pad;
};

struct ColWork {         // 56 bytes: one work group's tiles and its segment's program
  uint64_t c0;           // column byte of its first tile (a multiple of the tile size)
  uint64_t s0, s1;       // the segment's column bytes
  uint32_t loads, ops, stores;
  uint32_t part;         // checksums: its nop partial sums go to partial[part .. part + nop)
  uint16_t nload, nop, nstore;
  uint16_t ntiles;       // consecutive tiles from c0
  uint16_t nfirst, pad0, pad1, pad2;
};

// Row checksums of the column kernel: every work group stores op k's wave
// total to its own slot (no atomics); a row's checksum is the sum of the
// slots of the ops that carry its value, over the work groups of every
// segment it covers.  One ColRef per (row, segment): `count` slots from
// `first`, `stride` apart (a segment's work groups store their nop partial
// sums one after the other).
struct ColRef {          // 16 bytes
  uint32_t first, count, stride, pad;
};

struct ColArgs {
  const ColWork* work;
  const ColInstr* code;
  uint64_t* partial;         // checksums: partial sums, one per (work group, op); else nullptr
  RankPtrs p;
};

// What a column-kernel launch passes: ColArgs with room for P ranks' buffer
// addresses (lane r of a work group reads rank r's).  The host time of a
// launch grows with its argument block, so calls over at most 16 ranks pass
// 16 addresses a side (280 bytes in all), the others 64 (1,048 bytes), not
// the 128 of RankPtrs (2,072 bytes): measured on MI355X, the host time per
// 4-rank AllReduce call through the C ABI fell from 5.1 to 4.7 us.
template <int P>
struct ColLaunchArgs {
  const ColWork* work;
  const ColInstr* code;
  uint64_t* partial;
  uint64_t send[P];
  uint64_t recv[P];
};

// Slices of a row's partial sums the checksum fold adds in parallel.
constexpr uint32_t COL_FOLD_SLICES = 32;

// Threads of a column-kernel work group (one wave).  Lane r also holds rank
// r's buffer addresses, so programs name at most COL_THREADS ranks.
constexpr int COL_THREADS = 64;
static_assert(COL_THREADS <= COLL_MAX_RANKS, "lane r reads rank r's pointers");

// Copy rows that depend on nothing but the send buffers (Pairwise AllToAll:
// every block read from its sender's send buffer, written to its receiver's
// receive buffer), all of one length: row r copies row_bytes from rank src's
// send buffer at src_off to rank dst's receive buffer at dst_off (bytes).
struct CopyRow {                      // 24 bytes
  uint32_t src, dst;
  uint64_t src_off, dst_off;
};

struct CopyRowsArgs {
  const CopyRow* rows;
  uint64_t* partial;                  // checksums: one slot per work group; else nullptr
  RankPtrs p;
  uint64_t row_bytes;                 // a multiple of 16
  uint32_t wgs_per_row;               // work group w copies 1 KiB tile w % wgs_per_row of row w / wgs_per_row
};

struct PermArgs {                     // staged permutation kernel (AllToAll)
  const DevItem* items;
  const DevStep* steps;
  uint64_t* sums;                     // partial row checksums (SUM_LANES per row) or nullptr
  uint32_t s0, s1;
  uint32_t lg_upl;                    // log2 of the units each lane holds per row and tile
  uint32_t ncols_units;               // block width in units
  uint32_t nontemporal;               // nonzero: nontemporal loads and stores
  uint32_t pad;
  RankPtrs p;
};

}  // namespace coll
