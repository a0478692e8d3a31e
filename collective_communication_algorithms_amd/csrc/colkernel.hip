// Column kernel for gfx950 (CDNA4, wave64): runs the host-compiled column
// programs of a schedule (device_types.h, colprog.h).
//
// Every schedule but AllToAll keeps each element at its column, so rank r's
// final value at column x is a fixed expression over the ranks' inputs at x:
// the rows that cover x, applied step by step ("集合通信算法延迟公式" gives the
// step structure of every algorithm here: Ring ReduceScatter / AllGather,
// Recursive Halving-Doubling, Double Binary Tree, Tree Reduce; "一对多通信：
// Broadcast 与 Scatter" the Broadcast, Scatter and Gather trees and pipelines).
// A work group is one wave; lane l takes bytes [16l, 16l + 16) of every
// 1 KiB tile of its segment.  Per tile it
//   * loads the program's leaves (each rank input the program needs, once)
//     into register slots, all loads in flight together (programs with more
//     leaves than slots bring them in batches: an op flagged RELOAD first
//     refills slots 0 .. m-1 (m <= 8) with the next leaves, once the batch
//     before is consumed);
//   * runs the ops in the rows' order: a recv_and_reduce row combines its old
//     destination value with its source value (A (+) B, the same element
//     arithmetic as the row kernel, so float results keep the schedule's
//     association), a copy row passes a value on; `y` holds the last result,
//     other values live in slots;
//   * adds every op's value to its checksum accumulator (same words, same
//     rotation as the row kernel; a row whose value an op carries already
//     shares that op's sum);
//   * stores each rank's final value where the collective defines it.
// What the schedule's steps would have passed through memory stays in
// registers, so the kernel moves each leaf once and each stored output once:
// for an in-place AllReduce over N ranks of M bytes, 2NM bytes.  No work group
// reads or writes another's columns, so nothing waits on anything.  Row
// checksums: each work group stores its per-op totals to slots of its own,
// and a fold kernel adds up each row's slots (device-scope atomics from one
// work group per KiB of columns cost more than the whole copy).
#include <hip/hip_runtime.h>

#include <mutex>
#include <unordered_map>

#include "device_common.h"
#include "device_types.h"
#include "launch.h"

namespace coll {
namespace {

// NL slots of 16 bytes in registers, indexed by a wave-uniform slot number:
// the compiler moves them with relative register addressing, which it does
// for vectors of up to 32 dwords, so larger files are two such halves.
template <int NL>
struct Slots {
  static constexpr int DW = NL * 4;                    // dwords
  static constexpr int HALF = DW > 32 ? DW / 2 : DW;   // dwords per part
  static_assert(DW <= 64 && DW % 4 == 0, "at most two 32-dword parts");
  typedef uint32_t V __attribute__((ext_vector_type(HALF)));
  V lo, hi;  // hi is unused when DW <= 32
};

template <int NL>
__device__ __forceinline__ uint32_t slot_word(const Slots<NL>& s, uint32_t i) {
  typedef Slots<NL> S;
  if constexpr (S::DW <= 32) return s.lo[i];
  else return i < uint32_t(S::HALF) ? s.lo[i] : s.hi[i - S::HALF];
}

template <int NL>
__device__ __forceinline__ void slot_word_set(Slots<NL>& s, uint32_t i, uint32_t v) {
  typedef Slots<NL> S;
  if constexpr (S::DW <= 32) {
    s.lo[i] = v;
  } else {
    if (i < uint32_t(S::HALF)) s.lo[i] = v;
    else s.hi[i - S::HALF] = v;
  }
}

template <int NL>
__device__ __forceinline__ u32x4 slot_get(const Slots<NL>& s, uint32_t k) {
  u32x4 r;
  r.x = slot_word(s, 4 * k);
  r.y = slot_word(s, 4 * k + 1);
  r.z = slot_word(s, 4 * k + 2);
  r.w = slot_word(s, 4 * k + 3);
  return r;
}

template <int NL>
__device__ __forceinline__ void slot_set(Slots<NL>& s, uint32_t k, u32x4 v) {
  slot_word_set(s, 4 * k, v.x);
  slot_word_set(s, 4 * k + 1, v.y);
  slot_word_set(s, 4 * k + 2, v.z);
  slot_word_set(s, 4 * k + 3, v.w);
}

// The row-checksum words of the 16-byte unit at column x (a multiple of 16),
// over the bytes of [s0, s1) in it, rotated by the row start's misalignment
// `shift`.
template <int DT>
__device__ __forceinline__ uint64_t unit_words(u32x4 v, uint64_t x, uint64_t s0, uint64_t s1, bool full,
                                               uint32_t shift) {
  if (full) return words16(v, shift * 8u);
  constexpr int SZ = elem_size<DT>(), E = 16 / SZ;
  const uint32_t r0 = s0 > x ? uint32_t(s0 - x) : 0u, r1 = s1 < x + 16 ? uint32_t(s1 - x) : 16u;
  uint64_t acc = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t b = uint32_t(e * SZ);
    if (b >= r0 && b < r1) acc += uint64_t(elem_of<DT>(v, e) << (8u * ((b + shift) & 3u)));
  }
  return acc;
}

// Stores the unit's bytes that lie in [s0, s1), element by element.
template <int DT>
__device__ __forceinline__ void store_part(char* p, u32x4 v, uint64_t x, uint64_t s0, uint64_t s1) {
  constexpr int SZ = elem_size<DT>(), E = 16 / SZ;
  const uint32_t r0 = s0 > x ? uint32_t(s0 - x) : 0u, r1 = s1 < x + 16 ? uint32_t(s1 - x) : 16u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t b = uint32_t(e * SZ);
    if (b >= r0 && b < r1) st_elem<DT>(p + b, elem_of<DT>(v, e));
  }
}

__device__ __forceinline__ uint64_t lane_u64(uint32_t lo, uint32_t hi, uint32_t lane) {
  return uint64_t(uint32_t(__builtin_amdgcn_readlane(int(lo), int(lane)))) |
         (uint64_t(uint32_t(__builtin_amdgcn_readlane(int(hi), int(lane)))) << 32);
}

// NA u64 checksum accumulators (NA <= 16: 32 dwords), indexed by the
// wave-uniform op number, like the slots.
template <int NA>
struct Accs {
  static_assert(NA <= 16, "one 32-dword file");
  typedef uint64_t V __attribute__((ext_vector_type(NA)));
  V lo;
  __device__ __forceinline__ void clear() { lo = 0; }
  __device__ __forceinline__ void add(uint32_t k, uint64_t v) { lo[k] += v; }
  __device__ __forceinline__ uint64_t get(uint32_t k) const { return lo[k]; }
};
template <>
struct Accs<0> {};
// NA < 0: no accumulator file; each op's words are reduced across the wave
// per tile as the ops arrive (any op count up to 64), like the digits of a
// binary counter: a level-j group holds the partial sums of 2^j consecutive
// ops, two lanes per pair of ops apart.  Merging the level-j groups A (the
// earlier ops) and B pairs every lane with a partner (level 0: l ^ 7 by
// row_half_mirror, 1: l ^ 1 and 2: l ^ 2 by quad permutes, 3: l ^ 8 by
// row_ror:8, 4: l ^ 16 and 5: l ^ 32 by the permlane swaps): a lane whose
// level bit is clear keeps A's words plus its partner's, the other B's.
// Each level pairs lanes that hold the same op, so after six levels lane l
// holds the wave total of op op_of_lane(l).  A 64-op group costs 63 merges
// of a few instructions each, against 64 full wave sums.
template <>
struct Accs<-1> {
  uint64_t l[6];  // the pending group at each level
};
// NA = -2: the same merged sums, with the leaves loaded in pairs (below).
template <>
struct Accs<-2> : Accs<-1> {};
// NA = -3: no checksums, the leaves loaded in pairs, launched at most 16 work
// groups per CU (COL_PAIRED_LDS).
template <>
struct Accs<-3> {};

// The lane that carries op o after six merge levels (the inverse of the
// level bits chosen above: op bit 0 is lane bit 2, op bits 1 and 2 are lane
// bits 0 and 1, op bits 3 .. 5 are lane bits 3 .. 5).
__device__ __forceinline__ uint32_t op_of_lane(uint32_t lane) {
  return ((lane >> 2) & 1u) | ((lane & 3u) << 1) | (lane & 0x38u);
}

template <int J>
__device__ __forceinline__ uint32_t partner_word(uint32_t v) {
  // row_half_mirror, quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_ror:8
  constexpr int ctrl = J == 0 ? 0x141 : J == 1 ? 0xB1 : J == 2 ? 0x4E : 0x128;
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), ctrl, 0xf, 0xf, false));
}

template <int J>
__device__ __forceinline__ uint64_t merge_level(uint64_t a, uint64_t b, uint32_t lane) {
  if constexpr (J < 4) {
    constexpr uint32_t bit = J == 0 ? 4u : J == 1 ? 1u : J == 2 ? 2u : 8u;
    const bool second = (lane & bit) != 0;
    const uint64_t keep = second ? b : a, give = second ? a : b;
    const uint64_t got = uint64_t(partner_word<J>(uint32_t(give))) |
                         (uint64_t(partner_word<J>(uint32_t(give >> 32))) << 32);
    return keep + got;
  } else {
    // the swap exchanges the second half of rows (J = 4: the odd 16-lane
    // rows; J = 5: the upper 32 lanes) of its first operand with the first
    // half of its second: afterwards the two registers hold, lane for lane,
    // A's words and its partner's where the level bit is clear, B's where it
    // is set
    const auto lo = J == 4 ? __builtin_amdgcn_permlane16_swap(uint32_t(a), uint32_t(b), false, false)
                           : __builtin_amdgcn_permlane32_swap(uint32_t(a), uint32_t(b), false, false);
    const auto hi = J == 4 ? __builtin_amdgcn_permlane16_swap(uint32_t(a >> 32), uint32_t(b >> 32), false, false)
                           : __builtin_amdgcn_permlane32_swap(uint32_t(a >> 32), uint32_t(b >> 32), false, false);
    return ((uint64_t(hi[0]) << 32) | lo[0]) + ((uint64_t(hi[1]) << 32) | lo[1]);
  }
}

// Op k's words c enter at level 0; every set bit of k below the first clear
// one completes a group, which merges with the pending group of its level.
// A completed 64-op group is added to the lane's running total.
template <int J>
__device__ __forceinline__ void push_op(Accs<-1>& s, uint64_t c, uint32_t k, uint32_t lane, uint64_t& total) {
  if constexpr (J == 6) {
    total += c;
  } else {
    if (k & (1u << J)) push_op<J + 1>(s, merge_level<J>(s.l[J], c, lane), k, lane, total);
    else s.l[J] = c;
  }
}

// After n ops (n <= 64): the pending groups (one per set bit of n, earlier
// ops at higher levels) and a partial group carried up from below merge
// into one 64-op group whose missing ops are zero.
template <int J>
__device__ __forceinline__ uint64_t flush_ops(const Accs<-1>& s, uint32_t n, uint64_t c, uint32_t lane) {
  if constexpr (J == 6) {
    return c;
  } else {
    if (n & (1u << J)) c = merge_level<J>(s.l[J], c, lane);
    else if (n & ((1u << J) - 1u)) c = merge_level<J>(c, 0, lane);
    return flush_ops<J + 1>(s, n, c, lane);
  }
}

// 16 bytes per lane and column; NL slots; NA checksum accumulators (0: no
// checksums; 16: a per-lane file; -1: per-tile wave sums, for every program
// a 16-entry file with 8 slots does not hold: larger files cost more in
// occupancy than the sums cost in instructions); NTM: nontemporal loads
// (NT_SRC) / stores (NT_DST); BT: programs
// may bring leaves in batches (the RELOAD path costs registers, so the other
// variants leave it out).  Batched programs keep leaves in slots 0 .. 7 and
// only partial results above, which are written once and read once per
// subtree: with BT those slots live in LDS (1 KiB each per work group), so
// the wave keeps the registers of the 8-slot variant and its occupancy.
template <int DT, int OP, int NL, int NA, int NTM, bool BT, int P>
__global__ __launch_bounds__(COL_THREADS) void col_kernel(const ColLaunchArgs<P> a) {
  typedef u32x4 U;
  constexpr uint64_t UNIT = 16;
  constexpr uint64_t TB = uint64_t(COL_THREADS) * UNIT;
  constexpr int NR = (BT && NL > int(COL_BATCH)) ? int(COL_BATCH) : NL;  // slots in registers
  constexpr int NS = NL - NR;                                            // slots in LDS
  __shared__ U lds_slot[NS > 0 ? NS : 1][COL_THREADS];
  const ColWork wk = cload(a.work + blockIdx.x);
  const uint32_t lane = threadIdx.x;
  // lane r holds rank r's buffer addresses, lane k entry k of each list
  static_assert(P <= COL_THREADS, "lane r holds rank r's addresses");
  const uint64_t sp = lane < uint32_t(P) ? a.send[lane] : 0, rp = lane < uint32_t(P) ? a.recv[lane] : 0;
  const uint32_t sp_lo = uint32_t(sp), sp_hi = uint32_t(sp >> 32), rp_lo = uint32_t(rp), rp_hi = uint32_t(rp >> 32);
  uint32_t ld_w1 = 0, op_w0 = 0, op_w1 = 0, st_w0 = 0, st_w1 = 0;
  if (lane < wk.nload) ld_w1 = *gptr<uint32_t>(reinterpret_cast<const char*>(a.code + wk.loads + lane) + 4);
  if (lane < wk.nop) {
    const uint64_t v = *gptr<uint64_t>(reinterpret_cast<const char*>(a.code + wk.ops + lane));
    op_w0 = uint32_t(v);
    op_w1 = uint32_t(v >> 32);
  }
  if (lane < wk.nstore) {
    const uint64_t v = *gptr<uint64_t>(reinterpret_cast<const char*>(a.code + wk.stores + lane));
    st_w0 = uint32_t(v);
    st_w1 = uint32_t(v >> 32);
  }
  // The tile loop reads the lists and addresses above with v_readlane.  Wait
  // for them once here: the compiler cannot tell, in blocks a uniform branch
  // may skip, that they have arrived, and would otherwise wait for every
  // outstanding load (vmcnt(0)) before each leaf load.
  __builtin_amdgcn_s_waitcnt(0);
  const uint32_t nfirst = wk.nfirst, nop = wk.nop, nstore = wk.nstore;
  const uint64_t s0 = wk.s0, s1 = wk.s1, xs = s0 & ~(UNIT - 1);
  constexpr bool MERGED = NA == -1 || NA == -2;            // checksums as merged wave sums
  constexpr bool PAIRS = NA > 0 || NA == -2 || NA == -3;    // leaves loaded in pairs
  Accs<NA> acc;
  if constexpr (NA > 0) acc.clear();
  if constexpr (MERGED)
    for (int j = 0; j < 6; ++j) acc.l[j] = 0;
  uint64_t mine = 0;  // MERGED: lane l's running total of op op_of_lane(l)
  for (uint32_t t = 0; t < wk.ntiles; ++t) {
    const uint64_t x = wk.c0 + uint64_t(t) * TB + uint64_t(lane) * UNIT;
    const bool any = x < s1 && x + UNIT > s0;
    const bool full = x >= s0 && x + UNIT <= s1;
    // a lane outside the segment loads the segment's first unit instead: the
    // loads need no branch (a branch around each makes the compiler wait for
    // every load before issuing the next), and what that lane computes is
    // neither stored nor summed
    const uint64_t xl = any ? x : xs;
    Slots<NR> v;
    auto sget = [&](uint32_t i) -> U {
      if constexpr (NS > 0) {
        if (i >= uint32_t(NR)) return lds_slot[i - NR][lane];
      }
      return slot_get(v, i);
    };
    auto sset = [&](uint32_t i, U u) {
      // a batched program writes partial results only, to slots NR and up
      // (leaves arrive by loads): the register slots are never written here
      if constexpr (NS > 0) lds_slot[i - NR][lane] = u;
      else slot_set(v, i, u);
    };
    if constexpr (BT) {
      // a batched program's first batch (1 .. 8 leaves): slots past it load
      // its last leaf again (a cache hit, never read), so that no slot
      // depends on a branch
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const uint32_t jj = uint32_t(j) < nfirst ? uint32_t(j) : nfirst - 1u;
        const uint32_t rk = uint32_t(__builtin_amdgcn_readlane(int(ld_w1), int(jj)));
        const char* base = reinterpret_cast<const char*>(lane_u64(sp_lo, sp_hi, rk));
        slot_set(v, uint32_t(j), ld16<(NTM & NT_SRC) != 0>(base + xl));
      }
    } else if constexpr (PAIRS) {
      // the checksum variants of up to 16 ops (4-6 waves per SIMD where the
      // plain one holds 8): leaves in pairs, one branch per pair (a slot
      // past the leaves loads the last leaf again), which the compiler
      // issues with at most two loads in flight per wave.  Measured on
      // MI355X with row checksums: Ring AllReduce fp32 8 x 256 MiB 0.741 ->
      // 0.726 ms, bf16 0.830 -> 0.750 ms, tree Reduce 0.461 -> 0.425 ms;
      // pairs without checksums were slower (0.737 -> 0.758 ms), and so
      // were all eight loads in flight together (0.764 ms).  Single-leaf
      // programs load one at a time (NA = -1): AllGather bf16 8 x 256 MiB
      // 0.418 ms in pairs (the leaf loaded twice), 0.394 ms alone.
#pragma unroll
      for (int j0 = 0; j0 < NR; j0 += 2) {
        if (uint32_t(j0) < nfirst) {
#pragma unroll
          for (int j = j0; j < j0 + 2; ++j) {
            const uint32_t jj = uint32_t(j) < nfirst ? uint32_t(j) : nfirst - 1u;
            const uint32_t rk = uint32_t(__builtin_amdgcn_readlane(int(ld_w1), int(jj)));
            const char* base = reinterpret_cast<const char*>(lane_u64(sp_lo, sp_hi, rk));
            slot_set(v, uint32_t(j), ld16<(NTM & NT_SRC) != 0>(base + xl));
          }
        }
      }
    } else {
      // one branch per leaf: the compiler waits for each load before the
      // next, which keeps one load in flight per wave; at the plain
      // variant's occupancy that beats issuing them together
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        if (uint32_t(j) < nfirst) {
          const uint32_t rk = uint32_t(__builtin_amdgcn_readlane(int(ld_w1), j));
          const char* base = reinterpret_cast<const char*>(lane_u64(sp_lo, sp_hi, rk));
          slot_set(v, uint32_t(j), ld16<(NTM & NT_SRC) != 0>(base + xl));
        }
      }
    }
    U y{};
    uint32_t next = nfirst;  // leaves loaded so far
    for (uint32_t k = 0; k < nop; ++k) {
      const uint32_t w0 = uint32_t(__builtin_amdgcn_readlane(int(op_w0), int(k)));
      if (BT && (w0 & CI_RELOAD)) {
        // before this op: the next m leaves into slots 0 .. m-1, all loads in
        // flight together.  The batch before is consumed; saying so (an
        // explicit wait, free here) keeps the compiler from waiting between
        // these loads for loads it cannot tell have arrived.
        __builtin_amdgcn_s_waitcnt(0);
        const uint32_t m = (uint32_t(__builtin_amdgcn_readlane(int(op_w1), int(k))) >> 8) & 0xffu;
        // (slots past m load leaf m-1 again, as for the first batch)
#pragma unroll
        for (uint32_t j = 0; j < COL_BATCH; ++j) {
          const uint32_t jj = next + (j < m ? j : m - 1u);
          const uint32_t rk = uint32_t(__builtin_amdgcn_readlane(int(ld_w1), int(jj)));
          const char* base = reinterpret_cast<const char*>(lane_u64(sp_lo, sp_hi, rk));
          slot_set(v, j, ld16<(NTM & NT_SRC) != 0>(base + xl));
        }
        next += m;
      }
      const U A = (w0 & CI_A_Y) ? y : sget((w0 >> 8) & 0xffu);
      U val = A;
      if (w0 & CI_COMBINE) {
        const U B = (w0 & CI_B_Y) ? y : sget((w0 >> 16) & 0xffu);
        y = combine16<DT, OP>(A, B);
        if (w0 & CI_WRITE) sset(w0 >> 24, y);
        val = y;
      }
      if constexpr (NA > 0) {
        const uint32_t shift = uint32_t(__builtin_amdgcn_readlane(int(op_w1), int(k))) & 3u;
        if (any) acc.add(k, unit_words<DT>(val, x, s0, s1, full, shift));
      } else if constexpr (MERGED) {
        const uint32_t shift = uint32_t(__builtin_amdgcn_readlane(int(op_w1), int(k))) & 3u;
        const uint64_t w = any ? unit_words<DT>(val, x, s0, s1, full, shift) : 0;
        push_op<0>(acc, w, k, lane, mine);  // every lane takes part
      }
    }
    if constexpr (MERGED) mine += flush_ops<0>(acc, nop, 0, lane);
    // Batched programs: every load of this tile has been consumed (each leaf
    // an op or a store reads); an explicit wait tells the compiler so, which
    // it cannot see across the dynamic op loop, and would otherwise wait for
    // every outstanding load before each leaf load of the next tile's first
    // batch.  (The other variants issue their first loads in branches of
    // their own and measure faster without it.)
    if constexpr (BT) __builtin_amdgcn_s_waitcnt(0);
    for (uint32_t j = 0; j < nstore; ++j) {
      const uint32_t w0 = uint32_t(__builtin_amdgcn_readlane(int(st_w0), int(j)));
      const uint32_t rk = uint32_t(__builtin_amdgcn_readlane(int(st_w1), int(j)));
      const U val = (w0 & CI_A_Y) ? y : sget((w0 >> 8) & 0xffu);
      char* base = reinterpret_cast<char*>(lane_u64(rp_lo, rp_hi, rk));
      if (full) st16<(NTM & NT_DST) != 0>(base + x, val);
      else if (any) store_part<DT>(base + x, val, x, s0, s1);
    }
  }
  // op k's wave total goes to one lane, which stores it in this work group's
  // own slot: no atomics, every slot written once per call
  if constexpr (NA > 0) {
    for (uint32_t k = 0; k < nop; ++k) {
      const uint64_t tot = wave_sum(acc.get(k));
      if (lane == k) mine = tot;
    }
    if (lane < nop) *gptr<uint64_t>(reinterpret_cast<char*>(a.partial + wk.part + lane)) = mine;
  } else if constexpr (MERGED) {
    const uint32_t o = op_of_lane(lane);  // a permutation of 0 .. 63
    if (o < nop) *gptr<uint64_t>(reinterpret_cast<char*>(a.partial + wk.part + o)) = mine;
  }
}

// Row checksums from the column kernel's partial sums, in two launches: work
// group (r, q) adds slice q (of COL_FOLD_SLICES) of the slots row r's ColRefs
// name into tmp[r * COL_FOLD_SLICES + q]; then one wave per row adds its
// slices into out[r].  A row of the headline call has 8,000-33,000 slots,
// which one work group per row would take longer to add than the slices do.
__global__ __launch_bounds__(BLOCK_THREADS) void col_fold_kernel(const ColRef* refs, const uint32_t* row_off,
                                                                  const uint64_t* partial, uint64_t* tmp) {
  __shared__ uint64_t wsum[BLOCK_THREADS / 64];
  const uint32_t r = blockIdx.x / COL_FOLD_SLICES, q = blockIdx.x % COL_FOLD_SLICES;
  const uint32_t i0 = cload(row_off + r), i1 = cload(row_off + r + 1);
  uint64_t acc = 0;
  for (uint32_t i = i0; i < i1; ++i) {
    const ColRef c = cload(refs + i);
    const uint32_t w0 = uint32_t((uint64_t(c.count) * q) / COL_FOLD_SLICES);
    const uint32_t w1 = uint32_t((uint64_t(c.count) * (q + 1)) / COL_FOLD_SLICES);
    for (uint32_t w = w0 + threadIdx.x; w < w1; w += BLOCK_THREADS)
      acc += *gptr<uint64_t>(reinterpret_cast<const char*>(partial + c.first + uint64_t(w) * c.stride));
  }
  acc = wave_sum(acc);
  if ((threadIdx.x & 63u) == 0) wsum[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t t = 0;
    for (int k = 0; k < BLOCK_THREADS / 64; ++k) t += wsum[k];
    *gptr<uint64_t>(reinterpret_cast<char*>(tmp + blockIdx.x)) = t;
  }
}

__global__ __launch_bounds__(BLOCK_THREADS) void col_fold_rows_kernel(const uint64_t* tmp, uint64_t* out,
                                                                       uint64_t nrows) {
  static_assert(COL_FOLD_SLICES <= 64, "one lane per slice");
  const uint64_t r = uint64_t(blockIdx.x) * (BLOCK_THREADS / 64) + (threadIdx.x >> 6);
  if (r >= nrows) return;  // uniform across the wave
  const uint32_t lane = threadIdx.x & 63u;
  const uint64_t v = lane < COL_FOLD_SLICES ? *gptr<uint64_t>(reinterpret_cast<const char*>(tmp + r * COL_FOLD_SLICES + lane)) : 0;
  const uint64_t t = wave_sum(v);
  if (lane == 0) *gptr<uint64_t>(reinterpret_cast<char*>(out + r)) = t;
}

// Row checksums equal to others already folded: out[r] = src[idx[r]] (the
// rows of an AllToAll run as one direct copy take the sums of the blocks they
// carry).  Every idx[r] indexes src; the host builds both.
__global__ __launch_bounds__(BLOCK_THREADS) void gather_sums_kernel(const uint32_t* idx, const uint64_t* src,
                                                                     uint64_t* out, uint64_t n) {
  const uint64_t r = uint64_t(blockIdx.x) * BLOCK_THREADS + threadIdx.x;
  if (r >= n) return;
  const uint32_t i = *gptr<uint32_t>(reinterpret_cast<const char*>(idx + r));
  *gptr<uint64_t>(reinterpret_cast<char*>(out + r)) = *gptr<uint64_t>(reinterpret_cast<const char*>(src + i));
}

template <int P>
using ColFn = void (*)(ColLaunchArgs<P>);

template <int DT, int OP, int NL, int NA, bool BT, int P>
ColFn<P> col_fn_nt(bool nt) {
  return nt ? col_kernel<DT, OP, NL, NA, NT_SRC | NT_DST, BT, P> : col_kernel<DT, OP, NL, NA, 0, BT, P>;
}

// Unbatched programs hold at most 8 slots; accs -1: no checksums, leaves in
// pairs, at most 16 work groups per CU; checksums of up to 8 ops: merged
// wave sums, the leaves in pairs (one leaf: alone); 9 .. 16 ops: a per-lane
// file; more: merged wave sums.  Batched programs: 8 slots, or 16 with slots
// 8 and up in LDS; checksums: merged wave sums.
template <int DT, int OP, bool BT, int P>
ColFn<P> col_fn_variant(int leaves, int accs, bool nt) {
  if constexpr (BT) {
    if (accs > 0) return leaves <= 8 ? col_fn_nt<DT, OP, 8, -1, BT, P>(nt) : col_fn_nt<DT, OP, 16, -1, BT, P>(nt);
    return leaves <= 8 ? col_fn_nt<DT, OP, 8, 0, BT, P>(nt) : col_fn_nt<DT, OP, 16, 0, BT, P>(nt);
  } else {
    if (accs < 0) return col_fn_nt<DT, OP, 8, -3, BT, P>(nt);
    if (accs > 16) return col_fn_nt<DT, OP, 8, -1, BT, P>(nt);
    if (accs > 8) return col_fn_nt<DT, OP, 8, 16, BT, P>(nt);
    if (accs > 0) return leaves <= 1 ? col_fn_nt<DT, OP, 8, -1, BT, P>(nt) : col_fn_nt<DT, OP, 8, -2, BT, P>(nt);
    return col_fn_nt<DT, OP, 8, 0, BT, P>(nt);
  }
}

// batched programs (over 16 leaves) only come with over 16 ranks: P = 64
template <int DT, int P>
ColFn<P> col_fn_op(int op, int leaves, int accs, bool batched, bool nt) {
  if constexpr (P > 16) {
    if (batched) {
      switch (op) {
        case OP_SUM: return col_fn_variant<DT, OP_SUM, true, P>(leaves, accs, nt);
        case OP_MAX: return col_fn_variant<DT, OP_MAX, true, P>(leaves, accs, nt);
        default: return col_fn_variant<DT, OP_MIN, true, P>(leaves, accs, nt);
      }
    }
  }
  switch (op) {
    case OP_SUM: return col_fn_variant<DT, OP_SUM, false, P>(leaves, accs, nt);
    case OP_MAX: return col_fn_variant<DT, OP_MAX, false, P>(leaves, accs, nt);
    default: return col_fn_variant<DT, OP_MIN, false, P>(leaves, accs, nt);
  }
}

template <int P>
ColFn<P> pick_col(int dtype, int op, int leaves, int accs, bool batched, bool nt) {
  switch (dtype) {
    case DT_I32: return col_fn_op<DT_I32, P>(op, leaves, accs, batched, nt);
    case DT_U8: return col_fn_op<DT_U8, P>(op, leaves, accs, batched, nt);
    case DT_F32: return col_fn_op<DT_F32, P>(op, leaves, accs, batched, nt);
    default: return col_fn_op<DT_BF16, P>(op, leaves, accs, batched, nt);
  }
}

template <int P>
hipError_t launch_col_p(const ColArgs& a, int dtype, int op, int leaves, int accs, bool batched, bool capped,
                        bool nt, uint32_t grid, hipStream_t stream) {
  ColLaunchArgs<P> c;
  c.work = a.work;
  c.code = a.code;
  c.partial = a.partial;
  for (int i = 0; i < P; ++i) {
    c.send[i] = a.p.send[i];
    c.recv[i] = a.p.recv[i];
  }
  // the variants for many-store programs reserve LDS they never touch, so
  // that a CU holds fewer of their work groups: the paired one at most 16 (4
  // waves per SIMD), capped batched ones fewer still
  const size_t lds = accs < 0 ? COL_PAIRED_LDS : capped ? COL_BATCHED_CAP_LDS : 0;
  hipLaunchKernelGGL(pick_col<P>(dtype, op, leaves, accs, batched, nt), dim3(grid), dim3(COL_THREADS), lds, stream, c);
  return hipGetLastError();
}

// Device memory of coll_allreduce_noalloc: its programs, work table, row
// references, partial checksum sums and fold slices, for callers that cannot
// allocate.  Each GPU the library runs on holds its own copy until the process
// ends.  In host code the name stands for no device address: host code uses
// the per-device address from noalloc_scratch() only.
static __device__ __align__(256) uint8_t scratch[COLL_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch_ptr;  // device -> address of that device's scratch

}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    it = g_scratch_ptr.emplace(dev, p).first;
  }
  *out = it->second;
  return hipSuccess;
}

hipError_t launch_col(const ColArgs& a, int nranks, int dtype, int op, int unit, int leaves, int accs, bool batched,
                      bool capped, bool nt, uint32_t grid, hipStream_t stream) {
  (void)unit;  // every variant takes 16-byte units
  if (nranks < 1 || nranks > COL_THREADS) return hipErrorInvalidValue;
  if (nranks <= 16 && !batched) return launch_col_p<16>(a, dtype, op, leaves, accs, batched, capped, nt, grid, stream);
  return launch_col_p<64>(a, dtype, op, leaves, accs, batched, capped, nt, grid, stream);
}

hipError_t launch_gather_sums(const uint32_t* idx, const uint64_t* src, uint64_t* out, uint64_t n,
                              hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const uint64_t grid = (n + BLOCK_THREADS - 1) / BLOCK_THREADS;
  if (grid > 0x7fffffffu) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_sums_kernel, dim3(uint32_t(grid)), dim3(BLOCK_THREADS), 0, stream, idx, src, out, n);
  return hipGetLastError();
}

hipError_t launch_col_fold(const ColRef* refs, const uint32_t* row_off, const uint64_t* partial, uint64_t* tmp,
                           uint64_t* out, uint64_t nrows, hipStream_t stream) {
  if (nrows == 0) return hipSuccess;
  if (nrows * COL_FOLD_SLICES > 0x7fffffffu) return hipErrorInvalidValue;
  hipLaunchKernelGGL(col_fold_kernel, dim3(uint32_t(nrows * COL_FOLD_SLICES)), dim3(BLOCK_THREADS), 0, stream, refs,
                     row_off, partial, tmp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint64_t per = BLOCK_THREADS / 64;
  hipLaunchKernelGGL(col_fold_rows_kernel, dim3(uint32_t((nrows + per - 1) / per)), dim3(BLOCK_THREADS), 0, stream,
                     tmp, out, nrows);
  return hipGetLastError();
}

}  // namespace coll
