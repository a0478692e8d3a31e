// Device kernels for gfx950 (CDNA4, wave64).
//
//  rows_kernel  copy and recv_and_reduce rows of a schedule ("集合通信算法延迟公式",
//               Ring ReduceScatter: each step a rank reduces the chunk it receives
//               into its own; the HCCL blog's recv_and_reduce).  One launch can run
//               every step of a call: each work group walks a host-built list of
//               row pieces inside the column groups it owns (see device_types.h),
//               so no flags or barriers are needed between steps.  128-bit loads
//               and stores, nontemporal hints per operand.
//  perm_kernel  in-place block shifts of the Bruck and Ring AllToAll rounds and their
//               final rotation ("集合通信算法延迟公式", AllToAll 算法怎么选): each
//               staging group is read into registers, the
//               work group meets at a barrier, then the values are written
//               permuted, so every read of a group precedes every write.
//  fill / calib plain helpers: clear checksum slots, stream copy / add.
//  spin         a register-only stand-in for compute, for overlap measurements.
//
// No MFMA: nothing here is a contraction.  Every kernel is bound by memory.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "device_types.h"
#include "launch.h"

namespace coll {

// ---- row kernel --------------------------------------------------------------

struct ItemView {
  const char* src;   // address of column 0 on the source side
  const char* dsrc;  // address of column 0 for the old destination value
  char* dst;         // address of column 0 on the destination side
  bool reduce;
  uint32_t shift;    // (-row start) mod 4
};

// One 16-byte column unit x of the item, clipped to [lo, hi).
//  vec: the unit is 16-byte aligned on every side, so it is loaded whole even
//    when the row covers it only in part (an aligned 16-byte block never
//    crosses a page, so the bytes outside the row are as readable as the ones
//    inside; this thread is the only one that touches the unit in any step, so
//    nothing else writes them meanwhile); only the row's elements are stored.
//  otherwise: element by element, in batches of up to 8 whose loads are all
//    issued before the batch's first store (a store may alias a later load's
//    address, so a load placed after it would wait a full memory round trip).
template <int DT, int OP, bool CKS, int NTM>
__device__ __forceinline__ void do_unit(const ItemView& v, uint64_t x, uint64_t lo, uint64_t hi, bool vec,
                                        uint64_t& acc) {
  if (x + 16 <= lo || x >= hi) return;
  constexpr int SZ = elem_size<DT>(), E = 16 / SZ;
  if (vec) {
    u32x4 s = ld16<(NTM & NT_SRC) != 0>(v.src + x);
    if (v.reduce) s = combine16<DT, OP>(ld16<(NTM & NT_DSRC) != 0>(v.dsrc + x), s);
    if (x >= lo && x + 16 <= hi) {
      st16<(NTM & NT_DST) != 0>(v.dst + x, s);
      if constexpr (CKS) acc += words16(s, v.shift * 8u);
      return;
    }
    // the row's bytes of this unit: [r0, r1) counted from x
    const uint32_t r0 = lo > x ? uint32_t(lo - x) : 0u, r1 = hi < x + 16 ? uint32_t(hi - x) : 16u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (uint32_t(e * SZ) >= r0 && uint32_t(e * SZ) < r1) {
        const uint32_t val = elem_of<DT>(s, e);
        st_elem<DT>(v.dst + x + e * SZ, val);
        if constexpr (CKS) acc += uint64_t(val << (8u * ((uint32_t(e * SZ) + v.shift) & 3u)));
      }
    }
    return;
  }
  const uint32_t r0 = lo > x ? uint32_t(lo - x) : 0u, r1 = hi < x + 16 ? uint32_t(hi - x) : 16u;
  constexpr int B = E < 8 ? E : 8;  // elements per batch of loads (bounds the registers held)
#pragma unroll
  for (int e0 = 0; e0 < E; e0 += B) {
    uint32_t s[B], d[B];
#pragma unroll
    for (int e = 0; e < B; ++e) {
      const uint32_t b = uint32_t((e0 + e) * SZ);
      const bool in = b >= r0 && b < r1;
      s[e] = in ? ld_elem<DT>(v.src + x + b) : 0u;
      d[e] = in && v.reduce ? ld_elem<DT>(v.dsrc + x + b) : 0u;
    }
#pragma unroll
    for (int e = 0; e < B; ++e) {
      const uint32_t b = uint32_t((e0 + e) * SZ);
      if (b >= r0 && b < r1) {
        const uint32_t val = v.reduce ? combine_elem<DT, OP>(d[e], s[e]) : s[e];
        st_elem<DT>(v.dst + x + b, val);
        if constexpr (CKS) acc += uint64_t(val << (8u * ((b + v.shift) & 3u)));
      }
    }
  }
}

// U full, aligned units at x0, x0 + 4 KiB, ...: all loads issued before the stores.
template <int U, int DT, int OP, bool CKS, int NTM>
__device__ __forceinline__ void do_batch(const ItemView& v, uint64_t x0, uint64_t& acc) {
  u32x4 s[U];
#pragma unroll
  for (int k = 0; k < U; ++k) s[k] = ld16<(NTM & NT_SRC) != 0>(v.src + x0 + uint64_t(k) * TILE_BYTES);
  if (v.reduce) {
    u32x4 d[U];
#pragma unroll
    for (int k = 0; k < U; ++k) d[k] = ld16<(NTM & NT_DSRC) != 0>(v.dsrc + x0 + uint64_t(k) * TILE_BYTES);
#pragma unroll
    for (int k = 0; k < U; ++k) s[k] = combine16<DT, OP>(d[k], s[k]);
  }
#pragma unroll
  for (int k = 0; k < U; ++k) {
    st16<(NTM & NT_DST) != 0>(v.dst + x0 + uint64_t(k) * TILE_BYTES, s[k]);
    if constexpr (CKS) acc += words16(s[k], v.shift * 8u);
  }
}

__device__ __forceinline__ ItemView view_of(const RowsArgs& a, const DevItem& it) {
  ItemView v;
  v.src = reinterpret_cast<const char*>((it.flags & ITEM_SRC_SEND) ? a.p.send[it.src_rank]
                                                                   : a.p.recv[it.src_rank]) + it.src_delta;
  v.dsrc = reinterpret_cast<const char*>((it.flags & ITEM_DSRC_SEND) ? a.p.send[it.dst_rank]
                                                                     : a.p.recv[it.dst_rank]) + it.dst_delta;
  v.dst = reinterpret_cast<char*>(a.p.recv[it.dst_rank]) + it.dst_delta;
  v.reduce = (it.flags & ITEM_REDUCE) != 0;
  v.shift = (it.flags >> ITEM_CKS_SHIFT) & 3u;
  return v;
}

// One piece: columns [col0, col1) of one row, inside one column group.  Thread t
// handles bytes [16t, 16t + 16) of every 4 KiB tile the piece touches.
template <int DT, int OP, bool CKS, int NTM>
__device__ __forceinline__ void do_piece(const RowsArgs& a, const DevItem& it, uint64_t tofs, uint64_t& acc) {
  const ItemView v = view_of(a, it);
  const bool vec = a.bases16 && (it.flags & ITEM_VEC);
  const uint64_t t0 = it.col0 / TILE_BYTES, t1 = (it.col1 - 1) / TILE_BYTES;
  if (!vec) {
    for (uint64_t t = t0; t <= t1; ++t) do_unit<DT, OP, CKS, NTM>(v, t * TILE_BYTES + tofs, it.col0, it.col1, false, acc);
    return;
  }
  // whole tiles [m0, m1) go through batched loads; a partly covered first or
  // last tile (a row that starts or ends inside a tile) unit by unit
  const uint64_t m0 = (it.col0 + TILE_BYTES - 1) / TILE_BYTES, m1 = it.col1 / TILE_BYTES;
  if (m0 >= m1) {
    for (uint64_t t = t0; t <= t1; ++t) do_unit<DT, OP, CKS, NTM>(v, t * TILE_BYTES + tofs, it.col0, it.col1, true, acc);
    return;
  }
  if (t0 < m0) do_unit<DT, OP, CKS, NTM>(v, t0 * TILE_BYTES + tofs, it.col0, it.col1, true, acc);
  uint64_t t = m0;
  for (; t + 4 <= m1; t += 4) do_batch<4, DT, OP, CKS, NTM>(v, t * TILE_BYTES + tofs, acc);
  for (; t < m1; ++t) do_batch<1, DT, OP, CKS, NTM>(v, t * TILE_BYTES + tofs, acc);
  if (t1 >= m1) do_unit<DT, OP, CKS, NTM>(v, t1 * TILE_BYTES + tofs, it.col0, it.col1, true, acc);
}

// A piece of at most FWD_TILES whole tiles (fwd_eligible), for the forwarding
// variant: `held[k]` holds the unit this thread stored in tile k of the
// previous eligible piece of its list.  An ITEM_SRC_FWD / ITEM_DSRC_FWD piece
// takes its source / old destination from there instead of loading what this
// thread itself just stored; every other operand is loaded, all loads first.
// The piece's results replace `held`; an ITEM_NO_STORE piece does not store them.
template <int DT, int OP, bool CKS, int NTM>
__device__ __forceinline__ void do_piece_fwd(const RowsArgs& a, const DevItem& it, uint64_t tofs,
                                             u32x4 (&held)[FWD_TILES], uint64_t& acc) {
  const ItemView v = view_of(a, it);
  const uint32_t nt = uint32_t((it.col1 - it.col0) / TILE_BYTES);
  const uint64_t x0 = it.col0 + tofs;
  const bool fs = (it.flags & ITEM_SRC_FWD) != 0, fd = (it.flags & ITEM_DSRC_FWD) != 0;
  const bool store = (it.flags & ITEM_NO_STORE) == 0;
  u32x4 s[FWD_TILES], d[FWD_TILES];
#pragma unroll
  for (uint32_t k = 0; k < FWD_TILES; ++k) {
    if (k < nt) {
      if (!fs) s[k] = ld16<(NTM & NT_SRC) != 0>(v.src + x0 + uint64_t(k) * TILE_BYTES);
      if (v.reduce && !fd) d[k] = ld16<(NTM & NT_DSRC) != 0>(v.dsrc + x0 + uint64_t(k) * TILE_BYTES);
    }
  }
#pragma unroll
  for (uint32_t k = 0; k < FWD_TILES; ++k) {
    if (k < nt) {
      u32x4 y = fs ? held[k] : s[k];
      if (v.reduce) y = combine16<DT, OP>(fd ? held[k] : d[k], y);
      if (store) st16<(NTM & NT_DST) != 0>(v.dst + x0 + uint64_t(k) * TILE_BYTES, y);
      held[k] = y;
      if constexpr (CKS) acc += words16(y, v.shift * 8u);
    }
  }
}

__device__ __forceinline__ bool one_tile(const DevItem& it) {
  return it.col0 / TILE_BYTES == (it.col1 - 1) / TILE_BYTES;
}

// A run of up to RUN_MAX pieces that each lie inside one tile and may run
// together (same step, no common destination bytes: ITEM_BATCH_NEXT); bit k
// of `mine` is set for the members this wave has bytes in.  Every lane issues
// the loads of its whole unit in every such piece first, then combines and
// stores, so the run costs one memory round trip, not one per piece.  Units a
// piece covers only in part take the element path afterwards.
template <int DT, int OP, bool CKS, int NTM>
__device__ __forceinline__ void do_run(const RowsArgs& a, const DevItem (&r)[RUN_MAX], uint32_t mine, uint64_t tofs) {
  u32x4 s[RUN_MAX], d[RUN_MAX];
  bool whole[RUN_MAX];
#pragma unroll
  for (uint32_t k = 0; k < RUN_MAX; ++k) {
    whole[k] = false;
    if (mine & (1u << k)) {
      const ItemView v = view_of(a, r[k]);
      const uint64_t x = (r[k].col0 / TILE_BYTES) * TILE_BYTES + tofs;
      whole[k] = a.bases16 && (r[k].flags & ITEM_VEC) && x >= r[k].col0 && x + 16 <= r[k].col1;
      if (whole[k]) {
        s[k] = ld16<(NTM & NT_SRC) != 0>(v.src + x);
        if (v.reduce) d[k] = ld16<(NTM & NT_DSRC) != 0>(v.dsrc + x);
      }
    }
  }
#pragma unroll
  for (uint32_t k = 0; k < RUN_MAX; ++k) {
    if (mine & (1u << k)) {
      const ItemView v = view_of(a, r[k]);
      const uint64_t x = (r[k].col0 / TILE_BYTES) * TILE_BYTES + tofs;
      uint64_t acc = 0;
      if (whole[k]) {
        u32x4 y = s[k];
        if (v.reduce) y = combine16<DT, OP>(d[k], y);
        st16<(NTM & NT_DST) != 0>(v.dst + x, y);
        if constexpr (CKS) acc += words16(y, v.shift * 8u);
      } else {
        do_unit<DT, OP, CKS, NTM>(v, x, r[k].col0, r[k].col1, a.bases16 && (r[k].flags & ITEM_VEC), acc);
      }
      if constexpr (CKS) add_row_sum(a.sums, r[k].row, acc);
    }
  }
}

// Work-list entries held across a wave: lane l keeps the 12 words of entry
// base + l.  One coalesced load fills 64 entries; an entry is then read into
// scalar registers with v_readlane, so walking a list of many small pieces
// costs no memory round trip per entry (a load of the entry inside the loop
// would be a vector load, and waiting for it would also wait for the stores
// of the piece before).
struct LaneList {
  uint32_t w[12];
  uint32_t base;
};

__device__ __forceinline__ void lane_fill(LaneList& c, const DevItem* list, uint32_t base, uint32_t e1) {
  c.base = base;
  const uint32_t i = base + (threadIdx.x & 63u);
#pragma unroll
  for (int q = 0; q < 12; ++q) c.w[q] = 0;
  if (i < e1) {
    const char* p = reinterpret_cast<const char*>(list + i);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const u32x4 v = *gptr<u32x4>(p + 16 * q);
      c.w[4 * q] = v.x;
      c.w[4 * q + 1] = v.y;
      c.w[4 * q + 2] = v.z;
      c.w[4 * q + 3] = v.w;
    }
  }
}

// word q of entry e (10: flags, 11: the wave mask)
template <int Q>
__device__ __forceinline__ uint32_t lane_word(const LaneList& c, uint32_t e) {
  return __builtin_amdgcn_readlane(c.w[Q], e - c.base);
}

__device__ __forceinline__ DevItem lane_get(const LaneList& c, uint32_t e) {
  const uint32_t j = e - c.base;
  uint32_t x[12];
#pragma unroll
  for (int q = 0; q < 12; ++q) x[q] = __builtin_amdgcn_readlane(c.w[q], j);
  DevItem it;
  __builtin_memcpy(&it, x, sizeof(it));
  return it;
}

// Work group w walks its slice of the launch's work list in order (the host
// built it in step order; every piece of one column group is in one slice, so
// values written in one step are read back by the same threads in the next).
//
// FINE = false (lists of large pieces): the next entry is fetched before the
// current piece is processed; every piece goes alone.
// FINE = true (lists of small pieces; more registers, so launched only for
// them): entries come from a LaneList; a wave reads only the flags and wave
// mask of an entry it has no bytes in and moves on; a run of
// ITEM_BATCH_NEXT-linked pieces (each inside one tile, as the host builds
// them) is processed together.  Both orders are correct: runs never hold two
// pieces with common destination bytes.
template <int DT, int OP, bool CKS, int NTM, bool FINE, bool FWD>
__global__ __launch_bounds__(BLOCK_THREADS) void rows_kernel(const RowsArgs a) {
  const uint32_t e0 = cload(a.off + blockIdx.x), e1 = cload(a.off + blockIdx.x + 1);
  if (e0 >= e1) return;
  const uint64_t tofs = uint64_t(threadIdx.x) * 16u;
  if constexpr (FINE) {
    const uint32_t wbit = 1u << __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    LaneList c;
    lane_fill(c, a.list, e0, e1);
    uint32_t e = e0;
    while (e < e1) {
      if (e + RUN_MAX > c.base + 64u) lane_fill(c, a.list, e, e1);
      const uint32_t avail = e1 - e < RUN_MAX ? e1 - e : RUN_MAX;
      uint32_t n = 1, mine = (lane_word<11>(c, e) & wbit) ? 1u : 0u;
      uint32_t fl = lane_word<10>(c, e);
#pragma unroll
      for (uint32_t k = 1; k < RUN_MAX; ++k) {
        if (n == k && k < avail && (fl & ITEM_BATCH_NEXT)) {
          fl = lane_word<10>(c, e + k);
          if (lane_word<11>(c, e + k) & wbit) mine |= 1u << k;
          n = k + 1;
        }
      }
      if (n == 1) {
        if (mine) {
          const DevItem it = lane_get(c, e);
          uint64_t acc = 0;
          do_piece<DT, OP, CKS, NTM>(a, it, tofs, acc);
          if constexpr (CKS) add_row_sum(a.sums, it.row, acc);
        }
      } else if (mine) {
        // members are read whole (scalar registers); `mine` decides which run
        DevItem r[RUN_MAX];
#pragma unroll
        for (uint32_t k = 0; k < RUN_MAX; ++k) r[k] = lane_get(c, e + (k < n ? k : 0));
        do_run<DT, OP, CKS, NTM>(a, r, mine, tofs);
      }
      e += n;
    }
  } else {
    u32x4 held[FWD_TILES];  // FWD: this thread's units of the last eligible piece
    DevItem next = cload(a.list + e0);
    for (uint32_t e = e0; e < e1; ++e) {
      const DevItem it = next;
      if (e + 1 < e1) next = cload(a.list + e + 1);
      uint64_t acc = 0;
      if (FWD && a.bases16 && fwd_eligible(it.col0, it.col1, it.flags))
        do_piece_fwd<DT, OP, CKS, NTM>(a, it, tofs, held, acc);
      else
        do_piece<DT, OP, CKS, NTM>(a, it, tofs, acc);
      if constexpr (CKS) add_row_sum(a.sums, it.row, acc);
    }
  }
}

// ---- staged permutation kernel (AllToAll) -------------------------------------------

template <int U>
struct UnitT;
template <> struct UnitT<16> { typedef u32x4 T; };
template <> struct UnitT<8> { typedef uint64_t T; };
template <> struct UnitT<4> { typedef uint32_t T; };
template <> struct UnitT<2> { typedef uint16_t T; };
template <> struct UnitT<1> { typedef uint8_t T; };

template <int U, bool NT>
__device__ __forceinline__ typename UnitT<U>::T ld_unit(const char* p) {
  typedef typename UnitT<U>::T T;
  if constexpr (NT && U >= 4) return __builtin_nontemporal_load(gptr<T>(p));
  else return *gptr<T>(p);
}

template <int U, bool NT>
__device__ __forceinline__ void st_unit(char* p, typename UnitT<U>::T v) {
  typedef typename UnitT<U>::T T;
  if constexpr (NT && U >= 4) __builtin_nontemporal_store(v, gptr<T>(p));
  else *gptr<T>(p) = v;
}

template <int U>
__device__ __forceinline__ uint64_t unit_words(typename UnitT<U>::T v, uint64_t col) {
  if constexpr (U == 16) return words16(v, 0);
  else if constexpr (U == 8) return uint64_t(uint32_t(v)) + uint32_t(v >> 32);
  else if constexpr (U == 4) return v;
  else return uint64_t(uint32_t(v) << (8u * uint32_t(col & 3u)));
}

// Columns are unit indices inside a block; every staged row keeps its offset
// inside the block, so a tile of block columns is a closed world: work group w
// owns tiles w, w + G, ... and nothing outside it ever reads or writes them.
// A staging group is the gs rows that permute one set of cells (the N ranks'
// copies of one block slot in a Bruck or Ring round, or the N blocks of one rank in the
// final rotation).  Per group and tile, wave v takes rows v, v+4, ... of the
// group; lane l holds units l, l+64, ... (upl of them) of each such row in
// registers: all rows' sources are loaded, the work group meets at a barrier
// (every read of the group precedes every write), then the same lanes store
// the values to the rows' destinations.  A barrier ends each step.
// HOIST (groups of more than 32 rows, 9 to 16 or more per wave): a wave
// reads its rows' descriptors once per group, before the group's first tile,
// and issues every data load of a tile with no branch around it (a slot past
// the group's rows loads the group's last row again, a lane past the block's
// end the block's last unit: in bounds, never stored).  Otherwise each slot
// reads its row's descriptor in the tile loop, which makes each data load
// wait for the one before: measured on MI355X, that is faster up to 32 rows
// (Bruck bf16 8 x 256 MiB 2.64 against 2.80 ms, 32 x 128 MiB perm rounds
// 7.18 against 7.38 ms per call) and slower above (64 x 64 MiB 8.80 against
// 8.01 ms), where a wave holds more rows.
template <int U, int SLOTS, bool CKS, bool NT, bool HOIST>
__global__ __launch_bounds__(BLOCK_THREADS) void perm_kernel(const PermArgs a) {
  typedef typename UnitT<U>::T T;
  const uint32_t G = gridDim.x, w = blockIdx.x;
  // the wave index is the same for all 64 lanes: say so, so that row descriptors
  // and base addresses live in scalar registers
  const uint32_t lane = threadIdx.x & 63u, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t ncol = a.ncols_units;
  const uint32_t lg = a.lg_upl;
  const uint32_t tu = 64u << lg;            // units of one row in one tile
  const uint32_t ntiles = (ncol + tu - 1) / tu;
  for (uint32_t s = a.s0; s < a.s1; ++s) {
    const DevStep st = cload(a.steps + s);
    const uint32_t gs = st.gsize;
    const uint32_t ngroups = st.nitems / gs;
    for (uint32_t grp = 0; grp < ngroups && w < ntiles; ++grp) {
      const uint32_t ib = st.item0 + grp * gs;
      const char* src[SLOTS];
      char* dst[SLOTS];
      uint32_t row[SLOTS];
      if constexpr (HOIST) {
#pragma unroll
        for (int r = 0; r < SLOTS; ++r) {
          const uint32_t m = wave + 4u * (uint32_t(r) >> lg);
          const DevItem it = cload(a.items + ib + (m < gs ? m : gs - 1u));
          src[r] = reinterpret_cast<const char*>(a.p.recv[it.src_rank]) + it.src_delta;
          dst[r] = reinterpret_cast<char*>(a.p.recv[it.dst_rank]) + it.dst_delta;
          row[r] = it.row;
        }
      }
      for (uint32_t tile = w; tile < ntiles; tile += G) {
        const uint32_t c0 = tile * tu;
        T v[SLOTS];
#pragma unroll
        for (int r = 0; r < SLOTS; ++r) {
          const uint32_t c = c0 + lane + 64u * (uint32_t(r) & ((1u << lg) - 1u));
          if constexpr (HOIST) {
            v[r] = ld_unit<U, NT>(src[r] + uint32_t((c < ncol ? c : ncol - 1u) * U));
          } else {
            const uint32_t m = wave + 4u * (uint32_t(r) >> lg);
            if (m < gs) {  // uniform across the wave
              const DevItem it = cload(a.items + ib + m);
              const char* base = reinterpret_cast<const char*>(a.p.recv[it.src_rank]) + it.src_delta;
              if (c < ncol) v[r] = ld_unit<U, NT>(base + uint32_t(c * U));
            }
          }
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < SLOTS; ++r) {
          const uint32_t m = wave + 4u * (uint32_t(r) >> lg);
          if (m < gs) {  // uniform across the wave
            const uint32_t c = c0 + lane + 64u * (uint32_t(r) & ((1u << lg) - 1u));
            char* base;
            uint32_t rw;
            if constexpr (HOIST) {
              base = dst[r];
              rw = row[r];
            } else {
              const DevItem it = cload(a.items + ib + m);
              base = reinterpret_cast<char*>(a.p.recv[it.dst_rank]) + it.dst_delta;
              rw = it.row;
            }
            uint64_t acc = 0;
            if (c < ncol) {
              st_unit<U, NT>(base + uint32_t(c * U), v[r]);
              if constexpr (CKS) acc = unit_words<U>(v[r], uint64_t(c) * U);
            }
            if constexpr (CKS) add_row_sum(a.sums, rw, acc);
          }
        }
      }
    }
    __syncthreads();
  }
}

// ---- helpers -----------------------------------------------------------------------

__global__ void fill_u64_kernel(uint64_t* p, uint64_t n, uint64_t value) {
  for (uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += uint64_t(gridDim.x) * blockDim.x)
    *gptr<uint64_t>(reinterpret_cast<char*>(p + i)) = value;
}

// One wave per row: lane p loads partial slot p and sets it back to zero for
// the next call, the wave sums the loaded values.
__global__ __launch_bounds__(BLOCK_THREADS) void fold_sums_kernel(uint64_t* partial, uint64_t* out, uint64_t nrows) {
  static_assert(SUM_LANES == 64, "one lane per partial slot");
  const uint64_t r = uint64_t(blockIdx.x) * (BLOCK_THREADS / 64) + (threadIdx.x >> 6);
  if (r >= nrows) return;  // uniform across the wave
  char* slot = reinterpret_cast<char*>(partial + r * SUM_LANES + (threadIdx.x & 63u));
  const uint64_t v = *gptr<uint64_t>(slot);
  *gptr<uint64_t>(slot) = 0;
  const uint64_t t = wave_sum(v);
  if ((threadIdx.x & 63u) == 0) *gptr<uint64_t>(reinterpret_cast<char*>(out + r)) = t;
}

// Independent copy rows (Pairwise AllToAll) in the shape of the plain copy
// stream: a one-wave work group copies one 1 KiB tile of one row, 16 bytes
// per lane, nontemporal when NT.  Nothing is read twice, so every block is
// read once and written once.  With checksums each work group stores the u64
// sum of the words it wrote to a slot of its own; the column kernel's fold
// adds a row's slots.
template <bool CKS, bool NT>
__global__ __launch_bounds__(64) void copy_rows_kernel(const CopyRowsArgs a) {
  const uint32_t r = blockIdx.x / a.wgs_per_row, q = blockIdx.x % a.wgs_per_row;
  const CopyRow row = cload(a.rows + r);
  const uint64_t off = uint64_t(q) * 1024u + uint64_t(threadIdx.x) * 16u;
  // lanes past the row's end (its last tile) copy nothing; they load the
  // row's last unit so that the load needs no branch
  const bool in = off < a.row_bytes;
  const uint64_t offl = in ? off : a.row_bytes - 16u;
  const char* src = reinterpret_cast<const char*>(a.p.send[row.src]) + row.src_off;
  char* dst = reinterpret_cast<char*>(a.p.recv[row.dst]) + row.dst_off;
  const u32x4 v = ld16<NT>(src + offl);
  if (in) st16<NT>(dst + off, v);
  if constexpr (CKS) {
    // rows start at multiples of 16 bytes: no rotation
    const uint64_t t = wave_sum(in ? words16(v, 0) : 0);
    if (threadIdx.x == 0) *gptr<uint64_t>(reinterpret_cast<char*>(a.partial + blockIdx.x)) = t;
  }
}

// Plain streams for the achievable-rate ceiling: one-wave work groups, one
// 16-byte unit per lane, nontemporal loads and stores, as the column kernel
// runs.  Measured on MI355X for a 2 GiB copy, 64-lane work groups of one 1
// KiB tile each: 6.71 TB/s; four tiles each 6.15; 256-lane work groups of
// four 4 KiB tiles 5.77; 32 or 64 bytes per lane (two or four adjacent
// 16-byte accesses) 3.7 and 1.4.
constexpr int CALIB_THREADS = 64;

template <bool ADD>
__global__ __launch_bounds__(CALIB_THREADS) void calib_kernel(char* dst, const char* a, const char* b, uint64_t units) {
  const uint64_t u = uint64_t(blockIdx.x) * CALIB_THREADS + threadIdx.x;
  if (u >= units) return;
  u32x4 x = ld16<true>(a + u * 16);
  if constexpr (ADD) x = combine16<DT_F32, OP_SUM>(x, ld16<true>(b + u * 16));
  st16<true>(dst + u * 16, x);
}

// Access patterns of the column kernel's programs, without the programs:
// one-wave work groups, one 1 KiB tile per buffer (16 B per lane), L loads at
// the same offset of L buffers (all in flight together, eight at a time),
// their u32 word sum, then S stores of it at the same offset of S buffers;
// nontemporal.  L = 0 stores a constant (a fill).  Buffers may repeat (in
// place: the stores go where the loads came from).  Lane r holds load
// buffer r's and store buffer r's addresses.  A launch may reserve LDS it
// never touches, to cap the work groups a CU holds at once.
template <int L, int S>
__global__ __launch_bounds__(64) void calib_pattern_kernel(const RankPtrs p) {
  const uint32_t lane = threadIdx.x;
  const uint64_t lp = p.send[lane], sp = p.recv[lane];
  const uint32_t lp_lo = uint32_t(lp), lp_hi = uint32_t(lp >> 32), sp_lo = uint32_t(sp), sp_hi = uint32_t(sp >> 32);
  const uint64_t off = uint64_t(blockIdx.x) * 1024u + uint64_t(lane) * 16u;
  u32x4 acc = {lane, uint32_t(blockIdx.x), 0u, 0u};
  if constexpr (L > 0) acc = u32x4{0u, 0u, 0u, 0u};
  constexpr int B = L < 8 ? L : 8;
#pragma unroll
  for (int b = 0; b < L; b += B) {
    u32x4 v[B > 0 ? B : 1];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const uint64_t base = uint64_t(uint32_t(__builtin_amdgcn_readlane(int(lp_lo), b + j))) |
                            (uint64_t(uint32_t(__builtin_amdgcn_readlane(int(lp_hi), b + j))) << 32);
      v[j] = ld16<true>(reinterpret_cast<const char*>(base) + off);
    }
#pragma unroll
    for (int j = 0; j < B; ++j) acc += v[j];
  }
#pragma unroll
  for (int k = 0; k < S; ++k) {
    const uint64_t base = uint64_t(uint32_t(__builtin_amdgcn_readlane(int(sp_lo), k))) |
                          (uint64_t(uint32_t(__builtin_amdgcn_readlane(int(sp_hi), k))) << 32);
    st16<true>(reinterpret_cast<char*>(base) + off, acc);
  }
}

// ---- host-side dispatch ---------------------------------------------------------------

typedef void (*RowsFn)(RowsArgs);

template <int DT, int OP, bool CKS>
static RowsFn rows_fn_nt(uint32_t nt, bool fine, bool fwd) {
  // lists of small pieces come from small footprints, which stay in the
  // caches: the fine variant exists for the all-cached mask only; the
  // forwarding variant for the masks the automatic policy picks for it (none,
  // source loads, source loads and stores)
  if (fine && (nt & 7u) == 0) return rows_kernel<DT, OP, CKS, 0, true, false>;
  if (fwd && (nt & 7u) == 0) return rows_kernel<DT, OP, CKS, 0, false, true>;
  if (fwd && (nt & 7u) == NT_SRC) return rows_kernel<DT, OP, CKS, NT_SRC, false, true>;
  if (fwd && (nt & 7u) == (NT_SRC | NT_DST)) return rows_kernel<DT, OP, CKS, NT_SRC | NT_DST, false, true>;
  switch (nt & 7u) {
    case 0: return rows_kernel<DT, OP, CKS, 0, false, false>;
    case 1: return rows_kernel<DT, OP, CKS, 1, false, false>;
    case 2: return rows_kernel<DT, OP, CKS, 2, false, false>;
    case 3: return rows_kernel<DT, OP, CKS, 3, false, false>;
    case 4: return rows_kernel<DT, OP, CKS, 4, false, false>;
    case 5: return rows_kernel<DT, OP, CKS, 5, false, false>;
    case 6: return rows_kernel<DT, OP, CKS, 6, false, false>;
    default: return rows_kernel<DT, OP, CKS, 7, false, false>;
  }
}

template <int DT, int OP>
static RowsFn rows_fn(bool cks, uint32_t nt, bool fine, bool fwd) {
  return cks ? rows_fn_nt<DT, OP, true>(nt, fine, fwd) : rows_fn_nt<DT, OP, false>(nt, fine, fwd);
}

template <int DT>
static RowsFn rows_fn_op(int op, bool cks, uint32_t nt, bool fine, bool fwd) {
  switch (op) {
    case OP_SUM: return rows_fn<DT, OP_SUM>(cks, nt, fine, fwd);
    case OP_MAX: return rows_fn<DT, OP_MAX>(cks, nt, fine, fwd);
    default: return rows_fn<DT, OP_MIN>(cks, nt, fine, fwd);
  }
}

static RowsFn pick_rows(int dtype, int op, bool cks, uint32_t nt, bool fine, bool fwd) {
  switch (dtype) {
    case DT_I32: return rows_fn_op<DT_I32>(op, cks, nt, fine, fwd);
    case DT_U8: return rows_fn_op<DT_U8>(op, cks, nt, fine, fwd);
    case DT_F32: return rows_fn_op<DT_F32>(op, cks, nt, fine, fwd);
    default: return rows_fn_op<DT_BF16>(op, cks, nt, fine, fwd);
  }
}

typedef void (*PermFn)(PermArgs);

template <int U, int SLOTS, bool HOIST>
static PermFn perm_fn(bool cks, bool nt) {
  if (cks) return nt ? perm_kernel<U, SLOTS, true, true, HOIST> : perm_kernel<U, SLOTS, true, false, HOIST>;
  return nt ? perm_kernel<U, SLOTS, false, true, HOIST> : perm_kernel<U, SLOTS, false, false, HOIST>;
}

template <int SLOTS, bool HOIST>
static PermFn pick_perm_slots(int unit, bool cks, bool nt) {
  switch (unit) {
    case 16: return perm_fn<16, SLOTS, HOIST>(cks, nt);
    case 8: return perm_fn<8, SLOTS, HOIST>(cks, nt);
    case 4: return perm_fn<4, SLOTS, HOIST>(cks, nt);
    case 2: return perm_fn<2, SLOTS, HOIST>(cks, nt);
    default: return perm_fn<1, SLOTS, HOIST>(cks, nt);
  }
}

// slots 8 (17-32 ranks), 16 (up to 16 ranks; hoisted for 33-64), 32 (hoisted, over 64)
static PermFn pick_perm(int unit, int slots, bool hoist, bool cks, bool nt) {
  if (slots <= 8) return pick_perm_slots<8, false>(unit, cks, nt);
  if (slots > 16) return pick_perm_slots<32, true>(unit, cks, nt);
  return hoist ? pick_perm_slots<16, true>(unit, cks, nt) : pick_perm_slots<16, false>(unit, cks, nt);
}

hipError_t launch_rows(const RowsArgs& a, int dtype, int op, bool cks, uint32_t nt, bool fine, bool fwd,
                       uint32_t grid, hipStream_t stream) {
  RowsFn f = pick_rows(dtype, op, cks, nt, fine, fwd);
  hipLaunchKernelGGL(f, dim3(grid), dim3(BLOCK_THREADS), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_perm(const PermArgs& a, int unit, int slots, bool hoist, bool cks, uint32_t grid,
                       hipStream_t stream) {
  PermFn f = pick_perm(unit, slots, hoist, cks, a.nontemporal != 0);
  hipLaunchKernelGGL(f, dim3(grid), dim3(BLOCK_THREADS), 0, stream, a);
  return hipGetLastError();
}

int rows_blocks_per_cu(int dtype, int op, bool cks, uint32_t nt) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, pick_rows(dtype, op, cks, nt, false, false), BLOCK_THREADS,
                                                   0) !=
      hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

int perm_blocks_per_cu(int unit, int slots, bool hoist, bool cks, bool nt) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, pick_perm(unit, slots, hoist, cks, nt), BLOCK_THREADS, 0) !=
      hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

// Four independent fp32 FMA chains per thread, `iters` rounds, all in
// registers; one float per thread is stored at the end so that the work cannot
// be dropped.  No other memory traffic: the kernel occupies compute units and
// issue slots only, like the compute a collective is meant to hide behind.
__global__ __launch_bounds__(BLOCK_THREADS) void spin_kernel(float* out, uint32_t iters) {
  const uint32_t t = blockIdx.x * BLOCK_THREADS + threadIdx.x;
  float a0 = 1.0f + float(t & 1023u) * 1e-6f, a1 = a0 + 0.25f, a2 = a0 + 0.5f, a3 = a0 + 0.75f;
  const float m = 0.9999999f, c = 1e-7f;
  for (uint32_t i = 0; i < iters; ++i) {
    a0 = __builtin_fmaf(a0, m, c);
    a1 = __builtin_fmaf(a1, m, c);
    a2 = __builtin_fmaf(a2, m, c);
    a3 = __builtin_fmaf(a3, m, c);
  }
  *gptr<float>(reinterpret_cast<char*>(out + t)) = (a0 + a1) + (a2 + a3);
}

hipError_t launch_spin(float* out, uint32_t iters, uint32_t grid, hipStream_t stream) {
  hipLaunchKernelGGL(spin_kernel, dim3(grid), dim3(BLOCK_THREADS), 0, stream, out, iters);
  return hipGetLastError();
}

hipError_t launch_fill_u64(uint64_t* p, uint64_t n, uint64_t value, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const uint32_t grid = uint32_t(n < 256 * 1024 ? (n + BLOCK_THREADS - 1) / BLOCK_THREADS : 1024);
  hipLaunchKernelGGL(fill_u64_kernel, dim3(grid), dim3(BLOCK_THREADS), 0, stream, p, n, value);
  return hipGetLastError();
}

hipError_t launch_fold_sums(uint64_t* partial, uint64_t* out, uint64_t nrows, hipStream_t stream) {
  if (nrows == 0) return hipSuccess;
  const uint64_t rows_per_block = BLOCK_THREADS / 64;
  const uint32_t grid = uint32_t((nrows + rows_per_block - 1) / rows_per_block);
  hipLaunchKernelGGL(fold_sums_kernel, dim3(grid), dim3(BLOCK_THREADS), 0, stream, partial, out, nrows);
  return hipGetLastError();
}

hipError_t launch_copy_rows(const CopyRowsArgs& a, uint64_t nrows, bool cks, bool nt, hipStream_t stream) {
  const uint64_t g = nrows * uint64_t(a.wgs_per_row);
  if (g == 0) return hipSuccess;
  if (g > 0x7fffffffu || a.row_bytes % 16u) return hipErrorInvalidValue;
  const uint32_t grid = uint32_t(g);
  auto fn = cks ? (nt ? copy_rows_kernel<true, true> : copy_rows_kernel<true, false>)
                : (nt ? copy_rows_kernel<false, true> : copy_rows_kernel<false, false>);
  hipLaunchKernelGGL(fn, dim3(grid), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_calib_pattern(const RankPtrs& p, int nloads, int nstores, uint64_t bytes, uint32_t lds_bytes,
                                hipStream_t stream) {
  void (*f)(RankPtrs) = nullptr;
  if (nloads == 0 && nstores == 1) f = calib_pattern_kernel<0, 1>;
  else if (nloads == 8 && nstores == 8) f = calib_pattern_kernel<8, 8>;
  else if (nloads == 8 && nstores == 1) f = calib_pattern_kernel<8, 1>;
  else if (nloads == 1 && nstores == 7) f = calib_pattern_kernel<1, 7>;
  else if (nloads == 64 && nstores == 1) f = calib_pattern_kernel<64, 1>;
  else if (nloads == 1 && nstores == 63) f = calib_pattern_kernel<1, 63>;
  if (!f || bytes % 1024u) return hipErrorInvalidValue;
  const uint64_t g = bytes / 1024u;
  if (g == 0) return hipSuccess;
  if (g > 0x7fffffffu) return hipErrorInvalidValue;
  hipLaunchKernelGGL(f, dim3(uint32_t(g)), dim3(64), lds_bytes, stream, p);
  return hipGetLastError();
}

hipError_t launch_calib(void* dst, const void* a, const void* b, uint64_t bytes, hipStream_t stream) {
  const uint64_t units = bytes / 16;
  const uint64_t g = (units + CALIB_THREADS - 1) / CALIB_THREADS;
  if (g == 0) return hipSuccess;
  if (g > 0x7fffffffu) return hipErrorInvalidValue;
  const uint32_t grid = uint32_t(g);
  if (b)
    hipLaunchKernelGGL(calib_kernel<true>, dim3(grid), dim3(CALIB_THREADS), 0, stream, reinterpret_cast<char*>(dst),
                       reinterpret_cast<const char*>(a), reinterpret_cast<const char*>(b), units);
  else
    hipLaunchKernelGGL(calib_kernel<false>, dim3(grid), dim3(CALIB_THREADS), 0, stream, reinterpret_cast<char*>(dst),
                       reinterpret_cast<const char*>(a), nullptr, units);
  return hipGetLastError();
}

}  // namespace coll
