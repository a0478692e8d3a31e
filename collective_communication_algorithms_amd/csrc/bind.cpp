#include "bind.h"

#include <algorithm>
#include <iterator>
#include <map>
#include <stdexcept>

namespace coll {
namespace {

// Disjoint element intervals of one rank's receive buffer written so far.
class Written {
 public:
  void add(int64_t a, int64_t b) {
    if (a >= b) return;
    auto it = iv_.upper_bound(a);
    if (it != iv_.begin() && std::prev(it)->second >= a) {
      --it;
      a = it->first;
    }
    while (it != iv_.end() && it->first <= b) {
      b = std::max(b, it->second);
      it = iv_.erase(it);
    }
    iv_[a] = b;
  }
  // Boundaries inside (a, b) where written / unwritten changes.
  void cuts(int64_t a, int64_t b, std::vector<int64_t>& out) const {
    auto it = iv_.upper_bound(a);
    if (it != iv_.begin()) --it;
    for (; it != iv_.end() && it->first < b; ++it) {
      if (it->first > a) out.push_back(it->first);
      if (it->second > a && it->second < b) out.push_back(it->second);
    }
  }
  bool covers(int64_t a, int64_t b) const {  // [a, b) entirely written (a < b)
    auto it = iv_.upper_bound(a);
    if (it == iv_.begin()) return false;
    --it;
    return it->first <= a && it->second >= b;
  }
  // Parts of [a, b) not yet written.
  void gaps(int64_t a, int64_t b, std::vector<std::pair<int64_t, int64_t>>& out) const {
    int64_t x = a;
    auto it = iv_.upper_bound(a);
    if (it != iv_.begin()) --it;
    for (; it != iv_.end() && it->first < b; ++it) {
      if (it->second <= x) continue;
      if (it->first > x) out.push_back({x, std::min(it->first, b)});
      x = std::max(x, it->second);
      if (x >= b) break;
    }
    if (x < b) out.push_back({x, b});
  }

 private:
  std::map<int64_t, int64_t> iv_;
};

uint32_t vec_flag(int64_t src_delta, int64_t dst_delta) {
  return (src_delta % 16 == 0 && dst_delta % 16 == 0) ? ITEM_VEC : 0u;
}

uint32_t shift_flag(int64_t row_start_byte) {
  return uint32_t(((-row_start_byte) % 4 + 4) % 4) << ITEM_CKS_SHIFT;
}

}  // namespace

std::vector<std::pair<int64_t, int64_t>> defined_output(const Schedule& s, int rank) {
  const int64_t lo = (int64_t(rank) * s.count) / s.N, hi = (int64_t(rank + 1) * s.count) / s.N;
  switch (s.kind) {
    case COLL_K_REDUCESCATTER:
    case COLL_K_SCATTER: return {{lo, hi}};
    case COLL_K_GATHER:
    case COLL_K_REDUCE:
      if (rank == s.root) return {{0, s.count}};
      return {};
    default: return {{0, s.count}};
  }
}

Bound bind_schedule(const Schedule& s, int sz, bool inplace) {
  Bound b;
  b.nrows = int64_t(s.rows.size());
  b.defined.resize(size_t(s.N));
  for (int rank = 0; rank < s.N; ++rank)
    for (auto& reg : defined_output(s, rank))
      if (reg.second > reg.first) b.defined[size_t(rank)].push_back({uint64_t(reg.first * sz), uint64_t(reg.second * sz)});
  b.counts = count_schedule(s, sz);
  const bool a2a = s.kind == COLL_K_ALLTOALL;
  // staged AllToAll steps (Bruck's and the Ring's rounds, the final rotation)
  // are block permutations: they run in the permutation kernel, which needs
  // them after every ordinary step
  auto perm = [&](size_t si) { return a2a && si < s.steps.size() && s.steps[si].staged; };
  size_t first_perm = s.steps.size();
  for (size_t si = 0; si < s.steps.size(); ++si)
    if (perm(si)) {
      first_perm = si;
      break;
    }
  const bool has_perm = first_perm < s.steps.size();
  for (size_t si = first_perm; si < s.steps.size(); ++si)
    if (!perm(si)) throw std::logic_error("ordinary AllToAll step after a staged one");
  std::vector<std::vector<DevItem>> per_step(s.steps.size());
  std::vector<Written> written(a2a || inplace ? 0 : size_t(s.N));

  for (size_t si = 0; si < s.steps.size(); ++si) {
    const Step& st = s.steps[si];
    const bool perm_step = perm(si);
    for (int64_t ri = st.first; ri < st.first + st.nrows; ++ri) {
      const Row& r = s.rows[size_t(ri)];
      DevItem it{};
      it.row = uint32_t(ri);
      it.src_rank = uint16_t(r.src);
      it.dst_rank = uint16_t(r.dst);
      const int64_t row_start = r.dst_off * sz;
      if (perm_step) {
        // column = byte offset inside the block; the item moves one whole block
        it.col0 = 0;
        it.col1 = uint64_t(r.n * sz);
        it.src_delta = r.src_off * sz;
        it.dst_delta = r.dst_off * sz;
        it.flags = vec_flag(it.src_delta, it.dst_delta) | shift_flag(row_start);
        per_step[si].push_back(it);
        continue;
      }
      const int64_t sd = (r.src_off - r.dst_off) * sz;
      it.src_delta = sd;
      it.dst_delta = 0;
      const uint32_t base = (r.reduce ? ITEM_REDUCE : 0u) | vec_flag(sd, 0) | shift_flag(row_start);
      if (a2a || inplace) {
        it.col0 = uint64_t(r.dst_off * sz);
        it.col1 = uint64_t((r.dst_off + r.n) * sz);
        it.flags = base | (r.from_send ? ITEM_SRC_SEND : 0u);
        per_step[si].push_back(it);
        continue;
      }
      // Out of place: split where the source or the old destination changes
      // between "already written on the receive side" and "still only in send".
      const int64_t a = r.dst_off, z = r.dst_off + r.n;
      std::vector<int64_t> cut{a, z};
      written[size_t(r.src)].cuts(r.src_off, r.src_off + r.n, cut);  // src_off == dst_off here
      if (r.reduce) written[size_t(r.dst)].cuts(a, z, cut);
      std::sort(cut.begin(), cut.end());
      cut.erase(std::unique(cut.begin(), cut.end()), cut.end());
      for (size_t k = 0; k + 1 < cut.size(); ++k) {
        const int64_t lo = cut[k], hi = cut[k + 1];
        DevItem p = it;
        p.col0 = uint64_t(lo * sz);
        p.col1 = uint64_t(hi * sz);
        p.flags = base;
        if (!written[size_t(r.src)].covers(lo + (r.src_off - r.dst_off), hi + (r.src_off - r.dst_off)))
          p.flags |= ITEM_SRC_SEND;
        if (r.reduce && !written[size_t(r.dst)].covers(lo, hi)) p.flags |= ITEM_DSRC_SEND;
        per_step[si].push_back(p);
      }
      written[size_t(r.dst)].add(a, z);
    }
  }

  if (!a2a && !inplace) {
    // defined output that no row writes: copy it from send to receive
    std::vector<DevItem> copies;
    for (int rank = 0; rank < s.N; ++rank) {
      for (auto& reg : defined_output(s, rank)) {
        std::vector<std::pair<int64_t, int64_t>> g;
        written[size_t(rank)].gaps(reg.first, reg.second, g);
        for (auto& q : g) {
          if (q.second <= q.first) continue;
          DevItem it{};
          it.row = NO_ROW;
          it.src_rank = it.dst_rank = uint16_t(rank);
          it.col0 = uint64_t(q.first * sz);
          it.col1 = uint64_t(q.second * sz);
          it.flags = ITEM_SRC_SEND | ITEM_VEC;
          copies.push_back(it);
          b.counts.hbm_bytes += 2 * (q.second - q.first) * sz;
        }
      }
    }
    if (!copies.empty()) {
      if (per_step.empty()) per_step.emplace_back();
      per_step[0].insert(per_step[0].end(), copies.begin(), copies.end());
    }
  }

  uint64_t rows_cols = 0, perm_cols = 0;
  for (size_t si = 0; si < per_step.size(); ++si) {
    DevStep d{};
    d.item0 = uint32_t(b.items.size());
    d.nitems = uint32_t(per_step[si].size());
    const bool perm_step = perm(si);
    d.flags = perm_step ? STEP_STAGED : 0u;
    d.gsize = perm_step ? uint32_t(s.N) : 1u;
    // same-destination accumulation (a Double Binary Tree parent with two
    // children) must keep row order; every other step may be walked backwards
    if (!perm_step) {
      std::vector<const DevItem*> v;
      for (auto& it : per_step[si]) v.push_back(&it);
      std::sort(v.begin(), v.end(), [](const DevItem* x, const DevItem* y) {
        return x->dst_rank != y->dst_rank ? x->dst_rank < y->dst_rank : x->col0 < y->col0;
      });
      for (size_t x = 1; x < v.size(); ++x)
        if (v[x]->dst_rank == v[x - 1]->dst_rank && v[x]->col0 < v[x - 1]->col1) d.flags |= STEP_ORDERED;
    }
    for (auto& it : per_step[si]) {
      if (perm_step) perm_cols = std::max(perm_cols, it.col1);
      else rows_cols = std::max(rows_cols, it.col1);
      b.items.push_back(it);
    }
    b.steps.push_back(d);
  }
  const uint32_t nsteps = uint32_t(b.steps.size());
  if (nsteps == 0 || b.items.empty()) return b;
  if (has_perm) {
    if (first_perm > 0) {
      Phase p1;
      p1.kind = Phase::ROWS;
      p1.s0 = 0;
      p1.s1 = uint32_t(first_perm);
      p1.colspace = rows_cols;
      b.phases.push_back(p1);
    }
    if (perm_cols > 0) {
      Phase p2;
      p2.kind = Phase::PERM;
      p2.s0 = uint32_t(first_perm);
      p2.s1 = nsteps;
      p2.colspace = perm_cols;
      b.phases.push_back(p2);
    }
    const int64_t blk = perm_cols > 0 ? int64_t(perm_cols) : 16;
    b.perm_unit = 1;
    for (int u : {16, 8, 4, 2}) {
      if (blk % u == 0) {
        b.perm_unit = u;
        break;
      }
    }
  } else {
    Phase p;
    p.kind = Phase::ROWS;
    p.s0 = 0;
    p.s1 = nsteps;
    p.colspace = rows_cols;
    b.phases.push_back(p);
  }
  for (Phase& p : b.phases) {
    if (p.kind != Phase::ROWS) continue;
    for (uint32_t s = p.s0; s < p.s1; ++s)
      for (uint32_t i = 0; i < b.steps[s].nitems; ++i) {
        const DevItem& it = b.items[b.steps[s].item0 + i];
        for (uint64_t c : {it.col0, it.col1})
          if (c > 0 && c < p.colspace) p.bounds.push_back(c);
      }
    std::sort(p.bounds.begin(), p.bounds.end());
    p.bounds.erase(std::unique(p.bounds.begin(), p.bounds.end()), p.bounds.end());
  }
  return b;
}

// Waves of a work group with bytes in the piece: within a tile, wave w handles
// bytes [w * WAVE_BYTES, (w + 1) * WAVE_BYTES).
uint32_t wave_mask(const DevItem& x) {
  const uint32_t waves = BLOCK_THREADS / 64;
  if (x.col1 - x.col0 >= TILE_BYTES) return (1u << waves) - 1u;
  uint32_t m = 0;
  for (uint64_t t = x.col0 / TILE_BYTES; t <= (x.col1 - 1) / TILE_BYTES; ++t)
    for (uint32_t w = 0; w < waves; ++w) {
      const uint64_t lo = t * TILE_BYTES + w * WAVE_BYTES, hi = lo + WAVE_BYTES;
      if (x.col0 < hi && lo < x.col1) m |= 1u << w;
    }
  return m;
}

bool several_pieces_per_step(const Bound& b, const Phase& ph) {
  const uint64_t gb = uint64_t(BLOCKED_GROUP_TILES_REDUCE) * TILE_BYTES;
  uint64_t pieces = 0;
  for (uint32_t s = ph.s0; s < ph.s1; ++s)
    for (uint32_t i = 0; i < b.steps[s].nitems; ++i) {
      const DevItem& it = b.items[b.steps[s].item0 + i];
      if (it.col1 > it.col0) pieces += (it.col1 - 1) / gb - it.col0 / gb + 1;
    }
  const uint64_t groups = (ph.colspace + gb - 1) / gb;
  return pieces >= 2 * groups * uint64_t(ph.s1 - ph.s0);
}

uint64_t phase_segment(const Phase& ph) { return ph.colspace / (uint64_t(ph.bounds.size()) + 1); }

uint32_t resident_group_tiles(uint64_t colspace, uint64_t max_groups) {
  const uint64_t tiles = (colspace + TILE_BYTES - 1) / TILE_BYTES;
  uint32_t gt = 8;
  while (gt > 1 && tiles / gt < max_groups) gt >>= 1;
  return gt;
}

std::vector<uint64_t> group_cuts(const Phase& ph, uint64_t gbytes) {
  std::vector<uint64_t> cuts;
  for (uint64_t c : ph.bounds)
    if (c % gbytes) cuts.push_back(c);
  return cuts;
}

void build_worklist(const Bound& b, const Phase& ph, uint32_t G, uint32_t group_tiles, bool reverse,
                    bool per_step, bool group_major, const std::vector<uint64_t>& cuts, std::vector<uint32_t>& off,
                    std::vector<DevItem>& list) {
  const uint64_t gbytes = uint64_t(group_tiles) * TILE_BYTES;
  const uint32_t launches = per_step ? ph.s1 - ph.s0 : 1;
  off.clear();
  list.clear();
  struct Piece {
    uint64_t group;
    uint32_t step;
    DevItem it;
  };
  std::vector<std::vector<Piece>> raw(G);
  std::vector<Piece> cut;  // pieces of one item
  std::vector<DevItem> per;
  // the entries of the current run (indices into per) and the run's step
  std::vector<size_t> run;
  uint32_t run_step = ~0u;
  auto one_tile = [](const DevItem& x) { return x.col0 / TILE_BYTES == (x.col1 - 1) / TILE_BYTES; };
  auto push = [&](uint32_t s, const DevItem& q) {
    bool join = !run.empty() && run_step == s && run.size() < RUN_MAX && one_tile(q) && one_tile(per[run.back()]);
    for (size_t i = 0; join && i < run.size(); ++i) {
      const DevItem& p = per[run[i]];
      // two accumulations into the same bytes must stay one after the other
      if (p.dst_rank == q.dst_rank && p.col0 < q.col1 && q.col0 < p.col1) join = false;
    }
    if (join) {
      per[run.back()].flags |= ITEM_BATCH_NEXT;
      run.push_back(per.size());
    } else {
      run.assign(1, per.size());
      run_step = s;
    }
    per.push_back(q);
  };
  // stores outside the defined output may be dropped only where nothing after
  // this list can read them (see below)
  bool zero_deltas = true;
  for (uint32_t s = ph.s0; s < ph.s1; ++s)
    for (uint32_t i = 0; i < b.steps[s].nitems; ++i) {
      const DevItem& it = b.items[b.steps[s].item0 + i];
      zero_deltas = zero_deltas && it.src_delta == 0 && it.dst_delta == 0;
    }
  const bool dead_at_end = group_major && !per_step && zero_deltas && ph.s1 == b.steps.size() &&
                           b.defined.size() > 0;
  auto defined_meets = [&](const DevItem& p) {
    if (p.dst_rank >= b.defined.size()) return true;
    for (auto& r : b.defined[p.dst_rank])
      if (r.first < p.col1 && p.col0 < r.second) return true;
    return false;
  };
  for (uint32_t j = 0; j < launches; ++j) {
    for (auto& v : raw) v.clear();
    const uint32_t sa = per_step ? ph.s0 + j : ph.s0, sb = per_step ? sa + 1 : ph.s1;
    for (uint32_t s = sa; s < sb; ++s) {
      const DevStep& st = b.steps[s];
      const bool rev = reverse && (s & 1u);
      const bool back = rev && !(st.flags & STEP_ORDERED);
      for (uint32_t n = 0; n < st.nitems; ++n) {
        const DevItem& it = b.items[st.item0 + (back ? st.nitems - 1 - n : n)];
        if (it.col1 <= it.col0) continue;
        // group of column c: its tile group plus the cuts at or below c
        size_t ci = size_t(std::upper_bound(cuts.begin(), cuts.end(), it.col0) - cuts.begin());
        cut.clear();
        for (uint64_t c0 = it.col0; c0 < it.col1;) {
          const uint64_t q = c0 / gbytes;
          uint64_t c1 = std::min(it.col1, (q + 1) * gbytes);
          if (ci < cuts.size() && cuts[ci] < c1) c1 = cuts[ci];
          DevItem piece = it;
          piece.col0 = c0;
          piece.col1 = c1;
          cut.push_back({q + ci, s, piece});
          c0 = c1;
          while (ci < cuts.size() && cuts[ci] <= c0) ++ci;
        }
        for (size_t k = 0; k < cut.size(); ++k) {
          Piece p = cut[rev ? cut.size() - 1 - k : k];
          uint32_t owner = uint32_t(p.group % G);
          if (per_step && rev) owner = G - 1 - owner;
          p.it.flags &= ~uint32_t(ITEM_BATCH_NEXT | ITEM_SRC_FWD | ITEM_DSRC_FWD | ITEM_NO_STORE);
          p.it.pad = wave_mask(p.it);
          raw[owner].push_back(p);
        }
      }
    }
    for (uint32_t w = 0; w < G; ++w) {
      // group-major: a work group takes each of its column groups through every
      // step before the next group (the columns of different groups never
      // meet, so any interleaving of groups is correct); step-major: every
      // group one step at a time
      if (group_major)
        std::stable_sort(raw[w].begin(), raw[w].end(), [](const Piece& x, const Piece& y) { return x.group < y.group; });
      per.clear();
      run.clear();
      run_step = ~0u;
      for (const Piece& p : raw[w]) push(p.step, p.it);
      // forwarding: an entry that reads, over the same whole-tile columns, the
      // bytes the entry before it wrote (its source in a later step, or its old
      // destination value) may take them from the registers of the threads that
      // stored them; no other work group writes these columns, and nothing else
      // in this list comes between the two
      for (size_t i = 1; i < per.size(); ++i) {
        const DevItem& p = per[i - 1];
        DevItem& q = per[i];
        if (!fwd_eligible(p.col0, p.col1, p.flags) || !fwd_eligible(q.col0, q.col1, q.flags)) continue;
        if (p.col0 != q.col0 || p.col1 != q.col1 || (p.flags & ITEM_BATCH_NEXT)) continue;
        if (!(q.flags & ITEM_SRC_SEND) && q.src_rank == p.dst_rank && q.src_delta == p.dst_delta &&
            raw[w][i].step > raw[w][i - 1].step)
          q.flags |= ITEM_SRC_FWD;
        if ((q.flags & ITEM_REDUCE) && !(q.flags & ITEM_DSRC_SEND) && q.dst_rank == p.dst_rank &&
            q.dst_delta == p.dst_delta)
          q.flags |= ITEM_DSRC_FWD;
      }
      // stores no one needs: the destination bytes of an eligible entry that a
      // later entry over the same columns overwrites before any entry between
      // them loads them (an operand taken from registers is no load; a load from
      // the rank's send buffer counts, which in place is the same memory).  In
      // Ring AllReduce these are the partial sums of the ReduceScatter half,
      // which the AllGather half overwrites: N-2 of each column's 2(N-1) stores.
      for (size_t i = 0; i < per.size(); ++i) {
        DevItem& p = per[i];
        if (!fwd_eligible(p.col0, p.col1, p.flags)) continue;
        const uint64_t width = p.col1 - p.col0;
        auto meets = [&](uint16_t rank, int64_t delta) {
          return rank == p.dst_rank && uint64_t(delta > p.dst_delta ? delta - p.dst_delta : p.dst_delta - delta) < width;
        };
        for (size_t j = i + 1; j < per.size(); ++j) {
          const DevItem& q = per[j];
          if (!fwd_eligible(q.col0, q.col1, q.flags) || q.col0 != p.col0 || q.col1 != p.col1) break;
          const bool loads = (!(q.flags & ITEM_SRC_FWD) && meets(q.src_rank, q.src_delta)) ||
                             ((q.flags & ITEM_REDUCE) && !(q.flags & ITEM_DSRC_FWD) && meets(q.dst_rank, q.dst_delta));
          if (loads) break;
          if (meets(q.dst_rank, q.dst_delta)) {
            if (q.dst_delta == p.dst_delta) p.flags |= ITEM_NO_STORE;
            break;
          }
        }
      }
      // stores no one reads before the call ends: in a group-major list of the
      // call's last phase, run in one launch, an eligible entry whose
      // destination bytes lie outside its rank's defined output and which no
      // later entry of its column group loads (the ReduceScatter partial sums
      // that stay on the ranks that do not own the chunk).  With every delta
      // zero a column is the same bytes on every rank, so entries of other
      // column groups, which other work groups or later parts of this list
      // run, never touch these bytes.
      if (dead_at_end) {
        for (size_t i = 0; i < per.size(); ++i) {
          DevItem& p = per[i];
          if ((p.flags & ITEM_NO_STORE) || !fwd_eligible(p.col0, p.col1, p.flags) || defined_meets(p)) continue;
          bool live = false;
          for (size_t j = i + 1; j < per.size() && raw[w][j].group == raw[w][i].group && !live; ++j) {
            const DevItem& q = per[j];
            const bool overlap = p.col0 < q.col1 && q.col0 < p.col1;
            const bool same = q.col0 == p.col0 && q.col1 == p.col1;
            live = overlap && ((q.src_rank == p.dst_rank && !(same && (q.flags & ITEM_SRC_FWD) && fwd_eligible(q.col0, q.col1, q.flags))) ||
                               (q.dst_rank == p.dst_rank));
          }
          if (!live) p.flags |= ITEM_NO_STORE;
        }
      }
      off.push_back(uint32_t(list.size()));
      list.insert(list.end(), per.begin(), per.end());
    }
    off.push_back(uint32_t(list.size()));
  }
}

RowsList plan_rows_list(const Bound& b, const Phase& ph, uint64_t cap, uint32_t group_tiles, bool reverse,
                        bool per_step, bool group_major) {
  RowsList r;
  const uint64_t gbytes = uint64_t(group_tiles) * TILE_BYTES;
  const uint64_t groups = std::max<uint64_t>(1, (ph.colspace + gbytes - 1) / gbytes);
  // Groups split at row boundaries when every group (split halves included)
  // gets a work group of its own.  A group holding the end of one row and the
  // start of the next would give its work group two chains of pieces to run one
  // after the other, twice the round trips of any other work group (8 x 64 MiB
  // uint8 Broadcast in 13 chunks: 160 -> 138 us).  With several groups per work
  // group a split adds as many pieces to some list as it saves.
  std::vector<uint64_t> cuts = group_cuts(ph, gbytes);
  if (groups + cuts.size() > cap) cuts.clear();
  r.G = uint32_t(std::min(groups + cuts.size(), cap));
  build_worklist(b, ph, r.G, group_tiles, reverse, per_step, group_major, cuts, r.off, r.list);
  // the fine variant pays off when pieces are small: some runs, or pieces of
  // less than one tile on average
  uint64_t piece_bytes = 0;
  bool runs = false;
  size_t marked = 0;
  for (const DevItem& x : r.list) {
    runs = runs || (x.flags & ITEM_BATCH_NEXT);
    piece_bytes += x.col1 - x.col0;
    marked += (x.flags & (ITEM_SRC_FWD | ITEM_DSRC_FWD)) != 0;
  }
  r.fine = runs || (!r.list.empty() && piece_bytes < uint64_t(TILE_BYTES) * r.list.size());
  // The forwarding variant holds 8 tiles of results in registers, which halves
  // the work groups a CU can hold.  It pays on the large grids of group-major
  // lists where most entries forward (chains: Ring AllReduce / AllGather, chain
  // pipelines, about 90 % of their entries; 8 x 256 MiB fp32 Ring 1.150 -> 0.948
  // ms), not where few do (trees and halving-doubling, 30-50 %: 9-14 % slower at
  // 8 x 256 MiB), nor on resident grids, which are sized for the plain kernel's
  // occupancy (Ring AllReduce 8 x 1-8 MiB: 22-100 % slower).
  r.fwd = group_major && marked > 0 && marked * 10 >= r.list.size() * 6;
  if (r.fwd)
    for (const DevItem& x : r.list) {
      if (!fwd_eligible(x.col0, x.col1, x.flags)) continue;
      const uint64_t w = x.col1 - x.col0;
      if (x.flags & ITEM_SRC_FWD) r.fwd_saved += w;
      if ((x.flags & ITEM_REDUCE) && (x.flags & ITEM_DSRC_FWD)) r.fwd_saved += w;
      if (x.flags & ITEM_NO_STORE) r.fwd_saved += w;
    }
  return r;
}

}  // namespace coll
