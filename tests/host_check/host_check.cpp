// Host-side invariants of schedule generation, binding and work-list layout,
// built with AddressSanitizer and UndefinedBehaviorSanitizer by the CPU tests.
// No GPU: only plan.cpp and bind.cpp are linked.
//
// For every shape in a grid of (collective, algorithm, N, count, root, k,
// element size, in place) it checks:
//   * build_schedule accepts the arguments and check_schedule finds no hazard;
//   * bind_schedule: per row, the items of a row-kernel step cover the row's
//     destination bytes exactly once;
//   * build_worklist, for several launch shapes, step-major and group-major,
//     with uniform column groups and with groups split at the rows' boundaries
//     (group_cuts): the pieces of every item cover its columns exactly once,
//     each piece lies inside one column group and sits in its owner's list,
//     with split groups every row boundary is a group boundary, every
//     forwarding mark (ITEM_SRC_FWD / ITEM_DSRC_FWD) names bytes the entry
//     just before it in the same list wrote, over the same whole-tile columns
//     (a source: in an earlier step), each group's
//     pieces are in step order (group-major lists: groups in order), the wave mask
//     is the set of waves whose bytes the piece touches, and every
//     ITEM_BATCH_NEXT run has at most RUN_MAX members of one step, each inside
//     one tile, with no two members writing common bytes of one rank;
//   * symbolic execution of every such list: each byte of every rank buffer
//     holds a 32-bit symbol, a copy moves it and a reduction replaces the old
//     destination symbol d by mix(d, s), which depends on the order of its
//     operands.  Running a launch's lists one work group after another, the
//     way the forwarding variant of the row kernel takes them (forwarded
//     operands from the previous piece's results, ITEM_NO_STORE stores
//     skipped), and again the way the plain variant does (every operand
//     loaded, every store made), must end in the same memory as running the
//     phase's items step by step (in the call's last phase: the same defined
//     output); and within one launch no byte that a work group writes is read
//     or written by another (column ownership).
//   * column programs (compile_colplan), with checksums and without: run on
//     symbols for every column of every segment (leaves into their slots, ops
//     reading their operands from y or a slot, stores), every store lands a
//     rank's final symbol from the schedule run row by row (snapshot per
//     step), every defined output byte whose final value is not its own
//     input (out of place: every defined byte) is stored exactly once and
//     nothing else is,
//     and each op's value is the symbol of its row's destination right after
//     the row, so the kernel's checksums are the rows' checksums;
//   * rows_shape picks the measured launch shapes (group size, grid cap, list
//     order) for the configurations its rules were measured on, asks whether
//     groups see several pieces per step only when a rule depends on it, and
//     several_pieces_per_step classifies real schedules as expected.
// Prints one line per failure and "host_check: N shapes, M lists, ok" at the end.
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <map>
#include <numeric>
#include <string>
#include <vector>

#include "bind.h"
#include "colprog.h"
#include "plan.h"

using namespace coll;

namespace {

int failures = 0;
long long fwd_marks = 0;       // forwarding marks checked
long long no_store_marks = 0;  // ITEM_NO_STORE marks checked
long long exec_lists = 0;      // launches' lists executed symbolically

#define CHECK(cond, ...)                  \
  do {                                    \
    if (!(cond)) {                        \
      ++failures;                         \
      if (failures < 50) {                \
        std::printf("FAIL %s: ", #cond);  \
        std::printf(__VA_ARGS__);         \
        std::printf("\n");                \
      }                                   \
    }                                     \
  } while (0)

struct Shape {
  coll_kind_t kind;
  coll_algo_t algo;
  int N;
  int64_t count;
  int root, k, sz;
  bool inplace;
};

std::string name(const Shape& s) {
  char b[160];
  std::snprintf(b, sizeof b, "kind %d algo %d N %d count %lld root %d k %d sz %d inplace %d", int(s.kind),
                int(s.algo), s.N, (long long)s.count, s.root, s.k, s.sz, int(s.inplace));
  return b;
}

uint32_t mask_of(uint64_t c0, uint64_t c1) {
  uint32_t m = 0;
  for (uint64_t t = c0 / TILE_BYTES; t <= (c1 - 1) / TILE_BYTES; ++t)
    for (uint32_t w = 0; w < BLOCK_THREADS / 64; ++w) {
      const uint64_t lo = t * TILE_BYTES + w * WAVE_BYTES, hi = lo + WAVE_BYTES;
      if (c0 < hi && lo < c1) m |= 1u << w;
    }
  return m;
}

// ---- symbolic execution ------------------------------------------------------

uint32_t mix(uint32_t d, uint32_t s) {
  uint32_t h = (d ^ 0x9E3779B9u) * 0x85EBCA6Bu;
  h ^= h >> 13;
  return h + s * 0xC2B2AE35u + 1u;
}

// Rank buffers as symbols, one array: buffer id 2*rank (send) or 2*rank + 1
// (receive) starts at base[id]; in place a rank's send and receive buffers are
// the same memory.  One symbol stands for q bytes: every item boundary and
// delta of the schedule, and the tile size, are multiples of q, so every item
// and every piece moves such a unit whole.
struct Mem {
  bool inplace = false;
  uint64_t q = 1;
  std::vector<uint64_t> base;
  std::vector<uint32_t> v;
  uint64_t id(bool send, int rank) const { return uint64_t(2 * rank) + ((send && !inplace) ? 0 : 1); }
  // index into v of the unit at column c of an item's operand
  uint64_t src(const DevItem& it, uint64_t c) const {
    return base[id((it.flags & ITEM_SRC_SEND) != 0, it.src_rank)] + uint64_t(int64_t(c) + it.src_delta) / q;
  }
  uint64_t dsrc(const DevItem& it, uint64_t c) const {
    return base[id((it.flags & ITEM_DSRC_SEND) != 0, it.dst_rank)] + uint64_t(int64_t(c) + it.dst_delta) / q;
  }
  uint64_t dst(const DevItem& it, uint64_t c) const {
    return base[id(false, it.dst_rank)] + uint64_t(int64_t(c) + it.dst_delta) / q;
  }
};

template <class F>
void for_row_items(const Bound& b, F&& f) {
  for (const Phase& ph : b.phases) {
    if (ph.kind != Phase::ROWS) continue;
    for (uint32_t s = ph.s0; s < ph.s1; ++s)
      for (uint32_t i = 0; i < b.steps[s].nitems; ++i) {
        const DevItem& it = b.items[b.steps[s].item0 + i];
        if (it.col1 > it.col0) f(it);
      }
  }
}

Mem initial_mem(const Bound& b, int N, bool inplace) {
  Mem m;
  m.inplace = inplace;
  m.q = TILE_BYTES;
  auto g = [&](int64_t x) { m.q = std::gcd(m.q, uint64_t(x < 0 ? -x : x)); };
  for_row_items(b, [&](const DevItem& it) {
    g(int64_t(it.col0));
    g(int64_t(it.col1));
    g(it.src_delta);
    g(it.dst_delta);
  });
  std::vector<uint64_t> ext(size_t(2 * N), 0);
  m.base.assign(ext.size() + 1, 0);  // all zero while measuring: index = unit offset
  for_row_items(b, [&](const DevItem& it) {
    const uint64_t c = it.col1 - m.q;
    uint64_t& e1 = ext[m.id((it.flags & ITEM_SRC_SEND) != 0, it.src_rank)];
    e1 = std::max(e1, m.src(it, c) + 1);
    uint64_t& e2 = ext[m.id((it.flags & ITEM_DSRC_SEND) != 0, it.dst_rank)];
    e2 = std::max(e2, m.dsrc(it, c) + 1);
    uint64_t& e3 = ext[m.id(false, it.dst_rank)];
    e3 = std::max(e3, m.dst(it, c) + 1);
  });
  for (size_t i = 0; i < ext.size(); ++i) m.base[i + 1] = m.base[i] + ext[i];
  m.v.resize(m.base.back());
  for (uint64_t x = 0; x < m.v.size(); ++x) {
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    m.v[x] = uint32_t(z ^ (z >> 31));
  }
  return m;
}

// The phase's items step by step, in item order.
void run_steps(Mem& m, const Bound& b, const Phase& ph) {
  for (uint32_t s = ph.s0; s < ph.s1; ++s)
    for (uint32_t i = 0; i < b.steps[s].nitems; ++i) {
      const DevItem& it = b.items[b.steps[s].item0 + i];
      for (uint64_t c = it.col0; c < it.col1; c += m.q) {
        uint32_t y = m.v[m.src(it, c)];
        if (it.flags & ITEM_REDUCE) y = mix(m.v[m.dsrc(it, c)], y);
        m.v[m.dst(it, c)] = y;
      }
    }
}

// The units of v that a phase's items write, as sorted disjoint ranges.
std::vector<std::pair<uint64_t, uint64_t>> written_units(const Mem& m, const Bound& b, const Phase& ph) {
  std::vector<std::pair<uint64_t, uint64_t>> r;
  for (uint32_t s = ph.s0; s < ph.s1; ++s)
    for (uint32_t i = 0; i < b.steps[s].nitems; ++i) {
      const DevItem& it = b.items[b.steps[s].item0 + i];
      if (it.col1 > it.col0) r.push_back({m.dst(it, it.col0), m.dst(it, it.col1 - m.q) + 1});
    }
  std::sort(r.begin(), r.end());
  std::vector<std::pair<uint64_t, uint64_t>> out;
  for (auto& x : r) {
    if (!out.empty() && x.first <= out.back().second) out.back().second = std::max(out.back().second, x.second);
    else out.push_back(x);
  }
  return out;
}

// Which work group of the current launch touched each unit: tag = (launch
// generation << 16) | (work group + 1); readers' tag ends in 0xFFFF once two
// work groups have read the unit.
struct Owners {
  std::vector<uint64_t> rd, wr;
  uint64_t gen = 0;
  explicit Owners(const Mem& m) : rd(m.v.size(), 0), wr(m.v.size(), 0) {}
  bool read(uint64_t i, uint32_t w) {
    const uint64_t tag = (gen << 16) | (w + 1);
    const uint64_t ww = wr[i];
    if ((ww >> 16) == gen && ww != tag) return false;
    uint64_t& r = rd[i];
    if ((r >> 16) != gen) r = tag;
    else if (r != tag) r = (gen << 16) | 0xFFFF;
    return true;
  }
  bool write(uint64_t i, uint32_t w) {
    const uint64_t tag = (gen << 16) | (w + 1);
    const uint64_t ww = wr[i], r = rd[i];
    if ((ww >> 16) == gen && ww != tag) return false;
    if ((r >> 16) == gen && r != tag) return false;
    wr[i] = tag;
    return true;
  }
};

// `units` (sorted disjoint unit ranges) cut down to the receive-buffer bytes
// each rank's output defines.
std::vector<std::pair<uint64_t, uint64_t>> defined_units(const Mem& m, const Bound& b,
                                                         const std::vector<std::pair<uint64_t, uint64_t>>& units) {
  std::vector<std::pair<uint64_t, uint64_t>> def, out;
  for (size_t rank = 0; rank < b.defined.size(); ++rank)
    for (auto& r : b.defined[rank]) {
      const uint64_t id = m.id(false, int(rank));
      const uint64_t lo = m.base[id] + r.first / m.q, hi = std::min(m.base[id] + (r.second + m.q - 1) / m.q, m.base[id + 1]);
      if (lo < hi) def.push_back({lo, hi});
    }
  std::sort(def.begin(), def.end());
  for (auto& u : units)
    for (auto& d : def) {
      const uint64_t lo = std::max(u.first, d.first), hi = std::min(u.second, d.second);
      if (lo < hi) out.push_back({lo, hi});
    }
  return out;
}

// Runs one phase's launches on `m` (the memory before the phase), each
// launch's work groups one after the other, as the forwarding variant (fwd) or
// the plain variant takes the lists; compares the units of `compare` with
// `after` and puts `before`'s values back on every unit of `written`.
void check_exec(const Shape& sh, uint32_t G, const std::vector<uint32_t>& off, const std::vector<DevItem>& list,
                const Mem& before, const Mem& after, const std::vector<std::pair<uint64_t, uint64_t>>& written,
                const std::vector<std::pair<uint64_t, uint64_t>>& compare, Owners& own, Mem& m, bool fwd) {
  const uint32_t launches = uint32_t(off.size() / (G + 1));
  bool race = false, stale = false;
  std::vector<uint32_t> held, next;
  for (uint32_t j = 0; j < launches; ++j) {
    ++own.gen;
    for (uint32_t w = 0; w < G; ++w) {
      bool have = false;
      uint64_t h0 = 0, h1 = 0;
      for (uint32_t e = off[size_t(j) * (G + 1) + w]; e < off[size_t(j) * (G + 1) + w + 1]; ++e) {
        const DevItem& it = list[e];
        const bool f = fwd && fwd_eligible(it.col0, it.col1, it.flags);
        const bool fs = f && (it.flags & ITEM_SRC_FWD), fd = f && (it.flags & ITEM_DSRC_FWD);
        const bool store = !(f && (it.flags & ITEM_NO_STORE));
        if ((fs || fd) && !(have && h0 == it.col0 && h1 == it.col1)) stale = true;
        next.assign(size_t((it.col1 - it.col0) / m.q), 0);
        for (uint64_t c = it.col0; c < it.col1; c += m.q) {
          const size_t k = size_t((c - it.col0) / m.q);
          uint32_t y;
          if (fs && !stale) {
            y = held[k];
          } else {
            const uint64_t i = m.src(it, c);
            race = race || !own.read(i, w);
            y = m.v[i];
          }
          if (it.flags & ITEM_REDUCE) {
            uint32_t d;
            if (fd && !stale) {
              d = held[k];
            } else {
              const uint64_t i = m.dsrc(it, c);
              race = race || !own.read(i, w);
              d = m.v[i];
            }
            y = mix(d, y);
          }
          if (store) {
            const uint64_t i = m.dst(it, c);
            race = race || !own.write(i, w);
            m.v[i] = y;
          }
          next[k] = y;
        }
        if (f) {
          held.swap(next);
          have = true;
          h0 = it.col0;
          h1 = it.col1;
        }
      }
    }
  }
  ++exec_lists;
  bool same = true;
  for (auto& r : compare)
    same = same && std::equal(m.v.begin() + r.first, m.v.begin() + r.second, after.v.begin() + r.first);
  for (auto& r : written) std::copy(before.v.begin() + r.first, before.v.begin() + r.second, m.v.begin() + r.first);
  const char* how = fwd ? "forwarding" : "plain";
  CHECK(!stale, "%s: %s variant: a forwarded operand with no matching piece before it", name(sh).c_str(), how);
  CHECK(!race, "%s: %s variant: two work groups of one launch touch a unit one of them writes", name(sh).c_str(),
        how);
  CHECK(same, "%s: %s variant, G %u: lists end in other memory than the steps", name(sh).c_str(), how, G);
}

// Which lists to execute symbolically, and how (--exec=...; every list of
// every shape takes about 20 minutes at -O2):
//   small (default): shapes of up to 1,000 elements, every launch layout;
//   sample: also shapes of up to 4,099 elements on grids of 3 and 257 work
//     groups, group-major lists in reversed order and step-major lists in step
//     order, and larger ones in the layout of large reductions (257 work
//     groups, 4-tile groups split at row boundaries, group-major) in the
//     forwarding variant only;
//   all: everything;  none: nothing.
enum ExecMode { EXEC_NONE, EXEC_SMALL, EXEC_SAMPLE, EXEC_ALL } exec_mode = EXEC_SMALL;
bool exec_shape(const Shape& sh) {
  return exec_mode == EXEC_ALL || exec_mode == EXEC_SAMPLE || (exec_mode == EXEC_SMALL && sh.count <= 1000);
}
bool exec_filter(const Shape& sh, uint32_t G, uint32_t gt, bool rev, bool per_step, bool gm, bool snap, bool fwd) {
  if (!exec_shape(sh)) return false;
  if (exec_mode == EXEC_ALL || sh.count <= 1000) return true;
  if (sh.count <= 4099) return G != 1 && rev == gm;
  return fwd && G == 257 && gt == 4 && gm && !per_step && rev && snap;
}

void check_lists(const Shape& sh, const Schedule& sched, const Bound& b, int& nlists) {
  // memory before and after each row phase, items run step by step
  std::vector<Mem> mems;
  mems.push_back(exec_shape(sh) ? initial_mem(b, sh.N, sh.inplace) : Mem{});
  Owners own(mems[0]);
  for (const Phase& ph : b.phases) {
    mems.push_back(mems.back());
    if (ph.kind == Phase::ROWS && exec_shape(sh)) run_steps(mems.back(), b, ph);
  }
  for (size_t pi = 0; pi < b.phases.size(); ++pi) {
    const Phase& ph = b.phases[pi];
    if (ph.kind != Phase::ROWS) continue;
    Mem work = mems[pi];
    const auto written = exec_shape(sh) ? written_units(work, b, ph) : std::vector<std::pair<uint64_t, uint64_t>>{};
    // the call's last phase: only the defined output has to match (stores
    // outside it that nothing reads afterwards may be skipped)
    const auto compare = exec_shape(sh) && ph.s1 == b.steps.size() ? defined_units(work, b, written) : written;
    for (uint32_t G : {1u, 3u, 257u})
      for (uint32_t gt : {1u, 4u})
        for (int rev = 0; rev < 2; ++rev)
          for (int per_step = 0; per_step < 2; ++per_step)
            for (int gm = 0; gm < 2; ++gm)
              for (int snap = 0; snap < (gm && !per_step ? 2 : 1); ++snap) {
            std::vector<uint32_t> off;
            std::vector<DevItem> list;
            const uint64_t gbytes = uint64_t(gt) * TILE_BYTES;
            std::vector<uint64_t> cuts;
            if (snap) {
              cuts = group_cuts(ph, gbytes);
              // the cuts: exactly the row boundaries strictly inside a group, sorted, once each
              std::vector<uint64_t> want_cuts;
              for (uint32_t s = ph.s0; s < ph.s1; ++s)
                for (uint32_t i = 0; i < b.steps[s].nitems; ++i) {
                  const DevItem& it = b.items[b.steps[s].item0 + i];
                  if (it.col1 <= it.col0) continue;
                  for (uint64_t c : {it.col0, it.col1})
                    if (c % gbytes && c < ph.colspace) want_cuts.push_back(c);
                }
              std::sort(want_cuts.begin(), want_cuts.end());
              want_cuts.erase(std::unique(want_cuts.begin(), want_cuts.end()), want_cuts.end());
              CHECK(cuts == want_cuts, "%s: group cuts", name(sh).c_str());
            }
            // group of a column: its tile group plus the cuts at or below it
            auto group_of = [&](uint64_t c) {
              return c / gbytes + uint64_t(std::upper_bound(cuts.begin(), cuts.end(), c) - cuts.begin());
            };
            // split groups: every row boundary is a group boundary
            if (snap)
              for (uint32_t s = ph.s0; s < ph.s1; ++s)
                for (uint32_t i = 0; i < b.steps[s].nitems; ++i) {
                  const DevItem& it = b.items[b.steps[s].item0 + i];
                  if (it.col1 <= it.col0) continue;
                  for (uint64_t c : {it.col0, it.col1})
                    if (c > 0 && c < ph.colspace)
                      CHECK(group_of(c - 1) != group_of(c), "%s: row boundary %llu inside a group", name(sh).c_str(),
                            (unsigned long long)c);
                }
            build_worklist(b, ph, G, gt, rev != 0, per_step != 0, gm != 0, cuts, off, list);
            ++nlists;
            const uint32_t launches = per_step ? ph.s1 - ph.s0 : 1;
            CHECK(off.size() == size_t(launches) * (G + 1), "%s: offsets", name(sh).c_str());
            if (off.size() != size_t(launches) * (G + 1)) continue;
            // coverage: the pieces of item (step, dst rank, col0..col1, row) re-assemble it.
            // Pieces carry no item index; match them to items by (row, dst_rank, src/dst delta, flags).
            std::map<std::vector<int64_t>, std::vector<std::pair<uint64_t, uint64_t>>> got, want;
            for (uint32_t s = ph.s0; s < ph.s1; ++s) {
              const DevStep& d = b.steps[s];
              for (uint32_t i = 0; i < d.nitems; ++i) {
                const DevItem& it = b.items[d.item0 + i];
                if (it.col1 <= it.col0) continue;
                std::vector<int64_t> key{int64_t(s), it.row, it.src_rank, it.dst_rank, it.src_delta, it.dst_delta,
                                         int64_t(it.flags & ~uint32_t(ITEM_BATCH_NEXT))};
                want[key].push_back({it.col0, it.col1});
              }
            }
            for (uint32_t j = 0; j < launches; ++j) {
              for (uint32_t w = 0; w < G; ++w) {
                const uint32_t a = off[size_t(j) * (G + 1) + w], z = off[size_t(j) * (G + 1) + w + 1];
                CHECK(a <= z && z <= list.size(), "%s: list bounds", name(sh).c_str());
                if (!(a <= z && z <= list.size())) continue;
                std::map<uint64_t, uint32_t> last_step;   // per column group
                uint64_t last_group = 0;
                for (uint32_t e = a; e < z; ++e) {
                  const DevItem& p = list[e];
                  CHECK(p.col0 < p.col1, "%s: empty piece", name(sh).c_str());
                  const uint64_t g = group_of(p.col0);
                  CHECK(group_of(p.col1 - 1) == g, "%s: piece crosses a group", name(sh).c_str());
                  CHECK(p.pad == mask_of(p.col0, p.col1), "%s: wave mask %u vs %u", name(sh).c_str(), p.pad,
                        mask_of(p.col0, p.col1));
                  // step of the piece: its row's step (copies of undefined-by-rows output: step 0)
                  CHECK(p.row == NO_ROW || p.row < sched.rows.size(), "%s: row index", name(sh).c_str());
                  if (p.row != NO_ROW && p.row >= sched.rows.size()) continue;
                  const uint32_t ps = p.row == NO_ROW ? 0u : uint32_t(sched.rows[p.row].step);
                  // owner: group g mod G; in per-step launches of reversed (odd) steps, mirrored
                  uint32_t owner = uint32_t(g % G);
                  if (per_step && rev && (ps & 1u)) owner = G - 1 - owner;
                  CHECK(owner == w, "%s: piece of step %u in the wrong list", name(sh).c_str(), ps);
                  CHECK(ps >= last_step[g], "%s: a group's pieces not in step order", name(sh).c_str());
                  last_step[g] = ps;
                  if (gm) {
                    CHECK(g >= last_group, "%s: group-major list not in group order", name(sh).c_str());
                    last_group = g;
                  }
                  std::vector<int64_t> key{int64_t(ps), p.row, p.src_rank, p.dst_rank, p.src_delta, p.dst_delta,
                                           int64_t(p.flags & ~uint32_t(ITEM_BATCH_NEXT | ITEM_SRC_FWD |
                                                                       ITEM_DSRC_FWD | ITEM_NO_STORE))};
                  if (p.flags & ITEM_NO_STORE) {
                    ++no_store_marks;
                    CHECK(fwd_eligible(p.col0, p.col1, p.flags), "%s: store skipped on a piece the forwarding "
                          "variant does not hold", name(sh).c_str());
                  }
                  // forwarding marks
                  if (p.flags & (ITEM_SRC_FWD | ITEM_DSRC_FWD)) {
                    ++fwd_marks;
                    CHECK(e > a, "%s: forwarding mark on a list's first entry", name(sh).c_str());
                    if (e > a) {
                      const DevItem& q = list[e - 1];
                      const uint32_t qs = q.row == NO_ROW ? 0u : uint32_t(sched.rows[q.row].step);
                      CHECK(fwd_eligible(q.col0, q.col1, q.flags) && fwd_eligible(p.col0, p.col1, p.flags) &&
                                q.col0 == p.col0 && q.col1 == p.col1 && !(q.flags & ITEM_BATCH_NEXT),
                            "%s: forwarding between pieces that are not the same whole tiles", name(sh).c_str());
                      if (p.flags & ITEM_SRC_FWD)
                        CHECK(!(p.flags & ITEM_SRC_SEND) && p.src_rank == q.dst_rank && p.src_delta == q.dst_delta &&
                                  ps > qs,
                              "%s: source forwarded from a piece that did not write it", name(sh).c_str());
                      if (p.flags & ITEM_DSRC_FWD)
                        CHECK((p.flags & ITEM_REDUCE) && !(p.flags & ITEM_DSRC_SEND) && p.dst_rank == q.dst_rank &&
                                  p.dst_delta == q.dst_delta && ps >= qs,
                              "%s: old destination forwarded from a piece that did not write it", name(sh).c_str());
                    }
                  }
                  got[key].push_back({p.col0, p.col1});
                  // runs
                  if (p.flags & ITEM_BATCH_NEXT) {
                    CHECK(e + 1 < z, "%s: run flag on the last entry", name(sh).c_str());
                    CHECK(p.col0 / TILE_BYTES == (p.col1 - 1) / TILE_BYTES, "%s: run member spans tiles",
                          name(sh).c_str());
                  }
                }
                // run structure: members of one run, same step, one tile, disjoint writes, <= RUN_MAX
                uint32_t e = a;
                while (e < z) {
                  uint32_t n = 1;
                  while (e + n < z && (list[e + n - 1].flags & ITEM_BATCH_NEXT)) ++n;
                  CHECK(n <= RUN_MAX, "%s: run of %u", name(sh).c_str(), n);
                  for (uint32_t x = e; x < e + n; ++x)
                    for (uint32_t y = x + 1; y < e + n; ++y) {
                      const DevItem& p = list[x];
                      const DevItem& q = list[y];
                      CHECK(!(p.dst_rank == q.dst_rank && p.col0 < q.col1 && q.col0 < p.col1),
                            "%s: run members write common bytes", name(sh).c_str());
                      CHECK(q.col0 / TILE_BYTES == (q.col1 - 1) / TILE_BYTES, "%s: run member spans tiles",
                            name(sh).c_str());
                    }
                  e += n;
                }
              }
            }
            // compare coverage
            for (auto& kv : want) {
              auto w = kv.second;
              auto it = got.find(kv.first);
              CHECK(it != got.end(), "%s: item without pieces", name(sh).c_str());
              if (it == got.end()) continue;
              auto g = it->second;
              std::sort(w.begin(), w.end());
              std::sort(g.begin(), g.end());
              // merge adjacent pieces and compare with the merged items
              auto merge = [](std::vector<std::pair<uint64_t, uint64_t>> v) {
                std::vector<std::pair<uint64_t, uint64_t>> out;
                for (auto& x : v) {
                  if (!out.empty() && out.back().second == x.first) out.back().second = x.second;
                  else out.push_back(x);
                }
                return out;
              };
              uint64_t wb = 0, gb = 0;
              for (auto& x : w) wb += x.second - x.first;
              for (auto& x : g) gb += x.second - x.first;
              CHECK(wb == gb, "%s: covered %llu of %llu bytes", name(sh).c_str(), (unsigned long long)gb,
                    (unsigned long long)wb);
              CHECK(merge(w) == merge(g), "%s: pieces do not re-assemble the items", name(sh).c_str());
            }
            CHECK(got.size() == want.size(), "%s: pieces of unknown items", name(sh).c_str());
            for (bool fwd : {true, false})
              if (exec_filter(sh, G, gt, rev != 0, per_step != 0, gm != 0, snap != 0, fwd))
                check_exec(sh, G, off, list, mems[pi], mems[pi + 1], written, compare, own, work, fwd);
          }
  }
}

}  // namespace

void check_launch_shapes() {
  struct Case {
    const char* what;
    coll_kind_t kind;
    coll_algo_t algo;
    int N, k;
    int64_t bytes;       // per rank
    int sz;
    bool per_step;
    int64_t forced_gt, forced_grid;
    int several;         // expected several_pieces_per_step, -1: not asked
    uint32_t gt;
    uint64_t cap;
    bool group_major;
    bool checksums = false;
  };
  const uint64_t big = uint64_t(1) << 20;
  const Case cases[] = {
      {"Ring AR fp32 8x256MiB", COLL_K_ALLREDUCE, COLL_ALGO_RING, 8, 1, 256 << 20, 4, false, 0, 0, 0, 4, big, true},
      {"Ring AR fp32 8x32MiB", COLL_K_ALLREDUCE, COLL_ALGO_RING, 8, 1, 32 << 20, 4, false, 0, 0, 0, 8, big, true},
      {"DBT AR fp32 8x256MiB", COLL_K_ALLREDUCE, COLL_ALGO_DBT, 8, 1, 256 << 20, 4, false, 0, 0, 1, 4, 512, true},
      {"RHD AR bf16 8x256MiB", COLL_K_ALLREDUCE, COLL_ALGO_RHD, 8, 1, 256 << 20, 2, false, 0, 0, 1, 4, 512, true},
      {"tree Reduce fp32 8x256MiB", COLL_K_REDUCE, COLL_ALGO_BINOMIAL, 8, 1, 256 << 20, 4, false, 0, 0, 1, 4, 512,
       true},
      {"Ring RS bf16 64x256MiB", COLL_K_REDUCESCATTER, COLL_ALGO_RING, 64, 1, 256 << 20, 2, false, 0, 0, 0, 8, big,
       true},
      {"RHD AG bf16 64x256MiB", COLL_K_ALLGATHER, COLL_ALGO_RHD, 64, 1, 256 << 20, 2, false, 0, 0, 1, 4, 512, true},
      {"Ring AG bf16 64x256MiB", COLL_K_ALLGATHER, COLL_ALGO_RING, 64, 1, 256 << 20, 2, false, 0, 0, 0, 8, big, true},
      {"binomial Bcast u8 8x64MiB", COLL_K_BROADCAST, COLL_ALGO_BINOMIAL, 8, 1, 64 << 20, 1, false, 0, 0, -1, 8, big,
       true},
      {"binomial Bcast u8 16x64MiB", COLL_K_BROADCAST, COLL_ALGO_BINOMIAL, 16, 1, 64 << 20, 1, false, 0, 0, 1, 4, 512,
       true},
      {"chain Bcast k=8 u8 16x64MiB", COLL_K_BROADCAST, COLL_ALGO_CHAIN_PIPE, 16, 8, 64 << 20, 1, false, 0, 0, 0, 8,
       big, true},
      {"Ring AR u8 8x256MiB", COLL_K_ALLREDUCE, COLL_ALGO_RING, 8, 1, 256 << 20, 1, false, 0, 0, -1, 4, big, true},
      {"Ring AR fp32 8x64MiB", COLL_K_ALLREDUCE, COLL_ALGO_RING, 8, 1, 64 << 20, 4, false, 0, 0, 0, 4, big, true},
      {"Ring AR bf16 16x192MiB", COLL_K_ALLREDUCE, COLL_ALGO_RING, 16, 1, 192 << 20, 2, false, 0, 0, 0, 4, big, true},
      {"Ring AR fp32 8x48MiB", COLL_K_ALLREDUCE, COLL_ALGO_RING, 8, 1, 48 << 20, 4, false, 0, 0, 0, 8, big, true},
      {"Ring AG bf16 8x128MiB", COLL_K_ALLGATHER, COLL_ALGO_RING, 8, 1, 128 << 20, 2, false, 0, 0, 0, 4, big, true},
      {"Ring AG bf16 8x256MiB", COLL_K_ALLGATHER, COLL_ALGO_RING, 8, 1, 256 << 20, 2, false, 0, 0, 0, 4, big, true},
      {"Ring AG bf16 8x96MiB", COLL_K_ALLGATHER, COLL_ALGO_RING, 8, 1, 96 << 20, 2, false, 0, 0, -1, 8, big, true},
      {"Ring AG bf16 32x256MiB", COLL_K_ALLGATHER, COLL_ALGO_RING, 32, 1, 256 << 20, 2, false, 0, 0, 0, 8, big, true},
      {"chain Bcast k=8 u8 8x256MiB", COLL_K_BROADCAST, COLL_ALGO_CHAIN_PIPE, 8, 8, 256 << 20, 1, false, 0, 0, 0, 4,
       big, true},
      {"binomial Bcast u8 8x256MiB", COLL_K_BROADCAST, COLL_ALGO_BINOMIAL, 8, 1, 256 << 20, 1, false, 0, 0, 1, 8,
       big, true},
      {"chain Bcast u8 8x64MiB", COLL_K_BROADCAST, COLL_ALGO_CHAIN_PIPE, 8, 1, 64 << 20, 1, false, 0, 0, -1, 8, big,
       true},
      {"chain Bcast u8 8x128MiB", COLL_K_BROADCAST, COLL_ALGO_CHAIN_PIPE, 8, 1, 128 << 20, 1, false, 0, 0, 0, 4, big,
       true},
      {"Ring AG bf16 4x64MiB", COLL_K_ALLGATHER, COLL_ALGO_RING, 4, 1, 64 << 20, 2, false, 0, 0, -1, 8, big, true},
      {"Ring AR fp32 8x256MiB checksums", COLL_K_ALLREDUCE, COLL_ALGO_RING, 8, 1, 256 << 20, 4, false, 0, 0, 0, 8, big,
       true, true},
      {"chain Bcast u8 8x128MiB checksums", COLL_K_BROADCAST, COLL_ALGO_CHAIN_PIPE, 8, 1, 128 << 20, 1, false, 0, 0, -1,
       8, big, true, true},
      {"Ring AR fp32 8x16MiB", COLL_K_ALLREDUCE, COLL_ALGO_RING, 8, 1, 16 << 20, 4, false, 0, 0, 0, 8, big, true},
      {"Ring AR fp32 8x4MiB", COLL_K_ALLREDUCE, COLL_ALGO_RING, 8, 1, 4 << 20, 4, false, 0, 0, -1, 1, 2048, false},
      {"Ring AR fp32 8x8MiB", COLL_K_ALLREDUCE, COLL_ALGO_RING, 8, 1, 8 << 20, 4, false, 0, 0, 0, 4, big, true},
      {"chain Bcast u8 8x8MiB", COLL_K_BROADCAST, COLL_ALGO_CHAIN_PIPE, 8, 1, 8 << 20, 1, false, 0, 0, -1, 4, big, true},
      {"Ring AR fp32 8x256MiB per step", COLL_K_ALLREDUCE, COLL_ALGO_RING, 8, 1, 256 << 20, 4, true, 0, 0, -1, 8, 8192,
       false},
      {"Ring AR fp32 8x256MiB forced", COLL_K_ALLREDUCE, COLL_ALGO_RING, 8, 1, 256 << 20, 4, false, 2, 100, -1, 2, 100,
       true},
  };
  for (const Case& c : cases) {
    Schedule s;
    std::string err;
    const int64_t count = c.bytes / c.sz;
    CHECK(build_schedule(c.kind, c.algo, c.N, count, 0, c.k, s, err) == COLL_OK, "%s: build (%s)", c.what,
          err.c_str());
    const Bound b = bind_schedule(s, c.sz, true);
    CHECK(!b.phases.empty() && b.phases[0].kind == Phase::ROWS, "%s: no row phase", c.what);
    if (b.phases.empty()) continue;
    const Phase& ph = b.phases[0];
    RowsShapeInput in;
    in.colspace = ph.colspace;
    in.segment = phase_segment(ph);
    in.checksums = c.checksums;
    in.has_reduce = c.kind == COLL_K_ALLREDUCE || c.kind == COLL_K_REDUCESCATTER || c.kind == COLL_K_REDUCE;
    in.elem_size = c.sz;
    in.nranks = c.N;
    in.cus = 256;
    in.resident = 2048;
    in.per_step = c.per_step;
    in.forced_group_tiles = c.forced_gt;
    in.forced_grid = c.forced_grid;
    int asked = 0;
    bool several = false;
    const RowsShape r = rows_shape(in, [&] {
      ++asked;
      several = several_pieces_per_step(b, ph);
      return several;
    });
    if (c.several < 0) {
      CHECK(asked == 0, "%s: asked about pieces per step", c.what);
    } else {
      CHECK(asked == 1, "%s: asked %d times about pieces per step", c.what, asked);
      CHECK(several == (c.several != 0), "%s: several pieces per step %d", c.what, int(several));
    }
    CHECK(r.group_tiles == c.gt, "%s: group tiles %u, want %u", c.what, r.group_tiles, c.gt);
    CHECK(r.cap == c.cap, "%s: grid cap %llu, want %llu", c.what, (unsigned long long)r.cap,
          (unsigned long long)c.cap);
    CHECK(r.group_major == c.group_major, "%s: group-major %d", c.what, int(r.group_major));
  }
}

// ---- column programs ---------------------------------------------------------

long long col_plans = 0;     // programs compiled and executed
long long col_fallbacks = 0; // shapes the column kernel leaves to the row kernel
long long col_batched = 0;   // programs that bring leaves in batches

// Element symbols: input of rank r at element e; reductions mix(d, s).
uint32_t input_sym(int r, int64_t e) { return uint32_t(r) * 0x9E3779B1u + uint32_t(e) * 0x7FEB352Du + 1u; }

void check_colplan(const Shape& sh, const Schedule& s, bool cks) {
  if (s.count > 5000) return;
  const ColPlan p = compile_colplan(s, sh.sz, sh.inplace, cks);
  if (!p.ok) {
    CHECK(sh.kind == COLL_K_ALLTOALL || sh.N > 16, "%s: no column program (%s)", name(sh).c_str(), p.why.c_str());
    ++col_fallbacks;
    return;
  }
  ++col_plans;
  const int N = s.N;
  const int64_t count = s.count;
  // the schedule row by row: final symbols, which elements a row wrote, and
  // each row's destination symbols right after it
  std::vector<std::vector<uint32_t>> cur(size_t(N), std::vector<uint32_t>(static_cast<size_t>(count)));
  std::vector<std::vector<char>> wrote(size_t(N), std::vector<char>(static_cast<size_t>(count), 0));
  for (int r = 0; r < N; ++r)
    for (int64_t e = 0; e < count; ++e) cur[size_t(r)][size_t(e)] = input_sym(r, e);
  std::vector<std::vector<uint32_t>> after(s.rows.size());
  for (const Step& st : s.steps) {
    std::vector<std::vector<uint32_t>> snap;
    for (int64_t i = st.first; i < st.first + st.nrows; ++i) {
      const Row& r = s.rows[size_t(i)];
      snap.emplace_back(cur[size_t(r.src)].begin() + r.src_off, cur[size_t(r.src)].begin() + r.src_off + r.n);
    }
    for (int64_t i = st.first; i < st.first + st.nrows; ++i) {
      const Row& r = s.rows[size_t(i)];
      const std::vector<uint32_t>& sv = snap[size_t(i - st.first)];
      for (int64_t e = 0; e < r.n; ++e) {
        uint32_t& d = cur[size_t(r.dst)][size_t(r.dst_off + e)];
        d = r.reduce ? mix(d, sv[size_t(e)]) : sv[size_t(e)];
        wrote[size_t(r.dst)][size_t(r.dst_off + e)] = 1;
      }
      after[size_t(i)].assign(cur[size_t(r.dst)].begin() + r.dst_off, cur[size_t(r.dst)].begin() + r.dst_off + r.n);
    }
  }
  std::vector<std::vector<int>> stored(size_t(N), std::vector<int>(static_cast<size_t>(count), 0));
  std::vector<int64_t> row_elems(s.rows.size(), 0);
  // refs of each segment
  std::vector<std::vector<ColRowRef>> seg_refs(p.segs.size());
  for (const ColRowRef& r : p.refs) {
    CHECK(r.seg < p.segs.size() && r.row < s.rows.size(), "%s: ref out of range", name(sh).c_str());
    if (r.seg < p.segs.size() && r.row < s.rows.size()) seg_refs[r.seg].push_back(r);
  }
  CHECK(cks || p.refs.empty(), "%s: refs without checksums", name(sh).c_str());
  for (size_t si = 0; si < p.segs.size(); ++si) {
    const ColSeg& sg = p.segs[si];
    CHECK(sg.s0 % uint64_t(sh.sz) == 0 && sg.s1 % uint64_t(sh.sz) == 0 && sg.s0 < sg.s1 && sg.s1 <= p.colspace,
          "%s: segment bytes", name(sh).c_str());
    CHECK(int(sg.nfirst) <= p.v.leaves && (sg.nfirst == sg.nload || sg.nfirst <= COL_BATCH) &&
              sg.nload <= COL_LIST_MAX && sg.nop <= COL_LIST_MAX &&
              sg.nstore <= COL_LIST_MAX && (!cks || int(sg.nop) <= p.v.accs),
          "%s: program exceeds its variant", name(sh).c_str());
    for (const ColRowRef& r : seg_refs[si]) {
      CHECK(r.op < sg.nop, "%s: ref to op %u of %u", name(sh).c_str(), r.op, unsigned(sg.nop));
      const Row& row = s.rows[r.row];
      CHECK(row.dst_off * sh.sz <= int64_t(sg.s0) && int64_t(sg.s1) <= (row.dst_off + row.n) * sh.sz,
            "%s: ref row does not cover its segment", name(sh).c_str());
      if (r.op < sg.nop)
        CHECK((p.code[sg.ops + r.op].arg & 3u) == uint32_t((((-(row.dst_off * sh.sz)) % 4) + 4) % 4),
              "%s: checksum shift", name(sh).c_str());
    }
    std::vector<uint32_t> opval(sg.nop);
    for (int64_t e = int64_t(sg.s0) / sh.sz; e < int64_t(sg.s1) / sh.sz; ++e) {
      std::vector<uint32_t> slot(size_t(p.v.leaves), 0xDEADBEEFu);
      std::vector<char> full(size_t(p.v.leaves), 0);
      // the kernel's loads: leaves 0 .. nfirst-1 into slots 0 .. nfirst-1,
      // then per RELOAD op the next m into slots 0 .. m-1
      for (uint32_t j = 0; j < sg.nload; ++j)
        CHECK(p.code[sg.loads + j].arg < uint32_t(N), "%s: leaf %u", name(sh).c_str(), j);
      for (uint32_t j = 0; j < sg.nfirst; ++j) {
        slot[j] = input_sym(int(p.code[sg.loads + j].arg), e);
        full[j] = 1;
      }
      uint32_t next = sg.nfirst;
      if (e == int64_t(sg.s0) / sh.sz && sg.nfirst < sg.nload) ++col_batched;
      uint32_t y = 0xBADC0DEu;
      bool yset = false;
      for (uint32_t k = 0; k < sg.nop; ++k) {
        const ColInstr& in = p.code[sg.ops + k];
        if (in.flags & CI_RELOAD) {
          const uint32_t m = (in.arg >> 8) & 0xffu;
          CHECK(m >= 1 && m <= COL_BATCH && next + m <= sg.nload, "%s: RELOAD of %u leaves", name(sh).c_str(),
                unsigned(m));
          for (uint32_t j = 0; j < m && next + j < sg.nload; ++j) {
            slot[j] = input_sym(int(p.code[sg.loads + next + j].arg), e);
            full[j] = 1;
          }
          next += m;
        }
        auto opnd = [&](uint8_t ybit, uint8_t sl) {
          if (in.flags & ybit) {
            CHECK(yset, "%s: y read before set", name(sh).c_str());
            return y;
          }
          CHECK(sl < p.v.leaves && full[sl], "%s: empty slot %u read", name(sh).c_str(), unsigned(sl));
          return slot[sl < p.v.leaves ? sl : 0];
        };
        uint32_t v;
        if (in.flags & CI_COMBINE) {
          const uint32_t A = opnd(CI_A_Y, in.a), B = opnd(CI_B_Y, in.b);
          y = mix(A, B);
          yset = true;
          v = y;
          if (in.flags & CI_WRITE) {
            CHECK(in.out < p.v.leaves, "%s: slot %u", name(sh).c_str(), unsigned(in.out));
            slot[in.out < p.v.leaves ? in.out : 0] = y;
            full[in.out < p.v.leaves ? in.out : 0] = 1;
          }
        } else {
          CHECK(cks, "%s: a copy op without checksums", name(sh).c_str());
          v = opnd(CI_A_Y, in.a);
        }
        CHECK(((in.flags & CI_CKS) != 0) == cks, "%s: checksum flag", name(sh).c_str());
        opval[k] = v;
      }
      CHECK(next >= sg.nload, "%s: leaves listed but never loaded", name(sh).c_str());
      for (const ColRowRef& r : seg_refs[si]) {
        const Row& row = s.rows[r.row];
        if (r.op >= sg.nop || e < row.dst_off || e >= row.dst_off + row.n) continue;
        CHECK(after[r.row][size_t(e - row.dst_off)] == opval[r.op], "%s: row %u checksum value at element %lld",
              name(sh).c_str(), r.row, (long long)e);
        ++row_elems[r.row];
      }
      for (uint32_t j = 0; j < sg.nstore; ++j) {
        const ColInstr& in = p.code[sg.stores + j];
        const uint32_t v = (in.flags & CI_A_Y) ? y : slot[in.a < p.v.leaves ? in.a : 0];
        CHECK(!(in.flags & CI_A_Y) || yset, "%s: store of an unset y", name(sh).c_str());
        CHECK(in.arg < uint32_t(N), "%s: store rank", name(sh).c_str());
        if (in.arg >= uint32_t(N)) continue;
        CHECK(v == cur[in.arg][size_t(e)], "%s: rank %u element %lld stored the wrong value", name(sh).c_str(),
              in.arg, (long long)e);
        ++stored[in.arg][size_t(e)];
      }
    }
  }
  // every defined element the schedule changed (out of place: every defined
  // element) is stored once, and nothing else is
  for (int r = 0; r < N; ++r) {
    std::vector<char> def(static_cast<size_t>(count), 0);
    for (auto& d : defined_output(s, r))
      for (int64_t e = d.first; e < d.second; ++e) def[size_t(e)] = 1;
    for (int64_t e = 0; e < count; ++e) {
      const bool changed = wrote[size_t(r)][size_t(e)] && cur[size_t(r)][size_t(e)] != input_sym(r, e);
      const int want = def[size_t(e)] && (changed || !sh.inplace) ? 1 : 0;
      CHECK(stored[size_t(r)][size_t(e)] == want, "%s: rank %d element %lld stored %d times, want %d",
            name(sh).c_str(), r, (long long)e, stored[size_t(r)][size_t(e)], want);
    }
  }
  if (cks)
    for (size_t r = 0; r < s.rows.size(); ++r)
      CHECK(row_elems[r] == s.rows[r].n, "%s: row %zu checksummed over %lld of %lld elements", name(sh).c_str(), r,
            (long long)row_elems[r], (long long)s.rows[r].n);
  // tiles: each segment's bytes are covered by its work groups' tiles
  // exactly; with checksums, the work groups' partial-sum slots are disjoint
  // and every row's refs name exactly its ops' slots in every work group of
  // each segment it covers
  const ColTables t = col_tables(p, 3, s.rows.size());
  const uint64_t tb = uint64_t(COL_THREADS) * uint64_t(p.v.unit);
  std::vector<uint64_t> covered(p.segs.size(), 0);
  std::map<uint64_t, size_t> seg_at;  // segments start at distinct columns
  for (size_t k = 0; k < p.segs.size(); ++k) seg_at[p.segs[k].s0] = k;
  std::vector<std::vector<uint32_t>> seg_parts(p.segs.size());
  std::vector<int> slot_writes(size_t(t.partials), 0);
  for (const ColWork& c : t.work) {
    auto it = seg_at.find(c.s0);
    CHECK(it != seg_at.end() && c.c0 % tb == 0 && c.ntiles >= 1 && c.ntiles <= 3, "%s: work", name(sh).c_str());
    if (it == seg_at.end()) continue;
    const size_t segi = it->second;
    const ColSeg& sg = p.segs[segi];
    CHECK(c.s0 == sg.s0 && c.s1 == sg.s1 && c.loads == sg.loads && c.ops == sg.ops && c.stores == sg.stores &&
              c.nfirst == sg.nfirst && c.nload == sg.nload && c.nop == sg.nop && c.nstore == sg.nstore,
          "%s: a work group's program is not its segment's", name(sh).c_str());
    const uint64_t lo = std::max<uint64_t>(c.c0, sg.s0), hi = std::min<uint64_t>(c.c0 + c.ntiles * tb, sg.s1);
    CHECK(lo < hi, "%s: a work group with no bytes of its segment", name(sh).c_str());
    if (lo < hi) covered[segi] += hi - lo;
    if (cks) {
      seg_parts[segi].push_back(c.part);
      for (uint32_t k = 0; k < c.nop; ++k)
        if (uint64_t(c.part) + k < t.partials) ++slot_writes[c.part + k];
        else CHECK(false, "%s: partial slot out of range", name(sh).c_str());
    }
  }
  for (size_t k = 0; k < p.segs.size(); ++k)
    CHECK(covered[k] == p.segs[k].s1 - p.segs[k].s0, "%s: segment %zu covered %llu bytes", name(sh).c_str(), k,
          (unsigned long long)covered[k]);
  if (cks) {
    for (size_t q = 0; q < slot_writes.size(); ++q)
      CHECK(slot_writes[q] == 1, "%s: partial slot %zu written %d times", name(sh).c_str(), q, slot_writes[q]);
    CHECK(t.row_off.size() == s.rows.size() + 1 && t.row_off.back() == t.refs.size(), "%s: row offsets",
          name(sh).c_str());
    // the slots each row adds, from its ColRefs, against its refs
    for (size_t r = 0; r < s.rows.size() && t.row_off.size() == s.rows.size() + 1; ++r) {
      std::vector<uint64_t> got, want;
      for (uint32_t i = t.row_off[r]; i < t.row_off[r + 1]; ++i)
        for (uint32_t w = 0; w < t.refs[i].count; ++w) got.push_back(uint64_t(t.refs[i].first) + uint64_t(w) * t.refs[i].stride);
      for (const ColRowRef& rf : p.refs)
        if (rf.row == r)
          for (uint32_t part : seg_parts[rf.seg]) want.push_back(uint64_t(part) + rf.op);
      std::sort(got.begin(), got.end());
      std::sort(want.begin(), want.end());
      CHECK(got == want, "%s: row %zu adds the wrong partial slots", name(sh).c_str(), r);
    }
  }
}

int main(int argc, char** argv) {
  for (int i = 1; i < argc; ++i) {
    const std::string a = argv[i];
    if (a == "--exec=none") exec_mode = EXEC_NONE;
    else if (a == "--exec=small") exec_mode = EXEC_SMALL;
    else if (a == "--exec=sample") exec_mode = EXEC_SAMPLE;
    else if (a == "--exec=all") exec_mode = EXEC_ALL;
    else {
      std::printf("unknown argument %s\n", a.c_str());
      return 2;
    }
  }
  check_launch_shapes();
  std::vector<Shape> shapes;
  const coll_kind_t kinds[] = {COLL_K_ALLREDUCE, COLL_K_REDUCESCATTER, COLL_K_ALLGATHER, COLL_K_BROADCAST,
                               COLL_K_SCATTER,   COLL_K_GATHER,        COLL_K_ALLTOALL,  COLL_K_REDUCE};
  for (coll_kind_t kind : kinds)
    for (int a = 1; a <= int(COLL_ALGO_BIDIR_RING); ++a) {
      if (a == int(COLL_ALGO_AUTO)) continue;
      for (int N : {1, 2, 3, 5, 8, 13, 16})
        for (int64_t count : {int64_t(0), int64_t(1), int64_t(7), int64_t(1000), int64_t(4099), int64_t(65536 + 77)})
          for (int sz : {1, 2, 4})
            for (int inplace = 0; inplace < 2; ++inplace) {
              const int root = N / 2;
              for (int k : {1, 3}) {
                Shape s{kind, coll_algo_t(a), N, count, root, k, sz, inplace != 0};
                if (kind == COLL_K_ALLTOALL) {
                  if (inplace || count % N) continue;
                }
                std::string err;
                if (validate_schedule_args(kind, s.algo, N, count, root, k, err) != COLL_OK) continue;
                if (!algo_pipelined(s.algo) && k != 1) continue;
                shapes.push_back(s);
              }
            }
      // more ranks than the column kernel's slots: batched leaves or the row kernel
      for (int N : {17, 32, 64})
        for (int64_t count : {int64_t(1), int64_t(77), int64_t(1000)})
          for (int sz : {2, 4})
            for (int inplace = 0; inplace < 2; ++inplace) {
              Shape s{kind, coll_algo_t(a), N, count * (kind == COLL_K_ALLTOALL ? N : 1), N / 3, 1, sz, inplace != 0};
              if (kind == COLL_K_ALLTOALL && inplace) continue;
              std::string err;
              if (validate_schedule_args(kind, s.algo, N, s.count, s.root, 1, err) != COLL_OK) continue;
              shapes.push_back(s);
            }
    }
  int nlists = 0;
  for (const Shape& sh : shapes) {
    Schedule s;
    std::string err;
    const coll_status_t st = build_schedule(sh.kind, sh.algo, sh.N, sh.count, sh.root, sh.k, s, err);
    CHECK(st == COLL_OK, "%s: build_schedule %d (%s)", name(sh).c_str(), int(st), err.c_str());
    if (st != COLL_OK) continue;
    const std::string hz = check_schedule(s);
    CHECK(hz.empty(), "%s: hazard %s", name(sh).c_str(), hz.c_str());
    const Bound b = bind_schedule(s, sh.sz, sh.inplace);
    // row-kernel steps: per row, the items cover the destination bytes once
    if (sh.kind != COLL_K_ALLTOALL) {
      std::map<uint32_t, uint64_t> bytes;
      for (const Phase& ph : b.phases)
        if (ph.kind == Phase::ROWS)
          for (uint32_t st2 = ph.s0; st2 < ph.s1; ++st2)
            for (uint32_t i = 0; i < b.steps[st2].nitems; ++i) {
              const DevItem& it = b.items[b.steps[st2].item0 + i];
              if (it.row != NO_ROW) bytes[it.row] += it.col1 - it.col0;
            }
      for (size_t r = 0; r < s.rows.size(); ++r)
        CHECK(bytes[uint32_t(r)] == uint64_t(s.rows[r].n) * uint64_t(sh.sz), "%s: row %zu covered %llu of %lld",
              name(sh).c_str(), r, (unsigned long long)bytes[uint32_t(r)], (long long)(s.rows[r].n * sh.sz));
    }
    check_lists(sh, s, b, nlists);
    if (exec_mode != EXEC_NONE || sh.count <= 1000) {
      check_colplan(sh, s, false);
      check_colplan(sh, s, true);
    }
  }
  CHECK(fwd_marks > 0, "no forwarding mark was made");
  CHECK(no_store_marks > 0, "no store was skipped");
  CHECK(exec_mode == EXEC_NONE || exec_lists > 0, "no list was executed");
  CHECK(col_plans > 0, "no column program was checked");
  CHECK(col_batched > 0, "no batched column program was checked");
  std::printf("host_check: %zu shapes, %d lists, %lld forwarding marks, %lld skipped stores, %lld list executions, "
              "%lld column programs (%lld batched; %lld shapes left to the row kernel), %s\n",
              shapes.size(), nlists, fwd_marks, no_store_marks, exec_lists, col_plans, col_batched, col_fallbacks,
              failures ? "FAILED" : "ok");
  return failures ? 1 : 0;
}
