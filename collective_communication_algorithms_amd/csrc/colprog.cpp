#include "colprog.h"

#include <algorithm>
#include <map>

#include "bind.h"

namespace coll {
namespace {

// A value a column holds somewhere in the schedule: an input (leaf) or the
// result of one recv_and_reduce row.
struct Node {
  bool leaf = true;
  int rank = -1;        // leaf: whose input
  int a = -1, b = -1;   // combine: old destination value, source value
};

struct Event {          // one covering row, in execution order
  int node = -1;        // reduce: the new value; copy: the value copied
  bool combine = false;
  uint32_t row = 0;
  uint32_t shift = 0;   // (-row start byte) mod 4
};

uint32_t row_shift(const Row& r, int sz) { return uint32_t((((-(r.dst_off * sz)) % 4) + 4) % 4); }

// Variants the column kernel is built in (colkernel.hip), smallest first.  A
// 64-slot variant of 4-byte units was built and measured: its 64-leaf
// programs are bound by instruction issue (64-rank ReduceScatter bf16 x 256
// MiB: Ring 10.6 ms, halving-doubling 11.2 ms, against 3.07 / 6.86 ms in the
// row kernel), so programs that need more than 16 slots run in the row kernel.
const ColVariant kVariants[] = {{16, 8, 0}, {16, 8, 16}, {16, 16, 0}, {16, 16, 32}};

}  // namespace

ColPlan compile_colplan(const Schedule& s, int sz, bool inplace, bool checksums, size_t max_segments) {
  ColPlan p;
  auto fail = [&](const char* w) {
    p.ok = false;
    p.why = w;
    p.segs.clear();
    p.code.clear();
    p.refs.clear();
    return p;
  };
  if (s.kind == COLL_K_ALLTOALL) return fail("AllToAll rows move data between offsets");
  if (s.N > COL_LIST_MAX) return fail("more ranks than a program list holds");
  for (const Step& st : s.steps)
    if (st.local || st.staged) return fail("a staged or local step");
  for (const Row& r : s.rows)
    if (r.src_off != r.dst_off || r.from_send) return fail("a row moves data between offsets");
  const int N = s.N;
  p.colspace = uint64_t(s.count) * uint64_t(sz);

  // segment boundaries: every row's ends and every defined output's ends
  std::vector<int64_t> cut{0, s.count};
  for (const Row& r : s.rows) {
    cut.push_back(r.dst_off);
    cut.push_back(r.dst_off + r.n);
  }
  std::vector<std::vector<std::pair<int64_t, int64_t>>> defined(static_cast<size_t>(N));
  for (int r = 0; r < N; ++r) {
    defined[size_t(r)] = defined_output(s, r);
    for (auto& d : defined[size_t(r)]) {
      cut.push_back(d.first);
      cut.push_back(d.second);
    }
  }
  std::sort(cut.begin(), cut.end());
  cut.erase(std::unique(cut.begin(), cut.end()), cut.end());
  while (!cut.empty() && cut.back() > s.count) cut.pop_back();
  const size_t nseg = cut.size() < 2 ? 0 : cut.size() - 1;
  if (nseg > max_segments) return fail("too many segments");

  // the covering rows of every segment, in row (hence step) order
  std::vector<std::vector<uint32_t>> cover(nseg);
  uint64_t work = 0;
  for (size_t ri = 0; ri < s.rows.size(); ++ri) {
    const Row& r = s.rows[ri];
    if (r.n <= 0) continue;
    const size_t a = size_t(std::lower_bound(cut.begin(), cut.end(), r.dst_off) - cut.begin());
    const size_t b = size_t(std::lower_bound(cut.begin(), cut.end(), r.dst_off + r.n) - cut.begin());
    for (size_t k = a; k < b; ++k) cover[k].push_back(uint32_t(ri));
    work += b - a;
    if (work > (uint64_t(1) << 26)) return fail("too many row pieces");
  }

  std::vector<Node> nodes;
  std::vector<Event> ev;
  std::vector<int> val(static_cast<size_t>(N)), srcv;
  std::vector<char> written(static_cast<size_t>(N));
  std::vector<std::pair<int, int>> stores;  // (rank, node)
  for (size_t k = 0; k < nseg; ++k) {
    const int64_t e0 = cut[k], e1 = cut[k + 1];
    nodes.clear();
    ev.clear();
    stores.clear();
    std::fill(val.begin(), val.end(), -1);
    std::fill(written.begin(), written.end(), 0);
    auto get = [&](int r) {
      if (val[size_t(r)] < 0) {
        Node n;
        n.rank = r;
        nodes.push_back(n);
        val[size_t(r)] = int(nodes.size()) - 1;
      }
      return val[size_t(r)];
    };
    const std::vector<uint32_t>& rows = cover[k];
    for (size_t i = 0; i < rows.size();) {
      size_t j = i;
      const int32_t step = s.rows[rows[i]].step;
      while (j < rows.size() && s.rows[rows[j]].step == step) ++j;
      // every source of the step is taken before any row of it applies
      srcv.clear();
      for (size_t q = i; q < j; ++q) srcv.push_back(get(s.rows[rows[q]].src));
      for (size_t q = i; q < j; ++q) {
        const Row& r = s.rows[rows[q]];
        Event e;
        e.row = rows[q];
        e.shift = row_shift(r, sz);
        if (r.reduce) {
          Node n;
          n.leaf = false;
          n.a = get(r.dst);
          n.b = srcv[q - i];
          nodes.push_back(n);
          e.node = int(nodes.size()) - 1;
          e.combine = true;
        } else {
          e.node = srcv[q - i];
        }
        val[size_t(r.dst)] = e.node;
        written[size_t(r.dst)] = 1;
        ev.push_back(e);
      }
      i = j;
    }
    for (int r = 0; r < N; ++r) {
      bool def = false;
      for (auto& d : defined[size_t(r)])
        if (d.first <= e0 && e1 <= d.second) def = true;
      if (!def) continue;
      if (!inplace) {
        stores.push_back({r, get(r)});
      } else if (written[size_t(r)]) {
        // in place, memory still holds the input until the stores: a rank
        // that ends with its own input needs none
        const Node& n = nodes[size_t(val[size_t(r)])];
        if (!(n.leaf && n.rank == r)) stores.push_back({r, val[size_t(r)]});
      }
    }

    // values something needs: the stores', every row's when checksums are on,
    // and their operands
    std::vector<char> live(nodes.size(), 0);
    for (auto& st : stores) live[size_t(st.second)] = 1;
    if (checksums)
      for (const Event& e : ev) live[size_t(e.node)] = 1;
    for (size_t n = nodes.size(); n-- > 0;)
      if (live[n] && !nodes[n].leaf) {
        live[size_t(nodes[n].a)] = 1;
        live[size_t(nodes[n].b)] = 1;
      }
    // with checksums: one op per combine, and one per copy whose value and
    // rotation no op before it carries; `carrier[i]`: the op whose value is
    // event i's row's checksum over this segment
    std::vector<Event> ops;
    std::vector<int> carrier(ev.size(), -1);
    std::map<std::pair<int, uint32_t>, int> carried;  // (value, shift) -> op
    for (size_t i = 0; i < ev.size(); ++i) {
      const Event& e = ev[i];
      if (checksums) {
        auto key = std::make_pair(e.node, e.shift);
        auto it = carried.find(key);
        if (!e.combine && it != carried.end()) {
          carrier[i] = it->second;
          continue;
        }
        carrier[i] = int(ops.size());
        carried[key] = int(ops.size());
        ops.push_back(e);
      } else if (e.combine && live[size_t(e.node)]) {
        ops.push_back(e);
      }
    }
    if (ops.empty() && stores.empty()) continue;  // nothing to load, compute or store

    // positions: op i at i, store j at ops.size() + j; the last use of each value
    const int K = int(ops.size());
    std::vector<int> last(nodes.size(), -1);
    for (int i = 0; i < K; ++i) {
      const Event& e = ops[size_t(i)];
      if (e.combine) {
        last[size_t(nodes[size_t(e.node)].a)] = i;
        last[size_t(nodes[size_t(e.node)].b)] = i;
      } else {
        last[size_t(e.node)] = i;
      }
    }
    for (size_t j = 0; j < stores.size(); ++j) last[size_t(stores[j].second)] = K + int(j);
    std::vector<int> next_comb(size_t(K), K);  // the first combine after op i (K: none)
    for (int i = K - 1, nxt = K; i >= 0; --i) {
      next_comb[size_t(i)] = nxt;
      if (ops[size_t(i)].combine) nxt = i;
    }

    ColSeg sg{};
    sg.s0 = uint64_t(e0) * uint64_t(sz);
    sg.s1 = uint64_t(e1) * uint64_t(sz);
    sg.loads = uint32_t(p.code.size());
    std::vector<int> slot(nodes.size(), -1), owner;
    for (size_t n = 0; n < nodes.size(); ++n)
      if (nodes[n].leaf && live[n]) {
        slot[n] = int(owner.size());
        owner.push_back(int(n));
        ColInstr in{};
        in.a = uint8_t(slot[n] & 0xff);
        in.arg = uint32_t(nodes[n].rank);
        p.code.push_back(in);
      }
    const int nload = int(owner.size());
    sg.ops = uint32_t(p.code.size());
    int y = -1;
    for (int i = 0; i < K; ++i) {
      const Event& e = ops[size_t(i)];
      ColInstr in{};
      in.arg = e.shift;
      auto operand = [&](int n, uint8_t ybit, uint8_t& field) {
        if (n == y) {
          in.flags |= ybit;
        } else {
          field = uint8_t(slot[size_t(n)] & 0xff);
          if (slot[size_t(n)] < 0) p.why = "internal: a value has no slot";
        }
      };
      if (e.combine) {
        const Node& n = nodes[size_t(e.node)];
        in.flags |= CI_COMBINE;
        operand(n.a, CI_A_Y, in.a);
        operand(n.b, CI_B_Y, in.b);
        const int nc = next_comb[size_t(i)];
        if (nc < K && last[size_t(e.node)] > nc) {
          // needed after the next combine replaces y: keep it in a slot whose
          // value is not needed after this op
          int s = -1;
          for (size_t q = 0; q < owner.size() && s < 0; ++q)
            if (owner[q] < 0 || last[size_t(owner[q])] <= i) s = int(q);
          if (s < 0) {
            s = int(owner.size());
            owner.push_back(-1);
          }
          if (owner[size_t(s)] >= 0) slot[size_t(owner[size_t(s)])] = -1;
          owner[size_t(s)] = e.node;
          slot[size_t(e.node)] = s;
          in.flags |= CI_WRITE;
          in.out = uint8_t(s & 0xff);
        }
        y = e.node;
      } else {
        operand(e.node, CI_A_Y, in.a);
      }
      if (checksums) in.flags |= CI_CKS;
      p.code.push_back(in);
    }
    sg.stores = uint32_t(p.code.size());
    for (auto& st : stores) {
      ColInstr in{};
      in.arg = uint32_t(st.first);
      if (st.second == y) {
        in.flags = CI_A_Y;
      } else {
        in.a = uint8_t(slot[size_t(st.second)] & 0xff);
        if (slot[size_t(st.second)] < 0) p.why = "internal: a stored value has no slot";
      }
      p.code.push_back(in);
    }
    if (!p.why.empty()) return fail("internal: a value has no slot");
    sg.nload = uint16_t(nload);
    sg.nop = uint16_t(K);
    sg.nstore = uint16_t(stores.size());
    if (nload > COL_LIST_MAX || K > COL_LIST_MAX || int(stores.size()) > COL_LIST_MAX)
      return fail("a program list longer than 64 instructions");
    p.max_leaves = std::max<uint32_t>(p.max_leaves, uint32_t(nload));
    p.max_slots = std::max<uint32_t>(p.max_slots, uint32_t(owner.size()));
    p.max_ops = std::max<uint32_t>(p.max_ops, uint32_t(K));
    p.max_stores = std::max<uint32_t>(p.max_stores, uint32_t(stores.size()));
    p.moved_bytes += uint64_t(nload + int(stores.size())) * (sg.s1 - sg.s0);
    if (checksums)
      for (size_t i = 0; i < ev.size(); ++i)
        p.refs.push_back(ColRowRef{ev[i].row, uint32_t(p.segs.size()), uint32_t(carrier[i])});
    p.segs.push_back(sg);
  }
  for (const ColVariant& v : kVariants) {
    if ((v.accs > 0) != checksums) continue;
    if (int(p.max_slots) > v.leaves || (checksums && int(p.max_ops) > v.accs) || sz > v.unit) continue;
    p.v = v;
    p.ok = true;
    return p;
  }
  return fail("no kernel variant holds the programs");
}

ColTables col_tables(const ColPlan& p, uint32_t tiles_per_group, size_t nrows) {
  ColTables t;
  const uint64_t tb = uint64_t(COL_THREADS) * uint64_t(p.v.unit);
  const uint32_t per = std::max<uint32_t>(1, std::min<uint32_t>(tiles_per_group, 65535));
  const bool cks = p.v.accs > 0;
  std::vector<uint64_t> base(p.segs.size()), groups(p.segs.size());
  for (size_t k = 0; k < p.segs.size(); ++k) {
    const ColSeg& sg = p.segs[k];
    const uint64_t t0 = sg.s0 / tb, t1 = (sg.s1 + tb - 1) / tb;
    base[k] = t.partials;
    groups[k] = 0;
    for (uint64_t q = t0; q < t1; q += per) {
      ColWork c{};
      c.c0 = q * tb;
      c.s0 = sg.s0;
      c.s1 = sg.s1;
      c.loads = sg.loads;
      c.ops = sg.ops;
      c.stores = sg.stores;
      c.part = uint32_t(cks ? t.partials : 0);
      c.nload = sg.nload;
      c.nop = sg.nop;
      c.nstore = sg.nstore;
      c.ntiles = uint16_t(std::min<uint64_t>(per, t1 - q));
      t.work.push_back(c);
      ++groups[k];
      if (cks) t.partials += sg.nop;
    }
  }
  if (cks) {
    t.row_off.assign(nrows + 1, 0);
    for (const ColRowRef& r : p.refs) ++t.row_off[r.row + 1];
    for (size_t r = 0; r < nrows; ++r) t.row_off[r + 1] += t.row_off[r];
    t.refs.resize(p.refs.size());
    std::vector<uint32_t> fill(t.row_off.begin(), t.row_off.end() - 1);
    for (const ColRowRef& r : p.refs) {
      ColRef c{};
      c.first = uint32_t(base[r.seg] + r.op);
      c.count = uint32_t(groups[r.seg]);
      c.stride = p.segs[r.seg].nop;
      t.refs[fill[r.row]++] = c;
    }
  }
  return t;
}

}  // namespace coll
