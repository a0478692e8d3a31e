#include "colprog.h"

#include <algorithm>
#include <cstdlib>
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

// Variants the column kernel is built in (colkernel.hip), smallest first.
// Programs over 8 slots bring their leaves in batches (batched variants,
// kPlainSlots) rather than holding all of them: a 64-slot variant of 4-byte
// units was built and measured, and its 64-leaf programs were bound by
// instruction issue (64-rank ReduceScatter bf16 x 256 MiB: Ring 10.6 ms,
// halving-doubling 11.2 ms, where batches of 8 run them in 2.9 ms).
// Checksums: a file of 16 per-lane accumulators for programs of up to 8
// leaves and 16 ops, wave sums merged across lanes as the ops arrive for the
// others (colkernel.hip).  Larger accumulator files cost occupancy more than
// the sums cost instructions: measured on MI355X with row checksums, files of
// 32 (16 slots, 191-260 VGPRs) against per-tile sums (104-114 VGPRs):
// AllReduce fp32 16 x 64 MiB Ring 0.620 against 0.451 ms, 32 x 64 MiB
// halving-doubling 1.392 against 0.840 ms, ReduceScatter bf16 32 x 256 MiB
// Ring 4.756 against 1.917 ms.  The 16-accumulator file (97 VGPRs for fp32)
// stays where it wins: Ring AllReduce fp32 8 x 256 MiB 0.724 ms against 0.758
// ms with merged sums (80 VGPRs): a wave that stores 8 buffers runs best at
// the file's lower occupancy, as the plain 8-load, 8-store pattern does at 4
// work groups per CU.  Programs of up to 8 ops and at most 2 stores run
// faster merged (bf16 8 x 256 MiB tree Reduce 0.464 -> 0.426 ms, Ring
// ReduceScatter 0.454 -> 0.416 ms), and so do single-leaf programs
// (AllGather bf16 8 x 256 MiB 0.418 -> 0.394 ms, its leaf loaded alone: the
// {1 slot, 8 ops} entry).
// Without checksums, programs of 2 or more leaves and 8 stores (the AllReduces
// over 8 ranks) load their leaves in pairs at 4 waves per SIMD, the shape the
// checksummed AllReduce runs at, where the plain variant holds 8 waves with one
// load in flight.  Measured on MI355X, plain -> paired, fp32 8 x 256 MiB Ring
// 0.736 -> 0.715 ms, halving-doubling 0.737 -> 0.722, double binary tree
// 0.737 -> 0.717, bf16 Ring 0.740 -> 0.729; Ring 8 x 128 MiB 0.370 -> 0.348,
// 8 x 32 MiB 0.094 -> 0.090 (pairs at 8 waves per SIMD: 0.764 ms at 256 MiB).
// Fewer stores lose (Ring AllReduce over 4 ranks 0.353 -> 0.373 ms), and so do
// small column spaces (abi.cpp: fit_col_variant); programs of one leaf or one
// store keep the plain variant's occupancy.
// Batched programs of 8 or more stores (AllReduces over 9-64 ranks) likewise
// run at fewer work groups per CU (`capped`: reserved LDS).  Without
// checksums: Ring AllReduce fp32 16 x 64 MiB 0.384 -> 0.360 ms,
// halving-doubling 32 x 64 MiB 0.811 -> 0.751, Ring 64 x 64 MiB 1.603 ->
// 1.572; with them: 0.412 -> 0.395, 0.819 -> 0.809, 1.796 -> 1.770 ms.
// One-store programs (ReduceScatter) lose (64 x 256 MiB bf16 2.96 -> 3.91 ms
// without checksums, 3.24 -> 3.40 ms with).
const ColVariant kVariants[] = {{16, 8, -1, false, COL_LIST_MAX_STORES, 8, 2},
                                {16, 8, 0, false},
                                {16, 1, 8, false},
                                {16, 8, 8, false, 2},
                                {16, 8, 16, false},
                                {16, 8, 64, false},
                                {16, 8, 0, true, COL_LIST_MAX_STORES, 8, 2, true},
                                {16, 16, 0, true, COL_LIST_MAX_STORES, 8, 2, true},
                                {16, 8, 0, true},
                                {16, 16, 0, true},
                                {16, 8, 64, true, COL_LIST_MAX_STORES, 8, 2, true},
                                {16, 16, 64, true, COL_LIST_MAX_STORES, 8, 2, true},
                                {16, 8, 64, true},
                                {16, 16, 64, true}};


// Register slots of the largest column-kernel variant.
constexpr int kMaxSlots = 16;
// Programs over this many slots run batched: leaves in 8 register slots,
// partial results in 8 more in LDS.  Measured on MI355X against holding 9-16
// slots in registers (116-127 VGPRs, 4 waves per SIMD, against 92-114 and
// 4-5), no checksums / checksums: ReduceScatter bf16 16 x 256 MiB 1.091 ->
// 0.777 / 1.36 -> 0.95 ms, Reduce fp32 16 x 64 MiB 0.291 -> 0.190 ms,
// AllReduce fp32 16 x 64 MiB halving-doubling 0.431 -> 0.384 / 0.511 ->
// 0.409 ms, Ring 0.399 -> 0.382 ms.
constexpr int kPlainSlots = 8;

// One segment's program as instruction lists.
struct Emitted {
  std::vector<ColInstr> loads, ops, stores;
  std::vector<int> pos;   // ops[] index of each input op (the program may reorder them)
  int nfirst = 0;         // leaves loaded before the ops
  int slots = 0;          // register slots the program uses
};

// The ops whose value stays in y until the next combine: positions of the
// first combine after each op (K: none).
std::vector<int> next_combine(const std::vector<Event>& ops) {
  const int K = int(ops.size());
  std::vector<int> nc(size_t(K), K);
  for (int i = K - 1, nxt = K; i >= 0; --i) {
    nc[size_t(i)] = nxt;
    if (ops[size_t(i)].combine) nxt = i;
  }
  return nc;
}

// Last use of every value: op i at position i, store j at ops.size() + j.
std::vector<int> last_uses(const std::vector<Node>& nodes, const std::vector<Event>& ops,
                           const std::vector<std::pair<int, int>>& stores) {
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
  return last;
}

// Every live leaf loaded before the ops, into slots 0 .. L-1, the ops in the
// rows' order; a value that outlives y goes to a slot no later op needs.
bool emit_plain(const std::vector<Node>& nodes, const std::vector<char>& live, const std::vector<Event>& ops,
                const std::vector<std::pair<int, int>>& stores, bool checksums, Emitted& em) {
  const int K = int(ops.size());
  const std::vector<int> last = last_uses(nodes, ops, stores);
  const std::vector<int> next_comb = next_combine(ops);
  bool ok = true;
  std::vector<int> slot(nodes.size(), -1), owner;
  for (size_t n = 0; n < nodes.size(); ++n)
    if (nodes[n].leaf && live[n]) {
      slot[n] = int(owner.size());
      owner.push_back(int(n));
      ColInstr in{};
      in.a = uint8_t(slot[n] & 0xff);
      in.arg = uint32_t(nodes[n].rank);
      em.loads.push_back(in);
    }
  em.nfirst = int(em.loads.size());
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
        if (slot[size_t(n)] < 0) ok = false;
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
    em.ops.push_back(in);
    em.pos.push_back(i);
  }
  for (auto& st : stores) {
    ColInstr in{};
    in.arg = uint32_t(st.first);
    if (st.second == y) {
      in.flags = CI_A_Y;
    } else {
      in.a = uint8_t(slot[size_t(st.second)] & 0xff);
      if (slot[size_t(st.second)] < 0) ok = false;
    }
    em.stores.push_back(in);
  }
  em.slots = int(owner.size());
  return ok;
}

// Programs with more leaves than slots: the combines in depth-first order
// from the final values (each value after its operands, old destination
// value first; a combine and
// its operands are the schedule's, so the arithmetic is unchanged), leaves in
// order of first use, brought in batches of up to COL_BATCH into slots 0 ..
// COL_BATCH-1 (a RELOAD flag on the op that first needs a batch) once the
// batch before is consumed, a batch ending early rather than between the two
// leaf operands of one combine; values that outlive y go to slots COL_BATCH ..
// kMaxSlots-1.  False when the order does not allow it (a
// batch boundary between two leaves one combine needs, a copy's checksum of
// a leaf, a stored leaf outside the last batch, more than kMaxSlots slots).
bool emit_batched(const std::vector<Node>& nodes, const std::vector<Event>& ops_in,
                  const std::vector<std::pair<int, int>>& stores, bool checksums, Emitted& em) {
  const int B = int(COL_BATCH);
  // each combine's event, and the copies' checksum events per value
  std::vector<int> event_of(nodes.size(), -1);
  std::vector<std::vector<int>> copies_of(nodes.size());
  for (size_t i = 0; i < ops_in.size(); ++i) {
    if (ops_in[i].combine) event_of[size_t(ops_in[i].node)] = int(i);
    else if (nodes[size_t(ops_in[i].node)].leaf) return false;
    else copies_of[size_t(ops_in[i].node)].push_back(int(i));
  }
  // depth-first order of the combines, from the values the events and the
  // stores need
  std::vector<int> order;
  std::vector<char> seen(nodes.size(), 0);
  std::vector<std::pair<int, int>> stack;  // (node, next child to visit)
  auto visit = [&](int root) {
    if (nodes[size_t(root)].leaf || seen[size_t(root)]) return;
    stack.push_back({root, 0});
    seen[size_t(root)] = 1;
    while (!stack.empty()) {
      auto& top = stack.back();
      const Node& n = nodes[size_t(top.first)];
      if (top.second < 2) {
        const int c = top.second == 0 ? n.a : n.b;
        ++top.second;
        if (!nodes[size_t(c)].leaf && !seen[size_t(c)]) {
          seen[size_t(c)] = 1;
          stack.push_back({c, 0});
        }
      } else {
        order.push_back(top.first);
        stack.pop_back();
      }
    }
  };
  // roots first (the stored values, then values no combine reads), so that
  // each subtree is finished before the next starts
  std::vector<char> operand(nodes.size(), 0);
  for (const Event& e : ops_in)
    if (e.combine) {
      operand[size_t(nodes[size_t(e.node)].a)] = 1;
      operand[size_t(nodes[size_t(e.node)].b)] = 1;
    }
  for (auto& st : stores) visit(st.second);
  for (const Event& e : ops_in)
    if (!operand[size_t(e.node)]) visit(e.node);
  for (const Event& e : ops_in) visit(e.node);
  // the ops in that order, each combine followed by the copies of its value
  std::vector<Event> ops;
  std::vector<int> src;  // ops_in index of each op
  for (int n : order) {
    if (event_of[size_t(n)] < 0) return false;  // a needed value no event computes
    ops.push_back(ops_in[size_t(event_of[size_t(n)])]);
    src.push_back(event_of[size_t(n)]);
    for (int c : copies_of[size_t(n)]) {
      ops.push_back(ops_in[size_t(c)]);
      src.push_back(c);
    }
  }
  if (ops.size() != ops_in.size()) return false;
  // leaves in order of first use
  std::vector<int> leaves;
  std::vector<int> leaf_idx(nodes.size(), -1);
  auto take = [&](int n) {
    if (nodes[size_t(n)].leaf && leaf_idx[size_t(n)] < 0) {
      leaf_idx[size_t(n)] = int(leaves.size());
      leaves.push_back(n);
    }
  };
  for (const Event& e : ops)
    if (e.combine) {
      take(nodes[size_t(e.node)].a);
      take(nodes[size_t(e.node)].b);
    }
  for (auto& st : stores) take(st.second);
  const int K = int(ops.size());
  const std::vector<int> last = last_uses(nodes, ops, stores);
  const std::vector<int> next_comb = next_combine(ops);
  for (int n : leaves) {
    ColInstr in{};
    in.a = uint8_t(leaf_idx[size_t(n)] % B);
    in.arg = uint32_t(nodes[size_t(n)].rank);
    em.loads.push_back(in);
  }
  // a batch holds up to B leaves, fewer where the next would split the two
  // leaf operands of one combine
  std::vector<int> pair_of(nodes.size(), -1);
  for (const Event& e : ops)
    if (e.combine && nodes[size_t(nodes[size_t(e.node)].a)].leaf && nodes[size_t(nodes[size_t(e.node)].b)].leaf) {
      pair_of[size_t(nodes[size_t(e.node)].a)] = nodes[size_t(e.node)].b;
      pair_of[size_t(nodes[size_t(e.node)].b)] = nodes[size_t(e.node)].a;
    }
  auto batch_size = [&](int from) {
    int m = std::min(B, int(leaves.size()) - from);
    if (from + m < int(leaves.size()) && m > 1 && pair_of[size_t(leaves[size_t(from + m - 1)])] == leaves[size_t(from + m)])
      --m;
    return m;
  };
  std::vector<int> slot(nodes.size(), -1), owner(size_t(kMaxSlots), -1);
  int next_leaf = batch_size(0);  // leaves[0 .. next_leaf) are or were loaded
  em.nfirst = next_leaf;
  for (int q = 0; q < next_leaf; ++q) {
    slot[size_t(leaves[size_t(q)])] = q;
    owner[size_t(q)] = leaves[size_t(q)];
  }
  int y = -1, slots = next_leaf;
  em.pos.assign(ops_in.size(), -1);
  int reload_next = 0;  // leaves the next op brings in first
  auto reload = [&](int at) {
    // every loaded leaf must be consumed before op `at`
    for (int q = 0; q < B; ++q)
      if (owner[size_t(q)] >= 0 && last[size_t(owner[size_t(q)])] >= at) return false;
    const int m = batch_size(next_leaf);
    if (m <= 0 || reload_next) return false;
    reload_next = m;
    for (int q = 0; q < B; ++q) {
      if (owner[size_t(q)] >= 0) slot[size_t(owner[size_t(q)])] = -1;
      owner[size_t(q)] = -1;
    }
    for (int q = 0; q < m; ++q) {
      slot[size_t(leaves[size_t(next_leaf + q)])] = q;
      owner[size_t(q)] = leaves[size_t(next_leaf + q)];
    }
    slots = std::max(slots, m);
    next_leaf += m;
    return true;
  };
  for (int i = 0; i < K; ++i) {
    const Event& e = ops[size_t(i)];
    if (e.combine) {
      for (int c : {nodes[size_t(e.node)].a, nodes[size_t(e.node)].b})
        if (nodes[size_t(c)].leaf && slot[size_t(c)] < 0) {
          if (leaf_idx[size_t(c)] != next_leaf || !reload(i)) return false;
        }
      // both leaf operands must be in slots now (a reload may not evict the other)
      for (int c : {nodes[size_t(e.node)].a, nodes[size_t(e.node)].b})
        if (c != y && slot[size_t(c)] < 0) return false;
    }
    ColInstr in{};
    in.arg = e.shift;
    auto operand = [&](int n, uint8_t ybit, uint8_t& field) {
      if (n == y) {
        in.flags |= ybit;
        return true;
      }
      field = uint8_t(slot[size_t(n)] & 0xff);
      return slot[size_t(n)] >= 0;
    };
    if (e.combine) {
      const Node& n = nodes[size_t(e.node)];
      in.flags |= CI_COMBINE;
      if (!operand(n.a, CI_A_Y, in.a) || !operand(n.b, CI_B_Y, in.b)) return false;
      const int nc = next_comb[size_t(i)];
      if (nc < K && last[size_t(e.node)] > nc) {
        int s = -1;
        for (int q = B; q < kMaxSlots && s < 0; ++q)
          if (owner[size_t(q)] < 0 || last[size_t(owner[size_t(q)])] <= i) s = q;
        if (s < 0) return false;
        if (owner[size_t(s)] >= 0) slot[size_t(owner[size_t(s)])] = -1;
        owner[size_t(s)] = e.node;
        slot[size_t(e.node)] = s;
        slots = std::max(slots, s + 1);
        in.flags |= CI_WRITE;
        in.out = uint8_t(s);
      }
      y = e.node;
    } else if (!operand(e.node, CI_A_Y, in.a)) {
      return false;
    }
    if (checksums) in.flags |= CI_CKS;
    if (reload_next) {
      in.flags |= CI_RELOAD;
      in.arg |= uint32_t(reload_next) << 8;
    }
    reload_next = 0;
    em.pos[size_t(src[size_t(i)])] = int(em.ops.size());
    em.ops.push_back(in);
  }
  if (next_leaf != int(leaves.size())) return false;
  for (auto& st : stores) {
    ColInstr in{};
    in.arg = uint32_t(st.first);
    if (st.second == y) {
      in.flags = CI_A_Y;
    } else {
      if (slot[size_t(st.second)] < 0) return false;
      in.a = uint8_t(slot[size_t(st.second)]);
    }
    em.stores.push_back(in);
  }
  em.slots = slots;
  return true;
}

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

    Emitted em;
    if (!emit_plain(nodes, live, ops, stores, checksums, em)) return fail("internal: a value has no slot");
    if (em.slots > kPlainSlots) {
      Emitted eb;
      if (!emit_batched(nodes, ops, stores, checksums, eb)) return fail("a program needs more than 16 slots, in batches too");
      em = std::move(eb);
    }
    ColSeg sg{};
    sg.s0 = uint64_t(e0) * uint64_t(sz);
    sg.s1 = uint64_t(e1) * uint64_t(sz);
    sg.loads = uint32_t(p.code.size());
    p.code.insert(p.code.end(), em.loads.begin(), em.loads.end());
    sg.ops = uint32_t(p.code.size());
    p.code.insert(p.code.end(), em.ops.begin(), em.ops.end());
    sg.stores = uint32_t(p.code.size());
    p.code.insert(p.code.end(), em.stores.begin(), em.stores.end());
    const int nload = int(em.loads.size()), K = int(em.ops.size());
    sg.nfirst = uint16_t(em.nfirst);
    if (em.nfirst < nload) p.batched = true;
    sg.nload = uint16_t(nload);
    sg.nop = uint16_t(K);
    sg.nstore = uint16_t(em.stores.size());
    if (nload > COL_LIST_MAX || K > COL_LIST_MAX || int(em.stores.size()) > COL_LIST_MAX)
      return fail("a program list longer than 64 instructions");
    p.max_leaves = std::max<uint32_t>(p.max_leaves, uint32_t(nload));
    p.max_slots = std::max<uint32_t>(p.max_slots, uint32_t(em.slots));
    p.max_ops = std::max<uint32_t>(p.max_ops, uint32_t(K));
    p.max_stores = std::max<uint32_t>(p.max_stores, uint32_t(em.stores.size()));
    p.moved_bytes += uint64_t(nload + int(em.stores.size())) * (sg.s1 - sg.s0);
    if (checksums)
      for (size_t i = 0; i < ev.size(); ++i)
        p.refs.push_back(ColRowRef{ev[i].row, uint32_t(p.segs.size()), uint32_t(em.pos[size_t(carrier[i])])});
    p.segs.push_back(sg);
  }
  for (const ColVariant& v : kVariants) {
    if ((v.accs > 0) != checksums || v.batched != p.batched) continue;
    if (int(p.max_slots) > v.leaves || (checksums && int(p.max_ops) > v.accs) || sz > v.unit ||
        int(p.max_stores) > v.stores || int(p.max_stores) < v.min_stores || int(p.max_leaves) < v.min_leaves)
      continue;
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
      c.nfirst = sg.nfirst;
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
