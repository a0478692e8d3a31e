// Row tables of every supported schedule.
//
// A row is "in step s rank src sends n elements at src_off to rank dst, which
// stores them at dst_off (copy) or reduces them into its own elements
// (recv_and_reduce)".  All rows of one step read the state before the step.
//
// Readings of points the pages leave open (they are shared with the CPU
// checker because both follow the same text; no code is shared):
//  * chunk c of N = elements [c*count/N, (c+1)*count/N) (floor partition);
//  * after ReduceScatter rank i owns chunk i;
//  * recursive halving pairs at distance N/2 first, lower rank keeps the lower half;
//  * Double Binary Tree: tree 1 = rank 0 above the tree over 1..N-1 whose node in
//    [lo, hi) is the element with most trailing zero bits; tree 2 = tree 1 + 1 mod N;
//  * Scatter / Gather keep chunks at their in-place offsets;
//  * Pairwise round k sends block (i+k) mod N of rank i to rank (i+k) mod N;
//  * Bruck = rotate, log2 rounds of shifts by 2^k, rotate back;
//  * Ring AllToAll = rotate, N-1 store-and-forward rounds to the next rank
//    (round t moves slots t..N-1), rotate back.
#include "plan.h"

#include <algorithm>
#include <functional>
#include <map>
#include <sstream>

namespace coll {
namespace {

int ceil_log2(int64_t n) {
  int k = 0;
  while ((int64_t(1) << k) < n) ++k;
  return k;
}

bool pow2(int64_t n) { return n >= 1 && (n & (n - 1)) == 0; }

// Start of part c when `count` elements are split into `parts` (floor).
int64_t part_start(int64_t count, int64_t parts, int64_t c) {
  // c*count fits: count < 2^48 and parts <= 2^16 in every accepted call.
  return (c * count) / parts;
}

int mod(int64_t a, int64_t n) { return int(((a % n) + n) % n); }

struct Emitter {
  Schedule& s;
  int cur = -1;
  explicit Emitter(Schedule& sch) : s(sch) {}
  void step(bool local = false, bool staged = false) {
    Step st;
    st.first = int64_t(s.rows.size());
    st.local = local;
    st.staged = staged;
    s.steps.push_back(st);
    cur = int(s.steps.size()) - 1;
  }
  void row(int src, int dst, int64_t src_off, int64_t dst_off, int64_t n, bool reduce,
           bool from_send = false) {
    if (n <= 0) return;
    Row r{};
    r.step = cur;
    r.src = src;
    r.dst = dst;
    r.reduce = reduce;
    r.local = s.steps[cur].local;
    r.from_send = from_send;
    r.staged = s.steps[cur].staged;
    r.src_off = src_off;
    r.dst_off = dst_off;
    r.n = n;
    s.rows.push_back(r);
    s.steps[cur].nrows++;
  }
  // chunks [a, b) of the N-way floor partition, same offsets on both sides
  void chunks(int src, int dst, int64_t a, int64_t b, bool reduce) {
    const int64_t lo = part_start(s.count, s.N, a), hi = part_start(s.count, s.N, b);
    row(src, dst, lo, lo, hi - lo, reduce);
  }
};

// ---- Ring ("集合通信算法延迟公式", Ring AllReduce; Ring AllGather / ReduceScatter)
// ReduceScatter: at step s every rank r passes chunk (r-s-1) mod N on to r+1,
// which reduces it into its own copy; after N-1 steps rank i holds chunk i.
void ring_reduce_scatter(Emitter& e) {
  const int N = e.s.N;
  for (int s = 0; s + 1 < N; ++s) {
    e.step();
    for (int r = 0; r < N; ++r) {
      const int c = mod(r - s - 1, N);
      e.chunks(r, (r + 1) % N, c, c + 1, true);
    }
  }
}

// AllGather: at step s rank r forwards chunk (r-s) mod N, the one it received
// last (its own at s = 0), to r+1.
void ring_all_gather(Emitter& e) {
  const int N = e.s.N;
  for (int s = 0; s + 1 < N; ++s) {
    e.step();
    for (int r = 0; r < N; ++r) {
      const int c = mod(r - s, N);
      e.chunks(r, (r + 1) % N, c, c + 1, false);
    }
  }
}

// ---- Recursive Halving-Doubling (eq:model-algo-rhd-rs / -ag)
// Halving: the live chunk window of every rank halves each round; partners at
// distance d = N/2, N/4, ..., 1 exchange halves and reduce the half they keep.
void rhd_reduce_scatter(Emitter& e) {
  const int N = e.s.N;
  std::vector<int64_t> lo(N, 0), hi(N, N);
  for (int d = N / 2; d >= 1; d /= 2) {
    e.step();
    for (int r = 0; r < N; ++r) {
      const int64_t mid = (lo[r] + hi[r]) / 2;
      if (r & d) lo[r] = mid; else hi[r] = mid;
      e.chunks(r ^ d, r, lo[r], hi[r], true);
    }
  }
}

// Doubling: rank r starts with chunk r; at distance d = 1, 2, ..., N/2 it
// copies in the partner's aligned window of d chunks, doubling its own.
void rhd_all_gather(Emitter& e) {
  const int N = e.s.N;
  for (int d = 1; d < N; d *= 2) {
    e.step();
    for (int r = 0; r < N; ++r) {
      const int p = r ^ d;
      const int64_t start = p & ~(d - 1);
      e.chunks(p, r, start, start + d, false);
    }
  }
}

// Halving-doubling AllReduce for N that is not a power of two (the page needs
// N = 2^n; the source it cites folds the surplus first): with P the largest
// power of two below N and r = N - P, rank 2i reduces its whole buffer into
// rank 2i+1 (i < r); ranks 2i+1 (i < r) and 2r..N-1 form a core of P ranks
// that halves and doubles over the P-way partition; rank 2i+1 then copies the
// result back to rank 2i.
void rhd_all_reduce_folded(Emitter& e) {
  const int N = e.s.N;
  int P = 1;
  while (P * 2 <= N) P *= 2;
  const int r = N - P;
  std::vector<int> core;
  for (int i = 0; i < r; ++i) core.push_back(2 * i + 1);
  for (int i = 2 * r; i < N; ++i) core.push_back(i);
  const int64_t count = e.s.count;
  auto cut = [&](int64_t c) { return part_start(count, P, c); };
  e.step();
  for (int i = 0; i < r; ++i) e.row(2 * i, 2 * i + 1, 0, 0, count, true);
  std::vector<int64_t> lo(P, 0), hi(P, P);
  for (int d = P / 2; d >= 1; d /= 2) {
    e.step();
    for (int j = 0; j < P; ++j) {
      const int64_t mid = (lo[j] + hi[j]) / 2;
      if (j & d) lo[j] = mid; else hi[j] = mid;
      e.row(core[j ^ d], core[j], cut(lo[j]), cut(lo[j]), cut(hi[j]) - cut(lo[j]), true);
    }
  }
  for (int d = 1; d < P; d *= 2) {
    e.step();
    for (int j = 0; j < P; ++j) {
      const int64_t start = (j ^ d) & ~(d - 1);
      e.row(core[j ^ d], core[j], cut(start), cut(start), cut(start + d) - cut(start), false);
    }
  }
  e.step();
  for (int i = 0; i < r; ++i) e.row(2 * i + 1, 2 * i, 0, 0, count, false);
}

// ---- Double Binary Tree (eq:model-algo-dbt-ar)
struct Tree {
  int root = 0;
  std::vector<std::vector<int>> kids;
  std::vector<int> height, depth;
};

// Node of the balanced tree over [lo, hi): the element with the most trailing
// zero bits, i.e. hi-1 with every bit below the highest bit in which lo and
// hi-1 differ cleared.
int tree_node(int lo, int hi) {
  const unsigned a = unsigned(lo), b = unsigned(hi - 1);
  if (a == b) return lo;
  const unsigned top = 31u - unsigned(__builtin_clz(a ^ b));
  return int(b & ~((1u << top) - 1u));
}

int build_tree(Tree& t, int lo, int hi) {
  if (lo >= hi) return -1;
  const int m = tree_node(lo, hi);
  const int l = build_tree(t, lo, m), r = build_tree(t, m + 1, hi);
  if (l >= 0) t.kids[m].push_back(l);
  if (r >= 0) t.kids[m].push_back(r);
  return m;
}

void tree_levels(Tree& t) {
  const int N = int(t.kids.size());
  t.height.assign(N, 0);
  t.depth.assign(N, 0);
  std::function<int(int, int)> walk = [&](int u, int dep) {
    t.depth[u] = dep;
    int h = 0;
    for (int c : t.kids[u]) h = std::max(h, 1 + walk(c, dep + 1));
    t.height[u] = h;
    return h;
  };
  walk(t.root, 0);
}

void dbt_trees(int N, Tree& t1, Tree& t2) {
  t1.kids.assign(N, {});
  t1.root = 0;
  const int top = build_tree(t1, 1, N);
  if (top >= 0) t1.kids[0].push_back(top);
  t2.kids.assign(N, {});
  t2.root = 1 % N;
  for (int u = 0; u < N; ++u)
    for (int c : t1.kids[u]) t2.kids[(u + 1) % N].push_back((c + 1) % N);
  tree_levels(t1);
  tree_levels(t2);
}

// Reduce up both trees level by level (by height; left child before right,
// tree 1 before tree 2), then broadcast down (by depth).  Tree 1 carries
// elements [0, count/2), tree 2 the rest.
void dbt_all_reduce(Emitter& e) {
  const int N = e.s.N;
  if (N < 2) return;
  Tree t[2];
  dbt_trees(N, t[0], t[1]);
  const int H = ceil_log2(N);
  const int64_t half[3] = {0, e.s.count / 2, e.s.count};
  for (int h = 1; h <= H; ++h) {
    e.step();
    for (int k = 0; k < 2; ++k)
      for (int p = 0; p < N; ++p)
        for (int c : t[k].kids[p])
          if (t[k].height[c] == h - 1) e.row(c, p, half[k], half[k], half[k + 1] - half[k], true);
  }
  for (int j = 1; j <= H; ++j) {
    e.step();
    for (int k = 0; k < 2; ++k)
      for (int p = 0; p < N; ++p)
        if (t[k].depth[p] == j - 1)
          for (int c : t[k].kids[p]) e.row(p, c, half[k], half[k], half[k + 1] - half[k], false);
  }
}

// ---- One-to-many ("一对多通信：Broadcast 与 Scatter")
// Sub-step j (1-based) of the binomial tree, relative ranks: every v that is a
// multiple of 2d, d = 2^(L-j), hands on to v+d when v+d < N.
template <class F>
void binomial_substep(int N, int j, F&& f) {
  const int L = ceil_log2(N);
  const int d = 1 << (L - j);
  for (int v = 0; v + d < N; v += 2 * d) f(v, v + d, d);
}

int abs_rank(int root, int v, int N) { return (root + v) % N; }

// eq:binomial-bcast: ceil(log2 N) steps of the whole message.
void bcast_binomial(Emitter& e) {
  const int N = e.s.N, L = ceil_log2(N), root = e.s.root;
  for (int j = 1; j <= L; ++j) {
    e.step();
    binomial_substep(N, j, [&](int v, int w, int) {
      e.row(abs_rank(root, v, N), abs_rank(root, w, N), 0, 0, e.s.count, false);
    });
  }
}

// eq:pipe-chain-bcast: chunk c crosses hop h (relative rank h -> h+1) at step c+h.
void bcast_chain_pipe(Emitter& e) {
  const int N = e.s.N, k = e.s.chunks, root = e.s.root;
  if (N < 2) return;
  for (int t = 0; t < N + k - 2; ++t) {
    e.step();
    for (int c = std::max(0, t - (N - 2)); c <= std::min(t, k - 1); ++c) {
      const int h = t - c;
      const int64_t lo = part_start(e.s.count, k, c), hi = part_start(e.s.count, k, c + 1);
      e.row(abs_rank(root, h, N), abs_rank(root, h + 1, N), lo, lo, hi - lo, false);
    }
  }
}

// eq:pipe-tree-bcast: chunk c takes binomial sub-step j+1 at step c+j.
void bcast_binomial_pipe(Emitter& e) {
  const int N = e.s.N, k = e.s.chunks, root = e.s.root, L = ceil_log2(N);
  if (L == 0) return;
  for (int t = 0; t < L + k - 1; ++t) {
    e.step();
    for (int c = std::max(0, t - (L - 1)); c <= std::min(t, k - 1); ++c) {
      const int64_t lo = part_start(e.s.count, k, c), hi = part_start(e.s.count, k, c + 1);
      binomial_substep(N, t - c + 1, [&](int v, int w, int) {
        e.row(abs_rank(root, v, N), abs_rank(root, w, N), lo, lo, hi - lo, false);
      });
    }
  }
}

// "一对多通信：Broadcast 与 Scatter", SCCL 的 Broadcast 实现: the root feeds both
// directions of a bidirectional ring at once.  The clockwise chain reaches
// relative ranks 1..floor(N/2), the counter-clockwise one N-1 down to
// floor(N/2)+1; chunk c crosses hop h of either chain at step c+h.
void bcast_bidir_ring(Emitter& e) {
  const int N = e.s.N, k = e.s.chunks, root = e.s.root;
  if (N < 2) return;
  const int cw = N / 2, ccw = (N - 1) / 2;
  for (int t = 0; t < cw + k - 1; ++t) {
    e.step();
    for (int c = std::max(0, t - (cw - 1)); c <= std::min(t, k - 1); ++c) {
      const int h = t - c;
      const int64_t lo = part_start(e.s.count, k, c), hi = part_start(e.s.count, k, c + 1);
      e.row(abs_rank(root, h, N), abs_rank(root, h + 1, N), lo, lo, hi - lo, false);
      if (h < ccw) e.row(abs_rank(root, N - h, N), abs_rank(root, N - h - 1, N), lo, lo, hi - lo, false);
    }
  }
}

// Relative chunks [a, b) between relative ranks, split where the absolute
// chunk index wraps past N-1.
void relative_chunks(Emitter& e, int v_src, int v_dst, int a, int b) {
  const int N = e.s.N, root = e.s.root;
  const int first = (root + a) % N;
  const int n = b - a;
  const int head = std::min(n, N - first);
  e.chunks(abs_rank(root, v_src, N), abs_rank(root, v_dst, N), first, first + head, false);
  if (n > head) e.chunks(abs_rank(root, v_src, N), abs_rank(root, v_dst, N), 0, n - head, false);
}

// eq:binomial-scatter: at sub-step j the holder v gives v+d the chunks of the
// subtree rooted at v+d, relative chunks [v+d, v+2d).
void scatter_binomial(Emitter& e) {
  const int N = e.s.N, L = ceil_log2(N);
  for (int j = 1; j <= L; ++j) {
    e.step();
    binomial_substep(N, j, [&](int v, int w, int d) { relative_chunks(e, v, w, w, std::min(w + d, N)); });
  }
}

// eq:onetoall-gather-scatter-duality: Scatter's steps in reverse order with
// every edge reversed.
void gather_binomial(Emitter& e) {
  const int N = e.s.N, L = ceil_log2(N);
  for (int j = L; j >= 1; --j) {
    e.step();
    binomial_substep(N, j, [&](int v, int w, int d) { relative_chunks(e, w, v, w, std::min(w + d, N)); });
  }
}

// eq:onetoall-scatter-naive: the root sends rank root+i its chunk at step i.
void scatter_linear(Emitter& e) {
  const int N = e.s.N, root = e.s.root;
  for (int i = 1; i < N; ++i) {
    e.step();
    const int a = abs_rank(root, i, N);
    e.chunks(root, a, a, a + 1, false);
  }
}

// Tree Reduce ("集合通信算法延迟公式", eq:model-algo-reduce-tree): the tree
// Broadcast run backwards; at step j every relative rank v with lowest set bit
// 2^(j-1) reduces its partial result into v - 2^(j-1).
void reduce_binomial(Emitter& e) {
  const int N = e.s.N, L = ceil_log2(N), root = e.s.root;
  for (int j = L; j >= 1; --j) {
    e.step();
    binomial_substep(N, j, [&](int v, int w, int) {
      e.row(abs_rank(root, w, N), abs_rank(root, v, N), 0, 0, e.s.count, true);
    });
  }
}

// ---- AllToAll (eq:model-algo-a2a-pairwise / -bruck)
void a2a_pairwise(Emitter& e) {
  const int N = e.s.N;
  const int64_t B = e.s.count / N;
  e.step(true);
  for (int i = 0; i < N; ++i) e.row(i, i, i * B, i * B, B, false, true);
  for (int k = 1; k < N; ++k) {
    e.step();
    for (int i = 0; i < N; ++i) {
      const int j = (i + k) % N;
      e.row(i, j, j * B, i * B, B, false, true);
    }
  }
}

// Bruck's local phases, also the storage of the Ring AllToAll: rotate in,
// tmp_i[j] = send_i[(i+j) mod N] (slot j holds the block for rank i+j), and
// rotate out, recv_i[(i-j) mod N] = tmp_i[j].  tmp is the receive buffer.
void a2a_rotate_in(Emitter& e, int64_t B) {
  const int N = e.s.N;
  e.step(true);
  for (int i = 0; i < N; ++i)
    for (int j = 0; j < N; ++j) e.row(i, i, int64_t((i + j) % N) * B, j * B, B, false, true);
}

void a2a_rotate_out(Emitter& e, int64_t B) {
  const int N = e.s.N;
  e.step(true, true);
  for (int i = 0; i < N; ++i)
    for (int j = 0; j < N; ++j) e.row(i, i, j * B, int64_t(mod(i - j, N)) * B, B, false);
}

// eq:model-algo-a2a-bruck: round k shifts every block index with bit k set by
// 2^k ranks, all such blocks packed into one message.
void a2a_bruck(Emitter& e) {
  const int N = e.s.N;
  const int64_t B = e.s.count / N;
  a2a_rotate_in(e, B);
  for (int k = 0; (1 << k) < N; ++k) {
    e.step(false, true);
    for (int j = 0; j < N; ++j)
      if ((j >> k) & 1)
        for (int i = 0; i < N; ++i) e.row(i, (i + (1 << k)) % N, j * B, j * B, B, false);
  }
  a2a_rotate_out(e, B);
}

// eq:model-algo-a2a-ring: N-1 rounds between ring neighbours only, read as
// store-and-forward.  In the rotated storage a block in slot j still has j
// hops to go before round 1; round t moves slots t..N-1 one rank on, so the
// block in slot t arrives and stays.  Each slot's move is a cyclic shift over
// all N ranks (a closed group), as in Bruck's rounds.
void a2a_ring(Emitter& e) {
  const int N = e.s.N;
  const int64_t B = e.s.count / N;
  a2a_rotate_in(e, B);
  for (int t = 1; t < N; ++t) {
    e.step(false, true);
    for (int j = t; j < N; ++j)
      for (int i = 0; i < N; ++i) e.row(i, (i + 1) % N, j * B, j * B, B, false);
  }
  a2a_rotate_out(e, B);
}

bool algo_valid(coll_kind_t kind, coll_algo_t a) {
  switch (kind) {
    case COLL_K_ALLREDUCE: return a == COLL_ALGO_RING || a == COLL_ALGO_RHD || a == COLL_ALGO_DBT;
    case COLL_K_REDUCESCATTER:
    case COLL_K_ALLGATHER: return a == COLL_ALGO_RING || a == COLL_ALGO_RHD;
    case COLL_K_BROADCAST:
      return a == COLL_ALGO_BINOMIAL || a == COLL_ALGO_CHAIN_PIPE || a == COLL_ALGO_BINOMIAL_PIPE ||
             a == COLL_ALGO_SCATTER_ALLGATHER || a == COLL_ALGO_BIDIR_RING;
    case COLL_K_SCATTER: return a == COLL_ALGO_BINOMIAL || a == COLL_ALGO_LINEAR;
    case COLL_K_GATHER:
    case COLL_K_REDUCE: return a == COLL_ALGO_BINOMIAL;
    case COLL_K_ALLTOALL: return a == COLL_ALGO_PAIRWISE || a == COLL_ALGO_BRUCK || a == COLL_ALGO_RING;
  }
  return false;
}

}  // namespace

int64_t Schedule::counted_steps() const {
  int64_t n = 0;
  for (const Step& s : steps) n += s.local ? 0 : 1;
  return n;
}

coll_algo_t resolve_algo(coll_kind_t kind, coll_algo_t algo) {
  if (algo != COLL_ALGO_DEFAULT) return algo;
  switch (kind) {
    case COLL_K_ALLREDUCE:
    case COLL_K_REDUCESCATTER:
    case COLL_K_ALLGATHER: return COLL_ALGO_RING;
    case COLL_K_BROADCAST:
    case COLL_K_SCATTER:
    case COLL_K_GATHER:
    case COLL_K_REDUCE: return COLL_ALGO_BINOMIAL;
    case COLL_K_ALLTOALL: return COLL_ALGO_PAIRWISE;
  }
  return algo;
}

coll_status_t validate_schedule_args(coll_kind_t kind, coll_algo_t algo_in, int N, int64_t count, int root,
                                     int chunks, std::string& err) {
  if (int(kind) < 0 || int(kind) > int(COLL_K_REDUCE)) {
    err = "unknown collective";
    return COLL_ERR_INVALID_ARG;
  }
  if (N < 1) {
    err = "nranks must be at least 1";
    return COLL_ERR_INVALID_ARG;
  }
  if (N > COLL_MAX_RANKS) {
    err = "nranks above COLL_MAX_RANKS";
    return COLL_ERR_UNSUPPORTED;
  }
  if (count < 0 || count >= (int64_t(1) << 47)) {
    err = "count out of range";
    return COLL_ERR_INVALID_ARG;
  }
  const coll_algo_t algo = resolve_algo(kind, algo_in);
  if (algo == COLL_ALGO_AUTO) {
    err = "COLL_ALGO_AUTO is resolved before a schedule is built";
    return COLL_ERR_INVALID_ARG;
  }
  if (int(algo) < 1 || int(algo) > int(COLL_ALGO_BIDIR_RING) || !algo_valid(kind, algo)) {
    err = "algorithm not defined for this collective";
    return COLL_ERR_UNSUPPORTED;
  }
  if (algo == COLL_ALGO_RHD && kind != COLL_K_ALLREDUCE && !pow2(N)) {
    err = "recursive halving-doubling ReduceScatter / AllGather need a power-of-two N";
    return COLL_ERR_UNSUPPORTED;
  }
  const bool rooted =
      kind == COLL_K_BROADCAST || kind == COLL_K_SCATTER || kind == COLL_K_GATHER || kind == COLL_K_REDUCE;
  if (rooted && (root < 0 || root >= N)) {
    err = "root outside [0, nranks)";
    return COLL_ERR_INVALID_ARG;
  }
  const bool pipe = algo_pipelined(algo);
  if (pipe && count > 0 && (chunks < 1 || int64_t(chunks) > count)) {
    err = "chunks must be in [1, count]";
    return COLL_ERR_INVALID_ARG;
  }
  if (pipe && chunks > 65536) {
    err = "chunks above 65536";
    return COLL_ERR_UNSUPPORTED;
  }
  if (kind == COLL_K_ALLTOALL && count % N) {
    err = "alltoall needs count divisible by nranks";
    return COLL_ERR_INVALID_ARG;
  }
  return COLL_OK;
}

coll_status_t build_schedule(coll_kind_t kind, coll_algo_t algo_in, int N, int64_t count, int root,
                             int chunks, Schedule& out, std::string& err) {
  const coll_status_t st = validate_schedule_args(kind, algo_in, N, count, root, chunks, err);
  if (st != COLL_OK) return st;
  const coll_algo_t algo = resolve_algo(kind, algo_in);
  const bool rooted =
      kind == COLL_K_BROADCAST || kind == COLL_K_SCATTER || kind == COLL_K_GATHER || kind == COLL_K_REDUCE;
  const bool pipe = algo_pipelined(algo);
  out = Schedule{};
  out.kind = kind;
  out.algo = algo;
  out.N = N;
  out.count = count;
  out.root = rooted ? root : 0;
  out.chunks = pipe ? std::max(1, chunks) : 1;
  if (pipe && count == 0) out.chunks = 1;
  Emitter e(out);
  switch (kind) {
    case COLL_K_ALLREDUCE:
      if (algo == COLL_ALGO_RING) { ring_reduce_scatter(e); ring_all_gather(e); }
      else if (algo == COLL_ALGO_RHD) {
        if (pow2(N)) { rhd_reduce_scatter(e); rhd_all_gather(e); }
        else rhd_all_reduce_folded(e);
      }
      else dbt_all_reduce(e);
      break;
    case COLL_K_REDUCESCATTER:
      if (algo == COLL_ALGO_RING) ring_reduce_scatter(e); else rhd_reduce_scatter(e);
      break;
    case COLL_K_ALLGATHER:
      if (algo == COLL_ALGO_RING) ring_all_gather(e); else rhd_all_gather(e);
      break;
    case COLL_K_BROADCAST:
      if (algo == COLL_ALGO_BINOMIAL) bcast_binomial(e);
      else if (algo == COLL_ALGO_CHAIN_PIPE) bcast_chain_pipe(e);
      else if (algo == COLL_ALGO_BINOMIAL_PIPE) bcast_binomial_pipe(e);
      else if (algo == COLL_ALGO_BIDIR_RING) bcast_bidir_ring(e);
      else {
        // "一对多通信：Broadcast 与 Scatter", Broadcast 与 Scatter 的关系: chunks stay
        // at their offsets, so after the Scatter rank i holds chunk i, which
        // is what the Ring AllGather starts from
        scatter_binomial(e);
        ring_all_gather(e);
      }
      break;
    case COLL_K_SCATTER:
      if (algo == COLL_ALGO_BINOMIAL) scatter_binomial(e); else scatter_linear(e);
      break;
    case COLL_K_GATHER: gather_binomial(e); break;
    case COLL_K_REDUCE: reduce_binomial(e); break;
    case COLL_K_ALLTOALL:
      if (algo == COLL_ALGO_PAIRWISE) a2a_pairwise(e);
      else if (algo == COLL_ALGO_BRUCK) a2a_bruck(e);
      else a2a_ring(e);
      break;
  }
  return COLL_OK;
}

coll_status_t choose_algo(coll_kind_t kind, int N, int64_t count, int elem_size, int root, const CostModel& m,
                          coll_algo_t& out, std::string& err, const std::function<PlannedCost(const Schedule&)>* cost) {
  std::vector<coll_algo_t> cand;
  switch (kind) {
    case COLL_K_ALLREDUCE: cand = {COLL_ALGO_DBT, COLL_ALGO_RHD, COLL_ALGO_RING}; break;
    case COLL_K_REDUCESCATTER:
    case COLL_K_ALLGATHER:
      if (pow2(N)) cand.push_back(COLL_ALGO_RHD);
      cand.push_back(COLL_ALGO_RING);
      break;
    case COLL_K_BROADCAST:
      cand = {COLL_ALGO_BINOMIAL, COLL_ALGO_CHAIN_PIPE, COLL_ALGO_SCATTER_ALLGATHER, COLL_ALGO_BIDIR_RING};
      break;
    case COLL_K_SCATTER: cand = {COLL_ALGO_BINOMIAL, COLL_ALGO_LINEAR}; break;
    case COLL_K_GATHER:
    case COLL_K_REDUCE: cand = {COLL_ALGO_BINOMIAL}; break;
    case COLL_K_ALLTOALL: cand = {COLL_ALGO_PAIRWISE, COLL_ALGO_BRUCK, COLL_ALGO_RING}; break;
    default:
      err = "unknown collective";
      return COLL_ERR_INVALID_ARG;
  }
  double best = 0;
  bool have = false;
  for (coll_algo_t a : cand) {
    Schedule s;
    std::string e2;
    const coll_status_t st = build_schedule(kind, a, N, count, root, 1, s, e2);
    if (st != COLL_OK) {
      err = e2;
      if (!have && a == cand.back()) return st;
      continue;
    }
    PlannedCost pc;
    if (cost) {
      pc = (*cost)(s);
    } else {
      const coll_counts_t c = count_schedule(s, elem_size);
      pc.round_trips = c.steps;
      pc.bytes = c.hbm_bytes;
    }
    const double t = double(pc.round_trips) * m.alpha_s + double(pc.bytes) / m.beta_Bps;
    if (!have || t < best) {
      best = t;
      out = a;
      have = true;
    }
  }
  return have ? COLL_OK : COLL_ERR_UNSUPPORTED;
}

coll_counts_t count_schedule(const Schedule& s, int elem_size) {
  coll_counts_t c{};
  c.steps = s.counted_steps();
  c.round_trips = c.steps;
  c.rows = int64_t(s.rows.size());
  for (const Step& st : s.steps) {
    std::map<std::pair<int, int>, int64_t> edge;
    for (int64_t i = st.first; i < st.first + st.nrows; ++i) {
      const Row& r = s.rows[size_t(i)];
      edge[{r.src, r.dst}] += r.n;
      c.hbm_bytes += (r.reduce ? 3 : 2) * r.n * elem_size;
      c.moved_bytes += (r.reduce ? 3 : 2) * r.n * elem_size;
    }
    if (!st.local) {
      int64_t m = 0;
      for (auto& kv : edge) m = std::max(m, kv.second);
      c.crit_bytes += m * elem_size;
    }
  }
  return c;
}

std::string check_schedule(const Schedule& s) {
  // Per step and rank: written intervals must not overlap unless both rows
  // reduce (they accumulate in row order), and no row may read what another
  // row of the same step writes.  Staged steps only need disjoint writes.
  struct Iv { int64_t lo, hi, row; bool reduce; };
  for (size_t si = 0; si < s.steps.size(); ++si) {
    const Step& st = s.steps[si];
    std::map<int, std::vector<Iv>> writes, reads;
    for (int64_t i = st.first; i < st.first + st.nrows; ++i) {
      const Row& r = s.rows[size_t(i)];
      writes[r.dst].push_back({r.dst_off, r.dst_off + r.n, i, bool(r.reduce)});
      if (!r.from_send) reads[r.src].push_back({r.src_off, r.src_off + r.n, i, false});
    }
    for (auto& kv : writes) {
      auto& w = kv.second;
      std::sort(w.begin(), w.end(), [](const Iv& a, const Iv& b) { return a.lo < b.lo; });
      for (size_t a = 0; a < w.size(); ++a)
        for (size_t b = a + 1; b < w.size() && w[b].lo < w[a].hi; ++b)
          if (st.staged || !(w[a].reduce && w[b].reduce)) {
            std::ostringstream os;
            os << "step " << si << ": rows " << w[a].row << " and " << w[b].row << " both write rank "
               << kv.first;
            return os.str();
          }
    }
    if (st.staged) continue;
    for (auto& kv : reads) {
      auto it = writes.find(kv.first);
      if (it == writes.end()) continue;
      for (const Iv& rd : kv.second)
        for (const Iv& wr : it->second)
          if (wr.row != rd.row && wr.lo < rd.hi && rd.lo < wr.hi) {
            std::ostringstream os;
            os << "step " << si << ": row " << rd.row << " reads rank " << kv.first << " where row "
               << wr.row << " writes";
            return os.str();
          }
    }
  }
  return "";
}

}  // namespace coll
