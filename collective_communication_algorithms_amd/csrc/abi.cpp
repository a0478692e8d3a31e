// The C ABI: argument checks, the schedule cache, launches.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "bind.h"
#include "coll.h"
#include "colprog.h"
#include "launch.h"
#include "plan.h"

namespace coll {
namespace {

thread_local std::string t_err;
thread_local coll_counts_t t_last{};
thread_local uint64_t* t_sums = nullptr;
// COLL_OPT_TIMING: the last timed call's events on this thread (one pair per device)
struct TimingEvents {
  int dev = -1;
  hipEvent_t start = nullptr, stop = nullptr;
  bool recorded = false;
};
thread_local std::vector<TimingEvents> t_timing;
thread_local TimingEvents* t_last_timed = nullptr;
thread_local size_t t_sums_cap = 0;

std::atomic<int64_t> opt_exec{0};      // 0: column kernel where it applies, else one row-kernel launch per
                                       // phase; 1: one row-kernel launch per step; 2: one per phase
std::atomic<int64_t> opt_col_tiles{0}; // column kernel: tiles per work group (0: automatic)
std::atomic<int64_t> opt_timing{0};    // 1: HIP events around each call's main kernels
std::atomic<int64_t> opt_group{0};     // 0: automatic
std::atomic<int64_t> opt_grid{0};      // 0: automatic
std::atomic<int64_t> opt_nt{-1};       // -1: automatic, else an NT_* mask
std::atomic<int64_t> opt_reverse{1};
std::atomic<int64_t> opt_alpha_ns{1060};   // COLL_ALGO_AUTO: fitted per-step cost on MI355X
std::atomic<int64_t> opt_beta_gbps{8200};  // COLL_ALGO_AUTO: fitted schedule-byte rate on MI355X
std::atomic<int64_t> opt_cache_bytes{int64_t(1) << 31};  // device memory the schedule cache may hold
std::atomic<int64_t> opt_a2a_direct{1};  // 1: an AllToAll of whole-block rows as one direct copy of its blocks
std::atomic<bool> g_debug{false};      // COLL_DEBUG: one line per call on stderr

const char* kind_name(coll_kind_t k) {
  static const char* n[] = {"allreduce", "reducescatter", "allgather", "broadcast", "scatter", "gather",
                            "alltoall", "reduce"};
  return int(k) >= 0 && int(k) < 8 ? n[int(k)] : "?";
}

const char* algo_name(coll_algo_t a) {
  static const char* n[] = {"default", "ring", "rhd", "dbt", "binomial", "chain_pipe", "binomial_pipe",
                            "pairwise", "bruck", "linear", "scatter_allgather", "auto", "bidir_ring"};
  return int(a) >= 0 && int(a) < 13 ? n[int(a)] : "?";
}

// Working sets up to the 256 MiB memory-side cache of MI355X stay there between
// steps when accessed normally; larger ones stream, and then nontemporal source
// loads (whose data is consumed once per step) keep the cache for the stores
// the next step reads back.  Measured on the Ring / Halving-Doubling / tree
// AllReduce, Broadcast and ReduceScatter / AllGather sweeps.  AllToAll never
// reads back what it writes, so there the stores are nontemporal too (32 x
// 128 MiB bf16 Pairwise 1.67 -> 1.61 ms; the Bruck rounds are unchanged).
constexpr uint64_t CACHE_RESIDENT_BYTES = uint64_t(256) << 20;

uint32_t auto_nt(uint64_t footprint, bool alltoall) {
  if (footprint <= CACHE_RESIDENT_BYTES) return 0u;
  return alltoall ? (NT_SRC | NT_DST) : NT_SRC;
}


coll_status_t fail(coll_status_t st, const std::string& msg) {
  t_err = msg;
  return st;
}

coll_status_t hip_fail(hipError_t e, const char* what) {
  t_err = std::string(what) + ": " + hipGetErrorString(e);
  return COLL_ERR_HIP;
}

int elem_size(coll_dtype_t d) {
  switch (d) {
    case COLL_INT32: return 4;
    case COLL_UINT8: return 1;
    case COLL_FLOAT32: return 4;
    case COLL_BFLOAT16: return 2;
  }
  return 0;
}

struct Key {
  int dev, kind, algo, N;
  int64_t count;
  int sz, root, chunks, inplace;
  bool operator==(const Key& o) const {
    return dev == o.dev && kind == o.kind && algo == o.algo && N == o.N && count == o.count && sz == o.sz &&
           root == o.root && chunks == o.chunks && inplace == o.inplace;
  }
};

struct KeyHash {
  size_t operator()(const Key& k) const {
    uint64_t h = 1469598103934665603ull;
    auto mix = [&](uint64_t v) { h = (h ^ v) * 1099511628211ull; };
    mix(uint64_t(k.dev));
    mix(uint64_t(k.kind));
    mix(uint64_t(k.algo));
    mix(uint64_t(k.N));
    mix(uint64_t(k.count));
    mix(uint64_t(k.sz));
    mix(uint64_t(k.root));
    mix(uint64_t(k.chunks));
    mix(uint64_t(k.inplace));
    return size_t(h);
  }
};

struct DevList {                // work lists of one row phase for one launch shape
  bool pinned = false;          // used by a captured call: kept until coll_finalize
  size_t phase = 0;
  uint64_t cap = 0;             // grid cap asked for
  uint32_t G = 0, gt = 0;       // grid used, group tiles
  bool reverse = false, per_step = false, group_major = false;
  uint32_t launches = 0;
  bool fine = false;            // small pieces: launch the row kernel's fine variant
  bool fwd = false;             // launch the forwarding variant (most entries take an operand from registers)
  uint64_t fwd_saved = 0;       // bytes that variant neither loads nor stores
  uint32_t* d_off = nullptr;
  DevItem* d_list = nullptr;
  uint64_t bytes = 0;           // device memory held
};

// A schedule's column programs on the device (one per checksum mode).
struct ColDev {
  bool tried = false;
  bool pinned = false;          // used by a captured call: tables kept until coll_finalize
  ColPlan plan;                 // plan.ok false: the row kernel runs this schedule
  uint32_t tiles = 0;           // tiles per work group of d_work
  uint32_t nwork = 0;
  uint64_t partials = 0;        // checksums: partial-sum slots the work groups write
  ColWork* d_work = nullptr;
  ColInstr* d_code = nullptr;
  uint32_t* d_row_off = nullptr;  // checksums: ColRefs of each row
  ColRef* d_refs = nullptr;
  uint64_t code_bytes = 0, table_bytes = 0;  // device memory held
};

// The direct copy of an AllToAll's leading independent rows
// (copy_rows_kernel): its row table and, for checksums, the fold's
// references (one per row: its work groups' slots).
struct CopyDev {
  bool tried = false, ok = false;
  bool whole = false;           // the whole schedule; else the rows of phase 0
  bool pinned = false;          // used by a captured call: tables kept until coll_finalize
  uint32_t nrows = 0, wgs_per_row = 0;  // copy rows
  uint32_t nfold = 0;           // schedule rows whose checksums the copy's slots make
  uint32_t* d_idx = nullptr;    // a whole AllToAll's rows: the copy row (block) each carries; refs are per block
  uint64_t row_bytes = 0;
  CopyRow* d_rows = nullptr;
  uint32_t* d_row_off = nullptr;
  ColRef* d_refs = nullptr;
  uint64_t bytes = 0;           // device memory held
};

struct Entry {
  Schedule sched;
  Bound bound;
  ColDev col[2];                // [checksums on]
  CopyDev copy[2];              // [COLL_OPT_A2A_DIRECT]
  bool pinned = false;          // used by a captured call: never evicted before coll_finalize
  std::vector<int8_t> multi;    // per phase: groups average two or more pieces per step (-1: not known yet)
  int dev = 0;
  DevItem* d_items = nullptr;
  DevStep* d_steps = nullptr;
  std::vector<DevList> lists;
  uint64_t last_use = 0;
  uint64_t bytes = 0;           // device memory held by the tables and lists
};

struct DevInfo {
  int cus = 0;
};

std::mutex g_mu;
std::unordered_map<Key, std::unique_ptr<Entry>, KeyHash> g_cache;
std::unordered_map<int, DevInfo> g_dev;
std::unordered_map<uint64_t, int> g_occ;  // (kernel variant, device) -> blocks per CU
uint64_t g_tick = 0;

// Partial row-checksum slots (SUM_LANES per row), one buffer per (device,
// caller's checksum buffer): calls that share a checksum buffer are ordered by
// the caller anyway, and calls with different buffers never share slots.
struct SumScratch {
  int dev = 0;
  const uint64_t* user = nullptr;
  uint64_t* d = nullptr;
  size_t cap = 0;               // slots
  uint64_t last_use = 0;
  bool clean = false;           // every slot is zero once the queued work is done (the fold
                                // kernel zeroes what it reads); else the next call clears them
  bool pinned = false;          // used by a captured call: neither freed nor moved before coll_finalize
};
std::vector<SumScratch> g_sum_scratch;
// Device buffers a captured graph may still use, released by coll_finalize:
// pinned tables that a later call had to replace.
std::vector<void*> g_retired;
constexpr size_t SUM_SCRATCH_MAX = 16;  // buffers kept; the least recently used goes first
constexpr size_t CACHE_CAP = 512;  // schedules kept
uint64_t g_cache_bytes = 0;        // device memory they hold (COLL_OPT_CACHE_BYTES caps it)
std::map<std::vector<int64_t>, coll_algo_t> g_auto;  // COLL_ALGO_AUTO decisions

CostModel cost_model() {
  CostModel m;
  m.alpha_s = double(opt_alpha_ns.load()) * 1e-9;
  m.beta_Bps = double(opt_beta_gbps.load()) * 1e9;
  return m;
}

// Compute units assumed when planning without a device (coll_plan): MI355X's.
constexpr uint32_t PLAN_CUS = 256;

// Whether a row phase's launches run the forwarding variant with its marks
// honoured: the variant exists for the nontemporal masks of ordinary
// footprints (none, source loads; without either, a list of small pieces takes
// the fine variant instead), and it honours its marks only when every rank
// buffer is 16-byte aligned.
bool forwarding_runs(bool fwd, bool fine, uint32_t ntmask, bool bases16) {
  return fwd && bases16 && (ntmask == NT_SRC || ntmask == (NT_SRC | NT_DST) || (ntmask == 0 && !fine));
}

// The nontemporal mask of a row phase's launches: the call's, except that
// under the automatic policy a forwarding list of a reducing schedule whose
// footprint is past the memory-side cache (source loads nontemporal) also
// stores nontemporally.  Its stores are the results, which nothing in the
// call reads back (the forwarded operands never left the registers).
// Measured for Ring AllReduce 8 ranks fp32 / bf16: 48 MiB 184 -> 156 / 185 ->
// 151 us, 64 MiB 247 -> 203 / 249 -> 190 us, 128 MiB 452 -> 430 / 453 -> 426
// us, 256 MiB 0.860 -> 0.833 / 0.864 -> 0.837 ms; AllGather (copies) lost 2 %,
// so copy-only schedules keep their mask.
uint32_t rows_ntmask(uint32_t ntmask, bool fwd, bool has_reduce) {
  if (opt_nt.load() < 0 && fwd && has_reduce && ntmask == NT_SRC) return NT_SRC | NT_DST;
  return ntmask;
}

// Whether the column kernel may run calls (the automatic execution mode).
bool col_mode() { return opt_exec.load() == 0; }

// What a call costs, as planned for an in-place call on 16-byte-aligned
// buffers with the current options on a device of `cus` compute units.  Where
// the column kernel runs the schedule: one memory round trip, and the bytes
// its programs load and store.  Elsewhere: a round trip per step, and the
// schedule's bytes less, in every row phase whose lists the forwarding variant
// runs, the operands it takes from registers and the stores it skips (only
// large column spaces get group-major lists, so only they build lists here).
// The rows of an AllToAll's steps before its first staged step, when every
// one of them reads the send buffers and writes the receive buffers, all of
// one length, a multiple of 16 bytes, and the direct copy's grid fits: they
// are then independent and run in one launch of copy_rows_kernel.  That is
// every row of the Pairwise schedule, and the first rotation of Bruck's and
// of the Ring AllToAll (the rounds after it run in the permutation kernel).
// 0: none.
size_t copy_prefix_rows(const Schedule& s, int sz) {
  if (s.kind != COLL_K_ALLTOALL || s.rows.empty()) return 0;
  size_t nrows = 0;
  for (const Step& st : s.steps) {
    if (st.staged) break;
    nrows = size_t(st.first + st.nrows);
  }
  if (nrows == 0) return 0;
  const int64_t n = s.rows[0].n;
  for (size_t i = 0; i < nrows; ++i) {
    const Row& r = s.rows[i];
    if (!r.from_send || r.reduce || r.n != n) return 0;
  }
  const uint64_t row_bytes = uint64_t(n) * uint64_t(sz);
  if (row_bytes == 0 || row_bytes % 16u) return 0;
  return (row_bytes + 1023u) / 1024u * nrows <= 0x7fffffffu ? nrows : 0;
}

// The send block each row of an AllToAll carries (block j of rank i: i * N +
// j), when every row moves one whole block of count / N elements: the
// schedule run on block identities with the pages' step model (every source
// of a step is read before any row of it writes).  Empty when a row moves
// anything else, reads a block no row has written, two rows of a step write
// one block, or the receive buffers end other than the AllToAll defines
// (block i of recv_j = block j of send_i).  Since the rows only move
// blocks, a row's destination after it holds exactly the block it carries.
std::vector<uint32_t> alltoall_carried(const Schedule& s) {
  if (s.kind != COLL_K_ALLTOALL || s.rows.empty() || s.N < 1) return {};
  const int64_t N = s.N, B = s.count / N;
  if (B <= 0 || N * N >= int64_t(0xffffffff)) return {};
  constexpr uint32_t NONE = 0xffffffffu;
  std::vector<uint32_t> recv(size_t(N * N), NONE), carried(s.rows.size(), NONE);
  std::vector<uint8_t> hit(size_t(N * N), 0);
  for (const Step& st : s.steps) {
    const size_t r0 = size_t(st.first), r1 = size_t(st.first + st.nrows);
    for (size_t i = r0; i < r1; ++i) {
      const Row& r = s.rows[i];
      if (r.reduce || r.n != B || r.src < 0 || r.src >= N || r.dst < 0 || r.dst >= N || r.src_off < 0 ||
          r.dst_off < 0 || r.src_off % B || r.dst_off % B || r.src_off / B >= N || r.dst_off / B >= N)
        return {};
      const size_t from = size_t(int64_t(r.src) * N + r.src_off / B);
      const uint32_t id = r.from_send ? uint32_t(from) : recv[from];
      if (id == NONE) return {};
      carried[i] = id;
    }
    for (size_t i = r0; i < r1; ++i) {
      const Row& r = s.rows[i];
      const size_t to = size_t(int64_t(r.dst) * N + r.dst_off / B);
      if (hit[to]) return {};
      hit[to] = 1;
      recv[to] = carried[i];
    }
    for (size_t i = r0; i < r1; ++i) hit[size_t(int64_t(s.rows[i].dst) * N + s.rows[i].dst_off / B)] = 0;
  }
  for (int64_t i = 0; i < N; ++i)
    for (int64_t j = 0; j < N; ++j)
      if (recv[size_t(j * N + i)] != uint32_t(i * N + j)) return {};
  return carried;
}

// Copy rows of the one direct copy that runs a whole AllToAll, or 0.
// Pairwise's rows are that copy as they stand; with COLL_OPT_A2A_DIRECT, any
// AllToAll whose rows each move one whole block runs as the copy of its N * N
// blocks (`carried`: the block each row carries).  Blocks must be multiples
// of 16 bytes, and the copy's grid must fit.
uint64_t whole_copy_rows(const Schedule& s, int sz, bool direct, std::vector<uint32_t>* carried) {
  if (s.kind != COLL_K_ALLTOALL || s.rows.empty()) return 0;
  if (copy_prefix_rows(s, sz) == s.rows.size()) return s.rows.size();
  if (!direct) return 0;
  const uint64_t n = uint64_t(s.N) * uint64_t(s.N), row_bytes = uint64_t(s.count / s.N) * uint64_t(sz);
  if (row_bytes == 0 || row_bytes % 16u || (row_bytes + 1023u) / 1024u * n > 0x7fffffffu) return 0;
  std::vector<uint32_t> c = alltoall_carried(s);
  if (c.empty()) return 0;
  if (carried) *carried = std::move(c);
  return n;
}

PlannedCost planned_cost(const Schedule& s, int sz, uint32_t cus) {
  if (col_mode() && s.kind != COLL_K_ALLTOALL) {
    const ColPlan cp = compile_colplan(s, sz, true, t_sums != nullptr);
    if (cp.ok) return PlannedCost{1, int64_t(cp.moved_bytes)};
  }
  if (col_mode() && s.kind == COLL_K_ALLTOALL) {
    // every block read once and written once
    const uint64_t n = whole_copy_rows(s, sz, opt_a2a_direct.load() != 0, nullptr);
    if (n) return PlannedCost{1, int64_t(2 * n * uint64_t(s.count / s.N) * uint64_t(sz))};
  }
  const Bound b = bind_schedule(s, sz, true);
  int64_t moved = b.counts.hbm_bytes;
  const bool a2a = s.kind == COLL_K_ALLTOALL;
  const uint64_t footprint = uint64_t(s.N) * uint64_t(s.count) * uint64_t(sz);
  const uint32_t ntmask = opt_nt.load() < 0 ? auto_nt(footprint, a2a) : uint32_t(opt_nt.load());
  const bool has_reduce =
      s.kind == COLL_K_ALLREDUCE || s.kind == COLL_K_REDUCESCATTER || s.kind == COLL_K_REDUCE;
  for (const Phase& ph : b.phases) {
    if (ph.kind != Phase::ROWS) continue;
    RowsShapeInput in;
    in.colspace = ph.colspace;
    in.segment = phase_segment(ph);
    in.has_reduce = has_reduce;
    in.checksums = t_sums != nullptr;
    in.elem_size = sz;
    in.nranks = s.N;
    in.cus = cus;
    in.resident = uint64_t(cus) * 8u;  // only resident grids use it, and they never forward
    in.per_step = opt_exec.load() == 1;
    in.forced_group_tiles = opt_group.load();
    in.forced_grid = opt_grid.load();
    const RowsShape shape = rows_shape(in, [&] { return several_pieces_per_step(b, ph); });
    if (!shape.group_major) continue;
    const RowsList rl = plan_rows_list(b, ph, std::max<uint64_t>(shape.cap, 1), shape.group_tiles,
                                       opt_reverse.load() != 0, in.per_step, shape.group_major);
    if (forwarding_runs(rl.fwd, rl.fine, rows_ntmask(ntmask, rl.fwd, has_reduce), true)) moved -= int64_t(rl.fwd_saved);
  }
  return PlannedCost{b.counts.steps, moved};
}

coll_status_t auto_algo(coll_kind_t kind, int N, int64_t count, int sz, int root, uint32_t cus, coll_algo_t& out) {
  const std::vector<int64_t> key{int64_t(kind), N, count, sz, root, opt_alpha_ns.load(), opt_beta_gbps.load(),
                                 int64_t(cus), opt_nt.load(), opt_exec.load(), opt_group.load(), opt_grid.load(),
                                 opt_reverse.load(), t_sums != nullptr ? 1 : 0, opt_a2a_direct.load()};
  auto it = g_auto.find(key);
  if (it != g_auto.end()) {
    out = it->second;
    return COLL_OK;
  }
  std::string err;
  const std::function<PlannedCost(const Schedule&)> cost = [&](const Schedule& s) {
    return planned_cost(s, sz, cus);
  };
  const coll_status_t st = choose_algo(kind, N, count, sz, root, cost_model(), out, err, &cost);
  if (st != COLL_OK) return fail(st, err);
  if (g_auto.size() > 4096) g_auto.clear();
  g_auto[key] = out;
  return COLL_OK;
}

// Frees a device buffer, or keeps it until coll_finalize when a captured
// graph may still read it.
void release(void* p, bool pinned) {
  if (!p) return;
  if (pinned) g_retired.push_back(p);
  else (void)hipFree(p);
}

void free_col(ColDev& c) {
  release(c.d_work, c.pinned);
  release(c.d_code, c.pinned);
  release(c.d_row_off, c.pinned);
  release(c.d_refs, c.pinned);
  c = ColDev{};
}

void free_copy(CopyDev& c) {
  release(c.d_idx, c.pinned);
  release(c.d_rows, c.pinned);
  release(c.d_row_off, c.pinned);
  release(c.d_refs, c.pinned);
  c = CopyDev{};
}

void free_entry(Entry& e) {
  release(e.d_items, e.pinned);
  release(e.d_steps, e.pinned);
  for (DevList& l : e.lists) {
    release(l.d_off, l.pinned || e.pinned);
    release(l.d_list, l.pinned || e.pinned);
  }
  for (ColDev& c : e.col) {
    c.pinned = c.pinned || e.pinned;
    free_col(c);
  }
  for (CopyDev& c : e.copy) {
    c.pinned = c.pinned || e.pinned;
    free_copy(c);
  }
  e.lists.clear();
  e.d_items = nullptr;
  e.d_steps = nullptr;
  g_cache_bytes -= e.bytes;
  e.bytes = 0;
}

// Drops the least recently used schedule other than `keep` that no captured
// call uses; its tables may still be read by queued work, so its device is
// synchronised first.  Returns false when there is nothing to drop.
bool evict_lru(const Entry* keep, coll_status_t& st) {
  st = COLL_OK;
  auto lru = g_cache.end();
  for (auto i = g_cache.begin(); i != g_cache.end(); ++i)
    if (i->second.get() != keep && !i->second->pinned &&
        (lru == g_cache.end() || i->second->last_use < lru->second->last_use))
      lru = i;
  if (lru == g_cache.end()) return false;
  int cur = 0;
  hipError_t he = hipGetDevice(&cur);
  if (he == hipSuccess && lru->second->dev != cur) he = hipSetDevice(lru->second->dev);
  if (he == hipSuccess) he = hipDeviceSynchronize();
  if (lru->second->dev != cur) (void)hipSetDevice(cur);
  if (he != hipSuccess) {
    st = hip_fail(he, "hipDeviceSynchronize");
    return false;
  }
  free_entry(*lru->second);
  g_cache.erase(lru);
  return true;
}

// Keeps the cache within COLL_OPT_CACHE_BYTES of device memory (`keep` stays).
coll_status_t trim_cache(const Entry* keep) {
  coll_status_t st = COLL_OK;
  while (g_cache_bytes > uint64_t(opt_cache_bytes.load()) && evict_lru(keep, st)) {
  }
  return st;
}

// Frees one partial-slot buffer after its device has finished the work queued
// on it (the kernels that use it may still be running); a buffer a captured
// call uses is kept until coll_finalize instead.
void free_sum_scratch(SumScratch& s) {
  if (s.d && s.pinned) {
    g_retired.push_back(s.d);
  } else if (s.d) {
    int cur = 0;
    const bool have_cur = hipGetDevice(&cur) == hipSuccess;
    if (hipSetDevice(s.dev) == hipSuccess) (void)hipDeviceSynchronize();
    (void)hipFree(s.d);
    if (have_cur) (void)hipSetDevice(cur);
  }
  s.d = nullptr;
  s.cap = 0;
  s.pinned = false;
}

// Partial checksum slots for `n` slots on device `dev`, for the caller's
// buffer `user` (allocated, or grown, on first use).
coll_status_t sum_scratch(int dev, const uint64_t* user, size_t n, SumScratch*& out) {
  SumScratch* hit = nullptr;
  for (SumScratch& s : g_sum_scratch)
    if (s.dev == dev && s.user == user) hit = &s;
  if (!hit) {
    if (g_sum_scratch.size() >= SUM_SCRATCH_MAX) {
      auto lru = g_sum_scratch.end();
      for (auto i = g_sum_scratch.begin(); i != g_sum_scratch.end(); ++i)
        if (!i->pinned && (lru == g_sum_scratch.end() || i->last_use < lru->last_use)) lru = i;
      if (lru != g_sum_scratch.end()) {
        free_sum_scratch(*lru);
        g_sum_scratch.erase(lru);
      }
    }
    g_sum_scratch.push_back(SumScratch{});
    hit = &g_sum_scratch.back();
    hit->dev = dev;
    hit->user = user;
  }
  hit->last_use = ++g_tick;
  if (hit->cap < n) {
    free_sum_scratch(*hit);
    hipError_t he = hipMalloc(reinterpret_cast<void**>(&hit->d), n * sizeof(uint64_t));
    if (he != hipSuccess) {
      hit->d = nullptr;
      return fail(COLL_ERR_NO_MEMORY, std::string("hipMalloc: ") + hipGetErrorString(he));
    }
    hit->cap = n;
    hit->clean = false;
  }
  out = hit;
  return COLL_OK;
}

// The work lists of phase `pi` for a grid of at most `cap` work groups and
// column groups of `gt` tiles (plan_rows_list), built and uploaded on first use.
coll_status_t get_list(Entry& e, size_t pi, uint64_t cap, uint32_t gt, bool reverse, bool per_step, bool group_major,
                       DevList*& out) {
  for (DevList& l : e.lists)
    if (l.phase == pi && l.cap == cap && l.gt == gt && l.reverse == reverse && l.per_step == per_step &&
        l.group_major == group_major) {
      out = &l;
      return COLL_OK;
    }
  // a few launch shapes per schedule are plenty: drop the oldest one no
  // captured call uses
  size_t unpinned = 0, oldest = e.lists.size();
  for (size_t i = 0; i < e.lists.size(); ++i)
    if (!e.lists[i].pinned && !e.pinned) {
      ++unpinned;
      if (oldest == e.lists.size()) oldest = i;
    }
  if (unpinned >= 8 && oldest < e.lists.size()) {
    hipError_t he = hipDeviceSynchronize();
    if (he != hipSuccess) return hip_fail(he, "hipDeviceSynchronize");
    DevList& l = e.lists[oldest];
    (void)hipFree(l.d_off);
    (void)hipFree(l.d_list);
    e.bytes -= l.bytes;
    g_cache_bytes -= l.bytes;
    e.lists.erase(e.lists.begin() + long(oldest));
  }
  const Phase& ph = e.bound.phases[pi];
  RowsList rl = plan_rows_list(e.bound, ph, cap, gt, reverse, per_step, group_major);
  const std::vector<uint32_t>& off = rl.off;
  const std::vector<DevItem>& list = rl.list;
  DevList l;
  l.phase = pi;
  l.cap = cap;
  l.G = rl.G;
  l.gt = gt;
  l.reverse = reverse;
  l.per_step = per_step;
  l.group_major = group_major;
  l.launches = per_step ? ph.s1 - ph.s0 : 1;
  l.fine = rl.fine;
  l.fwd = rl.fwd;
  l.fwd_saved = rl.fwd_saved;
  hipError_t he = hipMalloc(reinterpret_cast<void**>(&l.d_off), off.size() * sizeof(uint32_t));
  if (he != hipSuccess) return fail(COLL_ERR_NO_MEMORY, std::string("hipMalloc: ") + hipGetErrorString(he));
  he = hipMalloc(reinterpret_cast<void**>(&l.d_list), std::max<size_t>(list.size(), 1) * sizeof(DevItem));
  if (he != hipSuccess) {
    (void)hipFree(l.d_off);
    return fail(COLL_ERR_NO_MEMORY, std::string("hipMalloc: ") + hipGetErrorString(he));
  }
  he = hipMemcpy(l.d_off, off.data(), off.size() * sizeof(uint32_t), hipMemcpyHostToDevice);
  if (he == hipSuccess && !list.empty())
    he = hipMemcpy(l.d_list, list.data(), list.size() * sizeof(DevItem), hipMemcpyHostToDevice);
  if (he != hipSuccess) {
    (void)hipFree(l.d_off);
    (void)hipFree(l.d_list);
    return hip_fail(he, "hipMemcpy");
  }
  l.bytes = off.size() * sizeof(uint32_t) + std::max<size_t>(list.size(), 1) * sizeof(DevItem);
  e.bytes += l.bytes;
  g_cache_bytes += l.bytes;
  e.lists.push_back(l);
  out = &e.lists.back();
  return trim_cache(&e);
}

template <class T>
coll_status_t upload(const std::vector<T>& v, T*& d) {
  d = nullptr;
  hipError_t he = hipMalloc(reinterpret_cast<void**>(&d), std::max<size_t>(v.size(), 1) * sizeof(T));
  if (he != hipSuccess) {
    d = nullptr;
    return fail(COLL_ERR_NO_MEMORY, std::string("hipMalloc: ") + hipGetErrorString(he));
  }
  if (!v.empty()) he = hipMemcpy(d, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice);
  if (he != hipSuccess) {
    (void)hipFree(d);
    d = nullptr;
    return hip_fail(he, "hipMemcpy");
  }
  return COLL_OK;
}

// Column kernel: tiles per work group.  Column spaces under 64 tiles per CU:
// 1, so that every compute unit gets work.  Without checksums: 2 from 128 up
// to 512 tiles per CU for unbatched programs, 4 above for single-leaf ones,
// else 1 (a work group that ends
// after one tile never waits for its stores, which pays where the whole call
// fits the memory-side cache and where it streams; batched programs hold
// fewer waves per CU and lose with 2: ReduceScatter bf16 32 x 64 MiB 0.389
// against 0.422 ms).  With row checksums more tiles make the
// partial sums fewer for the fold to add, but fewer, longer work groups leave
// a tail: 2, and 4 from 1,024 tiles per CU.  Measured on Ring AllReduce fp32
// over 8 ranks, each call after a restore of its inputs, ms per call with
// checksums, 2 / 4 tiles: 64 MiB per rank 0.195 / 0.225, 128 MiB 0.364 /
// 0.371, 256 MiB 5.75 / 5.81 TB/s; without, 1 / 2 tiles: 16 MiB 0.0421 /
// 0.0426 ms, 24 MiB 0.0688 / 0.0704, 32 MiB 0.1022 / 0.0921, 48 MiB 0.1421 /
// 0.1343, 64 MiB 0.1946 / 0.1921, 96 MiB 0.302 / 0.289, 128 MiB 0.367 /
// 0.377, 256 MiB 5.78 / 5.71 TB/s; 8 ranks x 64 MiB, 1 / 2 tiles: Ring
// ReduceScatter bf16 0.1256 / 0.1215 ms, AllGather 0.0975 / 0.0954, tree
// Reduce fp32 0.1228 / 0.1199, Broadcast 0.0975 / 0.0959.  From 512 tiles
// per CU single-leaf programs (AllGather, Broadcast: one load, many stores)
// take 4: 256 MiB per rank, 1 / 2 / 4 / 8 tiles, Broadcast uint8 8 ranks
// 0.420 / 0.414 / 0.389 / 0.402 ms, AllGather bf16 8 ranks 0.406 / 0.417 /
// 0.390 / 0.403 ms, 64 ranks 3.336 / 3.276 / 3.304 / 3.396 ms; the Ring
// AllReduce fp32 8 ranks 0.738 / 0.743 / 0.770 / 0.793 ms.
uint64_t col_tile_count(const ColPlan& p) {
  const uint64_t tb = uint64_t(COL_THREADS) * uint64_t(p.v.unit);
  uint64_t tiles = 0;
  for (const ColSeg& sg : p.segs) tiles += (sg.s1 + tb - 1) / tb - sg.s0 / tb;
  return tiles;
}

uint32_t auto_col_tiles(const ColPlan& p, uint32_t cus) {
  const uint64_t tiles = col_tile_count(p);
  if (tiles < uint64_t(cus) * 64u) return 1;
  if (p.v.accs <= 0) {
    if (p.batched || tiles < uint64_t(cus) * 128u) return 1;
    if (tiles < uint64_t(cus) * 512u) return 2;
    return p.max_leaves <= 1 ? 4 : 1;  // single-leaf programs: 1 load, many stores per tile
  }
  return tiles >= uint64_t(cus) * 1024u ? 4 : 2;
}

// The column kernel's paired variant without checksums (4 waves per SIMD)
// and the capped batched ones pay from 128 tiles per CU; below, the plain
// variants run the same programs (Ring AllReduce fp32 8 x 16 MiB, 64 tiles per
// CU: 0.0422 ms plain, 0.0446 ms paired).
void fit_col_variant(ColPlan& p, uint32_t cus) {
  if (!p.ok || (p.v.accs >= 0 && !p.v.capped) || col_tile_count(p) >= uint64_t(cus) * 128u) return;
  if (p.v.accs < 0) p.v.accs = 0;
  p.v.capped = false;
}

// Column kernel: nontemporal loads and stores once the call's buffers exceed
// twice the memory-side cache (a call reads and writes each byte once).
// Below that, part of the inputs is still in the cache from whatever wrote
// them.  Measured as above, ordinary / nontemporal, 1 tile without
// checksums: 48 MiB per rank (384 MiB of buffers) 5.54 / 5.14 TB/s, 64 MiB
// 5.46 / 5.33, 80 MiB 5.45 / 5.40, 96 MiB 5.26 / 5.45, 128 MiB 5.50 / 5.79,
// 256 MiB 5.38 / 5.78.
constexpr uint64_t COL_NT_BYTES = 2 * CACHE_RESIDENT_BYTES;

// The column programs of a schedule for this call's checksum mode, compiled
// and uploaded on first use, with work groups of `tiles` tiles.  out->plan.ok
// false: the row kernel runs the schedule.
coll_status_t get_col(Entry& e, const Key& k, bool cks, uint32_t cus, ColDev*& out) {
  ColDev& c = e.col[cks ? 1 : 0];
  out = &c;
  if (!c.tried) {
    c.tried = true;
    c.plan = compile_colplan(e.sched, k.sz, k.inplace != 0, cks);
    if (!c.plan.ok) return COLL_OK;
    fit_col_variant(c.plan, cus);
    const coll_status_t st = upload(c.plan.code, c.d_code);
    if (st != COLL_OK) {
      free_col(c);
      return st;
    }
    c.tried = true;
    c.code_bytes = std::max<size_t>(c.plan.code.size(), 1) * sizeof(ColInstr);
    e.bytes += c.code_bytes;
    g_cache_bytes += c.code_bytes;
  }
  if (!c.plan.ok) return COLL_OK;
  const uint32_t tiles = opt_col_tiles.load() > 0 ? uint32_t(opt_col_tiles.load()) : auto_col_tiles(c.plan, cus);
  if (c.d_work && c.tiles == tiles) return COLL_OK;
  const ColTables t = col_tables(c.plan, tiles, size_t(e.bound.nrows));
  ColWork* dw = nullptr;
  uint32_t* dro = nullptr;
  ColRef* drf = nullptr;
  coll_status_t st = upload(t.work, dw);
  if (st == COLL_OK && cks) st = upload(t.row_off, dro);
  if (st == COLL_OK && cks) st = upload(t.refs, drf);
  if (st != COLL_OK) {
    if (dw) (void)hipFree(dw);
    if (dro) (void)hipFree(dro);
    return st;
  }
  if (c.d_work && !c.pinned) {
    // queued calls may still read the old tables
    const hipError_t he = hipDeviceSynchronize();
    if (he != hipSuccess) {
      (void)hipFree(dw);
      if (dro) (void)hipFree(dro);
      if (drf) (void)hipFree(drf);
      return hip_fail(he, "hipDeviceSynchronize");
    }
  }
  release(c.d_work, c.pinned);
  release(c.d_row_off, c.pinned);
  release(c.d_refs, c.pinned);
  c.d_work = dw;
  c.d_row_off = dro;
  c.d_refs = drf;
  c.tiles = tiles;
  c.nwork = uint32_t(t.work.size());
  c.partials = t.partials;
  const uint64_t old = c.table_bytes;
  c.table_bytes = std::max<size_t>(t.work.size(), 1) * sizeof(ColWork) +
                  (cks ? std::max<size_t>(t.row_off.size(), 1) * sizeof(uint32_t) +
                             std::max<size_t>(t.refs.size(), 1) * sizeof(ColRef)
                       : 0);
  e.bytes = e.bytes - old + c.table_bytes;
  g_cache_bytes = g_cache_bytes - old + c.table_bytes;
  return trim_cache(&e);
}

// The direct-copy tables of a whole AllToAll (whole_copy_rows) or of its
// leading independent rows (copy_prefix_rows); built and uploaded on first
// use.  Leading rows replace the schedule's first phase, which must cover
// exactly those rows' steps.  out->ok false: the row kernels run them.
coll_status_t get_copy(Entry& e, const Key& k, bool direct, CopyDev*& out) {
  CopyDev& c = e.copy[direct ? 1 : 0];
  out = &c;
  if (c.tried) return COLL_OK;
  c.tried = true;
  const Schedule& s = e.sched;
  std::vector<uint32_t> carried;
  const uint64_t nwhole = whole_copy_rows(s, k.sz, direct, &carried);
  const bool mapped = !carried.empty();  // the copy rows are the blocks, not the schedule's rows
  const size_t n0 = nwhole ? size_t(nwhole) : copy_prefix_rows(s, k.sz);
  if (n0 == 0) return COLL_OK;
  const bool whole = nwhole != 0;
  if (!whole) {
    // the rows kernel's first phase is these rows' steps, the rest staged
    const Bound& b = e.bound;
    if (b.phases.size() != 2 || b.phases[0].kind != Phase::ROWS || b.phases[1].kind != Phase::PERM) return COLL_OK;
    const uint32_t s1 = b.phases[0].s1;
    if (b.phases[0].s0 != 0 || s1 == 0 || s1 > s.steps.size() ||
        size_t(s.steps[s1 - 1].first + s.steps[s1 - 1].nrows) != n0)
      return COLL_OK;
  }
  const uint64_t row_bytes = uint64_t(s.rows[0].n) * uint64_t(k.sz);
  const uint64_t wgs = (row_bytes + 1023u) / 1024u;
  const size_t nfold = mapped ? s.rows.size() : n0;
  // the fold's references: one per copy row (its work groups' slots); a
  // mapped schedule's rows then take their block's sum through idx
  std::vector<CopyRow> rows(n0);
  std::vector<uint32_t> row_off(n0 + 1), idx;
  std::vector<ColRef> refs(n0);
  for (size_t i = 0; i < n0; ++i) {
    row_off[i] = uint32_t(i);
    refs[i] = ColRef{uint32_t(i * wgs), uint32_t(wgs), 1u, 0u};
  }
  row_off[n0] = uint32_t(n0);
  if (mapped) {
    // send block j of rank i is copy row ((j - i) mod N) * N + i, Pairwise's
    // order (round k: every rank's block k ahead)
    const int64_t N = s.N, B = s.count / N;
    const auto copy_row = [N](int64_t i, int64_t j) { return uint32_t(((j - i + N) % N) * N + i); };
    for (int64_t i = 0; i < N; ++i)
      for (int64_t j = 0; j < N; ++j)
        rows[copy_row(i, j)] = CopyRow{uint32_t(i), uint32_t(j), uint64_t(j * B) * uint64_t(k.sz),
                                       uint64_t(i * B) * uint64_t(k.sz)};
    idx.resize(nfold);
    for (size_t r = 0; r < nfold; ++r) idx[r] = copy_row(carried[r] / N, carried[r] % N);
  } else {
    for (size_t i = 0; i < n0; ++i) {
      const Row& r = s.rows[i];
      rows[i] = CopyRow{uint32_t(r.src), uint32_t(r.dst), uint64_t(r.src_off) * uint64_t(k.sz),
                        uint64_t(r.dst_off) * uint64_t(k.sz)};
    }
  }
  CopyRow* dr = nullptr;
  uint32_t* dro = nullptr;
  ColRef* drf = nullptr;
  uint32_t* dix = nullptr;
  coll_status_t st = upload(rows, dr);
  if (st == COLL_OK) st = upload(row_off, dro);
  if (st == COLL_OK) st = upload(refs, drf);
  if (st == COLL_OK && mapped) st = upload(idx, dix);
  if (st != COLL_OK) {
    if (dr) (void)hipFree(dr);
    if (dro) (void)hipFree(dro);
    if (drf) (void)hipFree(drf);
    return st;
  }
  c.d_rows = dr;
  c.d_row_off = dro;
  c.d_refs = drf;
  c.d_idx = dix;
  c.nrows = uint32_t(n0);
  c.nfold = uint32_t(nfold);
  c.whole = whole;
  c.wgs_per_row = uint32_t(wgs);
  c.row_bytes = row_bytes;
  c.ok = true;
  c.bytes = rows.size() * sizeof(CopyRow) + (row_off.size() + idx.size()) * sizeof(uint32_t) +
            refs.size() * sizeof(ColRef);
  e.bytes += c.bytes;
  g_cache_bytes += c.bytes;
  return trim_cache(&e);
}

coll_status_t device_info(int dev, DevInfo*& out) {
  auto it = g_dev.find(dev);
  if (it == g_dev.end()) {
    DevInfo di;
    hipError_t e = hipDeviceGetAttribute(&di.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    it = g_dev.emplace(dev, di).first;
  }
  out = &it->second;
  return COLL_OK;
}

int occupancy_rows(int dev, int dt, int op, bool cks, uint32_t nt) {
  const uint64_t key = (uint64_t(dev) << 32) | uint64_t(dt * 256 + op * 32 + (cks ? 16 : 0) + nt);
  auto it = g_occ.find(key);
  if (it != g_occ.end()) return it->second;
  const int n = rows_blocks_per_cu(dt, op, cks, nt);
  g_occ[key] = n;
  return n;
}

int occupancy_perm(int dev, int unit, int slots, bool hoist, bool cks, bool nt) {
  const uint64_t key = (uint64_t(dev) << 32) | (uint64_t(1) << 31) | (uint64_t(hoist) << 20) |
                       uint64_t(slots * 256 + unit * 4 + (cks ? 2 : 0) + (nt ? 1 : 0));
  auto it = g_occ.find(key);
  if (it != g_occ.end()) return it->second;
  const int n = perm_blocks_per_cu(unit, slots, hoist, cks, nt);
  g_occ[key] = n;
  return n;
}

coll_status_t get_entry(const Key& k, Entry*& out) {
  auto it = g_cache.find(k);
  if (it != g_cache.end()) {
    it->second->last_use = ++g_tick;
    out = it->second.get();
    return COLL_OK;
  }
  if (g_cache.size() >= CACHE_CAP) {
    coll_status_t st = COLL_OK;
    evict_lru(nullptr, st);
    if (st != COLL_OK) return st;
  }
  Schedule s;
  std::string err;
  coll_status_t st = build_schedule(coll_kind_t(k.kind), coll_algo_t(k.algo), k.N, k.count, k.root, k.chunks, s, err);
  if (st != COLL_OK) return fail(st, err);
  const std::string hz = check_schedule(s);
  if (!hz.empty()) return fail(COLL_ERR_UNSUPPORTED, "internal schedule conflict: " + hz);
  auto e = std::make_unique<Entry>();
  e->bound = bind_schedule(s, k.sz, k.inplace != 0);
  e->sched = std::move(s);
  const Bound& b = e->bound;
  if (!b.items.empty()) {
    hipError_t he = hipMalloc(reinterpret_cast<void**>(&e->d_items), b.items.size() * sizeof(DevItem));
    if (he != hipSuccess) return fail(COLL_ERR_NO_MEMORY, std::string("hipMalloc: ") + hipGetErrorString(he));
    he = hipMalloc(reinterpret_cast<void**>(&e->d_steps), b.steps.size() * sizeof(DevStep));
    if (he != hipSuccess) {
      free_entry(*e);
      return fail(COLL_ERR_NO_MEMORY, std::string("hipMalloc: ") + hipGetErrorString(he));
    }
    he = hipMemcpy(e->d_items, b.items.data(), b.items.size() * sizeof(DevItem), hipMemcpyHostToDevice);
    if (he == hipSuccess)
      he = hipMemcpy(e->d_steps, b.steps.data(), b.steps.size() * sizeof(DevStep), hipMemcpyHostToDevice);
    if (he != hipSuccess) {
      free_entry(*e);
      return hip_fail(he, "hipMemcpy");
    }
  }
  e->dev = k.dev;
  if (e->d_items) e->bytes = b.items.size() * sizeof(DevItem) + b.steps.size() * sizeof(DevStep);
  g_cache_bytes += e->bytes;
  e->last_use = ++g_tick;
  out = e.get();
  g_cache.emplace(k, std::move(e));
  return trim_cache(out);
}

// Pointer checks: non-null, element-aligned, no overlap between distinct rank
// buffers, in place either for every rank or for none.
coll_status_t check_buffers(void* const* send, void* const* recv, int N, int64_t count, int sz, bool a2a,
                            bool& inplace) {
  if (!send) return fail(COLL_ERR_INVALID_ARG, "sendbufs is NULL");
  inplace = true;
  // nothing is read or written: empty buffers may share any pointer
  if (count == 0) return COLL_OK;
  if (recv) {
    int same = 0;
    for (int i = 0; i < N; ++i) same += recv[i] == send[i];
    if (same != 0 && same != N) return fail(COLL_ERR_INVALID_ARG, "recvbufs alias sendbufs for some ranks only");
    inplace = same == N;
  }
  if (a2a && inplace) return fail(COLL_ERR_INVALID_ARG, "alltoall must be out of place");
  // all rank buffers have the same length, so sorting the start addresses
  // and comparing neighbours finds any overlap
  uint64_t starts[2 * COLL_MAX_RANKS];
  int n = 0;
  const uint64_t bytes = uint64_t(count) * uint64_t(sz);
  for (int side = 0; side < (inplace ? 1 : 2); ++side) {
    void* const* v = side ? recv : send;
    for (int i = 0; i < N; ++i) {
      const uint64_t p = reinterpret_cast<uint64_t>(v[i]);
      if (!p) return fail(COLL_ERR_INVALID_ARG, "a rank buffer is NULL");
      if (p % uint64_t(sz)) return fail(COLL_ERR_INVALID_ARG, "a rank buffer is not aligned to the element size");
      starts[n++] = p;
    }
  }
  std::sort(starts, starts + n);
  for (int i = 1; i < n; ++i)
    if (starts[i] - starts[i - 1] < bytes) return fail(COLL_ERR_INVALID_ARG, "rank buffers overlap");
  return COLL_OK;
}

// Every check of a collective call's arguments that needs no HIP call: sizes,
// pointers, aliasing, the algorithm and scalars (no rows built), also when
// there is nothing to move.
coll_status_t check_call(coll_kind_t kind, void* const* send, void* const* recv, int N, size_t count_in,
                         coll_dtype_t dtype, coll_op_t op, coll_algo_t algo, int root, int chunks, int& sz,
                         int64_t& count, bool& inplace) {
  sz = elem_size(dtype);
  if (!sz) return fail(COLL_ERR_INVALID_ARG, "unknown dtype");
  if (int(op) < 0 || int(op) > 2) return fail(COLL_ERR_INVALID_ARG, "unknown op");
  if (N < 1) return fail(COLL_ERR_INVALID_ARG, "nranks must be at least 1");
  if (N > COLL_MAX_RANKS) return fail(COLL_ERR_UNSUPPORTED, "nranks above COLL_MAX_RANKS");
  if (count_in > (size_t(1) << 44) / size_t(sz)) return fail(COLL_ERR_INVALID_ARG, "count too large");
  count = int64_t(count_in);
  inplace = true;
  coll_status_t st = check_buffers(send, recv, N, count, sz, kind == COLL_K_ALLTOALL, inplace);
  if (st != COLL_OK) return st;
  const bool automatic = algo == COLL_ALGO_AUTO;
  std::string err;
  st = validate_schedule_args(kind, automatic ? COLL_ALGO_DEFAULT : algo, N, count, root, automatic ? 1 : chunks, err);
  if (st != COLL_OK) return fail(st, err);
  // the permutation kernel addresses a block with 32-bit unit offsets
  if (kind == COLL_K_ALLTOALL && uint64_t(count / N) * uint64_t(sz) >= (uint64_t(1) << 31))
    return fail(COLL_ERR_UNSUPPORTED, "AllToAll blocks of 2 GiB or more");
  return COLL_OK;
}

// One kernel launch of a call, planned before anything is enqueued.
struct Launch {
  enum Kind { COL, COPY, ROWS, PERM } kind = ROWS;
  // COL
  const ColWork* work = nullptr;
  const ColInstr* code = nullptr;
  const uint32_t* row_off = nullptr;
  const ColRef* refs = nullptr;
  ColVariant v;
  uint32_t grid = 0;
  bool nt = false;
  // ROWS
  const DevItem* list = nullptr;
  const uint32_t* off = nullptr;
  uint32_t launches = 0;
  uint32_t ntmask = 0;
  bool fine = false, fwd = false;
  // PERM
  uint32_t s0 = 0, s1 = 0, lg = 0, ncols = 0;
  int unit = 16, slots = 8;
  bool hoist = false;           // descriptors once per group (groups over 32 rows)
};

coll_status_t run(coll_kind_t kind, void* const* send, void* const* recv, int N, size_t count_in, coll_dtype_t dtype,
                  coll_op_t op, coll_algo_t algo, int root, int chunks, void* stream_v) {
  int sz = 0;
  int64_t count = 0;
  bool inplace = true;
  coll_status_t st = check_call(kind, send, recv, N, count_in, dtype, op, algo, root, chunks, sz, count, inplace);
  if (st != COLL_OK) return st;
  const bool automatic = algo == COLL_ALGO_AUTO;
  if (automatic) chunks = 1;
  t_last = coll_counts_t{};
  if (count == 0) return COLL_OK;

  int dev = 0;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return hip_fail(he, "hipGetDevice");
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);

  std::lock_guard<std::mutex> lock(g_mu);
  DevInfo* di = nullptr;
  st = device_info(dev, di);
  if (st != COLL_OK) return st;
  coll_algo_t chosen = algo;
  if (automatic) {
    st = auto_algo(kind, N, count, sz, root, uint32_t(di->cus), chosen);
    if (st != COLL_OK) return st;
  }
  const coll_algo_t ra = resolve_algo(kind, chosen);
  const bool rooted =
      kind == COLL_K_BROADCAST || kind == COLL_K_SCATTER || kind == COLL_K_GATHER || kind == COLL_K_REDUCE;
  const bool pipe = algo_pipelined(ra);
  Key k{dev, int(kind), int(ra), N, count, sz, rooted ? root : 0, pipe ? chunks : 1, inplace ? 1 : 0};
  Entry* e = nullptr;
  st = get_entry(k, e);
  if (st != COLL_OK) return st;
  const Bound& b = e->bound;

  // ---- plan every launch and allocate what it needs; nothing is enqueued
  // before this part has succeeded, so an error leaves no partial work
  const bool cks = t_sums != nullptr;
  if (cks && size_t(b.nrows) > t_sums_cap) return fail(COLL_ERR_INVALID_ARG, "checksum buffer smaller than the schedule");
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const bool capturing = hipStreamIsCapturing(stream, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone;
  const uint64_t footprint = uint64_t(N) * uint64_t(count) * uint64_t(sz) * (inplace ? 1u : 2u);
  const uint32_t ntmask = opt_nt.load() < 0 ? auto_nt(footprint, kind == COLL_K_ALLTOALL) : uint32_t(opt_nt.load());
  const bool step_mode = opt_exec.load() == 1;

  RankPtrs ptrs;
  uint64_t align_or = 0;
  for (int i = 0; i < N; ++i) {
    ptrs.send[i] = reinterpret_cast<uint64_t>(send[i]);
    ptrs.recv[i] = reinterpret_cast<uint64_t>(inplace ? send[i] : recv[i]);
    align_or |= ptrs.send[i] | ptrs.recv[i];
  }
  for (int i = N; i < COLL_MAX_RANKS; ++i) ptrs.send[i] = ptrs.recv[i] = 0;
  const bool bases16 = (align_or % 16) == 0;

  const int dt = int(dtype) == COLL_INT32 ? DT_I32 : int(dtype) == COLL_UINT8 ? DT_U8
               : int(dtype) == COLL_FLOAT32 ? DT_F32 : DT_BF16;
  const bool has_reduce = kind == COLL_K_ALLREDUCE || kind == COLL_K_REDUCESCATTER || kind == COLL_K_REDUCE;
  std::vector<Launch> plan;
  std::string dbg;    // launch shapes, for COLL_DEBUG
  int64_t moved = b.counts.hbm_bytes;
  ColDev* cd = nullptr;
  CopyDev* xd = nullptr;
  if (col_mode() && bases16 && kind != COLL_K_ALLTOALL) {
    st = get_col(*e, k, cks, uint32_t(di->cus), cd);
    if (st != COLL_OK) return st;
    if (!cd->plan.ok) cd = nullptr;
  }
  if (col_mode() && bases16 && kind == COLL_K_ALLTOALL) {
    st = get_copy(*e, k, opt_a2a_direct.load() != 0, xd);
    if (st != COLL_OK) return st;
    if (!xd->ok) xd = nullptr;
  }
  // a copy of leading rows that are not the whole schedule stands for phase 0
  const bool copy_part = xd && !xd->whole;
  const uint64_t n0 = xd ? xd->nfold : 0;  // schedule rows the direct copy makes
  if (xd) {
    Launch L;
    L.kind = Launch::COPY;
    L.nt = ntmask != 0;
    L.grid = xd->nrows * xd->wgs_per_row;
    if (L.grid) plan.push_back(L);
    if (g_debug.load())
      dbg += " | copy rows: " + std::to_string(xd->nrows) + " rows of " + std::to_string(xd->row_bytes) + " bytes, grid " +
             std::to_string(L.grid) + (L.nt ? " nontemporal" : "") +
             (xd->nfold != xd->nrows ? ", the blocks of " + std::to_string(xd->nfold) + " schedule rows" : "");
  }
  if (xd && xd->whole) {
    moved = int64_t(2 * uint64_t(xd->nrows) * xd->row_bytes);  // every block read once, written once
  } else if (cd) {
    Launch L;
    L.kind = Launch::COL;
    L.work = cd->d_work;
    L.code = cd->d_code;
    L.row_off = cd->d_row_off;
    L.refs = cd->d_refs;
    L.v = cd->plan.v;
    L.grid = cd->nwork;
    // nothing is read twice: past twice the memory-side cache every access streams
    L.nt = opt_nt.load() < 0 ? footprint > COL_NT_BYTES : (ntmask & (NT_SRC | NT_DST)) != 0;
    if (L.grid) plan.push_back(L);
    moved = int64_t(cd->plan.moved_bytes);
    if (g_debug.load())
      dbg += " | columns: " + std::to_string(cd->plan.segs.size()) + " segments, grid " + std::to_string(L.grid) +
             " tiles " + std::to_string(cd->tiles) + " unit " + std::to_string(L.v.unit) + " slots " +
             std::to_string(L.v.leaves) + (L.v.accs > 0 ? " checksum ops " + std::to_string(L.v.accs) : "") +
             (L.v.accs < 0 ? " paired" : "") + (L.v.capped ? " capped" : "") +
             (L.v.batched ? " batched" : "") + (L.nt ? " nontemporal" : "");
  } else {
    for (size_t pi = copy_part ? 1 : 0; pi < b.phases.size(); ++pi) {
      const Phase& ph = b.phases[pi];
      Launch L;
      if (ph.kind == Phase::ROWS) {
        RowsShapeInput in;
        in.colspace = ph.colspace;
        in.segment = phase_segment(ph);
        in.has_reduce = has_reduce;
        in.checksums = cks;
        in.elem_size = sz;
        in.nranks = N;
        in.cus = uint32_t(di->cus);
        in.resident = uint64_t(di->cus) * uint64_t(occupancy_rows(dev, dt, int(op), cks, ntmask));
        in.per_step = step_mode;
        in.forced_group_tiles = opt_group.load();
        in.forced_grid = opt_grid.load();
        const RowsShape shape = rows_shape(in, [&] {
          if (e->multi.size() != b.phases.size()) e->multi.assign(b.phases.size(), int8_t(-1));
          if (e->multi[pi] < 0) e->multi[pi] = several_pieces_per_step(b, ph) ? 1 : 0;
          return e->multi[pi] != 0;
        });
        DevList* D = nullptr;
        st = get_list(*e, pi, std::max<uint64_t>(shape.cap, 1), shape.group_tiles, opt_reverse.load() != 0, step_mode,
                      shape.group_major, D);
        if (st != COLL_OK) return st;
        if (capturing) D->pinned = true;
        L.kind = Launch::ROWS;
        L.list = D->d_list;
        L.off = D->d_off;
        L.grid = D->G;
        L.launches = D->launches;
        L.fine = D->fine;
        L.fwd = D->fwd;
        L.ntmask = rows_ntmask(ntmask, D->fwd, has_reduce);
        if (forwarding_runs(D->fwd, D->fine, L.ntmask, bases16)) moved -= int64_t(D->fwd_saved);
        if (g_debug.load())
          dbg += " | rows steps " + std::to_string(ph.s0) + ".." + std::to_string(ph.s1) + " grid " +
                 std::to_string(L.grid) + " group_tiles " + std::to_string(shape.group_tiles) +
                 (L.fine ? " fine" : "") + (forwarding_runs(D->fwd, D->fine, L.ntmask, bases16) ? " forwarding" : "") +
                 " nt " + std::to_string(L.ntmask) + " launches " + std::to_string(L.launches);
      } else {
        L.kind = Launch::PERM;
        int unit = b.perm_unit;
        while (unit > 1 && (align_or % uint64_t(unit))) unit >>= 1;
        L.unit = unit;
        L.ncols = uint32_t(ph.colspace / uint64_t(unit));
        // every staged AllToAll step permutes groups of N rows; each of the 4 waves
        // holds ceil(N/4) rows, 2^lg units per lane of each
        const uint32_t ipw = uint32_t(N + 3) / 4;
        // slots per lane: measured at 32 ranks (5-8 rows per wave) 8 slots, one
        // unit per row, beat 16 (Bruck 7.5 vs 8.0 ms); at 8 and 16 ranks 16 slots
        // beat 8 (0.68 vs 0.72 ms, 1.63 vs 1.77 ms)
        L.slots = ipw > 4 && ipw <= 8 ? 8 : ipw <= 16 ? 16 : 32;
        L.hoist = N > 32;
        uint32_t lg = 0;
        while ((ipw << (lg + 1)) <= uint32_t(L.slots) && (64u << (lg + 1)) <= std::max<uint32_t>(L.ncols, 64)) ++lg;
        L.lg = lg;
        const uint64_t tu = uint64_t(64) << lg;
        const uint64_t ntiles = (uint64_t(L.ncols) + tu - 1) / tu;
        uint64_t cap = uint64_t(di->cus) * uint64_t(occupancy_perm(dev, unit, L.slots, L.hoist, cks, ntmask != 0));
        if (opt_grid.load() > 0) cap = uint64_t(opt_grid.load());
        // the same number of tiles for every work group
        const uint64_t per_wg = std::max<uint64_t>(1, (ntiles + cap - 1) / cap);
        L.grid = uint32_t(std::max<uint64_t>(1, (ntiles + per_wg - 1) / per_wg));
        L.s0 = ph.s0;
        L.s1 = ph.s1;
        L.ntmask = ntmask;
        if (g_debug.load())
          dbg += " | perm steps " + std::to_string(ph.s0) + ".." + std::to_string(ph.s1) + " grid " +
                 std::to_string(L.grid) + " unit " + std::to_string(unit) + " slots " + std::to_string(L.slots) +
                 (L.hoist ? " hoisted" : "");
      }
      plan.push_back(L);
    }
  }
  uint64_t* partial = nullptr;  // SUM_LANES slots per row, folded into t_sums after the kernels
  uint64_t* copy_partial = nullptr;  // the direct copy's slot per work group, then the fold's slices
  SumScratch* scratch = nullptr;
  const uint64_t copy_slots = xd ? uint64_t(xd->nrows) * xd->wgs_per_row : 0;
  if (cks) {
    // the row kernels' SUM_LANES slots per row, or the column kernel's partial
    // sums and the fold's slices; a direct copy's slots and slices after the
    // row kernels' slots, if any
    const size_t rows_slots = (cd || (xd && xd->whole)) ? 0 : std::max<size_t>(size_t(b.nrows), 1) * SUM_LANES;
    // (a whole AllToAll's copy: its blocks' fold slices and sums, which its
    // rows then gather)
    const size_t copy_fold = !xd ? 0 : xd->d_idx ? size_t(xd->nrows) * (COL_FOLD_SLICES + 1) : size_t(n0) * COL_FOLD_SLICES;
    const size_t slots = cd ? size_t(cd->partials) + std::max<size_t>(size_t(b.nrows), 1) * COL_FOLD_SLICES
                            : rows_slots + (xd ? size_t(copy_slots) + copy_fold : 0);
    st = sum_scratch(dev, t_sums, slots, scratch);
    if (st != COLL_OK) return st;
    partial = scratch->d;
    if (xd) copy_partial = partial + rows_slots;
  }
  if (capturing) {
    // a graph replays this call later without the library: keep what it
    // reads until coll_finalize
    e->pinned = true;
    if (cd) cd->pinned = true;
    if (xd) xd->pinned = true;
    if (scratch) scratch->pinned = true;
  }

  // ---- enqueue
  if (cks && !cd && !(xd && xd->whole)) {
    // the row kernels add into zeroed slots.  A call being captured into a
    // graph runs later, once per replay: it clears the slots itself and
    // leaves the flag to the calls that run now
    if (!scratch->clean || capturing) {
      he = launch_fill_u64(partial, scratch->cap, 0, stream);
      if (he != hipSuccess) return hip_fail(he, "checksum clear");
    }
    if (!capturing) scratch->clean = false;  // until this call's fold is queued
  }
  TimingEvents* te = nullptr;
  if (opt_timing.load() == 1 && !capturing && !plan.empty()) {
    for (TimingEvents& x : t_timing)
      if (x.dev == dev) te = &x;
    if (!te) {
      TimingEvents x;
      x.dev = dev;
      he = hipEventCreate(&x.start);
      if (he == hipSuccess) he = hipEventCreate(&x.stop);
      if (he != hipSuccess) return hip_fail(he, "hipEventCreate");
      t_timing.push_back(x);
      te = &t_timing.back();
    }
    he = hipEventRecord(te->start, stream);
    if (he != hipSuccess) return hip_fail(he, "hipEventRecord");
  }
  for (const Launch& L : plan) {
    if (L.kind == Launch::COL) {
      ColArgs a{};
      a.work = L.work;
      a.code = L.code;
      a.partial = partial;
      a.p = ptrs;
      he = launch_col(a, N, dt, int(op), L.v.unit, L.v.leaves, L.v.accs, L.v.batched, L.v.capped, L.nt, L.grid, stream);
      if (he != hipSuccess) return hip_fail(he, "column kernel launch");
    } else if (L.kind == Launch::COPY) {
      CopyRowsArgs a{};
      a.rows = xd->d_rows;
      a.partial = copy_partial;
      a.p = ptrs;
      a.row_bytes = xd->row_bytes;
      a.wgs_per_row = xd->wgs_per_row;
      he = launch_copy_rows(a, xd->nrows, cks, L.nt, stream);
      if (he != hipSuccess) return hip_fail(he, "copy kernel launch");
    } else if (L.kind == Launch::ROWS) {
      RowsArgs a{};
      a.list = L.list;
      a.sums = partial;
      a.bases16 = bases16;
      a.p = ptrs;
      for (uint32_t j = 0; j < L.launches; ++j) {
        a.off = L.off + size_t(j) * (L.grid + 1);
        he = launch_rows(a, dt, int(op), cks, L.ntmask, L.fine, L.fwd, L.grid, stream);
        if (he != hipSuccess) return hip_fail(he, "row kernel launch");
      }
    } else {
      PermArgs a{};
      a.items = e->d_items;
      a.steps = e->d_steps;
      a.sums = partial;
      a.nontemporal = L.ntmask;
      a.p = ptrs;
      a.ncols_units = L.ncols;
      a.lg_upl = L.lg;
      for (uint32_t s0 = L.s0; s0 < L.s1; s0 = step_mode ? s0 + 1 : L.s1) {
        a.s0 = s0;
        a.s1 = step_mode ? s0 + 1 : L.s1;
        he = launch_perm(a, L.unit, L.slots, L.hoist, cks, L.grid, stream);
        if (he != hipSuccess) return hip_fail(he, "permutation kernel launch");
      }
    }
  }
  if (te) {
    he = hipEventRecord(te->stop, stream);
    if (he != hipSuccess) return hip_fail(he, "hipEventRecord");
    te->recorded = true;
    t_last_timed = te;
  }
  if (cks && copy_part) {
    // the row kernels' rows after the copy's, then the copy's rows; the copy's
    // slots are not zero for a later row-kernel call
    he = launch_fold_sums(partial + n0 * SUM_LANES, t_sums + n0, uint64_t(b.nrows) - n0, stream);
    if (he == hipSuccess)
      he = launch_col_fold(xd->d_refs, xd->d_row_off, copy_partial, copy_partial + copy_slots, t_sums, n0, stream);
    if (he != hipSuccess) return hip_fail(he, "checksum fold");
    if (!capturing) scratch->clean = false;
  } else if (cks && xd && xd->d_idx) {
    // each block's sum once, then every row takes the sum of the block it
    // carries
    uint64_t* tmp = copy_partial + copy_slots;
    uint64_t* block_sums = tmp + uint64_t(xd->nrows) * COL_FOLD_SLICES;
    he = launch_col_fold(xd->d_refs, xd->d_row_off, copy_partial, tmp, block_sums, xd->nrows, stream);
    if (he == hipSuccess) he = launch_gather_sums(xd->d_idx, block_sums, t_sums, uint64_t(b.nrows), stream);
    if (he != hipSuccess) return hip_fail(he, "checksum fold");
    if (!capturing) scratch->clean = false;
  } else if (cks && (cd || xd)) {
    // every partial slot was written by this call: nothing to clear, but the
    // slots are no longer zero for a row-kernel call
    const uint64_t nslots = cd ? cd->partials : copy_slots;
    he = launch_col_fold(cd ? cd->d_refs : xd->d_refs, cd ? cd->d_row_off : xd->d_row_off,
                         cd ? partial : copy_partial, (cd ? partial : copy_partial) + nslots, t_sums,
                         uint64_t(b.nrows), stream);
    if (he != hipSuccess) return hip_fail(he, "checksum fold");
    if (!capturing) scratch->clean = false;
  } else if (cks) {
    he = launch_fold_sums(partial, t_sums, uint64_t(b.nrows), stream);
    if (he != hipSuccess) return hip_fail(he, "checksum fold");
    if (!capturing) scratch->clean = true;
  }
  if (g_debug.load())
    std::fprintf(stderr, "coll: %s algo %s N %d count %lld dtype-size %d %s steps %lld rows %lld sched_bytes %lld%s\n",
                 kind_name(kind), algo_name(ra), N, (long long)count, sz, inplace ? "in-place" : "out-of-place",
                 (long long)b.counts.steps, (long long)b.counts.rows, (long long)b.counts.hbm_bytes, dbg.c_str());
  t_last = b.counts;
  t_last.moved_bytes = moved;
  t_last.round_trips = (cd || (xd && xd->whole)) ? 1 : b.counts.steps;
  return COLL_OK;
}


// ---- the allocation-free AllReduce -------------------------------------------------

// What a device's allocation-free scratch holds: the tables of the last call
// that uploaded, and where they lie in it (byte offsets).  The host copies
// stay alive as long as they are the scratch's contents.
struct NoallocState {
  bool valid = false;
  std::vector<int64_t> key;       // schedule key, checksum mode, tiles
  ColPlan plan;
  ColTables tables;
  coll_counts_t counts{};         // the schedule's
  size_t nrows = 0;
  uint32_t tiles = 0;
  uint64_t off_code = 0, off_work = 0, off_row_off = 0, off_refs = 0, off_part = 0, off_tmp = 0, end = 0;
};
std::unordered_map<int, NoallocState> g_noalloc;

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

// The layout of a plan's tables in the scratch with `tiles` per work group.
void noalloc_layout(NoallocState& n, size_t nrows, bool cks) {
  uint64_t o = 0;
  n.off_code = o;
  o = align256(o + n.plan.code.size() * sizeof(ColInstr));
  n.off_work = o;
  o = align256(o + n.tables.work.size() * sizeof(ColWork));
  n.off_row_off = o;
  o = align256(o + (cks ? n.tables.row_off.size() * sizeof(uint32_t) : 0));
  n.off_refs = o;
  o = align256(o + (cks ? n.tables.refs.size() * sizeof(ColRef) : 0));
  n.off_part = o;
  o = align256(o + (cks ? n.tables.partials * sizeof(uint64_t) : 0));
  n.off_tmp = o;
  o = align256(o + (cks ? std::max<size_t>(nrows, 1) * COL_FOLD_SLICES * sizeof(uint64_t) : 0));
  n.end = o;
}

coll_status_t run_noalloc(void* const* send, void* const* recv, int N, size_t count_in, coll_dtype_t dtype,
                          coll_op_t op, coll_algo_t algo, int root, int chunks, void* stream_v) {
  const coll_kind_t kind = COLL_K_ALLREDUCE;
  int sz = 0;
  int64_t count = 0;
  bool inplace = true;
  coll_status_t st = check_call(kind, send, recv, N, count_in, dtype, op, algo, root, chunks, sz, count, inplace);
  if (st != COLL_OK) return st;
  t_last = coll_counts_t{};
  if (count == 0) return COLL_OK;
  uint64_t align_or = 0;
  RankPtrs ptrs;
  for (int i = 0; i < N; ++i) {
    ptrs.send[i] = reinterpret_cast<uint64_t>(send[i]);
    ptrs.recv[i] = reinterpret_cast<uint64_t>(inplace ? send[i] : recv[i]);
    align_or |= ptrs.send[i] | ptrs.recv[i];
  }
  for (int i = N; i < COLL_MAX_RANKS; ++i) ptrs.send[i] = ptrs.recv[i] = 0;
  if (align_or % 16) return fail(COLL_ERR_UNSUPPORTED, "the allocation-free AllReduce needs 16-byte aligned rank buffers");
  int dev = 0;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return hip_fail(he, "hipGetDevice");
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
  std::lock_guard<std::mutex> lock(g_mu);
  DevInfo* di = nullptr;
  st = device_info(dev, di);
  if (st != COLL_OK) return st;
  coll_algo_t chosen = algo;
  if (algo == COLL_ALGO_AUTO) {
    st = auto_algo(kind, N, count, sz, root, uint32_t(di->cus), chosen);
    if (st != COLL_OK) return st;
  }
  const coll_algo_t ra = resolve_algo(kind, chosen);
  const bool cks = t_sums != nullptr;
  void* base = nullptr;
  he = noalloc_scratch(&base);
  if (he != hipSuccess) return hip_fail(he, "hipGetSymbolAddress");
  NoallocState& cur = g_noalloc[dev];
  const std::vector<int64_t> key{int64_t(ra), N, count, sz, inplace ? 1 : 0, cks ? 1 : 0, opt_col_tiles.load()};
  if (!cur.valid || cur.key != key) {
    NoallocState n;
    n.key = key;
    Schedule s;
    std::string err;
    st = build_schedule(kind, ra, N, count, 0, 1, s, err);
    if (st != COLL_OK) return fail(st, err);
    n.plan = compile_colplan(s, sz, inplace, cks);
    if (!n.plan.ok)
      return fail(COLL_ERR_UNSUPPORTED, "the allocation-free AllReduce runs the column kernel only: " + n.plan.why);
    fit_col_variant(n.plan, uint32_t(di->cus));
    // tiles per work group: the automatic choice, more while the tables and
    // partial sums exceed the scratch
    uint32_t tiles = opt_col_tiles.load() > 0 ? uint32_t(opt_col_tiles.load()) : auto_col_tiles(n.plan, uint32_t(di->cus));
    for (;;) {
      n.tables = col_tables(n.plan, tiles, s.rows.size());
      noalloc_layout(n, s.rows.size(), cks);
      if (n.end <= COLL_NOALLOC_SCRATCH_BYTES || tiles >= 65535) break;
      tiles = std::min<uint32_t>(65535, tiles * 2);
    }
    if (n.end > COLL_NOALLOC_SCRATCH_BYTES)
      return fail(COLL_ERR_INVALID_ARG, "the allocation-free AllReduce needs " + std::to_string(n.end) +
                                            " bytes of scratch, more than COLL_NOALLOC_SCRATCH_BYTES");
    n.tiles = tiles;
    n.counts = count_schedule(s, sz);
    n.nrows = s.rows.size();
    n.valid = true;
    if (cks && n.nrows > t_sums_cap) return fail(COLL_ERR_INVALID_ARG, "checksum buffer smaller than the schedule");
    // the scratch's old tables may still be read by work queued on this
    // stream: wait for it before replacing them (and their host copies)
    if (cur.valid) {
      he = hipStreamSynchronize(stream);
      if (he != hipSuccess) return hip_fail(he, "hipStreamSynchronize");
    }
    cur = NoallocState{};
    char* b = static_cast<char*>(base);
    auto put = [&](uint64_t off, const void* src, size_t bytes) {
      return bytes ? hipMemcpyAsync(b + off, src, bytes, hipMemcpyHostToDevice, stream) : hipSuccess;
    };
    he = put(n.off_code, n.plan.code.data(), n.plan.code.size() * sizeof(ColInstr));
    if (he == hipSuccess) he = put(n.off_work, n.tables.work.data(), n.tables.work.size() * sizeof(ColWork));
    if (he == hipSuccess && cks) he = put(n.off_row_off, n.tables.row_off.data(), n.tables.row_off.size() * sizeof(uint32_t));
    if (he == hipSuccess && cks) he = put(n.off_refs, n.tables.refs.data(), n.tables.refs.size() * sizeof(ColRef));
    if (he != hipSuccess) return hip_fail(he, "hipMemcpyAsync");
    cur = std::move(n);
  }
  if (cks && cur.nrows > t_sums_cap) return fail(COLL_ERR_INVALID_ARG, "checksum buffer smaller than the schedule");
  char* b = static_cast<char*>(base);
  ColArgs a{};
  a.work = reinterpret_cast<const ColWork*>(b + cur.off_work);
  a.code = reinterpret_cast<const ColInstr*>(b + cur.off_code);
  a.partial = cks ? reinterpret_cast<uint64_t*>(b + cur.off_part) : nullptr;
  a.p = ptrs;
  const uint64_t footprint = uint64_t(N) * uint64_t(count) * uint64_t(sz) * (inplace ? 1u : 2u);
  const bool nt = opt_nt.load() < 0 ? footprint > COL_NT_BYTES : (uint32_t(opt_nt.load()) & (NT_SRC | NT_DST)) != 0;
  const int dt = int(dtype) == COLL_INT32 ? DT_I32 : int(dtype) == COLL_UINT8 ? DT_U8
               : int(dtype) == COLL_FLOAT32 ? DT_F32 : DT_BF16;
  const uint32_t grid = uint32_t(cur.tables.work.size());
  if (grid) {
    he = launch_col(a, N, dt, int(op), cur.plan.v.unit, cur.plan.v.leaves, cur.plan.v.accs, cur.plan.v.batched,
                    cur.plan.v.capped, nt,
                     grid, stream);
    if (he != hipSuccess) return hip_fail(he, "column kernel launch");
  }
  if (cks) {
    he = launch_col_fold(reinterpret_cast<const ColRef*>(b + cur.off_refs),
                         reinterpret_cast<const uint32_t*>(b + cur.off_row_off),
                         reinterpret_cast<const uint64_t*>(b + cur.off_part), reinterpret_cast<uint64_t*>(b + cur.off_tmp),
                         t_sums, uint64_t(cur.nrows), stream);
    if (he != hipSuccess) return hip_fail(he, "checksum fold");
  }
  t_last = cur.counts;
  t_last.moved_bytes = int64_t(cur.plan.moved_bytes);
  t_last.round_trips = 1;
  return COLL_OK;
}
}  // namespace

// the calls' error reporting, for the calibration entry points (calib.cpp)
coll_status_t report_error(coll_status_t st, const char* msg) { return fail(st, msg); }
coll_status_t report_hip_error(hipError_t e, const char* what) { return hip_fail(e, what); }

}  // namespace coll

using namespace coll;

extern "C" {

#define COLL_ENTRY(name, kind)                                                                                 \
  coll_status_t name(void* const* sendbufs, void* const* recvbufs, int nranks, size_t count, coll_dtype_t dtype, \
                     coll_op_t op, coll_algo_t algo, int root, int chunks, void* stream) {                        \
    try {                                                                                                       \
      return run(kind, sendbufs, recvbufs, nranks, count, dtype, op, algo, root, chunks, stream);              \
    } catch (const std::bad_alloc&) {                                                                           \
      return fail(COLL_ERR_NO_MEMORY, "host allocation failed");                                               \
    } catch (...) {                                                                                             \
      return fail(COLL_ERR_INVALID_ARG, "unexpected host exception");                                         \
    }                                                                                                           \
  }

COLL_ENTRY(coll_allreduce, COLL_K_ALLREDUCE)
COLL_ENTRY(coll_reducescatter, COLL_K_REDUCESCATTER)
COLL_ENTRY(coll_allgather, COLL_K_ALLGATHER)
COLL_ENTRY(coll_broadcast, COLL_K_BROADCAST)
COLL_ENTRY(coll_scatter, COLL_K_SCATTER)
COLL_ENTRY(coll_gather, COLL_K_GATHER)
COLL_ENTRY(coll_alltoall, COLL_K_ALLTOALL)
COLL_ENTRY(coll_reduce, COLL_K_REDUCE)

coll_status_t coll_allreduce_noalloc(void* const* sendbufs, void* const* recvbufs, int nranks, size_t count,
                                     coll_dtype_t dtype, coll_op_t op, coll_algo_t algo, int root, int chunks,
                                     void* stream) {
  try {
    return run_noalloc(sendbufs, recvbufs, nranks, count, dtype, op, algo, root, chunks, stream);
  } catch (const std::bad_alloc&) {
    return fail(COLL_ERR_NO_MEMORY, "host allocation failed");
  } catch (...) {
    return fail(COLL_ERR_INVALID_ARG, "unexpected host exception");
  }
}

coll_status_t coll_plan(coll_kind_t kind, coll_algo_t algo, int nranks, size_t count, coll_dtype_t dtype, int root,
                        int chunks, coll_row_t* rows, size_t* nrows, coll_counts_t* counts) {
  try {
    const int sz = elem_size(dtype);
    if (!sz) return fail(COLL_ERR_INVALID_ARG, "unknown dtype");
    if (!nrows) return fail(COLL_ERR_INVALID_ARG, "nrows is NULL");
    if (count > (size_t(1) << 44) / size_t(sz)) return fail(COLL_ERR_INVALID_ARG, "count too large");
    Schedule s;
    std::string err;
    if (algo == COLL_ALGO_AUTO) {
      coll_status_t st = build_schedule(kind, COLL_ALGO_DEFAULT, nranks, 0, root, 1, s, err);
      if (st != COLL_OK) return fail(st, err);
      const std::function<PlannedCost(const Schedule&)> cost = [&](const Schedule& x) {
        return planned_cost(x, sz, PLAN_CUS);
      };
      st = choose_algo(kind, nranks, int64_t(count), sz, root, cost_model(), algo, err, &cost);
      if (st != COLL_OK) return fail(st, err);
      chunks = 1;
    }
    coll_status_t st = build_schedule(kind, algo, nranks, int64_t(count), root, chunks, s, err);
    if (st != COLL_OK) return fail(st, err);
    const size_t cap = *nrows;
    *nrows = s.rows.size();
    if (counts) {
      *counts = count_schedule(s, sz);
      const PlannedCost pc = planned_cost(s, sz, PLAN_CUS);
      counts->moved_bytes = pc.bytes;
      counts->round_trips = pc.round_trips;
    }
    if (rows) {
      if (cap < s.rows.size()) return fail(COLL_ERR_INVALID_ARG, "row capacity too small");
      for (size_t i = 0; i < s.rows.size(); ++i) {
        const Row& r = s.rows[i];
        coll_row_t& o = rows[i];
        o.step = r.step;
        o.src = r.src;
        o.dst = r.dst;
        o.reduce = r.reduce;
        o.local = r.local;
        o.from_send = r.from_send;
        o.staged = r.staged;
        o.src_off = r.src_off;
        o.dst_off = r.dst_off;
        o.n = r.n;
      }
    }
    return COLL_OK;
  } catch (const std::bad_alloc&) {
    return fail(COLL_ERR_NO_MEMORY, "host allocation failed");
  }
}

coll_status_t coll_get_stats(coll_counts_t* last) {
  if (!last) return fail(COLL_ERR_INVALID_ARG, "NULL");
  *last = t_last;
  return COLL_OK;
}

coll_status_t coll_set_checksums(uint64_t* dev_sums, size_t capacity) {
  if (dev_sums && capacity == 0) return fail(COLL_ERR_INVALID_ARG, "capacity is 0");
  t_sums = dev_sums;
  t_sums_cap = dev_sums ? capacity : 0;
  return COLL_OK;
}

coll_status_t coll_set_option(coll_option_t key, int64_t value) {
  switch (key) {
    case COLL_OPT_EXEC:
      if (value < 0 || value > 2) return fail(COLL_ERR_INVALID_ARG, "exec mode is 0, 1 or 2");
      opt_exec = value;
      return COLL_OK;
    case COLL_OPT_COL_TILES:
      if (value < 0 || value > 65535) return fail(COLL_ERR_INVALID_ARG, "column tiles in [0, 65535]");
      opt_col_tiles = value;
      return COLL_OK;
    case COLL_OPT_TIMING:
      if (value != 0 && value != 1) return fail(COLL_ERR_INVALID_ARG, "timing is 0 or 1");
      opt_timing = value;
      return COLL_OK;
    case COLL_OPT_REVERSE:
      opt_reverse = value ? 1 : 0;
      return COLL_OK;
    case COLL_OPT_MODEL_ALPHA_NS:
      if (value < 0 || value > 1000000000) return fail(COLL_ERR_INVALID_ARG, "alpha out of range");
      opt_alpha_ns = value;
      return COLL_OK;
    case COLL_OPT_MODEL_BETA_GBPS:
      if (value < 1 || value > 1000000000) return fail(COLL_ERR_INVALID_ARG, "beta out of range");
      opt_beta_gbps = value;
      return COLL_OK;
    case COLL_OPT_GROUP_TILES:
      if (value < 0 || value > 64) return fail(COLL_ERR_INVALID_ARG, "group tiles in [0, 64]");
      opt_group = value;
      return COLL_OK;
    case COLL_OPT_MAX_GRID:
      if (value < 0 || value > (int64_t(1) << 20)) return fail(COLL_ERR_INVALID_ARG, "grid cap out of range");
      opt_grid = value;
      return COLL_OK;
    case COLL_OPT_NONTEMPORAL:
      if (value < -1 || value > 7) return fail(COLL_ERR_INVALID_ARG, "nontemporal mask in [-1, 7]");
      opt_nt = value;
      return COLL_OK;
    case COLL_OPT_CACHE_BYTES:
      if (value < 0) return fail(COLL_ERR_INVALID_ARG, "cache budget below 0");
      opt_cache_bytes = value;
      return COLL_OK;
    case COLL_OPT_A2A_DIRECT:
      if (value != 0 && value != 1) return fail(COLL_ERR_INVALID_ARG, "a2a_direct is 0 or 1");
      opt_a2a_direct = value;
      return COLL_OK;
  }
  return fail(COLL_ERR_INVALID_ARG, "unknown option");
}

coll_status_t coll_last_kernel_ms(float* ms) {
  if (!ms) return fail(COLL_ERR_INVALID_ARG, "ms is NULL");
  TimingEvents* te = t_last_timed;
  if (!te || !te->recorded) return fail(COLL_ERR_INVALID_ARG, "no call on this thread was timed");
  hipError_t he = hipEventSynchronize(te->stop);
  if (he == hipSuccess) he = hipEventElapsedTime(ms, te->start, te->stop);
  if (he != hipSuccess) return hip_fail(he, "hipEventElapsedTime");
  return COLL_OK;
}

coll_status_t coll_check(void* stream) {
  hipError_t he = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
  if (he == hipSuccess) he = hipGetLastError();
  if (he != hipSuccess) return hip_fail(he, "stream work");
  return COLL_OK;
}

coll_status_t coll_get_option(coll_option_t key, int64_t* value) {
  if (!value) return fail(COLL_ERR_INVALID_ARG, "value is NULL");
  switch (key) {
    case COLL_OPT_EXEC: *value = opt_exec.load(); return COLL_OK;
    case COLL_OPT_GROUP_TILES: *value = opt_group.load(); return COLL_OK;
    case COLL_OPT_MAX_GRID: *value = opt_grid.load(); return COLL_OK;
    case COLL_OPT_NONTEMPORAL: *value = opt_nt.load(); return COLL_OK;
    case COLL_OPT_REVERSE: *value = opt_reverse.load(); return COLL_OK;
    case COLL_OPT_MODEL_ALPHA_NS: *value = opt_alpha_ns.load(); return COLL_OK;
    case COLL_OPT_MODEL_BETA_GBPS: *value = opt_beta_gbps.load(); return COLL_OK;
    case COLL_OPT_CACHE_BYTES: *value = opt_cache_bytes.load(); return COLL_OK;
    case COLL_OPT_COL_TILES: *value = opt_col_tiles.load(); return COLL_OK;
    case COLL_OPT_TIMING: *value = opt_timing.load(); return COLL_OK;
    case COLL_OPT_A2A_DIRECT: *value = opt_a2a_direct.load(); return COLL_OK;
  }
  return fail(COLL_ERR_INVALID_ARG, "unknown option");
}

coll_status_t coll_cache_info(int64_t* schedules, int64_t* device_bytes) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (schedules) *schedules = int64_t(g_cache.size());
  if (device_bytes) *device_bytes = int64_t(g_cache_bytes);
  return COLL_OK;
}

const char* coll_status_string(coll_status_t s) {
  switch (s) {
    case COLL_OK: return "COLL_OK";
    case COLL_ERR_INVALID_ARG: return "COLL_ERR_INVALID_ARG";
    case COLL_ERR_UNSUPPORTED: return "COLL_ERR_UNSUPPORTED";
    case COLL_ERR_HIP: return "COLL_ERR_HIP";
    case COLL_ERR_NO_MEMORY: return "COLL_ERR_NO_MEMORY";
  }
  return "unknown status";
}

const char* coll_last_error(void) { return t_err.c_str(); }

void coll_finalize(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  // queued calls may still read the tables: wait for every device that holds some
  int cur = 0;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  std::vector<int> devs;
  for (auto& kv : g_cache)
    if (std::find(devs.begin(), devs.end(), kv.second->dev) == devs.end()) devs.push_back(kv.second->dev);
  for (int d : devs)
    if (hipSetDevice(d) == hipSuccess) (void)hipDeviceSynchronize();
  if (have_cur && !devs.empty()) (void)hipSetDevice(cur);
  for (auto& kv : g_cache) {
    kv.second->pinned = false;
    for (DevList& l : kv.second->lists) l.pinned = false;
    for (ColDev& c : kv.second->col) c.pinned = false;
    free_entry(*kv.second);
  }
  for (SumScratch& s : g_sum_scratch) {
    s.pinned = false;
    free_sum_scratch(s);
  }
  g_sum_scratch.clear();
  // buffers that captured graphs kept: the caller has stopped replaying them
  int ndev = 0;
  if (!g_retired.empty() && hipGetDeviceCount(&ndev) == hipSuccess)
    for (int d = 0; d < ndev; ++d)
      if (hipSetDevice(d) == hipSuccess) (void)hipDeviceSynchronize();
  if (have_cur && !g_retired.empty()) (void)hipSetDevice(cur);
  for (void* p : g_retired) (void)hipFree(p);
  g_retired.clear();
  g_cache.clear();
  g_cache_bytes = 0;
  g_occ.clear();
  g_dev.clear();
}

}  // extern "C"

namespace {

// Initial option values from the environment (read once, when the library is
// loaded): COLL_EXEC, COLL_GROUP_TILES, COLL_MAX_GRID, COLL_NONTEMPORAL,
// COLL_REVERSE, COLL_MODEL_ALPHA_NS, COLL_MODEL_BETA_GBPS, COLL_CACHE_BYTES,
// COLL_COL_TILES, COLL_TIMING (integers, as for coll_set_option; an invalid one is reported on stderr and
// ignored), and COLL_DEBUG (set and not "0": one line per call on stderr).
struct EnvOptions {
  EnvOptions() {
    static const struct {
      const char* name;
      coll_option_t key;
    } vars[] = {{"COLL_EXEC", COLL_OPT_EXEC},
                {"COLL_GROUP_TILES", COLL_OPT_GROUP_TILES},
                {"COLL_MAX_GRID", COLL_OPT_MAX_GRID},
                {"COLL_NONTEMPORAL", COLL_OPT_NONTEMPORAL},
                {"COLL_REVERSE", COLL_OPT_REVERSE},
                {"COLL_MODEL_ALPHA_NS", COLL_OPT_MODEL_ALPHA_NS},
                {"COLL_MODEL_BETA_GBPS", COLL_OPT_MODEL_BETA_GBPS},
                {"COLL_CACHE_BYTES", COLL_OPT_CACHE_BYTES},
                {"COLL_COL_TILES", COLL_OPT_COL_TILES},
                {"COLL_TIMING", COLL_OPT_TIMING},
                {"COLL_A2A_DIRECT", COLL_OPT_A2A_DIRECT}};
    for (const auto& v : vars) {
      const char* s = std::getenv(v.name);
      if (!s || !*s) continue;
      char* end = nullptr;
      const long long x = std::strtoll(s, &end, 10);
      if (*end != '\0' || coll_set_option(v.key, int64_t(x)) != COLL_OK)
        std::fprintf(stderr, "coll: ignoring %s=%s\n", v.name, s);
    }
    const char* d = std::getenv("COLL_DEBUG");
    coll::g_debug = d && *d && std::strcmp(d, "0") != 0;
  }
};
EnvOptions g_env_options;

}  // namespace
