/*
 * coll.h — collective-communication schedules executed over N virtual ranks
 * whose buffers all sit in one MI355X's HBM.
 *
 * Every collective is run as the step-by-step schedule its algorithm defines:
 * in each step some ranks "send" a chunk to another rank, which either stores
 * it (copy) or reduces it into its own chunk (recv_and_reduce).  On one GPU a
 * send is a device-to-device move performed by this library's HIP kernels.
 *
 * Sources (pages, by title and section):
 *   [P1] "一对多通信：Broadcast 与 Scatter" — Broadcast / Scatter semantics,
 *        binomial and chunked-pipeline Broadcast, binomial Scatter, Gather.
 *   [P2] HCCL blog on Ring / Mesh / Tree AllReduce — the hccl_allreduce call
 *        (element count, data type, SUM / MAX / MIN, in place when sendbuf ==
 *        recvbuf, stream-ordered), and the Ring chunk walk.
 *   [P3] "集合通信算法延迟公式" — Ring / Recursive Halving-Doubling / Double
 *        Binary Tree AllReduce, Ring AllGather / ReduceScatter, Pairwise and
 *        Bruck AllToAll, busbw coefficients.
 *
 * Conventions shared by all eight collective calls
 *   sendbufs[i], recvbufs[i]  device pointers of virtual rank i, each holding
 *                `count` elements of `dtype` (the pages' message size M =
 *                count * sizeof(dtype) bytes per rank).  Pointers must be
 *                aligned to the element size; 16-byte alignment takes the
 *                128-bit load/store path.
 *   recvbufs == NULL, or recvbufs[i] == sendbufs[i] for every i: in place.
 *                Mixing the two, or any overlap between distinct rank buffers,
 *                is COLL_ERR_INVALID_ARG.  AllToAll must be out of place.
 *   count == 0   nothing is read or written: once the scalar arguments are
 *                valid the call returns COLL_OK without looking at the rank
 *                pointers (no NULL, alignment or aliasing check; empty
 *                framework tensors may all share one pointer, often NULL).
 *   chunk c of a rank buffer = elements [c*count/N, (c+1)*count/N) (floor).
 *   op     ignored by collectives that do not reduce.
 *   root   used by broadcast / scatter / gather / reduce only; 0 <= root < N.
 *   chunks pipeline chunk count k for COLL_ALGO_CHAIN_PIPE,
 *          COLL_ALGO_BINOMIAL_PIPE and COLL_ALGO_BIDIR_RING (1 <= k <= count);
 *          ignored otherwise.
 *   stream a hipStream_t; the work is enqueued on it and the call returns
 *          without waiting (stream-ordered, like hccl_allreduce's stream).
 *
 * Ownership: the caller owns every buffer and keeps it alive until the stream
 * work has finished.  The library never allocates, frees or retains user
 * memory; it owns only its schedule cache (host and device copies) and, while
 * checksums are on, its partial checksum slots, all freed by coll_finalize().
 *
 * Errors: every argument is checked on the host before anything is enqueued,
 * so an error return leaves no partial work.  No exception crosses the ABI.
 * A failing HIP call returns COLL_ERR_HIP with the HIP error text in
 * coll_last_error() (thread-local).
 */
#ifndef COLL_H
#define COLL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  COLL_OK = 0,
  COLL_ERR_INVALID_ARG = 1,  /* bad pointer, size, root, chunks, aliasing          */
  COLL_ERR_UNSUPPORTED = 2,  /* algorithm not defined for this collective or N    */
  COLL_ERR_HIP = 3,          /* a HIP runtime call failed                         */
  COLL_ERR_NO_MEMORY = 4     /* host or device allocation for the schedule failed */
} coll_status_t;

typedef enum { COLL_INT32 = 0, COLL_UINT8 = 1, COLL_FLOAT32 = 2, COLL_BFLOAT16 = 3 } coll_dtype_t;

/* dst <- dst (+) src per element.  int32 / uint8 sums wrap; float32 is one
 * IEEE binary32 add (round to nearest even, subnormals kept); bfloat16 widens
 * both operands to binary32, adds once and rounds to nearest even (NaN ->
 * 0x7FC0) after every row.  max / min pick src when it compares greater /
 * smaller, else keep dst.  [P2] hccl_allreduce parameter list (SUM/MAX/MIN). */
typedef enum { COLL_SUM = 0, COLL_MAX = 1, COLL_MIN = 2 } coll_op_t;

typedef enum {
  COLL_ALGO_DEFAULT = 0,       /* ring / binomial / pairwise for the collective */
  COLL_ALGO_RING = 1,          /* [P3] Ring AllReduce, Ring AllGather / ReduceScatter, Ring
                                  AllToAll (store-and-forward between neighbours)              */
  COLL_ALGO_RHD = 2,           /* [P3] Recursive Halving-Doubling; ReduceScatter / AllGather need
                                  N = 2^n; AllReduce folds the surplus ranks of any N first     */
  COLL_ALGO_DBT = 3,           /* [P3] Double Binary Tree (any N)                              */
  COLL_ALGO_BINOMIAL = 4,      /* [P1] binomial-tree Broadcast / Scatter / Gather              */
  COLL_ALGO_CHAIN_PIPE = 5,    /* [P1] chunked chain pipeline Broadcast (k = 1: chain)         */
  COLL_ALGO_BINOMIAL_PIPE = 6, /* [P1] chunked binomial-tree pipeline Broadcast (k = 1: tree)  */
  COLL_ALGO_PAIRWISE = 7,      /* [P3] Pairwise AllToAll, N-1 rounds                           */
  COLL_ALGO_BRUCK = 8,         /* [P3] Bruck AllToAll, ceil(log2 N) rounds plus rotations      */
  COLL_ALGO_LINEAR = 9,        /* [P1] naive Scatter: the root sends each chunk directly      */
  COLL_ALGO_SCATTER_ALLGATHER = 10, /* [P1] Broadcast as binomial Scatter + Ring AllGather    */
  COLL_ALGO_AUTO = 11,         /* the candidate with the least predicted time, t = round_trips *
                                  alpha + moved_bytes / beta (coll_counts_t; [P3]'s alpha-beta
                                  model with this device's fitted constants, COLL_OPT_MODEL_*,
                                  over what the kernels that run it take); ties go to the
                                  first of: AllReduce DBT, RHD, Ring; ReduceScatter / AllGather
                                  RHD, Ring; Broadcast binomial, chain, Scatter+AllGather,
                                  bidirectional ring; Scatter binomial, linear; AllToAll
                                  Pairwise, Bruck, Ring.  `chunks` is ignored (one GPU moves the
                                  same bytes for any k). */
  COLL_ALGO_BIDIR_RING = 12    /* [P1] Broadcast over both directions of a ring at once (SCCL's
                                  4-chip scheme, any N), pipelined in `chunks` chunks */
} coll_algo_t;

typedef enum {
  COLL_K_ALLREDUCE = 0, COLL_K_REDUCESCATTER = 1, COLL_K_ALLGATHER = 2, COLL_K_BROADCAST = 3,
  COLL_K_SCATTER = 4, COLL_K_GATHER = 5, COLL_K_ALLTOALL = 6, COLL_K_REDUCE = 7
} coll_kind_t;

/* Largest N the kernels accept (all rank pointers travel as kernel arguments). */
#define COLL_MAX_RANKS 128

/* ------------------------------------------------------------------------- */
/* The eight collectives.  Same parameters for all; see the conventions above. */

/* [P3] AllReduce: every rank ends with the elementwise reduction over ranks.
 * Input all of buf_i; output all of buf_i.  algo: RING (default; [P3] Ring
 * AllReduce：带宽最优, eq:model-algo-ring-ar: ReduceScatter then AllGather,
 * 2(N-1) steps), RHD ([P3] Recursive Halving-Doubling, eq:model-algo-rhd-ar:
 * 2 log2 N steps), DBT ([P3] Double Binary Tree, eq:model-algo-dbt-ar). */
coll_status_t coll_allreduce(void* const* sendbufs, void* const* recvbufs, int nranks, size_t count,
                             coll_dtype_t dtype, coll_op_t op, coll_algo_t algo, int root, int chunks,
                             void* stream);

/* [P3] ReduceScatter: rank i ends with chunk i of the reduction; its other
 * chunks are left unspecified.  algo: RING (default; [P3] Ring
 * ReduceScatter, eq:model-algo-ring-reducescatter: N-1 steps of M/N), RHD
 * ([P3] Recursive Halving-Doubling, eq:model-algo-rhd-rs: log2 N halving
 * rounds; N = 2^n). */
coll_status_t coll_reducescatter(void* const* sendbufs, void* const* recvbufs, int nranks, size_t count,
                                 coll_dtype_t dtype, coll_op_t op, coll_algo_t algo, int root, int chunks,
                                 void* stream);

/* [P3] AllGather: rank i contributes chunk i of its buffer; every rank ends
 * with all N chunks.  algo: RING (default; [P3] Ring AllGather,
 * eq:model-algo-ring-allgather: N-1 steps of M/N), RHD ([P3] Recursive
 * Halving-Doubling, eq:model-algo-rhd-ag: log2 N doubling rounds; N = 2^n). */
coll_status_t coll_allgather(void* const* sendbufs, void* const* recvbufs, int nranks, size_t count,
                             coll_dtype_t dtype, coll_op_t op, coll_algo_t algo, int root, int chunks,
                             void* stream);

/* [P1] Broadcast (eq:onetoall-bcast-semantic): every buffer ends equal to the
 * root's.  algo: BINOMIAL (default), CHAIN_PIPE, BINOMIAL_PIPE with `chunks`,
 * SCATTER_ALLGATHER (binomial Scatter, then Ring AllGather; [P1] "Broadcast 与
 * Scatter 的关系"), BIDIR_RING with `chunks` ([P1] "SCCL 的 Broadcast 实现":
 * the root sends clockwise and counter-clockwise at once; floor(N/2) + k - 1
 * steps of M/k bytes). */
coll_status_t coll_broadcast(void* const* sendbufs, void* const* recvbufs, int nranks, size_t count,
                             coll_dtype_t dtype, coll_op_t op, coll_algo_t algo, int root, int chunks,
                             void* stream);

/* [P1] Scatter (eq:onetoall-scatter-semantic): the root's chunk i lands in
 * chunk i of rank i; other chunks of non-root buffers are staging space and
 * left unspecified.  algo: BINOMIAL (default), LINEAR (eq:onetoall-scatter-naive). */
coll_status_t coll_scatter(void* const* sendbufs, void* const* recvbufs, int nranks, size_t count,
                           coll_dtype_t dtype, coll_op_t op, coll_algo_t algo, int root, int chunks,
                           void* stream);

/* [P1] Gather (eq:onetoall-gather-scatter-duality, Scatter reversed): chunk i
 * of rank i lands in chunk i of the root; non-root buffers are left
 * unspecified.  algo: BINOMIAL. */
coll_status_t coll_gather(void* const* sendbufs, void* const* recvbufs, int nranks, size_t count,
                          coll_dtype_t dtype, coll_op_t op, coll_algo_t algo, int root, int chunks,
                          void* stream);

/* [P3] Tree Reduce (eq:model-algo-reduce-tree, the mirror of the tree
 * Broadcast): the root ends with the elementwise reduction over ranks; the
 * other buffers hold partial results (unspecified).  algo: BINOMIAL. */
coll_status_t coll_reduce(void* const* sendbufs, void* const* recvbufs, int nranks, size_t count,
                          coll_dtype_t dtype, coll_op_t op, coll_algo_t algo, int root, int chunks,
                          void* stream);

/* [P3] AllToAll (AllToAll 算法怎么选): send_i holds N blocks of count/N
 * elements, block j meant for rank j; afterwards block i of recv_j = block j
 * of send_i.  Out of place only; count must be a multiple of N.  algo:
 * PAIRWISE (default; eq:model-algo-a2a-pairwise: in round k rank i sends to
 * i+k, N-1 rounds), BRUCK (eq:model-algo-a2a-bruck: ceil(log2 N) rounds with
 * local rotations), RING (eq:model-algo-a2a-ring: N-1 rounds between
 * neighbours i -> i+1; round t forwards the N-t blocks still in transit, so
 * each link carries (N-1)M/2 bytes in all, against the printed formula's
 * (N-1)M/N).  Every row of these schedules moves one whole block, so with
 * blocks of a multiple of 16 bytes on 16-byte aligned buffers a call runs as
 * one direct copy of every block whatever the algorithm (one launch,
 * coll_get_stats().round_trips 1, moved_bytes 2 * N * count * element size),
 * the rows' checksums those of the blocks they carry (COLL_OPT_A2A_DIRECT). */
coll_status_t coll_alltoall(void* const* sendbufs, void* const* recvbufs, int nranks, size_t count,
                            coll_dtype_t dtype, coll_op_t op, coll_algo_t algo, int root, int chunks,
                            void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): an
 * AllReduce with the same arguments, results and row checksums as
 * coll_allreduce, that calls no hipMalloc, hipFree or other allocating
 * routine.  It runs the column kernel only, with its programs, work table and
 * checksum partial sums in a library array of COLL_NOALLOC_SCRATCH_BYTES per
 * GPU (held until the process ends); the schedule is compiled on the host.
 * The array keeps the last call's tables: a call for the same schedule,
 * options and checksum mode uploads nothing, any other uploads its tables
 * (hipMemcpyAsync on `stream`) and first waits for `stream`.  Calls that
 * overlap on one GPU (other streams or threads) race on the array.
 * Errors: as coll_allreduce; COLL_ERR_UNSUPPORTED when the column kernel does
 * not run the call (rank buffers not 16-byte aligned, or more than 64 ranks,
 * whose programs no kernel variant holds); COLL_ERR_INVALID_ARG when its
 * tables and partial
 * sums do not fit the array even with the fewest work groups (the message
 * says how many bytes they need).  Not in coll_get_stats' schedule cache. */
#define COLL_NOALLOC_SCRATCH_BYTES (16u << 20)
coll_status_t coll_allreduce_noalloc(void* const* sendbufs, void* const* recvbufs, int nranks, size_t count,
                                     coll_dtype_t dtype, coll_op_t op, coll_algo_t algo, int root, int chunks,
                                     void* stream);

/* ------------------------------------------------------------------------- */
/* Schedules and statistics (host only; no GPU needed). */

/* One row of a schedule: in step `step`, rank `src` sends n elements at
 * element offset src_off to rank `dst`, which stores them at dst_off
 * (reduce = 0) or reduces them into its own elements there (reduce = 1).
 * local: a rank-internal move (AllToAll rearrangement), not a counted step.
 * from_send: the source is the send buffer (AllToAll).  staged: a step that
 * permutes in place; all its reads happen before its writes. */
typedef struct {
  int32_t step, src, dst;
  uint8_t reduce, local, from_send, staged;
  int64_t src_off, dst_off, n;
} coll_row_t;

/* steps: counted communication steps (the pages' closed forms, e.g. 2(N-1)
 * for Ring AllReduce); rows: schedule rows; crit_bytes: per step the largest
 * byte total on one (src, dst) edge, summed over steps (the beta term of
 * [P3]'s alpha-beta model); hbm_bytes: bytes the rows read and write (copy
 * 2*n*size, reduce 3*n*size); moved_bytes: the part of hbm_bytes that goes
 * through memory.  The column kernel (COLL_OPT_EXEC) loads each input its
 * programs need once and stores each defined output once: an in-place
 * AllReduce moves 2NM for every algorithm, ReduceScatter (N+1)M, AllGather
 * and Broadcast NM.  The row kernel moves the schedule's bytes, less the
 * operands its forwarding variant passes from step to step in registers and
 * the stores it skips (lists over 8 MiB or more of columns whose entries
 * mostly form chains, as Ring's do).  round_trips: dependent memory round
 * trips of the kernels: 1 for the column kernel, a step each for the row
 * kernel (the alpha term of COLL_ALGO_AUTO). */
typedef struct { int64_t steps, rows, crit_bytes, hbm_bytes, moved_bytes, round_trips; } coll_counts_t;

/* Build the in-place schedule of a collective.  rows may be NULL; *nrows is
 * the capacity on input and the number of rows on output (COLL_ERR_INVALID_ARG
 * if the capacity is too small, with *nrows set to what is needed).  counts
 * may be NULL; its moved_bytes is planned for an in-place call on 16-byte
 * aligned buffers with the current options on MI355X's 256 compute units.
 * Validation as for the collective calls (without pointers).  COLL_ALGO_AUTO
 * picks the candidate that minimises steps * alpha + moved_bytes / beta
 * (COLL_OPT_MODEL_ALPHA_NS / _BETA_GBPS), planned so here and for the calling
 * device's compute units in a collective call. */
coll_status_t coll_plan(coll_kind_t kind, coll_algo_t algo, int nranks, size_t count, coll_dtype_t dtype,
                        int root, int chunks, coll_row_t* rows, size_t* nrows, coll_counts_t* counts);

/* Counts of the last successful collective call on this thread, as executed
 * (an out-of-place call adds local copies to hbm_bytes; moved_bytes counts
 * what the launched kernels moved). */
coll_status_t coll_get_stats(coll_counts_t* last);

/* Per-row checksums.  When `dev_sums` is non-NULL (a device array of
 * `capacity` uint64), every later collective call on this thread writes
 * dev_sums[0 .. rows), stream-ordered: for schedule row r (in coll_plan's
 * order), the sum modulo 2^64 of the little-endian uint32 words of the row's
 * destination region right after the row (words counted from the region's
 * first byte, the last one zero-padded).  The kernels accumulate into 64
 * partial slots per row in a library buffer kept per (device, dev_sums),
 * allocated on the first call that needs it or needs more (outside graph
 * capture, like the schedule), and a last kernel folds them into dev_sums;
 * calls that share dev_sums must be ordered with each other.  A call with more
 * rows than `capacity` fails with COLL_ERR_INVALID_ARG.  NULL switches
 * checksums off. */
coll_status_t coll_set_checksums(uint64_t* dev_sums, size_t capacity);

/* Process-wide execution options (defaults in brackets).
 * COLL_OPT_EXEC            0: automatic [0]: every collective but AllToAll, on
 *                          16-byte aligned buffers, runs in the column kernel
 *                          (its schedule compiled per column segment, see
 *                          above), and an AllToAll whose blocks are
 *                          multiples of 16 bytes in one direct copy
 *                          (COLL_OPT_A2A_DIRECT); where neither applies,
 *                          one row-kernel
 *                          launch runs every step of the call (each work
 *                          group owns fixed columns, so the steps need no
 *                          synchronisation between work groups).
 *                          1: the row kernel, one launch per step (the
 *                          launches order the steps).
 *                          2: the row kernel, one launch for every step.
 * COLL_OPT_GROUP_TILES     4 KiB column tiles per work-group column group, 1..64
 *                          [0: automatic.  Column spaces of 8 MiB or more:
 *                          int32 / fp32 / bf16 reductions whose groups see two
 *                          or more rows per step (trees, halving-doubling),
 *                          and copy-only schedules over 16 or more ranks that
 *                          do, use 4-tile groups on 2 work groups per CU, each
 *                          work group taking its groups one at a time; other
 *                          schedules one group per work group, 8 tiles; 4 for
 *                          uint8 reductions, where 8-tile groups would number
 *                          fewer than 2 per CU, and where rows start or end
 *                          no more often than every 8 MiB over 64 MiB of
 *                          columns or more (reductions), or every 16 MiB over
 *                          128 MiB or more (copies), on average, in calls
 *                          without row checksums.  Smaller column spaces: up to 8
 *                          tiles over a grid of the work groups that fit on
 *                          the device at once.  Whenever every group has a work
 *                          group of its own, groups are also split where a row
 *                          starts or ends inside them].
 * COLL_OPT_MAX_GRID        cap on work groups per launch, up to 2^20 [0: automatic].
 * COLL_OPT_NONTEMPORAL     bit mask of nontemporal accesses: 1 source loads,
 *                          2 old-destination loads, 4 stores; -1: automatic
 *                          [-1]: in the row kernel none while all rank
 *                          buffers together fit the 256 MiB memory-side
 *                          cache, else source loads only (AllToAll, and the
 *                          row lists of reducing calls that pass results
 *                          between steps in registers: source loads and
 *                          stores); in the column kernel, where every access
 *                          is a load or a store of its own, none up to twice
 *                          that size, else all.  Any mask with a bit of 1 or
 *                          4 makes the column kernel's accesses nontemporal.
 * COLL_OPT_REVERSE         1: odd steps walk their columns backwards, so data
 *                          written last is read first [1]; 0: always forwards.
 * COLL_OPT_MODEL_ALPHA_NS  per-step cost used by COLL_ALGO_AUTO, in ns [1060].
 * COLL_OPT_MODEL_BETA_GBPS moved-byte rate used by COLL_ALGO_AUTO, in GB/s [8200].
 * COLL_OPT_COL_TILES       column kernel: tiles (64 lanes x 16 bytes) per
 *                          work group, up to 65535 [0: automatic: 1 under 64
 *                          tiles per CU; without row checksums, for programs
 *                          that hold all their leaves in registers, 2 from
 *                          128 to 511 tiles per CU and 4 above for programs
 *                          of one leaf (AllGather, Broadcast), else 1; with
 *                          them 2, from 1,024 tiles per CU 4].
 * COLL_OPT_TIMING          1: every call made outside graph capture records a
 *                          HIP event before its first data-moving kernel and
 *                          one after its last (not around the checksum
 *                          clearing or folding), for coll_last_kernel_ms [0].
 * COLL_OPT_CACHE_BYTES     device memory the schedule cache may hold, in bytes
 *                          [2^31]; least recently used schedules are dropped
 *                          (after synchronising their device) when a call
 *                          takes it above; 0 keeps only the schedule in use.
 *                          A lower value applies from the next call on.
 * COLL_OPT_A2A_DIRECT      with COLL_OPT_EXEC 0 and 16-byte aligned buffers:
 *                          1: an AllToAll whose every row moves one whole
 *                          block (Pairwise, Bruck, the Ring AllToAll) and
 *                          whose blocks are multiples of 16 bytes runs as one
 *                          direct copy of its N * N blocks, each read once and
 *                          written once [1].  An AllToAll only moves blocks,
 *                          so the host runs the schedule on block identities
 *                          (every source of a step read before any row of it
 *                          writes, the pages' step model) and each row's
 *                          checksum is that of the send block it carries,
 *                          summed by the copy.  0: only the rows a direct copy
 *                          makes as they stand (all of Pairwise; Bruck's and
 *                          the Ring AllToAll's first rotation), the rounds
 *                          after them in the permutation kernel.
 * Every setting other than the model constants gives bit-identical results;
 * they only change the speed or the memory held. */
typedef enum {
  COLL_OPT_EXEC = 0,
  COLL_OPT_GROUP_TILES = 1,
  COLL_OPT_MAX_GRID = 2,
  COLL_OPT_NONTEMPORAL = 3,
  COLL_OPT_REVERSE = 4,
  COLL_OPT_MODEL_ALPHA_NS = 5,
  COLL_OPT_MODEL_BETA_GBPS = 6,
  COLL_OPT_CACHE_BYTES = 7,
  COLL_OPT_COL_TILES = 8,
  COLL_OPT_TIMING = 9,
  COLL_OPT_A2A_DIRECT = 10
} coll_option_t;
coll_status_t coll_set_option(coll_option_t key, int64_t value);
/* The current value of an option; INVALID_ARG for an unknown key or NULL value. */
coll_status_t coll_get_option(coll_option_t key, int64_t* value);
/* Schedules in the cache and the device bytes their tables and work lists
 * hold, summed over devices (either pointer may be NULL). */
coll_status_t coll_cache_info(int64_t* schedules, int64_t* device_bytes);

/* The time between the events of the last call this thread made with
 * COLL_OPT_TIMING on, in ms (waits for that call's kernels; [P3]'s step
 * model is checked against such times).  INVALID_ARG for NULL or when no call
 * was timed; COLL_ERR_HIP when the events fail. */
coll_status_t coll_last_kernel_ms(float* ms);

/* Waits for the work enqueued on `stream` (a hipStream_t; NULL: the null
 * stream) and reports whether it failed: COLL_ERR_HIP with the HIP error text
 * in coll_last_error(), else COLL_OK.  No kernel of this library waits on a
 * flag written by another work group (every column has one owner), so no call
 * can hang on one and there is no time-out status. */
coll_status_t coll_check(void* stream);

const char* coll_status_string(coll_status_t status);
const char* coll_last_error(void);   /* thread-local detail of the last error */
void coll_finalize(void);            /* frees the schedule cache and the checksum slots after
                                        waiting for every device that holds part of them (work
                                        queued there finishes first) */

/* ------------------------------------------------------------------------- */
/* Calibration kernels: plain streams over `bytes` bytes (multiple of 16) for
 * measuring the achievable HBM rate beside the schedule kernels.
 * copy: dst = src (1 read + 1 write); add: dst = a + b as float32 (2 reads + 1
 * write). */
coll_status_t coll_calib_copy(void* dst, const void* src, size_t bytes, void* stream);
coll_status_t coll_calib_add(void* dst, const void* a, const void* b, size_t bytes, void* stream);

/* The column kernel's access patterns without its programs, as ceilings for
 * it: one-wave work groups, one 1 KiB tile of each buffer per work group;
 * the tile is loaded from each of the nloads buffers (all loads in flight,
 * eight at a time), summed as u32 words, and the sum stored to each of the
 * nstores buffers at the same offset; nontemporal; nloads 0 stores a
 * constant.  (nloads, nstores): (0, 1) a fill, (8, 8) an 8-rank AllReduce
 * (pass the same buffers twice for in place), (8, 1) an 8-rank Reduce, (1, 7)
 * an 8-rank Broadcast, (64, 1) a 64-rank ReduceScatter segment, (1, 63) a
 * 64-rank AllGather segment.  Each buffer holds `bytes` bytes (a multiple of
 * 1024), 16-byte aligned, owned by the caller; the stores overwrite them.
 * groups_per_cu: 0 for no cap, or COLL_CALIB_MIN_GROUPS .. COLL_CALIB_MAX_GROUPS
 * to hold each CU to at most that many work groups at once (by reserving
 * LDS the kernel never touches, 160 KiB per CU).  Errors: UNSUPPORTED for
 * any other pair; INVALID_ARG for NULL or misaligned buffers or sizes, or
 * groups_per_cu out of range. */
#define COLL_CALIB_MIN_GROUPS 3
#define COLL_CALIB_MAX_GROUPS 32
coll_status_t coll_calib_pattern(void* const* loads, int nloads, void* const* stores, int nstores, size_t bytes,
                                 int groups_per_cu, void* stream);

/* A stand-in for compute, for measuring how far a collective on a side stream
 * hides behind it ([P2] 延迟掩盖：计算与通信的Overlap; Overlap的性能收益).
 * `grid` work groups of 256 threads each run `iters` rounds of four dependent
 * fp32 FMA chains in registers, then write one float per thread to
 * out[0 .. grid*256); there is no other memory traffic.  The duration grows
 * linearly with iters.  out: device memory of grid*256 floats, 4-byte aligned,
 * owned by the caller.  Errors: INVALID_ARG for NULL or misaligned out, grid
 * outside [1, COLL_SPIN_MAX_GRID] or iters above COLL_SPIN_MAX_ITERS. */
#define COLL_SPIN_MAX_GRID 65536
#define COLL_SPIN_MAX_ITERS (1u << 28)
coll_status_t coll_calib_spin(float* out, uint32_t iters, uint32_t grid, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* COLL_H */
