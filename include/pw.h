/*
 * pw.h -- C ABI of the sharded-dataflow hot path on one MI355X (gfx950).
 *
 * The method is the one described on the PATHWAYS page ("PATHWAYS:
 * Asynchronous Distributed Dataflow for ML"):
 *   - section 4.3 "Coordination implementation": a chain of two N-sharded
 *     computations is the four-node graph Arg -> Compute(A) -> Compute(B) ->
 *     Result; each node emits tuples tagged with destination shards; messages
 *     travel among dynamically chosen subsets of shards along a sharded edge
 *     and progress tracking decides when a shard has received all of them;
 *   - sections 4.4 and 4.5: computations consume buffer futures and a
 *     successor starts as soon as its input futures are ready; regular
 *     (statically shaped) subgraphs are prepared ahead of time and handed
 *     over in one message (parallel asynchronous dispatch);
 *   - section 4.2 and 4.6: a sharded buffer is one logical object, referred
 *     to by handle, bookkept once for all of its shards; allocation failure
 *     means backpressure rather than a crash.
 *
 * Conventions for every entry point:
 *   - Every pointer named "device" is device memory the CALLER owns and keeps
 *     alive until the future returned by the call has fired; the library
 *     never allocates, frees or retains device memory of its own, except
 *     the one extent an object store (pw_store_*) takes when the caller
 *     creates it. Host structs passed in are read during the call only.
 *   - A stream argument is a hipStream_t passed as void* (NULL = the null
 *     stream). Calls are stream ordered and return before the device work
 *     finishes.
 *   - Every function returns a status code (PW_OK or a negative PW_ERR_*).
 *     On failure nothing was enqueued, and pw_last_error() (thread local)
 *     describes the cause. Errors found by kernels (a destination out of
 *     range, an expired wait) are latched in the plan's device status word,
 *     tagged with the epoch of the call that raised them, and reported by the
 *     first pw_future_wait on a future of that call or a later one.
 *   - Nothing aborts or throws across this ABI.
 *   - No HIP call is made before the first call that needs the device
 *     (sizing and validation in pw_plan with ws == NULL are host-only).
 */
#ifndef PW_H_
#define PW_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PW_ABI_VERSION 1u

/* ---- status codes -------------------------------------------------------- */
#define PW_OK                0
#define PW_ERR_INVALID      -1  /* bad argument, descriptor or shape mismatch          */
#define PW_ERR_NOMEM        -2  /* workspace too small: the caller must grow it and retry
                                   (the backpressure of section 4.6)                  */
#define PW_ERR_DEVICE       -3  /* a HIP call failed; pw_last_error() holds its text    */
#define PW_ERR_TIMEOUT      -4  /* a host wait, or a bounded device wait, expired       */
#define PW_ERR_BAD_DEST     -5  /* a tuple named a destination outside [0, N); the
                                   kernels dropped it                                 */
#define PW_ERR_STATE        -6  /* wrong call order (stale future, destroyed plan, ...) */
#define PW_ERR_UNSUPPORTED  -7  /* a valid request the library does not implement         */

/* ---- element types ------------------------------------------------------- */
typedef enum { PW_F32 = 0, PW_BF16 = 1 } pw_dtype;

/* ---- graph kinds (one plan = one statically shaped program) -------------- */
typedef enum {
  PW_GRAPH_EXCHANGE = 0, /* Arg -> A -> sparse exchange -> B -> Result (section 4.3)          */
  PW_GRAPH_CHAIN    = 1, /* K chained steps Arg -> A -> B -> Result, identity routing (5.1)   */
  PW_GRAPH_MOE      = 2, /* A = router + top-k gate, exchange to experts, B = expert FFN,
                            gated combine back to token order (section 6.3)                 */
  PW_GRAPH_PIPELINE = 3  /* S stages x M microbatches, GPipe fill/drain (5.3, Table 2)        */
} pw_graph_kind;

/* ---- elementwise node bodies --------------------------------------------- */
typedef enum {
  PW_OP_IDENTITY = 0, /* y = x, bit copy (any dtype)                                   */
  PW_OP_AFFINE   = 1, /* y = a*x + b in fp32, rounded once (fused multiply-add); fp32 */
  PW_OP_ROWSUM   = 2  /* B only: one fp32 per tuple, the sum of its P elements; fp32  */
} pw_op_kind;

typedef struct {
  uint32_t kind; /* pw_op_kind */
  float a;
  float b;
} pw_op;

/* ---- chain execution modes (section 5.1: OpByOp / Chained / Fused) ------- */
typedef enum {
  PW_CHAIN_CHAINED = 0, /* one launch runs every step; each node waits on its input futures
                           in the HBM future table and fires its own                        */
  PW_CHAIN_OPBYOP  = 1, /* one host launch per node per step                                 */
  PW_CHAIN_FUSED   = 2, /* one launch, one node per shard looping over the steps, no futures */
  PW_CHAIN_SPLIT   = 3  /* as CHAINED, but A[i] and B[i] run on different waves, of different
                           workgroups, with A preferably on the first half of the XCDs and B on
                           the other: every gate is a cross-workgroup handoff, the producer's
                           agent-coherent stores and epoch, the consumer's poll and coherent
                           loads (section 4.5, parallel asynchronous dispatch). Needs all the
                           waves resident at once (else pw_plan returns PW_ERR_UNSUPPORTED)  */
} pw_chain_mode;

/* ---- plan flags ----------------------------------------------------------- */
#define PW_FLAG_TRACE   0x1u /* record a device timestamp for every future fire          */
#define PW_FLAG_TIMING  0x2u /* record HIP events around every kernel (pw_plan_kernel_times) */
#define PW_FLAG_STAGE_WINDOWS 0x4u /* PIPELINE: claim tiles stage by stage within windows of 16
                                      microbatches instead of in GPipe lock-step ticks; the same
                                      dependencies and per-stage microbatch order, fewer waits  */
#define PW_FLAG_ONE_LAUNCH 0x8u /* EXCHANGE: where the step is small enough (<= 64 destinations,
                                   <= 256 slabs of <= 32 KiB of payload, rows of 16..512 bytes),
                                   run the whole step as one co-resident launch in which B of each
                                   segment waits on that segment's EXCHANGE future inside the
                                   launch (sections 4.4-4.5); otherwise, and by default, as
                                   separate launches (rank and scan, scatter, B). Same results   */

/* ---- plan descriptor ------------------------------------------------------ */
typedef struct {
  uint32_t abi_version;      /* must be PW_ABI_VERSION                                        */
  uint32_t kind;             /* pw_graph_kind                                                  */
  uint32_t num_shards;       /* EXCHANGE/CHAIN: N shards; MOE: experts E; PIPELINE: stages S   */
  uint32_t num_src_shards;   /* EXCHANGE/MOE: source shards (0 = num_shards)                   */
  uint64_t tuples_per_shard; /* EXCHANGE: tuples per source shard T; MOE: tokens per source
                                shard; CHAIN: fp32 elements per shard; PIPELINE: rows per
                                microbatch                                                     */
  uint32_t payload_elems;    /* EXCHANGE: elements per tuple P; MOE/PIPELINE: model width d    */
  uint32_t dtype;            /* EXCHANGE payload dtype (pw_dtype); MOE/PIPELINE: PW_BF16       */
  pw_op a_op;                /* EXCHANGE/CHAIN: A's body                                       */
  pw_op b_op;                /* EXCHANGE/CHAIN: B's body                                       */
  uint32_t top_k;            /* MOE: tuples per token (2)                                      */
  uint32_t hidden;           /* MOE: expert FFN hidden width (multiple of 256; d = payload_elems
                                a multiple of 256, <= 1280)                                      */
  uint32_t microbatches;     /* PIPELINE: M                                                    */
  uint32_t chain_mode;       /* CHAIN: pw_chain_mode                                           */
  uint32_t flags;            /* PW_FLAG_*                                                      */
  uint32_t capacity;         /* MOE: tuples each expert keeps, the first in tuple order
                                g = 2 * token + slot (0 = no limit); the rest are dropped and
                                add nothing to their token's combine. Other kinds: 0         */
  uint64_t spin_limit_ns;    /* bound of every device-side wait (0 = 2 s); an expired wait
                                latches PW_ERR_TIMEOUT and the waiting work is skipped        */
  /* Weights are stored [in][out], row-major. They are read once, when the plan is built
     (pw_plan with ws != NULL packs them K-contiguous into the workspace); later changes
     to these buffers are not seen by the plan. */
  const void* w_router;      /* MOE: device bf16 [d][E]                                        */
  const void* w1;            /* MOE: device bf16 [E][d][hidden]; PIPELINE: bf16 [S][d][d]      */
  const void* w2;            /* MOE: device bf16 [E][hidden][d]                                */
} pw_plan_desc;

/* ---- sharded buffer: one logical buffer over N shards (section 4.2) ------- */
typedef struct {
  void* base;               /* device: tuple 0 of shard 0; tuples are rows of elems_per_tuple */
  uint64_t num_tuples;      /* rows over all shards                                          */
  uint32_t num_shards;
  uint32_t elems_per_tuple;
  uint32_t dtype;           /* pw_dtype                                                      */
  uint32_t reserved0;
  int64_t* shard_offsets;   /* device [num_shards + 1] row offsets of the shards. Inputs:
                               NULL = uniform shards. Exchange outputs: written by the call
                               (the CSR of the destination segments), may be NULL            */
} pw_sharded_buf;

/* ---- futures (sections 4.4-4.5) -------------------------------------------
 * A future names one (node, shard) of one plan and one epoch. Epochs count
 * calls (EXCHANGE, MOE, PIPELINE) or steps (CHAIN) and start at 1. It is a
 * value type: nothing to free. */
typedef enum {
  PW_NODE_ARG = 0, PW_NODE_A = 1, PW_NODE_EXCHANGE = 2, PW_NODE_B = 3, PW_NODE_RESULT = 4,
  PW_NODE_STAGE = 5 /* PIPELINE: shard = stage * M + microbatch */
} pw_node;

typedef struct {
  uint64_t plan_id;
  uint32_t node;   /* pw_node                                  */
  int32_t shard;   /* -1 = the whole node (Result)              */
  uint64_t epoch;
} pw_future_t;

typedef struct pw_plan_s* pw_plan_t;

/* ---- exchange call arguments ---------------------------------------------- */
typedef struct {
  pw_sharded_buf src;   /* EXCHANGE: [G][P] rows, shard-major (tuple g = s*T + i).
                           MOE: the tokens [tokens][d] bf16                                 */
  const int32_t* dest;  /* EXCHANGE: device [G] destination per tuple. MOE: NULL (A routes) */
  pw_sharded_buf dst;   /* [G][P] A(src) rows in exchange order: destination-major, source
                           order inside a destination. MOE: [k*tokens][d] dispatched rows;
                           dst.shard_offsets (nullable) receives the N+1 segment offsets     */
  int32_t* src_index;   /* device [G]: source tuple index held by each output slot (nullable
                           for EXCHANGE; MOE: tuple g = k*token + slot)                      */
  int32_t* counts;      /* device [num_src][N]: tuples per (source, destination); nullable   */
  void* b_out;          /* EXCHANGE: B's output in exchange order -- ROWSUM: fp32 [G];
                           AFFINE: fp32 [G][P]; IDENTITY: unused. MOE: expert outputs
                           [k*tokens][d] bf16 (required)                                     */
  void* result;         /* MOE: combined output [tokens][d] bf16 (required)                  */
  float* logits;        /* MOE: router logits fp32 [tokens][E]; nullable                     */
  int32_t* experts;     /* MOE: [tokens][k] chosen experts, best first; nullable             */
  float* gates;         /* MOE: [tokens][k] gate values; nullable                            */
} pw_exchange_io;

/* ---- per-kernel timing (PW_FLAG_TIMING) ----------------------------------- */
typedef struct {
  char name[32];
  uint64_t launches;
  double total_ms;  /* sum of HIP-event durations over the launches */
} pw_kernel_time;

/* ======================================================================== */

/* ABI version of the loaded library (PW_ABI_VERSION it was built with). */
uint32_t pw_abi_version(void);

/* Static text for a status code. Never NULL. */
const char* pw_strerror(int status);

/* Thread-local text of this thread's last failure ("" if none). */
const char* pw_last_error(void);

/*
 * pw_plan -- build a statically shaped program once (PATHWAYS page, section
 * 4.5: host work for every node is done before any node runs, from the known
 * shapes; section 3 and Appendix B: compiled functions have static shapes).
 *
 * Two calls. With ws == NULL it validates `d` on the host only and stores the
 * workspace size in *ws_required (out may be NULL). With ws != NULL (device
 * memory of ws_bytes >= *ws_required, 256-byte aligned, caller-owned, kept
 * alive until pw_plan_destroy) it lays out the tables in ws, clears them,
 * and returns an opaque handle in *out. ws_bytes too small -> PW_ERR_NOMEM.
 * The plan holds host metadata only; weights in `d` are packed into the
 * workspace during this second call (device work, synchronised before return).
 */
int pw_plan(const pw_plan_desc* d, void* ws, size_t ws_bytes, size_t* ws_required, pw_plan_t* out);

/* Release the plan's host metadata (not ws; the caller owns and frees it).
 * PATHWAYS page, section 4.2: objects are referred to by handle and their
 * lifetime is the client's to end; section 4.6: buffers stay allocated until
 * the client releases them. PW_ERR_STATE if the plan's last call may still be
 * running (wait on its future first); PW_ERR_STATE for a handle that is not
 * a live plan (destroyed twice, forged). */
int pw_plan_destroy(pw_plan_t plan);

/*
 * pw_exchange -- one step Arg -> Compute(A) -> sparse exchange -> Compute(B)
 * -> Result (PATHWAYS page, section 4.3; for MOE also section 6.3).
 *
 * EXCHANGE: every tuple of src goes, transformed by A, to the segment of its
 * destination in dst; segments are in destination order and keep source
 * order inside (a stable sort by destination); src_index/counts/segment
 * offsets describe the move. The future of destination d (node EXCHANGE)
 * fires once all of its tuples are written; B runs on segment d only after
 * that future fired and fires node B; Result fires after every B.
 * MOE: A is the router GEMM with top-k gating (tuple g = k*token + slot goes
 * to expert experts[token][slot]); B is the expert FFN on each expert's
 * segment, gated on that expert's future; the combine gathers each token's
 * k expert rows back and sums them weighted by the gates into `result`.
 *
 * Stream ordered; *done receives the Result future. Argument errors return
 * PW_ERR_INVALID before anything is enqueued. The calls of one plan share its
 * workspace (tables, counters, futures): issue them on one stream or order
 * them across streams; calls of one plan that overlap on the device race.
 * A call's epoch (and, one-launch, its slab-table tag) is fixed when the call
 * is made, and a graph replay would reuse them: on a stream under HIP graph
 * capture every call of a plan returns PW_ERR_UNSUPPORTED before enqueueing
 * anything (pw_exchange_scratch is the capturable form of the step).
 */
int pw_exchange(pw_plan_t plan, const pw_exchange_io* io, void* stream, pw_future_t* done);

/*
 * pw_exchange_begin / pw_exchange_end -- the same step in two calls, split
 * where its output sizes become known (PATHWAYS page, section 4.5: a node
 * whose resource needs depend on its predecessor's results falls back to
 * sequential scheduling; here, the rows an MOE step dispatches under an
 * expert capacity).
 *
 * begin enqueues Compute(A) (MOE: router and top-k gate), the histogram and
 * the scan on `stream`, then BLOCKS until they finish and copies the
 * destination segment offsets to offsets_host[0..N] (caller's host memory,
 * N + 1 int64; for MOE with a capacity, of the kept tuples). It reads src,
 * dest (EXCHANGE) and logits / experts / gates / counts (MOE, nullable) of
 * io; the output fields are not read.
 * end enqueues the scatter, B and the Result and returns at once; *done
 * receives the Result future. Its io must name the src, dest, logits,
 * experts, gates and counts begin was given (else PW_ERR_INVALID); dst and
 * b_out need only hold offsets_host[N] rows.
 * While a step is open (begin returned, end not yet called) pw_exchange and
 * pw_exchange_begin on the plan return PW_ERR_STATE; pw_exchange_end
 * without begin returns PW_ERR_STATE.
 *
 * pw_exchange needs dst and b_out of the static bound instead: G rows for
 * EXCHANGE, 2 * tokens for MOE, or min(2 * tokens, E * capacity).
 */
int pw_exchange_begin(pw_plan_t plan, const pw_exchange_io* io, void* stream, int64_t* offsets_host);
int pw_exchange_end(pw_plan_t plan, const pw_exchange_io* io, void* stream, pw_future_t* done);

/*
 * pw_exchange_scratch -- the EXCHANGE step of pw_exchange with no plan and no
 * workspace, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. It
 * allocates nothing (no hipMalloc, hipFree, events or pinned memory) and
 * enqueues only kernel launches on `stream`.
 *
 * `d` is an EXCHANGE descriptor with flags = 0; `io` as for pw_exchange, with
 * dst of G rows and dst.shard_offsets (device, N + 1 int64) required: tuples
 * whose destination is outside [0, N) are dropped, and G - offsets[N] tells
 * how many (there is no future to report it through). The step's tables live
 * in a static device array of 8 MiB per GPU, held from the library's load
 * until the process ends; a descriptor whose tables need more returns
 * PW_ERR_INVALID before anything is enqueued (the error text names both
 * sizes). Each call clears what must start at zero; every call on one GPU
 * shares the array, so calls that overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller. Results are those of
 * pw_exchange on the same inputs, bit for bit.
 */
int pw_exchange_scratch(const pw_plan_desc* d, const pw_exchange_io* io, void* stream);

/*
 * pw_chain_run -- run a chained program in one call (PATHWAYS page, section
 * 3 "program tracer", section 4.5 parallel asynchronous dispatch, section 5.1
 * chained execution).
 *
 * CHAIN: `steps` repetitions of Arg -> A -> B -> Result over `state` (N shards
 * of tuples_per_shard fp32, one tuple per shard, identity routing). The
 * Result of step k is the Arg of step k + 1; on return of the device work
 * `state` holds the last Result. `aux` (nullable, device, same shape as state)
 * receives A's last output. Mode per plan (chain_mode). `state->base` and
 * `aux` must be 16-byte aligned (else PW_ERR_INVALID).
 * PIPELINE: steps must be 1. `state` holds the M microbatches [M][rows][d]
 * bf16; `aux` (device, required) receives every stage output [S][M][rows][d]
 * bf16. Item (s, m) (stage s of microbatch m) reads the output of (s-1, m)
 * only once that row block's future fired; items of one stage start in
 * ascending m on each XCD (microbatch m runs on XCD m mod 8), and items of
 * different XCDs run concurrently.
 *
 * *done receives the future of the last Result.
 */
int pw_chain_run(pw_plan_t plan, uint64_t steps, pw_sharded_buf* state, void* aux, void* stream,
                 pw_future_t* done);

/*
 * pw_future_wait -- block the calling host thread until `f` fired or
 * timeout_ns passed (< 0: no limit). PATHWAYS page, section 4.4: every
 * computation consumes and produces futures (of sharded buffers); section 4.5:
 * a node's successor may start as soon as the node's output future is ready,
 * before the rest of the program finished.
 *
 * A shard's future (shard >= 0, any node but RESULT) is resolved from its own
 * word in the plan's device future table, which the kernels store at system
 * scope when the (node, shard) completes: the wait polls that word (a 4-byte
 * read-back on a stream of the plan's own, spinning for 100 us, then every
 * 20 us) and returns once it holds f.epoch or later, which can be long before
 * the call's Result. The RESULT future (shard -1) waits for the call's
 * completion. A fired future means the device work of that (node, shard) is
 * complete in device memory; host reads of the buffers it guards still go
 * through the caller's stream.
 *
 * Returns PW_OK; PW_ERR_TIMEOUT; a device error latched by f's call or an
 * earlier call of the plan (PW_ERR_BAD_DEST, PW_ERR_TIMEOUT), reported once
 * and then cleared (an error latched by a later call is left for the waits of
 * that call); PW_ERR_STATE if the future belongs to no live plan, its epoch
 * was never launched, or its call completed without firing it;
 * PW_ERR_INVALID for a node or shard outside the plan's table.
 */
int pw_future_wait(pw_future_t f, int64_t timeout_ns);

/* Non-blocking form of pw_future_wait (same sections, same resolution and
 * errors): *fired = 1 if f has fired, else 0. */
int pw_future_query(pw_future_t f, int* fired);

/*
 * pw_plan_read_futures -- copy the plan's device future table to host memory
 * after waiting for its last call: epochs[node * width + shard] (the last
 * epoch each future fired for), fires[...] (how many times it fired since
 * the plan was built) and, with PW_FLAG_TRACE, stamps[...] (device clock at
 * the last fire, 100 MHz ticks). Any pointer may be NULL. *width receives
 * the number of shard slots per node, *nodes the number of node rows.
 */
int pw_plan_read_futures(pw_plan_t plan, uint32_t* epochs, uint32_t* fires, uint64_t* stamps,
                         size_t capacity, uint32_t* nodes, uint32_t* width);

/*
 * pw_plan_chain_placement -- where the last PW_CHAIN_SPLIT call of a CHAIN
 * plan ran each node (PATHWAYS page, section 4.1: the system, not the
 * program, maps computations onto physical devices; section 4.5: the nodes of
 * a chain are dispatched to their devices ahead of time). Waits for the
 * plan's last call, then copies 2 N words: xcc[2 i] the XCD (accelerator die)
 * of the wave that ran A[i], xcc[2 i + 1] that of B[i]. PW_ERR_INVALID if the
 * plan is not a CHAIN plan in PW_CHAIN_SPLIT mode or capacity < 2 N.
 */
int pw_plan_chain_placement(pw_plan_t plan, uint32_t* xcc, size_t capacity);

/* Per-kernel launch counts and HIP-event times accumulated under
 * PW_FLAG_TIMING (waits for pending events). *n receives the entry count. */
int pw_plan_kernel_times(pw_plan_t plan, pw_kernel_time* out, int max, int* n);

/* Clear the accumulated kernel times. */
int pw_plan_reset_times(pw_plan_t plan);

/* ======================================================================== *
 * Multi-tenant scheduler (PATHWAYS page, section 5.2 "Multi-tenancy",
 * Figures 8 and 9; Appendix D, Figure 11): programs of several clients are
 * gang-scheduled onto the whole GPU one after another, interleaved at the
 * granularity of one program, and each client receives accelerator time in
 * proportion to its weight (e.g. 1:1:1:1 or 1:2:4:8).
 *
 * Policy (the pages name none): stride scheduling in integers. Client c has
 * weight w_c and stride floor(2^32 / w_c); among clients with queued
 * programs the smallest pass dispatches its oldest program (ties: lowest
 * client number) and advances by cost * stride; a client whose queue was
 * empty resumes at max(its pass, the pass of the last dispatch).
 *
 * One dispatch thread per scheduler issues the programs, in that order, on
 * one stream the scheduler owns (default priority), keeping at most
 * max_inflight of them queued on the device so that the order decided on
 * the host is close to the order the device runs. A plan submitted here
 * must not be used by other callers while it has programs pending; its
 * buffers stay the caller's, alive until pw_sched_wait returned for the
 * program. Thread safety: every pw_sched_* call may come from any thread.
 * ======================================================================== */
typedef struct pw_sched_s* pw_sched_t;

typedef enum { PW_PROG_CHAIN = 0, PW_PROG_EXCHANGE = 1 } pw_prog_kind;

typedef struct {
  uint32_t kind;          /* pw_prog_kind                                                    */
  uint32_t cost;          /* accelerator time charged to the client, caller's units, 1..2^20  */
  pw_plan_t plan;         /* CHAIN or PIPELINE plan for PW_PROG_CHAIN; EXCHANGE or MOE plan   */
  uint64_t steps;         /* PW_PROG_CHAIN: pw_chain_run's steps                              */
  pw_sharded_buf state;   /* PW_PROG_CHAIN: pw_chain_run's state (copied at submission)        */
  void* aux;              /* PW_PROG_CHAIN: pw_chain_run's aux                                */
  pw_exchange_io io;      /* PW_PROG_EXCHANGE: pw_exchange's arguments (copied at submission) */
} pw_program;

typedef struct {
  uint64_t ticket;        /* as returned by pw_sched_submit                                   */
  uint32_t client;
  int32_t status;         /* the launch call's status                                         */
  uint64_t dispatch;      /* position in the dispatch order, from 0                           */
  double start_ms;        /* device time the program started / ended, in ms after the         */
  double end_ms;          /* scheduler's first dispatch (HIP events on its stream)            */
} pw_sched_record;

/* Create a scheduler on the current HIP device. max_inflight in [1, 64].
 * Creates its stream and its dispatch thread. */
int pw_sched_create(uint32_t max_inflight, pw_sched_t* out);

/* Add a client with weight in [1, 65536]; *client receives its number
 * (0, 1, ... in call order). */
int pw_sched_add_client(pw_sched_t s, uint32_t weight, uint32_t* client);

/* Queue a program for `client`. Validates the kind, cost and plan handle
 * (argument errors of the launch itself surface at pw_sched_wait); copies
 * *prog. *ticket receives the program's ticket (1, 2, ...). */
int pw_sched_submit(pw_sched_t s, uint32_t client, const pw_program* prog, uint64_t* ticket);

/* Block until the program of `ticket` has finished on the device or
 * timeout_ns passed (< 0: no limit). Returns the launch status, else the
 * plan's latched device status (as pw_future_wait), else PW_OK. A ticket is
 * waited at most once: afterwards it is unknown (PW_ERR_STATE). */
int pw_sched_wait(pw_sched_t s, uint64_t ticket, int64_t timeout_ns);

/* hold != 0: dispatch nothing until called again with 0 (programs keep
 * queuing; what is already on the device runs on). */
int pw_sched_hold(pw_sched_t s, int hold);

/* Copy the records of finished programs, in dispatch order, from the
 * oldest not yet read: up to `capacity` into out; *n receives the count.
 * Records are dropped once read. */
int pw_sched_records(pw_sched_t s, pw_sched_record* out, size_t capacity, size_t* n);

/* Wait for every queued and running program, stop the thread, destroy the
 * stream. Tickets not yet waited are dropped. */
int pw_sched_destroy(pw_sched_t s);

/* ======================================================================== *
 * HBM object store (PATHWAYS page, section 4.6 "Data management"): buffers
 * in device memory named by handle and labelled with an owner, so that all
 * buffers of a failed client or program can be released at once; an
 * allocation that does not fit because other programs' buffers occupy the
 * memory stalls (backpressure) instead of failing.
 *
 * One extent of device memory, taken by pw_store_create. Sizes round up to
 * 256 bytes; placement is first fit by address and freed extents merge with
 * free neighbours; waiting requests are served in arrival order (a later
 * request never overtakes a waiting one). Frees are stream ordered: the
 * extent is reused only after the work enqueued on the given stream before
 * the free has finished. Every call may come from any thread.
 * ======================================================================== */
typedef struct pw_store_s* pw_store_t;

typedef struct {
  uint64_t base;          /* device address of the extent                    */
  uint64_t capacity;      /* bytes                                            */
  uint64_t in_use;        /* bytes held by live objects                       */
  uint64_t pending_free;  /* bytes freed whose stream work is still running   */
  uint64_t largest_free;  /* longest free extent now                          */
  uint64_t objects;       /* live objects                                     */
  uint64_t waiting;       /* allocations waiting now                          */
  uint64_t stalls;        /* allocations that had to wait, so far             */
  double stalled_ms;      /* host time they spent waiting, so far             */
} pw_store_stats;

/* Take `bytes` (rounded down to 256) of device memory on the current device.
 * PW_ERR_NOMEM if the device cannot provide it. */
int pw_store_create(size_t bytes, pw_store_t* out);

/* Allocate `bytes` for `owner`. If they do not fit now, wait until frees
 * make room (backpressure) for up to timeout_ns (< 0: no limit, 0: no wait);
 * PW_ERR_NOMEM on expiry, and at once if bytes exceed the whole store.
 * *object receives the handle (never 0), *device_ptr the address (256-byte
 * aligned; contents undefined). */
int pw_store_alloc(pw_store_t s, size_t bytes, uint32_t owner, int64_t timeout_ns, uint64_t* object,
                   void** device_ptr);

/* Free an object; its memory is reused once the work enqueued on `stream`
 * (hipStream_t as void*, NULL = null stream) before this call has finished.
 * PW_ERR_STATE if the handle is not live. */
int pw_store_free(pw_store_t s, uint64_t object, void* stream);

/* Free every live object of `owner` (e.g. after that client failed), stream
 * ordered as pw_store_free; *released (nullable) receives how many. */
int pw_store_release_owner(pw_store_t s, uint32_t owner, void* stream, uint64_t* released);

/* Occupancy and backpressure counters. */
int pw_store_get_stats(pw_store_t s, pw_store_stats* out);

/* Release the extent (waits for frees in flight). Live objects become
 * invalid. PW_ERR_STATE while an allocation is waiting. */
int pw_store_destroy(pw_store_t s);

#ifdef __cplusplus
}
#endif

#endif /* PW_H_ */
