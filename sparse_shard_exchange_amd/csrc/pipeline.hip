// GPipe forward pipeline of S stages over M microbatches in one launch.
//
// PATHWAYS page ("PATHWAYS: Asynchronous Distributed Dataflow for ML"),
// section 5.3 "Large-scale model performance" and Table 2: a model split into
// S balanced stages on distinct device sets, run with a GPipe-like schedule
// over M microbatches; sections 4.4-4.5: each computation starts when the
// buffer futures of its inputs are ready, and the whole statically shaped
// program is handed over at once. NEST page, Algorithm 1: fill and drain of
// such a pipeline take M + S - 1 stage slots.
//
// On one GPU the stages are shards of the program. Stage s of microbatch m is
// h[s][m] = bf16(GELU(h[s-1][m] . W_s)) (rows x d times d x d). The work is cut
// into 256 x 256 output tiles (s, m, r, c): row block r, column block c. The
// plan uploads the claim order: items in GPipe lock-step order (tick s + m
// ascending, then stage), microbatch m's items in the queue of XCD m mod 8,
// each item's tiles consecutive. Persistent workgroups claim tiles from
// their own XCD's queue only. Tile (s, m, r, c) waits for the row-block
// future (s - 1, m, r) (all column tiles of that row block of the previous
// stage written), so a row block flows to the next stage before the rest of
// its microbatch is done.
//
// Producer and consumer of every activation block share an XCD, and with it
// the L2, the coherence point of the XCD's CUs: a tile's plain stores are
// complete (every wave waited for them) before the row-block counter add
// that publishes them, and the consumer reads the block with loads that skip
// its CU's L1 (sc0), after it saw the counter. No agent-scope release or
// acquire is needed, each of which would write back or invalidate the XCD's
// whole L2. (Each activation block is written once per launch and read only
// after it is complete, and the L1s start the launch empty.)
#include "device.h"
#include "gemm.h"

namespace pw {

namespace {

__device__ __forceinline__ bool reached(uint32_t v, uint32_t target) { return (int32_t)(v - target) >= 0; }

constexpr uint32_t kNone = 0xFFFFFFFFu;
constexpr int kPastL1 = 1;  // sc0 in the cache-policy operand: the load is served by the L2, never a CU's L1

__global__ void k_pipe_reset(PipeArgs a) {
  if (threadIdx.x < a.nq) a.qctr[threadIdx.x] = 0;
}

// Row block (s, m, r) of stage s is complete once all its column tiles have
// been published (cumulative counter, target per call).
__device__ __forceinline__ const uint32_t* gate_of(const PipeArgs& a, uint32_t s, uint32_t m, uint32_t r) {
  return a.rb_ctr + ((uint64_t)(s - 1) * a.M + m) * a.RB + r;
}

struct PipeTile {
  uint32_t s, m, r, c;
};

// Tickets and tile codes are wave-uniform; readfirstlane says so. The loop
// over tiles carries only the 32-bit code of a tile and recomputes its
// pointers where they are used, so that little state lives across the K loop.
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ PipeTile unpack(uint32_t code) {
  return {code & 0xFF, (code >> 8) & 0xFF, (code >> 16) & 0xFF, code >> 24};
}

__device__ __forceinline__ uint32_t code_at(const PipeArgs& a, uint32_t t) { return uniform(a.order[t]); }

__device__ __forceinline__ mm::Tile tile_of(const PipeArgs& a, const PipeTile& p) {
  const uint64_t item_elems = (uint64_t)a.rows * a.d;
  const __bf16* in = p.s == 0 ? a.x + (uint64_t)p.m * item_elems : a.acts + ((uint64_t)(p.s - 1) * a.M + p.m) * item_elems;
  mm::Tile tile;
  tile.A = in + (uint64_t)p.r * mm::BM * a.d;
  tile.lda = a.d;
  tile.rows = min((int)mm::BM, (int)a.rows - (int)(p.r * mm::BM));
  tile.Bt = a.wt + (uint64_t)p.s * a.d * a.d + (uint64_t)p.c * mm::BN * a.d;
  tile.ldb = a.d;
  tile.K = a.d;
  return tile;
}

// Thread 0: count tile p as done; the last tile of a row block completes it,
// the last row block of an item fires the item's future. Every wave waited
// for its stores of the tile before the barrier that precedes this call, and
// the consumers share this XCD's L2, so the add needs no release.
__device__ __forceinline__ void publish(const PipeArgs& a, const PipeTile& p) {
  uint32_t* ctr = a.rb_ctr + ((uint64_t)p.s * a.M + p.m) * a.RB + p.r;
  const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (reached(old + 1, a.rb_target)) {
    uint32_t* ic = a.item_ctr + (uint64_t)p.s * a.M + p.m;
    const uint32_t io = __hip_atomic_fetch_add(ic, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (reached(io + 1, a.item_target)) fire(a.f, NODE_STAGE, p.s * a.M + p.m, a.epoch);
  }
}

// Thread 0: is tile p's input row block complete (relaxed: no ordering yet)?
__device__ __forceinline__ bool gate_open(const PipeArgs& a, const PipeTile& p) {
  return p.s == 0 ||
         reached(__hip_atomic_load(gate_of(a, p.s, p.m, p.r), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), a.rb_target);
}

// Thread 0: is tile p's input row block complete? With `block`, wait for it,
// bounded by the spin limit (false once it expires). No acquire: the tile
// reads its activation operand from this XCD's L2, past the L1.
__device__ __forceinline__ bool input_ready(const PipeArgs& a, const PipeTile& p, bool block) {
  if (p.s == 0) return true;
  bool ok = gate_open(a, p);
  if (!ok && !block) return false;
  const uint64_t t0 = ok ? 0 : wall_clock64();
  while (!ok) {
    __builtin_amdgcn_s_sleep(2);
    ok = gate_open(a, p);
    if (!ok && wall_clock64() - t0 > a.f.spin_ticks) {
      latch(a.f, ST_TIMEOUT);
      return false;
    }
  }
  return true;
}

struct Claims {
  uint32_t next;   // the ticket after the current candidate (thread 0 writes it)
  uint32_t ready;  // thread 0's answer: is the candidate's input complete
  uint32_t start;  // start_blocking: the ticket thread 0 chose to start, or kNone
  uint32_t cand;   // start_blocking: the candidate after an expired wait
};

// Thread 0's claim pipeline. A claim is an atomic add on the counter of the
// XCD's queue, a round trip of several microseconds; its result is needed
// only a whole tile later. So take() hands out the ticket claimed on the
// previous call and issues the next claim without waiting for it (`raw`
// holds the counter value in flight); once the queue is exhausted the
// workgroup is done (it never takes work from another XCD's queue: the
// activations it would read sit in that XCD's L2). Before the workgroup
// waits for an input, resolve() turns the claim in flight into a held
// ticket, so that the wait can take it too (see start_blocking); take()
// hands out a held ticket first.
struct Claimer {
  uint32_t raw;   // value returned by the add in flight on queue q
  uint32_t q;     // this XCD's queue
  uint32_t held;  // a claimed ticket not handed out yet, or kNone
  bool live;      // an add is in flight
  bool done;      // the queue is empty
  __device__ void issue(const PipeArgs& a) {
    raw = __hip_atomic_fetch_add(&a.qctr[q], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    live = true;
  }
  __device__ uint32_t take(const PipeArgs& a) {  // thread 0
    if (held != kNone) {
      const uint32_t t = held;
      held = kNone;
      if (!live && !done) issue(a);  // claim ahead again
      return t;
    }
    if (done) return kNone;
    if (!live) issue(a);  // nothing in flight (resolved into a ticket earlier): claim now
    const uint32_t t = raw < a.qlen[q] ? a.qstart[q] + raw : kNone;
    if (t == kNone) {
      done = true;
      live = false;
    } else {
      issue(a);
    }
    return t;
  }
  __device__ void resolve(const PipeArgs& a) {  // thread 0
    if (live && held == kNone && raw < a.qlen[q]) {
      held = a.qstart[q] + raw;
      live = false;
    }
  }
};

// Thread 0: which of the tiles at tickets t, n and h (n, h may be kNone) has
// its input complete first: 0, 1 or 2, or -1 once the spin limit expired
// (latched as a timeout). The gates are polled with relaxed loads, all in
// flight together (no acquire, as in input_ready).
__device__ int await_any(const PipeArgs& a, uint32_t t, uint32_t n, uint32_t h) {
  const uint32_t* g[3] = {nullptr, nullptr, nullptr};
  const uint32_t tk[3] = {t, n, h};
  bool open0[3] = {false, false, false};
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    if (tk[i] == kNone) continue;
    const PipeTile p = unpack(a.order[tk[i]]);
    if (p.s == 0) open0[i] = true;
    else g[i] = gate_of(a, p.s, p.m, p.r);
  }
  const uint64_t t0 = wall_clock64();
  while (true) {
    uint32_t v[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) v[i] = g[i] ? __hip_atomic_load(g[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    int which = -1;
#pragma unroll
    for (int i = 2; i >= 0; --i)
      if (open0[i] || (g[i] && reached(v[i], a.rb_target))) which = i;  // the earliest held ticket wins ties
    if (which >= 0) return which;
    if (wall_clock64() - t0 > a.f.spin_ticks) {
      latch(a.f, ST_TIMEOUT);
      return -1;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Starting from candidate ticket t (cl.next holds the one after it), wait
// until one of the tiles the workgroup holds has its input complete and issue
// its first stages. The workgroup holds at most three unstarted tickets: t,
// cl.next, and the claim that was in flight, resolved into a ticket first;
// the others stay held, t still the candidate. Progress, per queue (a tile's
// inputs are earlier tiles of its own queue): let E be the earliest
// unfinished tile of a queue. E's input is complete; if a waiting workgroup
// holds E, it polls E and starts it; if nobody holds E, E is not claimed
// yet, every claimed ticket of the queue precedes it and is finished, so no
// workgroup of the XCD is waiting, and one of them claims E when it has
// finished its tile. A tile whose wait expires (the spin limit) is
// published as done, so nothing downstream waits forever, and the next ticket
// is taken. Returns false once the queues are empty.
__device__ bool start_blocking(const PipeArgs& a, unsigned char* lds, Claims& cl, Claimer& cr, uint32_t t,
                               uint32_t& code) {
  while (t != kNone) {
    if (threadIdx.x == 0) {
      cr.resolve(a);
      const uint32_t n = cl.next, h = cr.held;
      const int which = await_any(a, t, n, h);
      if (which == 0) {
        cl.start = t;
      } else if (which == 1) {
        cl.start = n;
        cl.next = t;
      } else if (which == 2) {
        cl.start = h;
        cr.held = n;  // handed out after t
        cl.next = t;
      } else {
        publish(a, unpack(a.order[t]));
        cl.start = kNone;
        cl.cand = n;
        cl.next = n != kNone ? cr.take(a) : kNone;
      }
    }
    __syncthreads();
    const uint32_t s = uniform(cl.start);
    if (s != kNone) {
      code = code_at(a, s);
      mm::tile_start<kPastL1>(tile_of(a, unpack(code)), lds);
      return true;
    }
    t = uniform(cl.cand);
    __syncthreads();  // every thread has read start and cand before thread 0 writes them again
  }
  return false;
}

// Publishes the previous tile from inside the next tile's K loop, once every
// wave's stores of it are complete.
struct PublishPrev {
  const PipeArgs* a;
  uint32_t code;
  bool pending;
  __device__ bool active() const { return pending; }
  __device__ void operator()() {
    if (pending && threadIdx.x == 0) publish(*a, unpack(code));
    pending = false;
  }
};

// Persistent: one workgroup per CU loops over tiles of its XCD's queue (all
// the items of the microbatches pinned to that XCD, in GPipe order), so an
// item's activation rows and weight columns are shared through that XCD's
// L2. Each queue is in dependency order, so the earliest unfinished tile of
// each queue is always held or next in line. (A tile, not a whole row
// block, is the unit of work: one GPipe tick holds at most S items, and only
// at tile granularity do they outnumber the workgroups.)
//
// Tile t's epilogue overlaps both neighbours: once its K loop ends, the first
// stages of tile t+1 are issued (and kept if t+1's input row block is already
// complete, by one non-blocking check), then t is stored, and t+1's K loop
// publishes t a few stages in (its stores long complete by then). If the
// check failed, t is published first and only then does the workgroup wait
// for t+1's input: t+1 may depend on t itself.
__global__ __launch_bounds__(256, 1) void k_pipeline(PipeArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __shared__ Claims cl;
  const uint32_t tid = threadIdx.x;
  const uint64_t item_elems = (uint64_t)a.rows * a.d;
  // Own queue: the one of the XCD this workgroup runs on (the plan makes one
  // queue per XCD and the grid fills every CU, so every queue has owners).
  Claimer cr{0, xcc_id() % a.nq, kNone, false, false};
  if (tid == 0) {
    cr.issue(a);
    cl.next = cr.take(a);
  }
  __syncthreads();
  const uint32_t first = uniform(cl.next);
  __syncthreads();
  if (tid == 0 && first != kNone) cl.next = cr.take(a);
  uint32_t cur = 0;  // code of the tile in hand
  PublishPrev prev{&a, 0, false};
  bool have = start_blocking(a, lds, cl, cr, first, cur);
  // The candidate after the tile in hand and its code, loaded a tile ahead so
  // that the check below does not wait for the order table.
  uint32_t nxt = uniform(cl.next);
  uint32_t nxt_code = nxt != kNone ? code_at(a, nxt) : 0;
  while (have) {
    mm::f32x16 acc[4][4];
    mm::tile_finish<kPastL1>(tile_of(a, unpack(cur)), lds, acc, prev);  // may publish the previous tile; ends with a barrier
    const uint32_t t2 = nxt, code2 = nxt_code;
    // every thread read cl.next and cl.ready before the barriers of the K loop
    if (tid == 0) {
      cl.ready = t2 != kNone && input_ready(a, unpack(code2), false);
      if (t2 != kNone) cl.next = cr.take(a);
    }
    __syncthreads();
    const bool started = uniform(cl.ready) != 0;
    uint32_t nxt_raw = 0;  // the load is issued here, its value taken after the epilogue
    if (started) {
      nxt = uniform(cl.next);
      if (nxt != kNone) nxt_raw = a.order[nxt];
    }
    // Issued without a branch (a conditional start here makes the compiler
    // read the accumulators out before the branch, which doubles the register
    // demand of the epilogue and spills); when not started the loads are out
    // of range and touch no memory, and the ring contents are discarded below
    // once every wave has waited for them. (code2 is a valid tile even when
    // there is no candidate.)
    mm::tile_start_if<kPastL1>(tile_of(a, unpack(code2)), lds, started);
    const PipeTile p = unpack(cur);
    __bf16* out = a.acts + ((uint64_t)p.s * a.M + p.m) * item_elems + (uint64_t)p.r * mm::BM * a.d +
                  (uint64_t)p.c * mm::BN;
    mm::store_tile<true>(acc, out, a.d, min((int)mm::BM, (int)a.rows - (int)(p.r * mm::BM)));
    nxt_code = uniform(nxt_raw);
    prev.code = cur;
    prev.pending = true;
    if (started) {
      cur = code2;
    } else {  // publish now: the wait below may be for this very tile
      mm::wait_stores();
      __syncthreads();  // every wave's stores and ring loads complete; every thread has read ready
      prev();
      have = start_blocking(a, lds, cl, cr, t2, cur);
      nxt = uniform(cl.next);
      nxt_code = nxt != kNone ? code_at(a, nxt) : 0;
    }
  }
  if (prev.pending) {  // uniform
    mm::wait_stores();
    __syncthreads();
    prev();
  }
  if (tid == 0) {
    const uint32_t dn = __hip_atomic_fetch_add(a.done_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (reached(dn + 1, a.done_target)) fire(a.f, NODE_RESULT, 0, a.epoch);
  }
}

}  // namespace

hipError_t launch_pipeline(const PipeArgs& a, uint32_t grid, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k_pipeline, hipFuncAttributeMaxDynamicSharedMemorySize, mm::kLdsTotal);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(k_pipe_reset, dim3(1), dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_pipeline, dim3(grid), dim3(mm::NT), mm::kLdsTotal, s, a);
  return hipGetLastError();
}

}  // namespace pw
