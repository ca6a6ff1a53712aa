// Host runtime of the pw C ABI: plan building (workspace layout, static
// launch shapes), argument validation, stream-ordered launches, futures and
// kernel timing. It allocates no device memory: the caller hands in the
// workspace and every buffer.
//
// PATHWAYS page ("PATHWAYS: Asynchronous Distributed Dataflow for ML"),
// section 4.5: because compiled functions have static shapes, all host work
// for a program (buffer layout, launch shapes, future slots) is done once, up
// front; afterwards a call only enqueues device work. Section 4.2: the plan
// keeps one record per logical sharded buffer, never one per shard.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <map>
#include <mutex>
#include <string>
#include <thread>
#include <unordered_map>
#include <vector>

#include "pw.h"
#include "internal.h"
#include "runtime.h"

namespace pw {

// ------------------------------------------------------------------ errors
static thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

int hip_fail(hipError_t e, const char* what) {
  return fail(PW_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------------- registry
static std::mutex g_reg_mu;
static std::unordered_map<uint64_t, Plan*> g_plans;
static uint64_t g_next_id = 1;

Plan* lookup(uint64_t id) {
  std::lock_guard<std::mutex> lk(g_reg_mu);
  auto it = g_plans.find(id);
  return it == g_plans.end() ? nullptr : it->second;
}

// A handle is live if the registry holds it; the pointer itself is never
// dereferenced before that check, so stale or forged handles are safe.
bool is_live(const Plan* p) {
  if (!p) return false;
  std::lock_guard<std::mutex> lk(g_reg_mu);
  for (const auto& kv : g_plans)
    if (kv.second == p) return true;
  return false;
}

// ------------------------------------------------------------------ layout
static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  }
};

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static uint32_t ceil_log2(uint32_t n) {
  uint32_t b = 0;
  while ((1ull << b) < n) ++b;
  return b;
}

// Tuples per ranking tile: at least 2048 tiles while the tile can grow
// (up to 4096 tuples), and 512 from 16 Ki tuples on: half the tiles of 256
// means half the scan table, which keeps more mid-size steps within the scan
// fused into the ranking launch (64 x 512 x 64 fp32: 28.2 -> 25.5 us per
// step; 8 x 8192 and 16 x 4096: 36 -> 34; the 8-shard step equal).
static uint32_t pick_tile(uint64_t G) {
  uint32_t tile = G >= 16384 ? 512 : 256;
  while (tile < 4096 && G / ((uint64_t)tile * 2) >= 2048) tile *= 2;
  return tile;
}

int plan_layout(const pw_plan_desc& d, Layout& L) {
  L = Layout{};
  Carver c;
  L.ctl = c.take(256);
  switch (d.kind) {
    case PW_GRAPH_EXCHANGE:
    case PW_GRAPH_MOE: {
      const uint32_t N = d.num_shards;
      const uint32_t S = d.num_src_shards ? d.num_src_shards : d.num_shards;
      const uint64_t fan = d.kind == PW_GRAPH_MOE ? d.top_k : 1;
      L.G = (uint64_t)S * d.tuples_per_shard * fan;
      L.tile = pick_tile(L.G);
      L.num_tiles = (uint32_t)std::max<uint64_t>(1, (L.G + L.tile - 1) / L.tile);
      // 16 tiles per scan block (more only beyond 4096 tiles): at most 256
      // blocks, so the scan's second level holds every block total of a
      // destination in 16 threads x 16 registers
      L.scan_tiles = 16;
      while ((uint64_t)L.scan_tiles * 256 < L.num_tiles) L.scan_tiles *= 2;
      L.num_blk = (L.num_tiles + L.scan_tiles - 1) / L.scan_tiles;
      L.width = std::max<uint32_t>(std::max(N, S), 1);
      L.fut = c.take((size_t)kNodes * L.width * 4);
      L.fires = c.take((size_t)kNodes * L.width * 4);
      if (d.flags & PW_FLAG_TRACE) L.stamps = c.take((size_t)kNodes * L.width * 8);
      L.arrived = c.take((size_t)N * 4);
      L.expected = c.take((size_t)N * 4);
      L.b_arrived = c.take((size_t)N * 4);
      L.seg = c.take((size_t)(N + 1) * 8);
      L.tile_base = c.take((size_t)N * L.num_tiles * 4);
      L.blk_base = c.take((size_t)N * L.num_blk * 4);
      L.tile_cnt = c.take((size_t)N * L.num_tiles * 4);
      L.tile_done = c.take((size_t)L.num_tiles * 4);
      L.rank = c.take(L.G * 2);
      if (d.kind == PW_GRAPH_EXCHANGE) {
        const uint32_t row = (d.dtype == PW_F32 ? 4u : 2u) * d.payload_elems;
        L.slab = exchange_small_slab(L.G, N, row, d.b_op.kind, d.dtype == PW_F32);
        if (L.slab) {
          L.small_grid = (uint32_t)((L.G + L.slab - 1) / L.slab);
          L.slab_cnt = c.take((size_t)L.small_grid * N * 8);
          L.small_tab = c.take((size_t)2 * (2 * N + 1) * 4);
        }
      }
      if (d.kind == PW_GRAPH_MOE) {
        const uint64_t tokens = (uint64_t)S * d.tuples_per_shard;
        L.experts = c.take(tokens * d.top_k * 4);
        L.gates = c.take(tokens * d.top_k * 4);
        L.slot_of = c.take(L.G * 4);
        L.hidden_act = c.take(moe_static_rows(d) * (uint64_t)d.hidden * 2);
        L.rb_start = c.take((size_t)(N + 1) * 4);
        L.b_done = c.take((size_t)N * 4);
        L.w1t = c.take((size_t)N * d.hidden * d.payload_elems * 2);
        L.w2t = c.take((size_t)N * d.hidden * d.payload_elems * 2);
        L.wrt = c.take((size_t)64 * d.payload_elems * 2);
      }
      break;
    }
    case PW_GRAPH_CHAIN: {
      L.width = d.num_shards;
      L.fut = c.take((size_t)kNodes * L.width * 4);
      L.fires = c.take((size_t)kNodes * L.width * 4);
      if (d.flags & PW_FLAG_TRACE) L.stamps = c.take((size_t)kNodes * L.width * 8);
      L.a_buf = c.take((size_t)d.num_shards * d.tuples_per_shard * 4);
      L.place = c.take((size_t)d.num_shards * 2 * 4);
      break;
    }
    case PW_GRAPH_PIPELINE: {
      const uint64_t S = d.num_shards, M = d.microbatches;
      const uint64_t RB = (d.tuples_per_shard + 255) / 256, CT = d.payload_elems / 256;
      L.width = (uint32_t)(S * M);
      L.fut = c.take((size_t)kNodes * L.width * 4);
      L.fires = c.take((size_t)kNodes * L.width * 4);
      if (d.flags & PW_FLAG_TRACE) L.stamps = c.take((size_t)kNodes * L.width * 8);
      L.pipe_ctl = c.take(256);
      L.rb_ctr = c.take(S * M * RB * 4);
      L.item_ctr = c.take(S * M * 4);
      L.order = c.take(S * M * RB * CT * 4);
      L.w1t = c.take(S * d.payload_elems * d.payload_elems * 2);
      break;
    }
    default:
      return fail(PW_ERR_INVALID, "unknown graph kind %u", d.kind);
  }
  L.total = c.off;
  return PW_OK;
}

static int validate_op(const pw_op& op, bool allow_rowsum, const char* which) {
  if (op.kind > PW_OP_ROWSUM) return fail(PW_ERR_INVALID, "%s: unknown op kind %u", which, op.kind);
  if (op.kind == PW_OP_ROWSUM && !allow_rowsum) return fail(PW_ERR_INVALID, "%s: ROWSUM is only a B body", which);
  return PW_OK;
}

int validate_desc(const pw_plan_desc* d) {
  if (!d) return fail(PW_ERR_INVALID, "descriptor is NULL");
  if (d->abi_version != PW_ABI_VERSION)
    return fail(PW_ERR_INVALID, "abi_version %u != %u", d->abi_version, PW_ABI_VERSION);
  if (d->flags & ~(PW_FLAG_TRACE | PW_FLAG_TIMING | PW_FLAG_STAGE_WINDOWS | PW_FLAG_ONE_LAUNCH))
    return fail(PW_ERR_INVALID, "unknown flags 0x%x", d->flags);
  if ((d->flags & PW_FLAG_ONE_LAUNCH) && d->kind != PW_GRAPH_EXCHANGE)
    return fail(PW_ERR_INVALID, "PW_FLAG_ONE_LAUNCH is for EXCHANGE plans");
  if ((d->flags & PW_FLAG_STAGE_WINDOWS) && d->kind != PW_GRAPH_PIPELINE)
    return fail(PW_ERR_INVALID, "PW_FLAG_STAGE_WINDOWS is for PIPELINE plans");
  if (d->capacity && d->kind != PW_GRAPH_MOE) return fail(PW_ERR_INVALID, "capacity is for MOE plans only");
  switch (d->kind) {
    case PW_GRAPH_EXCHANGE: {
      // the scatter keeps 5 words per destination in LDS (160 KiB per CU)
      if (d->num_shards == 0 || d->num_shards > 8192) return fail(PW_ERR_INVALID, "num_shards must be in [1, 8192]");
      const uint64_t S = d->num_src_shards ? d->num_src_shards : d->num_shards;
      const uint64_t G = S * d->tuples_per_shard;
      if (G > 0x7fffffffull) return fail(PW_ERR_INVALID, "more than 2^31-1 tuples");
      if (d->dtype != PW_F32 && d->dtype != PW_BF16) return fail(PW_ERR_INVALID, "unknown dtype %u", d->dtype);
      const uint64_t esz = d->dtype == PW_F32 ? 4 : 2;
      if (d->payload_elems == 0) return fail(PW_ERR_INVALID, "payload_elems must be > 0");
      const uint64_t row = esz * d->payload_elems;
      if (row % 4 != 0 || row > (1u << 20)) return fail(PW_ERR_INVALID, "payload row must be a multiple of 4 bytes, <= 1 MiB");
      int st;
      if ((st = validate_op(d->a_op, false, "a_op"))) return st;
      if ((st = validate_op(d->b_op, true, "b_op"))) return st;
      if (d->dtype != PW_F32 && (d->a_op.kind != PW_OP_IDENTITY || d->b_op.kind != PW_OP_IDENTITY))
        return fail(PW_ERR_INVALID, "A/B bodies other than IDENTITY need fp32 payloads");
      if ((uint64_t)d->num_shards * std::max<uint64_t>(1, (G + 255) / 256) > (1ull << 31))
        return fail(PW_ERR_INVALID, "destination x tile table too large");
      return PW_OK;
    }
    case PW_GRAPH_CHAIN:
    case PW_GRAPH_MOE:
    case PW_GRAPH_PIPELINE:
      return validate_desc_more(d);
    default:
      return fail(PW_ERR_INVALID, "unknown graph kind %u", d->kind);
  }
}

// ---------------------------------------------------------------- timing
void Plan::launch_begin(const char* name, hipStream_t s) {
  if (!(desc.flags & PW_FLAG_TIMING)) return;
  Pending p;
  p.name = name;
  p.e0 = get_event();
  p.e1 = get_event();
  (void)hipEventRecord(p.e0, s);
  pending.push_back(p);
}

void Plan::launch_end(hipStream_t s) {
  if (!(desc.flags & PW_FLAG_TIMING) || pending.empty()) return;
  (void)hipEventRecord(pending.back().e1, s);
  if (pending.size() > 4096) resolve_times();
}

hipEvent_t Plan::get_event() {
  if (!event_pool.empty()) {
    hipEvent_t e = event_pool.back();
    event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  (void)hipEventCreate(&e);
  return e;
}

void Plan::resolve_times() {
  for (auto& p : pending) {
    (void)hipEventSynchronize(p.e1);
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, p.e0, p.e1);
    auto& t = times[p.name];
    t.launches += 1;
    t.total_ms += ms;
    event_pool.push_back(p.e0);
    event_pool.push_back(p.e1);
  }
  pending.clear();
}

// --------------------------------------------------------- call bookkeeping
int Plan::begin_call(hipStream_t s) {
  if (device < 0) {
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  }
  int cur = -1;
  (void)hipGetDevice(&cur);
  if (cur != device) return fail(PW_ERR_STATE, "plan built on device %d, current device is %d", device, cur);
  // A call's epoch (and the one-launch table tag) is fixed here, on the host:
  // a graph replay would reuse it, so capture is refused before anything is
  // enqueued (pw_exchange_scratch is the capturable form of the step).
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone)
    return fail(PW_ERR_UNSUPPORTED, "a plan's calls cannot be captured into a HIP graph (each call's epoch is fixed "
                "when it is made); pw_exchange_scratch can be");
  return PW_OK;
}

int Plan::end_call(hipStream_t s, uint64_t epoch_hi) {
  hipEvent_t e = nullptr;
  if (!done_pool.empty()) {
    e = done_pool.back();
    done_pool.pop_back();
  } else {
    hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (err != hipSuccess) return hip_fail(err, "hipEventCreate");
  }
  hipError_t err = hipEventRecord(e, s);
  if (err != hipSuccess) return hip_fail(err, "hipEventRecord");
  done.push_back({epoch_hi, e});
  while (done.size() > 16) {
    done_pool.push_back(done.front().event);
    done.pop_front();
  }
  return PW_OK;
}

hipEvent_t Plan::event_for(uint64_t epoch) const {
  for (const auto& d : done)
    if (d.epoch_hi >= epoch) return d.event;
  return done.empty() ? nullptr : done.back().event;
}

Futures Plan::futures() const {
  Futures f{};
  auto* base = static_cast<unsigned char*>(ws);
  f.status = reinterpret_cast<uint64_t*>(base + L.ctl);
  f.epoch = reinterpret_cast<uint32_t*>(base + L.fut);
  f.fires = reinterpret_cast<uint32_t*>(base + L.fires);
  f.stamps = (desc.flags & PW_FLAG_TRACE) ? reinterpret_cast<uint64_t*>(base + L.stamps) : nullptr;
  f.width = L.width;
  const uint64_t ns = desc.spin_limit_ns ? desc.spin_limit_ns : 2000000000ull;
  f.spin_ticks = (uint32_t)std::min<uint64_t>(0xffffffffull, ns / 10);  // 100 MHz wall clock
  f.call_epoch = (uint32_t)(epoch + 1);  // the call about to be launched
  return f;
}

int Plan::clear_status() {
  uint64_t* st = reinterpret_cast<uint64_t*>(static_cast<unsigned char*>(ws) + L.ctl);
  hipError_t e = hipMemsetAsync(st, 0, 8, aux);
  if (e == hipSuccess) e = hipStreamSynchronize(aux);
  if (e != hipSuccess) return hip_fail(e, "clearing the status word");
  return PW_OK;
}

// The status word and one future's epoch with a single round trip: two small
// copies into pinned host memory on the read-back stream, one synchronize.
int Plan::read_status_and_epoch(uint32_t node, uint32_t shard, uint64_t* status, uint32_t* epoch) {
  if (node >= kNodes || shard >= L.width) return fail(PW_ERR_INVALID, "future (%u, %u) outside the table", node, shard);
  if (!aux) {
    hipError_t e = hipStreamCreateWithFlags(&aux, hipStreamNonBlocking);
    if (e != hipSuccess) return hip_fail(e, "hipStreamCreate");
  }
  if (!host_words) {
    hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&host_words), 4 * sizeof(uint32_t), hipHostMallocDefault);
    if (e != hipSuccess) {
      host_words = nullptr;
      return hip_fail(e, "hipHostMalloc");
    }
  }
  auto* base = static_cast<unsigned char*>(ws);
  const uint32_t* fut = reinterpret_cast<const uint32_t*>(base + L.fut) + node * L.width + shard;
  hipError_t e = hipMemcpyAsync(host_words, base + L.ctl, 8, hipMemcpyDeviceToHost, aux);
  if (e == hipSuccess) e = hipMemcpyAsync(host_words + 2, fut, 4, hipMemcpyDeviceToHost, aux);
  if (e == hipSuccess) e = hipStreamSynchronize(aux);
  if (e != hipSuccess) return hip_fail(e, "reading the status word and the future table");
  *status = (uint64_t)host_words[0] | (uint64_t)host_words[1] << 32;
  *epoch = host_words[2];
  return PW_OK;
}

static int status_to_code(uint32_t st) {
  switch (st) {
    case ST_OK: return PW_OK;
    case ST_BAD_DEST: return fail(PW_ERR_BAD_DEST, "a tuple named a destination outside [0, N)");
    case ST_TIMEOUT: return fail(PW_ERR_TIMEOUT, "a device-side wait on a future expired");
    default: return fail(PW_ERR_DEVICE, "unknown device status %u", st);
  }
}

// ------------------------------------------------------------ exchange call

// After the first half of a split step: wait for it, hand the segment
// offsets to the host and remember the inputs the second half must match.
int finish_begin(Plan* p, const pw_exchange_io* io, hipStream_t s, int64_t* offsets_host) {
  const uint32_t N = p->desc.num_shards;
  const int64_t* seg = reinterpret_cast<const int64_t*>(p->base() + p->L.seg);
  hipError_t e = hipMemcpyAsync(offsets_host, seg, (N + 1) * sizeof(int64_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading the segment offsets");
  Plan::Open& o = p->open;
  o.active = true;
  o.rows = (uint64_t)offsets_host[N];
  o.src = io->src.base;
  o.dest = io->dest;
  o.logits = io->logits;
  o.experts = io->experts;
  o.gates = io->gates;
  o.counts = io->counts;
  return PW_OK;
}

// The second half of a split step must name the inputs of the first.
int check_end(Plan* p, const pw_exchange_io* io) {
  const Plan::Open& o = p->open;
  if (!o.active) return fail(PW_ERR_STATE, "pw_exchange_end without pw_exchange_begin");
  if (io->src.base != o.src || io->dest != o.dest || io->logits != o.logits || io->experts != o.experts ||
      io->gates != o.gates || io->counts != o.counts)
    return fail(PW_ERR_INVALID, "pw_exchange_end must name the src, dest, logits, experts, gates and counts of begin");
  if (io->dst.num_tuples < o.rows) return fail(PW_ERR_INVALID, "dst holds %llu rows, the step writes %llu",
                                               (unsigned long long)io->dst.num_tuples, (unsigned long long)o.rows);
  return PW_OK;
}

// The io of an EXCHANGE step against its descriptor (need_dst: the step
// writes dst and B's output; dst_rows: the rows dst must hold).
int validate_exchange_io(const pw_plan_desc& d, const Layout& L, const pw_exchange_io* io, bool need_dst,
                         uint64_t dst_rows) {
  if (L.G && (!io->src.base || !io->dest || (need_dst && !io->dst.base)))
    return fail(PW_ERR_INVALID, "src, dest and dst are required");
  if (io->src.num_tuples != L.G || io->src.elems_per_tuple != d.payload_elems || io->src.dtype != d.dtype)
    return fail(PW_ERR_INVALID, "src does not match the plan (tuples %llu, elems %u, dtype %u)",
                (unsigned long long)io->src.num_tuples, io->src.elems_per_tuple, io->src.dtype);
  if (io->src.shard_offsets) return fail(PW_ERR_UNSUPPORTED, "non-uniform source shards");
  if (need_dst && (io->dst.num_tuples < dst_rows || io->dst.elems_per_tuple != d.payload_elems ||
                   io->dst.dtype != d.dtype))
    return fail(PW_ERR_INVALID, "dst does not match the plan");
  if (!aligned16(io->src.base) || (need_dst && !aligned16(io->dst.base)))
    return fail(PW_ERR_INVALID, "src/dst must be 16-byte aligned");
  if (need_dst && d.b_op.kind != PW_OP_IDENTITY && !io->b_out)
    return fail(PW_ERR_INVALID, "b_out is required when B is not IDENTITY");
  return PW_OK;
}

// Kernel arguments of an EXCHANGE step whose tables are laid out by L from
// `base` (a plan's workspace, or the static scratch array).
void exchange_args(const pw_plan_desc& d, const Layout& L, unsigned char* base, const pw_exchange_io* io,
                   uint32_t epoch, const Futures& f, ExchangeArgs& a) {
  const uint32_t N = d.num_shards;
  const uint32_t S = d.num_src_shards ? d.num_src_shards : N;
  const uint32_t esz = d.dtype == PW_F32 ? 4 : 2;
  const uint32_t row = esz * d.payload_elems;
  a = ExchangeArgs{};
  a.src = static_cast<const unsigned char*>(io->src.base);
  a.dest = io->dest;
  a.dst = static_cast<unsigned char*>(io->dst.base);
  a.src_index = io->src_index;
  a.slot_of = nullptr;
  a.counts = io->counts;
  a.offsets_out = io->dst.shard_offsets;
  a.b_out = io->b_out;
  a.G = L.G;
  a.dst_rows = std::min<uint64_t>(io->dst.num_tuples, L.G);  // also bounds src_index (G entries)
  a.capacity = 0;
  a.T = d.tuples_per_shard;
  a.N = N;
  a.num_src = S;
  a.row_bytes = row;
  a.fanout = 1;
  a.tile = L.tile;
  a.num_tiles = L.num_tiles;
  a.scan_tiles = L.scan_tiles;
  a.num_blk = L.num_blk;
  // few tiles: the last ranking workgroup runs the scan (one block, or one
  // (block, destination) column per thread of a workgroup), saving the scan's
  // launch (8-shard step: 27.0 -> 25.6-26.0 us warm; 8 x 8192 tuples equal)
  a.fuse_scan = L.num_blk == 1 || (L.num_blk <= 16 && (uint64_t)L.num_blk * N <= 256);
  a.nbits = ceil_log2(N);
  a.is_f32 = d.dtype == PW_F32;
  a.a_kind = d.a_op.kind; a.a_a = d.a_op.a; a.a_b = d.a_op.b;
  a.b_kind = d.b_op.kind; a.b_a = d.b_op.a; a.b_b = d.b_op.b;
  a.epoch = epoch;
  a.b_gated = d.b_op.kind != PW_OP_IDENTITY;
  a.f = f;
  a.arrived = reinterpret_cast<uint32_t*>(base + L.arrived);
  a.expected = reinterpret_cast<uint32_t*>(base + L.expected);
  a.b_arrived = reinterpret_cast<uint32_t*>(base + L.b_arrived);
  a.ctl = reinterpret_cast<uint32_t*>(base + L.ctl + 64);
  a.tile_base = reinterpret_cast<uint32_t*>(base + L.tile_base);
  a.blk_base = reinterpret_cast<uint32_t*>(base + L.blk_base);
  a.tile_cnt = reinterpret_cast<uint32_t*>(base + L.tile_cnt);
  a.tile_done = reinterpret_cast<uint32_t*>(base + L.tile_done);
  a.rank = reinterpret_cast<uint16_t*>(base + L.rank);
  a.chunk = scatter_chunk(L.tile, row, a.fanout);
  a.seg = reinterpret_cast<int64_t*>(base + L.seg);
  a.slab = L.slab;
  a.call = 0;
  a.slab_cnt = L.slab ? reinterpret_cast<uint64_t*>(base + L.slab_cnt) : nullptr;
  a.small_tab = L.slab ? reinterpret_cast<uint32_t*>(base + L.small_tab) : nullptr;
}

int run_exchange(Plan* p, const pw_exchange_io* io, hipStream_t s, pw_future_t* done, Phase ph, int64_t* offsets_host) {
  const pw_plan_desc& d = p->desc;
  const Layout& L = p->L;
  const bool need_dst = ph != Phase::kBegin;
  int st = validate_exchange_io(d, L, io, need_dst, ph == Phase::kEnd ? p->open.rows : L.G);
  if (st) return st;
  if (ph == Phase::kEnd && (st = check_end(p, io))) return st;
  if ((st = p->begin_call(s))) return st;

  ExchangeArgs a;
  exchange_args(d, L, p->base(), io, (uint32_t)(p->epoch + 1), p->futures(), a);

  hipError_t e = hipSuccess;
  if (ph == Phase::kAll && p->small_ok) {  // the whole step in one launch
    if (io->counts) {
      p->launch_begin("src_counts", s);
      e = launch_src_counts(a, s);
      p->launch_end(s);
      if (e != hipSuccess) return hip_fail(e, "launch src_counts");
    }
    a.call = (uint32_t)(p->small_calls + 1);
    p->launch_begin("exchange_small", s);
    e = launch_exchange_small(a, s);
    p->launch_end(s);
    if (e != hipSuccess) return hip_fail(e, "launch exchange_small");
    p->small_calls += 1;
    p->epoch += 1;
    st = p->end_call(s, p->epoch);
    if (st) return st;
    if (done) *done = pw_future_t{p->id, PW_NODE_RESULT, -1, p->epoch};
    return PW_OK;
  }
  if (ph != Phase::kEnd) {
    if (io->counts) {
      p->launch_begin("src_counts", s);
      e = launch_src_counts(a, s);
      p->launch_end(s);
      if (e != hipSuccess) return hip_fail(e, "launch src_counts");
    }
    p->launch_begin(a.fuse_scan ? "rank_scan" : "rank", s);
    e = launch_rank(a, s);
    p->launch_end(s);
    if (e != hipSuccess) return hip_fail(e, "launch rank");
    if (!a.fuse_scan) {
      p->launch_begin("scan", s);
      e = launch_scan(a, s);
      p->launch_end(s);
      if (e != hipSuccess) return hip_fail(e, "launch scan");
    }
    if (ph == Phase::kBegin) return finish_begin(p, io, s, offsets_host);
  }
  p->open.active = false;
  p->launch_begin("scatter", s);
  e = launch_scatter(a, s);
  p->launch_end(s);
  if (e != hipSuccess) return hip_fail(e, "launch scatter");
  if (a.b_gated) {
    p->launch_begin("b", s);
    e = launch_b(a, s);
    p->launch_end(s);
    if (e != hipSuccess) return hip_fail(e, "launch b");
  }
  p->epoch += 1;
  st = p->end_call(s, p->epoch);
  if (st) return st;
  if (done) *done = pw_future_t{p->id, PW_NODE_RESULT, -1, p->epoch};
  return PW_OK;
}

}  // namespace pw

// ======================================================================= ABI
using namespace pw;

extern "C" {

uint32_t pw_abi_version(void) { return PW_ABI_VERSION; }

const char* pw_strerror(int status) {
  switch (status) {
    case PW_OK: return "ok";
    case PW_ERR_INVALID: return "invalid argument";
    case PW_ERR_NOMEM: return "workspace too small";
    case PW_ERR_DEVICE: return "HIP runtime error";
    case PW_ERR_TIMEOUT: return "timed out";
    case PW_ERR_BAD_DEST: return "destination out of range";
    case PW_ERR_STATE: return "invalid state";
    case PW_ERR_UNSUPPORTED: return "unsupported";
    default: return "unknown status";
  }
}

const char* pw_last_error(void) { return g_last_error.c_str(); }

int pw_plan(const pw_plan_desc* d, void* ws, size_t ws_bytes, size_t* ws_required, pw_plan_t* out) {
  g_last_error.clear();
  int st = validate_desc(d);
  if (st) return st;
  Layout L;
  if ((st = plan_layout(*d, L))) return st;
  if (ws_required) *ws_required = L.total;
  if (!ws) {
    if (out) *out = nullptr;
    return PW_OK;
  }
  if (!out) return fail(PW_ERR_INVALID, "out is NULL");
  if (((uintptr_t)ws & 255u) != 0) return fail(PW_ERR_INVALID, "workspace must be 256-byte aligned");
  if (ws_bytes < L.total)
    return fail(PW_ERR_NOMEM, "workspace has %zu bytes, the plan needs %zu", ws_bytes, L.total);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  e = hipMemset(ws, 0, L.total);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "clearing the workspace");
  Plan* p = new Plan();
  p->desc = *d;
  p->L = L;
  p->ws = ws;
  p->ws_bytes = ws_bytes;
  p->device = dev;
  {
    std::lock_guard<std::mutex> lk(g_reg_mu);
    p->id = g_next_id++;
    g_plans[p->id] = p;
  }
  if (d->kind == PW_GRAPH_EXCHANGE && L.slab && (d->flags & PW_FLAG_ONE_LAUNCH))
    p->small_ok = exchange_small_resident(dev) >= L.small_grid;  // the one launch needs every workgroup resident
  st = plan_init_kind(p);
  if (st) {
    std::lock_guard<std::mutex> lk(g_reg_mu);
    g_plans.erase(p->id);
    delete p;
    return st;
  }
  *out = reinterpret_cast<pw_plan_t>(p);
  return PW_OK;
}

int pw_plan_destroy(pw_plan_t plan) {
  g_last_error.clear();
  Plan* p = reinterpret_cast<Plan*>(plan);
  if (!is_live(p)) return fail(PW_ERR_STATE, "not a live plan");
  if (!p->done.empty()) {
    hipError_t e = hipEventQuery(p->done.back().event);
    if (e == hipErrorNotReady) return fail(PW_ERR_STATE, "the plan's last call is still running");
  }
  p->resolve_times();
  {
    std::lock_guard<std::mutex> lk(g_reg_mu);
    g_plans.erase(p->id);
  }
  for (auto& dn : p->done) (void)hipEventDestroy(dn.event);
  for (auto e : p->done_pool) (void)hipEventDestroy(e);
  for (auto e : p->event_pool) (void)hipEventDestroy(e);
  if (p->aux) (void)hipStreamDestroy(p->aux);
  if (p->host_words) (void)hipHostFree(p->host_words);
  plan_release_kind(p);
  delete p;
  return PW_OK;
}

static int exchange_phase(pw_plan_t plan, const pw_exchange_io* io, void* stream, pw_future_t* done, Phase ph,
                          int64_t* offsets_host) {
  g_last_error.clear();
  Plan* p = reinterpret_cast<Plan*>(plan);
  if (!is_live(p)) return fail(PW_ERR_STATE, "not a live plan");
  if (!io) return fail(PW_ERR_INVALID, "io is NULL");
  if (ph == Phase::kBegin && !offsets_host) return fail(PW_ERR_INVALID, "offsets_host is NULL");
  std::lock_guard<std::mutex> lk(p->mu);
  if (ph != Phase::kEnd && p->open.active) return fail(PW_ERR_STATE, "a split step is open: call pw_exchange_end first");
  if (ph == Phase::kEnd && !p->open.active) return fail(PW_ERR_STATE, "pw_exchange_end without pw_exchange_begin");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (p->desc.kind == PW_GRAPH_EXCHANGE) return run_exchange(p, io, s, done, ph, offsets_host);
  if (p->desc.kind == PW_GRAPH_MOE) return run_moe(p, io, s, done, ph, offsets_host);
  return fail(PW_ERR_INVALID, "an EXCHANGE or MOE plan is needed");
}

int pw_exchange(pw_plan_t plan, const pw_exchange_io* io, void* stream, pw_future_t* done) {
  return exchange_phase(plan, io, stream, done, Phase::kAll, nullptr);
}

int pw_exchange_begin(pw_plan_t plan, const pw_exchange_io* io, void* stream, int64_t* offsets_host) {
  return exchange_phase(plan, io, stream, nullptr, Phase::kBegin, offsets_host);
}

int pw_exchange_end(pw_plan_t plan, const pw_exchange_io* io, void* stream, pw_future_t* done) {
  return exchange_phase(plan, io, stream, done, Phase::kEnd, nullptr);
}

int pw_chain_run(pw_plan_t plan, uint64_t steps, pw_sharded_buf* state, void* aux, void* stream, pw_future_t* done) {
  g_last_error.clear();
  Plan* p = reinterpret_cast<Plan*>(plan);
  if (!is_live(p)) return fail(PW_ERR_STATE, "not a live plan");
  std::lock_guard<std::mutex> lk(p->mu);
  if (p->desc.kind == PW_GRAPH_CHAIN) return run_chain(p, steps, state, aux, static_cast<hipStream_t>(stream), done);
  if (p->desc.kind == PW_GRAPH_PIPELINE) return run_pipeline(p, steps, state, aux, static_cast<hipStream_t>(stream), done);
  return fail(PW_ERR_INVALID, "pw_chain_run needs a CHAIN or PIPELINE plan");
}

static int future_common(pw_future_t f, Plan** out) {
  Plan* p = lookup(f.plan_id);
  if (!p) return fail(PW_ERR_STATE, "future of plan %llu: no such live plan", (unsigned long long)f.plan_id);
  if (f.epoch == 0 || f.epoch > p->epoch) return fail(PW_ERR_STATE, "epoch %llu was never launched", (unsigned long long)f.epoch);
  if (f.node >= kNodes) return fail(PW_ERR_INVALID, "node %u", f.node);
  *out = p;
  return PW_OK;
}

// One read of the status word and of future f's epoch. A latched device
// error counts for f if the call that raised it is f's call or an earlier
// one (its epoch tag <= f.epoch): it is then reported, and cleared for later
// calls; an error raised by a later call is left for the waits of that call.
// *fired = 1 once the future holds f.epoch (or a later one).
static int poll_future(Plan* p, pw_future_t f, int* fired) {
  uint64_t st = 0;
  uint32_t v = 0;
  const uint32_t shard = f.shard < 0 ? 0u : (uint32_t)f.shard;
  int rc = p->read_status_and_epoch(f.node, shard, &st, &v);
  if (rc) return rc;
  const uint32_t code = (uint32_t)st, at = (uint32_t)(st >> 32);
  if (code && (int32_t)((uint32_t)f.epoch - at) >= 0) {
    if ((rc = p->clear_status())) return rc;
    return status_to_code(code);
  }
  *fired = (int32_t)(v - (uint32_t)f.epoch) >= 0;
  return PW_OK;
}

// After the call of f completed: its status, and f must have fired.
static int check_fired(Plan* p, pw_future_t f) {
  int fired = 0;
  int rc = poll_future(p, f, &fired);
  if (rc) return rc;
  if (!fired)
    return fail(PW_ERR_STATE, "future (%u, %d) did not fire for epoch %llu although its call completed", f.node,
                f.shard, (unsigned long long)f.epoch);
  return PW_OK;
}

static int64_t elapsed_ns(std::chrono::steady_clock::time_point t0) {
  return std::chrono::duration_cast<std::chrono::nanoseconds>(std::chrono::steady_clock::now() - t0).count();
}

// Spin for the first 100 us (short device work completes with no sleep
// latency), then poll every 20 us.
static void backoff(int64_t el) {
  if (el > 100000) std::this_thread::sleep_for(std::chrono::microseconds(20));
}

int pw_future_wait(pw_future_t f, int64_t timeout_ns) {
  g_last_error.clear();
  Plan* p = nullptr;
  int rc = future_common(f, &p);
  if (rc) return rc;
  std::lock_guard<std::mutex> lk(p->mu);
  hipEvent_t e = p->event_for(f.epoch);
  if (!e) return fail(PW_ERR_STATE, "no call recorded");
  const auto t0 = std::chrono::steady_clock::now();
  if (f.shard >= 0 && f.node != PW_NODE_RESULT) {
    // A shard's future: poll its own word in the device future table (the
    // kernels store it at system scope), so the wait returns as soon as that
    // (node, shard) fired, possibly long before the rest of the call.
    if ((uint32_t)f.shard >= p->L.width) return fail(PW_ERR_INVALID, "shard %d outside the future table", f.shard);
    while (true) {
      int fired = 0;
      if ((rc = poll_future(p, f, &fired))) return rc;
      if (fired) return PW_OK;
      const hipError_t q = hipEventQuery(e);
      if (q == hipSuccess) return check_fired(p, f);  // the call is over: one last read decides
      if (q != hipErrorNotReady) return hip_fail(q, "hipEventQuery");
      const int64_t el = elapsed_ns(t0);
      if (timeout_ns >= 0 && el >= timeout_ns)
        return fail(PW_ERR_TIMEOUT, "future not fired within %lld ns", (long long)timeout_ns);
      backoff(el);
    }
  }
  // The Result (the whole call): its completion event.
  if (timeout_ns < 0) {
    hipError_t err = hipEventSynchronize(e);
    if (err != hipSuccess) return hip_fail(err, "hipEventSynchronize");
  } else {
    while (true) {
      hipError_t err = hipEventQuery(e);
      if (err == hipSuccess) break;
      if (err != hipErrorNotReady) return hip_fail(err, "hipEventQuery");
      const int64_t el = elapsed_ns(t0);
      if (el >= timeout_ns) return fail(PW_ERR_TIMEOUT, "future not fired within %lld ns", (long long)timeout_ns);
      backoff(el);
    }
  }
  return check_fired(p, f);
}

int pw_future_query(pw_future_t f, int* fired) {
  g_last_error.clear();
  if (!fired) return fail(PW_ERR_INVALID, "fired is NULL");
  *fired = 0;
  Plan* p = nullptr;
  int rc = future_common(f, &p);
  if (rc) return rc;
  std::lock_guard<std::mutex> lk(p->mu);
  hipEvent_t e = p->event_for(f.epoch);
  const bool shard_future = f.shard >= 0 && f.node != PW_NODE_RESULT;
  if (shard_future && (uint32_t)f.shard >= p->L.width) return fail(PW_ERR_INVALID, "shard %d outside the future table", f.shard);
  if (shard_future) {
    if ((rc = poll_future(p, f, fired))) return rc;
    if (*fired) return PW_OK;
  }
  hipError_t err = hipEventQuery(e);
  if (err == hipErrorNotReady) return PW_OK;
  if (err != hipSuccess) return hip_fail(err, "hipEventQuery");
  rc = check_fired(p, f);
  if (rc == PW_OK) *fired = 1;
  return rc;
}

int pw_plan_read_futures(pw_plan_t plan, uint32_t* epochs, uint32_t* fires, uint64_t* stamps, size_t capacity,
                         uint32_t* nodes, uint32_t* width) {
  g_last_error.clear();
  Plan* p = reinterpret_cast<Plan*>(plan);
  if (!is_live(p)) return fail(PW_ERR_STATE, "not a live plan");
  std::lock_guard<std::mutex> lk(p->mu);
  if (nodes) *nodes = kNodes;
  if (width) *width = p->L.width;
  const size_t n = (size_t)kNodes * p->L.width;
  if ((epochs || fires || stamps) && capacity < n) return fail(PW_ERR_INVALID, "capacity %zu < %zu", capacity, n);
  if (!p->done.empty()) {
    hipError_t e = hipEventSynchronize(p->done.back().event);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
  }
  if (!p->aux) {
    hipError_t e = hipStreamCreateWithFlags(&p->aux, hipStreamNonBlocking);
    if (e != hipSuccess) return hip_fail(e, "hipStreamCreate");
  }
  auto* base = static_cast<unsigned char*>(p->ws);
  hipError_t e = hipSuccess;
  if (epochs) e = hipMemcpyAsync(epochs, base + p->L.fut, n * 4, hipMemcpyDeviceToHost, p->aux);
  if (e == hipSuccess && fires) e = hipMemcpyAsync(fires, base + p->L.fires, n * 4, hipMemcpyDeviceToHost, p->aux);
  if (e == hipSuccess && stamps) {
    if (!(p->desc.flags & PW_FLAG_TRACE)) return fail(PW_ERR_INVALID, "stamps need PW_FLAG_TRACE");
    e = hipMemcpyAsync(stamps, base + p->L.stamps, n * 8, hipMemcpyDeviceToHost, p->aux);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(p->aux);
  if (e != hipSuccess) return hip_fail(e, "reading the future table");
  return PW_OK;
}

int pw_plan_chain_placement(pw_plan_t plan, uint32_t* xcc, size_t capacity) {
  g_last_error.clear();
  Plan* p = reinterpret_cast<Plan*>(plan);
  if (!is_live(p)) return fail(PW_ERR_STATE, "not a live plan");
  if (p->desc.kind != PW_GRAPH_CHAIN || p->desc.chain_mode != PW_CHAIN_SPLIT)
    return fail(PW_ERR_INVALID, "a CHAIN plan in PW_CHAIN_SPLIT mode is needed");
  const size_t n = (size_t)p->desc.num_shards * 2;
  if (!xcc || capacity < n) return fail(PW_ERR_INVALID, "capacity %zu < %zu", capacity, n);
  std::lock_guard<std::mutex> lk(p->mu);
  if (!p->done.empty()) {
    hipError_t e = hipEventSynchronize(p->done.back().event);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
  }
  hipError_t e = hipMemcpy(xcc, p->base() + p->L.place, n * 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "reading the placement table");
  return PW_OK;
}

int pw_plan_kernel_times(pw_plan_t plan, pw_kernel_time* out, int max, int* n) {
  g_last_error.clear();
  Plan* p = reinterpret_cast<Plan*>(plan);
  if (!is_live(p)) return fail(PW_ERR_STATE, "not a live plan");
  std::lock_guard<std::mutex> lk(p->mu);
  p->resolve_times();
  int i = 0;
  for (auto& kv : p->times) {
    if (out && i < max) {
      pw_kernel_time t{};
      snprintf(t.name, sizeof(t.name), "%s", kv.first.c_str());
      t.launches = kv.second.launches;
      t.total_ms = kv.second.total_ms;
      out[i] = t;
    }
    ++i;
  }
  if (n) *n = i;
  return PW_OK;
}

int pw_plan_reset_times(pw_plan_t plan) {
  g_last_error.clear();
  Plan* p = reinterpret_cast<Plan*>(plan);
  if (!is_live(p)) return fail(PW_ERR_STATE, "not a live plan");
  std::lock_guard<std::mutex> lk(p->mu);
  p->resolve_times();
  p->times.clear();
  return PW_OK;
}

}  // extern "C"

// The status of a call known to have finished (its completion event
// passed): the plan's latched device status, then the future's epoch.
int pw::future_check(pw_future_t f) {
  Plan* p = nullptr;
  int rc = future_common(f, &p);
  if (rc) return rc;
  std::lock_guard<std::mutex> lk(p->mu);
  return check_fired(p, f);
}
