// CHAIN, MOE and PIPELINE programs of the pw library (host side).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "runtime.h"

namespace pw {

namespace {

constexpr uint32_t kQueues = 8;  // claim queues at most (one per XCD)

struct KindState {
  uint64_t calls = 0;  // calls launched so far (targets of the cumulative device counters)
  uint32_t grid = 0;   // PIPELINE, MOE: persistent workgroups (one per CU)
  uint32_t nq = 0;     // PIPELINE: claim queues (one per XCD; never more than workgroups)
};

}  // namespace

int validate_desc_more(const pw_plan_desc* d) {
  switch (d->kind) {
    case PW_GRAPH_CHAIN: {
      if (d->num_shards == 0 || d->num_shards > (1u << 20)) return fail(PW_ERR_INVALID, "num_shards must be in [1, 2^20]");
      if (d->tuples_per_shard == 0 || d->tuples_per_shard > (1u << 20))
        return fail(PW_ERR_INVALID, "CHAIN: tuples_per_shard (fp32 elements per shard) must be in [1, 2^20]");
      if ((uint64_t)d->num_shards * d->tuples_per_shard > (1ull << 31))
        return fail(PW_ERR_INVALID, "CHAIN: state larger than 2^31 elements");
      if (d->dtype != PW_F32) return fail(PW_ERR_INVALID, "CHAIN: state must be fp32");
      for (const pw_op* o : {&d->a_op, &d->b_op})
        if (o->kind != PW_OP_IDENTITY && o->kind != PW_OP_AFFINE)
          return fail(PW_ERR_INVALID, "CHAIN: A and B must be IDENTITY or AFFINE");
      if (d->chain_mode > PW_CHAIN_SPLIT) return fail(PW_ERR_INVALID, "CHAIN: unknown chain_mode %u", d->chain_mode);
      return PW_OK;
    }
    case PW_GRAPH_PIPELINE: {
      if (d->num_shards == 0 || d->num_shards > 255) return fail(PW_ERR_INVALID, "PIPELINE: stages must be in [1, 255]");
      if (d->microbatches == 0 || d->microbatches > 255) return fail(PW_ERR_INVALID, "PIPELINE: microbatches must be in [1, 255]");
      if (d->tuples_per_shard == 0 || d->tuples_per_shard > 255 * 256)
        return fail(PW_ERR_INVALID, "PIPELINE: rows per microbatch must be in [1, 65280]");
      if (d->payload_elems == 0 || d->payload_elems % 256 || d->payload_elems > 255 * 256)
        return fail(PW_ERR_INVALID, "PIPELINE: width d must be a positive multiple of 256");
      if (d->dtype != PW_BF16) return fail(PW_ERR_INVALID, "PIPELINE: activations and weights are bf16");
      if (!d->w1) return fail(PW_ERR_INVALID, "PIPELINE: stage weights (w1) are required");
      const uint64_t elems = (uint64_t)d->num_shards * d->microbatches * d->tuples_per_shard * d->payload_elems;
      if (elems > (1ull << 40)) return fail(PW_ERR_INVALID, "PIPELINE: too large");
      return PW_OK;
    }
    case PW_GRAPH_MOE: {
      if (d->num_shards < 2 || d->num_shards > 64) return fail(PW_ERR_INVALID, "MOE: experts must be in [2, 64]");
      if (d->top_k != 2) return fail(PW_ERR_UNSUPPORTED, "MOE: only top-2 routing is built");
      const uint64_t S = d->num_src_shards ? d->num_src_shards : d->num_shards;
      const uint64_t tokens = S * d->tuples_per_shard;
      if (tokens == 0 || tokens > (1ull << 28)) return fail(PW_ERR_INVALID, "MOE: token count must be in [1, 2^28]");
      // the router keeps W_r^T (64 x d bf16) in one CU's 160 KiB of LDS
      if (d->payload_elems == 0 || d->payload_elems % 256 || d->payload_elems > 1280)
        return fail(PW_ERR_INVALID, "MOE: d must be a positive multiple of 256, <= 1280");
      if (d->hidden == 0 || d->hidden % 256 || d->hidden > 65536)
        return fail(PW_ERR_INVALID, "MOE: hidden must be a positive multiple of 256");
      if (d->dtype != PW_BF16) return fail(PW_ERR_INVALID, "MOE: tokens and weights are bf16");
      if (!d->w_router || !d->w1 || !d->w2) return fail(PW_ERR_INVALID, "MOE: w_router, w1 and w2 are required");
      if ((uint64_t)d->payload_elems * d->hidden * 2 > 0xffffffffull)
        return fail(PW_ERR_INVALID, "MOE: one expert weight must stay below 4 GiB");
      if (d->capacity > 2 * tokens) return fail(PW_ERR_INVALID, "MOE: capacity above the tuple count");
      return PW_OK;
    }
    default:
      return fail(PW_ERR_INVALID, "unknown graph kind %u", d->kind);
  }
}

int plan_init_kind(Plan* p) {
  auto* ks = new KindState();
  p->kind_state = ks;
  if (p->desc.kind == PW_GRAPH_PIPELINE) {
    // Items in GPipe lock-step order (tick t = s + m ascending, then stage),
    // or with PW_FLAG_STAGE_WINDOWS stage by stage within windows of
    // kWindow microbatches (item (s, m) then comes a whole window of items
    // after (s - 1, m), so its input is long complete, and a window's
    // activations stay in the last-level cache), go to one queue per XCD by
    // microbatch: every stage of microbatch m runs on XCD m mod nq, so each
    // activation block is written and read through one L2 and the handoff
    // needs no cache-wide fence. An item's tiles (row block, then column
    // block) stay together in its queue. Both orders keep each stage's
    // microbatches in ascending order and every item after its predecessor
    // stage. Uploaded once.
    const pw_plan_desc& d = p->desc;
    const uint32_t S = d.num_shards, M = d.microbatches;
    const uint32_t RB = (uint32_t)((d.tuples_per_shard + 255) / 256), CT = d.payload_elems / 256;
    int cus = 0;
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, p->device);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    ks->grid = (uint32_t)std::max(1, cus);
    // one queue per XCD: a workgroup owns the queue of the XCD it runs on, so
    // every queue has owners (the grid fills every CU) and an item's tiles
    // share one L2
    int xccs = 0;
    if (hipDeviceGetAttribute(&xccs, hipDeviceAttributeNumberOfXccs, p->device) != hipSuccess || xccs <= 0) xccs = 1;
    // every queue must belong to exactly one XCD (its activations stay in
    // that XCD's L2)
    if ((uint32_t)xccs > kQueues) return fail(PW_ERR_UNSUPPORTED, "PIPELINE: %d XCDs, at most %u supported", xccs, kQueues);
    const uint32_t nq = std::min<uint32_t>((uint32_t)xccs, ks->grid);
    ks->nq = nq;
    std::vector<std::vector<uint32_t>> queues(nq);
    auto deal = [&](uint32_t s, uint32_t m) {
      auto& q = queues[m % nq];
      for (uint32_t r = 0; r < RB; ++r)
        for (uint32_t c = 0; c < CT; ++c) q.push_back(s | m << 8 | r << 16 | c << 24);
    };
    if (d.flags & PW_FLAG_STAGE_WINDOWS) {
      constexpr uint32_t kWindow = 16;
      for (uint32_t w0 = 0; w0 < M; w0 += kWindow)
        for (uint32_t s = 0; s < S; ++s)
          for (uint32_t m = w0; m < std::min(M, w0 + kWindow); ++m) deal(s, m);
    } else {
      for (uint32_t t = 0; t + 1 < S + M; ++t)
        for (uint32_t s = 0; s < S; ++s)
          if (t >= s && t - s < M) deal(s, t - s);
    }
    std::vector<uint32_t> order, head(nq), len(nq);
    order.reserve((size_t)S * M * RB * CT);
    for (uint32_t q = 0; q < nq; ++q) {
      head[q] = (uint32_t)order.size();
      len[q] = (uint32_t)queues[q].size();
      order.insert(order.end(), queues[q].begin(), queues[q].end());
    }
    hipError_t e0 = hipMemcpy(p->base() + p->L.pipe_ctl + 64, head.data(), nq * 4, hipMemcpyHostToDevice);
    if (e0 == hipSuccess) e0 = hipMemcpy(p->base() + p->L.pipe_ctl + 128, len.data(), nq * 4, hipMemcpyHostToDevice);
    if (e0 != hipSuccess) return hip_fail(e0, "uploading the pipeline queues");
    e = hipMemcpy(p->base() + p->L.order, order.data(), order.size() * 4, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "uploading the pipeline order");
    // stage weights [S][d][d] -> packed W_s^T, once
    e = hipDeviceSynchronize();
    if (e == hipSuccess)
      e = launch_pack_t(static_cast<const __bf16*>(d.w1), reinterpret_cast<__bf16*>(p->base() + p->L.w1t), S,
                        d.payload_elems, d.payload_elems, d.payload_elems, nullptr);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "packing the stage weights");
  }
  if (p->desc.kind == PW_GRAPH_CHAIN && p->desc.chain_mode == PW_CHAIN_SPLIT) {
    if (!chain_split_fits(p->device, p->desc.num_shards, (uint32_t)p->desc.tuples_per_shard))
      return fail(PW_ERR_UNSUPPORTED, "CHAIN split placement: %u waves must be resident at once", 2 * p->desc.num_shards);
    int xccs = 0;
    if (hipDeviceGetAttribute(&xccs, hipDeviceAttributeNumberOfXccs, p->device) != hipSuccess || xccs <= 0) xccs = 1;
    ks->nq = (uint32_t)xccs;
  }
  if (p->desc.kind == PW_GRAPH_MOE) {
    // expert and router weights -> packed K-contiguous copies, once
    const pw_plan_desc& d = p->desc;
    const uint32_t E = d.num_shards, D = d.payload_elems, H = d.hidden;
    int cus = 0;
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, p->device);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    ks->grid = (uint32_t)std::max(1, cus);
    e = hipDeviceSynchronize();
    if (e == hipSuccess)
      e = launch_pack_t(static_cast<const __bf16*>(d.w1), reinterpret_cast<__bf16*>(p->base() + p->L.w1t), E, D, H, H,
                        nullptr);
    if (e == hipSuccess)
      e = launch_pack_t(static_cast<const __bf16*>(d.w2), reinterpret_cast<__bf16*>(p->base() + p->L.w2t), E, H, D, D,
                        nullptr);
    if (e == hipSuccess)
      e = launch_pack_t(static_cast<const __bf16*>(d.w_router), reinterpret_cast<__bf16*>(p->base() + p->L.wrt), 1, D,
                        E, 64, nullptr);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "packing the expert weights");
  }
  return PW_OK;
}

void plan_release_kind(Plan* p) {
  delete static_cast<KindState*>(p->kind_state);
  p->kind_state = nullptr;
}

// -------------------------------------------------------------------- MOE
// Rows the dispatch can write at most: every tuple, or with a capacity C
// per expert, E C if that is fewer.
uint64_t moe_static_rows(const pw_plan_desc& d) {
  const uint64_t S = d.num_src_shards ? d.num_src_shards : d.num_shards;
  const uint64_t tuples = 2 * S * d.tuples_per_shard;
  return d.capacity ? std::min<uint64_t>(tuples, (uint64_t)d.num_shards * d.capacity) : tuples;
}

int run_moe(Plan* p, const pw_exchange_io* io, hipStream_t s, pw_future_t* done, Phase ph, int64_t* offsets_host) {
  const pw_plan_desc& d = p->desc;
  const Layout& L = p->L;
  const uint32_t E = d.num_shards;
  const uint32_t S = d.num_src_shards ? d.num_src_shards : E;
  const uint64_t tokens = (uint64_t)S * d.tuples_per_shard;
  const uint32_t D = d.payload_elems;
  const bool outs = ph != Phase::kBegin;  // the second half writes dst, b_out and result
  const uint64_t rows = ph == Phase::kEnd ? p->open.rows : moe_static_rows(d);
  if (!io->src.base || io->src.num_tuples != tokens || io->src.elems_per_tuple != D || io->src.dtype != PW_BF16)
    return fail(PW_ERR_INVALID, "src must be %llu tokens x %u bf16", (unsigned long long)tokens, D);
  if (outs && (!io->dst.base || io->dst.num_tuples < rows || io->dst.elems_per_tuple != D || io->dst.dtype != PW_BF16))
    return fail(PW_ERR_INVALID, "dst must hold %llu dispatched rows of %u bf16", (unsigned long long)rows, D);
  if (outs && (!io->b_out || !io->result)) return fail(PW_ERR_INVALID, "b_out (expert outputs) and result are required");
  if (io->dest) return fail(PW_ERR_INVALID, "MOE routes with its router: dest must be NULL");
  const uintptr_t al = outs ? ((uintptr_t)io->src.base | (uintptr_t)io->dst.base | (uintptr_t)io->b_out |
                               (uintptr_t)io->result)
                            : (uintptr_t)io->src.base;
  if (al & 15u) return fail(PW_ERR_INVALID, "buffers must be 16-byte aligned");
  int st = ph == Phase::kEnd ? check_end(p, io) : PW_OK;
  if (st) return st;
  if ((st = p->begin_call(s))) return st;
  unsigned char* base = p->base();

  MoeArgs m{};
  m.x = static_cast<const __bf16*>(io->src.base);
  m.w1t = reinterpret_cast<const __bf16*>(base + L.w1t);
  m.w2t = reinterpret_cast<const __bf16*>(base + L.w2t);
  m.wrt = reinterpret_cast<const __bf16*>(base + L.wrt);
  m.xd = static_cast<__bf16*>(io->dst.base);
  m.h = reinterpret_cast<__bf16*>(base + L.hidden_act);
  m.y = static_cast<__bf16*>(io->b_out);
  m.out = static_cast<__bf16*>(io->result);
  m.logits = io->logits;
  m.experts = io->experts ? io->experts : reinterpret_cast<int32_t*>(base + L.experts);
  m.gates = io->gates ? io->gates : reinterpret_cast<float*>(base + L.gates);
  m.slot_of = reinterpret_cast<int32_t*>(base + L.slot_of);
  m.tokens = tokens;
  m.d = D;
  m.hidden = d.hidden;
  m.E = E;
  m.max_row_blocks = (uint32_t)((moe_static_rows(d) + 255) / 256 + E);
  m.seg = reinterpret_cast<const int64_t*>(base + L.seg);
  m.rb_start = reinterpret_cast<uint32_t*>(base + L.rb_start);
  m.b_done = reinterpret_cast<uint32_t*>(base + L.b_done);
  m.ctl = reinterpret_cast<uint32_t*>(base + L.ctl + 64);
  m.epoch = (uint32_t)(p->epoch + 1);
  m.f = p->futures();

  ExchangeArgs a{};
  a.src = static_cast<const unsigned char*>(io->src.base);
  a.dest = m.experts;
  a.dst = static_cast<unsigned char*>(io->dst.base);
  a.src_index = io->src_index;
  a.slot_of = m.slot_of;
  a.counts = io->counts;
  a.offsets_out = io->dst.shard_offsets;
  a.b_out = nullptr;
  a.G = L.G;
  a.dst_rows = outs ? std::min<uint64_t>(io->dst.num_tuples, L.G) : 0;  // also bounds src_index (G entries)
  a.capacity = d.capacity;
  a.T = 2 * d.tuples_per_shard;
  a.N = E;
  a.num_src = S;
  a.row_bytes = 2 * D;
  a.fanout = 2;
  a.tile = L.tile;
  a.num_tiles = L.num_tiles;
  a.scan_tiles = L.scan_tiles;
  a.num_blk = L.num_blk;
  a.nbits = 0;
  while ((1u << a.nbits) < E) ++a.nbits;
  a.is_f32 = 0;
  a.a_kind = OP_IDENTITY;
  a.b_kind = OP_IDENTITY;
  a.epoch = m.epoch;
  a.b_gated = 1;  // the expert FFN fires B
  a.f = m.f;
  a.arrived = reinterpret_cast<uint32_t*>(base + L.arrived);
  a.expected = reinterpret_cast<uint32_t*>(base + L.expected);
  a.b_arrived = reinterpret_cast<uint32_t*>(base + L.b_arrived);
  a.ctl = m.ctl;
  a.tile_base = reinterpret_cast<uint32_t*>(base + L.tile_base);
  a.blk_base = reinterpret_cast<uint32_t*>(base + L.blk_base);
  a.tile_cnt = reinterpret_cast<uint32_t*>(base + L.tile_cnt);
  a.tile_done = reinterpret_cast<uint32_t*>(base + L.tile_done);
  a.rank = reinterpret_cast<uint16_t*>(base + L.rank);
  a.chunk = scatter_chunk(L.tile, a.row_bytes, a.fanout);
  a.seg = reinterpret_cast<int64_t*>(base + L.seg);

  hipError_t e = hipSuccess;
#define PW_STEP(label, call)           \
  do {                                 \
    p->launch_begin(label, s);         \
    e = (call);                        \
    p->launch_end(s);                  \
    if (e != hipSuccess) return hip_fail(e, "launch " label); \
  } while (0)
  if (ph != Phase::kEnd) {
    PW_STEP("router", launch_router(m, s));
    if (io->counts) PW_STEP("src_counts", launch_src_counts(a, s));
    PW_STEP("rank", launch_rank(a, s));
    PW_STEP("scan", launch_scan(a, s));
    if (ph == Phase::kBegin) return finish_begin(p, io, s, offsets_host);
  }
  p->open.active = false;
  PW_STEP("scatter", launch_scatter(a, s));
  PW_STEP("moe_prefix", launch_moe_prefix(m, s));
  const uint32_t cus = static_cast<KindState*>(p->kind_state)->grid;
  PW_STEP("ffn1", launch_ffn(m, false, cus, s));
  PW_STEP("ffn2", launch_ffn(m, true, cus, s));
  PW_STEP("combine", launch_combine(m, s));
#undef PW_STEP
  p->epoch += 1;
  st = p->end_call(s, p->epoch);
  if (st) return st;
  if (done) *done = pw_future_t{p->id, PW_NODE_RESULT, -1, p->epoch};
  return PW_OK;
}

// ------------------------------------------------------------------ CHAIN
int run_chain(Plan* p, uint64_t steps, pw_sharded_buf* state, void* aux, hipStream_t s, pw_future_t* done) {
  const pw_plan_desc& d = p->desc;
  if (!state || !state->base) return fail(PW_ERR_INVALID, "state is required");
  if (state->num_tuples != d.num_shards || state->elems_per_tuple != d.tuples_per_shard || state->dtype != PW_F32)
    return fail(PW_ERR_INVALID, "state must be %u shards x one tuple of %llu fp32", d.num_shards,
                (unsigned long long)d.tuples_per_shard);
  if (steps == 0) return fail(PW_ERR_INVALID, "steps must be >= 1");
  if ((uintptr_t)state->base % 16 || (uintptr_t)aux % 16)
    return fail(PW_ERR_INVALID, "state and aux must be 16-byte aligned");
  if (p->epoch + steps > 0x7fffffffull) return fail(PW_ERR_INVALID, "epoch would pass 2^31");
  int st = p->begin_call(s);
  if (st) return st;
  auto* ks = static_cast<KindState*>(p->kind_state);

  ChainArgs a{};
  a.state = static_cast<float*>(state->base);
  a.abuf = aux ? static_cast<float*>(aux) : reinterpret_cast<float*>(p->base() + p->L.a_buf);
  a.N = d.num_shards;
  a.E = (uint32_t)d.tuples_per_shard;
  a.a_kind = d.a_op.kind; a.a_a = d.a_op.a; a.a_b = d.a_op.b;
  a.b_kind = d.b_op.kind; a.b_a = d.b_op.a; a.b_b = d.b_op.b;
  a.f = p->futures();
  a.done_ctr = reinterpret_cast<uint32_t*>(p->base() + p->L.ctl + 64);
  a.done_target = (uint32_t)((ks->calls + 1) * (uint64_t)d.num_shards);
  a.role_ctr = a.done_ctr + 8;
  a.place = reinterpret_cast<uint32_t*>(p->base() + p->L.place);
  a.nxcc = ks->nq ? ks->nq : 1;

  hipError_t e = hipSuccess;
  if (d.chain_mode == PW_CHAIN_OPBYOP) {
    for (uint64_t j = 1; j <= steps && e == hipSuccess; ++j) {
      a.epoch0 = (uint32_t)(p->epoch + j - 1);
      a.steps = 1;
      a.node = NODE_A;
      uint32_t* dc = a.done_ctr;
      a.done_ctr = nullptr;
      p->launch_begin("chain_node_a", s);
      e = launch_chain(a, 1, s);
      p->launch_end(s);
      if (e != hipSuccess) break;
      a.node = NODE_B;
      a.done_ctr = j == steps ? dc : nullptr;
      p->launch_begin("chain_node_b", s);
      e = launch_chain(a, 1, s);
      p->launch_end(s);
      a.done_ctr = dc;
    }
  } else {
    a.epoch0 = (uint32_t)p->epoch;
    a.steps = (uint32_t)steps;
    const bool fused = d.chain_mode == PW_CHAIN_FUSED, split = d.chain_mode == PW_CHAIN_SPLIT;
    p->launch_begin(fused ? "chain_fused" : split ? "chain_split" : "chain_chained", s);
    e = launch_chain(a, fused ? 2 : split ? 3 : 0, s);
    p->launch_end(s);
  }
  if (e != hipSuccess) return hip_fail(e, "launch chain");
  ks->calls += 1;
  p->epoch += steps;
  st = p->end_call(s, p->epoch);
  if (st) return st;
  if (done) *done = pw_future_t{p->id, PW_NODE_RESULT, -1, p->epoch};
  return PW_OK;
}

// --------------------------------------------------------------- PIPELINE
int run_pipeline(Plan* p, uint64_t steps, pw_sharded_buf* state, void* aux, hipStream_t s, pw_future_t* done) {
  const pw_plan_desc& d = p->desc;
  const uint32_t S = d.num_shards, M = d.microbatches, R = (uint32_t)d.tuples_per_shard, D = d.payload_elems;
  if (steps != 1) return fail(PW_ERR_INVALID, "PIPELINE runs one pass per call (steps = 1)");
  if (!state || !state->base || !aux) return fail(PW_ERR_INVALID, "state (microbatches) and aux (stage outputs) are required");
  if (state->num_tuples != (uint64_t)M * R || state->elems_per_tuple != D || state->dtype != PW_BF16)
    return fail(PW_ERR_INVALID, "state must be %u microbatches x %u rows x %u bf16", M, R, D);
  if (((uintptr_t)state->base | (uintptr_t)aux) & 15u) return fail(PW_ERR_INVALID, "buffers must be 16-byte aligned");
  int st = p->begin_call(s);
  if (st) return st;
  auto* ks = static_cast<KindState*>(p->kind_state);
  const uint32_t RB = (R + 255) / 256, CT = D / 256;
  const uint64_t call = ks->calls + 1;

  PipeArgs a{};
  a.x = static_cast<const __bf16*>(state->base);
  a.acts = static_cast<__bf16*>(aux);
  a.wt = reinterpret_cast<const __bf16*>(p->base() + p->L.w1t);
  a.order = reinterpret_cast<const uint32_t*>(p->base() + p->L.order);
  uint32_t* ctl = reinterpret_cast<uint32_t*>(p->base() + p->L.pipe_ctl);
  a.done_ctr = ctl;
  a.qctr = ctl + 4;
  a.qstart = ctl + 16;
  a.qlen = ctl + 32;
  a.nq = ks->nq;
  a.rb_ctr = reinterpret_cast<uint32_t*>(p->base() + p->L.rb_ctr);
  a.item_ctr = reinterpret_cast<uint32_t*>(p->base() + p->L.item_ctr);
  a.rb_target = (uint32_t)(call * CT);
  a.item_target = (uint32_t)(call * RB);
  a.done_target = (uint32_t)(call * ks->grid);
  a.S = S; a.M = M; a.rows = R; a.d = D; a.RB = RB; a.CT = CT;
  a.epoch = (uint32_t)(p->epoch + 1);
  a.f = p->futures();
  p->launch_begin("pipeline", s);
  hipError_t e = launch_pipeline(a, ks->grid, s);
  p->launch_end(s);
  if (e != hipSuccess) return hip_fail(e, "launch pipeline");
  ks->calls += 1;
  p->epoch += 1;
  st = p->end_call(s, p->epoch);
  if (st) return st;
  if (done) *done = pw_future_t{p->id, PW_NODE_RESULT, -1, p->epoch};
  return PW_OK;
}

}  // namespace pw
