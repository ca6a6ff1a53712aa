// CHAIN, MOE and PIPELINE programs of the pw library (host side).
#include <hip/hip_runtime.h>

#include "runtime.h"

namespace pw {

namespace {

struct KindState {
  uint64_t calls = 0;  // completed-call counter target of the device done counter
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
      if (d->chain_mode > PW_CHAIN_FUSED) return fail(PW_ERR_INVALID, "CHAIN: unknown chain_mode %u", d->chain_mode);
      return PW_OK;
    }
    case PW_GRAPH_MOE:
    case PW_GRAPH_PIPELINE:
      return fail(PW_ERR_UNSUPPORTED, "graph kind %u is not built yet", d->kind);
    default:
      return fail(PW_ERR_INVALID, "unknown graph kind %u", d->kind);
  }
}

int plan_init_kind(Plan* p) {
  p->kind_state = new KindState();
  return PW_OK;
}

void plan_release_kind(Plan* p) {
  delete static_cast<KindState*>(p->kind_state);
  p->kind_state = nullptr;
}

int run_moe(Plan*, const pw_exchange_io*, hipStream_t, pw_future_t*) {
  return fail(PW_ERR_UNSUPPORTED, "MOE is not built yet");
}

// ------------------------------------------------------------------ CHAIN
int run_chain(Plan* p, uint64_t steps, pw_sharded_buf* state, void* aux, hipStream_t s, pw_future_t* done) {
  const pw_plan_desc& d = p->desc;
  if (!state || !state->base) return fail(PW_ERR_INVALID, "state is required");
  if (state->num_tuples != d.num_shards || state->elems_per_tuple != d.tuples_per_shard || state->dtype != PW_F32)
    return fail(PW_ERR_INVALID, "state must be %u shards x one tuple of %llu fp32", d.num_shards,
                (unsigned long long)d.tuples_per_shard);
  if (steps == 0) return fail(PW_ERR_INVALID, "steps must be >= 1");
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
    const bool fused = d.chain_mode == PW_CHAIN_FUSED;
    p->launch_begin(fused ? "chain_fused" : "chain_chained", s);
    e = launch_chain(a, fused ? 2 : 0, s);
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

int run_pipeline(Plan*, uint64_t, pw_sharded_buf*, void*, hipStream_t, pw_future_t*) {
  return fail(PW_ERR_UNSUPPORTED, "PIPELINE is not built yet");
}

}  // namespace pw
