// CHAIN, MOE and PIPELINE programs of the pw library (host side).
#include <hip/hip_runtime.h>

#include "runtime.h"

namespace pw {

int validate_desc_more(const pw_plan_desc* d) {
  switch (d->kind) {
    case PW_GRAPH_CHAIN:
    case PW_GRAPH_MOE:
    case PW_GRAPH_PIPELINE:
      return fail(PW_ERR_UNSUPPORTED, "graph kind %u is not built yet", d->kind);
    default:
      return fail(PW_ERR_INVALID, "unknown graph kind %u", d->kind);
  }
}

int plan_init_kind(Plan*) { return PW_OK; }
void plan_release_kind(Plan*) {}

int run_moe(Plan*, const pw_exchange_io*, hipStream_t, pw_future_t*) {
  return fail(PW_ERR_UNSUPPORTED, "MOE is not built yet");
}
int run_chain(Plan*, uint64_t, pw_sharded_buf*, void*, hipStream_t, pw_future_t*) {
  return fail(PW_ERR_UNSUPPORTED, "CHAIN is not built yet");
}
int run_pipeline(Plan*, uint64_t, pw_sharded_buf*, void*, hipStream_t, pw_future_t*) {
  return fail(PW_ERR_UNSUPPORTED, "PIPELINE is not built yet");
}

}  // namespace pw
