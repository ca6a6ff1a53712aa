// Host-side plan object of the pw library (internal).
#pragma once

#include <hip/hip_runtime.h>

#include <deque>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "pw.h"
#include "internal.h"

namespace pw {

// Byte offsets of the tables a plan keeps in the caller's workspace.
struct Layout {
  size_t ctl = 0;         // 256 B: [0] status word, [64..] control counters
  size_t fut = 0;         // [kNodes][width] u32 epochs
  size_t fires = 0;       // [kNodes][width] u32 fire counts
  size_t stamps = 0;      // [kNodes][width] u64 (PW_FLAG_TRACE)
  size_t arrived = 0, expected = 0, b_arrived = 0;  // [N] u32
  size_t seg = 0;         // [N+1] i64 segment offsets
  size_t tile_base = 0;   // [num_tiles][N] u32
  size_t blk_base = 0;    // [num_blk][N] u32
  size_t tile_cnt = 0;    // [num_tiles][N] u32
  size_t tile_done = 0;   // [num_tiles] u32
  size_t rank = 0;        // [G] u16
  size_t slab_cnt = 0;    // [grid][N] u64 (one-launch path): count | call << 32
  size_t small_tab = 0;   // [2][2N + 1] u32 (one-launch path counters, by call parity)
  size_t experts = 0, gates = 0, slot_of = 0, hidden_act = 0;  // MOE
  size_t rb_start = 0, b_done = 0;                              // MOE
  size_t w1t = 0, w2t = 0, wrt = 0;  // packed (K-contiguous) weights: MOE W1^T, W2^T, W_r^T; PIPELINE W^T in w1t
  size_t a_buf = 0;       // CHAIN: A's output buffer
  size_t place = 0;       // CHAIN: [N][2] u32 XCD of the waves that ran A[i] and B[i] (split placement)
  size_t pipe_ctl = 0;    // PIPELINE: [0] ticket, [1] done counter
  size_t rb_ctr = 0, item_ctr = 0, order = 0;  // PIPELINE tables
  size_t total = 0;
  uint64_t G = 0;         // tuples per exchange
  uint32_t tile = 0, num_tiles = 0, width = 0;
  uint32_t scan_tiles = 0, num_blk = 0;  // tiles per scan block, scan blocks
  uint32_t slab = 0, small_grid = 0;     // one-launch path: tuples per workgroup, workgroups (0: none)
};

struct Plan {
  uint64_t id = 0;
  pw_plan_desc desc{};
  Layout L;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  int device = -1;
  uint64_t epoch = 0;     // last epoch launched
  bool small_ok = false;  // EXCHANGE: whole steps run as one co-resident launch
  uint64_t small_calls = 0;  // one-launch calls so far
  std::mutex mu;

  struct Done {
    uint64_t epoch_hi;
    hipEvent_t event;
  };
  std::deque<Done> done;  // completion events of the latest calls
  std::vector<hipEvent_t> done_pool;
  hipStream_t aux = nullptr;  // non-blocking stream for small read-backs
  uint32_t* host_words = nullptr;  // pinned: [0..1] status word, [2] one future epoch, read back together

  struct Pending {
    const char* name;
    hipEvent_t e0, e1;
  };
  struct Acc {
    uint64_t launches = 0;
    double total_ms = 0;
  };
  std::vector<Pending> pending;
  std::vector<hipEvent_t> event_pool;
  std::map<std::string, Acc> times;

  void* kind_state = nullptr;  // per-kind host state

  // Between pw_exchange_begin and pw_exchange_end: the inputs begin was
  // given and the output rows it reported.
  struct Open {
    bool active = false;
    uint64_t rows = 0;
    const void* src = nullptr;
    const int32_t* dest = nullptr;
    float* logits = nullptr;
    int32_t* experts = nullptr;
    float* gates = nullptr;
    int32_t* counts = nullptr;
  } open;

  void launch_begin(const char* name, hipStream_t s);
  void launch_end(hipStream_t s);
  hipEvent_t get_event();
  void resolve_times();
  int begin_call(hipStream_t s);
  int end_call(hipStream_t s, uint64_t epoch_hi);
  hipEvent_t event_for(uint64_t epoch) const;
  Futures futures() const;
  int clear_status();
  int read_status_and_epoch(uint32_t node, uint32_t shard, uint64_t* status, uint32_t* epoch);
  unsigned char* base() const { return static_cast<unsigned char*>(ws); }
};

int fail(int code, const char* fmt, ...);
int hip_fail(hipError_t e, const char* what);
void clear_error();                 // empty this thread's pw_last_error()
bool is_live(const Plan* p);        // the registry holds p
int future_check(pw_future_t f);    // latched device status of a call known to have finished

// graphs.cpp: the CHAIN, MOE and PIPELINE programs.
int validate_desc_more(const pw_plan_desc* d);
int plan_init_kind(Plan* p);
void plan_release_kind(Plan* p);
// A step whole (kAll), or split where its output sizes become known: kBegin
// runs A, the histogram and the scan and returns the segment offsets to the
// host; kEnd runs the rest.
enum class Phase { kAll, kBegin, kEnd };
int run_exchange(Plan* p, const pw_exchange_io* io, hipStream_t s, pw_future_t* done, Phase ph, int64_t* offsets_host);
int plan_layout(const pw_plan_desc& d, Layout& L);
int validate_desc(const pw_plan_desc* d);
int validate_exchange_io(const pw_plan_desc& d, const Layout& L, const pw_exchange_io* io, bool need_dst,
                         uint64_t dst_rows);
void exchange_args(const pw_plan_desc& d, const Layout& L, unsigned char* base, const pw_exchange_io* io,
                   uint32_t epoch, const Futures& f, ExchangeArgs& a);
int run_moe(Plan* p, const pw_exchange_io* io, hipStream_t s, pw_future_t* done, Phase ph, int64_t* offsets_host);
int finish_begin(Plan* p, const pw_exchange_io* io, hipStream_t s, int64_t* offsets_host);
uint64_t moe_static_rows(const pw_plan_desc& d);  // dispatched rows at most (graphs.cpp)
int check_end(Plan* p, const pw_exchange_io* io);
int run_chain(Plan* p, uint64_t steps, pw_sharded_buf* state, void* aux, hipStream_t s, pw_future_t* done);
int run_pipeline(Plan* p, uint64_t steps, pw_sharded_buf* state, void* aux, hipStream_t s, pw_future_t* done);

}  // namespace pw
