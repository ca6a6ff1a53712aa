// Multi-tenant scheduler: programs of several clients gang-scheduled onto
// the whole GPU in proportional shares.
//
// PATHWAYS page ("PATHWAYS: Asynchronous Distributed Dataflow for ML"),
// section 5.2 "Multi-tenancy" with Figures 8 and 9, Appendix D with
// Figure 11: the accelerators are time-multiplexed among the programs of
// concurrent clients, each program runs on all cores, programs interleave at
// (sub-)millisecond granularity, and the scheduler controls the accelerator
// time each client gets (proportional shares such as 1:2:4:8).
//
// On one GPU a program (a chain run, an exchange step) already uses every
// CU, so gang scheduling is running programs one after another on one
// stream. The scheduler owns that stream and one dispatch thread. The
// policy is stride scheduling in integers (the pages name no policy): the
// client with the smallest pass among those with queued programs goes next
// (ties: lowest client number) and its pass grows by cost * floor(2^32 / w);
// a client whose queue ran empty resumes at max(its pass, the pass of the
// last dispatch), so idle time earns no credit. At most max_inflight
// programs sit on the device at a time, so the host-side order is the
// device-side order within that window. Each program is bracketed by two
// timing events; the records give its device start and end.
#include <hip/hip_runtime.h>

#include <chrono>
#include <condition_variable>
#include <deque>
#include <mutex>
#include <string>
#include <thread>
#include <unordered_map>
#include <vector>

#include "pw.h"
#include "runtime.h"

namespace pw {

namespace {

constexpr uint64_t kStrideOne = 1ull << 32;
constexpr uint32_t kMaxCost = 1u << 20;
constexpr uint32_t kMaxWeight = 1u << 16;
constexpr uint64_t kRebase = 1ull << 62;  // passes stay below 2^62 + 2^52
constexpr size_t kMaxRecords = 1u << 20;  // unread records beyond this are dropped, oldest first

struct Queued {
  uint64_t ticket;
  pw_program prog;
};

struct Client {
  uint64_t stride = 0;
  uint64_t pass = 0;
  std::deque<Queued> queue;
};

struct Ticket {
  enum State { kQueued, kRunning, kDone } state = kQueued;
  int status = PW_OK;
  std::string error;  // the launch call's error text
  pw_future_t done{};
};

struct InFlight {
  uint64_t ticket;
  uint32_t client;
  uint64_t dispatch;
  hipEvent_t e0, e1;
  int status;
};

}  // namespace
}  // namespace pw

struct pw_sched_s {
  int device = -1;
  hipStream_t stream = nullptr;
  uint32_t max_inflight = 1;

  std::mutex mu;
  std::condition_variable cv_work;  // dispatcher: programs queued, hold lifted, stop
  std::condition_variable cv_done;  // waiters: a program finished
  std::vector<pw::Client> clients;
  std::unordered_map<uint64_t, pw::Ticket> tickets;  // node-based: references stay valid
  std::deque<pw_sched_record> records;
  uint64_t vtime = 0, next_ticket = 1, dispatched = 0;
  size_t queued = 0;
  bool hold = false, stop = false;
  std::string thread_error;  // a HIP failure of the dispatch thread itself

  // dispatch thread only
  std::deque<pw::InFlight> inflight;
  std::vector<hipEvent_t> pool;
  hipEvent_t base = nullptr;  // recorded before the first dispatch
  bool based = false;
  std::thread th;
};

namespace pw {
namespace {

using Sched = pw_sched_s;

hipEvent_t take_event(Sched* s) {
  if (!s->pool.empty()) {
    hipEvent_t e = s->pool.back();
    s->pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Pick and launch one program. Called with the lock held and at least one
// queued program; returns with the lock held.
void dispatch_one(Sched* s, std::unique_lock<std::mutex>& lk) {
  uint32_t best = UINT32_MAX;
  for (uint32_t c = 0; c < s->clients.size(); ++c)
    if (!s->clients[c].queue.empty() && (best == UINT32_MAX || s->clients[c].pass < s->clients[best].pass)) best = c;
  Client& cl = s->clients[best];
  Queued q = cl.queue.front();
  cl.queue.pop_front();
  --s->queued;
  s->vtime = cl.pass;
  cl.pass += (uint64_t)q.prog.cost * cl.stride;
  if (s->vtime >= kRebase) {  // order-preserving: every queued client's pass is >= vtime
    for (auto& c : s->clients) c.pass = c.pass > s->vtime ? c.pass - s->vtime : 0;
    s->vtime = 0;
  }
  Ticket& tk = s->tickets[q.ticket];
  tk.state = Ticket::kRunning;
  const uint64_t index = s->dispatched++;
  lk.unlock();

  int rc = PW_OK;
  std::string err;
  pw_future_t done{};
  hipEvent_t e0 = take_event(s), e1 = take_event(s);
  if (!s->based && s->base == nullptr) {
    if (hipEventCreate(&s->base) != hipSuccess) s->base = nullptr;
  }
  if (!e0 || !e1 || !s->base) {
    rc = PW_ERR_DEVICE;
    err = "hipEventCreate failed in the dispatch thread";
  } else {
    if (!s->based) {
      (void)hipEventRecord(s->base, s->stream);
      s->based = true;
    }
    (void)hipEventRecord(e0, s->stream);
    if (q.prog.kind == PW_PROG_CHAIN) {
      pw_sharded_buf st = q.prog.state;
      rc = pw_chain_run(q.prog.plan, q.prog.steps, &st, q.prog.aux, s->stream, &done);
    } else {
      rc = pw_exchange(q.prog.plan, &q.prog.io, s->stream, &done);
    }
    if (rc != PW_OK) err = pw_last_error();
    (void)hipEventRecord(e1, s->stream);
  }

  lk.lock();
  tk.status = rc;
  tk.error = err;
  tk.done = done;
  if (e0 && e1) {
    s->inflight.push_back({q.ticket, best, index, e0, e1, rc});
  } else {  // nothing enqueued: finished now
    if (e0) s->pool.push_back(e0);
    if (e1) s->pool.push_back(e1);
    tk.state = Ticket::kDone;
    s->records.push_back({q.ticket, best, rc, index, 0.0, 0.0});
    s->cv_done.notify_all();
  }
}

// Retire finished programs, oldest first (one stream: they finish in order).
// Called with the lock held.
void retire(Sched* s, std::unique_lock<std::mutex>& lk) {
  while (!s->inflight.empty()) {
    InFlight f = s->inflight.front();
    lk.unlock();
    hipError_t q = hipEventQuery(f.e1);
    float t0 = 0.f, t1 = 0.f;
    if (q == hipSuccess) {
      (void)hipEventElapsedTime(&t0, s->base, f.e0);
      (void)hipEventElapsedTime(&t1, s->base, f.e1);
    }
    lk.lock();
    if (q == hipErrorNotReady) return;
    s->inflight.pop_front();
    s->pool.push_back(f.e0);
    s->pool.push_back(f.e1);
    auto it = s->tickets.find(f.ticket);
    if (it != s->tickets.end()) {
      it->second.state = Ticket::kDone;
      if (q != hipSuccess && it->second.status == PW_OK) {
        it->second.status = PW_ERR_DEVICE;
        it->second.error = std::string("hipEventQuery: ") + hipGetErrorString(q);
      }
    }
    s->records.push_back({f.ticket, f.client, f.status, f.dispatch, (double)t0, (double)t1});
    while (s->records.size() > kMaxRecords) s->records.pop_front();
    s->cv_done.notify_all();
  }
}

void dispatch_loop(Sched* s) {
  if (hipSetDevice(s->device) != hipSuccess) {
    std::lock_guard<std::mutex> g(s->mu);
    s->thread_error = "hipSetDevice failed in the dispatch thread";
  }
  std::unique_lock<std::mutex> lk(s->mu);
  while (true) {
    retire(s, lk);
    if (!s->hold && s->queued > 0 && s->inflight.size() < s->max_inflight) {
      dispatch_one(s, lk);
      continue;
    }
    if (s->inflight.empty()) {
      if (s->stop && s->queued == 0) break;
      s->cv_work.wait(lk);  // nothing on the device: sleep until a submission, a lifted hold or stop
      continue;
    }
    // programs on the device and nothing to dispatch: poll their completion
    lk.unlock();
    std::this_thread::yield();
    lk.lock();
  }
}

}  // namespace
}  // namespace pw

using pw::fail;

int pw_sched_create(uint32_t max_inflight, pw_sched_t* out) {
  pw::clear_error();
  if (!out) return fail(PW_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (max_inflight < 1 || max_inflight > 64) return fail(PW_ERR_INVALID, "max_inflight %u outside [1, 64]", max_inflight);
  auto* s = new pw_sched_s();
  s->max_inflight = max_inflight;
  hipError_t e = hipGetDevice(&s->device);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&s->stream, hipStreamNonBlocking);
  if (e != hipSuccess) {
    delete s;
    return pw::hip_fail(e, "scheduler stream");
  }
  try {
    s->th = std::thread(pw::dispatch_loop, s);
  } catch (...) {
    (void)hipStreamDestroy(s->stream);
    delete s;
    return fail(PW_ERR_DEVICE, "could not start the dispatch thread");
  }
  *out = s;
  return PW_OK;
}

int pw_sched_add_client(pw_sched_t s, uint32_t weight, uint32_t* client) {
  pw::clear_error();
  if (!s || !client) return fail(PW_ERR_INVALID, "NULL argument");
  if (weight < 1 || weight > pw::kMaxWeight) return fail(PW_ERR_INVALID, "weight %u outside [1, 65536]", weight);
  std::lock_guard<std::mutex> g(s->mu);
  pw::Client c;
  c.stride = pw::kStrideOne / weight;
  c.pass = s->vtime;
  s->clients.push_back(c);
  *client = (uint32_t)(s->clients.size() - 1);
  return PW_OK;
}

int pw_sched_submit(pw_sched_t s, uint32_t client, const pw_program* prog, uint64_t* ticket) {
  pw::clear_error();
  if (!s || !prog || !ticket) return fail(PW_ERR_INVALID, "NULL argument");
  if (prog->kind != PW_PROG_CHAIN && prog->kind != PW_PROG_EXCHANGE) return fail(PW_ERR_INVALID, "program kind %u", prog->kind);
  if (prog->cost < 1 || prog->cost > pw::kMaxCost) return fail(PW_ERR_INVALID, "cost %u outside [1, 2^20]", prog->cost);
  if (!pw::is_live(reinterpret_cast<const pw::Plan*>(prog->plan))) return fail(PW_ERR_STATE, "not a live plan");
  std::lock_guard<std::mutex> g(s->mu);
  if (s->stop) return fail(PW_ERR_STATE, "scheduler is being destroyed");
  if (client >= s->clients.size()) return fail(PW_ERR_INVALID, "client %u of %zu", client, s->clients.size());
  pw::Client& c = s->clients[client];
  if (c.queue.empty() && c.pass < s->vtime) c.pass = s->vtime;  // idle time earns no credit
  const uint64_t t = s->next_ticket++;
  c.queue.push_back({t, *prog});
  s->tickets.emplace(t, pw::Ticket{});
  ++s->queued;
  *ticket = t;
  s->cv_work.notify_one();
  return PW_OK;
}

int pw_sched_wait(pw_sched_t s, uint64_t ticket, int64_t timeout_ns) {
  pw::clear_error();
  if (!s) return fail(PW_ERR_INVALID, "NULL scheduler");
  std::unique_lock<std::mutex> lk(s->mu);
  auto it = s->tickets.find(ticket);
  if (it == s->tickets.end()) return fail(PW_ERR_STATE, "unknown ticket %llu", (unsigned long long)ticket);
  pw::Ticket& tk = it->second;
  auto finished = [&] { return tk.state == pw::Ticket::kDone; };
  if (timeout_ns < 0) {
    s->cv_done.wait(lk, finished);
  } else if (!s->cv_done.wait_for(lk, std::chrono::nanoseconds(timeout_ns), finished)) {
    return fail(PW_ERR_TIMEOUT, "program %llu not finished within %lld ns", (unsigned long long)ticket,
                (long long)timeout_ns);
  }
  const int status = tk.status;
  const std::string err = tk.error;
  const pw_future_t done = tk.done;
  s->tickets.erase(it);
  lk.unlock();
  if (status != PW_OK) return fail(status, "%s", err.c_str());
  return pw::future_check(done);
}

int pw_sched_hold(pw_sched_t s, int hold) {
  pw::clear_error();
  if (!s) return fail(PW_ERR_INVALID, "NULL scheduler");
  std::lock_guard<std::mutex> g(s->mu);
  s->hold = hold != 0;
  s->cv_work.notify_one();
  return PW_OK;
}

int pw_sched_records(pw_sched_t s, pw_sched_record* out, size_t capacity, size_t* n) {
  pw::clear_error();
  if (!s || !n || (capacity && !out)) return fail(PW_ERR_INVALID, "NULL argument");
  std::lock_guard<std::mutex> g(s->mu);
  size_t k = 0;
  while (k < capacity && !s->records.empty()) {
    out[k++] = s->records.front();
    s->records.pop_front();
  }
  *n = k;
  if (!s->thread_error.empty()) return fail(PW_ERR_DEVICE, "%s", s->thread_error.c_str());
  return PW_OK;
}

int pw_sched_destroy(pw_sched_t s) {
  pw::clear_error();
  if (!s) return fail(PW_ERR_INVALID, "NULL scheduler");
  {
    std::lock_guard<std::mutex> g(s->mu);
    s->stop = true;
    s->hold = false;
    s->cv_work.notify_one();
  }
  if (s->th.joinable()) s->th.join();
  for (auto e : s->pool) (void)hipEventDestroy(e);
  if (s->base) (void)hipEventDestroy(s->base);
  (void)hipStreamSynchronize(s->stream);
  (void)hipStreamDestroy(s->stream);
  delete s;
  return PW_OK;
}
