// HBM object store: buffers held in device memory, named by handle, labelled
// with an owner, allocated with backpressure.
//
// PATHWAYS page ("PATHWAYS: Asynchronous Distributed Dataflow for ML"),
// section 4.6 "Data management": a per-host object store tracks the buffers
// in accelerator memory; clients refer to them by opaque handles; ownership
// labels let the buffers of a failed client or program be garbage
// collected; when an allocation fails because other programs' buffers
// occupy the memory, simple backpressure stalls the computation instead of
// failing it.
//
// One extent of device memory, taken once at creation. Placement is first
// fit by address over the free extents (std::map offset -> length), and a
// freed extent merges with its free neighbours. A request that does not fit
// waits; waiters are served strictly in arrival order, so a large request is
// not starved by small ones. Frees are stream ordered: the extent returns to
// the free list once an event recorded on the caller's stream at the time of
// the free has completed (the work already enqueued that may still use it),
// so an object can be freed right after the launches that use it. Waiting
// allocations poll those events every 20 us while any are outstanding.
#include <hip/hip_runtime.h>

#include <chrono>
#include <condition_variable>
#include <deque>
#include <map>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "pw.h"
#include "runtime.h"

namespace pw {
namespace {

constexpr size_t kAlign = 256;

struct Obj {
  size_t off, len;
  uint32_t owner;
};

struct PendingFree {
  size_t off, len;
  hipEvent_t ev;
};

}  // namespace
}  // namespace pw

struct pw_store_s {
  int device = -1;
  unsigned char* base = nullptr;
  size_t size = 0;

  std::mutex mu;
  std::condition_variable cv;
  std::map<size_t, size_t> free_ext;  // offset -> length; no two adjacent
  std::unordered_map<uint64_t, pw::Obj> live;
  std::vector<pw::PendingFree> pending;
  std::deque<uint64_t> waiters;  // tickets in arrival order
  std::vector<hipEvent_t> pool;
  uint64_t next_obj = 1, next_ticket = 1;
  size_t in_use = 0, pending_bytes = 0;
  uint64_t stalls = 0;
  double stalled_ms = 0;
};

namespace pw {
namespace {

using Store = pw_store_s;

void give_back(Store* s, size_t off, size_t len) {
  auto next = s->free_ext.lower_bound(off);
  if (next != s->free_ext.end() && off + len == next->first) {  // merge with the extent after
    len += next->second;
    next = s->free_ext.erase(next);
  }
  if (next != s->free_ext.begin()) {
    auto prev = std::prev(next);
    if (prev->first + prev->second == off) {  // merge with the extent before
      prev->second += len;
      return;
    }
  }
  s->free_ext.emplace(off, len);
}

// First fit by address; returns false if no extent is long enough.
bool take(Store* s, size_t len, size_t* off) {
  for (auto it = s->free_ext.begin(); it != s->free_ext.end(); ++it) {
    if (it->second < len) continue;
    *off = it->first;
    const size_t rest = it->second - len, at = it->first + len;
    s->free_ext.erase(it);
    if (rest) s->free_ext.emplace(at, rest);
    return true;
  }
  return false;
}

// Return the extents of completed stream-ordered frees. Lock held.
bool reclaim(Store* s) {
  bool any = false;
  for (size_t i = 0; i < s->pending.size();) {
    PendingFree& p = s->pending[i];
    if (hipEventQuery(p.ev) == hipErrorNotReady) {
      ++i;
      continue;
    }
    give_back(s, p.off, p.len);
    s->pending_bytes -= p.len;
    s->pool.push_back(p.ev);
    p = s->pending.back();
    s->pending.pop_back();
    any = true;
  }
  return any;
}

// Free one object: its extent comes back once the work enqueued on `stream`
// so far has finished. Lock held.
int release(Store* s, uint64_t obj, hipStream_t stream) {
  auto it = s->live.find(obj);
  if (it == s->live.end()) return fail(PW_ERR_STATE, "object %llu is not live in this store", (unsigned long long)obj);
  hipEvent_t ev = nullptr;
  if (!s->pool.empty()) {
    ev = s->pool.back();
    s->pool.pop_back();
  } else {
    hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
  }
  hipError_t e = hipEventRecord(ev, stream);
  if (e != hipSuccess) {
    s->pool.push_back(ev);
    return hip_fail(e, "hipEventRecord");
  }
  const Obj o = it->second;
  s->live.erase(it);
  s->in_use -= o.len;
  s->pending.push_back({o.off, o.len, ev});
  s->pending_bytes += o.len;
  return PW_OK;
}

}  // namespace
}  // namespace pw

using pw::fail;

int pw_store_create(size_t bytes, pw_store_t* out) {
  pw::clear_error();
  if (!out) return fail(PW_ERR_INVALID, "out is NULL");
  *out = nullptr;
  bytes -= bytes % pw::kAlign;
  if (bytes == 0) return fail(PW_ERR_INVALID, "a store needs at least %zu bytes", pw::kAlign);
  auto* s = new pw_store_s();
  hipError_t e = hipGetDevice(&s->device);
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&s->base), bytes);
  if (e != hipSuccess) {
    delete s;
    return e == hipErrorOutOfMemory ? fail(PW_ERR_NOMEM, "hipMalloc of %zu bytes", bytes) : pw::hip_fail(e, "store");
  }
  s->size = bytes;
  s->free_ext.emplace(0, bytes);
  *out = s;
  return PW_OK;
}

int pw_store_alloc(pw_store_t s, size_t bytes, uint32_t owner, int64_t timeout_ns, uint64_t* object, void** device_ptr) {
  pw::clear_error();
  if (!s || !object || !device_ptr) return fail(PW_ERR_INVALID, "NULL argument");
  const size_t len = (std::max<size_t>(bytes, 1) + pw::kAlign - 1) / pw::kAlign * pw::kAlign;
  if (len > s->size) return fail(PW_ERR_NOMEM, "%zu bytes exceed the whole store (%zu)", bytes, s->size);
  const auto t0 = std::chrono::steady_clock::now();
  std::unique_lock<std::mutex> lk(s->mu);
  const uint64_t ticket = s->next_ticket++;
  s->waiters.push_back(ticket);
  bool stalled = false;
  while (true) {
    pw::reclaim(s);
    size_t off = 0;
    if (s->waiters.front() == ticket && pw::take(s, len, &off)) {
      s->waiters.pop_front();
      const uint64_t id = s->next_obj++;
      s->live.emplace(id, pw::Obj{off, len, owner});
      s->in_use += len;
      if (stalled) {
        ++s->stalls;
        s->stalled_ms += std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
      }
      *object = id;
      *device_ptr = s->base + off;
      s->cv.notify_all();  // the next waiter may fit too
      return PW_OK;
    }
    const int64_t el = std::chrono::duration_cast<std::chrono::nanoseconds>(std::chrono::steady_clock::now() - t0).count();
    if (timeout_ns >= 0 && el >= timeout_ns) {
      for (auto it = s->waiters.begin(); it != s->waiters.end(); ++it)
        if (*it == ticket) {
          s->waiters.erase(it);
          break;
        }
      if (stalled) {
        ++s->stalls;
        s->stalled_ms += (double)el * 1e-6;
      }
      s->cv.notify_all();
      return fail(PW_ERR_NOMEM, "%zu bytes not available within %lld ns (in use %zu, freeing %zu of %zu)", bytes,
                  (long long)timeout_ns, s->in_use, s->pending_bytes, s->size);
    }
    stalled = true;
    // frees in flight complete without a notification: poll them
    auto wait = std::chrono::nanoseconds(s->pending.empty() ? 1000000000ll : 20000ll);
    if (timeout_ns >= 0) wait = std::min(wait, std::chrono::nanoseconds(timeout_ns - el));
    s->cv.wait_for(lk, wait);
  }
}

int pw_store_free(pw_store_t s, uint64_t object, void* stream) {
  pw::clear_error();
  if (!s) return fail(PW_ERR_INVALID, "NULL store");
  std::lock_guard<std::mutex> g(s->mu);
  const int rc = pw::release(s, object, static_cast<hipStream_t>(stream));
  s->cv.notify_all();
  return rc;
}

int pw_store_release_owner(pw_store_t s, uint32_t owner, void* stream, uint64_t* released) {
  pw::clear_error();
  if (!s) return fail(PW_ERR_INVALID, "NULL store");
  std::lock_guard<std::mutex> g(s->mu);
  std::vector<uint64_t> ids;
  for (const auto& kv : s->live)
    if (kv.second.owner == owner) ids.push_back(kv.first);
  uint64_t n = 0;
  int rc = PW_OK;
  for (uint64_t id : ids) {
    if ((rc = pw::release(s, id, static_cast<hipStream_t>(stream)))) break;
    ++n;
  }
  if (released) *released = n;
  s->cv.notify_all();
  return rc;
}

int pw_store_get_stats(pw_store_t s, pw_store_stats* out) {
  pw::clear_error();
  if (!s || !out) return fail(PW_ERR_INVALID, "NULL argument");
  std::lock_guard<std::mutex> g(s->mu);
  pw::reclaim(s);
  size_t largest = 0;
  for (const auto& kv : s->free_ext) largest = std::max(largest, kv.second);
  out->base = reinterpret_cast<uint64_t>(s->base);
  out->capacity = s->size;
  out->in_use = s->in_use;
  out->pending_free = s->pending_bytes;
  out->largest_free = largest;
  out->objects = s->live.size();
  out->waiting = s->waiters.size();
  out->stalls = s->stalls;
  out->stalled_ms = s->stalled_ms;
  return PW_OK;
}

int pw_store_destroy(pw_store_t s) {
  pw::clear_error();
  if (!s) return fail(PW_ERR_INVALID, "NULL store");
  {
    std::lock_guard<std::mutex> g(s->mu);
    if (!s->waiters.empty()) return fail(PW_ERR_STATE, "allocations are waiting on this store");
  }
  for (auto& p : s->pending) {
    (void)hipEventSynchronize(p.ev);
    (void)hipEventDestroy(p.ev);
  }
  for (auto e : s->pool) (void)hipEventDestroy(e);
  (void)hipFree(s->base);
  delete s;
  return PW_OK;
}
