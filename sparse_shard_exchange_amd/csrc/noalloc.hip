// pw_exchange_scratch: the EXCHANGE step of pw_exchange with no plan and no
// workspace, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// The step's tables (status and future words, arrival counters, segment
// offsets, the tile x destination count tables, the in-tile ranks) live in
// one file-scope device array, `scratch`, of kScratchBytes per GPU, which the
// code object holds from the library's load until the process ends. The
// kernels are pw_exchange's own (exchange.hip); only where their tables live
// differs. Every call on a GPU uses that GPU's copy of the array and leaves
// its contents behind: each call first clears, with a fill kernel on the
// caller's stream (no memset node, so the call can be captured), the words
// that must start at zero (status, control counters, future table); the other
// tables are fully written by the step before they are read. Calls that
// overlap on one GPU (two streams, two threads) race on the array.
#include "device.h"
#include "runtime.h"

#include <mutex>

namespace pw {

namespace {

constexpr size_t kScratchBytes = (size_t)8 << 20;

// The array itself. In host code its name is a host-side stand-in, not a
// device address: host code only ever uses the address hipGetSymbolAddress
// returned for the current device (scratch_ptr below).
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this GPU's copy of `scratch`, looked up once per
// device, with that device current.
int scratch_ptr(int dev, unsigned char** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(PW_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(PW_ERR_DEVICE, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<unsigned char*>(g_scratch_ptr[dev]);
  return PW_OK;
}

// Zero n 16-byte words (the scratch array is 256-byte aligned and the region
// cleared is a multiple of 256 bytes).
__global__ __launch_bounds__(256) void k_clear(uint4* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = uint4{0, 0, 0, 0};
}

}  // namespace

}  // namespace pw

using namespace pw;

extern "C" int pw_exchange_scratch(const pw_plan_desc* d, const pw_exchange_io* io, void* stream) {
  clear_error();
  int st = validate_desc(d);
  if (st) return st;
  if (d->kind != PW_GRAPH_EXCHANGE) return fail(PW_ERR_INVALID, "pw_exchange_scratch takes an EXCHANGE descriptor");
  if (d->flags) return fail(PW_ERR_INVALID, "pw_exchange_scratch takes no flags (no trace, no timing)");
  if (!io) return fail(PW_ERR_INVALID, "io is NULL");
  Layout L;
  if ((st = plan_layout(*d, L))) return st;
  if (L.total > kScratchBytes)
    return fail(PW_ERR_INVALID, "this exchange needs %zu bytes of tables; the static scratch holds %zu (use pw_plan "
                "and pw_exchange with a workspace)", L.total, kScratchBytes);
  if ((st = validate_exchange_io(*d, L, io, true, L.G))) return st;
  if (L.G && !io->dst.shard_offsets)
    return fail(PW_ERR_INVALID, "dst.shard_offsets is required: it reports the tuples placed (dropped = G - offsets[N])");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  unsigned char* base = nullptr;
  if ((st = scratch_ptr(dev, &base))) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);

  // status, control counters and the future table (the first tables of the
  // layout) start at zero; the step uses epoch 1
  Futures f{};
  f.status = reinterpret_cast<uint64_t*>(base + L.ctl);
  f.epoch = reinterpret_cast<uint32_t*>(base + L.fut);
  f.fires = reinterpret_cast<uint32_t*>(base + L.fires);
  f.stamps = nullptr;
  f.width = L.width;
  const uint64_t ns = d->spin_limit_ns ? d->spin_limit_ns : 2000000000ull;
  f.spin_ticks = (uint32_t)std::min<uint64_t>(0xffffffffull, ns / 10);
  f.call_epoch = 1;
  const uint32_t words = (uint32_t)(L.arrived / 16);  // [0, arrived): ctl, fut, fires (256-byte aligned)
  hipLaunchKernelGGL(k_clear, dim3(std::min<uint32_t>(64, (words + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<uint4*>(base), words);
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "launch clear");

  ExchangeArgs a;
  exchange_args(*d, L, base, io, 1u, f, a);
  if (io->counts && (e = launch_src_counts(a, s)) != hipSuccess) return hip_fail(e, "launch src_counts");
  if ((e = launch_rank(a, s)) != hipSuccess) return hip_fail(e, "launch rank");
  if (!a.fuse_scan && (e = launch_scan(a, s)) != hipSuccess) return hip_fail(e, "launch scan");
  if ((e = launch_scatter(a, s)) != hipSuccess) return hip_fail(e, "launch scatter");
  if (a.b_gated && (e = launch_b(a, s)) != hipSuccess) return hip_fail(e, "launch b");
  return PW_OK;
}
