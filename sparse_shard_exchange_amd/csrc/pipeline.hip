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
// ascending, then stage) dealt round-robin to one queue per XCD, each item's
// tiles consecutive. Persistent workgroups claim tiles from their XCD's
// queue. Tile (s, m, r, c) waits for the row-block future (s - 1, m, r) (all
// column tiles of that row block of the previous stage written), so a row
// block flows to the next stage before the rest of its microbatch is done.
#include "device.h"
#include "gemm.h"

namespace pw {

namespace {

__device__ __forceinline__ bool reached(uint32_t v, uint32_t target) { return (int32_t)(v - target) >= 0; }

constexpr uint32_t kNone = 0xFFFFFFFFu;

// Which XCD (accelerator complex die, with its own L2) this wave runs on.
__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v;
}

// Claim the next tile: this XCD's queue first; only once it is empty, the
// other queues in turn. Returns an index into the order table or kNone.
__device__ __forceinline__ uint32_t claim(const PipeArgs& a, uint32_t home) {
  for (uint32_t q = 0; q < a.nq; ++q) {
    const uint32_t qi = (home + q) % a.nq;
    const uint32_t k = __hip_atomic_fetch_add(&a.qctr[qi], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (k < a.qlen[qi]) return a.qstart[qi] + k;
  }
  return kNone;
}

__global__ void k_pipe_reset(PipeArgs a) {
  if (threadIdx.x < a.nq) a.qctr[threadIdx.x] = 0;
}

// Persistent: one workgroup per CU loops over tiles. The plan puts all 32
// tiles of an item in one XCD's queue (items dealt round-robin to the 8
// queues in GPipe order), so the item's activation rows and weight columns
// are shared through that XCD's L2. Each queue is in dependency order and a
// workgroup leaves its own queue only once it is empty, so the earliest
// unfinished tile is always held or next in line: no deadlock.
__global__ __launch_bounds__(256, 1) void k_pipeline(PipeArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __shared__ uint32_t next;
  __shared__ uint32_t go;
  const uint32_t tid = threadIdx.x;
  const uint64_t item_elems = (uint64_t)a.rows * a.d;
  uint32_t home = 0;
  if (tid == 0) {
    home = xcc_id() % a.nq;
    next = claim(a, home);
  }
  __syncthreads();
  while (true) {
    const uint32_t t = next;
    if (t == kNone) break;  // uniform: every thread read the same value
    const uint32_t code = a.order[t];
    const uint32_t s = code & 0xFF, m = (code >> 8) & 0xFF, r = (code >> 16) & 0xFF, c = code >> 24;
    __syncthreads();  // all threads have read `next`
    if (tid == 0) {
      bool ok = true;
      if (s > 0) {  // gate on the row-block future of the previous stage
        const uint32_t* ctr = a.rb_ctr + ((uint64_t)(s - 1) * a.M + m) * a.RB + r;
        if (!reached(__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT), a.rb_target)) {
          const uint64_t t0 = wall_clock64();
          while (true) {
            __builtin_amdgcn_s_sleep(2);
            if (reached(__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT), a.rb_target)) break;
            if (wall_clock64() - t0 > a.f.spin_ticks) {
              latch(a.f.status, ST_TIMEOUT);
              ok = false;
              break;
            }
          }
        }
      }
      go = ok;
      next = claim(a, home);  // claimed now, used after this tile
    }
    __syncthreads();
    if (go) {
      const __bf16* in = s == 0 ? a.x + (uint64_t)m * item_elems : a.acts + ((uint64_t)(s - 1) * a.M + m) * item_elems;
      __bf16* out = a.acts + ((uint64_t)s * a.M + m) * item_elems;
      mm::Tile tile;
      tile.A = in + (uint64_t)r * mm::BM * a.d;
      tile.lda = a.d;
      tile.rows = min((int)mm::BM, (int)a.rows - (int)(r * mm::BM));
      tile.Bt = a.wt + (uint64_t)s * a.d * a.d + (uint64_t)c * mm::BN * a.d;
      tile.ldb = a.d;
      tile.K = a.d;
      mm::f32x16 acc[4][4];
      mm::tile_mma(tile, lds, acc);
      mm::store_tile<true>(acc, lds, out + (uint64_t)r * mm::BM * a.d + (uint64_t)c * mm::BN, a.d, tile.rows);
    }
    // publish: every wave's stores complete, then one release per tile. A tile
    // whose wait expired still counts, so nothing downstream waits forever.
    mm::wait_stores();
    __syncthreads();
    if (tid == 0) {
      uint32_t* ctr = a.rb_ctr + ((uint64_t)s * a.M + m) * a.RB + r;
      const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      if (reached(old + 1, a.rb_target)) {  // row block complete
        uint32_t* ic = a.item_ctr + (uint64_t)s * a.M + m;
        const uint32_t io = __hip_atomic_fetch_add(ic, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (reached(io + 1, a.item_target)) fire(a.f, NODE_STAGE, s * a.M + m, a.epoch, false);
      }
    }
  }
  if (tid == 0) {
    const uint32_t dn = __hip_atomic_fetch_add(a.done_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (reached(dn + 1, a.done_target)) fire(a.f, NODE_RESULT, 0, a.epoch, false);
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
