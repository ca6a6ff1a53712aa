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
// plan uploads one claim order for all tiles, the GPipe lock-step order
// (tick s + m ascending, then stage, row block, column block), and the
// workgroups of one launch claim tiles from a ticket counter in that order (one workgroup per tile; the ticket, not the launch order,
// decides which tile a workgroup computes). Tile (s, m, r, c) waits for the
// row-block future (s - 1, m, r) (all column tiles of that row block of the
// previous stage written), so a row block flows to the next stage before the
// rest of its microbatch is done. Claims are in dependency order and each
// workgroup holds one tile, so every awaited tile was claimed earlier by a
// workgroup that is already running: no deadlock whatever the residency.
#include "device.h"
#include "gemm.h"

namespace pw {

namespace {

__device__ __forceinline__ bool reached(uint32_t v, uint32_t target) { return (int32_t)(v - target) >= 0; }

__global__ __launch_bounds__(256, 1) void k_pipeline(PipeArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __shared__ uint32_t tk;
  __shared__ uint32_t go;
  const uint32_t tid = threadIdx.x;
  const uint64_t item_elems = (uint64_t)a.rows * a.d;
  // Claim the next tile in the plan's order (launch order of workgroups is
  // not the claim order; the ticket is).
  if (tid == 0) tk = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - a.ticket_base;
  __syncthreads();
  const uint32_t t = tk;
  if (t >= a.total_tiles) return;  // cannot happen: one workgroup per tile
  const uint32_t code = a.order[t];
  const uint32_t s = code & 0xFF, m = (code >> 8) & 0xFF, r = (code >> 16) & 0xFF, c = code >> 24;
  // gate on the row-block future of the previous stage
  if (tid == 0) {
    bool ok = true;
    if (s > 0) {
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
  }
  __syncthreads();
  if (go) {
    const __bf16* in = s == 0 ? a.x + (uint64_t)m * item_elems : a.acts + ((uint64_t)(s - 1) * a.M + m) * item_elems;
    __bf16* out = a.acts + ((uint64_t)s * a.M + m) * item_elems;
    mm::Tile tile;
    tile.A = in + (uint64_t)r * mm::BM * a.d;
    tile.lda = a.d;
    tile.rows = min((int)mm::BM, (int)a.rows - (int)(r * mm::BM));
    tile.B = a.w + (uint64_t)s * a.d * a.d + (uint64_t)c * mm::BN;
    tile.ldb = a.d;
    tile.K = a.d;
    mm::f32x16 acc[4][4];
    mm::tile_mma(tile, lds, acc);
    mm::store_tile<true>(acc, out + (uint64_t)r * mm::BM * a.d + (uint64_t)c * mm::BN, a.d, tile.rows);
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
    const uint32_t dn = __hip_atomic_fetch_add(a.done_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (reached(dn + 1, a.done_target)) fire(a.f, NODE_RESULT, 0, a.epoch, false);
  }
}

}  // namespace

hipError_t launch_pipeline(const PipeArgs& a, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k_pipeline, hipFuncAttributeMaxDynamicSharedMemorySize, mm::kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(k_pipeline, dim3(a.total_tiles), dim3(mm::NT), mm::kLdsBytes, s, a);
  return hipGetLastError();
}

}  // namespace pw
