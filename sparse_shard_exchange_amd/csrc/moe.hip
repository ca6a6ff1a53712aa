// Mixture-of-experts step: router + top-2 gate (A), dispatch exchange, expert
// FFN (B) gated on each expert's future, gated combine (Result).
//
// PATHWAYS page ("PATHWAYS: Asynchronous Distributed Dataflow for ML"),
// section 6.3 "Data-dependent vectorized control flow": sub-examples are
// routed by a learned function to the accelerators that hold different
// weights (mixture of experts), which needs fine-grained data-dependent
// exchanges; section 4.3: the exchange with progress tracking; section 4.5:
// when a node's resource needs depend on its predecessor's output the runtime
// schedules it after that output exists. Here the expert segment sizes are
// data dependent, so the FFN launches read them on the device (a row-block
// prefix computed after the exchange) instead of the host sizing them.
//
// Token t emits tuples 2t (top-1 expert) and 2t + 1 (top-2 expert); the
// exchange (exchange.hip) moves token rows into expert segments and records
// slot_of[g], the inverse of the permutation, which the combine reads.
#include <algorithm>

#include "device.h"
#include "gemm.h"

namespace pw {

namespace {

constexpr int kRouterThreads = 512;  // router workgroup: 8 waves, 2 per SIMD, one workgroup per CU
constexpr int kRouterTokens = kRouterThreads;  // 64 tokens per wave in the GEMM, one per thread in the top-2
constexpr int kMaxExperts = 64;
constexpr int kRouterUnroll = 8;  // k-steps of 16 per block of token loads (128 k)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

// logits[t][e] = sum_k x[t][k] w[k][e] with bf16 products and fp32
// accumulation (v_mfma_f32_32x32x16_bf16), then per token: the two largest
// logits (ties to the lower expert id), gates = softmax over those two.
// LDS holds the packed W^T ([64][d], k contiguous, 16-byte chunks swizzled by
// row), then is reused for the logits of the workgroup's tokens.
//
// The token rows stream from HBM once, in blocks of kRouterUnroll k-steps
// (128 k): each lane keeps two blocks of 16-byte loads in registers, and the
// loads of block s + 1 are issued before the MFMAs of block s, so a wave
// never waits a whole memory round trip between blocks. Block 0's loads are
// issued before the W^T fill. kBlocks = d / 128 (d a multiple of 256).
template <int kBlocks>
__global__ __launch_bounds__(kRouterThreads, 1) void k_router(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int d = (int)a.d, E = (int)a.E;
  const int chunks = d / 8;  // 16-byte chunks per W^T row
  const int64_t t0 = (int64_t)blockIdx.x * kRouterTokens + w * 64;  // this wave's 64 tokens
  const int64_t r0 = min<int64_t>(t0 + (lane & 31), a.tokens - 1);
  const int64_t r1 = min<int64_t>(t0 + 32 + (lane & 31), a.tokens - 1);
  // lanes 32..63 hold the second 8 k of each 16-k step (MFMA operand layout)
  const __bf16* x0 = a.x + r0 * d + (lane >> 5) * 8;
  const __bf16* x1 = a.x + r1 * d + (lane >> 5) * 8;
  bf16x8 buf[2][2][kRouterUnroll];  // [register buffer][token half][k-step]
  auto load_block = [&](bf16x8 (&b)[2][kRouterUnroll], int k0) {
#pragma unroll
    for (int u = 0; u < kRouterUnroll; ++u) {
      b[0][u] = *reinterpret_cast<const bf16x8*>(x0 + k0 + 16 * u);
      b[1][u] = *reinterpret_cast<const bf16x8*>(x1 + k0 + 16 * u);
    }
  };
  load_block(buf[0], 0);
  // packed W_r^T [64][d] (experts >= E are zero rows) -> LDS, 16-byte chunks
  // (16 loads per thread in flight before their LDS stores)
  constexpr int kFill = 16;
  for (int i0 = tid; i0 < kMaxExperts * chunks; i0 += kRouterThreads * kFill) {
    bf16x8 v[kFill];
#pragma unroll
    for (int u = 0; u < kFill; ++u) {
      const int i = i0 + u * kRouterThreads;
      if (i < kMaxExperts * chunks) {
        const int e = i / chunks, ch = i - e * chunks;
        v[u] = *reinterpret_cast<const bf16x8*>(a.wrt + (int64_t)e * d + ch * 8);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kFill; ++u) {
      const int i = i0 + u * kRouterThreads;
      if (i < kMaxExperts * chunks) {
        const int e = i / chunks, ch = i - e * chunks;
        *reinterpret_cast<bf16x8*>(lds + ((int64_t)e * chunks + (ch ^ (e & 7))) * 16) = v[u];
      }
    }
  }
  __syncthreads();

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
#pragma unroll
  for (int s = 0; s < kBlocks; ++s) {
    if (s + 1 < kBlocks) load_block(buf[(s + 1) & 1], (s + 1) * 16 * kRouterUnroll);
    __builtin_amdgcn_sched_barrier(0);  // the next block's loads stay above these MFMAs
#pragma unroll
    for (int u = 0; u < kRouterUnroll; ++u) {
      const int ch = ((s * 16 * kRouterUnroll + 16 * u) >> 3) + (lane >> 5);
      bf16x8 bv[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = j * 32 + (lane & 31);
        bv[j] = *reinterpret_cast<const bf16x8*>(lds + ((int64_t)e * chunks + (ch ^ (e & 7))) * 16);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(buf[s & 1][0][u], bv[j], acc[0][j], 0, 0, 0);
        acc[1][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(buf[s & 1][1][u], bv[j], acc[1][j], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // every wave is done with W^T: reuse LDS for logits
  float* lg = reinterpret_cast<float*>(lds);  // [kRouterTokens][65] (padded row)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = w * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int col = j * 32 + (lane & 31);
        lg[row * 65 + col] = acc[i][j][r];
      }
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kRouterTokens + tid;
  if (t < a.tokens) {
    const float* row = lg + tid * 65;
    int e0 = 0, e1 = -1;
    float l0 = row[0], l1 = 0.f;
    for (int e = 1; e < E; ++e) {
      const float v = row[e];
      if (v > l0) {  // strictly larger: ties keep the lower id
        e1 = e0; l1 = l0;
        e0 = e; l0 = v;
      } else if (e1 < 0 || v > l1) {
        e1 = e; l1 = v;
      }
    }
    const float z = expf(l1 - l0);  // <= 1
    const float g0 = 1.0f / (1.0f + z), g1 = z / (1.0f + z);
    a.experts[t * 2] = e0;
    a.experts[t * 2 + 1] = e1;
    a.gates[t * 2] = g0;
    a.gates[t * 2 + 1] = g1;
    if (a.logits)
      for (int e = 0; e < E; ++e) a.logits[t * E + e] = row[e];
  }
}

// Row-block prefix of the expert segments (data-dependent sizes), and the
// per-call reset of the FFN and combine counters. One workgroup.
__global__ void k_moe_prefix(MoeArgs a) {
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (uint32_t e = 0; e < a.E; ++e) {
      a.rb_start[e] = run;
      const int64_t n = a.seg[e + 1] - a.seg[e];
      run += (uint32_t)((n + mm::BM - 1) / mm::BM);
      a.b_done[e] = 0;
    }
    a.rb_start[a.E] = run;
    a.ctl[2] = 0;  // combine done counter
  }
}

// Largest e with rb_start[e] <= v.
__device__ __forceinline__ uint32_t expert_of(const uint32_t* rb_start, uint32_t E, uint32_t v) {
  uint32_t lo = 0, hi = E - 1;
  while (lo < hi) {
    const uint32_t mid = (lo + hi + 1) >> 1;
    if (rb_start[mid] <= v) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Workgroups -> tiles. The hardware deals consecutive workgroups to the 8
// XCDs in turn, so workgroup b runs on XCD b % 8 and each XCD holds about 32
// at a time (one per CU). An XCD's run of 32 workgroups covers an R x C patch
// of tiles (R row blocks x C column tiles, R C = 32) whose R activation panels
// and C weight panels are fetched from HBM once and shared through the XCD's
// L2; an XCD's successive patches walk the column groups of one row group
// before the next. (Placement only: the map is one-to-one whatever the
// dispatch order.)
constexpr uint32_t kXcds = 8, kPatch = 32;

__device__ __forceinline__ uint32_t patch_cols(uint32_t CT) {
  return CT % 8 == 0 ? 8 : CT % 4 == 0 ? 4 : CT % 2 == 0 ? 2 : 1;
}

__device__ __forceinline__ void tile_at(uint32_t b, uint32_t CT, uint32_t& rbg, uint32_t& c) {
  const uint32_t C = patch_cols(CT), R = kPatch / C, groups = CT / C;
  const uint32_t x = b % kXcds, s = b / kXcds, p = s % kPatch, k = s / kPatch;
  rbg = ((k / groups) * kXcds + x) * R + p / C;
  c = (k % groups) * C + p % C;
}

// Per-workgroup copies of the segment tables and the set of experts whose
// exchange future has fired (their input rows are complete).
struct FfnShared {
  uint32_t rb_start[kMaxExperts + 1];
  int64_t seg[kMaxExperts + 1];
  uint32_t ok[2];  // bit e: expert e may be read
};

// One 256 x 256 output tile of an expert FFN GEMM (wave-uniform).
struct FfnTile {
  uint32_t e, c;
  int64_t row0;  // first row of the tile in the expert-sorted activations
  int rows;      // valid rows (1..256)
};

__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint64_t u = (uint64_t)v;
  return (int64_t)((uint64_t)uniform((uint32_t)(u >> 32)) << 32 | uniform((uint32_t)u));
}

__device__ __forceinline__ FfnTile ffn_tile(const FfnShared& sh, uint32_t E, uint32_t rbg, uint32_t c) {
  FfnTile t;
  t.e = uniform(expert_of(sh.rb_start, E, rbg));
  const uint32_t rb = rbg - uniform(sh.rb_start[t.e]);
  const int64_t seg0 = uniform64(sh.seg[t.e]), n_e = uniform64(sh.seg[t.e + 1]) - seg0;
  t.row0 = seg0 + (int64_t)rb * mm::BM;
  t.rows = (int)uniform((uint32_t)min<int64_t>(mm::BM, n_e - (int64_t)rb * mm::BM));
  t.c = c;
  return t;
}

// The first tile index at or after b (stride: the grid) whose row block
// exists for this call's expert segments and whose expert's input is
// complete; ~0u if none.
__device__ __forceinline__ uint32_t next_tile(const FfnShared& sh, uint32_t E, uint32_t CT, uint32_t total_rb,
                                              uint32_t b, uint32_t nb, FfnTile& t) {
  for (; b < nb; b += gridDim.x) {
    uint32_t rbg, c;
    tile_at(b, CT, rbg, c);
    if (rbg >= total_rb) continue;
    t = ffn_tile(sh, E, rbg, c);
    if ((uniform(sh.ok[t.e >> 5]) >> (t.e & 31)) & 1u) return b;
  }
  return ~0u;
}

template <bool kSecond>
__device__ __forceinline__ mm::Tile ffn_operands(const MoeArgs& a, const FfnTile& t) {
  const uint32_t K = kSecond ? a.hidden : a.d, N = kSecond ? a.d : a.hidden;
  mm::Tile tile;
  tile.A = (kSecond ? a.h : a.xd) + t.row0 * K;
  tile.lda = K;
  tile.rows = t.rows;
  tile.Bt = (kSecond ? a.w2t : a.w1t) + (int64_t)t.e * K * N + (int64_t)t.c * mm::BN * K;
  tile.ldb = K;
  tile.K = (int)K;
  return tile;
}

// FFN2: a finished tile counts towards its expert; the expert's last tile
// fires B[e]. Called once every wave's stores of the tile have completed (after
// the next tile's K loop); the consumer (the combine) is a later launch on the
// same stream, so the kernel boundary makes the rows visible to it.
struct CountTile {
  const MoeArgs* a;
  uint32_t e, tiles_e;
  bool pending;
  __device__ void operator()() {
    if (pending && threadIdx.x == 0) {
      const uint32_t old = __hip_atomic_fetch_add(&a->b_done[e], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old + 1 == tiles_e) fire(a->f, NODE_B, e, a->epoch);
    }
    pending = false;
  }
};

// Expert FFN GEMM, persistent: one workgroup per CU walks the tiles
// b = blockIdx.x + k * gridDim.x (grid a multiple of 8, so all of a
// workgroup's tiles map to the XCD it runs on; see tile_at). kSecond: input
// H, weights W2 [E][hidden][d], output Y (no activation); otherwise input the
// dispatched rows, W1 [E][d][hidden], output H through GELU.
//
// B is gated on the exchange: before touching any rows, lane e of wave 0
// waits for expert e's exchange future (all experts at once); tiles of an
// expert whose wait expired are skipped (its B future then never fires and
// the combine reports the timeout). Each tile's epilogue overlaps the next
// tile's first loads, issued through size-predicated buffer loads (a branch
// there would make the compiler move the accumulators out early).
template <bool kSecond>
__global__ __launch_bounds__(256, 1) void k_ffn(MoeArgs a, uint32_t nb) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __shared__ FfnShared sh;
  const uint32_t tid = threadIdx.x, E = a.E;
  const uint32_t CT = (kSecond ? a.d : a.hidden) / mm::BN;
  const uint32_t N = kSecond ? a.d : a.hidden;
  if (tid <= E) {
    sh.rb_start[tid] = a.rb_start[tid];
    sh.seg[tid] = a.seg[tid];
  }
  if (tid < 2) sh.ok[tid] = 0;
  __syncthreads();
  if (tid < E) {
    const bool go = await_prior(a.f, NODE_EXCH, tid, a.epoch);  // the expert's input is complete
    if (go) atomicOr(&sh.ok[tid >> 5], 1u << (tid & 31));
  }
  __syncthreads();
  const uint32_t total_rb = uniform(sh.rb_start[E]);
  FfnTile cur;
  uint32_t b = next_tile(sh, E, CT, total_rb, blockIdx.x, nb, cur);
  if (b == ~0u) return;  // uniform
  mm::tile_start(ffn_operands<kSecond>(a, cur), lds);
  CountTile count{&a, 0, 0, false};
  while (true) {
    // the next tile is looked up before the K loop: control flow between the
    // K loop and the epilogue would also make the accumulators move early
    FfnTile nxt = cur;
    const uint32_t b2 = next_tile(sh, E, CT, total_rb, b + gridDim.x, nb, nxt);
    mm::f32x16 acc[4][4];
    mm::NoHook none;
    mm::tile_finish(ffn_operands<kSecond>(a, cur), lds, acc, none);
    mm::tile_start_if(ffn_operands<kSecond>(a, nxt), lds, b2 != ~0u);
    mm::store_tile<!kSecond>(acc, (kSecond ? a.y : a.h) + cur.row0 * N + (int64_t)cur.c * mm::BN, N, cur.rows);
    if (kSecond) {
      // every wave waited for all its memory operations inside the K loop
      // above, then met at its final barrier: the previous tile's stores are
      // complete (counted only here, after the epilogue, because a branch
      // between the K loop and the epilogue makes the accumulators move early)
      count();
      count.e = cur.e;
      count.tiles_e = uniform((uint32_t)((sh.seg[cur.e + 1] - sh.seg[cur.e] + mm::BM - 1) / mm::BM)) * CT;
      count.pending = true;
    }
    if (b2 == ~0u) break;
    b = b2;
    cur = nxt;
  }
  mm::wait_stores();  // also the out-of-range loads of the start above
  __syncthreads();
  if (kSecond) count();
}

// out[t] = bf16(g0 * Y[slot(2t)] + g1 * Y[slot(2t + 1)]), fp32 sum with the
// top-1 term first; a tuple dropped by the expert capacity (slot -1) adds
// nothing. Gating: each workgroup first checks the B futures of all experts
// (thread e: expert e) and combines only the tokens whose two experts fired.
// Then one wave handles kCombineTokens tokens per pass: their metadata
// (experts, gates, slots) in one round of loads, then every row chunk of both
// tokens in flight before any is used (16-byte chunks, lane l: chunks l and
// l + 64 of each row). The row loads are unconditional (a dropped tuple reads
// row 0 and masks it to zero), since a load under a branch would make the
// compiler wait for each load in turn. Rows are read and written
// nontemporally: the gather reads each Y row once (measured on this shape:
// 142 against 153 us with cached loads), nothing in the step reads the output
// again, and output rows left dirty in the caches would be written back while
// the next step's router streams the tokens (a read-bound kernel after 256 MiB
// of plain stores runs 30-35 us longer). The grid is bounded (grid-stride over
// tokens): every workgroup adds once to the done counter, and adds to one
// address serialize at the memory side.
constexpr uint32_t kCombineBlocks = 2048;
constexpr int kCombineTokens = 2;

__global__ __launch_bounds__(256) void k_combine(MoeArgs a) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  __shared__ uint32_t s_ok[2];
  const uint32_t tid = threadIdx.x;
  const int lane = tid & 63;
  if (tid < 2) s_ok[tid] = 0;
  __syncthreads();
  if (tid < a.E && await_prior(a.f, NODE_B, tid, a.epoch)) atomicOr(&s_ok[tid >> 5], 1u << (tid & 31));
  __syncthreads();
  const uint64_t ok = (uint64_t)s_ok[0] | (uint64_t)s_ok[1] << 32;
  const uint32_t nch = a.d / 8;  // 16-byte chunks per row
  const u32x4* y = reinterpret_cast<const u32x4*>(a.y);
  u32x4* out = reinterpret_cast<u32x4*>(a.out);
  const int64_t stride = (int64_t)gridDim.x * 4 * kCombineTokens;
  for (int64_t t0 = ((int64_t)blockIdx.x * 4 + (tid >> 6)) * kCombineTokens; t0 < (int64_t)a.tokens; t0 += stride) {
    int slot[kCombineTokens][2];
    float gate[kCombineTokens][2];
    bool live[kCombineTokens];
#pragma unroll
    for (int k = 0; k < kCombineTokens; ++k) {
      const int64_t t = min<int64_t>(t0 + k, (int64_t)a.tokens - 1);
      const int2 e = *reinterpret_cast<const int2*>(a.experts + t * 2);
      const float2 g = *reinterpret_cast<const float2*>(a.gates + t * 2);
      const int2 sl = *reinterpret_cast<const int2*>(a.slot_of + t * 2);
      const int e0 = __builtin_amdgcn_readfirstlane(e.x), e1 = __builtin_amdgcn_readfirstlane(e.y);
      live[k] = t0 + k < (int64_t)a.tokens && ((ok >> (e0 & 63)) & (ok >> (e1 & 63)) & 1u);
      slot[k][0] = __builtin_amdgcn_readfirstlane(sl.x);
      slot[k][1] = __builtin_amdgcn_readfirstlane(sl.y);
      gate[k][0] = g.x;
      gate[k][1] = g.y;
    }
    for (uint32_t c0 = 0; c0 < nch; c0 += 128) {
      u32x4 v[kCombineTokens][2][2];  // [token][tuple][chunk]
#pragma unroll
      for (int k = 0; k < kCombineTokens; ++k)
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const uint32_t ch = min(c0 + lane + 64 * c, nch - 1);
            v[k][r][c] = __builtin_nontemporal_load(y + (int64_t)max(slot[k][r], 0) * nch + ch);
          }
#pragma unroll
      for (int k = 0; k < kCombineTokens; ++k) {
        const uint32_t m0 = slot[k][0] >= 0 ? ~0u : 0u, m1 = slot[k][1] >= 0 ? ~0u : 0u;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const uint32_t ch = c0 + lane + 64 * c;
          const bf16x8 u = __builtin_bit_cast(bf16x8, v[k][0][c] & m0);
          const bf16x8 w = __builtin_bit_cast(bf16x8, v[k][1][c] & m1);
          bf16x8 r;
#pragma unroll
          for (int j = 0; j < 8; ++j) r[j] = (__bf16)fmaf(gate[k][1], (float)w[j], gate[k][0] * (float)u[j]);
          if (live[k] && ch < nch) __builtin_nontemporal_store(__builtin_bit_cast(u32x4, r), out + (t0 + k) * nch + ch);
        }
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&a.ctl[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 == gridDim.x) fire(a.f, NODE_RESULT, 0, a.epoch);
  }
}

}  // namespace

size_t router_lds_bytes(uint32_t d) { return (size_t)kMaxExperts * d * 2 > (size_t)kRouterTokens * 65 * 4 ? (size_t)kMaxExperts * d * 2 : (size_t)kRouterTokens * 65 * 4; }

template <int kBlocks>
static hipError_t launch_router_blocks(const MoeArgs& a, hipStream_t s) {
  const size_t lds = router_lds_bytes(a.d);
  hipError_t e = hipFuncSetAttribute((const void*)k_router<kBlocks>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const uint64_t blocks = (a.tokens + kRouterTokens - 1) / kRouterTokens;
  hipLaunchKernelGGL(k_router<kBlocks>, dim3((uint32_t)blocks), dim3(kRouterThreads), lds, s, a);
  return hipGetLastError();
}

// d is a multiple of 256 and at most 1280 (checked at plan time)
hipError_t launch_router(const MoeArgs& a, hipStream_t s) {
  switch (a.d) {
    case 256: return launch_router_blocks<2>(a, s);
    case 512: return launch_router_blocks<4>(a, s);
    case 768: return launch_router_blocks<6>(a, s);
    case 1024: return launch_router_blocks<8>(a, s);
    case 1280: return launch_router_blocks<10>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_moe_prefix(const MoeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_moe_prefix, dim3(1), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ffn(const MoeArgs& a, bool second, uint32_t cus, hipStream_t s) {
  // tile indices: enough whole patch rounds to cover max_row_blocks row
  // blocks (see tile_at); persistent grid: one workgroup per CU, a multiple of 8
  const uint32_t CT = (second ? a.d : a.hidden) / mm::BN;
  const uint32_t C = CT % 8 == 0 ? 8 : CT % 4 == 0 ? 4 : CT % 2 == 0 ? 2 : 1, R = kPatch / C;
  const uint64_t row_groups = ((uint64_t)a.max_row_blocks + R - 1) / R;
  const uint64_t nb = (row_groups + kXcds - 1) / kXcds * kXcds * R * CT;
  const uint32_t grid = (uint32_t)std::min<uint64_t>(nb, std::max<uint32_t>(kXcds, cus / kXcds * kXcds));
  const void* fn = second ? (const void*)k_ffn<true> : (const void*)k_ffn<false>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, mm::kLdsTotal);
  if (e != hipSuccess) return e;
  if (second)
    hipLaunchKernelGGL(k_ffn<true>, dim3(grid), dim3(mm::NT), mm::kLdsTotal, s, a, (uint32_t)nb);
  else
    hipLaunchKernelGGL(k_ffn<false>, dim3(grid), dim3(mm::NT), mm::kLdsTotal, s, a, (uint32_t)nb);
  return hipGetLastError();
}

hipError_t launch_combine(const MoeArgs& a, hipStream_t s) {
  const uint64_t blocks = std::min<uint64_t>((a.tokens + 4 * kCombineTokens - 1) / (4 * kCombineTokens), kCombineBlocks);
  hipLaunchKernelGGL(k_combine, dim3((uint32_t)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pw
