// The whole exchange step in one launch, for small steps: Arg -> A ->
// histogram, scan, stable scatter -> progress futures -> B, gated on those
// futures inside the launch -> Result. Taken when the plan asks for it
// (PW_FLAG_ONE_LAUNCH).
//
// PATHWAYS page ("PATHWAYS: Asynchronous Distributed Dataflow for ML"),
// section 4.3: progress tracking decides when a shard has received all of its
// messages; sections 4.4-4.5: B consumes the exchange's buffer futures and a
// successor starts as soon as its input future is ready, not when the whole
// previous program ends. Here one co-resident grid does the whole step:
//
//   1. workgroup b ranks the tuples of its slab of S consecutive tuples per
//      destination, 64 at a time by wave ballots (stable: chunk order, then
//      lane order), and loads the slab's payload (<= 32 KiB) into registers;
//   2. wave 0 publishes the slab's per-destination counts as a row of the
//      slab table, each entry tagged with the call;
//   3. every workgroup reads the whole table (at most 8192 entries), waiting
//      (bounded) until every entry carries this call's tag: the one
//      device-wide step the counting sort needs, since a destination's
//      segment start depends on every earlier destination's total. From it,
//      the totals, the segment offsets and its own run start inside each
//      segment; then it stores its rows straight from registers (A applied);
//   4. once its row stores have completed, an add per destination it wrote
//      to; the add that completes a destination fires EXCHANGE[d];
//   5. B: workgroup b takes output rows [b S, (b + 1) S); it waits for the
//      EXCHANGE futures of the destinations those rows belong to, so B of a
//      segment starts as soon as that segment is complete, while other
//      workgroups still scatter. The add that completes a segment's B fires
//      B[d]; the last B fires the Result.
//
// Everything handed between workgroups here (table entries, rows) is
// written and read with agent-coherent accesses (device.h), never through an
// agent-scope release or acquire fence: on this part such a fence writes
// back or invalidates a whole XCD's L2 and costs microseconds per workgroup
// (the fenced form of this kernel ran 28 us per 8-shard step, this one
// about 19). Each hop still costs about a microsecond or two of memory
// latency.
//
// The grid must be co-resident (step 3 waits for every workgroup); the plan
// takes this path only for grids of at most 256 workgroups of 256 threads,
// after checking the occupancy. Every wait is bounded by the plan's spin
// limit; an expired wait latches a timeout and the workgroup leaves. The
// table's tags make it safe to reuse across calls without clearing. The
// arrival counters come in two sets used by alternate calls; a call clears
// the other set (which the previous call used) for the next one, so no
// clearing races with this call's adds.
#include <algorithm>

#include "device.h"

namespace pw {

namespace {

constexpr uint32_t kBlock = 256;
constexpr uint32_t kUnits = 8;       // 16-byte payload units held per thread: 32 KiB per workgroup
constexpr uint32_t kMaxN = 64;       // destinations
constexpr uint32_t kMaxSlab = 1024;  // tuples per workgroup
constexpr uint32_t kMaxChunks = kMaxSlab / 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct SmallShared {
  uint32_t cnt[kMaxChunks][kMaxN];  // per 64-tuple chunk: counts, then the chunk's start inside the slab's run
  uint32_t mine[kMaxN];             // the slab's tuples per destination
  uint32_t tot[kMaxN], pre[kMaxN];  // all slabs' tuples per destination; the earlier slabs' tuples
  uint32_t seg[kMaxN + 1];          // segment offsets
  uint32_t tup[kMaxSlab];           // rank inside its chunk's group | destination << 16; ~0: dropped
  int slot[kMaxSlab];
  uint32_t red_t[kBlock], red_p[kBlock];
};

__device__ __forceinline__ u32x4 affine4(u32x4 v, float ca, float cb) {
  f32x4 f = __builtin_bit_cast(f32x4, v);
  f.x = fmaf(ca, f.x, cb);
  f.y = fmaf(ca, f.y, cb);
  f.z = fmaf(ca, f.z, cb);
  f.w = fmaf(ca, f.w, cb);
  return __builtin_bit_cast(u32x4, f);
}

// Bytes of the destination rows, as a buffer size (< 2^31: the one-launch
// path holds at most 256 Ki tuples of at most 512 bytes, so every slot it
// writes lies below it). Offsets at or past it read zero.
__device__ __forceinline__ uint32_t dst_bytes(const ExchangeArgs& a) {
  return (uint32_t)min<uint64_t>((uint64_t)a.dst_rows * a.row_bytes, 0x7fffffffu);
}

// Row sums of output rows [r0, r1) (fp32, P elements, P % 4 == 0): 16 lanes
// per row, 16 rows per pass, each lane summing float4 chunks l16, l16 + 16,
// ... as (x + y) + (z + w), then a butterfly over the 16 lanes. The loads of
// kPasses passes (128 rows: a whole slab of 256-byte rows) are in flight
// together; they are coherent loads (the rows were written by other
// workgroups of this launch), and those of rows past r1 or chunks past the
// row end go out of range and read zero. The same arithmetic, in the same
// order, as the separate B kernel, so both paths give the same bits.
__device__ __forceinline__ void rowsum_rows(const ExchangeArgs& a, __amdgpu_buffer_rsrc_t rows, int64_t r0,
                                            int64_t r1) {
  constexpr uint32_t kPasses = 8;
  const uint32_t P4 = a.row_bytes / 16u;  // float4 chunks per row (<= 32)
  const uint32_t oob = dst_bytes(a);
  float* out = reinterpret_cast<float*>(a.b_out);
  const uint32_t l16 = threadIdx.x & 15, r = threadIdx.x >> 4;
  for (int64_t base = r0; base < r1; base += 16 * kPasses) {
    f32x4 v0[kPasses], v1[kPasses];
#pragma unroll
    for (uint32_t p = 0; p < kPasses; ++p) {
      const int64_t s = base + p * 16 + r;
      const uint32_t c = (uint32_t)s * P4 + l16;
      const uint32_t o0 = s < r1 && l16 < P4 ? c * 16u : oob;
      const uint32_t o1 = s < r1 && l16 + 16 < P4 ? (c + 16) * 16u : oob;
      v0[p] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rows, o0, 0, kCoherent));
      v1[p] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rows, o1, 0, kCoherent));
    }
#pragma unroll
    for (uint32_t p = 0; p < kPasses; ++p) {
      const int64_t s = base + p * 16 + r;
      float x = 0.f;
      if (l16 < P4) x += (v0[p].x + v0[p].y) + (v0[p].z + v0[p].w);
      if (l16 + 16 < P4) x += (v1[p].x + v1[p].y) + (v1[p].z + v1[p].w);
      x += __shfl_xor(x, 8, 16);
      x += __shfl_xor(x, 4, 16);
      x += __shfl_xor(x, 2, 16);
      x += __shfl_xor(x, 1, 16);
      if (s < r1 && l16 == 0) out[s] = x;
    }
  }
}

// This thread's payload units of the slab: i = u * kBlock + tid for u <
// kUnits (16-byte units; unit i is unit i % vu of tuple i / vu). Every load
// is issued unconditionally, units past the slab's end re-reading its last
// unit (values never used): a load under a branch makes the compiler merge
// its value with the other path right after the branch, i.e. wait for it,
// which serialised the 8 loads.
__device__ __forceinline__ void load_payload(const ExchangeArgs& a, uint64_t g0, uint32_t units, uint32_t vu,
                                             u32x4 (&v)[kUnits]) {
#pragma unroll
  for (uint32_t u = 0; u < kUnits; ++u) {
    const uint32_t i = min(u * kBlock + threadIdx.x, units - 1);
    const uint32_t t = i / vu;
    v[u] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(a.src + (g0 + t) * a.row_bytes + (uint64_t)(i - t * vu) * 16u));
  }
}

template <bool kAffine>
__global__ __launch_bounds__(kBlock) void k_exchange_small(ExchangeArgs a) {
  __shared__ SmallShared sh;
  const uint32_t N = a.N, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint32_t b = blockIdx.x, S = a.slab, grid = gridDim.x;
  const uint64_t g0 = (uint64_t)b * S;
  const uint32_t nt = (uint32_t)min<uint64_t>(S, a.G - g0);  // tuples of this slab (>= 1)
  const uint32_t vu = a.row_bytes / 16u;
  const uint32_t units = nt * vu;
  const uint32_t chunks = (nt + 63) / 64;
  // this call's counters (arrivals, B arrivals, finished destinations) and
  // the next call's, cleared here: calls alternate between the two sets
  const uint32_t stride = 2 * N + 1;
  uint32_t* arrived = a.small_tab + (a.call & 1) * stride;
  uint32_t* b_arrived = arrived + N;
  uint32_t* done = arrived + 2 * N;
  if (b == 0) {
    uint32_t* next = a.small_tab + ((a.call & 1) ^ 1) * stride;
    for (uint32_t i = tid; i < stride; i += kBlock) next[i] = 0;
  }

  // 1. the destinations first (wave w ranks chunks w, w + 4, ...), then the
  //    payload
  constexpr uint32_t kPerWave = kMaxChunks / 4;
  int dv[kPerWave];
  uint32_t in_range = 0;
#pragma unroll
  for (uint32_t j = 0; j < kPerWave; ++j) {  // unconditional loads (see load_payload)
    const uint32_t t = (w + 4 * j) * 64 + lane;
    in_range |= (uint32_t)(t < nt) << j;
    dv[j] = a.dest[g0 + min(t, nt - 1)];
  }
  u32x4 v[kUnits];
  load_payload(a, g0, units, vu, v);
  for (uint32_t i = tid; i < chunks * kMaxN; i += kBlock) sh.cnt[i / kMaxN][i % kMaxN] = 0;
  __syncthreads();
  bool bad = false;
#pragma unroll
  for (uint32_t j = 0; j < kPerWave; ++j) {
    const uint32_t c = w + 4 * j;
    if (c >= chunks) break;  // uniform
    const bool ir = (in_range >> j) & 1u;
    const bool okd = ir && dv[j] >= 0 && (uint32_t)dv[j] < N;
    bad |= ir && !okd;
    const int d = okd ? dv[j] : -1;
    const uint64_t peers = match_peers(d, d >= 0, a.nbits);
    uint32_t code = ~0u;
    if (d >= 0) {
      const uint32_t r = (uint32_t)__popcll(peers & lanemask_lt(lane)), n = (uint32_t)__popcll(peers);
      if (r == 0) atomicAdd(&sh.cnt[c][d], n);
      code = r | (uint32_t)d << 16;
    }
    if (ir) sh.tup[c * 64 + lane] = code;
  }
  __syncthreads();
  // 2. wave 0: the slab's counts and its row of the slab table, each entry
  //    tagged with the call (one coherent 64-bit store: count | call << 32)
  if (tid < N) {
    uint32_t run = 0;
    for (uint32_t c = 0; c < chunks; ++c) {
      const uint32_t x = sh.cnt[c][tid];
      sh.cnt[c][tid] = run;
      run += x;
    }
    sh.mine[tid] = run;
    __hip_atomic_store(&a.slab_cnt[(uint64_t)b * N + tid], (uint64_t)a.call << 32 | run, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }

  // 3. totals, segment offsets and this slab's run starts, from the table
  //    (thread t reads column t % N of rows t / N, t / N + R, ...; 8 rows per
  //    round of coherent loads). The one device-wide step of the counting
  //    sort, since a destination's segment start depends on every earlier
  //    destination's total: an entry counts once it carries this call's tag;
  //    the loads of a round are repeated until all do (bounded).
  const uint32_t R = kBlock / N;
  bool ok = true;
  if (tid < R * N) {
    const uint32_t d = tid % N;
    uint32_t tt = 0, pp = 0;
    const uint64_t t0 = wall_clock64();
    for (uint32_t r0 = tid / N; r0 < grid && ok; r0 += 8 * R) {
      const uint64_t* e[8];
      uint64_t x[8];
#pragma unroll
      for (uint32_t u = 0; u < 8; ++u) {  // unconditional loads (see load_payload)
        e[u] = &a.slab_cnt[(uint64_t)min(r0 + u * R, grid - 1) * N + d];
        x[u] = __hip_atomic_load(e[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      while (true) {
        bool all = true;
#pragma unroll
        for (uint32_t u = 0; u < 8; ++u) all &= (uint32_t)(x[u] >> 32) == a.call;
        if (all) break;
        if (wall_clock64() - t0 > a.f.spin_ticks) {
          latch(a.f, ST_TIMEOUT);
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (uint32_t u = 0; u < 8; ++u)
          if ((uint32_t)(x[u] >> 32) != a.call) x[u] = __hip_atomic_load(e[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (uint32_t u = 0; u < 8; ++u) {
        const uint32_t r = r0 + u * R, n = (uint32_t)x[u];
        tt += r < grid ? n : 0u;
        pp += r < b ? n : 0u;
      }
    }
    sh.red_t[tid] = tt;
    sh.red_p[tid] = pp;
  }
  if (!__syncthreads_and(ok)) return;  // a slab never published: the call's waits time out
  if (tid < N) {
    uint32_t tt = 0, pp = 0;
    for (uint32_t r = 0; r < R; ++r) {
      tt += sh.red_t[r * N + tid];
      pp += sh.red_p[r * N + tid];
    }
    sh.tot[tid] = tt;
    sh.pre[tid] = pp;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t run = 0;
    for (uint32_t d = 0; d < N; ++d) {
      sh.seg[d] = run;
      run += sh.tot[d];
    }
    sh.seg[N] = run;
  }
  __syncthreads();
  if (b == 0) {
    if (tid <= N) {
      a.seg[tid] = sh.seg[tid];
      if (a.offsets_out) a.offsets_out[tid] = sh.seg[tid];
    }
    if (tid < N) a.expected[tid] = sh.tot[tid];
    if (tid < N && sh.tot[tid] == 0) {  // nothing will arrive: its input (and B, which has no rows) is complete
      fire(a.f, NODE_EXCH, tid, a.epoch);
      fire(a.f, NODE_B, tid, a.epoch);
      const uint32_t r = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (r + 1 == N) fire(a.f, NODE_RESULT, 0, a.epoch);
    }
  }
  for (uint32_t t = tid; t < nt; t += kBlock) {
    const uint32_t code = sh.tup[t];
    int slot = -1;
    if (code != ~0u) {
      const uint32_t d = code >> 16;
      const uint64_t sl = (uint64_t)sh.seg[d] + sh.pre[d] + sh.cnt[t / 64][d] + (code & 0xffffu);
      if (sl < a.dst_rows) {
        slot = (int)sl;
        if (a.src_index) a.src_index[sl] = (int32_t)(g0 + t);
      } else {
        bad = true;
      }
    }
    sh.slot[t] = slot;
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t out_rows = raw_buffer(a.dst, dst_bytes(a));
#pragma unroll
  for (uint32_t u = 0; u < kUnits; ++u) {
    const uint32_t i = u * kBlock + tid;
    if (i < units) {
      const uint32_t t = i / vu;
      const int slot = sh.slot[t];
      if (slot >= 0) {
        const u32x4 x = kAffine ? affine4(v[u], a.a_a, a.a_b) : v[u];
        __builtin_amdgcn_raw_buffer_store_b128(x, out_rows, (uint32_t)slot * a.row_bytes + (i - t * vu) * 16u, 0,
                                               kCoherent);
      }
    }
  }
  if (bad) latch(a.f, ST_BAD_DEST);

  // 4. progress: every wave's coherent row stores have completed, then an
  //    add per destination written; the add that completes one fires its
  //    future (every slab's rows of d were complete before its add)
  wait_vmem_all();
  __syncthreads();
  if (tid < N && sh.mine[tid]) {
    const uint32_t n = sh.mine[tid];
    const uint32_t old = __hip_atomic_fetch_add(&arrived[tid], n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + n == sh.tot[tid]) {
      fire(a.f, NODE_EXCH, tid, a.epoch);
      if (!a.b_gated) {  // B has no work of its own: it completes with its input
        fire(a.f, NODE_B, tid, a.epoch);
        const uint32_t r = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (r + 1 == N) fire(a.f, NODE_RESULT, 0, a.epoch);
      }
    }
  }
  if (!a.b_gated) return;

  // 5. B over output rows [b S, (b + 1) S), gated on the futures of the
  //    segments they belong to
  const int64_t r0 = (int64_t)b * S, r1 = min<int64_t>((int64_t)(b + 1) * S, sh.seg[N]);
  if (r0 >= r1) return;  // uniform
  bool in = false;
  bool ready = true;
  if (tid < N) {
    in = sh.tot[tid] && sh.seg[tid] < r1 && sh.seg[tid + 1] > r0;
    if (in) ready = await_coherent(a.f, NODE_EXCH, tid, a.epoch);
  }
  if (!__syncthreads_and(ready)) return;
  const __amdgpu_buffer_rsrc_t in_rows = raw_buffer(a.dst, dst_bytes(a));
  if (a.b_kind == OP_ROWSUM) {
    rowsum_rows(a, in_rows, r0, r1);
  } else if (a.b_kind == OP_AFFINE) {
    const uint32_t P = a.row_bytes / 4u;
    float* out = reinterpret_cast<float*>(a.b_out);
    for (uint32_t i = (uint32_t)r0 * P + tid; i < (uint32_t)r1 * P; i += kBlock)
      out[i] = fmaf(a.b_a, __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(in_rows, i * 4u, 0, kCoherent)),
                    a.b_b);
  }
  __syncthreads();
  if (in) {
    const int64_t lo = max<int64_t>(r0, sh.seg[tid]), hi = min<int64_t>(r1, sh.seg[tid + 1]);
    const uint32_t n = (uint32_t)(hi - lo);
    const uint32_t old = __hip_atomic_fetch_add(&b_arrived[tid], n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + n == sh.tot[tid]) {
      fire(a.f, NODE_B, tid, a.epoch);
      const uint32_t r = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (r + 1 == N) fire(a.f, NODE_RESULT, 0, a.epoch);
    }
  }
}

}  // namespace

// The slab size of the one-launch path for N destinations and rows of
// row_bytes, or 0 if the step does not fit it: 16-byte payload units, at most
// kUnits per thread and kMaxSlab tuples per workgroup, whole 64-tuple chunks,
// at most 256 workgroups (one per CU: co-resident), at most 256 Ki tuples
// (every workgroup reads all destinations), at most 64 destinations.
uint32_t exchange_small_slab(uint64_t G, uint32_t N, uint32_t row_bytes, uint32_t b_kind, bool f32) {
  if (G == 0 || N > kMaxN || row_bytes % 16 || row_bytes > 512) return 0;
  if (b_kind == OP_ROWSUM && (!f32 || row_bytes % 16)) return 0;
  const uint32_t slab = std::min<uint32_t>(kMaxSlab, kUnits * kBlock * 16 / row_bytes) / 64 * 64;
  if (slab < 64) return 0;
  const uint64_t grid = (G + slab - 1) / slab;
  if (grid > 256 || grid * N > 8192) return 0;  // every workgroup reads the whole slab table
  return slab;
}

uint32_t exchange_small_resident(int device) {
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)k_exchange_small<true>, kBlock, 0) !=
      hipSuccess)
    return 0;
  int per_cu2 = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu2, (const void*)k_exchange_small<false>, kBlock, 0) !=
      hipSuccess)
    return 0;
  return (uint32_t)std::max(0, cus * std::min(per_cu, per_cu2));
}

hipError_t launch_exchange_small(const ExchangeArgs& a, hipStream_t s) {
  const uint32_t grid = (uint32_t)((a.G + a.slab - 1) / a.slab);
  if (a.a_kind == OP_AFFINE)
    hipLaunchKernelGGL(k_exchange_small<true>, dim3(grid), dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL(k_exchange_small<false>, dim3(grid), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace pw
