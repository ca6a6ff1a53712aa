// Sparse shard-to-shard exchange on one MI355X.
//
// PATHWAYS page ("PATHWAYS: Asynchronous Distributed Dataflow for ML"),
// section 4.3 "Coordination implementation": every node emits tuples tagged
// with a destination shard, the runtime moves them among dynamically chosen
// shards along the sharded edge, and progress tracking decides when a shard
// has all of its messages; sections 4.4-4.5: the successor consumes buffer
// futures and the interconnect writes straight into the successor's input
// buffers. On one GPU the "interconnect" is HBM, and the exchange is a stable
// counting sort by destination done in three launches:
//
//   hist    one workgroup per tile of `tile` consecutive tuples counts its
//           destinations (LDS atomics) and writes the row tile_base[tile][*];
//   scan    one workgroup per block of scan_tiles tiles runs, per
//           destination, down its rows (where each tile's run of d starts
//           inside the block) and writes the block totals; the last
//           workgroup to finish scans those over the blocks and the
//           destination totals into segment offsets, sets the expected count
//           of every destination and fires the futures of destinations that
//           receive nothing;
//   scatter one workgroup per tile re-ranks its tuples (stable: wave by wave,
//           in source order), applies A and writes each payload row with
//           16-byte vector stores straight into its destination segment,
//           then adds its per-destination counts to the arrival counters;
//           the workgroup whose add completes a destination fires that
//           destination's future.
//
// B (exchange.hip: k_b) runs per block of output slots and starts only after
// the futures of every destination those slots belong to have fired.

#include "device.h"

namespace pw {

namespace {

constexpr uint32_t kBlock = 256;
constexpr uint32_t kWaves = kBlock / 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Destination of tuple g, or -1 (past the end, or out of range: latched).
__device__ __forceinline__ int load_dest(const ExchangeArgs& a, uint64_t g, bool& bad) {
  if (g >= a.G) return -1;
  const int d = a.dest[g];
  if (d < 0 || (uint32_t)d >= a.N) {
    bad = true;
    return -1;
  }
  return d;
}

// Exclusive scan of one u32 per thread over a 256-thread block.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const uint32_t lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (uint32_t o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (uint32_t i = 0; i < kWaves; ++i) {
    if (i < w) pre += wsum[i];
    tot += wsum[i];
  }
  __syncthreads();
  total = tot;
  return pre + x - v;
}

// ---------------------------------------------------------------- histogram
// A wave's destinations, loaded before any is used (up to kMaxChunks chunks
// of 64 tuples: tile <= 4096 split over 4 waves), so that the loads of its
// whole sub-tile are in flight together.
constexpr uint32_t kMaxChunks = 16;

struct WaveDests {
  int d[kMaxChunks];
};

__device__ __forceinline__ WaveDests load_wave_dests(const ExchangeArgs& a, uint64_t g0, uint32_t sub, uint32_t lane,
                                                     bool& bad) {
  WaveDests w;
#pragma unroll
  for (uint32_t i = 0; i < kMaxChunks; ++i) w.d[i] = i * 64 < sub ? load_dest(a, g0 + i * 64 + lane, bad) : -1;
  return w;
}

__global__ __launch_bounds__(kBlock) void k_hist(ExchangeArgs a) {
  extern __shared__ uint32_t lds[];
  uint32_t* cnt = lds;  // [N]
  for (uint32_t d = threadIdx.x; d < a.N; d += kBlock) cnt[d] = 0;
  __syncthreads();
  const uint32_t w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t sub = a.tile / kWaves;
  const uint64_t g0 = (uint64_t)blockIdx.x * a.tile + (uint64_t)w * sub;
  bool bad = false;
  const WaveDests wd = load_wave_dests(a, g0, sub, lane, bad);
  // counts need no order: one LDS atomic per tuple (the LDS serializes
  // lanes that hit one counter, which is cheaper than matching them)
#pragma unroll
  for (uint32_t i = 0; i < kMaxChunks; ++i)
    if (wd.d[i] >= 0) atomicAdd(&cnt[wd.d[i]], 1u);
  if (bad) latch(a.f.status, ST_BAD_DEST);
  __syncthreads();
  for (uint32_t d = threadIdx.x; d < a.N; d += kBlock) a.tile_base[(uint64_t)blockIdx.x * a.N + d] = cnt[d];
}

// ------------------------------------------------- per-source counts export
__global__ __launch_bounds__(kBlock) void k_src_counts(ExchangeArgs a) {
  extern __shared__ uint32_t lds[];
  uint32_t* cnt = lds;  // [N]
  for (uint32_t d = threadIdx.x; d < a.N; d += kBlock) cnt[d] = 0;
  __syncthreads();
  const uint64_t beg = (uint64_t)blockIdx.x * a.T, end = beg + a.T;
  bool bad = false;
  for (uint64_t g = beg + threadIdx.x; g < end; g += kBlock) {
    const int d = load_dest(a, g, bad);
    if (d >= 0) atomicAdd(&cnt[d], 1u);  // counts need no order
  }
  __syncthreads();
  for (uint32_t d = threadIdx.x; d < a.N; d += kBlock) a.counts[(uint64_t)blockIdx.x * a.N + d] = cnt[d];
}

// --------------------------------------------------------------------- scan
// Exclusive running sum, in place, of the column d of rows [r0, r1) of a
// row-major [rows][N] table; returns the column total. The loads of 16 rows
// are issued before any is needed.
__device__ __forceinline__ uint32_t column_scan(uint32_t* t, uint32_t N, uint32_t d, uint32_t r0, uint32_t r1) {
  constexpr uint32_t kB = 16;
  uint32_t run = 0;
  for (uint32_t r = r0; r < r1; r += kB) {
    uint32_t v[kB];
#pragma unroll
    for (uint32_t u = 0; u < kB; ++u) v[u] = r + u < r1 ? t[(uint64_t)(r + u) * N + d] : 0u;
#pragma unroll
    for (uint32_t u = 0; u < kB; ++u) {
      if (r + u < r1) t[(uint64_t)(r + u) * N + d] = run;
      run += v[u];
    }
  }
  return run;
}

__global__ __launch_bounds__(kBlock) void k_scan(ExchangeArgs a) {
  __shared__ uint32_t wsum[kWaves];
  __shared__ uint32_t is_last;
  __shared__ uint32_t zero_count[kWaves];
  {
    const uint32_t t0 = blockIdx.x * a.scan_tiles, t1 = min(a.num_tiles, t0 + a.scan_tiles);
    for (uint32_t d = threadIdx.x; d < a.N; d += kBlock)
      a.blk_base[(uint64_t)blockIdx.x * a.N + d] = column_scan(a.tile_base, a.N, d, t0, t1);
  }
  // The last workgroup to finish scans the block totals and turns the
  // destination totals into segment offsets.
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) is_last = atomicAdd(&a.ctl[1], 1u) == gridDim.x - 1;
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  for (uint32_t d = threadIdx.x; d < a.N; d += kBlock) {
    const uint32_t total = column_scan(a.blk_base, a.N, d, 0, a.num_blk);
    a.expected[d] = a.capacity ? min(total, a.capacity) : total;  // the tuples d keeps
  }
  __syncthreads();

  const uint32_t N = a.N;
  const uint32_t per = (N + kBlock - 1) / kBlock;
  const uint32_t lo = min(N, threadIdx.x * per), hi = min(N, lo + per);
  uint32_t local = 0;
  for (uint32_t d = lo; d < hi; ++d) local += __hip_atomic_load(&a.expected[d], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t total;
  const uint32_t ex = block_exclusive_scan(local, wsum, total);
  int64_t run = ex;
  uint32_t zeros = 0;
  for (uint32_t d = lo; d < hi; ++d) {
    const uint32_t e = __hip_atomic_load(&a.expected[d], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a.seg[d] = run;
    if (a.offsets_out) a.offsets_out[d] = run;
    run += e;
    a.arrived[d] = 0;
    a.b_arrived[d] = 0;
    if (e == 0) {  // nothing will arrive: the input of B[d] is complete now
      fire(a.f, NODE_EXCH, d, a.epoch, false);
      fire(a.f, NODE_B, d, a.epoch, false);
      ++zeros;
    }
  }
  if (threadIdx.x == kBlock - 1) {
    a.seg[N] = (int64_t)total;
    if (a.offsets_out) a.offsets_out[N] = (int64_t)total;
  }
  // count the destinations completed here
  uint32_t z = zeros;
#pragma unroll
  for (uint32_t o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o, 64);
  if ((threadIdx.x & 63) == 0) zero_count[threadIdx.x >> 6] = z;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t zt = 0;
    for (uint32_t i = 0; i < kWaves; ++i) zt += zero_count[i];
    __hip_atomic_store(&a.ctl[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // next call
    __hip_atomic_store(&a.ctl[0], zt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // B futures fired
    if (zt == N) fire(a.f, NODE_RESULT, 0, a.epoch, false);
  }
}

// ------------------------------------------------------------------ scatter
template <typename U>
__device__ __forceinline__ U apply_a(U v, const ExchangeArgs& a);

template <>
__device__ __forceinline__ u32x4 apply_a<u32x4>(u32x4 v, const ExchangeArgs& a) {
  f32x4 f = __builtin_bit_cast(f32x4, v);
  f.x = fmaf(a.a_a, f.x, a.a_b);
  f.y = fmaf(a.a_a, f.y, a.a_b);
  f.z = fmaf(a.a_a, f.z, a.a_b);
  f.w = fmaf(a.a_a, f.w, a.a_b);
  return __builtin_bit_cast(u32x4, f);
}
template <>
__device__ __forceinline__ uint32_t apply_a<uint32_t>(uint32_t v, const ExchangeArgs& a) {
  const float f = fmaf(a.a_a, __uint_as_float(v), a.a_b);
  return __float_as_uint(f);
}

// Copy the payload rows of one 64-tuple chunk: tuple t of the chunk (lane t
// holds its slot and source row) goes to slot __shfl(slot, t). Unit U is 16
// bytes when rows are a multiple of 16 bytes, else 4 bytes;
// v_units = row_bytes / sizeof(U). kCopyBatch units per lane are loaded
// before any is stored, so each wave keeps 16 KiB of reads in flight (a
// whole chunk of 256-byte rows; measured 2% faster than 8 KiB).
constexpr uint32_t kCopyBatch = 16;

template <typename U, bool kAffine>
__device__ __forceinline__ void copy_chunk(const ExchangeArgs& a, uint32_t lane, int slot, uint32_t srow,
                                           bool valid, uint32_t v_units, uint32_t v_shift, bool v_pow2) {
  const uint32_t total = 64u * v_units;
  for (uint32_t j0 = 0; j0 < total; j0 += 64u * kCopyBatch) {
    U v[kCopyBatch];
    int dslot[kCopyBatch];
    uint32_t unit[kCopyBatch];
    bool ok[kCopyBatch];
#pragma unroll
    for (uint32_t u = 0; u < kCopyBatch; ++u) {
      const uint32_t i = j0 + u * 64u + lane;
      const bool in = (j0 + u * 64u) < total;  // wave-uniform
      uint32_t t = 0, k = 0;
      if (in) {
        if (v_pow2) {
          t = i >> v_shift;
          k = i & (v_units - 1);
        } else {
          t = i / v_units;
          k = i - t * v_units;
        }
      }
      const int ts = __shfl(slot, (int)t, 64);
      const int tv = __shfl((int)valid, (int)t, 64);
      const uint32_t tr = (uint32_t)__shfl((int)srow, (int)t, 64);
      ok[u] = in && tv;
      dslot[u] = ts;
      unit[u] = k;
      if (ok[u]) {
        const U* src = reinterpret_cast<const U*>(a.src + (uint64_t)tr * a.row_bytes);
        v[u] = __builtin_nontemporal_load(src + k);
      }
    }
#pragma unroll
    for (uint32_t u = 0; u < kCopyBatch; ++u) {
      if (ok[u]) {
        U x = v[u];
        if (kAffine) x = apply_a<U>(x, a);
        U* dst = reinterpret_cast<U*>(a.dst + (uint64_t)dslot[u] * a.row_bytes);
        __builtin_nontemporal_store(x, dst + unit[u]);
      }
    }
  }
}

// kCap: each destination keeps its first `capacity` tuples in tuple order.
// Then wrun holds ranks inside the destination (not slots), a tuple is kept
// if its rank is below the capacity, and its slot is the segment start
// (segl) plus the rank; a dropped tuple moves nothing and its slot_of is -1.
template <bool kAffine, bool kCap>
__global__ __launch_bounds__(kBlock) void k_scatter(ExchangeArgs a) {
  extern __shared__ uint32_t lds[];
  const uint32_t N = a.N;
  uint32_t* wrun = lds;            // [kWaves][N]: next slot (kCap: rank) of each destination, per wave
  uint32_t* tcnt = lds + kWaves * N;  // [N]: tuples of this tile per destination that are kept
  uint32_t* segl = tcnt + N;          // [N] kCap: segment starts
  for (uint32_t i = threadIdx.x; i < kWaves * N; i += kBlock) wrun[i] = 0;
  __syncthreads();

  const uint32_t w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t sub = a.tile / kWaves;
  const uint64_t g0 = (uint64_t)blockIdx.x * a.tile + (uint64_t)w * sub;
  uint32_t* mine = wrun + w * N;
  bool bad = false;

  // 1. per-wave counts of this wave's contiguous sub-tile
  {
    const WaveDests wd = load_wave_dests(a, g0, sub, lane, bad);
#pragma unroll
    for (uint32_t i = 0; i < kMaxChunks; ++i)
      if (wd.d[i] >= 0) atomicAdd(&mine[wd.d[i]], 1u);
  }
  __syncthreads();

  // 2. first slot of each (wave, destination): segment start + this tile's
  //    start inside the segment + the counts of earlier waves
  for (uint32_t d = threadIdx.x; d < N; d += kBlock) {
    const uint32_t rank0 = a.blk_base[(uint64_t)(blockIdx.x / a.scan_tiles) * N + d] +
                           a.tile_base[(uint64_t)blockIdx.x * N + d];
    const uint32_t base = kCap ? rank0 : (uint32_t)a.seg[d] + rank0;
    uint32_t run = base;
#pragma unroll
    for (uint32_t ww = 0; ww < kWaves; ++ww) {
      const uint32_t c = wrun[ww * N + d];
      wrun[ww * N + d] = run;
      run += c;
    }
    if (kCap) {
      tcnt[d] = min(run, a.capacity) - min(base, a.capacity);
      segl[d] = (uint32_t)a.seg[d];
    } else {
      tcnt[d] = run - base;
    }
  }
  __syncthreads();

  // 3. stable rank inside each 64-tuple chunk, then move the rows
  const uint32_t unit_bytes = (a.row_bytes % 16u == 0) ? 16u : 4u;
  const uint32_t v_units = a.row_bytes / unit_bytes;
  const bool v_pow2 = (v_units & (v_units - 1)) == 0;
  const uint32_t v_shift = v_pow2 ? (uint32_t)__builtin_ctz(v_units) : 0u;
  for (uint32_t c = 0; c < sub && g0 + c < a.G; c += 64) {
    const uint64_t g = g0 + c + lane;
    const int d = load_dest(a, g, bad);
    const bool valid_d = d >= 0;
    const uint64_t peers = match_peers(d, valid_d, a.nbits);
    const uint32_t rank = (uint32_t)__popcll(peers & lanemask_lt(lane));
    int slot = 0;
    bool keep = valid_d;
    if (valid_d) {
      const uint32_t r = mine[d] + rank;  // kCap: rank inside d; else the slot
      // every lane has read mine[] before the group's leader advances it
      if (rank == 0) mine[d] = r + (uint32_t)__popcll(peers);
      if (kCap) {
        keep = r < a.capacity;
        slot = (int)(segl[d] + r);
      } else {
        slot = (int)r;
      }
    }
    // a slot past the end can only come from dest changing between the
    // histogram and this pass; never write outside the output
    const bool valid = keep && (uint64_t)slot < a.dst_rows;
    if (keep && !valid) bad = true;
    if (valid && a.src_index) a.src_index[slot] = (int32_t)g;
    if (valid_d && a.slot_of) a.slot_of[g] = valid ? slot : -1;
    const uint32_t srow = valid ? (uint32_t)(g / a.fanout) : 0u;
    if (unit_bytes == 16u)
      copy_chunk<u32x4, kAffine>(a, lane, slot, srow, valid, v_units, v_shift, v_pow2);
    else
      copy_chunk<uint32_t, kAffine>(a, lane, slot, srow, valid, v_units, v_shift, v_pow2);
  }
  if (bad) latch(a.f.status, ST_BAD_DEST);
  __syncthreads();

  // 4. progress: count this tile's arrivals; completing a destination fires it
  for (uint32_t d = threadIdx.x; d < N; d += kBlock) {
    const uint32_t n = tcnt[d];
    if (n == 0) continue;
    const uint32_t old = __hip_atomic_fetch_add(&a.arrived[d], n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + n == a.expected[d]) {
      fire(a.f, NODE_EXCH, d, a.epoch, false);
      if (!a.b_gated) {  // B has no work of its own: it completes with its input
        fire(a.f, NODE_B, d, a.epoch, false);
        const uint32_t r = __hip_atomic_fetch_add(&a.ctl[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (r + 1 == N) fire(a.f, NODE_RESULT, 0, a.epoch, false);
      }
    }
  }
}

// ------------------------------------------------------------------------ B
// Largest d with seg[d] <= s (s < seg[N]).
__device__ __forceinline__ uint32_t segment_of(const int64_t* seg, uint32_t N, int64_t s) {
  uint32_t lo = 0, hi = N - 1;
  while (lo < hi) {
    const uint32_t mid = (lo + hi + 1) >> 1;
    if (seg[mid] <= s) lo = mid; else hi = mid - 1;
  }
  return lo;
}

constexpr uint32_t kBRows = 256;  // output slots per B workgroup

__global__ __launch_bounds__(kBlock) void k_b(ExchangeArgs a) {
  __shared__ uint32_t range[2];
  __shared__ uint32_t go;
  const int64_t total = a.seg[a.N];
  const int64_t s0 = (int64_t)blockIdx.x * kBRows;
  if (s0 >= total) return;
  const int64_t s1 = min<int64_t>(total, s0 + kBRows);
  if (threadIdx.x == 0) {
    const uint32_t d0 = segment_of(a.seg, a.N, s0), d1 = segment_of(a.seg, a.N, s1 - 1);
    bool ok = true;
    for (uint32_t d = d0; d <= d1 && ok; ++d) ok = await_prior(a.f, NODE_EXCH, d, a.epoch);
    range[0] = d0;
    range[1] = d1;
    go = ok;
  }
  __syncthreads();
  if (!go) return;

  const uint32_t P = a.row_bytes / 4u;
  const float* y = reinterpret_cast<const float*>(a.dst);
  float* out = reinterpret_cast<float*>(a.b_out);
  if (a.b_kind == OP_ROWSUM) {
    // 16 lanes per row, 16 rows per pass of the workgroup
    const uint32_t l16 = threadIdx.x & 15, r = threadIdx.x >> 4;
    const bool vec = (P % 4u) == 0;
    const int64_t passes = (s1 - s0 + 15) / 16;
    for (int64_t p = 0; p < passes; ++p) {
      const int64_t s = s0 + p * 16 + r;
      float acc = 0.f;
      const bool in = s < s1;
      if (in) {
        const float* row = y + s * (int64_t)P;
        if (vec) {
          for (uint32_t e = l16; e < P / 4u; e += 16) {
            const float4 v = reinterpret_cast<const float4*>(row)[e];
            acc += (v.x + v.y) + (v.z + v.w);
          }
        } else {
          for (uint32_t e = l16; e < P; e += 16) acc += row[e];
        }
      }
      acc += __shfl_xor(acc, 8, 16);
      acc += __shfl_xor(acc, 4, 16);
      acc += __shfl_xor(acc, 2, 16);
      acc += __shfl_xor(acc, 1, 16);
      if (in && l16 == 0) out[s] = acc;
    }
  } else if (a.b_kind == OP_AFFINE) {
    const int64_t n = (s1 - s0) * (int64_t)P;
    for (int64_t i = threadIdx.x; i < n; i += kBlock) {
      const int64_t k = s0 * (int64_t)P + i;
      out[k] = fmaf(a.b_a, y[k], a.b_b);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (uint32_t d = range[0]; d <= range[1]; ++d) {
      const int64_t lo = max<int64_t>(s0, a.seg[d]), hi = min<int64_t>(s1, a.seg[d + 1]);
      if (hi <= lo) continue;
      const uint32_t n = (uint32_t)(hi - lo);
      const uint32_t old = __hip_atomic_fetch_add(&a.b_arrived[d], n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old + n == a.expected[d]) {
        fire(a.f, NODE_B, d, a.epoch, false);
        const uint32_t r = __hip_atomic_fetch_add(&a.ctl[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (r + 1 == a.N) fire(a.f, NODE_RESULT, 0, a.epoch, false);
      }
    }
  }
}

}  // namespace

// wrun and tcnt, plus segl with a capacity (MOE plans only: N <= 64)
size_t scatter_lds_bytes(uint32_t N, bool cap) { return (size_t)(kWaves + (cap ? 2 : 1)) * N * sizeof(uint32_t); }

hipError_t launch_hist(const ExchangeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_hist, dim3(a.num_tiles), dim3(kBlock), a.N * sizeof(uint32_t), s, a);
  return hipGetLastError();
}

hipError_t launch_src_counts(const ExchangeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_src_counts, dim3(a.num_src), dim3(kBlock), a.N * sizeof(uint32_t), s, a);
  return hipGetLastError();
}

hipError_t launch_scan(const ExchangeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_scan, dim3(a.num_blk), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scatter(const ExchangeArgs& a, hipStream_t s) {
  const bool cap = a.capacity != 0;
  const size_t lds = scatter_lds_bytes(a.N, cap);
  if (cap && a.a_kind == OP_AFFINE)
    hipLaunchKernelGGL((k_scatter<true, true>), dim3(a.num_tiles), dim3(kBlock), lds, s, a);
  else if (cap)
    hipLaunchKernelGGL((k_scatter<false, true>), dim3(a.num_tiles), dim3(kBlock), lds, s, a);
  else if (a.a_kind == OP_AFFINE)
    hipLaunchKernelGGL((k_scatter<true, false>), dim3(a.num_tiles), dim3(kBlock), lds, s, a);
  else
    hipLaunchKernelGGL((k_scatter<false, false>), dim3(a.num_tiles), dim3(kBlock), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_b(const ExchangeArgs& a, hipStream_t s) {
  const uint64_t blocks = (a.G + kBRows - 1) / kBRows;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_b, dim3((uint32_t)blocks), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace pw
