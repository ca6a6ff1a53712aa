// Sparse shard-to-shard exchange on one MI355X.
//
// PATHWAYS page ("PATHWAYS: Asynchronous Distributed Dataflow for ML"),
// section 4.3 "Coordination implementation": every node emits tuples tagged
// with a destination shard, the runtime moves them among dynamically chosen
// shards along the sharded edge, and progress tracking decides when a shard
// has all of its messages; sections 4.4-4.5: the successor consumes buffer
// futures and the interconnect writes straight into the successor's input
// buffers. On one GPU the "interconnect" is HBM, and the exchange is a stable
// counting sort by destination done in three launches (two for tiny ones):
//
//   rank    one workgroup per tile of `tile` consecutive tuples matches the
//           tuples of each 64-tuple chunk by destination (ballots), counts
//           its destinations (one LDS atomic per group), writes the row
//           tile_base[tile][*] (and a copy, tile_cnt), and ranks each tuple
//           among the tuples of the tile with the same destination, in tuple
//           order (wave by wave), into rank[g] (16 bits); with few tiles
//           (one scan block, or at most 16 blocks with at most 256 (block,
//           destination) columns in all) its last workgroup also runs the
//           scan below, one column per thread;
//   scan    one workgroup per block of 16 tiles runs, per destination, down
//           its rows (where each tile's run of d starts inside the block)
//           and writes the block totals; those are scanned over the blocks
//           (by the last block workgroup for up to 16 blocks, else by a
//           second launch with 16 threads per destination), and the last
//           workgroup turns the destination totals into segment offsets,
//           sets the expected count of every destination and fires the
//           futures of destinations that receive nothing;
//   scatter one short-lived workgroup per chunk of ~16 KiB of payload (64
//           rows of 256 bytes) finds each tuple's slot (segment start + the
//           tile's run start + its rank), applies A and writes each payload
//           row with 16-byte vector stores straight into its destination
//           segment. Each XCD takes one contiguous eighth of the chunks, in
//           order, and a CU holds 4 of these workgroups, so the workgroups
//           in flight on an XCD read one compact window of the input and
//           append to a few destination runs through one L2: measured on
//           this part, a copy split into 16 KiB pieces per workgroup runs at
//           ~6.3 TB/s, one whose workgroups each own 64 KiB or more at ~5.5,
//           and the scatter gained 8% from the per-XCD ranges. The last chunk of a
//           tile to finish adds the tile's per-destination counts to the
//           arrival counters; the add that completes a destination fires that
//           destination's future.
//
// B (exchange.hip: k_b) runs per block of output slots and computes only once
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

// ------------------------------------------------------------ scan helpers
// Exclusive running sum, in place, of the column d of rows [r0, r1) of a
// row-major [rows][N] table; returns the column total. The loads of 16 rows
// are issued before any is needed (unconditionally: rows past r1 re-read row
// r1 - 1 and count zero). kCoherent: the rows were written by other
// workgroups of the same launch, read with agent-coherent loads.
template <bool kCoherent = false>
__device__ __forceinline__ uint32_t column_scan(uint32_t* t, uint32_t N, uint32_t d, uint32_t r0, uint32_t r1) {
  constexpr uint32_t kB = 16;
  uint32_t run = 0;
  for (uint32_t r = r0; r < r1; r += kB) {
    uint32_t v[kB];
#pragma unroll
    for (uint32_t u = 0; u < kB; ++u) {
      uint32_t* e = &t[(uint64_t)min(r + u, r1 - 1) * N + d];
      v[u] = kCoherent ? __hip_atomic_load(e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *e;
    }
#pragma unroll
    for (uint32_t u = 0; u < kB; ++u) {
      if (r + u < r1) {
        t[(uint64_t)(r + u) * N + d] = run;
        run += v[u];
      }
    }
  }
  return run;
}

// Workgroup-shared state of the scan's last step.
struct ScanShared {
  uint32_t wsum[kWaves];
  uint32_t zero_count[kWaves];
  uint32_t is_last;
};

// True in the last workgroup of the grid to get here (counter ctl[1], reset
// by scan_finish). What that workgroup reads of the others' writes is
// written with agent-coherent stores, complete (every wave waits for its
// stores here) before the workgroup's count, and read with agent-coherent
// loads: no release or acquire fence, each of which would write back or
// invalidate the XCD's whole L2.
__device__ __forceinline__ bool last_to_arrive(const ExchangeArgs& a, ScanShared& sh) {
  wait_vmem_all();
  __syncthreads();
  if (threadIdx.x == 0) sh.is_last = atomicAdd(&a.ctl[1], 1u) == gridDim.x - 1;
  __syncthreads();
  return sh.is_last;
}

// The scan's last step, in one workgroup, once expected[d] (the tuples d
// keeps) is known for every destination (exp_of(d) reads it): segment
// offsets, the arrival counters cleared, and the futures of destinations
// that receive nothing fired now.
template <typename ExpOf>
__device__ __forceinline__ void scan_finish(const ExchangeArgs& a, ScanShared& sh, ExpOf exp_of) {
  const uint32_t N = a.N;
  const uint32_t per = (N + kBlock - 1) / kBlock;
  const uint32_t lo = min(N, threadIdx.x * per), hi = min(N, lo + per);
  uint32_t local = 0;
  for (uint32_t d = lo; d < hi; ++d) local += exp_of(d);
  uint32_t total;
  const uint32_t ex = block_exclusive_scan(local, sh.wsum, total);
  int64_t run = ex;
  uint32_t zeros = 0;
  for (uint32_t d = lo; d < hi; ++d) {
    const uint32_t e = exp_of(d);
    a.seg[d] = run;
    if (a.offsets_out) a.offsets_out[d] = run;
    run += e;
    a.arrived[d] = 0;
    a.b_arrived[d] = 0;
    if (e == 0) {  // nothing will arrive: the input of B[d] is complete now
      fire(a.f, NODE_EXCH, d, a.epoch);
      fire(a.f, NODE_B, d, a.epoch);
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
  if ((threadIdx.x & 63) == 0) sh.zero_count[threadIdx.x >> 6] = z;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t zt = 0;
    for (uint32_t i = 0; i < kWaves; ++i) zt += sh.zero_count[i];
    __hip_atomic_store(&a.ctl[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // next call
    __hip_atomic_store(&a.ctl[0], zt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // B futures fired
    if (zt == N) fire(a.f, NODE_RESULT, 0, a.epoch);
  }
}

// Both levels in one workgroup, for small tables (at most kOneMaxBlk blocks
// and at most one (block, destination) column per thread): thread b N + d
// runs down column d of block b (one round of loads) and leaves the block
// total in `part`; then every block's run start (the earlier blocks' totals
// of its destination) and the destination totals come from LDS, and the
// finish runs. kCoherent: the tile rows were written by other workgroups of
// the same launch (the fused scan of k_rank).
constexpr uint32_t kOneMaxBlk = 16;

template <bool kCoherent>
__device__ __forceinline__ void scan_one(const ExchangeArgs& a, ScanShared& sh, uint32_t* part, uint32_t* tot) {
  const uint32_t N = a.N, B = a.num_blk;
  const uint32_t b = threadIdx.x / N, d = threadIdx.x % N;
  const bool live = b < B;  // N * B <= kBlock
  if (live) {
    const uint32_t t0 = b * a.scan_tiles, t1 = min(a.num_tiles, t0 + a.scan_tiles);
    part[threadIdx.x] = column_scan<kCoherent>(a.tile_base, N, d, t0, t1);
  }
  __syncthreads();
  if (live) {
    uint32_t pre = 0, all = 0;
    for (uint32_t q = 0; q < B; ++q) {
      const uint32_t x = part[q * N + d];
      pre += q < b ? x : 0u;
      all += x;
    }
    a.blk_base[(uint64_t)b * N + d] = pre;
    if (b == 0) {
      const uint32_t e = a.capacity ? min(all, a.capacity) : all;  // the tuples d keeps
      a.expected[d] = e;
      tot[d] = e;
    }
  }
  __syncthreads();
  scan_finish(a, sh, [&](uint32_t dd) { return tot[dd]; });
}

// --------------------------------------------------------------------- rank
// A wave's destinations (kChunks chunks of 64 tuples: tile / 256), loaded
// before any is checked, so that the loads of its whole sub-tile are in
// flight together: the loads are unconditional (indices clamped to the last
// tuple) because a load under a branch, or one whose value is checked right
// away, makes the compiler wait for it before issuing the next. -1: past the
// end, or out of range (latched through `bad`).
template <uint32_t kChunks>
struct WaveDests {
  int d[kChunks];
};

template <uint32_t kChunks>
__device__ __forceinline__ WaveDests<kChunks> load_wave_dests(const ExchangeArgs& a, uint64_t g0, uint32_t lane,
                                                              bool& bad) {
  WaveDests<kChunks> w;
  if (a.G == 0) {  // uniform: an empty step reads nothing
#pragma unroll
    for (uint32_t i = 0; i < kChunks; ++i) w.d[i] = -1;
    return w;
  }
  if (g0 + kChunks * 64 <= a.G) {  // uniform: the whole sub-tile exists (every tile but the last)
    const int* p = a.dest + g0 + lane;
#pragma unroll
    for (uint32_t i = 0; i < kChunks; ++i) w.d[i] = p[i * 64];
#pragma unroll
    for (uint32_t i = 0; i < kChunks; ++i) {
      const bool in_range = (uint32_t)w.d[i] < a.N;  // also rejects negatives
      bad |= !in_range;
      w.d[i] = in_range ? w.d[i] : -1;
    }
    return w;
  }
  const uint64_t last = a.G - 1;
#pragma unroll
  for (uint32_t i = 0; i < kChunks; ++i) w.d[i] = a.dest[min<uint64_t>(g0 + i * 64 + lane, last)];
#pragma unroll
  for (uint32_t i = 0; i < kChunks; ++i) {
    const int d = w.d[i];
    const bool in_range = d >= 0 && (uint32_t)d < a.N;
    const bool exists = g0 + i * 64 + lane < a.G;
    bad |= exists && !in_range;
    w.d[i] = exists && in_range ? d : -1;
  }
  return w;
}

// At least 8 waves per SIMD (the compiler then keeps some scalars in vector
// lanes): 4096 ranking tiles are then exactly two rounds of resident
// workgroups instead of 2.3 (rank 60 -> 58 us).
//
// The ballot matching costs about eight vector instructions per key bit per
// chunk, and bounds this kernel by instruction issue. A tile usually holds far
// fewer distinct destinations than N (a source shard sends to a few shards),
// so the destinations present in the tile are first given dense ids (their
// order among the present ones) and the lanes are matched on the bits of
// those ids only: 2 bits instead of 8 for 4 destinations out of 256. Equal
// ids mean equal destinations, so the groups, and the ranks, are the same
// (rank 44 -> 30 us on 256 shards x 65536 tuples sent to 4 shards each).
// Tried and dropped: with at most 4 ids, one running count per id in scalar
// registers and one ballot per id and chunk instead of the matching (39 us).
template <uint32_t kChunks>
__global__ __launch_bounds__(kBlock, 8) void k_rank(ExchangeArgs a) {
  extern __shared__ uint32_t lds[];
  __shared__ uint32_t s_wsum[kWaves];
  const uint32_t N = a.N;
  uint32_t* wrun = lds;  // [kWaves][N]: counts of each wave's sub-tile, then its next rank per destination
  uint16_t* cid = reinterpret_cast<uint16_t*>(lds + kWaves * N);  // [N]: 1 if present, then the dense id
  for (uint32_t i = threadIdx.x; i < kWaves * N; i += kBlock) wrun[i] = 0;
  for (uint32_t i = threadIdx.x; i < N; i += kBlock) cid[i] = 0;
  const uint32_t w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr uint32_t sub = kChunks * 64;  // the wave's sub-tile (tile = 4 sub-tiles)
  const uint64_t g0 = (uint64_t)blockIdx.x * a.tile + (uint64_t)w * sub;
  uint32_t* mine = wrun + w * N;
  bool bad = false;
  const WaveDests<kChunks> wd = load_wave_dests<kChunks>(a, g0, lane, bad);
  __syncthreads();
  // 0. dense ids of the destinations present in the tile, 256 destinations
  //    at a time: a ballot of the present ones, offset by the earlier waves'
  //    and the earlier rounds' counts
#pragma unroll
  for (uint32_t i = 0; i < kChunks; ++i)
    if (wd.d[i] >= 0) cid[wd.d[i]] = 1;
  __syncthreads();
  uint32_t K = 0;  // destinations present (uniform)
  for (uint32_t d0 = 0; d0 < N; d0 += kBlock) {
    const uint32_t d = d0 + threadIdx.x;
    const bool present = d < N && cid[d] != 0;
    const uint64_t m = __ballot(present);
    if (lane == 0) s_wsum[w] = (uint32_t)__popcll(m);
    __syncthreads();
    uint32_t pre = K, tot = 0;
#pragma unroll
    for (uint32_t ww = 0; ww < kWaves; ++ww) {
      const uint32_t c = s_wsum[ww];
      pre += ww < w ? c : 0u;
      tot += c;
    }
    if (present) {
      const uint32_t id = pre + (uint32_t)__popcll(m & lanemask_lt(lane));
      cid[d] = (uint16_t)id;
    }
    K += tot;
    __syncthreads();
  }
  K = __builtin_amdgcn_readfirstlane(K);
  const uint32_t nb = K <= 1 ? 0u : 32u - (uint32_t)__builtin_clz(K - 1);  // bits of the largest id
  // 1. per-wave counts of its contiguous sub-tile: each 64-tuple chunk's
  //    lanes are matched by destination id once (ballots); the lowest lane of
  //    each group adds the group's size (one LDS atomic per group: one per
  //    lane queued up to 64 deep on a tile's few destinations) and every lane
  //    keeps its rank inside the group, 16 bits each, for step 3
  uint32_t grp[kChunks];  // rank inside the chunk's group | group size << 16
#pragma unroll
  for (uint32_t i = 0; i < kChunks; ++i) {
    grp[i] = 0;
    const int d = wd.d[i];
    const bool valid = d >= 0;
    const int c = valid ? (int)cid[d] : -1;
    const uint64_t peers = match_peers(c, valid, nb);
    if (valid) {
      const uint32_t rank = (uint32_t)__popcll(peers & lanemask_lt(lane)), n = (uint32_t)__popcll(peers);
      if (rank == 0) atomicAdd(&mine[d], n);
      grp[i] = rank | n << 16;
    }
  }
  __syncthreads();
  // 2. the tile's counts (for the scan, and kept for the arrival counts) and
  //    the first rank of each (wave, destination): the counts of earlier waves
  for (uint32_t d = threadIdx.x; d < N; d += kBlock) {
    uint32_t run = 0;
#pragma unroll
    for (uint32_t ww = 0; ww < kWaves; ++ww) {
      const uint32_t c = wrun[ww * N + d];
      wrun[ww * N + d] = run;
      run += c;
    }
    // coherent: with a fused scan the last workgroup reads it (below)
    __hip_atomic_store(&a.tile_base[(uint64_t)blockIdx.x * N + d], run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a.tile_cnt[(uint64_t)blockIdx.x * N + d] = run;
  }
  if (threadIdx.x == 0) a.tile_done[blockIdx.x] = 0;
  __syncthreads();
  // 3. stable rank inside the tile: the chunks in order, each group starting
  //    where the earlier chunks (and earlier waves) left its destination
#pragma unroll
  for (uint32_t i = 0; i < kChunks; ++i) {
    const int d = wd.d[i];
    if (d >= 0) {
      const uint32_t rank = grp[i] & 0xffffu;
      const uint32_t r = mine[d] + rank;
      // every lane has read mine[] before the group's leader advances it
      if (rank == 0) mine[d] = r + (grp[i] >> 16);
      a.rank[g0 + i * 64 + lane] = (uint16_t)r;
    }
  }
  if (bad) latch(a.f, ST_BAD_DEST);
  if (!a.fuse_scan) return;
  // Few tiles (one scan block, or a small table of blocks: the host decides):
  // the last workgroup to finish ranking runs the whole scan here instead of
  // in a launch of its own. With one block the destination totals pass
  // through LDS (wrun is free once every wave has ranked).
  __shared__ ScanShared sh;
  if (!last_to_arrive(a, sh)) return;
  if (a.num_blk > 1) {  // several scan blocks, one column of one block per thread
    __shared__ uint32_t part[kBlock], tot[kBlock];
    scan_one<true>(a, sh, part, tot);
    return;
  }
  uint32_t* exp_lds = wrun;
  for (uint32_t d = threadIdx.x; d < N; d += kBlock) {
    const uint32_t total = column_scan<true>(a.tile_base, N, d, 0, a.num_tiles);
    const uint32_t e = a.capacity ? min(total, a.capacity) : total;  // the tuples d keeps
    a.expected[d] = e;
    a.blk_base[d] = 0;  // the one scan block starts every run at 0 (the scatter adds this row)
    exp_lds[d] = e;
  }
  __syncthreads();
  scan_finish(a, sh, [&](uint32_t d) { return exp_lds[d]; });
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
// Level 1: block b of scan_tiles tiles (16 unless the step has more than 4096
// tiles) runs down each destination's column of its tiles: the exclusive
// prefix inside the block in place, the block total to blk_base[b] (the
// loads of a column are in flight together).
__global__ __launch_bounds__(kBlock) void k_scan_blocks(ExchangeArgs a) {
  const uint32_t t0 = blockIdx.x * a.scan_tiles, t1 = min(a.num_tiles, t0 + a.scan_tiles);
  for (uint32_t d = threadIdx.x; d < a.N; d += kBlock)
    a.blk_base[(uint64_t)blockIdx.x * a.N + d] = column_scan(a.tile_base, a.N, d, t0, t1);
}

// Both levels in one launch, for at most 16 blocks: level 1 as above, then
// the last workgroup to finish scans each destination's block totals (one
// round of loads) and turns the destination totals into segment offsets.
// With more blocks the second level runs as its own launch (k_scan_top):
// one workgroup walking 256 block rows per destination costs more than the
// launch (C2: 18.4 -> 14 us; for 8 blocks the extra launch costs ~2 us).
__global__ __launch_bounds__(kBlock) void k_scan(ExchangeArgs a) {
  __shared__ ScanShared sh;
  {
    const uint32_t t0 = blockIdx.x * a.scan_tiles, t1 = min(a.num_tiles, t0 + a.scan_tiles);
    for (uint32_t d = threadIdx.x; d < a.N; d += kBlock)
      __hip_atomic_store(&a.blk_base[(uint64_t)blockIdx.x * a.N + d], column_scan(a.tile_base, a.N, d, t0, t1),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!last_to_arrive(a, sh)) return;
  for (uint32_t d = threadIdx.x; d < a.N; d += kBlock) {
    const uint32_t total = column_scan<true>(a.blk_base, a.N, d, 0, a.num_blk);
    a.expected[d] = a.capacity ? min(total, a.capacity) : total;  // the tuples d keeps
  }
  __syncthreads();
  scan_finish(a, sh, [&](uint32_t d) {
    return __hip_atomic_load(&a.expected[d], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  });
}

// The scan in a launch of its own for small tables: one workgroup, no
// workgroup waiting for another, a single round of loads before its stores.
__global__ __launch_bounds__(kBlock) void k_scan_one(ExchangeArgs a) {
  __shared__ ScanShared sh;
  __shared__ uint32_t part[kBlock], tot[kBlock];
  scan_one<false>(a, sh, part, tot);
}

// Level 2: kTopDest destinations per workgroup and kTopLanes threads per
// destination, each holding up to 16 consecutive block totals (the layout
// keeps num_blk <= 256), loaded unconditionally so that all are in flight
// together: the block totals become exclusive prefixes in place and the
// destination total goes to expected[d]; the last workgroup to finish turns
// the totals into segment offsets.
constexpr uint32_t kTopDest = 16, kTopLanes = kBlock / kTopDest;

__global__ __launch_bounds__(kBlock) void k_scan_top(ExchangeArgs a) {
  __shared__ ScanShared sh;
  __shared__ uint32_t part[kTopLanes * kTopDest];
  const uint32_t N = a.N, B = a.num_blk;
  const uint32_t j = threadIdx.x % kTopDest, p = threadIdx.x / kTopDest;
  const uint32_t d = blockIdx.x * kTopDest + j;
  const bool live = d < N;
  const uint32_t per = (B + kTopLanes - 1) / kTopLanes;  // <= 16
  const uint32_t b0 = p * per;
  uint32_t v[16];
#pragma unroll
  for (uint32_t r = 0; r < 16; ++r) {
    const bool in = live && r < per && b0 + r < B;
    v[r] = a.blk_base[(uint64_t)(in ? b0 + r : 0) * N + (live ? d : 0)];
  }
  uint32_t local = 0;
#pragma unroll
  for (uint32_t r = 0; r < 16; ++r) {
    v[r] = live && r < per && b0 + r < B ? v[r] : 0u;
    local += v[r];
  }
  part[p * kTopDest + j] = local;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (uint32_t q = 0; q < kTopLanes; ++q) {
    const uint32_t x = part[q * kTopDest + j];
    pre += q < p ? x : 0u;
    tot += x;
  }
  uint32_t run = pre;
#pragma unroll
  for (uint32_t r = 0; r < 16; ++r) {
    if (live && r < per && b0 + r < B) a.blk_base[(uint64_t)(b0 + r) * N + d] = run;
    run += v[r];
  }
  if (live && p == 0)  // the tuples d keeps; the last workgroup reads them (coherent)
    __hip_atomic_store(&a.expected[d], a.capacity ? min(tot, a.capacity) : tot, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  if (!last_to_arrive(a, sh)) return;
  scan_finish(a, sh, [&](uint32_t dd) {
    return __hip_atomic_load(&a.expected[dd], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  });
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

// Tuples per scatter workgroup: about 16 KiB of payload, a power of two
// that divides the tile (tiles are powers of two >= 256), at most kMaxChunk.
constexpr uint32_t kMaxChunk = 1024;
constexpr uint32_t kCopyBatch = 4;  // units per thread loaded before any is stored (16 KiB per workgroup)

// The payload units of one batch (kCopyBatch per thread) of the chunk: unit
// i is unit i % vu of tuple i / vu. Source rows do not depend on the slots.
// kPairs (fan-out 2: tuples 2k and 2k + 1 carry the same row k): unit i is
// unit i % vu of the chunk's row i / vu, loaded once and stored to the slots
// of both its tuples.
template <typename U, bool kPairs>
struct Batch {
  U v[kCopyBatch];

  __device__ __forceinline__ void load(const ExchangeArgs& a, uint64_t g0, uint32_t j0, uint32_t total, uint32_t vu,
                                       bool pow2, uint32_t shift) {
#pragma unroll
    for (uint32_t u = 0; u < kCopyBatch; ++u) {
      const uint32_t i = j0 + u * kBlock + threadIdx.x;
      if (i < total) {
        const uint32_t t = pow2 ? i >> shift : i / vu;
        const uint64_t g = g0 + (kPairs ? 2 * t : t);  // the (first) tuple of the unit
        if (g < a.G) {
          const U* src = reinterpret_cast<const U*>(a.src + (kPairs ? g / 2 : g / a.fanout) * a.row_bytes);
          v[u] = __builtin_nontemporal_load(src + (i - t * vu));
        }
      }
    }
  }

  template <bool kAffine>
  __device__ __forceinline__ void store(const ExchangeArgs& a, const int* s_slot, uint32_t j0, uint32_t total,
                                        uint32_t vu, bool pow2, uint32_t shift) const {
#pragma unroll
    for (uint32_t u = 0; u < kCopyBatch; ++u) {
      const uint32_t i = j0 + u * kBlock + threadIdx.x;
      if (i < total) {
        const uint32_t t = pow2 ? i >> shift : i / vu;
        U x = v[u];
        if (kAffine) x = apply_a<U>(x, a);
#pragma unroll
        for (uint32_t c = 0; c < (kPairs ? 2u : 1u); ++c) {
          const int slot = s_slot[kPairs ? 2 * t + c : t];
          if (slot >= 0) {
            U* dst = reinterpret_cast<U*>(a.dst + (uint64_t)slot * a.row_bytes);
            // the MoE dispatch stores plainly (130-131 us against 135-136
            // with nontemporal stores; the expert FFN reading the rows next
            // runs the same either way)
            if (kPairs)
              dst[i - t * vu] = x;
            else
              __builtin_nontemporal_store(x, dst + (i - t * vu));
          }
        }
      }
    }
  }
};

// One workgroup per chunk of a.chunk consecutive tuples (inside one tile);
// chunks are dealt to XCDs in 8 contiguous ranges (xcd_contiguous).
// Unit U is 16 bytes when rows are a multiple of 16 bytes, else 4 bytes.
// The chunk's first batch of payload loads is issued before the slots are
// looked up, so the two round trips overlap. kCap: each destination keeps
// its first `capacity` tuples in tuple order: a tuple is kept if its rank
// inside the destination is below the capacity; a dropped tuple moves
// nothing and its slot_of is -1. kPairs: fan-out 2 with 16-byte units (the
// chunk is even and starts at an even tuple), each row loaded once.
template <typename U, bool kAffine, bool kCap, bool kPairs>
__global__ __launch_bounds__(kBlock) void k_scatter(ExchangeArgs a) {
  __shared__ int s_slot[kMaxChunk];  // destination slot of each tuple of the chunk, -1: nothing to move
  __shared__ uint32_t s_last;
  const uint32_t N = a.N, C = a.chunk;
  const uint64_t g0 = (uint64_t)xcd_contiguous(blockIdx.x, gridDim.x) * C;
  const uint32_t tile = (uint32_t)(g0 / a.tile);
  const uint32_t* tbase = a.tile_base + (uint64_t)tile * N;
  const uint32_t* bbase = a.blk_base + (uint64_t)(tile / a.scan_tiles) * N;
  const uint32_t vu = a.row_bytes / (uint32_t)sizeof(U);
  const bool pow2 = (vu & (vu - 1)) == 0;
  const uint32_t shift = pow2 ? (uint32_t)__builtin_ctz(vu) : 0u;
  const uint32_t total = (kPairs ? C / 2 : C) * vu;  // units to load
  Batch<U, kPairs> b;
  b.load(a, g0, 0, total, vu, pow2, shift);

  bool bad = false;
  for (uint32_t t = threadIdx.x; t < C; t += kBlock) {
    const uint64_t g = g0 + t;
    const int d = load_dest(a, g, bad);
    int slot = -1;
    if (d >= 0) {
      const uint32_t r = bbase[d] + tbase[d] + a.rank[g];  // rank inside destination d
      const bool keep = !kCap || r < a.capacity;
      const uint64_t sl = (uint64_t)a.seg[d] + r;
      // a slot past the end can only come from dest changing between the
      // ranking and this pass; never write outside the output
      const bool valid = keep && sl < a.dst_rows;
      if (keep && !valid) bad = true;
      if (valid) slot = (int)sl;
      if (valid && a.src_index) a.src_index[sl] = (int32_t)g;
      if (a.slot_of) a.slot_of[g] = slot;
    }
    s_slot[t] = slot;
  }
  __syncthreads();

  b.template store<kAffine>(a, s_slot, 0, total, vu, pow2, shift);
  for (uint32_t j0 = kBlock * kCopyBatch; j0 < total; j0 += kBlock * kCopyBatch) {
    b.load(a, g0, j0, total, vu, pow2, shift);
    b.template store<kAffine>(a, s_slot, j0, total, vu, pow2, shift);
  }
  if (bad) latch(a.f, ST_BAD_DEST);

  // progress: the last chunk of a tile to finish counts the tile's arrivals;
  // completing a destination fires it (consumers run in later launches: the
  // kernel boundary orders the rows before them)
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t t0 = (uint64_t)tile * a.tile;
    const uint64_t in_tile = min<uint64_t>(a.tile, a.G - t0);
    const uint32_t chunks = (uint32_t)((in_tile + C - 1) / C);
    const uint32_t old = __hip_atomic_fetch_add(&a.tile_done[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = old + 1 == chunks;
  }
  __syncthreads();
  if (!s_last) return;
  const uint32_t* tcnt = a.tile_cnt + (uint64_t)tile * N;
  for (uint32_t d = threadIdx.x; d < N; d += kBlock) {
    uint32_t n = tcnt[d];
    if (kCap && n) {
      const uint32_t base = bbase[d] + tbase[d];
      n = min(base + n, a.capacity) - min(base, a.capacity);  // the tuples of the tile that d keeps
    }
    if (n == 0) continue;
    const uint32_t old = __hip_atomic_fetch_add(&a.arrived[d], n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + n == a.expected[d]) {
      fire(a.f, NODE_EXCH, d, a.epoch);
      if (!a.b_gated) {  // B has no work of its own: it completes with its input
        fire(a.f, NODE_B, d, a.epoch);
        const uint32_t r = __hip_atomic_fetch_add(&a.ctl[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (r + 1 == N) fire(a.f, NODE_RESULT, 0, a.epoch);
      }
    }
  }
}

// ------------------------------------------------------------------------ B
// B over output slots [s0, s0 + kBRows) (kBRows: 64 or 128; row sums in
// passes of 16 rows of 16 lanes). The destinations whose non-empty
// segments overlap those slots are found, and their exchange futures checked,
// with one round of loads: each thread reads the segment bounds and the
// future of the destinations it owns (d = threadIdx.x + k * kBlock), and the
// overlapping ones (at most kBRows: each holds a slot of the range) go to an
// LDS list. After the rows, one thread per listed destination adds its slot
// count to the B arrivals. A segment's length is the tuple count its
// destination keeps, so the last adder knows it completed B[d].
//
// Row sums of rows of at most 256 bytes (one float4 per lane) load the rows
// before that round of checks, so that the two round trips overlap: the
// scatter ran in an earlier launch on this stream, so the rows are complete
// whatever the checks find, and the values are used only once every future
// checked has fired (rows past the buffer re-read its last row and are never
// stored).
template <uint32_t kBRows>
__global__ __launch_bounds__(kBlock) void k_b(ExchangeArgs a) {
  constexpr uint32_t kBPasses = kBRows / 16;
  __shared__ uint32_t n_over;
  __shared__ uint32_t over_d[kBRows];
  __shared__ int64_t over_lo[kBRows], over_hi[kBRows];
  if (threadIdx.x == 0) n_over = 0;
  const int64_t s0 = (int64_t)blockIdx.x * kBRows;
  const uint32_t P = a.row_bytes / 4u, P4 = P / 4u;
  const uint32_t l16 = threadIdx.x & 15, r = threadIdx.x >> 4;
  const bool early = a.b_kind == OP_ROWSUM && P % 4u == 0 && P4 <= 16 && a.dst_rows > 0;  // uniform
  float4 ev[kBPasses];
  if (early) {
    const float4* y4 = reinterpret_cast<const float4*>(a.dst);
#pragma unroll
    for (uint32_t p = 0; p < kBPasses; ++p) {  // unconditional loads: all in flight together
      const uint64_t row = min<uint64_t>((uint64_t)s0 + p * 16 + r, a.dst_rows - 1);
      ev[p] = y4[row * P4 + min(l16, P4 - 1)];
    }
  }
  __syncthreads();
  const int64_t total = a.seg[a.N];
  bool ok = true;
  for (uint32_t d = threadIdx.x; d < a.N; d += kBlock) {
    const int64_t lo = a.seg[d], hi = a.seg[d + 1];
    // volatile: issued with the segment loads, not sunk into the branch
    // below (which would add a round trip)
    const uint32_t v = *reinterpret_cast<const volatile uint32_t*>(&a.f.epoch[NODE_EXCH * a.f.width + d]);
    if (lo < hi && lo < s0 + kBRows && hi > s0) {
      if (!epoch_reached(v, a.epoch)) ok = ok && await_prior(a.f, NODE_EXCH, d, a.epoch);
      const uint32_t k = atomicAdd(&n_over, 1u);
      over_d[k] = d;
      over_lo[k] = lo;
      over_hi[k] = hi;
    }
  }
  if (!__syncthreads_and(ok) || s0 >= total) return;  // uniform
  const int64_t s1 = min<int64_t>(total, s0 + kBRows);

  const float* y = reinterpret_cast<const float*>(a.dst);
  float* out = reinterpret_cast<float*>(a.b_out);
  if (early) {  // the same sums, in the same order, as below
#pragma unroll
    for (uint32_t p = 0; p < kBPasses; ++p) {
      float x = 0.f;
      if (l16 < P4) x += (ev[p].x + ev[p].y) + (ev[p].z + ev[p].w);
      x += __shfl_xor(x, 8, 16);
      x += __shfl_xor(x, 4, 16);
      x += __shfl_xor(x, 2, 16);
      x += __shfl_xor(x, 1, 16);
      const int64_t s = s0 + p * 16 + r;
      if (s < s1 && l16 == 0) out[s] = x;
    }
  } else if (a.b_kind == OP_ROWSUM) {
    // 16 lanes per row, 16 rows per pass; the passes are unrolled so that
    // every lane's loads of all of them are in flight together
    const bool vec = (P % 4u) == 0;
    float acc[kBPasses];
#pragma unroll
    for (uint32_t p = 0; p < kBPasses; ++p) {
      const int64_t s = s0 + p * 16 + r;
      acc[p] = 0.f;
      if (s < s1) {
        const float* row = y + s * (int64_t)P;
        if (vec) {
          for (uint32_t e = l16; e < P / 4u; e += 16) {
            const float4 v = reinterpret_cast<const float4*>(row)[e];
            acc[p] += (v.x + v.y) + (v.z + v.w);
          }
        } else {
          for (uint32_t e = l16; e < P; e += 16) acc[p] += row[e];
        }
      }
    }
#pragma unroll
    for (uint32_t p = 0; p < kBPasses; ++p) {
      float x = acc[p];
      x += __shfl_xor(x, 8, 16);
      x += __shfl_xor(x, 4, 16);
      x += __shfl_xor(x, 2, 16);
      x += __shfl_xor(x, 1, 16);
      const int64_t s = s0 + p * 16 + r;
      if (s < s1 && l16 == 0) out[s] = x;
    }
  } else if (a.b_kind == OP_AFFINE) {
    const int64_t n = (s1 - s0) * (int64_t)P;
#pragma unroll 4
    for (int64_t i = threadIdx.x; i < n; i += kBlock) {
      const int64_t k = s0 * (int64_t)P + i;
      out[k] = fmaf(a.b_a, y[k], a.b_b);
    }
  }
  __syncthreads();
  if (threadIdx.x < n_over) {
    const uint32_t d = over_d[threadIdx.x];
    const int64_t lo = max<int64_t>(s0, over_lo[threadIdx.x]), hi = min<int64_t>(s1, over_hi[threadIdx.x]);
    const uint32_t n = (uint32_t)(hi - lo), want = (uint32_t)(over_hi[threadIdx.x] - over_lo[threadIdx.x]);
    const uint32_t old = __hip_atomic_fetch_add(&a.b_arrived[d], n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + n == want) {
      fire(a.f, NODE_B, d, a.epoch);
      const uint32_t r = __hip_atomic_fetch_add(&a.ctl[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (r + 1 == a.N) fire(a.f, NODE_RESULT, 0, a.epoch);
    }
  }
}

}  // namespace

// tile / 256 chunks of 64 tuples per wave (tiles are powers of two in
// [256, 4096], chosen at plan time)
hipError_t launch_rank(const ExchangeArgs& a, hipStream_t s) {
  // per-wave counts [kWaves][N] u32, then the dense ids [N] u16
  const size_t lds = (size_t)kWaves * a.N * sizeof(uint32_t) + ((size_t)a.N * 2 + 3) / 4 * 4;
  switch (a.tile) {
    case 256: hipLaunchKernelGGL(k_rank<1>, dim3(a.num_tiles), dim3(kBlock), lds, s, a); break;
    case 512: hipLaunchKernelGGL(k_rank<2>, dim3(a.num_tiles), dim3(kBlock), lds, s, a); break;
    case 1024: hipLaunchKernelGGL(k_rank<4>, dim3(a.num_tiles), dim3(kBlock), lds, s, a); break;
    case 2048: hipLaunchKernelGGL(k_rank<8>, dim3(a.num_tiles), dim3(kBlock), lds, s, a); break;
    case 4096: hipLaunchKernelGGL(k_rank<16>, dim3(a.num_tiles), dim3(kBlock), lds, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

uint32_t scatter_chunk(uint32_t tile, uint32_t row_bytes, uint32_t fanout) {
  // about 16 KiB loaded per chunk: with fan-out 2 (16-byte units) a chunk
  // loads each row once for two tuples, so it holds twice the tuples
  const uint32_t f = fanout == 2 && row_bytes % 16 == 0 ? 2 : 1;
  uint32_t c = f;
  while (c < kMaxChunk && c < tile && (uint64_t)c * 2 * row_bytes <= 16384ull * f) c *= 2;
  return c;
}

hipError_t launch_src_counts(const ExchangeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_src_counts, dim3(a.num_src), dim3(kBlock), a.N * sizeof(uint32_t), s, a);
  return hipGetLastError();
}

hipError_t launch_scan(const ExchangeArgs& a, hipStream_t s) {
  if (a.num_blk > 256) return hipErrorInvalidValue;  // the layout keeps it <= 256
  if (a.num_blk <= kOneMaxBlk && (uint64_t)a.num_blk * a.N <= kBlock) {
    hipLaunchKernelGGL(k_scan_one, dim3(1), dim3(kBlock), 0, s, a);
    return hipGetLastError();
  }
  if (a.num_blk <= 16) {
    hipLaunchKernelGGL(k_scan, dim3(a.num_blk), dim3(kBlock), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_scan_blocks, dim3(a.num_blk), dim3(kBlock), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_scan_top, dim3((a.N + kTopDest - 1) / kTopDest), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

// The scatter moves rows fastest with 4 resident workgroups per CU (the
// 160 KiB of LDS then holds 4 of them), not the 8 its registers allow:
// 1.545-1.551 ms against 1.572-1.575 at 8, 1.571-1.575 at 6 and 1.557-1.565
// at 3, on the large exchange. Fewer chunks in flight keep the addresses
// being read and written in a narrower window. The launch reserves the LDS
// that caps the count; the kernel does not use it. The MoE dispatch (fan-out
// 2: both tuples of a token copy the same 2 KiB row, so a chunk reads half
// the bytes it writes) is slower capped (175 against 151-163 us) and keeps
// the register-bound count.
constexpr size_t kScatterLdsReserve = 32 * 1024;

template <typename U, bool kPairs>
static hipError_t launch_scatter_u(const ExchangeArgs& a, uint32_t grid, hipStream_t s) {
  const bool cap = a.capacity != 0, aff = a.a_kind == OP_AFFINE;
  const size_t r = a.fanout == 1 ? kScatterLdsReserve : 0;
  if (cap && aff)
    hipLaunchKernelGGL((k_scatter<U, true, true, kPairs>), dim3(grid), dim3(kBlock), r, s, a);
  else if (cap)
    hipLaunchKernelGGL((k_scatter<U, false, true, kPairs>), dim3(grid), dim3(kBlock), r, s, a);
  else if (aff)
    hipLaunchKernelGGL((k_scatter<U, true, false, kPairs>), dim3(grid), dim3(kBlock), r, s, a);
  else
    hipLaunchKernelGGL((k_scatter<U, false, false, kPairs>), dim3(grid), dim3(kBlock), r, s, a);
  return hipGetLastError();
}

hipError_t launch_scatter(const ExchangeArgs& a, hipStream_t s) {
  const uint64_t grid = (a.G + a.chunk - 1) / a.chunk;
  if (grid == 0) return hipSuccess;
  if (a.row_bytes % 16u != 0) return launch_scatter_u<uint32_t, false>(a, (uint32_t)grid, s);
  // the pair path needs even chunks (scatter_chunk gives them for fan-out 2)
  if (a.fanout == 2 && a.chunk % 2 == 0) return launch_scatter_u<u32x4, true>(a, (uint32_t)grid, s);
  if (a.fanout > 2) return hipErrorInvalidValue;
  return launch_scatter_u<u32x4, false>(a, (uint32_t)grid, s);
}

// 128 output slots per B workgroup once that still gives every CU one (each
// then has twice the rows in flight, and a destination half the arrival adds:
// the 8-shard step's B 12.8 -> 10.4 us between events), else 64.
hipError_t launch_b(const ExchangeArgs& a, hipStream_t s) {
  if (a.G == 0) return hipSuccess;
  if (a.G >= 256ull * 128) {
    hipLaunchKernelGGL(k_b<128>, dim3((uint32_t)((a.G + 127) / 128)), dim3(kBlock), 0, s, a);
  } else {
    hipLaunchKernelGGL(k_b<64>, dim3((uint32_t)((a.G + 63) / 64)), dim3(kBlock), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pw
