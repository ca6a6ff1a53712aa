// Chained execution of Arg -> A -> B -> Result over N shards, K steps.
//
// PATHWAYS page ("PATHWAYS: Asynchronous Distributed Dataflow for ML"),
// section 5.1 "Single-controller dispatch overheads": a trivial computation
// repeated with each result fed into the next, submitted one call per
// computation (OpByOp), as one call for a whole chain (Chained), or as one
// node looping internally (Fused). Section 4.5: with static shapes all host
// work for the chain is done before it runs and the whole subgraph is handed
// over in one message; section 4.3: under data parallelism each of the N
// shards sends one tuple to the same shard of the next node.
//
// Split placement (k_chain_split): A[i] and B[i] on different workgroups,
// normally on different XCDs, so every gate is a handoff across CUs (coherent
// stores, an epoch store, coherent loads).
//
// Device mapping of the default chained kernel: one group of lanes per shard (the whole wave, or with
// 128-element shards and many shards half of it, so that the CUs hold fewer
// waves). The plan fixes the placement before the chain
// starts, so the producer of every future (A[i] of step k, B[i] of step k)
// and its consumer (B[i] of step k, A[i] of step k + 1) run on the same lanes:
// the gate is a load of the HBM future table ordered after the producer's
// stores by program order, with no cross-CU fence. Node outputs
// live in HBM buffers (state for B, a_buf for A), as the page's object store
// keeps them in accelerator memory.
#include "device.h"

namespace pw {

namespace {

__device__ __forceinline__ float body(uint32_t kind, float a, float b, float x) {
  return kind == OP_AFFINE ? fmaf(a, x, b) : x;
}

// Gate on a future these lanes produced themselves. The first lane of the
// shard's group both fires and reads every future of its shard, so program
// order makes the fire visible to the read and a relaxed load suffices; each
// lane only reads payload elements it wrote itself. The result is broadcast
// to the group. Bounded like every device wait.
__device__ __forceinline__ bool await_local_lane0(const Futures& f, uint32_t node, uint32_t shard, uint32_t epoch) {
  const uint32_t* p = &f.epoch[node * f.width + shard];
  if (epoch_reached(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT), epoch)) return true;
  const uint64_t t0 = wall_clock64();
  while (true) {
    __builtin_amdgcn_s_sleep(1);
    if (epoch_reached(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT), epoch)) return true;
    if (wall_clock64() - t0 > f.spin_ticks) {
      latch(f, ST_TIMEOUT);
      return false;
    }
  }
}

// `sub` is the lane's index inside its shard's lane group, `lead` the group's
// first lane (0 when the whole wave serves one shard).
__device__ __forceinline__ bool await_local(const Futures& f, uint32_t node, uint32_t shard, uint32_t epoch,
                                            uint32_t sub, uint32_t lead = 0) {
  bool ok = true;
  if (sub == 0) ok = await_local_lane0(f, node, shard, epoch);
  return __shfl((int)ok, (int)lead, 64) != 0;
}

// One count per shard; the last of them fires the Result.
__device__ __forceinline__ void finish_shard(const ChainArgs& a, uint32_t sub) {
  if (sub == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.done_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 == a.done_target) fire(a.f, NODE_RESULT, 0, a.epoch0 + a.steps);
  }
}

// One node (A or B) of one shard: out[e] = body(in[e]), E elements, lanes
// striding by 64 with two elements in flight per lane.
__device__ __forceinline__ void node_body(const float* in, float* out, uint32_t E, uint32_t lane, uint32_t kind,
                                          float ca, float cb) {
  uint32_t e = lane;
  for (; e + 64 < E; e += 128) {
    const float x0 = in[e], x1 = in[e + 64];
    out[e] = body(kind, ca, cb, x0);
    out[e + 64] = body(kind, ca, cb, x1);
  }
  if (e < E) out[e] = body(kind, ca, cb, in[e]);
}

// node_body for data handed across XCDs inside one launch: every load and
// store is agent-coherent (device.h), so that no fence is needed around it.
__device__ __forceinline__ void node_body_coherent(const float* in, float* out, uint32_t E, uint32_t lane,
                                                   uint32_t kind, float ca, float cb) {
  const __amdgpu_buffer_rsrc_t ri = raw_buffer(in, E * 4u), ro = raw_buffer(out, E * 4u);
  uint32_t e = lane;
  for (; e + 64 < E; e += 128) {
    const float x0 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ri, e * 4u, 0, kCoherent));
    const float x1 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ri, (e + 64) * 4u, 0, kCoherent));
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, body(kind, ca, cb, x0)), ro, e * 4u, 0, kCoherent);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, body(kind, ca, cb, x1)), ro, (e + 64) * 4u, 0,
                                          kCoherent);
  }
  if (e < E) {
    const float x = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ri, e * 4u, 0, kCoherent));
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, body(kind, ca, cb, x)), ro, e * 4u, 0, kCoherent);
  }
}

// Fire a future whose only consumer is this lane group (its first lane calls
// it): a plain store; the fire count and the stamp are kept in registers by
// the caller and written once when the launch ends.
__device__ __forceinline__ void fire_local(const Futures& f, uint32_t node, uint32_t shard, uint32_t epoch) {
  __hip_atomic_store(&f.epoch[node * f.width + shard], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
}

// One node of one shard with the gate folded in: the group's first lane reads
// the input future while every lane reads its input elements; the elements are
// used only once the future is known to have fired (else they are read again
// after the wait). With 128-element shards each of the 64/kG lanes of a group
// owns 2·kG consecutive elements; other sizes use a whole wave (kG = 1).
template <int kG>
__device__ __forceinline__ bool gated_node(const ChainArgs& a, uint32_t in_node, uint32_t shard, uint32_t need,
                                           const float* in, float* out, uint32_t sub, uint32_t lead, uint32_t kind,
                                           float ca, float cb) {
  uint32_t v = need;
  if (sub == 0) v = __hip_atomic_load(&a.f.epoch[in_node * a.f.width + shard], __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_WAVEFRONT);
  if (kG > 1 || a.E == 128) {
    using V = float __attribute__((ext_vector_type(2 * kG)));
    V x = reinterpret_cast<const V*>(in)[sub];
    // the group's answer from its first lane: a ballot (scalar) rather than
    // a lane shuffle through LDS, which cost ~50 ns per node here
    const bool ready = (__ballot(sub == 0 && epoch_reached(v, need)) >> lead) & 1ull;
    if (!ready) {
      if (!await_local(a.f, in_node, shard, need, sub, lead)) return false;
      x = reinterpret_cast<const V*>(in)[sub];
    }
#pragma unroll
    for (int e = 0; e < 2 * kG; ++e) x[e] = body(kind, ca, cb, x[e]);
    reinterpret_cast<V*>(out)[sub] = x;
    return true;
  }
  const bool ready = __shfl((int)epoch_reached(v, need), 0, 64) != 0;
  if (!ready && !await_local(a.f, in_node, shard, need, sub)) return false;
  node_body(in, out, a.E, sub, kind, ca, cb);
  return true;
}

template <int kG>
__global__ __launch_bounds__(256) void k_chain_chained(ChainArgs a) {
  constexpr uint32_t kLanes = 64 / kG;
  const uint32_t lane = threadIdx.x & 63, sub = lane % kLanes, lead = lane - sub;
  const uint32_t i = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kG + lane / kLanes;
  if (i >= a.N) return;  // whole lane groups only; no workgroup barrier below
  float* st = a.state + (uint64_t)i * a.E;
  float* ab = a.abuf + (uint64_t)i * a.E;
  uint32_t done = 0;
  for (uint32_t j = 1; j <= a.steps; ++j) {
    const uint32_t k = a.epoch0 + j;
    // A of step k consumes the Result of step k - 1 (B[i]; epoch0 = the Arg)
    if (!gated_node<kG>(a, NODE_B, i, k - 1, st, ab, sub, lead, a.a_kind, a.a_a, a.a_b)) break;
    if (sub == 0 && a.f.stamps && j == a.steps) a.f.stamps[NODE_A * a.f.width + i] = wall_clock64();
    if (sub == 0) fire_local(a.f, NODE_A, i, k);
    if (!gated_node<kG>(a, NODE_A, i, k, ab, st, sub, lead, a.b_kind, a.b_a, a.b_b)) break;
    if (sub == 0 && a.f.stamps && j == a.steps) a.f.stamps[NODE_B * a.f.width + i] = wall_clock64();
    if (sub == 0) fire_local(a.f, NODE_B, i, k);
    done = j;
  }
  if (sub == 0 && done) {
    for (uint32_t node : {NODE_A, NODE_B})
      __hip_atomic_fetch_add(&a.f.fires[node * a.f.width + i], done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  finish_shard(a, sub);
}

// Split placement: each wave claims one role (A or B) and a group of shards,
// so A[i] and B[i] run on different waves of different workgroups; A prefers
// the first half of the XCDs and B the second, so the two nodes of a shard
// normally sit on different XCDs and every future crosses them: the producer
// writes its node's output with agent-coherent stores, waits until they have
// completed and stores the epoch; the consumer polls the epoch, then reads
// with agent-coherent loads (no release or acquire fence, each of which
// would write back or invalidate the XCD's whole L2). The claim counters give every shard exactly one wave per role (the
// grid has one wave per (role, group) slot, plus at most three spare waves
// that find nothing and leave). With PW_FLAG_TRACE each node stamps its last
// fire at the moment it fires.
// kG shards per wave (64 / kG lanes each; with kG > 1 the shards have 128
// elements, 2 kG per lane): a wave claims a group of kG consecutive shards for
// one role, waits until every one of its shards' inputs fired, and publishes
// all of their outputs after one wait for its stores.
template <int kG>
__global__ __launch_bounds__(256) void k_chain_split(ChainArgs a) {
  constexpr uint32_t kLanes = 64 / kG;
  const uint32_t lane = threadIdx.x & 63, sub = lane % kLanes, grp = lane / kLanes;
  const uint32_t groups = (a.N + kG - 1) / kG;
  uint32_t role = 2, gi = 0;
  if (lane == 0) {
    const uint32_t x = xcc_id();
    const uint32_t pref = a.nxcc > 1 ? (x % a.nxcc < a.nxcc / 2 ? 0u : 1u) : ((blockIdx.x * 4 + (threadIdx.x >> 6)) & 1u);
    uint32_t k = __hip_atomic_fetch_add(&a.role_ctr[pref], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (k < groups) {
      role = pref;
      gi = k;
    } else {
      k = __hip_atomic_fetch_add(&a.role_ctr[pref ^ 1u], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (k < groups) {
        role = pref ^ 1u;
        gi = k;
      }
    }
  }
  role = __shfl(role, 0, 64);
  gi = __shfl(gi, 0, 64);
  if (role == 2) return;  // a spare wave
  const uint32_t i = gi * kG + grp;  // this lane group's shard
  const bool mine = i < a.N;
  if (mine && sub == 0) a.place[2 * i + role] = xcc_id();
  const uint32_t node = role == 0 ? NODE_A : NODE_B, in_node = role == 0 ? NODE_B : NODE_A;
  const uint32_t kind = role == 0 ? a.a_kind : a.b_kind;
  const float ca = role == 0 ? a.a_a : a.b_a, cb = role == 0 ? a.a_b : a.b_b;
  float* st = a.state + (uint64_t)(mine ? i : 0) * a.E;
  float* ab = a.abuf + (uint64_t)(mine ? i : 0) * a.E;
  const float* in = role == 0 ? st : ab;
  float* out = role == 0 ? ab : st;
  const uint32_t* gate = &a.f.epoch[in_node * a.f.width + (mine ? i : 0)];
  uint32_t done = 0;
  for (uint32_t j = 1; j <= a.steps; ++j) {
    const uint32_t k = a.epoch0 + j;
    // A of step k consumes B of step k - 1 (the Result; epoch0 = the Arg), B consumes A of step k.
    // Each group's first lane polls its shard's input future (relaxed); the
    // wave goes on once all have fired.
    const uint32_t need = role == 0 ? k - 1 : k;
    bool ok = true;
    if (sub == 0 && mine) ok = epoch_reached(__hip_atomic_load(gate, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), need);
    if (__ballot(!ok)) {
      const uint64_t t0 = wall_clock64();
      while (true) {
        __builtin_amdgcn_s_sleep(1);
        if (!ok) ok = epoch_reached(__hip_atomic_load(gate, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), need);
        if (!__ballot(!ok)) break;
        if (wall_clock64() - t0 > a.f.spin_ticks) {
          if (lane == 0) latch(a.f, ST_TIMEOUT);
          break;
        }
      }
      if (__ballot(!ok)) break;  // expired
    }
    if constexpr (kG > 1) {  // 2 kG consecutive elements per lane, as kG / 2 float4 (16-byte aligned)
      if (mine) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        typedef uint32_t u4 __attribute__((ext_vector_type(4)));
        constexpr int kQ = kG > 1 ? kG / 2 : 1;
        const __amdgpu_buffer_rsrc_t ri = raw_buffer(in, a.E * 4u), ro = raw_buffer(out, a.E * 4u);
        f4 x[kQ];
#pragma unroll
        for (int q = 0; q < kQ; ++q)
          x[q] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(ri, (sub * kQ + q) * 16u, 0, kCoherent));
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[q][e] = body(kind, ca, cb, x[q][e]);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, x[q]), ro, (sub * kQ + q) * 16u, 0,
                                                 kCoherent);
        }
      }
    } else {
      node_body_coherent(in, out, a.E, lane, kind, ca, cb);
    }
    wait_vmem_all();  // the wave's coherent stores of every output have completed, then the epochs
    if (sub == 0 && mine) {
      const uint32_t idx = node * a.f.width + i;
      if (a.f.stamps && j == a.steps) a.f.stamps[idx] = wall_clock64();
      __hip_atomic_store(&a.f.epoch[idx], k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    done = j;
  }
  if (sub == 0 && mine && done)
    __hip_atomic_fetch_add(&a.f.fires[node * a.f.width + i], done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (role == 1 && mine) finish_shard(a, sub);
}

__global__ void k_chain_reset(ChainArgs a) {
  if (threadIdx.x < 2) a.role_ctr[threadIdx.x] = 0;
}

// OpByOp: one launch per node per step. The input future was fired by the
// previous launch, so stream order already made it (and its buffer) visible.
__global__ __launch_bounds__(256) void k_chain_node(ChainArgs a) {
  const uint32_t i = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (i >= a.N) return;
  const uint32_t k = a.epoch0 + a.steps;  // the step this node belongs to
  float* st = a.state + (uint64_t)i * a.E;
  float* ab = a.abuf + (uint64_t)i * a.E;
  if (a.node == NODE_A) {
    if (!await_local(a.f, NODE_B, i, k - 1, lane)) return;
    node_body(st, ab, a.E, lane, a.a_kind, a.a_a, a.a_b);
    if (lane == 0) fire(a.f, NODE_A, i, k);
  } else {
    if (!await_local(a.f, NODE_A, i, k, lane)) return;
    node_body(ab, st, a.E, lane, a.b_kind, a.b_a, a.b_b);
    if (lane == 0) fire(a.f, NODE_B, i, k);
    if (a.done_ctr) finish_shard(a, lane);
  }
}

// Fused: one node per shard looping over every step in registers; only the
// final buffers and futures are written.
__global__ __launch_bounds__(256) void k_chain_fused(ChainArgs a) {
  const uint32_t i = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (i >= a.N) return;
  float* st = a.state + (uint64_t)i * a.E;
  float* ab = a.abuf + (uint64_t)i * a.E;
  if (!await_local(a.f, NODE_B, i, a.epoch0, lane)) return;
  for (uint32_t e = lane; e < a.E; e += 64) {
    float x = st[e], y = x;
    for (uint32_t j = 0; j < a.steps; ++j) {
      y = body(a.a_kind, a.a_a, a.a_b, x);
      x = body(a.b_kind, a.b_a, a.b_b, y);
    }
    ab[e] = y;
    st[e] = x;
  }
  if (lane == 0) {
    fire(a.f, NODE_A, i, a.epoch0 + a.steps);
    fire(a.f, NODE_B, i, a.epoch0 + a.steps);
  }
  finish_shard(a, lane);
}

}  // namespace

// Shards per wave for the chained kernel. A gated node's latency grows with
// the waves a CU holds (measured, one shard per wave: ~280 ns per node up to
// 4 waves per CU, ~360 at 6 to 8, ~405 at 16). Two 128-element shards per
// wave cost ~350 ns from 1024 to 2048 shards and ~395 at 4096, so only shard
// counts above 1536 pack them; four per wave were slower (~480-500).
static uint32_t chain_pack(uint32_t N, uint32_t E) { return E == 128 && N > 1536 ? 2 : 1; }

// Shards per wave of the split placement: one up to 128 shards, two above
// (128-element shards only). A wave goes on once the inputs of all its
// shards have fired, so it waits for the slowest of their producers: per
// gated node at 256 / 512 / 1024 / 2048 shards, one shard per wave 1.55 /
// 1.67 / 1.98 / 2.17 us, two 1.50 / 1.52 / 1.61 / 1.75, four 2.13 / 2.15 /
// 2.17 / 2.20, eight 4.17 / 4.25 / 4.26 / 4.22.
static uint32_t split_pack(uint32_t N, uint32_t E) { return E == 128 && N > 128 ? 2 : 1; }

// Workgroups of the split-placement kernel: one wave per (role, group of shards).
static uint32_t split_grid(uint32_t N, uint32_t g) { return (2 * ((N + g - 1) / g) + 3) / 4; }

static const void* split_kernel(uint32_t g) {
  return g == 2 ? (const void*)k_chain_split<2> : (const void*)k_chain_split<1>;
}

bool chain_split_fits(int device, uint32_t N, uint32_t E) {
  int cus = 0, per_cu = 0;
  const uint32_t g = split_pack(N, E);
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return false;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, split_kernel(g), 256, 0) != hipSuccess) return false;
  return (uint64_t)cus * per_cu >= split_grid(N, g);
}

hipError_t launch_chain(const ChainArgs& a, uint32_t mode, hipStream_t s) {
  const dim3 grid((a.N + 3) / 4), block(256);
  if (mode == 3) {
    hipLaunchKernelGGL(k_chain_reset, dim3(1), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const uint32_t g = split_pack(a.N, a.E);
    const dim3 sgrid(split_grid(a.N, g));
    if (g == 2)
      hipLaunchKernelGGL(k_chain_split<2>, sgrid, block, 0, s, a);
    else
      hipLaunchKernelGGL(k_chain_split<1>, sgrid, block, 0, s, a);
    return hipGetLastError();
  }
  if (mode == 0) {
    const uint32_t g = chain_pack(a.N, a.E), waves = (a.N + g - 1) / g;
    const dim3 cgrid((waves + 3) / 4);
    if (g == 2)
      hipLaunchKernelGGL(k_chain_chained<2>, cgrid, block, 0, s, a);
    else
      hipLaunchKernelGGL(k_chain_chained<1>, cgrid, block, 0, s, a);
  } else if (mode == 2)
    hipLaunchKernelGGL(k_chain_fused, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(k_chain_node, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace pw
