// Device helpers shared by the pw kernels: wave64 peer matching, the status
// latch, and firing / awaiting buffer futures in the HBM future table.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace pw {

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt(uint32_t lane) { return (1ull << lane) - 1ull; }

// Lanes of this wave holding the same destination as this lane, found with
// one ballot per destination bit (wave64 has no native match instruction).
// Lanes with valid == false match nothing and get 0.
// Must be called by all 64 lanes with the same nbits.
__device__ __forceinline__ uint64_t match_peers(int d, bool valid, uint32_t nbits) {
  uint64_t m = __ballot(valid);
  for (uint32_t b = 0; b < nbits; ++b) {
    const bool bit = (d >> b) & 1;
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return valid ? m : 0ull;
}

// Latch `code` in the plan's status word unless an error is latched already
// (the first one wins), tagged with the epoch of the call that raised it so
// that the host reports it to waits on that call and later ones only.
__device__ __forceinline__ void latch(const Futures& f, uint32_t code) {
  uint64_t expected = 0;
  __hip_atomic_compare_exchange_strong(f.status, &expected, (uint64_t)code | (uint64_t)f.call_epoch << 32,
                                       __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Fire future (node, shard) for `epoch`: the fire-count add, then the epoch
// stored at system scope, so that a host thread polling the future table
// sees it while the launch still runs. Orders nothing before it: consumers in
// the same launch read the producer's data with agent-coherent loads (the
// producer wrote it with agent-coherent stores and waited for them) or share
// its XCD (the pipeline); consumers in a later launch are ordered by the kernel
// boundary.
__device__ __forceinline__ void fire(const Futures& f, uint32_t node, uint32_t shard, uint32_t epoch) {
  const uint32_t i = node * f.width + shard;
  if (f.stamps) f.stamps[i] = wall_clock64();
  __hip_atomic_fetch_add(&f.fires[i], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&f.epoch[i], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ __forceinline__ bool epoch_reached(uint32_t v, uint32_t epoch) {
  return (int32_t)(v - epoch) >= 0;
}

// Wait on a future fired by an EARLIER launch on the same stream: the kernel
// boundary already orders the producer's writes before this launch, so the
// first check is an ordinary cacheable load (agent-scope loads of the few
// hot future words, one or two per token in the MoE combine, would all go to
// memory); only if that finds the epoch missing (the producer failed) does
// the bounded spin with relaxed agent-scope loads follow. Same bound and
// latch as await_coherent().
__device__ __forceinline__ bool await_prior(const Futures& f, uint32_t node, uint32_t shard, uint32_t epoch) {
  const uint32_t* p = &f.epoch[node * f.width + shard];
  if (epoch_reached(*p, epoch)) return true;
  const uint64_t t0 = wall_clock64();
  while (true) {
    __builtin_amdgcn_s_sleep(1);
    if (epoch_reached(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), epoch)) return true;
    if (wall_clock64() - t0 > f.spin_ticks) {
      latch(f, ST_TIMEOUT);
      return false;
    }
  }
}

// Agent-coherent accesses, for data handed between workgroups of one launch
// without cache-wide fences. Each XCD has its own L2: an agent-scope release
// fence writes back every dirty line of the XCD's L2 and an agent-scope
// acquire invalidates it (buffer_wbl2 / buffer_inv), several microseconds
// each, and the invalidation also throws away every other workgroup's cached
// data. Instead, each access to such data carries the agent-scope coherence
// bit (sc1), as the compiler's relaxed agent-scope atomic loads and stores
// do: such a store writes through to the memory side, such a load does not
// hit a possibly stale cached copy. A producer waits until its coherent
// stores have completed (vmcnt 0) before the counter add or flag store that
// publishes them; a consumer issues its coherent loads only after it has seen
// that flag (a value it branched on, or a barrier after the wait).
constexpr int kCoherent = 16;  // sc1 in the cache-policy operand of buffer instructions
constexpr int kRawBufWord3 = 0x00020000;  // gfx9 raw buffer: 32-bit format, stride 0, size in bytes

// A raw buffer resource over `bytes` bytes at p (bytes < 2^31); accesses past
// the end return zero / are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRawBufWord3);
}

// Wait until every vector-memory operation of this wave has completed; a
// compiler barrier as well.
__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until future (node, shard) fired for `epoch` or later, for consumers
// in the same launch whose reads of the producer's data are agent-coherent
// loads (so no acquire fence: one would invalidate the XCD's whole L2). The
// word is polled with relaxed agent-scope loads, bounded by f.spin_ticks of
// the 100 MHz wall clock; on expiry it latches ST_TIMEOUT and returns false
// so the caller skips its work and the wave still exits.
__device__ __forceinline__ bool await_coherent(const Futures& f, uint32_t node, uint32_t shard, uint32_t epoch) {
  const uint32_t* p = &f.epoch[node * f.width + shard];
  bool ok = epoch_reached(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), epoch);
  const uint64_t t0 = ok ? 0 : wall_clock64();
  while (!ok) {
    __builtin_amdgcn_s_sleep(1);
    ok = epoch_reached(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), epoch);
    if (!ok && wall_clock64() - t0 > f.spin_ticks) {
      latch(f, ST_TIMEOUT);
      return false;
    }
  }
  return true;
}

// Which XCD (accelerator complex die, with its own L2) this wave runs on.
__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xf;
}

// Workgroup b's item out of n when the hardware deals workgroups to the 8
// XCDs round robin (workgroup b to XCD b mod 8): XCD x takes the x-th of 8
// contiguous ranges of items, in order, so that each XCD's L2 sees one
// contiguous stream instead of every eighth item. A bijection for any n.
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t b, uint32_t n) {
  const uint32_t q = n / 8, r = n % 8, x = b % 8, k = b / 8;
  return x * q + min(x, r) + k;
}

}  // namespace pw
