// bf16 MFMA GEMM tile core for gfx950: C[256 x 256] (fp32) = A[256 x K] . B[K x 256].
//
// Operands are both K-contiguous: A is row-major [rows][K] (activations) and
// the weights come pre-packed as B^T [N][K] (pack.hip turns the stored
// [in][out] weights around once, when the plan is built). One workgroup of 4
// waves owns a 256 x 256 output tile; wave w computes the 128 x 128 quadrant
// (w >> 1, w & 1) as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16, accumulators
// in AGPRs. The MFMA is fed B^T as its first operand and A as its second, so
// each block accumulates C^T: a lane then holds 4 consecutive output columns
// of one row per register quad, and lanes l and l + 32 hold the two halves of
// 8 consecutive columns, which the epilogue joins with one lane swap.
//
// K streams through a ring of 4 LDS stages of 32 columns (A 256 x 32 and
// B^T 256 x 32 bf16 = 32 KiB per stage, 128 KiB in all) filled by direct
// global-to-LDS loads (global_load_lds_dwordx4: no staging registers). Each
// wave-wide load writes 1 KiB of LDS contiguously (16 bytes per lane), so the
// 16-byte chunks of each 64-byte LDS row are permuted by picking which global
// chunk each lane fetches: chunk c of row r sits at slot c ^ ((r >> 2) & 3),
// which makes the MFMA operand reads (lane l reads row l % 32, chunk l / 32 of
// the k-step) free of LDS bank conflicts.
//
// A stage is consumed in two halves (its two k-steps of 16). One workgroup
// barrier per stage, between the halves, publishes the next stage and frees
// the ring slot of the previous one. Stage j is loaded in two halves spread
// between the MFMAs of the second half of stage j - 3 and the first half of
// stage j - 2. Issued as one burst after the barrier, the 32 loads of the
// workgroup would queue up in the address unit and stall each wave's MFMA
// stream until its own loads were taken; spread out, they are accepted while
// the matrix core is busy. Waits on the vector-memory counter are explicit
// and exact: the loop is peeled so that every wait, load and fragment read is
// unconditional and the compiler can interleave them with the MFMAs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pw {
namespace mm {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int BM = 256, BN = 256, BK = 32, NT = 256;
constexpr int kStages = 4;                      // (5 stages, the whole LDS, measured slower)
constexpr int kHalf = BM * BK * 2;              // one operand block of a stage: 16 KiB
constexpr int kStageBytes = 2 * kHalf;          // 32 KiB
constexpr int kLdsBytes = kStages * kStageBytes;  // 128 KiB

// Byte offsets inside a tile (rows x K of A, 256 x K of B^T, the output tile)
// must stay below 4 GiB: they are 32-bit.
struct Tile {
  const __bf16* A;   // first row of the tile; rows are K-contiguous
  int64_t lda;       // elements between rows of A
  int rows;          // valid rows (1..BM); the rest are read from row rows-1 and never stored
  const __bf16* Bt;  // first row (output column) of the tile in B^T; K-contiguous
  int64_t ldb;       // elements between rows of B^T
  int K;             // multiple of BK
};

typedef __attribute__((address_space(3))) void* lds_ptr;

// Word 3 of a raw buffer resource on gfx9 parts: 32-bit data format, no
// swizzle, no index stride; with stride 0 the size field is in bytes.
constexpr int kBufWord3 = 0x00020000;

// Chunk permutation of 64-byte LDS rows. gfx950 serves a 16-byte-per-lane
// LDS read 16 lanes (256 bytes) at a time; lanes reading 16 consecutive rows
// at one logical chunk land in 16 distinct 16-byte bank groups with this
// permutation (measured: as fast as contiguous reads; (row >> 1) & 3 is ~20%
// slower, no permutation ~2.3x slower).
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

// Wait until at most n (< 64) vector-memory operations of this wave are
// outstanding; encodes vmcnt with expcnt and lgkmcnt left at their maxima.
template <int n>
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// threadIdx.x through an empty asm statement: values derived from it are
// recomputed at each call instead of being hoisted out of a loop over tiles
// and kept live across the K loop (per-lane offsets, 16+ registers).
__device__ __forceinline__ uint32_t opaque_tid() {
  uint32_t tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  return tid;
}

// Per-lane byte offsets (32-bit, from the tile's wave-uniform base pointers)
// of the global chunks this lane moves into LDS, for k0 = 0.
struct Lanes {
  uint32_t a[4], b[4];
};

// The row strides pass through an empty asm statement so that, in a loop
// over tiles, the compiler recomputes these offsets per tile instead of
// hoisting them (and keeping them live across the K loop).
__device__ __forceinline__ Lanes lane_offsets(const Tile& t) {
  const uint32_t tid = opaque_tid();
  const int lane = tid & 63, w = tid >> 6;
  uint32_t lda = (uint32_t)t.lda, ldb = (uint32_t)t.ldb;
  asm volatile("" : "+s"(lda), "+s"(ldb));
  Lanes o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (w * 4 + i) * 16 + (lane >> 2);  // 16 rows per wave-wide load
    const int c = (lane & 3) ^ swz(row);             // the chunk this lane's slot holds
    const int ra = row < t.rows ? row : t.rows - 1;
    o.a[i] = (uint32_t)ra * lda * 2u + (uint32_t)c * 16u;
    o.b[i] = (uint32_t)row * ldb * 2u + (uint32_t)c * 16u;
  }
  return o;
}

// Issue half h (0 or 1) of the direct-to-LDS loads of K columns [k0, k0 + 32)
// into one stage: loads 2h and 2h + 1 of A and of B^T (4 vector-memory
// operations per lane). kAuxA: cache-policy bits of the A loads (e.g. sc0,
// served past the CU's L1, when A was written by other CUs of the launch).
template <int kAuxA>
__device__ __forceinline__ void issue_half(const Tile& t, const Lanes& o, int k0, unsigned char* stage, int h) {
  const int w = threadIdx.x >> 6;
  const unsigned char* A = reinterpret_cast<const unsigned char*>(t.A) + (uint32_t)k0 * 2u;
  const unsigned char* B = reinterpret_cast<const unsigned char*>(t.Bt) + (uint32_t)k0 * 2u;
#pragma unroll
  for (int ii = 0; ii < 2; ++ii) {
    const int i = 2 * h + ii, group = w * 4 + i;
    __builtin_amdgcn_global_load_lds(A + o.a[i], (lds_ptr)(stage + group * 1024), 16, 0, kAuxA);
    __builtin_amdgcn_global_load_lds(B + o.b[i], (lds_ptr)(stage + kHalf + group * 1024), 16, 0, 0);
  }
}

// A workgroup barrier that the compiler may not move memory accesses across
// and that adds no wait of its own (the vector-memory waits are explicit).
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Byte offsets of this lane's fragment rows inside an operand block.
struct Frag {
  int a_row[4], a_sw[4], b_row[4], b_sw[4];
};

__device__ __forceinline__ Frag frag_offsets() {
  const uint32_t tid = opaque_tid();
  const int lane = tid & 63, w = tid >> 6;
  const int wm = (w >> 1) * 128, wn = (w & 1) * 128;
  Frag f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = wm + i * 32 + (lane & 31), rb = wn + i * 32 + (lane & 31);
    f.a_row[i] = ra * 64;
    f.a_sw[i] = swz(ra);
    f.b_row[i] = rb * 64;
    f.b_sw[i] = swz(rb);
  }
  return f;
}

// Read the 8 fragments (4 of A, 4 of B^T) of k-step kk of a stage.
__device__ __forceinline__ void read_frags(const unsigned char* stage, const Frag& f, int kk, bf16x8 (&a)[4],
                                           bf16x8 (&b)[4]) {
  const int c = 2 * kk + ((threadIdx.x & 63) >> 5);
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8*>(stage + f.a_row[i] + ((c ^ f.a_sw[i]) << 4));
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const bf16x8*>(stage + kHalf + f.b_row[j] + ((c ^ f.b_sw[j]) << 4));
}

// 16 MFMAs of one k-step.
__device__ __forceinline__ void mfma_step(const bf16x8 (&a)[4], const bf16x8 (&b)[4], f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
}

// Instruction order inside one half stage: the 8 fragment reads (of the next
// half) each follow an MFMA, so their latency hides under the matrix core;
// with kLoads, the 4 loads of a half ring stage sit between the remaining 8
// MFMAs. Scheduling-group masks: 0x008 MFMA, 0x100 LDS read, 0x020
// vector-memory read.
template <bool kLoads>
__device__ __forceinline__ void schedule_half() {
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  if (kLoads) {
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  } else {
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  }
  __builtin_amdgcn_sched_barrier(0);  // nothing crosses into the next half
}

__device__ __forceinline__ unsigned char* ring_slot(unsigned char* lds, int stage) {
  return lds + (stage % kStages) * kStageBytes;
}

// One stage ks of the K loop. On entry a0/b0 hold its first k-step's
// fragments; on exit they hold the first k-step's fragments of stage ks + 1.
// Stage j is loaded in two halves: the first during the second half of stage
// j - 3 (into the slot the barrier there freed), the second during the first
// half of stage j - 2. kLoadB / kLoadA: issue the second half of stage
// ks + 2 / the first half of stage ks + 3. kWait: vector-memory operations
// allowed in flight once stage ks + 1 has landed (those issued after it: the
// two halves of stage ks + 2, 8 operations, while there is one).
template <bool kLoadB, bool kLoadA, int kWait, int kAuxA>
__device__ __forceinline__ void k_stage(const Tile& t, const Lanes& o, const Frag& f, unsigned char* lds, int ks,
                                        bf16x8 (&a0)[4], bf16x8 (&b0)[4], bf16x8 (&a1)[4], bf16x8 (&b1)[4],
                                        f32x16 (&acc)[4][4]) {
  read_frags(ring_slot(lds, ks), f, 1, a1, b1);
  // loads after the reads in program order: the compiler keeps LDS-writing
  // loads behind earlier LDS reads (these go to another slot)
  if (kLoadB) issue_half<kAuxA>(t, o, (ks + kStages - 2) * BK, ring_slot(lds, ks + kStages - 2), 1);
  mfma_step(a0, b0, acc);
  schedule_half<kLoadB>();
  wait_vmem<kWait>();
  ring_barrier();  // every wave: stage ks+1 visible, done reading stage ks-1
  __builtin_amdgcn_sched_barrier(0);
  // (on the last stage this reads a stale slot, harmlessly: the reads stay
  // unconditional so that the counter waits stay exact)
  read_frags(ring_slot(lds, ks + 1), f, 0, a0, b0);
  if (kLoadA) issue_half<kAuxA>(t, o, (ks + kStages - 1) * BK, ring_slot(lds, ks + kStages - 1), 0);
  mfma_step(a1, b1, acc);
  schedule_half<kLoadA>();
}

// The loads of the first stages of a tile (stages 0 and 1, the first half of
// stage 2): issued ahead, e.g. while the previous tile's epilogue runs, once
// every wave has finished reading the ring. tile_finish must follow with the
// same tile (and the same kAuxA).
template <int kAuxA = 0>
__device__ __forceinline__ void tile_start(const Tile& t, unsigned char* lds) {
  const Lanes o = lane_offsets(t);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    issue_half<kAuxA>(t, o, s * BK, ring_slot(lds, s), 0);
    issue_half<kAuxA>(t, o, s * BK, ring_slot(lds, s), 1);
  }
  issue_half<kAuxA>(t, o, 2 * BK, ring_slot(lds, 2), 0);
}

// tile_start predicated on `live` without a branch: the same loads through
// buffer resources whose size is zero when !live, so that every one is out of
// range and returns without touching memory (the ring then holds junk, which
// the caller discards after waiting for it). Used where the next tile is
// started speculatively right before an epilogue: a conditional tile_start
// there makes the compiler move the accumulators out before the branch.
template <int kAuxA = 0>
__device__ __forceinline__ void tile_start_if(const Tile& t, unsigned char* lds, bool live) {
  const Lanes o = lane_offsets(t);
  const int w = threadIdx.x >> 6;
  const int n = live ? 0x7FFFFFFF : 0;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)t.A, (short)0, n, kBufWord3);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void*)t.Bt, (short)0, n, kBufWord3);
#pragma unroll
  for (int s = 0; s < 3; ++s)
#pragma unroll
    for (int h = 0; h < (s < 2 ? 2 : 1); ++h)
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * h + ii, group = w * 4 + i;
        unsigned char* stage = ring_slot(lds, s);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr)(stage + group * 1024), 16, o.a[i] + s * BK * 2, 0, 0,
                                                 kAuxA);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr)(stage + kHalf + group * 1024), 16, o.b[i] + s * BK * 2, 0, 0, 0);
      }
}

// Stage kHookStage of the K loop with a hook: if hook.active() (uniform),
// every wave waits for all of its vector-memory operations (so stores issued
// before the loop are complete), and after the barrier `hook()` runs (e.g.
// thread 0 publishes an earlier tile).
template <int kWait, int kAuxA, typename Hook>
__device__ __forceinline__ void k_stage_hook(const Tile& t, const Lanes& o, const Frag& f, unsigned char* lds, int ks,
                                             bf16x8 (&a0)[4], bf16x8 (&b0)[4], bf16x8 (&a1)[4], bf16x8 (&b1)[4],
                                             f32x16 (&acc)[4][4], Hook& hook) {
  read_frags(ring_slot(lds, ks), f, 1, a1, b1);
  issue_half<kAuxA>(t, o, (ks + kStages - 2) * BK, ring_slot(lds, ks + kStages - 2), 1);
  mfma_step(a0, b0, acc);
  schedule_half<true>();
  if (hook.active())
    wait_vmem<0>();
  else
    wait_vmem<kWait>();
  ring_barrier();
  __builtin_amdgcn_sched_barrier(0);
  hook();
  __builtin_amdgcn_sched_barrier(0);
  read_frags(ring_slot(lds, ks + 1), f, 0, a0, b0);
  issue_half<kAuxA>(t, o, (ks + kStages - 1) * BK, ring_slot(lds, ks + kStages - 1), 0);
  mfma_step(a1, b1, acc);
  schedule_half<true>();
}

struct NoHook {
  __device__ bool active() const { return false; }
  __device__ void operator()() const {}
};
constexpr int kHookStage = 2;

// The K loop of a tile whose first stages tile_start issued; K / BK must be
// at least kStages + kHookStage (every caller has K >= 256, i.e. 8 stages).
// `lds` holds kLdsBytes. Vector-memory operations issued between the two
// calls (epilogue stores) are allowed: loads complete in order among
// themselves, so each wait still covers the stage it names, and at worst it
// also waits for those stores. `hook` runs once, after the barrier of stage
// kHookStage; when hook.active(), every earlier vector-memory operation of
// every wave is complete by then. On return every wave has finished reading
// LDS and every load has landed.
template <int kAuxA = 0, typename Hook>
__device__ __forceinline__ void tile_finish(const Tile& t, unsigned char* lds, f32x16 (&acc)[4][4], Hook& hook) {
  constexpr int S = kStages, W = 8;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  const Frag f = frag_offsets();
  const Lanes o = lane_offsets(t);
  const int nk = t.K / BK;
  wait_vmem<12>();  // stage 0 landed: stage 1 and half of stage 2 (4 operations per half) may be in flight
  ring_barrier();
  bf16x8 a0[4], b0[4], a1[4], b1[4];
  read_frags(lds, f, 0, a0, b0);
  int ks = 0;
  for (; ks < kHookStage; ++ks) k_stage<true, true, W, kAuxA>(t, o, f, lds, ks, a0, b0, a1, b1, acc);
  k_stage_hook<W, kAuxA>(t, o, f, lds, ks++, a0, b0, a1, b1, acc, hook);
  for (; ks < nk - S + 1; ++ks) k_stage<true, true, W, kAuxA>(t, o, f, lds, ks, a0, b0, a1, b1, acc);
  k_stage<true, false, W, kAuxA>(t, o, f, lds, ks++, a0, b0, a1, b1, acc);  // issues the last half (stage nk-1)
  k_stage<false, false, 0, kAuxA>(t, o, f, lds, ks++, a0, b0, a1, b1, acc);
  k_stage<false, false, 0, kAuxA>(t, o, f, lds, ks, a0, b0, a1, b1, acc);
  ring_barrier();
}

__device__ __forceinline__ void tile_finish(const Tile& t, unsigned char* lds, f32x16 (&acc)[4][4]) {
  NoHook none;
  tile_finish(t, lds, acc, none);
}

__device__ __forceinline__ void tile_mma(const Tile& t, unsigned char* lds, f32x16 (&acc)[4][4]) {
  tile_start(t, lds);
  tile_finish(t, lds, acc);
}

// GELU(z) = z Phi(z). With h(a) = erfc(a / sqrt 2) / 2 for a = |z|, z Phi(z)
// is z (1 - h) for z >= 0 and z h for z < 0, i.e. max(z, 0) - |z| h: no
// select. h is evaluated as t 2^(P(t) - a^2 log2(e) / 2) with t = 1 / (1 + p a)
// (the form t exp(-x^2 + poly(t)) of Numerical Recipes' erfcc, section 6.2):
// the Gaussian factor is exact, and P, a degree-4 polynomial fitted minimax
// to log2(h / t) + a^2 log2(e) / 2 over a in [0, 16] (csrc/gelu_fit.py), makes
// the error RELATIVE: |h~ / h - 1| <= 3.9e-5 over the whole tail, and
// |GELU~(z) / GELU(z) - 1| <= 5.1e-5 for z in [-12, 12] in fp32 evaluation,
// below half a bf16 unit (2^-9), so the bf16 output is the correctly rounded
// one or its neighbour. 10 VALU + 2 transcendental instructions per element.
__device__ __forceinline__ float gelu(float z) {
  constexpr float kP = 0.2630000114440918f;
  constexpr float kC4 = -0.5329483f, kC3 = 0.994698f, kC2 = 0.28043312f, kC1 = 1.516207f, kC0 = -3.2584422f;
  const float a = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(kP, a, 1.0f));
  float q = fmaf(kC4, t, kC3);
  q = fmaf(q, t, kC2);
  q = fmaf(q, t, kC1);
  q = fmaf(q, t, kC0);
  const float e = __builtin_amdgcn_exp2f(fmaf(z * z, -0.72134752044448170f, q));  // -log2(e) / 2
  return fmaf(-a, t * e, fmaxf(z, 0.0f));
}

constexpr int kLdsTotal = kLdsBytes;  // the epilogue needs no LDS

// Store the tile as bf16 (round to nearest even), optionally through GELU,
// straight from the accumulators; rows >= `rows` are not stored. Block (i, j)
// holds C^T: register 4q + e of lane l is output row wm + 32 i + l % 32,
// column wn + 32 j + 8 q + 4 (l / 32) + e. For each pair of quads (2p, 2p+1)
// one v_permlane32_swap per packed dword hands lane l + 32's half of quad 2p
// to lane l and lane l's half of quad 2p + 1 to lane l + 32, so that lane l
// holds columns 16 p + [0, 8) and lane l + 32 columns 16 p + [8, 16) of the
// row: one 16-byte store each, 32 contiguous bytes per row and instruction.

template <bool kGelu>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[4][4], __bf16* out, int64_t ldo, int rows) {
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
  typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  const uint32_t tid = opaque_tid();
  const int lane = tid & 63, w = tid >> 6;
  const int wm = (w >> 1) * 128, wn = (w & 1) * 128;
  unsigned char* base = reinterpret_cast<unsigned char*>(out);
  uint32_t ld = (uint32_t)ldo;  // opaque per call, as in lane_offsets
  asm volatile("" : "+s"(ld));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wm + 32 * i + (lane & 31);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        bf16x4 v0, v1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = acc[i][j][8 * p + e], x1 = acc[i][j][8 * p + 4 + e];
          v0[e] = (__bf16)(kGelu ? gelu(x0) : x0);
          v1[e] = (__bf16)(kGelu ? gelu(x1) : x1);
        }
        const u32x2 d0 = __builtin_bit_cast(u32x2, v0), d1 = __builtin_bit_cast(u32x2, v1);
        // lanes 32..63 of the first operand trade places with lanes 0..31 of the second
        const auto lo = __builtin_amdgcn_permlane32_swap(d0.x, d1.x, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap(d0.y, d1.y, false, false);
        const u32x4 v = {lo[0], hi[0], lo[1], hi[1]};
        const int col = wn + 32 * j + 16 * p + 8 * (lane >> 5);
        if (row < rows)
          *reinterpret_cast<u32x4*>(base + ((uint32_t)row * ld + (uint32_t)col) * 2u) = v;
      }
  }
}

// Every wave's global stores have completed (vmcnt = 0) before the caller's
// barrier, so that one thread's publish afterwards covers the workgroup's
// output.
__device__ __forceinline__ void wait_stores() { wait_vmem<0>(); }

}  // namespace mm
}  // namespace pw
