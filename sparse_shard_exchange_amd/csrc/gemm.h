// bf16 MFMA GEMM tile core for gfx950: C[256 x 256] (fp32) = A[256 x K] . B[K x 256].
//
// A is row-major [rows][K] (activations, K contiguous); B is row-major [K][N]
// (weights stored [in][out], N contiguous). One workgroup of 4 waves owns a
// 256 x 256 output tile; wave w computes the 128 x 128 quadrant
// (w >> 1, w & 1) as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16.
//
// K advances 64 at a time through double-buffered LDS (2 x 64 KiB). A goes
// to LDS as [row][k]; B is transposed on the way in (each thread turns an
// 8 x 8 block of bf16 around in registers) to [n][k], so both MFMA operands
// are single 16-byte LDS reads: lane l reads row (l % 32) at k-chunk l / 32.
// The 16-byte chunks of every 128-byte LDS row are XOR-swizzled with
// (row ^ row >> 3) & 7, which keeps the row-wise reads of the MFMA operands
// and the transposed writes of B free of bank conflicts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pw {
namespace mm {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int BM = 256, BN = 256, BK = 64, NT = 256;
constexpr int kTileBytes = BM * BK * 2;            // one operand tile, 32 KiB
constexpr int kLdsBytes = 2 * 2 * kTileBytes;      // A and B, double buffered: 128 KiB

struct Tile {
  const __bf16* A;  // first row of the tile, column 0
  int64_t lda;
  int rows;         // valid rows (<= BM); the rest read as zero and are not stored
  const __bf16* B;  // row 0, first column of the tile
  int64_t ldb;
  int K;            // multiple of BK
};

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) { return (row * 8 + (chunk ^ swz(row))) * 16; }

struct Stage {
  u32x4 a[8];
  u32x4 b[8];
};

// Global -> registers for k columns [k0, k0 + 64). Addresses are 32-bit byte
// offsets from the tile's (wave-uniform) base pointers.
__device__ __forceinline__ void load_stage(const Tile& t, int k0, Stage& s) {
  const int tid = threadIdx.x;
  const unsigned char* A = reinterpret_cast<const unsigned char*>(t.A);
  const unsigned char* B = reinterpret_cast<const unsigned char*>(t.B);
  const uint32_t lda2 = (uint32_t)t.lda * 2u, ldb2 = (uint32_t)t.ldb * 2u;
  const uint32_t ch = tid & 7, row0 = tid >> 3;
  const uint32_t a_off = row0 * lda2 + (uint32_t)(k0 + ch * 8) * 2u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t row = row0 + i * (NT / 8);
    if ((int)row < t.rows)
      s.a[i] = *reinterpret_cast<const u32x4*>(A + a_off + (uint32_t)i * (NT / 8) * lda2);
    else
      s.a[i] = u32x4{0u, 0u, 0u, 0u};
  }
  const uint32_t nb = tid & 31, kg = tid >> 5;
  const uint32_t b_off = (uint32_t)(k0 + kg * 8) * ldb2 + nb * 16u;
#pragma unroll
  for (int r = 0; r < 8; ++r) s.b[r] = *reinterpret_cast<const u32x4*>(B + b_off + (uint32_t)r * ldb2);
}

// Registers -> LDS; B's 8 x 8 block (rows k, columns n) is written as 8 rows n.
__device__ __forceinline__ void store_stage(unsigned char* As, unsigned char* Bs, const Stage& s) {
  const int tid = threadIdx.x;
  const int ch = tid & 7, row0 = tid >> 3;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = row0 + i * (NT / 8);
    *reinterpret_cast<u32x4*>(As + lds_off(row, ch)) = s.a[i];
  }
  const int nb = tid & 31, kg = tid >> 5;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    u32x4 w;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t lo = s.b[2 * p][j >> 1], hi = s.b[2 * p + 1][j >> 1];
      w[p] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
    *reinterpret_cast<u32x4*>(Bs + lds_off(nb * 8 + j, kg)) = w;
  }
}

// Byte offsets (chunk 0 and the row's swizzle) of this lane's 4 A and 4 B
// fragment rows; chunk c of row k is at base + ((c ^ sw) << 4).
struct Frag {
  uint32_t a_base[4], a_sw[4], b_base[4], b_sw[4];
};

__device__ __forceinline__ Frag frag_offsets() {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = (w >> 1) * 128, wn = (w & 1) * 128;
  Frag f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = wm + i * 32 + (lane & 31), rb = wn + i * 32 + (lane & 31);
    f.a_base[i] = ra * 128;
    f.a_sw[i] = swz(ra);
    f.b_base[i] = rb * 128;
    f.b_sw[i] = swz(rb);
  }
  return f;
}

__device__ __forceinline__ void compute_stage(const unsigned char* As, const unsigned char* Bs, const Frag& f,
                                              f32x16 (&acc)[4][4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const uint32_t ch = 2 * kk + (lane >> 5);
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8*>(As + f.a_base[i] + ((ch ^ f.a_sw[i]) << 4));
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const bf16x8*>(Bs + f.b_base[j] + ((ch ^ f.b_sw[j]) << 4));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// The whole K loop of one tile. `lds` holds kLdsBytes.
__device__ __forceinline__ void tile_mma(const Tile& t, unsigned char* lds, f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  unsigned char* As[2] = {lds, lds + 2 * kTileBytes};
  unsigned char* Bs[2] = {lds + kTileBytes, lds + 3 * kTileBytes};
  Stage st;
  const Frag f = frag_offsets();
  const int nk = t.K / BK;
  load_stage(t, 0, st);
  store_stage(As[0], Bs[0], st);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < nk) load_stage(t, (ks + 1) * BK, st);
    compute_stage(As[cur], Bs[cur], f, acc);
    if (ks + 1 < nk) store_stage(As[cur ^ 1], Bs[cur ^ 1], st);
    __syncthreads();
  }
}

// Row / column (inside the tile) of accumulator register r of block (i, j).
__device__ __forceinline__ int acc_row(int i, int r) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  return (w >> 1) * 128 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}
__device__ __forceinline__ int acc_col(int j) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  return (w & 1) * 128 + j * 32 + (lane & 31);
}

// Exact GELU in fp32 with the device erff: z * Phi(z).
__device__ __forceinline__ float gelu(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

// Store the tile as bf16 (round to nearest even), optionally through GELU.
template <bool kGelu>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[4][4], __bf16* out, int64_t ldo, int rows) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = acc_row(i, r);
        if (m < rows) {
          float v = acc[i][j][r];
          if (kGelu) v = gelu(v);
          out[(int64_t)m * ldo + acc_col(j)] = (__bf16)v;
        }
      }
}

// Every wave's global stores have completed (vmcnt = 0) before the caller's
// barrier, so one thread's agent-scope release afterwards covers the
// workgroup's output.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace mm
}  // namespace pw
