// Weight packing: turn row-major [K][N] weights (stored [in][out]) into
// K-contiguous B^T [N_out][K] once, when a plan is built, so the GEMM tiles
// can stream both operands straight into LDS. Columns n >= N_in are zero
// (the router pads its expert count to 64).
#include "device.h"

namespace pw {

namespace {

__global__ __launch_bounds__(256) void k_pack_t(const __bf16* in, __bf16* out, uint32_t K, uint32_t N_in,
                                                uint32_t N_out) {
  __shared__ __bf16 tile[64][66];
  const uint64_t b = blockIdx.z;
  const uint32_t k0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const __bf16* src = in + b * (uint64_t)K * N_in;
  __bf16* dst = out + b * (uint64_t)N_out * K;
  for (uint32_t i = threadIdx.x; i < 64 * 64; i += 256) {
    const uint32_t r = i >> 6, c = i & 63;  // r: k, c: n
    const uint32_t k = k0 + r, n = n0 + c;
    tile[r][c] = (k < K && n < N_in) ? src[(uint64_t)k * N_in + n] : (__bf16)0.0f;
  }
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < 64 * 64; i += 256) {
    const uint32_t r = i >> 6, c = i & 63;  // r: n, c: k
    const uint32_t n = n0 + r, k = k0 + c;
    if (n < N_out && k < K) dst[(uint64_t)n * K + k] = tile[c][r];
  }
}

}  // namespace

hipError_t launch_pack_t(const __bf16* in, __bf16* out, uint32_t batch, uint32_t K, uint32_t N_in, uint32_t N_out,
                         hipStream_t s) {
  const dim3 grid((N_out + 63) / 64, (K + 63) / 64, batch);
  hipLaunchKernelGGL(k_pack_t, grid, dim3(256), 0, s, in, out, K, N_in, N_out);
  return hipGetLastError();
}

}  // namespace pw
