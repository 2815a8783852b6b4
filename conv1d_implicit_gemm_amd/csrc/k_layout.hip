// Layout change of the input: a channels-last fp32 x [N, T, C] transposed
// into [N, C, T] in the workspace, for the fp32 kernels that read positions
// contiguously.  A workgroup moves a 64 (positions) x 64 (channels) block
// through LDS: the loads run along the channels of a position, the stores
// along the positions of a channel, both in whole 256-byte rows of 64 lanes.
// The LDS rows have 65 entries so that the column reads of the store phase
// fall in distinct banks.
#include "common.hpp"
#include "launch.hpp"

namespace c1g {
namespace {

__global__ __launch_bounds__(256) void transpose_nlc_f32_kernel(const float* __restrict__ x,
                                                                float* __restrict__ xt,
                                                                int64_t T, int64_t C) {
  __shared__ float tile[64][65];
  const int64_t n = blockIdx.z;
  const int64_t t0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  const int lane = threadIdx.x & 63, row = threadIdx.x >> 6;  // 4 rows per pass
  const float* src = x + n * T * C;
#pragma unroll 4
  for (int r = row; r < 64; r += 4) {
    const int64_t t = t0 + r, c = c0 + lane;
    tile[r][lane] = (t < T && c < C) ? src[t * C + c] : 0.f;
  }
  __syncthreads();
  float* dst = xt + n * C * T;
#pragma unroll 4
  for (int r = row; r < 64; r += 4) {
    const int64_t c = c0 + r, t = t0 + lane;
    if (c < C && t < T) dst[c * T + t] = tile[lane][r];
  }
}

}  // namespace

hipError_t transpose_nlc_f32(const float* x, float* xt, int64_t N, int64_t T, int64_t C,
                             hipStream_t s) {
  const int64_t gt = (T + 63) / 64, gc = (C + 63) / 64;
  if (gt > 0x7fffffffll || gc > 65535 || N > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_nlc_f32_kernel, dim3((unsigned)gt, (unsigned)gc, (unsigned)N),
                     dim3(256), 0, s, x, xt, T, C);
  return hipGetLastError();
}

}  // namespace c1g
