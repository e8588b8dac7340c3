// Dense MLP block activation ("vllm-quantpack 0.1.0", exl3/linear.py module docstring: gate and up are two
// shards of one fused gate_up layer whose outputs are concatenated; the model's activation takes
// silu(gate) * up and feeds down_proj).
//
// h[m, j] = bf16(silu(g[m, j]) * u[m, j]) with g = gu[m, j], u = gu[m, I + j] read from the bf16 gate_up
// output [M, 2I]; silu in fp32, one round-to-nearest-even to bf16.  One thread per 8 outputs (16-byte loads
// of g and u, one 16-byte store); the kernel is HBM-bound on 6 bytes per output and at decode sizes
// launch-latency-bound.
#include "exl3_device.hpp"
#include "exl3_internal.hpp"
#include "k_silu.hpp"

namespace exl3 {

namespace {

__global__ __launch_bounds__(256) void silu_mul_kernel(uint16_t* __restrict__ h, const uint16_t* __restrict__ gu,
                                                       int64_t M, int64_t I) {
  const int64_t per_row = I / 8;
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= M * per_row) return;
  const int64_t m = t / per_row, j = (t % per_row) * 8;
  const u32x4 g = *reinterpret_cast<const u32x4*>(gu + m * 2 * I + j);
  const u32x4 u = *reinterpret_cast<const u32x4*>(gu + m * 2 * I + I + j);
  *reinterpret_cast<u32x4*>(h + m * I + j) = (u32x4){silu_mul_bf16x2(g[0], u[0]), silu_mul_bf16x2(g[1], u[1]),
                                                      silu_mul_bf16x2(g[2], u[2]), silu_mul_bf16x2(g[3], u[3])};
}

}  // namespace

hipError_t launch_silu_mul(void* h, const void* gu, int64_t M, int64_t I, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const int64_t threads = M * (I / 8);
  hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     static_cast<uint16_t*>(h), static_cast<const uint16_t*>(gu), M, I);
  return hipGetLastError();
}

}  // namespace exl3
