// Measurement hooks (not part of the layer): what the chip actually delivers, used as secondary
// denominators next to the published peaks when the layer's kernels are reported against a roofline.
//   * probe_read_kernel:  a plain streaming read of a large buffer, 16-byte loads (4 or 8 in flight per
//     thread, optionally non-temporal), grid-stride, one XOR per block written out so the loads cannot be
//     dropped;
//   * probe_mfma_kernel:  back-to-back independent MFMAs on register operands (4 or 8 accumulators per
//     wave, so every instruction is independent of the one before): f16 16x16x32, f16 32x32x16,
//     i8 16x16x64, i8 32x32x32.
#include "exl3_device.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

// U loads of 16 bytes in flight per thread and iteration; NT: non-temporal loads (no cache allocation).
template <int U, bool NT>
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
  uint32_t acc = 0u;
  const int64_t stride = int64_t(gridDim.x) * 256;
  int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = src[i];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0u;
    for (int j = 0; j < 256; ++j) t ^= red[j];
    sink[blockIdx.x] = t;
  }
}

typedef int int8v_i32x4 __attribute__((ext_vector_type(4)));

template <int KIND>
__global__ __launch_bounds__(256) void probe_mfma_kernel(float* __restrict__ sink, int iters, float seed) {
  const int lane = threadIdx.x & 63;
  const _Float16 h = (_Float16)(seed * float(lane + 1));
  half8 a = {h, h, h, h, h, h, h, h};
  half8 b = a;
  if constexpr (KIND == 0) {                          // f16 16x16x32: 16384 FLOP each
    float4v acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = (float4v){0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    sink[blockIdx.x * 256 + threadIdx.x] = s;
  } else if constexpr (KIND == 1) {                   // f16 32x32x16: 32768 FLOP each
    float16v acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[j][r];
    sink[blockIdx.x * 256 + threadIdx.x] = s;
  } else if constexpr (KIND == 3) {                   // i8 32x32x32: 65536 OP each
    const int w = int(seed * 7.f) * (lane + 1);
    const int8v_i32x4 ai = {w, w + 1, w + 2, w + 3};
    typedef int int16v_i32 __attribute__((ext_vector_type(16)));
    int16v_i32 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][r] = 0;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ai, ai, acc[j], 0, 0, 0);
    int s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[j][r];
    sink[blockIdx.x * 256 + threadIdx.x] = float(s);
  } else {                                            // i8 16x16x64: 32768 OP each
    const int w = int(seed * 7.f) * (lane + 1);
    const int8v_i32x4 ai = {w, w + 1, w + 2, w + 3};
    int8v_i32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = (int8v_i32x4){0, 0, 0, 0};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ai, ai, acc[j], 0, 0, 0);
    int s = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    sink[blockIdx.x * 256 + threadIdx.x] = float(s);
  }
}

hipError_t launch_probe_read(const void* src, size_t bytes, uint32_t* sink, int blocks, int variant,
                             hipStream_t stream) {
  const dim3 g((unsigned)blocks), b(256);
  const u32x4* p = (const u32x4*)src;
  const int64_t n16 = int64_t(bytes / 16);
  switch (variant) {
    case 0: hipLaunchKernelGGL((probe_read_kernel<4, false>), g, b, 0, stream, p, n16, sink); break;
    case 1: hipLaunchKernelGGL((probe_read_kernel<8, false>), g, b, 0, stream, p, n16, sink); break;
    case 2: hipLaunchKernelGGL((probe_read_kernel<8, true>), g, b, 0, stream, p, n16, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_probe_mfma(float* sink, int kind, int iters, int blocks, hipStream_t stream) {
  switch (kind) {
    case 0: hipLaunchKernelGGL(probe_mfma_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, stream, sink, iters, 0.001f); break;
    case 1: hipLaunchKernelGGL(probe_mfma_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, sink, iters, 0.001f); break;
    case 2: hipLaunchKernelGGL(probe_mfma_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, stream, sink, iters, 0.001f); break;
    case 3: hipLaunchKernelGGL(probe_mfma_kernel<3>, dim3((unsigned)blocks), dim3(256), 0, stream, sink, iters, 0.001f); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace exl3
