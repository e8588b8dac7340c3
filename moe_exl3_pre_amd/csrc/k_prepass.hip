// Activation pre-pass: xh = Had128((x * s_in) * rin) along the input features ("radiance_escha.py",
// module docstring: rin is a pre-scale applied before its Hadamard; "vLLM PR #190", commit message:
// input sign flip + Hadamard-128), then either
//   * fp16 (the GEMM operand; "vllm-quantpack 0.1.0", `Exl3LinearMethod._forward` casts to fp16), or
//   * per-row 8-bit codes with a float32 scale ("radiance_escha.py", `escha_linear_into` stages a
//     uint8 [M, IC] buffer and a float32 [M] scale): sc = max|xh| / 127, q = clamp(rne(xh / sc), +-127).
// One 256-thread block per row; each wave transforms whole 128-blocks, two features per lane.
#include "exl3_device.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

// Transform one 128-block: returns the normalised features 2*lane and 2*lane+1 in fp32.
__device__ __forceinline__ void rotate_block(const uint16_t* __restrict__ x, const uint16_t* __restrict__ s_in,
                                             const uint16_t* __restrict__ rin, int64_t k0, int lane,
                                             float& v0, float& v1) {
  const int64_t k = k0 + 2 * lane;
  const uint32_t xb = *reinterpret_cast<const uint32_t*>(x + k);
  const uint32_t sb = *reinterpret_cast<const uint32_t*>(s_in + k);
  const uint32_t rb = *reinterpret_cast<const uint32_t*>(rin + k);
  v0 = bf16_to_f32(xb & 0xFFFFu) * f16_to_f32(sb & 0xFFFFu) * f16_to_f32(rb & 0xFFFFu);
  v1 = bf16_to_f32(xb >> 16) * f16_to_f32(sb >> 16) * f16_to_f32(rb >> 16);
  had128_wave(v0, v1, lane);
  v0 *= kInvSqrt128;
  v1 *= kInvSqrt128;
}

// Destination index of feature k inside its 16-group for the permuted layout.
__device__ __forceinline__ int64_t dest_index(int64_t k, bool permuted) {
  return permuted ? ((k & ~int64_t(15)) | perm16_pos(int(k & 15))) : k;
}

// One wave per (row, 128-block): blockIdx.x * 4 + wave enumerates rows-major pairs.  Rows M .. M_pad-1
// are padding and are written as zeros (the decode-phase kernel reads whole 16-row blocks).
template <bool PERMUTED>
__global__ __launch_bounds__(256) void prepass_f16_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ s_in,
                                                          const uint16_t* __restrict__ rin,
                                                          uint16_t* __restrict__ xh, int64_t M, int64_t M_pad,
                                                          int64_t IC) {
  const int lane = threadIdx.x & 63;
  const int64_t nblk = IC / kHad;
  const int64_t pair = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (pair >= M_pad * nblk) return;
  const int64_t m = pair / nblk, q = pair % nblk;
  const int64_t k = q * kHad + 2 * lane;
  uint16_t* dst = xh + m * IC;
  if (m >= M) {
    *reinterpret_cast<uint32_t*>(dst + k) = 0u;
    return;
  }
  float v0, v1;
  rotate_block(x + m * IC, s_in, rin, q * kHad, lane, v0, v1);
  if (PERMUTED) {
    dst[dest_index(k, true)] = f32_to_f16(v0);
    dst[dest_index(k + 1, true)] = f32_to_f16(v1);
  } else {
    *reinterpret_cast<uint32_t*>(dst + k) = uint32_t(f32_to_f16(v0)) | (uint32_t(f32_to_f16(v1)) << 16);
  }
}

// 8-bit variant.  Two passes over the row: the first finds the amax, the second recomputes the same
// fp32 features (identical instruction sequence, so identical values) and quantises them.
template <bool PERMUTED>
__global__ __launch_bounds__(256) void prepass_i8_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ s_in,
                                                         const uint16_t* __restrict__ rin,
                                                         int8_t* __restrict__ q_out, float* __restrict__ scale,
                                                         int64_t M, int64_t IC) {
  __shared__ float red[4];
  const int64_t m = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint16_t* xr = x + m * IC;
  float amax = 0.f;
  for (int64_t q = wave; q < IC / kHad; q += 4) {
    float v0, v1;
    rotate_block(xr, s_in, rin, q * kHad, lane, v0, v1);
    amax = fmaxf(amax, fmaxf(fabsf(v0), fabsf(v1)));
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
  if (lane == 0) red[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = __fdiv_rn(amax, 127.0f);
  if (threadIdx.x == 0) scale[m] = sc;
  int8_t* dst = q_out + m * IC;
  for (int64_t q = wave; q < IC / kHad; q += 4) {
    float v0, v1;
    rotate_block(xr, s_in, rin, q * kHad, lane, v0, v1);
    int q0 = 0, q1 = 0;
    if (sc > 0.f) {
      q0 = (int)fminf(fmaxf(rintf(__fdiv_rn(v0, sc)), -127.f), 127.f);
      q1 = (int)fminf(fmaxf(rintf(__fdiv_rn(v1, sc)), -127.f), 127.f);
    }
    const int64_t k = q * kHad + 2 * lane;
    if (PERMUTED) {
      dst[dest_index(k, true)] = (int8_t)q0;
      dst[dest_index(k + 1, true)] = (int8_t)q1;
    } else {
      const uint16_t packed = uint16_t(uint8_t(q0)) | uint16_t(uint16_t(uint8_t(q1)) << 8);
      *reinterpret_cast<uint16_t*>(dst + k) = packed;
    }
  }
}

hipError_t launch_prepass_f16(const void* x, const void* s_in, const void* rin, void* xh, int64_t M, int64_t IC,
                              bool permuted, hipStream_t stream, int64_t M_pad) {
  if (M <= 0) return hipSuccess;
  const int64_t rows = M_pad > M ? M_pad : M;
  dim3 grid((unsigned)((rows * (IC / kHad) + 3) / 4)), block(256);
  if (permuted)
    hipLaunchKernelGGL(prepass_f16_kernel<true>, grid, block, 0, stream, (const uint16_t*)x, (const uint16_t*)s_in,
                       (const uint16_t*)rin, (uint16_t*)xh, M, rows, IC);
  else
    hipLaunchKernelGGL(prepass_f16_kernel<false>, grid, block, 0, stream, (const uint16_t*)x, (const uint16_t*)s_in,
                       (const uint16_t*)rin, (uint16_t*)xh, M, rows, IC);
  return hipGetLastError();
}

hipError_t launch_prepass_i8(const void* x, const void* s_in, const void* rin, void* q, float* scale, int64_t M,
                             int64_t IC, bool permuted, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  dim3 grid((unsigned)M), block(256);
  if (permuted)
    hipLaunchKernelGGL(prepass_i8_kernel<true>, grid, block, 0, stream, (const uint16_t*)x, (const uint16_t*)s_in,
                       (const uint16_t*)rin, (int8_t*)q, scale, M, IC);
  else
    hipLaunchKernelGGL(prepass_i8_kernel<false>, grid, block, 0, stream, (const uint16_t*)x, (const uint16_t*)s_in,
                       (const uint16_t*)rin, (int8_t*)q, scale, M, IC);
  return hipGetLastError();
}

}  // namespace exl3
