// Activation pre-pass: xh = Had128((x * s_in) * rin) along the input features ("radiance_escha.py",
// module docstring: rin is a pre-scale applied before its Hadamard; "vLLM PR #190", commit message:
// input sign flip + Hadamard-128), then either
//   * fp16 (the GEMM operand; "vllm-quantpack 0.1.0", `Exl3LinearMethod._forward` casts to fp16), or
//   * per-row 8-bit codes with a float32 scale ("radiance_escha.py", `escha_linear_into` stages a
//     uint8 [M, IC] buffer and a float32 [M] scale): sc = max|xh| / 127, q = clamp(rne(xh / sc), +-127).
// Layouts: natural row-major [M, IC] (exl3_rotate_activations), or the GEMM's fragment-major layout
// (PERM16 order inside every 16-feature group, then 1 KB per 16-row x 32-position MFMA A operand:
// row block rb, 64-position step s and half h hold lane (n, g) = row 16 rb + n, positions
// 64 s + 16 g + 8 h .. +8), with the rows up to the next multiple of 16 written as zeros.
#include "exl3_device.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

// Index (in halves) of PERM16 position P of row m in the fragment-major layout.
__device__ __forceinline__ int64_t frag_index(int64_t m, int64_t P, int64_t IC) {
  const int w = int(P & 63);
  return ((m >> 4) * (IC >> 6) + (P >> 6)) * 1024 + ((w >> 3) & 1) * 512 + (16 * (w >> 4) + int(m & 15)) * 8 + (w & 7);
}

// Transform one 128-block.  Natural order: lane l holds features 2l, 2l+1.  PERMUTED order: lane l holds
// features perm_pair_feature(l) and +8, which the PERM16 layout stores at positions 2l, 2l+1.
template <bool PERMUTED>
__device__ __forceinline__ void rotate_block(const uint16_t* __restrict__ x, const uint16_t* __restrict__ s_in,
                                             const uint16_t* __restrict__ rin, int64_t k0, int lane,
                                             float& v0, float& v1) {
  if (PERMUTED) {
    const int64_t f = k0 + perm_pair_feature(lane);
    v0 = bf16_to_f32(x[f]) * f16_to_f32(s_in[f]) * f16_to_f32(rin[f]);
    v1 = bf16_to_f32(x[f + 8]) * f16_to_f32(s_in[f + 8]) * f16_to_f32(rin[f + 8]);
  } else {
    const int64_t k = k0 + 2 * lane;
    const uint32_t xb = *reinterpret_cast<const uint32_t*>(x + k);
    const uint32_t sb = *reinterpret_cast<const uint32_t*>(s_in + k);
    const uint32_t rb = *reinterpret_cast<const uint32_t*>(rin + k);
    v0 = bf16_to_f32(xb & 0xFFFFu) * f16_to_f32(sb & 0xFFFFu) * f16_to_f32(rb & 0xFFFFu);
    v1 = bf16_to_f32(xb >> 16) * f16_to_f32(sb >> 16) * f16_to_f32(rb >> 16);
  }
  had128_wave(v0, v1, lane);
  v0 *= kInvSqrt128;
  v1 *= kInvSqrt128;
}

// One wave per 8 rows of one 128-block: the block's s_in / rin are loaded once, every input load is
// issued before any arithmetic (the kernel is latency-bound otherwise), and each row's result is one
// coalesced 256-byte store.  Rows M .. M_pad-1 are padding and are written as zeros (the decode-phase
// kernel reads whole 16-row blocks).
constexpr int kPrepassRows = 8;

template <bool PERMUTED>
__global__ __launch_bounds__(256) void prepass_f16_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ s_in,
                                                          const uint16_t* __restrict__ rin,
                                                          uint16_t* __restrict__ xh, int64_t M, int64_t M_pad,
                                                          int64_t IC) {
  const int lane = threadIdx.x & 63;
  const int64_t nblk = IC / kHad;
  const int64_t unit = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);   // (row group, block) pairs
  const int64_t ngroups = (M_pad + kPrepassRows - 1) / kPrepassRows;
  if (unit >= ngroups * nblk) return;
  const int64_t m0 = (unit / nblk) * kPrepassRows, q = unit % nblk;
  const int64_t k0 = q * kHad;
  // this lane's two features: natural (2l, 2l+1) or PERM16 pair (f, f+8) stored at (2l, 2l+1)
  const int64_t f0 = PERMUTED ? k0 + perm_pair_feature(lane) : k0 + 2 * lane;
  const int64_t f1 = PERMUTED ? f0 + 8 : f0 + 1;
  const float si0 = f16_to_f32(s_in[f0]), ri0 = f16_to_f32(rin[f0]);
  const float si1 = f16_to_f32(s_in[f1]), ri1 = f16_to_f32(rin[f1]);
  uint32_t xv[kPrepassRows];
#pragma unroll
  for (int r = 0; r < kPrepassRows; ++r) {
    const int64_t m = m0 + r < M ? m0 + r : M - 1;
    xv[r] = uint32_t(x[m * IC + f0]) | (uint32_t(x[m * IC + f1]) << 16);
  }
#pragma unroll
  for (int r = 0; r < kPrepassRows; ++r) {
    const int64_t m = m0 + r;
    if (m >= M_pad) break;
    uint32_t packed = 0u;
    if (m < M) {
      // (x * s_in) * rin, in the order the layer defines
      float v0 = bf16_to_f32(xv[r] & 0xFFFFu) * si0 * ri0;
      float v1 = bf16_to_f32(xv[r] >> 16) * si1 * ri1;
      had128_wave(v0, v1, lane);
      packed = uint32_t(f32_to_f16(v0 * kInvSqrt128)) | (uint32_t(f32_to_f16(v1 * kInvSqrt128)) << 16);
    }
    const int64_t at = PERMUTED ? frag_index(m, k0 + 2 * lane, IC) : m * IC + k0 + 2 * lane;
    *reinterpret_cast<uint32_t*>(xh + at) = packed;
  }
}

// 8-bit variant ("radiance_escha.py", `escha_linear_into`: an 8-bit activation buffer plus one float
// scale per row).  Two passes over the row: the first finds max |xh| over the row, the second recomputes
// the same fp32 features (identical instruction sequence, so identical values) and quantises them:
// sc = amax / 127, q = clamp(rne(xh / sc), -127, 127), and q = 0 for a row whose amax is 0.
// F16OUT writes each code as the fp16 number q (exact: |q| <= 127), which the fp16 MFMA GEMM consumes;
// otherwise the codes are written as int8.
template <bool PERMUTED, bool F16OUT>
__global__ __launch_bounds__(256) void prepass_i8_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ s_in,
                                                         const uint16_t* __restrict__ rin,
                                                         void* __restrict__ q_out, float* __restrict__ scale,
                                                         int64_t M, int64_t IC) {
  __shared__ float red[4];
  const int64_t m = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (m >= M) {                                        // padding row of the fragment-major layout: zeros
    if constexpr (F16OUT && PERMUTED) {
      for (int64_t q = wave; q < IC / kHad; q += 4)
        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(q_out) + frag_index(m, q * kHad + 2 * lane, IC)) = 0u;
    }
    return;
  }
  const uint16_t* xr = x + m * IC;
  float amax = 0.f;
  for (int64_t q = wave; q < IC / kHad; q += 4) {
    float v0, v1;
    rotate_block<PERMUTED>(xr, s_in, rin, q * kHad, lane, v0, v1);
    amax = fmaxf(amax, fmaxf(fabsf(v0), fabsf(v1)));
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
  if (lane == 0) red[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = __fdiv_rn(amax, 127.0f);
  if (threadIdx.x == 0) scale[m] = sc;
  for (int64_t q = wave; q < IC / kHad; q += 4) {
    float v0, v1;
    rotate_block<PERMUTED>(xr, s_in, rin, q * kHad, lane, v0, v1);
    int q0 = 0, q1 = 0;
    if (sc > 0.f) {
      q0 = (int)fminf(fmaxf(rintf(__fdiv_rn(v0, sc)), -127.f), 127.f);
      q1 = (int)fminf(fmaxf(rintf(__fdiv_rn(v1, sc)), -127.f), 127.f);
    }
    const int64_t k = q * kHad + 2 * lane;             // natural: features k, k+1; permuted: positions k, k+1
    if constexpr (F16OUT) {
      uint16_t* dst = static_cast<uint16_t*>(q_out) + (PERMUTED ? frag_index(m, k, IC) : m * IC + k);
      *reinterpret_cast<uint32_t*>(dst) = uint32_t(f32_to_f16(float(q0))) | (uint32_t(f32_to_f16(float(q1))) << 16);
    } else {
      int8_t* dst = static_cast<int8_t*>(q_out) + m * IC;
      *reinterpret_cast<uint16_t*>(dst + k) = uint16_t(uint8_t(q0)) | uint16_t(uint16_t(uint8_t(q1)) << 8);
    }
  }
}

hipError_t launch_prepass_f16(const void* x, const void* s_in, const void* rin, void* xh, int64_t M, int64_t IC,
                              bool permuted, hipStream_t stream, int64_t M_pad) {
  if (M <= 0) return hipSuccess;
  const int64_t rows = M_pad > M ? M_pad : M;
  const int64_t units = (rows + kPrepassRows - 1) / kPrepassRows * (IC / kHad);
  dim3 grid((unsigned)((units + 3) / 4)), block(256);
  if (permuted)
    hipLaunchKernelGGL(prepass_f16_kernel<true>, grid, block, 0, stream, (const uint16_t*)x, (const uint16_t*)s_in,
                       (const uint16_t*)rin, (uint16_t*)xh, M, rows, IC);
  else
    hipLaunchKernelGGL(prepass_f16_kernel<false>, grid, block, 0, stream, (const uint16_t*)x, (const uint16_t*)s_in,
                       (const uint16_t*)rin, (uint16_t*)xh, M, rows, IC);
  return hipGetLastError();
}

hipError_t launch_prepass_i8(const void* x, const void* s_in, const void* rin, void* q, float* scale, int64_t M,
                             int64_t IC, bool permuted, hipStream_t stream, bool f16_codes) {
  if (M <= 0) return hipSuccess;
  // the fragment-major layout (permuted fp16 codes) also gets its padding rows
  const int64_t rows = permuted && f16_codes ? (M + 15) / 16 * 16 : M;
  dim3 grid((unsigned)rows), block(256);
  const uint16_t *xx = (const uint16_t*)x, *si = (const uint16_t*)s_in, *ri = (const uint16_t*)rin;
  if (permuted && f16_codes)
    hipLaunchKernelGGL((prepass_i8_kernel<true, true>), grid, block, 0, stream, xx, si, ri, q, scale, M, IC);
  else if (permuted)
    hipLaunchKernelGGL((prepass_i8_kernel<true, false>), grid, block, 0, stream, xx, si, ri, q, scale, M, IC);
  else if (f16_codes)
    hipLaunchKernelGGL((prepass_i8_kernel<false, true>), grid, block, 0, stream, xx, si, ri, q, scale, M, IC);
  else
    hipLaunchKernelGGL((prepass_i8_kernel<false, false>), grid, block, 0, stream, xx, si, ri, q, scale, M, IC);
  return hipGetLastError();
}

}  // namespace exl3
