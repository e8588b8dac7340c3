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
#include "k_silu.hpp"

namespace exl3 {

// Transform one 128-block in natural order: lane l holds features 2l, 2l+1.
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
  v0 = rot_scale(v0);
  v1 = rot_scale(v1);
}

// Natural layout.  One wave per 8 rows of one 128-block: the block's s_in / rin are loaded once, every
// input load is issued before any arithmetic (the kernel is latency-bound otherwise), and each row's
// result is one coalesced 256-byte store.  Rows M .. M_pad-1, when asked for, are written as zeros.
constexpr int kPrepassRows = 8;

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
  const int64_t f0 = k0 + 2 * lane, f1 = f0 + 1;              // this lane's two features
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
      packed = rot_f16x2(v0, v1);
    }
    *reinterpret_cast<uint32_t*>(xh + m * IC + k0 + 2 * lane) = packed;
  }
}

// The GEMM's fragment-major layout, fp16.  One wave per (16-row block, 128-feature block): lane (n, g)
// holds row n's features of the 16-groups g and g + 4 (32 values), loaded as four coalesced 16-byte
// chunks.  The Hadamard-128 then runs as register butterflies over feature bits 0..3 and 6 and as
// lane-pair exchanges (v_permlane16_swap / v_permlane32_swap) over bits 4 and 5, and the wave's output is
// exactly 4 KB of the layout (the four 1 KB fragments of its two 64-position steps), written as four
// 1 KB wave stores.  Rows past M are written as zeros.
//
// The rotated features of one (16-row block rb, 128-block q) unit, before the 1/sqrt(128) normalisation:
// lane (n, g) ends with row 16 rb + n, features 16 (g + 4t) + w of the block in v[t][w] (zeros past M).
// SILU: x is the dense MLP block's gate_up output [M, 2 IC] and the transform's input is h = bf16(silu(g) * u)
// with g = x[row, k] and u = x[row, IC + k], formed exactly as the block's activation kernel forms it.
template <bool SILU = false>
__device__ __forceinline__ void frag_transform(const uint16_t* __restrict__ x, const uint16_t* __restrict__ s_in,
                                               const uint16_t* __restrict__ rin, int64_t M, int64_t IC, int64_t rb,
                                               int64_t q, int lane, float (&v)[2][16]) {
  const int n = lane & 15, g = lane >> 4;
  const int64_t row = rb * 16 + n;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int64_t f = q * kHad + 16 * (g + 4 * t);
    u32x4 sv[2], rv[2], xv[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      sv[c] = *reinterpret_cast<const u32x4*>(s_in + f + 8 * c);
      rv[c] = *reinterpret_cast<const u32x4*>(rin + f + 8 * c);
      if constexpr (SILU) {
        if (row < M) {
          const u32x4 g = *reinterpret_cast<const u32x4*>(x + row * 2 * IC + f + 8 * c);
          const u32x4 u = *reinterpret_cast<const u32x4*>(x + row * 2 * IC + IC + f + 8 * c);
          xv[c] = (u32x4){silu_mul_bf16x2(g[0], u[0]), silu_mul_bf16x2(g[1], u[1]), silu_mul_bf16x2(g[2], u[2]),
                          silu_mul_bf16x2(g[3], u[3])};
        } else {
          xv[c] = (u32x4){0u, 0u, 0u, 0u};
        }
      } else {
        xv[c] = row < M ? *reinterpret_cast<const u32x4*>(x + row * IC + f + 8 * c) : (u32x4){0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const uint32_t xw = xv[w >> 3][(w >> 1) & 3], sw = sv[w >> 3][(w >> 1) & 3], rw = rv[w >> 3][(w >> 1) & 3];
      const int sh = (w & 1) * 16;
      // (x * s_in) * rin, in the order the layer defines
      v[t][w] = bf16_to_f32((xw >> sh) & 0xFFFFu) * f16_to_f32(uint16_t(sw >> sh)) * f16_to_f32(uint16_t(rw >> sh));
    }
  }
  // feature bits 0..3: register butterflies inside each 16-group
#pragma unroll
  for (int b = 1; b < 16; b <<= 1)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int w = 0; w < 16; ++w)
        if (!(w & b)) {
          const float lo = v[t][w], hi = v[t][w | b];
          v[t][w] = lo + hi;
          v[t][w | b] = lo - hi;
        }
  // bits 4 and 5: lane pairs (lane bit 4, lane bit 5), two values per exchange
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int w = 0; w < 16; w += 2) lane_pair_bfly<false>(v[t][w], v[t][w + 1]);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int w = 0; w < 16; w += 2) lane_pair_bfly<true>(v[t][w], v[t][w + 1]);
  // bit 6: the two groups of the lane
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const float lo = v[0][w], hi = v[1][w];
    v[0][w] = lo + hi;
    v[1][w] = lo - hi;
  }
}

// Where a 16-row unit's values go.  Fragment (step 2q + t, half h), lane (n, g) holds PERM16 positions
// 8h .. 8h+7 of 16-group g + 4t, i.e. the features (4h + j, 4h + j + 8) for j = 0..3.
//   16-row layout (the 16x16x32 MFMA's A operand): per 16-row block rb, step s, half h, 1 KB with lane
//     (n, g) = row 16 rb + n, PERM16 positions 64 s + 16 g + 8 h .. +8;
//   32-row layout (the 32x32x16 MFMA's A operand): per 32-row block, step s, pair j, half h, 1 KB with
//     lane (m, k) = row 32 rb + m (m < 32), PERM16 positions 64 s + 16 (2 j + k) + 8 h .. +8, k < 2: the
//     two halves of the wave take the same positions of two different 16-groups.
template <bool R32>
__device__ __forceinline__ uint16_t* frag_addr(uint16_t* xf, int64_t IC, int64_t rb, int64_t q, int lane, int t,
                                               int h) {
  const int64_t step = 2 * q + t;
  if constexpr (!R32) {
    return xf + ((rb * (IC / 64) + step) * 2 + h) * 512 + lane * 8;
  } else {
    const int n = lane & 15, g = lane >> 4;
    const int lp = 16 * int(rb & 1) + n + 32 * (g & 1);
    return xf + ((((rb >> 1) * (IC / 64) + step) * 2 + (g >> 1)) * 2 + h) * 512 + lp * 8;
  }
}

// 16-row units a fragment-major launch covers: rows padded to 16, or to 32 for the 32-row layout.
__host__ __device__ inline int64_t frag_row_units(int64_t M, bool r32) {
  return r32 ? (M + 31) / 32 * 2 : (M + 15) / 16;
}

template <bool SILU, bool R32>
__global__ __launch_bounds__(256) void prepass_frag_f16_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ s_in,
                                                               const uint16_t* __restrict__ rin,
                                                               uint16_t* __restrict__ xf, int64_t M, int64_t IC) {
  // All parameters in one batch of scalar loads: otherwise the pointers are requested only after the sizes
  // have come back for the early exit, a second memory round trip before the first data load.
  asm volatile("" ::"s"(x), "s"(s_in), "s"(rin), "s"(xf), "s"(M), "s"(IC));
  const int lane = threadIdx.x & 63;
  const int64_t nq = IC / kHad;
  const int64_t unit = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (unit >= frag_row_units(M, R32) * nq) return;
  const int64_t rb = unit / nq, q = unit % nq;
  float v[2][16];
  frag_transform<SILU>(x, s_in, rin, M, IC, rb, q, lane, v);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[j] = rot_f16x2(v[t][4 * h + j], v[t][4 * h + j + 8]);
      *reinterpret_cast<u32x4*>(frag_addr<R32>(xf, IC, rb, q, lane, t, h)) = o;
    }
}

// 8-bit codes in the fragment-major layout, in three launches over the same units: the per-(row, block)
// max |xh| (frag_amax), the row scale sc = max / 127 (row_scale), and the codes q = clamp(rne(xh / sc),
// +-127) written as fp16 numbers (frag_codes; q = 0 for a row whose max is 0, zeros past M).  Both unit
// kernels compute xh with the same inlined transform, so the codes are taken on the values the scale
// came from.
__global__ __launch_bounds__(256) void prepass_frag_amax_kernel(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ s_in,
                                                                const uint16_t* __restrict__ rin,
                                                                float* __restrict__ part, int64_t M, int64_t IC) {
  asm volatile("" ::"s"(x), "s"(s_in), "s"(rin), "s"(part), "s"(M), "s"(IC));   // one batch (as above)
  const int lane = threadIdx.x & 63;
  const int64_t nq = IC / kHad;
  const int64_t unit = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (unit >= (M + 15) / 16 * nq) return;
  const int64_t rb = unit / nq, q = unit % nq;
  float v[2][16];
  frag_transform(x, s_in, rin, M, IC, rb, q, lane, v);
  float a = 0.f;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int w = 0; w < 16; ++w) a = fmaxf(a, fabsf(v[t][w] * kInvSqrt128));
  a = fmaxf(a, __shfl_xor(a, 16, 64));                     // the four lanes of row n
  a = fmaxf(a, __shfl_xor(a, 32, 64));
  const int64_t row = rb * 16 + (lane & 15);
  if (lane < 16 && row < M) part[row * nq + q] = a;
}

__global__ __launch_bounds__(256) void prepass_row_scale_kernel(const float* __restrict__ part,
                                                                float* __restrict__ scale, int64_t M, int64_t nq) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  float a = 0.f;
  for (int64_t q = lane; q < nq; q += 64) a = fmaxf(a, part[row * nq + q]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) a = fmaxf(a, __shfl_xor(a, d, 64));
  if (lane == 0) scale[row] = __fdiv_rn(a, 127.0f);
}

// FOLD: the row scale is not read from `scale` but formed here from the per-(row, block) maxima in `part`
// (max over the row's blocks, then / 127, the operations of prepass_row_scale_kernel, so the same value); the
// unit of block 0 writes it to `scale`.  This saves the row-scale launch where launches dominate (a few rows).
template <bool R32, bool FOLD = false>
__global__ __launch_bounds__(256) void prepass_frag_codes_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ s_in,
                                                                 const uint16_t* __restrict__ rin,
                                                                 float* __restrict__ scale,
                                                                 const float* __restrict__ part,
                                                                 uint16_t* __restrict__ xf, int64_t M, int64_t IC) {
  asm volatile("" ::"s"(x), "s"(s_in), "s"(rin), "s"(scale), "s"(part), "s"(xf), "s"(M), "s"(IC));   // one batch
  const int lane = threadIdx.x & 63;
  const int64_t nq = IC / kHad;
  const int64_t unit = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (unit >= frag_row_units(M, R32) * nq) return;
  const int64_t rb = unit / nq, q = unit % nq;
  const int64_t row = rb * 16 + (lane & 15);
  // FOLD: the four lanes of row n take every fourth block's maximum.  The first eight loads per lane are
  // issued before the transform's own loads, so both wait out one memory latency together.
  const float* pr = part + (row < M ? row : 0) * (FOLD ? nq : 0);
  const int64_t b0 = lane >> 4;
  float pm[8];
  if constexpr (FOLD) {
#pragma unroll
    for (int k = 0; k < 8; ++k) pm[k] = b0 + 4 * k < nq ? pr[b0 + 4 * k] : 0.f;
  }
  float v[2][16];
  frag_transform(x, s_in, rin, M, IC, rb, q, lane, v);
  float sc = 0.f;
  if constexpr (FOLD) {
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, pm[k]);
    for (int64_t bb = b0 + 32; bb < nq; bb += 4) m = fmaxf(m, pr[bb]);
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    if (row < M) {
      sc = __fdiv_rn(m, 127.0f);
      if (q == 0 && lane < 16) scale[row] = sc;
    }
  } else {
    sc = row < M ? scale[row] : 0.f;
  }
  auto code = [&](float xv) -> float {
    return sc > 0.f ? fminf(fmaxf(rintf(__fdiv_rn(xv * kInvSqrt128, sc)), -127.f), 127.f) : 0.f;
  };
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = f32x2_to_f16x2(code(v[t][4 * h + j]), code(v[t][4 * h + j + 8]));
      *reinterpret_cast<u32x4*>(frag_addr<R32>(xf, IC, rb, q, lane, t, h)) = o;
    }
}

// 8-bit variant, natural layout ("radiance_escha.py", `escha_linear_into`: an 8-bit activation buffer
// plus one float scale per row).  One block per row, two passes over it: the first finds max |xh| over
// the row, the second recomputes the same fp32 features (identical instruction sequence, so identical
// values) and quantises them: sc = amax / 127, q = clamp(rne(xh / sc), -127, 127), and q = 0 for a row
// whose amax is 0.
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
  for (int64_t q = wave; q < IC / kHad; q += 4) {
    float v0, v1;
    rotate_block(xr, s_in, rin, q * kHad, lane, v0, v1);
    int q0 = 0, q1 = 0;
    if (sc > 0.f) {
      q0 = (int)fminf(fmaxf(rintf(__fdiv_rn(v0, sc)), -127.f), 127.f);
      q1 = (int)fminf(fmaxf(rintf(__fdiv_rn(v1, sc)), -127.f), 127.f);
    }
    const int64_t k = q * kHad + 2 * lane;             // features k, k + 1
    *reinterpret_cast<uint16_t*>(q_out + m * IC + k) = uint16_t(uint8_t(q0)) | uint16_t(uint16_t(uint8_t(q1)) << 8);
  }
}

hipError_t launch_prepass_f16(const void* x, const void* s_in, const void* rin, void* xh, int64_t M, int64_t IC,
                              bool permuted, hipStream_t stream, int64_t M_pad, bool rows32) {
  if (M <= 0) return hipSuccess;
  if (permuted) {                                         // fragment-major: rows padded to 16 (32) with zeros
    const int64_t units = frag_row_units(M, rows32) * (IC / kHad);
    const dim3 g((unsigned)((units + 3) / 4)), b(256);
    if (rows32)
      hipLaunchKernelGGL((prepass_frag_f16_kernel<false, true>), g, b, 0, stream, (const uint16_t*)x,
                         (const uint16_t*)s_in, (const uint16_t*)rin, (uint16_t*)xh, M, IC);
    else
      hipLaunchKernelGGL((prepass_frag_f16_kernel<false, false>), g, b, 0, stream, (const uint16_t*)x,
                         (const uint16_t*)s_in, (const uint16_t*)rin, (uint16_t*)xh, M, IC);
    return hipGetLastError();
  }
  const int64_t rows = M_pad > M ? M_pad : M;
  const int64_t units = (rows + kPrepassRows - 1) / kPrepassRows * (IC / kHad);
  dim3 grid((unsigned)((units + 3) / 4)), block(256);
  hipLaunchKernelGGL(prepass_f16_kernel, grid, block, 0, stream, (const uint16_t*)x, (const uint16_t*)s_in,
                     (const uint16_t*)rin, (uint16_t*)xh, M, rows, IC);
  return hipGetLastError();
}

// The dense MLP block's down input straight from its gate_up output gu [M, 2 IC]: h = bf16(silu(g) * u)
// formed in registers, then the fragment-major fp16 rotation of launch_prepass_f16 (16- or 32-row fragments).
hipError_t launch_prepass_silu_f16(const void* gu, const void* s_in, const void* rin, void* xh, int64_t M, int64_t IC,
                                   hipStream_t stream, bool rows32) {
  if (M <= 0) return hipSuccess;
  const int64_t units = frag_row_units(M, rows32) * (IC / kHad);
  const dim3 g((unsigned)((units + 3) / 4)), b(256);
  if (rows32)
    hipLaunchKernelGGL((prepass_frag_f16_kernel<true, true>), g, b, 0, stream, (const uint16_t*)gu,
                       (const uint16_t*)s_in, (const uint16_t*)rin, (uint16_t*)xh, M, IC);
  else
    hipLaunchKernelGGL((prepass_frag_f16_kernel<true, false>), g, b, 0, stream, (const uint16_t*)gu,
                       (const uint16_t*)s_in, (const uint16_t*)rin, (uint16_t*)xh, M, IC);
  return hipGetLastError();
}

hipError_t launch_prepass_amax(const void* x, const void* s_in, const void* rin, float* part, int64_t M, int64_t IC,
                               hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const int64_t units = (M + 15) / 16 * (IC / kHad);
  hipLaunchKernelGGL(prepass_frag_amax_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, stream,
                     (const uint16_t*)x, (const uint16_t*)s_in, (const uint16_t*)rin, part, M, IC);
  return hipGetLastError();
}

hipError_t launch_prepass_i8(const void* x, const void* s_in, const void* rin, void* q, float* scale, int64_t M,
                             int64_t IC, bool permuted, hipStream_t stream, bool f16_codes, float* part, bool rows32) {
  if (M <= 0) return hipSuccess;
  if (permuted && f16_codes) {                            // fragment-major fp16 codes (the MFMA operand)
    if (!part) return hipErrorInvalidValue;
    const int64_t units = (M + 15) / 16 * (IC / kHad);
    const dim3 ug((unsigned)((units + 3) / 4)), blk(256);
    const uint16_t *xx = (const uint16_t*)x, *si = (const uint16_t*)s_in, *ri = (const uint16_t*)rin;
    hipLaunchKernelGGL(prepass_frag_amax_kernel, ug, blk, 0, stream, xx, si, ri, part, M, IC);
    const int64_t cunits = frag_row_units(M, rows32) * (IC / kHad);
    const dim3 cg((unsigned)((cunits + 3) / 4));
    if (rows32) {                                         // the prefill GEMM's operand: many rows, a scale launch
      hipLaunchKernelGGL(prepass_row_scale_kernel, dim3((unsigned)((M + 3) / 4)), blk, 0, stream, (const float*)part,
                         scale, M, IC / kHad);
      hipLaunchKernelGGL((prepass_frag_codes_kernel<true>), cg, blk, 0, stream, xx, si, ri, scale, (const float*)part,
                         (uint16_t*)q, M, IC);
    } else {                                              // the decode-phase operand (<= 32 rows): scales folded in
      hipLaunchKernelGGL((prepass_frag_codes_kernel<false, true>), cg, blk, 0, stream, xx, si, ri, scale,
                         (const float*)part, (uint16_t*)q, M, IC);
    }
    return hipGetLastError();
  }
  if (permuted || f16_codes) return hipErrorInvalidValue;  // natural layout: int8 codes only
  hipLaunchKernelGGL(prepass_i8_kernel, dim3((unsigned)M), dim3(256), 0, stream, (const uint16_t*)x,
                     (const uint16_t*)s_in, (const uint16_t*)rin, (int8_t*)q, scale, M, IC);
  return hipGetLastError();
}

}  // namespace exl3
