// The dense MLP block's activation value, shared by the activation kernel and the pre-pass that folds it
// into down's input rotation, so both take the same fp32 steps and the same bf16 rounding.
#pragma once
#include "exl3_device.hpp"

namespace exl3 {

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

// bf16(silu(g) * u) for two (g, u) pairs packed as bf16x2 words; returns the packed bf16x2 result.
__device__ __forceinline__ uint32_t silu_mul_bf16x2(uint32_t g, uint32_t u) {
  const float g0 = bf16_to_f32(g & 0xFFFFu), g1 = bf16_to_f32(g >> 16);
  const float u0 = bf16_to_f32(u & 0xFFFFu), u1 = bf16_to_f32(u >> 16);
  return f32x2_to_bf16x2(silu_f32(g0) * u0, silu_f32(g1) * u1);
}

}  // namespace exl3
