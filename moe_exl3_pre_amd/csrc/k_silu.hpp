// The dense MLP block's activation value, shared by the activation kernel and the pre-pass that folds it
// into down's input rotation, so both take the same fp32 steps and the same bf16 rounding.
#pragma once
#include "exl3_device.hpp"

namespace exl3 {

// silu(g) = g / (1 + e^-g), written with t = e^-|g| in (0, 1] so that nothing overflows: for g < 0 it is
// g t / (1 + t).  (The direct form overflows e^-g below g = -88.7 and returns -0 where the value is still
// a normal number, e.g. silu(-89) = -2e-37.)
__device__ __forceinline__ float silu_f32(float g) {
  const float t = expf(-fabsf(g));
  return (g >= 0.f ? g : g * t) / (1.0f + t);
}

// bf16(silu(g) * u) for two (g, u) pairs packed as bf16x2 words; returns the packed bf16x2 result.
__device__ __forceinline__ uint32_t silu_mul_bf16x2(uint32_t g, uint32_t u) {
  const float g0 = bf16_to_f32(g & 0xFFFFu), g1 = bf16_to_f32(g >> 16);
  const float u0 = bf16_to_f32(u & 0xFFFFu), u1 = bf16_to_f32(u >> 16);
  return f32x2_to_bf16x2(silu_f32(g0) * u0, silu_f32(g1) * u1);
}

}  // namespace exl3
