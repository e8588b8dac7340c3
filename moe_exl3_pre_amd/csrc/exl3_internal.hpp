// Internal interface between the C ABI (exl3_api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace exl3 {

constexpr int kGemvNB = 2;              // tile columns per wave in the decode-phase kernel
constexpr int kCounterSlots = 4096;     // split-K block counters at the head of every workspace
constexpr size_t kCounterBytes = kCounterSlots * sizeof(int);
constexpr size_t kAlign = 256;

inline size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }

struct GemvPlan {
  int mblocks;   // 16-row blocks per launch
  int steps;     // 64-feature k-steps over IC
  int sps;       // k-steps per split (compile-time variants 4 / 8 / 16)
  int S;         // splits
};

GemvPlan plan_gemv(int64_t M, int64_t IC, int64_t OC);

// Rows one decode-phase launch covers (bounded by the counter slots: mblocks * OC/128 <= kCounterSlots).
inline int64_t gemv_chunk_rows(int64_t M, int64_t OC) {
  const int64_t blocks = OC / 128;
  int64_t mb = kCounterSlots / (blocks > 0 ? blocks : 1);
  if (mb < 1) mb = 1;
  const int64_t need = (M + 15) / 16;
  return (need < mb ? need : mb) * 16;
}

// Rows [M, M_pad) of xh are written as zeros.
hipError_t launch_prepass_f16(const void* x, const void* s_in, const void* rin, void* xh, int64_t M, int64_t IC,
                              bool permuted, hipStream_t stream, int64_t M_pad = 0);
hipError_t launch_prepass_i8(const void* x, const void* s_in, const void* rin, void* q, float* scale, int64_t M,
                             int64_t IC, bool permuted, hipStream_t stream);
hipError_t launch_gemv(const GemvPlan& pl, const void* xh, const int16_t* code, int K, const void* rout,
                       const void* s_out, float* slab, int* counters, void* out, int64_t ldo, int64_t col0,
                       int64_t M, int64_t IC, int64_t OC, hipStream_t stream);
hipError_t launch_decode_tiles(void* w, const int16_t* code, int64_t IC, int64_t OC, int K, hipStream_t stream);

}  // namespace exl3
