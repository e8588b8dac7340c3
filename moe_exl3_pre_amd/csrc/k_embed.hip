// int8 embedding rows gathered by token id and dequantized ("vllm-quantpack 0.1.0", exl3/embedding.py,
// `Exl3EmbeddingMethod.embedding`): the table stays int8 with one scale per row, the rows of the requested
// ids are gathered and multiplied by their row's scale, so the table is never materialised in bf16.
//
// out[t, :] = bf16(table[ids[t], :] * scale[ids[t]]).  An int8 code times a bf16 scale is exact in fp32,
// so the one rounding is the conversion to bf16 (nearest, ties to even).  Ids outside [0, V) give zero
// rows (the page's tensor-parallel cut masks the ids a rank does not hold).
//
// One wave per (token, 1024 columns): each lane loads 16 codes as one 16-byte load and stores 16 bf16 as
// two 16-byte stores.  The kernel moves T*H bytes in and 2*T*H out; at decode sizes it is latency-bound.
#include "exl3_device.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

namespace {

constexpr int kEmbedChunk = 1024;   // columns one wave covers (64 lanes x 16)

__global__ __launch_bounds__(256) void embed_int8_kernel(uint16_t* __restrict__ out, const int8_t* __restrict__ table,
                                                         const uint16_t* __restrict__ scale, int64_t V, int64_t H,
                                                         const int32_t* __restrict__ ids, int64_t T) {
  const int lane = threadIdx.x & 63;
  const int64_t chunks = (H + kEmbedChunk - 1) / kEmbedChunk;
  const int64_t unit = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (unit >= T * chunks) return;
  const int64_t t = unit / chunks;
  const int64_t c = int64_t(unit % chunks) * kEmbedChunk + int64_t(lane) * 16;
  if (c >= H) return;                                        // H is a multiple of 16: whole lanes only
  const int id = ids[t];
  u32x4* dst = reinterpret_cast<u32x4*>(out + t * H + c);
  if (id < 0 || int64_t(id) >= V) {
    dst[0] = (u32x4){0u, 0u, 0u, 0u};
    dst[1] = (u32x4){0u, 0u, 0u, 0u};
    return;
  }
  const u32x4 q = *reinterpret_cast<const u32x4*>(table + int64_t(id) * H + c);
  const float s = bf16_to_f32(scale[id]);
  uint32_t o[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int32_t v = int32_t(q[w]);
    // bytes 0..3 of the word, sign-extended
    const float f0 = float((v << 24) >> 24) * s, f1 = float((v << 16) >> 24) * s;
    const float f2 = float((v << 8) >> 24) * s, f3 = float(v >> 24) * s;
    o[2 * w] = f32x2_to_bf16x2(f0, f1);
    o[2 * w + 1] = f32x2_to_bf16x2(f2, f3);
  }
  dst[0] = (u32x4){o[0], o[1], o[2], o[3]};
  dst[1] = (u32x4){o[4], o[5], o[6], o[7]};
}

}  // namespace

hipError_t launch_embed_int8(void* out, const int8_t* table, const void* scale, int64_t V, int64_t H,
                             const int32_t* ids, int64_t T, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int64_t units = T * ((H + kEmbedChunk - 1) / kEmbedChunk);
  hipLaunchKernelGGL(embed_int8_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, stream, (uint16_t*)out, table,
                     (const uint16_t*)scale, V, H, ids, T);
  return hipGetLastError();
}

}  // namespace exl3
