// int8 embedding rows gathered by token id and dequantized ("vllm-quantpack 0.1.0", exl3/embedding.py,
// `Exl3EmbeddingMethod.embedding`): the table is kept as int8 codes plus one scale per row, and only the
// rows a call asks for are dequantized; no bf16 copy of the whole table exists.
//
// out[t, :] = bf16(table[ids[t], :] * scale[ids[t]]).  An int8 code times a bf16 scale is exact in fp32,
// so the one rounding is the conversion to bf16 (nearest, ties to even).  Ids outside [0, V) give zero
// rows (the page's tensor-parallel cut masks the ids a rank does not hold).
//
// One wave per (token, 1024 columns): each lane loads 16 codes as one 16-byte load and stores 16 bf16 as
// two 16-byte stores.  The kernel moves T*H bytes in and 2*T*H out; at decode sizes it is latency-bound.
//
// The same table as the output head ("vllm-quantpack 0.1.0", exl3/embedding.py, `Exl3EmbeddingMethod.apply`):
// logits[m, v] = bf16(sum_h x[m, h] * w[v, h]) with every weight rounded once, w[v, h] = bf16(q[v, h] * s[v]),
// as the page dequantizes the table in bf16 before its linear map.  See lm_head_int8_kernel.
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

// ---------------------------------------------------------------------------------------------------
// Output head over the int8 table.  A workgroup of 4 waves owns 16 * G table rows; its waves split the
// H/64 feature steps into 4 contiguous parts, each wave streams its part of those rows once, and wave 0
// adds the four partial tiles from LDS in part order.  The x rows (up to 16 * MR) are the MFMA's other
// operand and come from the caches.  Small work items (V / 16G workgroups) keep the last round of
// workgroups short; more rows per wave (G) amortize the x loads when many x rows are live.
//
// Operands of v_mfma_f32_16x16x32_bf16: A = 16 table rows x 32 features, B = 32 features x 16 x rows.
// Lane l holds A row (l % 16) and B column (l % 16), features 8 * (l / 16) .. +8 of the instruction's 32.
// The 64 features of one step are split so that lane l owns features 16 * (l / 16) .. +16 of the step in
// both operands: one 16-byte load of int8 codes and two of bf16 x; the first 8 feed the first MFMA and the
// last 8 the second (the same permutation of the summation index on both sides).
//
// The weight: the code byte is biased to unsigned (q + 128, one xor per 4 codes), converted with the
// unsigned-byte conversion and scaled by fma(q + 128, s, -128 s) = q * s, exact in fp32 (at most 16
// significant bits), then rounded to bf16 by the hardware conversion: the page's bf16(q * s).
// The result D: lane l holds x row (l % 16) and table rows 4 * (l / 16) .. +4, written as 8 bytes when
// the output's base and row stride allow it (vec_store), else element by element.
//
// The summation order of a logit depends only on H (steps in order within a part, parts in order), not on
// M, G or MR, so a row's logits are the same bits whatever else is in the batch.
// ---------------------------------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kHeadParts = 4;   // waves per workgroup, each a contiguous quarter of the feature steps

__device__ __forceinline__ bf16x8 head_weights(uint32_t w0, uint32_t w1, float s, float c) {
  uint32_t o[4];
  const uint32_t u[2] = {w0 ^ 0x80808080u, w1 ^ 0x80808080u};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float f0 = fmaf(float(u[j] & 0xFFu), s, c), f1 = fmaf(float((u[j] >> 8) & 0xFFu), s, c);
    const float f2 = fmaf(float((u[j] >> 16) & 0xFFu), s, c), f3 = fmaf(float(u[j] >> 24), s, c);
    o[2 * j] = f32x2_to_bf16x2(f0, f1);
    o[2 * j + 1] = f32x2_to_bf16x2(f2, f3);
  }
  return __builtin_bit_cast(bf16x8, (u32x4){o[0], o[1], o[2], o[3]});
}

__device__ __forceinline__ float4v mfma_bf16(bf16x8 a, bf16x8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// MR groups of 16 x rows (M <= 16 * MR), G groups of 16 table rows per workgroup, U steps of 64 features
// loaded before they are used.
template <int MR, int G, int U>
__global__ __launch_bounds__(256) void lm_head_int8_kernel(uint16_t* __restrict__ out, int64_t ldo,
                                                           const uint16_t* __restrict__ x, int M,
                                                           const int8_t* __restrict__ table,
                                                           const uint16_t* __restrict__ scale, int64_t V, int64_t H,
                                                           bool vec_store) {
  __shared__ float4v red[kHeadParts][MR * G][64];
  const int lane = threadIdx.x & 63, part = threadIdx.x >> 6;
  const int r16 = lane & 15, quarter = lane >> 4;
  const int64_t v0 = int64_t(blockIdx.x) * 16 * G;
  const int64_t steps = H / 64;
  const int64_t h_lo = steps * part / kHeadParts * 64, h_hi = steps * (part + 1) / kHeadParts * 64;

  const int8_t* trow[G];
  bool tok[G];
  float s[G], c[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t v = v0 + 16 * g + r16;
    tok[g] = v < V;
    trow[g] = table + (tok[g] ? v : 0) * H + 16 * quarter;
    s[g] = tok[g] ? bf16_to_f32(scale[v]) : 0.0f;
    c[g] = -128.0f * s[g];
  }
  const uint16_t* xrow[MR];
  bool xok[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    const int m = 16 * r + r16;
    xok[r] = m < M;
    xrow[r] = x + int64_t(xok[r] ? m : 0) * H + 16 * quarter;
  }

  float4v acc[MR][G];
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int g = 0; g < G; ++g) acc[r][g] = (float4v){0.f, 0.f, 0.f, 0.f};

  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto step = [&](const u32x4 (&q)[G], const u32x4 (&xb)[MR][2]) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const bf16x8 w0 = head_weights(q[g][0], q[g][1], s[g], c[g]);
      const bf16x8 w1 = head_weights(q[g][2], q[g][3], s[g], c[g]);
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        acc[r][g] = mfma_bf16(w0, __builtin_bit_cast(bf16x8, xb[r][0]), acc[r][g]);
        acc[r][g] = mfma_bf16(w1, __builtin_bit_cast(bf16x8, xb[r][1]), acc[r][g]);
      }
    }
  };

  int64_t h = h_lo;
  for (; h + 64 * U <= h_hi; h += 64 * U) {
    u32x4 q[U][G], xb[U][MR][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int g = 0; g < G; ++g)
        q[u][g] = tok[g] ? *reinterpret_cast<const u32x4*>(trow[g] + h + 64 * u) : zero;
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        const u32x4* p = reinterpret_cast<const u32x4*>(xrow[r] + h + 64 * u);
        xb[u][r][0] = xok[r] ? p[0] : zero;
        xb[u][r][1] = xok[r] ? p[1] : zero;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) step(q[u], xb[u]);
  }
  for (; h < h_hi; h += 64) {
    u32x4 q[G], xb[MR][2];
#pragma unroll
    for (int g = 0; g < G; ++g) q[g] = tok[g] ? *reinterpret_cast<const u32x4*>(trow[g] + h) : zero;
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      const u32x4* p = reinterpret_cast<const u32x4*>(xrow[r] + h);
      xb[r][0] = xok[r] ? p[0] : zero;
      xb[r][1] = xok[r] ? p[1] : zero;
    }
    step(q, xb);
  }

  // partial tiles to LDS; wave 0 adds them in part order and writes the logits
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int g = 0; g < G; ++g) red[part][r * G + g][lane] = acc[r][g];
  __syncthreads();
  if (part != 0) return;
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    if (!xok[r]) continue;
    uint16_t* orow = out + int64_t(16 * r + r16) * ldo;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float4v t = red[0][r * G + g][lane];
#pragma unroll
      for (int k = 1; k < kHeadParts; ++k) t += red[k][r * G + g][lane];
      const int64_t v = v0 + 16 * g + 4 * quarter;
      const uint32_t lo = f32x2_to_bf16x2(t[0], t[1]);
      const uint32_t hi = f32x2_to_bf16x2(t[2], t[3]);
      if (vec_store && v + 4 <= V) {
        *reinterpret_cast<uint2*>(orow + v) = make_uint2(lo, hi);
      } else {
        const uint16_t e[4] = {uint16_t(lo), uint16_t(lo >> 16), uint16_t(hi), uint16_t(hi >> 16)};
        for (int i = 0; i < 4 && v + i < V; ++i) orow[v + i] = e[i];
      }
    }
  }
}

// 5..16 x rows, H a multiple of 256: x is the larger stream (as many bytes per 64-feature step as 64 table
// rows), so a workgroup of 4 waves owning 64 table rows stages each 256-feature slice of x in LDS once and
// every wave reads its B operands from there.  Each wave streams its own 16 rows over all of H, keeping
// one accumulator per quarter of the feature steps (the same quarters as lm_head_int8_kernel) and adding
// them in the same order, so the logits are the same bits as that kernel's.
constexpr int kHeadXStride = 256 + 8;   // halves per staged x row: 528 bytes, rows 4 banks apart

__global__ __launch_bounds__(256) void lm_head_int8_xlds_kernel(uint16_t* __restrict__ out, int64_t ldo,
                                                                const uint16_t* __restrict__ x, int M,
                                                                const int8_t* __restrict__ table,
                                                                const uint16_t* __restrict__ scale, int64_t V,
                                                                int64_t H, bool vec_store) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[16 * kHeadXStride];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, quarter = lane >> 4;
  const int64_t v = int64_t(blockIdx.x) * 64 + wave * 16 + r16;
  const bool tok = v < V;
  const int8_t* trow = table + (tok ? v : 0) * H + 16 * quarter;
  const float s = tok ? bf16_to_f32(scale[v]) : 0.0f, c = -128.0f * s;
  const int64_t steps = H / 64;
  int64_t bound[kHeadParts];
#pragma unroll
  for (int p = 0; p < kHeadParts; ++p) bound[p] = steps * (p + 1) / kHeadParts * 64;
  // staging: thread tid copies 16 features (32 bytes) of x row tid / 16
  const int sr = tid >> 4, sc = (tid & 15) * 16;
  const bool sok = sr < M;
  const uint16_t* xsrc = x + int64_t(sok ? sr : 0) * H + sc;

  float4v acc[kHeadParts];
#pragma unroll
  for (int p = 0; p < kHeadParts; ++p) acc[p] = (float4v){0.f, 0.f, 0.f, 0.f};
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int64_t h = 0; h < H; h += 256) {
    u32x4 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = tok ? *reinterpret_cast<const u32x4*>(trow + h + 64 * u) : zero;
    const u32x4 x0 = sok ? *reinterpret_cast<const u32x4*>(xsrc + h) : zero;
    const u32x4 x1 = sok ? *reinterpret_cast<const u32x4*>(xsrc + h + 8) : zero;
    __syncthreads();                                       // the previous slice is no longer read
    *reinterpret_cast<u32x4*>(xs + sr * kHeadXStride + sc) = x0;
    *reinterpret_cast<u32x4*>(xs + sr * kHeadXStride + sc + 8) = x1;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t hs = h + 64 * u;
      const int part = hs < bound[0] ? 0 : hs < bound[1] ? 1 : hs < bound[2] ? 2 : 3;
      const uint16_t* xp = xs + r16 * kHeadXStride + 64 * u + 16 * quarter;
      const u32x4 b0 = *reinterpret_cast<const u32x4*>(xp), b1 = *reinterpret_cast<const u32x4*>(xp + 8);
      const bf16x8 w0 = head_weights(q[u][0], q[u][1], s, c), w1 = head_weights(q[u][2], q[u][3], s, c);
      float4v t = acc[0];
      if (part == 1) t = acc[1];
      if (part == 2) t = acc[2];
      if (part == 3) t = acc[3];
      t = mfma_bf16(w0, __builtin_bit_cast(bf16x8, b0), t);
      t = mfma_bf16(w1, __builtin_bit_cast(bf16x8, b1), t);
      if (part == 0) acc[0] = t;
      if (part == 1) acc[1] = t;
      if (part == 2) acc[2] = t;
      if (part == 3) acc[3] = t;
    }
  }
  if (r16 >= M) return;
  float4v t = acc[0];
#pragma unroll
  for (int p = 1; p < kHeadParts; ++p) t += acc[p];
  uint16_t* orow = out + int64_t(r16) * ldo;
  const int64_t v4 = int64_t(blockIdx.x) * 64 + wave * 16 + 4 * quarter;
  const uint32_t lo = f32x2_to_bf16x2(t[0], t[1]);
  const uint32_t hi = f32x2_to_bf16x2(t[2], t[3]);
  if (vec_store && v4 + 4 <= V) {
    *reinterpret_cast<uint2*>(orow + v4) = make_uint2(lo, hi);
  } else {
    const uint16_t e[4] = {uint16_t(lo), uint16_t(lo >> 16), uint16_t(hi), uint16_t(hi >> 16)};
    for (int i = 0; i < 4 && v4 + i < V; ++i) orow[v4 + i] = e[i];
  }
}

template <int MR, int G, int U>
void launch_head(uint16_t* out, int64_t ldo, const uint16_t* x, int M, const int8_t* table, const uint16_t* scale,
                 int64_t V, int64_t H, bool vec_store, hipStream_t stream) {
  const int64_t blocks = (V + 16 * G - 1) / (16 * G);
  hipLaunchKernelGGL((lm_head_int8_kernel<MR, G, U>), dim3((unsigned)blocks), dim3(64 * kHeadParts), 0, stream, out,
                     ldo, x, M, table, scale, V, H, vec_store);
}

}  // namespace

// x rows in chunks of up to 64 (four 16-row MFMA groups); each chunk streams the whole table once.  Rows per
// workgroup by the number of live x rows, from a sweep at V = 248,320, H = 5120: 16 while few x lanes load
// (M <= 4), 32 up to 8 rows, 64 above (the x loads then cost as much as the table's).
hipError_t launch_lm_head_int8(void* out, int64_t ldo, const void* x, int64_t M, const int8_t* table,
                               const void* scale, int64_t V, int64_t H, hipStream_t stream) {
  const bool vec_store = ldo % 4 == 0 && reinterpret_cast<uintptr_t>(out) % 8 == 0;
  const uint16_t* sc = static_cast<const uint16_t*>(scale);
  for (int64_t m0 = 0; m0 < M; m0 += 64) {
    const int rows = int(M - m0 < 64 ? M - m0 : 64);
    uint16_t* o = static_cast<uint16_t*>(out) + m0 * ldo;
    const uint16_t* xs = static_cast<const uint16_t*>(x) + m0 * H;
    if (rows <= 4) launch_head<1, 1, 4>(o, ldo, xs, rows, table, sc, V, H, vec_store, stream);
    else if (rows <= 16 && H % 256 == 0)
      hipLaunchKernelGGL(lm_head_int8_xlds_kernel, dim3((unsigned)((V + 63) / 64)), dim3(256), 0, stream, o, ldo, xs,
                         rows, table, sc, V, H, vec_store);
    else if (rows <= 8) launch_head<1, 2, 4>(o, ldo, xs, rows, table, sc, V, H, vec_store, stream);
    else if (rows <= 16) launch_head<1, 4, 2>(o, ldo, xs, rows, table, sc, V, H, vec_store, stream);
    else if (rows <= 32) launch_head<2, 2, 2>(o, ldo, xs, rows, table, sc, V, H, vec_store, stream);
    else if (rows <= 48) launch_head<3, 1, 2>(o, ldo, xs, rows, table, sc, V, H, vec_store, stream);
    else launch_head<4, 1, 2>(o, ldo, xs, rows, table, sc, V, H, vec_store, stream);
    if (hipError_t e = hipGetLastError()) return e;
  }
  return hipSuccess;
}

hipError_t launch_embed_int8(void* out, const int8_t* table, const void* scale, int64_t V, int64_t H,
                             const int32_t* ids, int64_t T, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int64_t units = T * ((H + kEmbedChunk - 1) / kEmbedChunk);
  hipLaunchKernelGGL(embed_int8_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, stream, (uint16_t*)out, table,
                     (const uint16_t*)scale, V, H, ids, T);
  return hipGetLastError();
}

}  // namespace exl3
