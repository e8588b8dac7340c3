// Decode-phase kernel: a streaming split-K GEMM for small M.
//
// The weights are the whole cost at decode M, so the kernel is built around reading every trellis
// word exactly once, as early as possible:
//   * one wave owns NB adjacent tile columns (16*NB output features) over SPS k-steps of 64 features;
//     at entry it issues the loads for ALL of its words (one uint32 per lane per word it needs), so
//     the whole assignment is in flight at once;
//   * each arriving step is decoded in registers (exl3_device.hpp) straight into MFMA B fragments;
//     the rotated activations (fp16, permuted order) are the A fragments, 16 rows per M-block;
//   * every wave stores its fp32 partial [16 rows x 16*NB] into the split-K slab, then bumps the
//     counter of its 128-column block; the last arriving wave sums the splits in fixed order, applies
//     the output Hadamard-128, rout and s_out, rounds to bf16 and writes out[:, col0 + ...], then
//     resets the counter so the next launch (or graph replay) starts from zero.
// The slab and counters come from the caller's workspace ("radiance_escha.py", `_ensure_scratch`:
// split-K partial slab plus block counter, allocated once, never inside the launch).
#include "exl3_device.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

struct GemvArgs {
  const uint16_t* xh;      // fp16 [16 * mblocks, IC], PERM16 order within 16-groups, padding rows zero
  const uint32_t* code;    // tile words
  const uint16_t* rout;    // fp16 [OC]
  const uint16_t* s_out;   // fp16 [OC]
  float* slab;             // fp32 [S, M, OC]
  int* counters;           // [mblocks * OC/128]
  uint16_t* out;           // bf16 [M, ldo]
  int64_t ldo, col0;
  int M, IC, OC, S, steps;
  uint32_t code_bytes;     // size of the code tensor (buffer-resource range)
};

template <int K, int NB, int SPS>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs p) {
  using G = Geom<K>;
  // Activation slice of this block (16 rows x 64*SPS features, fp16), rows padded by 16 bytes so the
  // 16 lanes reading one fragment hit different banks.
  constexpr int kRowHalves = 64 * SPS + 8;
  __shared__ __attribute__((aligned(16))) uint16_t xs[16 * kRowHalves];

  const int lane = threadIdx.x & 63;
  const int ncg = p.OC / (16 * NB);                  // a multiple of 4: all waves of a block share s
  const int gw = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));   // wave-uniform
  const bool active = gw < ncg * p.S;
  const int mb = blockIdx.y;
  const int cg = gw % ncg, s = min(gw / ncg, p.S - 1);
  const int n = lane & 15, g = lane >> 4;
  const int st0 = s * SPS;                           // SPS divides the step count exactly
  const uint32_t tiles_per_row = uint32_t(p.OC / 16);

  // ---- 1. activation slice: issued first, so waiting for it never waits for the weight stream
  constexpr int kChunks = 16 * 8 * SPS;              // 16-byte chunks in the slice
  constexpr int kPerThread = (kChunks + 255) / 256;
  u32x4 xa[kPerThread];
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int c = threadIdx.x + 256 * q;
    if (c < kChunks) {
      const int r = c / (8 * SPS), c16 = c % (8 * SPS);
      xa[q] = *reinterpret_cast<const u32x4*>(p.xh + int64_t(mb * 16 + r) * p.IC + 64 * int64_t(st0) + 8 * c16);
    }
  }

  // ---- 2. every trellis word of this wave's assignment
  // Buffer loads: the resource covers the whole code tensor (reads past it return 0 instead of
  // faulting); byte offset = wave-uniform step base (scalar) + per-lane tile-row/word offset (vector)
  // + tile column j (immediate).
  int woff[G::kNW], shift;
  column_word_offsets<K>(n, woff, shift);
  const CodebookRegs cb = codebook_regs();
  constexpr bool kPrefetchAll = G::kNW * NB * SPS <= 128;
  uint32_t words[SPS][NB][G::kNW];
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(p.code), (short)0, (int)p.code_bytes, kBufferFlags);
  uint32_t lane_off[G::kNW];
#pragma unroll
  for (int w = 0; w < G::kNW; ++w) lane_off[w] = (uint32_t(g) * tiles_per_row * G::kWords + uint32_t(woff[w])) * 4u;
  const uint32_t wave_base = (4u * uint32_t(st0) * tiles_per_row + uint32_t(cg) * NB) * G::kWords * 4u;
  const uint32_t step_stride = 4u * tiles_per_row * G::kWords * 4u;
  auto load_step = [&](int st) {
    const uint32_t soff = wave_base + uint32_t(st) * step_stride;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
      for (int w = 0; w < G::kNW; ++w)
        words[st][j][w] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, lane_off[w] + uint32_t(j * G::kWords * 4), soff, 0);
    }
  };
  if constexpr (kPrefetchAll) {
    if (active) {
#pragma unroll
      for (int st = 0; st < SPS; ++st) load_step(st);
    }
  }

  // ---- 3. activations to LDS (the only barrier; every wave of the block reaches it)
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int c = threadIdx.x + 256 * q;
    if (c < kChunks) {
      const int r = c / (8 * SPS), c16 = c % (8 * SPS);
      *reinterpret_cast<u32x4*>(xs + r * kRowHalves + 8 * c16) = xa[q];
    }
  }
  __syncthreads();
  if (!active) return;

  // ---- 4. decode + MFMA, step by step as the words arrive
  float4v acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = (float4v){0.f, 0.f, 0.f, 0.f};
  const uint16_t* xl = xs + n * kRowHalves + 16 * g;   // A-operand row n, k-group g
#pragma unroll
  for (int st = 0; st < SPS; ++st) {
    if constexpr (!kPrefetchAll) load_step(st);
    const half8 a0 = *reinterpret_cast<const half8*>(xl + 64 * st);
    const half8 a1 = *reinterpret_cast<const half8*>(xl + 64 * st + 8);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      uint32_t b[8];
      decode_column<K>(words[st][j], shift, b, cb);
      acc[j] = mfma16(a0, as_half8(b[0], b[1], b[2], b[3]), acc[j]);
      acc[j] = mfma16(a1, as_half8(b[4], b[5], b[6], b[7]), acc[j]);
    }
  }

  // ---- partials: D fragment lane l holds rows 4*(l/16) + r of column l%16
  const int64_t M = p.M, OC = p.OC;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int64_t col = (int64_t(cg) * NB + j) * 16 + n;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mb * 16 + 4 * g + r;
      if (m < p.M) p.slab[(int64_t(s) * M + m) * OC + col] = acc[j][r];
    }
  }

  // ---- the last wave to finish a 128-column block of this M-block finishes it
  const int blk = (cg * NB * 16) / kHad;
  const int cidx = mb * (p.OC / kHad) + blk;
  const int contributors = p.S * (kHad / (16 * NB));
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");   // every lane's partial stores, before the count
  int old = 0;
  if (lane == 0)
    old = __hip_atomic_fetch_add(p.counters + cidx, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0, 64);
  if (old != contributors - 1) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // other waves' partials are visible from here

  const int64_t c0 = int64_t(blk) * kHad + 2 * lane;
  const float ro0 = f16_to_f32(p.rout[c0]), ro1 = f16_to_f32(p.rout[c0 + 1]);
  const float so0 = f16_to_f32(p.s_out[c0]), so1 = f16_to_f32(p.s_out[c0 + 1]);
  const int mend = min(p.M, mb * 16 + 16);
  for (int m = mb * 16; m < mend; ++m) {
    float v0 = 0.f, v1 = 0.f;
    for (int sp = 0; sp < p.S; ++sp) {
      const float* src = p.slab + (int64_t(sp) * M + m) * OC + c0;
      v0 += src[0];
      v1 += src[1];
    }
    had128_wave(v0, v1, lane);
    v0 = v0 * kInvSqrt128 * ro0 * so0;
    v1 = v1 * kInvSqrt128 * ro1 * so1;
    uint16_t* dst = p.out + int64_t(m) * p.ldo + p.col0 + c0;
    if (((p.ldo | p.col0) & 1) == 0) {
      *reinterpret_cast<uint32_t*>(dst) = f32_to_bf16(v0) | (f32_to_bf16(v1) << 16);
    } else {
      dst[0] = (uint16_t)f32_to_bf16(v0);
      dst[1] = (uint16_t)f32_to_bf16(v1);
    }
  }
  if (lane == 0) __hip_atomic_store(p.counters + cidx, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------------------------------
// Launch: pick the steps-per-split so that the grid has enough waves to cover the chip.
// ---------------------------------------------------------------------------------------------------
template <int K>
static hipError_t launch_k(const GemvPlan& pl, const GemvArgs& a, hipStream_t stream) {
  dim3 block(256);
  const int ncg = a.OC / (16 * kGemvNB);
  dim3 grid((unsigned)((ncg * a.S + 3) / 4), (unsigned)pl.mblocks);
  switch (pl.sps) {
    case 16: hipLaunchKernelGGL((gemv_kernel<K, kGemvNB, 16>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((gemv_kernel<K, kGemvNB, 8>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((gemv_kernel<K, kGemvNB, 4>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((gemv_kernel<K, kGemvNB, 2>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

GemvPlan plan_gemv(int64_t M, int64_t IC, int64_t OC) {
  GemvPlan pl;
  pl.mblocks = (int)((M + 15) / 16);
  pl.steps = (int)(IC / 64);                         // even, since IC is a multiple of 128
  const int64_t ncg = OC / (16 * kGemvNB);
  // Largest steps-per-split (16/8/4/2) dividing the step count that still gives ~6 waves per CU.
  pl.sps = 2;
  for (int c : {16, 8, 4}) {
    if (pl.steps % c) continue;
    if (ncg * (pl.steps / c) * pl.mblocks >= 1536 || c == 4) { pl.sps = c; break; }
  }
  if (pl.steps % pl.sps) pl.sps = 2;
  pl.S = pl.steps / pl.sps;
  return pl;
}

hipError_t launch_gemv(const GemvPlan& pl, const void* xh, const int16_t* code, int K, const void* rout,
                       const void* s_out, float* slab, int* counters, void* out, int64_t ldo, int64_t col0,
                       int64_t M, int64_t IC, int64_t OC, hipStream_t stream) {
  GemvArgs a;
  a.xh = (const uint16_t*)xh;
  a.code = (const uint32_t*)code;
  a.rout = (const uint16_t*)rout;
  a.s_out = (const uint16_t*)s_out;
  a.slab = slab;
  a.counters = counters;
  a.out = (uint16_t*)out;
  a.ldo = ldo;
  a.col0 = col0;
  a.M = (int)M;
  a.IC = (int)IC;
  a.OC = (int)OC;
  a.S = pl.S;
  a.steps = pl.steps;
  a.code_bytes = uint32_t(IC / 16 * (OC / 16) * 32 * K);
  switch (K) {
    case 1: return launch_k<1>(pl, a, stream);
    case 2: return launch_k<2>(pl, a, stream);
    case 3: return launch_k<3>(pl, a, stream);
    case 4: return launch_k<4>(pl, a, stream);
    case 5: return launch_k<5>(pl, a, stream);
    case 6: return launch_k<6>(pl, a, stream);
    case 7: return launch_k<7>(pl, a, stream);
    case 8: return launch_k<8>(pl, a, stream);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------------------------------
// Test hook: the decoded weight as fp16 [IC, OC], through decode_column.  One wave per 4 tiles of a
// tile row; lane (n, g) decodes column n of tile 4*wave_tile + g.
// ---------------------------------------------------------------------------------------------------
template <int K>
__global__ __launch_bounds__(256) void decode_tiles_kernel(uint16_t* __restrict__ w, const uint32_t* __restrict__ code,
                                                           int64_t IC, int64_t OC) {
  using G = Geom<K>;
  const int lane = threadIdx.x & 63;
  const int64_t ntiles = (IC / 16) * (OC / 16);
  const int64_t t = (int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  if (t >= ntiles) return;
  const int n = lane & 15;
  const int64_t a = t / (OC / 16), b = t % (OC / 16);
  int woff[G::kNW], shift;
  column_word_offsets<K>(n, woff, shift);
  uint32_t words[G::kNW];
  const uint32_t* tile = code + t * G::kWords;
#pragma unroll
  for (int j = 0; j < G::kNW; ++j) words[j] = tile[woff[j]];
  uint32_t v[8];
  decode_column<K>(words, shift, v, codebook_regs());
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    w[(16 * a + p) * OC + 16 * b + n] = uint16_t(v[p] & 0xFFFFu);
    w[(16 * a + p + 8) * OC + 16 * b + n] = uint16_t(v[p] >> 16);
  }
}

hipError_t launch_decode_tiles(void* w, const int16_t* code, int64_t IC, int64_t OC, int K, hipStream_t stream) {
  const int64_t ntiles = (IC / 16) * (OC / 16);
  if (ntiles == 0) return hipSuccess;
  dim3 block(256), grid((unsigned)((ntiles + 15) / 16));
  const uint32_t* c = (const uint32_t*)code;
  uint16_t* o = (uint16_t*)w;
  switch (K) {
    case 1: hipLaunchKernelGGL(decode_tiles_kernel<1>, grid, block, 0, stream, o, c, IC, OC); break;
    case 2: hipLaunchKernelGGL(decode_tiles_kernel<2>, grid, block, 0, stream, o, c, IC, OC); break;
    case 3: hipLaunchKernelGGL(decode_tiles_kernel<3>, grid, block, 0, stream, o, c, IC, OC); break;
    case 4: hipLaunchKernelGGL(decode_tiles_kernel<4>, grid, block, 0, stream, o, c, IC, OC); break;
    case 5: hipLaunchKernelGGL(decode_tiles_kernel<5>, grid, block, 0, stream, o, c, IC, OC); break;
    case 6: hipLaunchKernelGGL(decode_tiles_kernel<6>, grid, block, 0, stream, o, c, IC, OC); break;
    case 7: hipLaunchKernelGGL(decode_tiles_kernel<7>, grid, block, 0, stream, o, c, IC, OC); break;
    case 8: hipLaunchKernelGGL(decode_tiles_kernel<8>, grid, block, 0, stream, o, c, IC, OC); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace exl3
