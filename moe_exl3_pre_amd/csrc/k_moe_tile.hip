// MoE expert bank, the prefill-sized plan: grouped tiles of 64 gathered rows x 128 columns on the
// prefill GEMM's MFMA core.  Built apart from k_moe.hip with the iterative register scheduler the tile
// loops need.
#include <type_traits>

#include "k_moe.hpp"

namespace exl3 {

// ---------------------------------------------------------------------------------------------------
// Prefill-sized plan ("vLLM PR #190", commit message: a second MoE plan for prefill with 64-row blocks
// beside the decode plan).  With hundreds of rows per expert the streaming core of the decode-sized plan
// decodes each expert's weights once per 32-row chunk; here a slot's list is cut into chunks of
// kTileRows = 64 rows and each projection runs as tiles of 64 gathered rows x 128 columns with 32x32x16
// MFMAs (the prefill GEMM's operand layouts, k_gemm.hip; every decoded tile column feeds 4 of them), so
// every weight is decoded once per 64 rows.  A tile keeps 128 fp32 accumulators, so two waves share a
// SIMD and one wave's epilogue or memory wait overlaps the other's MFMAs.
//   * w13: a workgroup of two waves per (chunk, 128 intermediate features): wave 0 the w1 tile, wave 1 the
//     w3 tile of the same rows.  Both apply their output Hadamard-128 and svh in registers and swap half
//     of their rows through LDS, so that each wave holds h1 and h3 of 32 rows; each forms silu(h1) * h3 *
//     w2's suh for its rows, applies w2's input Hadamard (the same 128 features) and writes w2's fp16
//     operand.  As in the decode-sized plan h1, h3 and the product stay in fp32 until that operand.
//   * w2: a workgroup of four waves per (chunk, 512 output features), one 128-column tile each; output
//     Hadamard and svh; fp32 result per pair.
// Rows are gathered by pair id: each lane loads 16 bytes of its own row per A fragment (the rows are the
// rotated activations the route-and-rotate launch wrote, in PERM16 order), rows past the chunk read zeros.
// ---------------------------------------------------------------------------------------------------
constexpr int kMB = kTileRows / 32;               // 32-row groups per tile
constexpr int kGroupFloats = 4 * 16 * 64;          // one 32-row group of a 128-column tile, accumulator layout
// Waves per SIMD the tile kernels are built for: 128 accumulators leave room for two
constexpr int kTileWavesPerSimd = kMB <= 2 ? 2 : 1;

// One (32 MB) x 128 tile of one expert projection over `steps` 64-feature steps.  A holds fp16 rows of
// `lda` features; lane (c, k) gathers its row 32 mb + c from byte offset aoff[mb] (a_bytes or more reads
// zeros).  Trellis words as in the prefill GEMM: coalesced loads staged per wave in `slot`.
template <int K, int MB>
__device__ __forceinline__ void moe_tile_gemm(const uint16_t* code, uint32_t code_bytes, uint32_t tpr, int cb,
                                              const uint16_t* A, uint32_t a_bytes, const uint32_t (&aoff)[MB],
                                              int steps, char* slot, float16v (&acc)[MB][4]) {
  using G = Geom<K>;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;                   // staging: lane (n, g) loads and parks tile row g
  const int c = lane & 31, k = lane >> 5;                   // MFMA: lane (c, k)
  const __amdgpu_buffer_rsrc_t arsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A), (short)0, (int)a_bytes, kBufferFlags);
  char* my_row = slot + g * Slot<K>::kRowBytes;
  int woff[G::kNW], shift;
  column_word_offsets<K>(c & 15, woff, shift);
  const int tsel = c >> 4;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(code), (short)0, (int)code_bytes, kBufferFlags);
  const uint32_t lane_off = uint32_t(g) * tpr * G::kWords * 4u + uint32_t(n) * 16u;
  const uint32_t col_base = uint32_t(cb) * 8u * G::kWords * 4u;
  const uint32_t step_stride = 4u * tpr * G::kWords * 4u;
  auto load_t = [&](int st, u32x4 (&dst)[K]) {
    const uint32_t soff = uint32_t(st < steps ? st : steps - 1) * step_stride + col_base;
#pragma unroll
    for (int i = 0; i < K; ++i)
      dst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane_off + uint32_t(i * 256), soff, 0));
  };
  auto read_col = [&](int nb, int j, uint32_t (&dst)[G::kNW]) {
    const char* row = slot + (2 * j + k) * Slot<K>::kRowBytes;
#pragma unroll
    for (int w = 0; w < G::kNW; ++w)
      dst[w] = *reinterpret_cast<const uint32_t*>(row + ((2 * nb + tsel) * G::kWords + woff[w]) * 4);
  };
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;
  const CodebookRegs cbk = codebook_regs();
  u32x4 tn[K];
  auto park = [&]() {
    lane_exchange_fence();                                  // earlier reads of the slot come first
#pragma unroll
    for (int i = 0; i < K; ++i) *reinterpret_cast<u32x4*>(my_row + (i * 16 + n) * 16) = tn[i];
    lane_exchange_fence();                                  // later reads see these words
  };
  // The slot holds the words of the step being decoded; each lane reads one tile column ahead (two waves
  // share a SIMD, so one column of decode covers the LDS latency).  At the end of step st the words of
  // step st + 1 (loaded one step earlier) are parked and those of st + 2 requested.  The A fragments live
  // in one buffer: the tile columns run pair-half 0 first, so that half of the next step's fragments is
  // requested halfway through the step, the other half at its end.
  uint32_t wv[2][G::kNW];
  // VALU slots per MFMA in the schedule: the decode of one column feeds 2 MB MFMAs
  constexpr int kValuPerMfma = (K <= 1 ? 2 : K == 2 ? 3 : K <= 4 ? 5 : 8) * 4 / MB;
  half8 a[MB][2][2];
  auto load_a_half = [&](int st, int j) {
    st = st < steps ? st : steps - 1;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        a[mb][j][h] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(
            arsrc, aoff[mb] + uint32_t((64 * st + 16 * (2 * j + k) + 8 * h) * 2), 0, 0));
  };
  auto step = [&](int st) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = i >> 2, nb = i & 3;
      if (i + 1 < 8) read_col((i + 1) & 3, (i + 1) >> 2, wv[(i + 1) & 1]);
      uint32_t v[8];
      decode_column<K, (K <= 3)>(wv[i & 1], shift, v, cbk);
      const half8 b0 = as_half8(v[0], v[1], v[2], v[3]), b1 = as_half8(v[4], v[5], v[6], v[7]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb][nb] = mfma32(a[mb][j][0], b0, acc[mb][nb]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb][nb] = mfma32(a[mb][j][1], b1, acc[mb][nb]);
      if (i == 3) load_a_half(st + 1, 0);
    }
    load_a_half(st + 1, 1);
    park();
    load_t(st + 2, tn);
    read_col(0, 0, wv[0]);
#pragma unroll
    for (int i = 0; i < 16 * MB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
    }
  };
  load_t(0, tn);
  load_a_half(0, 0);
  load_a_half(0, 1);
  park();
  load_t(1, tn);
  read_col(0, 0, wv[0]);
  for (int st = 0; st < steps; ++st) {
    step(st);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The chunk's pair ids (-1 past its rows) in LDS, and this lane's gathered-row offsets.
__device__ __forceinline__ void moe_tile_rows(const MoeArgs& a, const int4v ch, int* pid, int lda, uint32_t a_bytes,
                                              uint32_t (&aoff)[kMB]) {
  const int row0 = ch[1], nrows = ch[2];
  for (int r = threadIdx.x; r < kTileRows; r += blockDim.x) pid[r] = r < nrows ? a.rows[row0 + r] : -1;
  __syncthreads();
  const int c = threadIdx.x & 31;
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) {
    const int q = pid[32 * mb + c];
    aoff[mb] = q >= 0 ? uint32_t(q) * uint32_t(lda) * 2u : a_bytes;
  }
}

// Row groups [mb0, mb0 + n) as compile-time constants: f(integral_constant<int, mb>) for each.
template <int MB0, int N, typename F>
__device__ __forceinline__ void for_groups(F&& f) {
  if constexpr (N > 0) {
    f(std::integral_constant<int, MB0>{});
    for_groups<MB0 + 1, N - 1>(f);
  }
}

// LDS of a w13 workgroup: the pair ids, then one region that holds the two waves' trellis slots during
// the main loop and the exchange tile (kMB groups of fp32) after it.
inline size_t moe_w13_tile_lds(size_t kslot) {
  const size_t xch = size_t(kMB) * kGroupFloats * 4;
  return 512 + (xch > 2 * kslot ? xch : 2 * kslot);
}

template <int K>
__device__ __forceinline__ void moe_w13_tile_block(const MoeArgs& a, const int4v ch, int ib, char* lds) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));   // wave 0: w1, wave 1: w3
  const int c = lane & 31, k = lane >> 5;
  const int slot = ch[0];
  int* pid = reinterpret_cast<int*>(lds);
  char* region = lds + 512;
  float* xch = reinterpret_cast<float*>(region);
  const uint32_t a_bytes = uint32_t(a.P) * uint32_t(a.ldx) * 2u;
  uint32_t aoff[kMB];
  moe_tile_rows(a, ch, pid, a.ldx, a_bytes, aoff);
  const int64_t off = wave == 0 ? a.off_w1[slot] : a.off_w3[slot];
  float16v acc[kMB][4];
  moe_tile_gemm<K, kMB>(a.w13 + off, uint32_t(int64_t(a.H) * a.I * K / 8), uint32_t(a.I / 16), ib,
                        a.xh13 + int64_t(wave) * a.P * a.ldx, a_bytes, aoff, a.H / 64, region + wave * Slot<K>::kBytes,
                        acc);
  const int col0 = ib * kHad;
  float sv[4], u2[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    sv[nb] = kInvSqrt128 * f16_to_f32(a.w13_svh[(int64_t(slot) * 2 + wave) * a.I + col0 + 32 * nb + c]);
    u2[nb] = f16_to_f32(a.w2_suh[int64_t(slot) * a.I + col0 + 32 * nb + c]);
  }
  // The per-32-row-group steps below take the group as a compile-time constant, so every accumulator
  // index is static and the accumulators stay in registers.
  // 1. each wave turns its own tile into h = svh * Had128(acc) / sqrt(128) (wave 0: h1, wave 1: h3), in place
  auto out_group = [&](auto mbc) {
    constexpr int mb = decltype(mbc)::value;
    float v[4][16];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) v[nb][r] = acc[mb][nb][r];
    had128_cols32(v, lane);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = v[nb][r] * sv[nb];
  };
  for_groups<0, kMB>(out_group);
  // 2. the waves split the row groups: wave 0 finishes groups [0, kMB / 2), wave 1 the others; each hands
  //    the other the groups it does not finish, through the exchange tile [wave][kMB / 2 groups][nb][r][lane],
  //    which overlays the trellis slots (hence the first barrier)
  constexpr int kHalfG = kMB / 2;
  __syncthreads();
  auto put_group = [&](auto mbc) {
    constexpr int mb = decltype(mbc)::value;
    float* dst = xch + (wave * kHalfG + mb % kHalfG) * kGroupFloats;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[(nb * 16 + r) * 64 + lane] = acc[mb][nb][r];
  };
  if (wave == 0)
    for_groups<kHalfG, kHalfG>(put_group);
  else
    for_groups<0, kHalfG>(put_group);
  __syncthreads();
  // 3. a = silu(h1) * h3 * w2's suh, w2's input rotation of these 128 features, fp16 in PERM16 order
  auto a_group = [&](auto mbc) {
    constexpr int mb = decltype(mbc)::value;
    const float* other = xch + ((1 - wave) * kHalfG + mb % kHalfG) * kGroupFloats;
    float v[4][16];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float mine = acc[mb][nb][r], theirs = other[(nb * 16 + r) * 64 + lane];
        const float h1 = wave == 0 ? mine : theirs, h3 = wave == 0 ? theirs : mine;
        // silu with the hardware reciprocal (one rounding more than a division, far below the fp16 step)
        v[nb][r] = h1 * __builtin_amdgcn_rcpf(1.0f + __expf(-h1)) * h3 * u2[nb];
      }
    had128_cols32(v, lane);                                 // w2's input rotation of these 128 features
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int q = pid[32 * mb + 8 * (r >> 2) + 4 * k + (r & 3)];
      if (q < 0) continue;
      uint16_t* dst = a.ah + int64_t(q) * a.ldh + col0;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int f = 32 * nb + c;                          // feature of the block, stored in PERM16 order
        dst[(f & ~15) + perm16_pos(f & 15)] = rot_f16(v[nb][r]);
      }
    }
  };
  if (wave == 0)
    for_groups<0, kHalfG>(a_group);
  else
    for_groups<kHalfG, kHalfG>(a_group);
}

template <int K>
__device__ __forceinline__ void moe_w2_tile_block(const MoeArgs& a, const int4v ch, int cg, char* lds) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int c = lane & 31, k = lane >> 5;
  const int slot = ch[0];
  int* pid = reinterpret_cast<int*>(lds);
  char* slots = lds + 512;
  const uint32_t a_bytes = uint32_t(a.P) * uint32_t(a.ldh) * 2u;
  uint32_t aoff[kMB];
  moe_tile_rows(a, ch, pid, a.ldh, a_bytes, aoff);
  const int hb = 4 * cg + wave;
  if (hb >= a.H / kHad) return;                             // past the last 128-column block (no barrier below)
  float16v acc[kMB][4];
  moe_tile_gemm<K, kMB>(a.w2 + a.off_w2[slot], uint32_t(int64_t(a.I) * a.H * K / 8), uint32_t(a.H / 16), hb, a.ah,
                        a_bytes, aoff, a.I / 64, slots + wave * Slot<K>::kBytes, acc);
  const int col0 = hb * kHad;
  float sv[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) sv[nb] = kInvSqrt128 * f16_to_f32(a.w2_svh[int64_t(slot) * a.H + col0 + 32 * nb + c]);
  auto o_group = [&](auto mbc) {
    constexpr int mb = decltype(mbc)::value;
    float v[4][16];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) v[nb][r] = acc[mb][nb][r];
    had128_cols32(v, lane);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int q = pid[32 * mb + 8 * (r >> 2) + 4 * k + (r & 3)];
      if (q < 0) continue;
      float* dst = a.o + int64_t(q) * a.H + col0 + c;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) dst[32 * nb] = v[nb][r] * sv[nb];
    }
  };
  for_groups<0, kMB>(o_group);
}

template <int KSET>
__global__ __launch_bounds__(128, kTileWavesPerSimd) void moe_w13_tile_kernel(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int c, ib;
  moe_tile(a.I / kHad, c, ib);
  int4v ch;
  if (!moe_chunk(a, c, ch)) return;
  moe_dispatch<KSET>(ch[3] & 0xFF, [&](auto k) { moe_w13_tile_block<decltype(k)::value>(a, ch, ib, lds); });
}

template <int KSET>
__global__ __launch_bounds__(256, kTileWavesPerSimd) void moe_w2_tile_kernel(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int c, cg;
  moe_tile((a.H / kHad + 3) / 4, c, cg);
  int4v ch;
  if (!moe_chunk(a, c, ch)) return;
  moe_dispatch<KSET>(ch[3] >> 8, [&](auto k) { moe_w2_tile_block<decltype(k)::value>(a, ch, cg, lds); });
}

// One pass of the prefill plan (0: w13, 1: w2) for the K set KS (0: the mixed set {2, 3, 4}); the grid
// covers `cgroups` chunk slots (moe_chunk_slots, see moe_tile) x the column groups.
template <int KS>
static void launch_tiles(const MoeArgs& a, int pass, size_t kslot, int64_t cgroups, hipStream_t stream) {
  if (pass == 0)
    hipLaunchKernelGGL(moe_w13_tile_kernel<KS>, dim3(unsigned(cgroups * (a.I / kHad))), dim3(128),
                       moe_w13_tile_lds(kslot), stream, a);
  else
    hipLaunchKernelGGL(moe_w2_tile_kernel<KS>, dim3(unsigned(cgroups * ((a.H / kHad + 3) / 4))), dim3(256),
                       512 + 4 * kslot, stream, a);
}

void launch_moe_tile_pass(const MoeArgs& a, int pass, int kset, size_t kslot, int64_t cgroups, hipStream_t stream) {
  switch (kset) {
    case 0: launch_tiles<0>(a, pass, kslot, cgroups, stream); break;
    case 1: launch_tiles<1>(a, pass, kslot, cgroups, stream); break;
    case 2: launch_tiles<2>(a, pass, kslot, cgroups, stream); break;
    case 3: launch_tiles<3>(a, pass, kslot, cgroups, stream); break;
    case 4: launch_tiles<4>(a, pass, kslot, cgroups, stream); break;
    case 5: launch_tiles<5>(a, pass, kslot, cgroups, stream); break;
    case 6: launch_tiles<6>(a, pass, kslot, cgroups, stream); break;
    case 7: launch_tiles<7>(a, pass, kslot, cgroups, stream); break;
    case 8: launch_tiles<8>(a, pass, kslot, cgroups, stream); break;
    default: break;
  }
}

}  // namespace exl3
