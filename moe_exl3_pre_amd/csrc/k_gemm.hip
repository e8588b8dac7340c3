// Prefill-phase kernel: at large M the layer really is a dense contraction, so it runs as a tiled MFMA
// GEMM whose B operand is produced by the trellis decode on the fly ("radiance_escha.py",
// `escha_linear_into`: prefill GEMM chosen inside the op by M).
//
//   * the activation pre-pass (k_prepass.hip) has written xh = Had128((x * s_in) * rin) in fp16, PERM16
//     order, to the workspace;
//   * a block of 4 waves owns a 256 x 128 output tile (one Hadamard-128 block of columns); wave (wm, wn)
//     owns 128 rows x 64 columns;
//   * per 64-feature step (4 tile rows) the block stages the A tile [256 rows x 64] through LDS (double
//     buffered, one barrier per step) and each wave streams the trellis words of its 8 tile columns
//     one step ahead; lane (n, g) decodes
//     column n of tile row g of each tile column in registers (exl3_device.hpp) -- the two halves of
//     that column are the B fragments of two MFMA 16x16x32 f16 -- and the wave issues 64 MFMAs into
//     128 fp32 accumulators; the next step's loads are in flight meanwhile;
//   * epilogue: Hadamard-128 over the block's 128 columns -- DPP across the 16 lanes of a column group,
//     register butterflies across a wave's 4 groups, and the last stage (columns c, c+64) between the
//     two waves of a row half through LDS -- then * 1/sqrt(128) * rout * s_out, bf16 into the slice;
//   * blocks are ordered so that the ~32 blocks running on one XCD (consecutive block ids go to
//     different XCDs) share 4 row tiles and 8 column tiles, keeping A and the trellis words in its L2.
#include "exl3_device.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

constexpr int kBM = 256, kBN = 128;       // block tile
constexpr int kWM = 128, kWN = 64;        // wave tile
constexpr int kNBW = kWN / 16;            // column groups per wave
constexpr int kGroupM = 4;                // row tiles per XCD group

struct GemmArgs {
  const uint16_t* xh;       // fp16 [M, IC], PERM16 order
  const uint32_t* code;
  const uint16_t* rout;
  const uint16_t* s_out;
  const float* row_scale;   // 8-bit path: per-row scale of the integer codes in xh (else null)
  uint16_t* out;            // bf16 [M, ldo]
  int64_t ldo, col0;
  int M, IC, OC;
  int mt, nt;               // row / column tiles
  uint32_t code_bytes;
};

// Hadamard butterflies across the 16 lanes of a 16x16 accumulator column group (lane bits 0..3 =
// column bits 0..3).
__device__ __forceinline__ float had16_lanes(float v, int lane) {
  v = bfly(v, dpp<kQuadXor1>(v), lane & 1);
  v = bfly(v, dpp<kQuadXor2>(v), lane & 2);
  v = bfly(v, lane_xor4(v), lane & 4);
  v = bfly(v, lane_xor8(v), lane & 8);
  return v;
}

template <int K>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p) {
  using G = Geom<K>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int n = lane & 15, g = lane >> 4;

  // ---- block -> (row tile, column tile): XCD-grouped order
  const int T = p.mt * p.nt;
  const int nxcd = 8;
  const int bid = blockIdx.x;
  const int xcd = bid % nxcd, j = bid / nxcd;
  const int per = T / nxcd, extra = T % nxcd;
  const int tile = xcd * per + (xcd < extra ? xcd : extra) + j;   // contiguous range per XCD
  const int group = tile / (kGroupM * p.nt);
  const int gm = (p.mt - group * kGroupM) < kGroupM ? (p.mt - group * kGroupM) : kGroupM;
  const int in_group = tile - group * kGroupM * p.nt;
  const int mtile = group * kGroupM + in_group % gm;
  const int ntile = in_group / gm;

  const int row0 = mtile * kBM + wm * kWM;                  // first output row of this wave
  const int col0 = ntile * kBN + wn * kWN;                  // first shard column of this wave
  const uint32_t tpr = uint32_t(p.OC / kTile);

  // ---- A tile of the block: rows mtile*256 .. +256, one 64-feature step per LDS buffer, stored in
  //      MFMA fragment order: fragment (wm, mb, h) is 64 slots of 16 bytes; lane (n, g) of it is row
  //      wm*128 + 16*mb + n, PERM16 features 16g + 8h .. +8 of the step, kept in slot
  //      (16g + n) ^ (4g + 2h).  The XOR keeps each 16-lane read group on one contiguous 256-byte span
  //      (the conflict-free ds_read_b128 pattern) and sends the 8 chunks of a row, which 8 consecutive
  //      threads write after a coalesced global load, to 8 different bank groups.
  constexpr int kAFrag = 64 * 8;                            // halves per fragment
  __shared__ __attribute__((aligned(16))) uint16_t As[2][2 * 8 * 2 * kAFrag];
  const int steps = p.IC / 64;
  // staging: thread t copies row (t + 256 q) / 8, chunk (t + 256 q) % 8 of the step (coalesced rows)
  const uint16_t* asrc[8];
  int adst[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int cidx = threadIdx.x + 256 * q, r = cidx >> 3, c = cidx & 7;
    const int grow = mtile * kBM + r;
    asrc[q] = p.xh + int64_t(grow < p.M ? grow : p.M - 1) * p.IC + 8 * c;
    const int fwm = r >> 7, fmb = (r >> 4) & 7, fn = r & 15, fg = c >> 1, fh = c & 1;
    const int frag = (fwm * 8 + fmb) * 2 + fh;
    adst[q] = (frag * 64 + ((16 * fg + fn) ^ (4 * fg + 2 * fh))) * 8;
  }
  u32x4 astage[8];
  auto load_a = [&](int st) {
    const int s = st < steps ? st : steps - 1;
#pragma unroll
    for (int q = 0; q < 8; ++q) astage[q] = *reinterpret_cast<const u32x4*>(asrc[q] + 64 * s);
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 8; ++q) *reinterpret_cast<u32x4*>(&As[buf][adst[q]]) = astage[q];
  };

  // ---- B: tile columns col0/16 + nb; lane (n, g) decodes column n of tile row 4*step + g
  int woff[G::kNW], shift;
  column_word_offsets<K>(n, woff, shift);
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(p.code), (short)0, (int)p.code_bytes, kBufferFlags);
  uint32_t lane_off[G::kNW];
#pragma unroll
  for (int w = 0; w < G::kNW; ++w) lane_off[w] = (uint32_t(g) * tpr * G::kWords + uint32_t(woff[w])) * 4u;
  const uint32_t col_base = uint32_t(col0 / kTile) * G::kWords * 4u;
  const uint32_t step_stride = 4u * tpr * G::kWords * 4u;   // four tile rows per 64-feature step
  uint32_t wcur[kNBW][G::kNW], wnext[kNBW][G::kNW];
  auto load_w = [&](int st, uint32_t (&dst)[kNBW][G::kNW]) {
    const int s = st < steps ? st : steps - 1;                // clamped: the data is simply not used
    const uint32_t soff = uint32_t(s) * step_stride + col_base;
#pragma unroll
    for (int nb = 0; nb < kNBW; ++nb)
#pragma unroll
      for (int w = 0; w < G::kNW; ++w)
        dst[nb][w] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, lane_off[w] + uint32_t(nb * G::kWords * 4), soff, 0);
  };

  float4v acc[8][kNBW];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNBW; ++nb) acc[mb][nb] = (float4v){0.f, 0.f, 0.f, 0.f};

  const CodebookRegs cb = codebook_regs();
  load_a(0);
  load_w(0, wcur);
  store_a(0);
  __syncthreads();
  const int aslot0 = wm * 16 * kAFrag + (lane ^ (4 * g)) * 8;       // fragment (wm, mb, 0)
  const int aslot1 = wm * 16 * kAFrag + (lane ^ (4 * g + 2)) * 8;   // fragment (wm, mb, 1), less kAFrag
  // One step per iteration (no unrolled pair: that makes the compiler move the accumulators between
  // register files at the back edge); the double buffers rotate by value instead.
  for (int st = 0; st < steps; ++st) {
    const int buf = st & 1;
    load_a(st + 1);
    load_w(st + 1, wnext);
    half8 a[8][2];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      a[mb][0] = *reinterpret_cast<const half8*>(&As[buf][aslot0 + (2 * mb) * kAFrag]);
      a[mb][1] = *reinterpret_cast<const half8*>(&As[buf][aslot1 + (2 * mb + 1) * kAFrag]);
    }
#pragma unroll
    for (int nb = 0; nb < kNBW; ++nb) {
      uint32_t v[8];
      decode_column<K>(wcur[nb], shift, v, cb);
      const half8 b0 = as_half8(v[0], v[1], v[2], v[3]), b1 = as_half8(v[4], v[5], v[6], v[7]);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        acc[mb][nb] = mfma16(a[mb][0], b0, acc[mb][nb]);
        acc[mb][nb] = mfma16(a[mb][1], b1, acc[mb][nb]);
      }
    }
    store_a(buf ^ 1);                                       // the other buffer: last read one step ago
#pragma unroll
    for (int nb = 0; nb < kNBW; ++nb)
#pragma unroll
      for (int w = 0; w < G::kNW; ++w) wcur[nb][w] = wnext[nb][w];
    __syncthreads();
  }

  // ---- epilogue, one 16-row group at a time: Hadamard-128 over the block's 128 columns (column =
  //      64*wn + 16*nb + n: lane bits give column bits 0..3, nb bits 4..5, wn bit 6), then
  //      * 1/sqrt(128) * rout * s_out, bf16 into the slice.  The last stage pairs column c of wave
  //      (wm, 0) with column c + 64 of wave (wm, 1): each wave publishes its values in LDS.
  float* xch = reinterpret_cast<float*>(&As[0][0]);        // [4 waves][4 regs][kNBW][64 lanes], reused
  float sc[kNBW];
#pragma unroll
  for (int nb = 0; nb < kNBW; ++nb) {
    const int c = col0 + 16 * nb + n;
    sc[nb] = kInvSqrt128 * f16_to_f32(p.rout[c]) * f16_to_f32(p.s_out[c]);
  }
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {                          // unrolled: acc must stay in registers
    float v[kNBW][4];
#pragma unroll
    for (int nb = 0; nb < kNBW; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) v[nb][r] = had16_lanes(acc[mb][nb][r], lane);
#pragma unroll
    for (int h = 1; h < kNBW; h <<= 1)
#pragma unroll
      for (int nb = 0; nb < kNBW; ++nb)
        if (!(nb & h))
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float lo = v[nb][r], hi = v[nb | h][r];
            v[nb][r] = lo + hi;
            v[nb | h][r] = lo - hi;
          }
    __syncthreads();                                        // previous group's reads (and the main loop) done
#pragma unroll
    for (int nb = 0; nb < kNBW; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) xch[((wave * 4 + r) * kNBW + nb) * 64 + lane] = v[nb][r];
    __syncthreads();
    const int partner = wave ^ 1;                           // same wm, other column half
#pragma unroll
    for (int nb = 0; nb < kNBW; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float o = xch[((partner * 4 + r) * kNBW + nb) * 64 + lane];
        v[nb][r] = wn == 0 ? v[nb][r] + o : o - v[nb][r];
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 16 * mb + 4 * g + r;
      if (row < p.M) {
        // the row scale commutes with the column transform; 1.0 on the 16-bit path (exact)
        const float rs = p.row_scale ? p.row_scale[row] : 1.0f;
        uint16_t* dst = p.out + int64_t(row) * p.ldo + p.col0 + col0 + n;
#pragma unroll
        for (int nb = 0; nb < kNBW; ++nb) dst[16 * nb] = (uint16_t)f32_to_bf16(v[nb][r] * rs * sc[nb]);
      }
    }
  }
}

hipError_t launch_gemm(const void* xh, const int16_t* code, int K, const void* rout, const void* s_out, void* out,
                       int64_t ldo, int64_t col0, int64_t M, int64_t IC, int64_t OC, hipStream_t stream,
                       const float* row_scale) {
  GemmArgs a;
  a.xh = (const uint16_t*)xh;
  a.row_scale = row_scale;
  a.code = (const uint32_t*)code;
  a.rout = (const uint16_t*)rout;
  a.s_out = (const uint16_t*)s_out;
  a.out = (uint16_t*)out;
  a.ldo = ldo;
  a.col0 = col0;
  a.M = (int)M;
  a.IC = (int)IC;
  a.OC = (int)OC;
  a.mt = (int)((M + kBM - 1) / kBM);
  a.nt = (int)((OC + kBN - 1) / kBN);
  a.code_bytes = uint32_t(IC / 16 * (OC / 16) * 32 * K);
  dim3 grid((unsigned)(a.mt * a.nt)), block(256);
  switch (K) {
    case 1: hipLaunchKernelGGL(gemm_kernel<1>, grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(gemm_kernel<2>, grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL(gemm_kernel<3>, grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL(gemm_kernel<4>, grid, block, 0, stream, a); break;
    case 5: hipLaunchKernelGGL(gemm_kernel<5>, grid, block, 0, stream, a); break;
    case 6: hipLaunchKernelGGL(gemm_kernel<6>, grid, block, 0, stream, a); break;
    case 7: hipLaunchKernelGGL(gemm_kernel<7>, grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL(gemm_kernel<8>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace exl3
