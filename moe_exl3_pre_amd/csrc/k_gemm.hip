// Prefill-phase GEMM, one wave per 128 x 128 output tile ("radiance_escha.py", `escha_linear_into`: at
// large M the layer is a dense contraction against the decoded weights).
//
// Why this shape on gfx950.  A 16x16x32 f16 MFMA keeps the matrix core busy for 16 cycles but holds the
// wave's issue port for about 8, and each VALU instruction costs about 4.5 more, so the trellis decode
// (the B operand) only hides behind the MFMAs when each decoded column feeds enough of them: here every
// column feeds 16 (8 row groups x 2 k-halves).  The A operand needs no LDS at all: the pre-pass writes
// the rotated activations fragment-major (below), so each A fragment is one contiguous 1 KB wave load
// that the four waves of a block share through L1.  With 128 columns per wave every wave owns one whole
// Hadamard-128 block of outputs, so the output transform is done in registers too: no barrier anywhere
// in the kernel, and each wave runs independently.
//
//   * fragment-major activations: for row block rb (16 rows), 64-feature step s and half h, 1 KB holds
//     lane (n, g) = row 16 rb + n, PERM16 positions 64 s + 16 g + 8 h .. +8 -- exactly the A operand
//     of one 16x16x32 MFMA (rows past M are zero);
//   * per step, the wave's trellis words arrive as K coalesced 16-byte loads per lane and pass through a
//     per-wave LDS slot (instead of several scattered word loads per tile column), lane
//     (n, g) decodes column n of tile row 4 s + g of each of the wave's 8 tile columns
//     (exl3_device.hpp) and the wave issues 128 MFMAs into 256 fp32 accumulators (accumulator VGPRs);
//     the next step's A fragments (two register buffers, the loop unrolled by two so neither is
//     copied) and the trellis words of the step after (parked in the slot at the end of each step) are
//     in flight meanwhile;
//   * epilogue per 16-row group: Hadamard-128 over the wave's columns (column = 16 nb + n: DPP
//     butterflies over the lane bits, stage by stage over all 32 values, register butterflies over nb),
//     * 1/sqrt(128) * rout * s_out (* the row scale first on the 8-bit path), bf16 into the slice;
//   * a block is 4 waves on the same 128 rows and 4 consecutive column blocks; blocks are ordered so
//     that the blocks running on one XCD (consecutive block ids go to different XCDs) share row tiles
//     and column groups in its L2.
#include "exl3_device.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

namespace {

constexpr int kRows = 128;                // rows per wave (and per block)
constexpr int kCols = 128;                // columns per wave
constexpr int kWavesN = 4;                // waves (column blocks) per block
constexpr int kGroupRows = 8;             // row tiles per XCD group

struct GemmArgs {
  const uint16_t* xf;       // fragment-major fp16 activations, M rounded up to 16 rows
  int64_t xf_bytes;
  const uint32_t* code;
  const uint16_t* rout;
  const uint16_t* s_out;
  const float* row_scale;   // 8-bit path: per-row scale of the integer codes (else null)
  uint16_t* out;            // bf16 [M, ldo]
  int64_t ldo, col0;
  int M, IC, OC;
  int mt, nt;               // row tiles (128 rows) / column groups (512 columns)
  uint32_t code_bytes;
  int splits, sps;          // K split: splits of sps 64-feature steps each (1: no split)
  int tile0, ntiles;        // this launch's blocks: tiles [tile0, tile0 + ntiles) of the mt x nt grid
  float4v* slab;            // splits > 1: [split][launch tile][wave][mb * 8 + nb][lane] partial sums
};

// Block tile -> (row tile, this wave's 128-column block).  Tiles run over groups of kGroupRows row tiles;
// inside a group, consecutive tiles walk down the rows first, so the blocks one XCD runs at a time (a
// contiguous range of tiles) share row tiles and column groups in its L2.
__device__ __forceinline__ void tile_coords(const GemmArgs& p, int tile, int wave, int& mtile, int& ctile) {
  const int group = tile / (kGroupRows * p.nt);
  const int gm = (p.mt - group * kGroupRows) < kGroupRows ? (p.mt - group * kGroupRows) : kGroupRows;
  const int in_group = tile - group * kGroupRows * p.nt;
  mtile = group * kGroupRows + in_group % gm;
  ctile = (in_group / gm) * kWavesN + wave;
}

// One butterfly stage of the Hadamard over the lane bits of a 16x16 accumulator group (lane bit b =
// column bit b), applied to all 32 values of a row group before the next stage so that the lane
// exchanges of different values fill each other's wait states.
template <int S>
__device__ __forceinline__ float lane_partner(float v) {
  if constexpr (S == 1) return dpp<kQuadXor1>(v);
  else if constexpr (S == 2) return dpp<kQuadXor2>(v);
  else if constexpr (S == 4) return lane_xor4(v);
  else return dpp<kRowRor8>(v);
}

template <int S>
__device__ __forceinline__ void lane_stage(float (&v)[8][4], int lane) {
  float q[8][4];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) q[nb][r] = lane_partner<S>(v[nb][r]);
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) v[nb][r] = bfly(v[nb][r], q[nb][r], lane & S);
}

// Output transform of one 16-row group of a 128-column tile (rows r0 .. r0+15, columns col0 .. +127 of
// the shard): v[nb][r] holds row r0 + 4g + r, column 16 nb + n.  Hadamard-128 over the columns, lane
// stages then register stages (the same butterflies in the same order for every value), * 1/sqrt(128) *
// rout * s_out (after * the row scale on the 8-bit path), rows 4g + r and 4g + r + 1 rounded to bf16
// together and stored as 2-byte halves.
__device__ __forceinline__ void column_scales(const GemmArgs& p, int col0, int n, float (&sc)[8]) {
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const int c = col0 + 16 * nb + n;
    sc[nb] = kInvSqrt128 * f16_to_f32(p.rout[c]) * f16_to_f32(p.s_out[c]);
  }
}

__device__ __forceinline__ void epilogue_group(const GemmArgs& p, float (&v)[8][4], const float (&sc)[8], int r0,
                                               int col0, int lane) {
  const int n = lane & 15, g = lane >> 4;
  lane_stage<1>(v, lane);
  lane_stage<2>(v, lane);
  lane_stage<4>(v, lane);
  lane_stage<8>(v, lane);
#pragma unroll
  for (int hb = 1; hb < 8; hb <<= 1)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      if (!(nb & hb))
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float lo = v[nb][r], hi = v[nb | hb][r];
          v[nb][r] = lo + hi;
          v[nb | hb][r] = lo - hi;
        }
  const int rbase = r0 + 4 * g;
  if (p.row_scale) {                                        // 8-bit path: the row scale first
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float rs = p.row_scale[rbase + r < p.M ? rbase + r : p.M - 1];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) v[nb][r] *= rs;
    }
  }
  const bool full = r0 + 16 <= p.M;                         // wave-uniform: no row of the group is past M
#pragma unroll
  for (int rp = 0; rp < 4; rp += 2) {
    uint16_t* d0 = p.out + int64_t(rbase + rp) * p.ldo + p.col0 + col0 + n;
    uint16_t* d1 = d0 + p.ldo;
    uint32_t w[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) w[nb] = f32x2_to_bf16x2(v[nb][rp] * sc[nb], v[nb][rp + 1] * sc[nb]);
    if (full) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        d0[16 * nb] = uint16_t(w[nb] & 0xFFFFu);
        d1[16 * nb] = uint16_t(w[nb] >> 16);
      }
    } else {
      const bool ok0 = rbase + rp < p.M, ok1 = rbase + rp + 1 < p.M;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        if (ok0) d0[16 * nb] = uint16_t(w[nb] & 0xFFFFu);
        if (ok1) d1[16 * nb] = uint16_t(w[nb] >> 16);
      }
    }
  }
}

template <int K, bool SPLIT>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs p) {
  using G = Geom<K>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;

  // ---- block -> (row tile, column group): a contiguous range of the launch's tiles per XCD
  const int T = p.ntiles;
  const int split = SPLIT ? __builtin_amdgcn_readfirstlane(int(blockIdx.x) / T) : 0;   // K split of this block
  const int nxcd = 8;
  const int bid = SPLIT ? int(blockIdx.x) - split * T : int(blockIdx.x);
  const int xcd = bid % nxcd, j = bid / nxcd;
  const int per = T / nxcd, extra = T % nxcd;
  const int lt = xcd * per + (xcd < extra ? xcd : extra) + j;   // tile of this launch
  int mtile, ctile;                                         // row tile, this wave's 128-column block
  tile_coords(p, p.tile0 + lt, wave, mtile, ctile);
  if (ctile * kCols >= p.OC) return;                        // past the last column block (no barriers below)

  const int row0 = mtile * kRows;
  const int col0 = ctile * kCols;
  const int steps = p.IC / 64;                              // even: IC is a multiple of 128
  const int s0 = SPLIT ? split * p.sps : 0;                 // this split's steps [s0, s1), an even count
  const int s1 = SPLIT ? (s0 + p.sps < steps ? s0 + p.sps : steps) : steps;

  // ---- A: a buffer resource based at this row tile; group mb, step st, half h of the lane's fragment is
  //      at mb * steps * 2048 + st * 2048 + h * 1024 + lane * 16 bytes.  The record count ends at the last
  //      written row block, so fragments of row blocks past it read as zeros (those rows are not stored).
  const int64_t tile_bytes = int64_t(row0 >> 4) * steps * 2048;
  const int64_t left = p.xf_bytes - tile_bytes;
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.xf) + tile_bytes / 2, (short)0, (int)(left < 0x7FFFFFFF ? left : 0x7FFFFFFF), kBufferFlags);
  const uint32_t lane_byte = uint32_t(lane) * 16u;
  const uint32_t mb_stride = uint32_t(steps) * 2048u;
  auto load_a = [&](int st, half8 (&dst)[8][2]) {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        dst[mb][h] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(
            arsrc, lane_byte + uint32_t(h * 1024), uint32_t(mb) * mb_stride + uint32_t(st) * 2048u, 0));
  };

  // ---- B: the words of one step of this wave's 8 tile columns are 4 tile rows x 256K contiguous bytes
  //      (tiles of a tile row are adjacent).  Lane group g loads its tile row with K coalesced 16-byte
  //      loads per lane; the wave parks them in its LDS slot (each row padded by 64 bytes so the four
  //      groups read different banks) and lane (n, g) reads the words of column n of each tile back.
  //      A step read past the shard re-reads the last one (the range check covers the vector offset only).
  __shared__ __attribute__((aligned(16))) char slots[kWavesN * Slot<K>::kBytes];
  char* my_row = slots + wave * Slot<K>::kBytes + g * Slot<K>::kRowBytes;
  int woff[G::kNW], shift;
  column_word_offsets<K>(n, woff, shift);
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(p.code), (short)0, (int)p.code_bytes, kBufferFlags);
  const uint32_t tpr = uint32_t(p.OC / kTile);
  const uint32_t lane_off = uint32_t(g) * tpr * G::kWords * 4u + uint32_t(n) * 16u;
  const uint32_t col_base = uint32_t(col0 / kTile) * G::kWords * 4u;
  const uint32_t step_stride = 4u * tpr * G::kWords * 4u;
  auto load_t = [&](int st, u32x4 (&dst)[K]) {
    const uint32_t soff = uint32_t(st) * step_stride + col_base;
#pragma unroll
    for (int i = 0; i < K; ++i)
      dst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane_off + uint32_t(i * 256), soff, 0));
  };
  auto read_col = [&](int nb, uint32_t (&dst)[G::kNW]) {
#pragma unroll
    for (int w = 0; w < G::kNW; ++w) dst[w] = *reinterpret_cast<const uint32_t*>(my_row + (nb * G::kWords + woff[w]) * 4);
  };

  float4v acc[8][8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[mb][nb] = (float4v){0.f, 0.f, 0.f, 0.f};

  const CodebookRegs cb = codebook_regs();
  // Trellis pipeline: the slot holds the current step's words, written at the end of the previous step;
  // the one register buffer tn holds the next step's, loaded a whole step before it is parked.  So a step
  // starts by reading its columns from LDS without waiting for any load, and every load has a step of
  // MFMAs to arrive in.  This wave's LDS operations complete in order, so parking the next step after the
  // current step's reads is safe.
  u32x4 tn[K];
  auto park = [&]() {
#pragma unroll
    for (int i = 0; i < K; ++i) *reinterpret_cast<u32x4*>(my_row + (i * 16 + n) * 16) = tn[i];
  };
  // One step: read every column's words at once (the LDS latency is paid once), then per tile column
  // decode and issue 16 MFMAs, then park the next step and load the one after.  The scheduling groups ask
  // for the LDS reads first and then one MFMA per kValuPerMfma VALU instructions, so the decode of the
  // next columns fills the MFMA issue gaps instead of running in bursts with the matrix core idle.
  constexpr int kValuPerMfma = K <= 1 ? 1 : K == 2 ? 2 : K <= 4 ? 3 : 4;
  auto step = [&](int st, const half8 (&a)[8][2]) {
    uint32_t wv[8][G::kNW];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) read_col(nb, wv[nb]);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      uint32_t v[8];
      decode_column<K, false>(wv[nb], shift, v, cb);
      const half8 b0 = as_half8(v[0], v[1], v[2], v[3]), b1 = as_half8(v[4], v[5], v[6], v[7]);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) acc[mb][nb] = mfma16(a[mb][0], b0, acc[mb][nb]);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) acc[mb][nb] = mfma16(a[mb][1], b1, acc[mb][nb]);
    }
    park();                                                 // step st + 1 (a clamped copy past the end)
    load_t(st + 2 < s1 ? st + 2 : s1 - 1, tn);
    __builtin_amdgcn_sched_group_barrier(0x100, 8 * G::kNW, 0);      // LDS reads
    // The MFMA/VALU groups also make the register allocator rotate the accumulators between the two
    // unrolled steps (~130 accumulator copies per step).  At K <= 2 the decode is short enough that the
    // copies cost more than the interleave gains (gate 5120 -> 17408 at M = 8192: -2% without the
    // groups, measured); at K >= 3 the interleave wins.
    if constexpr (K >= 3) {
#pragma unroll
      for (int i = 0; i < 128; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);  // then VALU
      }
    }
  };

  half8 a0[8][2], a1[8][2];
  load_t(s0, tn);
  load_a(s0, a0);
  park();
  load_t(s0 + 1, tn);
  // Two steps per iteration with the A buffers swapped, so neither is copied; the scheduling barriers
  // keep the halves apart so that the next step's A loads have a whole step of MFMAs to arrive in.
  for (int st = s0; st < s1; st += 2) {
    load_a(st + 1, a1);
    step(st, a0);
    __builtin_amdgcn_sched_barrier(0);
    load_a(st + 2 < s1 ? st + 2 : s1 - 1, a0);              // the last prefetch is not used
    step(st + 1, a1);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- a split parks its partial sums (1 KB wave stores; the reduction kernel finishes the tile)
  if constexpr (SPLIT) {
    float4v* dst = p.slab + ((int64_t(split) * p.ntiles + lt) * kWavesN + wave) * 4096 + lane;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) dst[(mb * 8 + nb) * 64] = acc[mb][nb];
  } else {
    // ---- epilogue, one 16-row group at a time
    float sc[8];
    column_scales(p, col0, n, sc);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      float v[8][4];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[nb][r] = acc[mb][nb][r];
      epilogue_group(p, v, sc, row0 + 16 * mb, col0, lane);
    }
  }
}

// K-split reduction over the launch's tiles: one wave per (16-row group, 128-column tile) sums the splits'
// partials in split order (fixed, so the result is deterministic) and applies the output transform.
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmArgs p) {
  const int lane = threadIdx.x & 63;
  const int64_t unit = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (unit >= int64_t(p.ntiles) * kWavesN * 8) return;
  const int lt = int(unit / (kWavesN * 8)), wave = int(unit / 8) % kWavesN, mb = int(unit & 7);
  int mtile, ctile;
  tile_coords(p, p.tile0 + lt, wave, mtile, ctile);
  if (ctile * kCols >= p.OC) return;                        // past the last column block
  const int r0 = mtile * kRows + 16 * mb;
  if (r0 >= p.M) return;                                    // the whole group is past M
  float4v sum[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) sum[nb] = (float4v){0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < p.splits; ++sp) {
    const float4v* src = p.slab + ((int64_t(sp) * p.ntiles + lt) * kWavesN + wave) * 4096 + mb * 8 * 64 + lane;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) sum[nb] += src[nb * 64];
  }
  float v[8][4], sc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) v[nb][r] = sum[nb][r];
  column_scales(p, ctile * kCols, lane & 15, sc);
  epilogue_group(p, v, sc, r0, ctile * kCols, lane);
}

}  // namespace

hipError_t launch_gemm(const void* xf, const int16_t* code, int K, const void* rout, const void* s_out, void* out,
                       int64_t ldo, int64_t col0, int64_t M, int64_t IC, int64_t OC, hipStream_t stream,
                       const float* row_scale, GemmSplit split, float* slab) {
  if ((split.splits > 1 || split.tail_splits > 1) && !slab) return hipErrorInvalidValue;
  GemmArgs a;
  a.xf = (const uint16_t*)xf;
  a.xf_bytes = (M + 15) / 16 * 16 * IC * 2;
  a.code = (const uint32_t*)code;
  a.rout = (const uint16_t*)rout;
  a.s_out = (const uint16_t*)s_out;
  a.row_scale = row_scale;
  a.out = (uint16_t*)out;
  a.ldo = ldo;
  a.col0 = col0;
  a.M = (int)M;
  a.IC = (int)IC;
  a.OC = (int)OC;
  a.mt = (int)((M + kRows - 1) / kRows);
  a.nt = (int)((OC + kCols * kWavesN - 1) / (kCols * kWavesN));
  a.code_bytes = uint32_t(IC / 16 * (OC / 16) * 32 * K);
  a.slab = reinterpret_cast<float4v*>(slab);
  const int T = a.mt * a.nt, steps = int(IC / 64);
  // One launch of tiles [tile0, tile0 + ntiles) with `splits` K splits of `sps` steps; a split launch is
  // followed by the reduction of the same tiles.
  auto launch_range = [&](int tile0, int ntiles, int splits, int sps) -> hipError_t {
    a.tile0 = tile0;
    a.ntiles = ntiles;
    a.splits = splits;
    a.sps = sps;
    dim3 grid((unsigned)(ntiles * splits)), block(64 * kWavesN);
#define EXL3_GEMM_CASE(KK)                                                                   \
  case KK:                                                                                   \
    if (splits > 1) hipLaunchKernelGGL((gemm_kernel<KK, true>), grid, block, 0, stream, a);    \
    else hipLaunchKernelGGL((gemm_kernel<KK, false>), grid, block, 0, stream, a);              \
    break;
    switch (K) {
      EXL3_GEMM_CASE(1)
      EXL3_GEMM_CASE(2)
      EXL3_GEMM_CASE(3)
      EXL3_GEMM_CASE(4)
      EXL3_GEMM_CASE(5)
      EXL3_GEMM_CASE(6)
      EXL3_GEMM_CASE(7)
      EXL3_GEMM_CASE(8)
      default: return hipErrorInvalidValue;
    }
#undef EXL3_GEMM_CASE
    if (splits > 1) {
      const int64_t units = int64_t(ntiles) * kWavesN * 8;
      hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
  };
  if (split.splits > 1) return launch_range(0, T, split.splits, split.sps);
  if (split.tail_blocks > 0 && split.tail_splits > 1 && split.tail_blocks < T) {
    if (hipError_t e = launch_range(0, T - split.tail_blocks, 1, steps); e != hipSuccess) return e;
    return launch_range(T - split.tail_blocks, split.tail_blocks, split.tail_splits, split.tail_sps);
  }
  return launch_range(0, T, 1, steps);
}

}  // namespace exl3
