// Prefill-phase GEMM, one wave per 128 x 128 output tile ("radiance_escha.py", `escha_linear_into`: at
// large M the layer is a dense contraction against the decoded weights).
//
// Why this shape on gfx950.  The 32x32x16 f16 MFMA does twice the work of the 16x16x32 one per issue and
// sustains more of the matrix core: back-to-back, independent 16x16x32 MFMAs reach ~1.27 PFLOP/s on this
// chip, 32x32x16 ones ~1.85 (measured with the library's MFMA probe).  The trellis decode (the B operand)
// is VALU work that must hide behind the MFMAs, so every decoded column feeds 8 of them (4 row groups of
// 32 x 2 halves) and one wave owns a whole 128 x 128 tile.  The A operand needs no LDS: the pre-pass
// writes the rotated activations in a 32-row fragment-major layout (below), so each A fragment is one
// contiguous 1 KB wave load that the four waves of a block share through L1.  With 128 columns per wave
// every wave owns one whole Hadamard-128 block of outputs, so the output transform is done in registers:
// no barrier anywhere, and each wave runs independently.
//
//   * MFMA operands (32x32x16): A lane (m, k) holds row m < 32, k-slots 8k .. 8k+7; B lane (c, k) holds
//     column c < 32, the same k-slots; D lane (c, k) holds column c, rows 8 i + 4 k + r (value 4 i + r).
//     The two halves of the wave (k = 0, 1) decode the same output column from two different tile rows:
//     per 64-feature step and 32-column group nb, lane (c, k) decodes column c % 16 of tile 2 nb + c / 16
//     in tile row 2 j + k (j = 0, 1), a whole tile column (exl3_device.hpp, register p = rows p, p + 8);
//     registers 0..3 feed the MFMA of half 0 and 4..7 the MFMA of half 1, whose k-slots are therefore the
//     PERM16 positions 8 h .. 8 h + 7 of 16-group 2 j + k;
//   * 32-row fragment-major activations: per 32-row block, step s, pair j and half h, 1 KB holds lane
//     (m, k) = row m, PERM16 positions 64 s + 16 (2 j + k) + 8 h .. +8 (rows past M are zero);
//   * per step, the wave's trellis words arrive as K coalesced 16-byte loads per lane and pass through a
//     per-wave LDS slot (instead of several scattered word loads per tile column), the wave decodes 8 tile
//     columns per lane and issues 64 MFMAs into 256 fp32 accumulators (accumulator VGPRs); the next step's
//     A fragments (two register buffers, the loop unrolled by two so neither is copied) and the trellis
//     words of the step after (parked in the slot at the end of each step) are in flight meanwhile;
//   * epilogue per 32-row group: Hadamard-128 over the wave's columns (column = 32 nb + c: DPP butterflies
//     over lane bits 0..3, lane-pair swaps over bit 4, register butterflies over nb), * 1/sqrt(128) * rout
//     * s_out (* the row scale first on the 8-bit path), bf16 into the slice;
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
  const uint16_t* xf;       // 32-row fragment-major fp16 activations, M rounded up to 32 rows
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

// Column scales of the wave's 4 column groups: 1/sqrt(128) * rout * s_out at column col0 + 32 nb + c.
__device__ __forceinline__ void column_scales(const GemmArgs& p, int col0, int c, float (&sc)[4]) {
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int col = col0 + 32 * nb + c;
    sc[nb] = kInvSqrt128 * f16_to_f32(p.rout[col]) * f16_to_f32(p.s_out[col]);
  }
}

// Output transform of one 32-row group of a 128-column tile (rows r0 .. r0+31, columns col0 .. +127 of the
// shard): v[nb][4 i + r] holds row r0 + 8 i + 4 k + r, column 32 nb + c (lane (c, k)).  Hadamard-128 over
// the columns -- lane bits 0..3 by DPP, bit 4 by lane-pair swaps, bits 5, 6 (nb) in registers; the same
// butterflies in the same order for every value -- then * 1/sqrt(128) * rout * s_out (after * the row scale
// on the 8-bit path), rows 4 k + r and 4 k + r + 1 rounded to bf16 together and stored as 2-byte halves.
__device__ __forceinline__ void epilogue_group(const GemmArgs& p, float (&v)[4][16], const float (&sc)[4], int r0,
                                               int col0, int lane) {
  const int c = lane & 31, k = lane >> 5;
  had128_cols32(v, lane);
  if (p.row_scale) {                                        // 8-bit path: the row scale first
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = r0 + 8 * (r >> 2) + 4 * k + (r & 3);
      const float rs = p.row_scale[row < p.M ? row : p.M - 1];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) v[nb][r] *= rs;
    }
  }
  const bool full = r0 + 32 <= p.M;                         // wave-uniform: no row of the group is past M
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const int row = r0 + 8 * (r >> 2) + 4 * k + (r & 3);
    uint16_t* d0 = p.out + int64_t(row) * p.ldo + p.col0 + col0 + c;
    uint16_t* d1 = d0 + p.ldo;
    uint32_t w[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) w[nb] = f32x2_to_bf16x2(v[nb][r] * sc[nb], v[nb][r + 1] * sc[nb]);
    if (full) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        d0[32 * nb] = uint16_t(w[nb] & 0xFFFFu);
        d1[32 * nb] = uint16_t(w[nb] >> 16);
      }
    } else {
      const bool ok0 = row < p.M, ok1 = row + 1 < p.M;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        if (ok0) d0[32 * nb] = uint16_t(w[nb] & 0xFFFFu);
        if (ok1) d1[32 * nb] = uint16_t(w[nb] >> 16);
      }
    }
  }
}

template <int K, bool SPLIT>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs p) {
  using G = Geom<K>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;                   // staging: lane (n, g) loads and parks tile row g
  const int c = lane & 31, k = lane >> 5;                   // MFMA: lane (c, k)

  // ---- block -> (row tile, column group): a contiguous range of the launch's tiles per XCD
  const int T = p.ntiles;
  const int split = SPLIT ? __builtin_amdgcn_readfirstlane(int(blockIdx.x) / T) : 0;   // K split of this block
  const int nxcd = 8;
  const int bid = SPLIT ? int(blockIdx.x) - split * T : int(blockIdx.x);
  const int xcd = bid % nxcd, j0 = bid / nxcd;
  const int per = T / nxcd, extra = T % nxcd;
  const int lt = xcd * per + (xcd < extra ? xcd : extra) + j0;  // tile of this launch
  int mtile, ctile;                                         // row tile, this wave's 128-column block
  tile_coords(p, p.tile0 + lt, wave, mtile, ctile);
  if (ctile * kCols >= p.OC) return;                        // past the last column block (no barriers below)

  const int row0 = mtile * kRows;
  const int col0 = ctile * kCols;
  const int steps = p.IC / 64;                              // even: IC is a multiple of 128
  const int s0 = SPLIT ? split * p.sps : 0;                 // this split's steps [s0, s1), an even count
  const int s1 = SPLIT ? (s0 + p.sps < steps ? s0 + p.sps : steps) : steps;

  // ---- A: a buffer resource based at this row tile; 32-row group mb, step st, pair j, half h of the
  //      lane's fragment is at mb * steps * 4096 + st * 4096 + (2 j + h) * 1024 + lane * 16 bytes.  The
  //      record count ends at the last written row block, so fragments of row blocks past it read as zeros
  //      (those rows are not stored).
  const int64_t tile_bytes = int64_t(row0 >> 5) * steps * 4096;
  const int64_t left = p.xf_bytes - tile_bytes;
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.xf) + tile_bytes / 2, (short)0, (int)(left < 0x7FFFFFFF ? left : 0x7FFFFFFF), kBufferFlags);
  const uint32_t lane_byte = uint32_t(lane) * 16u;
  const uint32_t mb_stride = uint32_t(steps) * 4096u;
  auto load_a = [&](int st, half8 (&dst)[4][2][2]) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          dst[mb][j][h] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(
              arsrc, lane_byte + uint32_t((2 * j + h) * 1024), uint32_t(mb) * mb_stride + uint32_t(st) * 4096u, 0));
  };

  // ---- B: the words of one step of this wave's 8 tile columns are 4 tile rows x 256K contiguous bytes
  //      (tiles of a tile row are adjacent).  Lane group g loads its tile row with K coalesced 16-byte
  //      loads per lane; the wave parks them in its LDS slot (each row padded by 64 bytes so the four
  //      groups read different banks) and lane (c, k) reads back the words of column c % 16 of tile
  //      2 nb + c / 16 in tile rows k and 2 + k.  A step read past the shard re-reads the last one (the range
  //      check covers the vector offset only).
  __shared__ __attribute__((aligned(16))) char slots[kWavesN * Slot<K>::kBytes];
  char* my_slot = slots + wave * Slot<K>::kBytes;
  char* my_row = my_slot + g * Slot<K>::kRowBytes;
  int woff[G::kNW], shift;
  column_word_offsets<K>(c & 15, woff, shift);
  const int tsel = c >> 4;
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
  auto read_col = [&](int nb, int j, uint32_t (&dst)[G::kNW]) {
    const char* row = my_slot + (2 * j + k) * Slot<K>::kRowBytes;
#pragma unroll
    for (int w = 0; w < G::kNW; ++w)
      dst[w] = *reinterpret_cast<const uint32_t*>(row + ((2 * nb + tsel) * G::kWords + woff[w]) * 4);
  };

  float16v acc[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;

  const CodebookRegs cb = codebook_regs();
  // Trellis pipeline, three steps deep: at the start of step st the registers wv hold step st's column
  // words, the LDS slot holds step st + 1's words and the register buffer tn step st + 2's (in flight).
  // As soon as a column of step st is decoded, its registers receive the same column of step st + 1 from
  // the slot; at the end of the step tn is parked in the slot (after those reads: this wave's LDS
  // operations complete in order) and step st + 3 is loaded into tn.  So no step waits on LDS at its
  // start, and every global load has two steps of MFMAs to arrive in.
  u32x4 tn[K];
  auto park = [&]() {
    lane_exchange_fence();                                  // earlier reads of the slot come first
#pragma unroll
    for (int i = 0; i < K; ++i) *reinterpret_cast<u32x4*>(my_row + (i * 16 + n) * 16) = tn[i];
    lane_exchange_fence();                                  // later reads see these words
  };
  uint32_t wv[4][2][G::kNW];
  // One step: per decoded tile column 8 MFMAs (the 4 row groups, half 0 then half 1, so no MFMA waits on
  // the one before) and the read of the next step's words for that column; then park and load.  The
  // scheduling groups interleave one MFMA with kValuPerMfma VALU instructions, so the decode of the next
  // columns fills the MFMA issue gaps instead of running in bursts with the matrix core idle.
  constexpr int kValuPerMfma = K <= 1 ? 2 : K == 2 ? 3 : K == 3 ? 4 : K == 4 ? 5 : 8;
  auto step = [&](int st, const half8 (&a)[4][2][2]) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint32_t v[8];
        // the 64-bit-shift decode where it fits the register file (K <= 3; at K >= 4 it spills)
        decode_column<K, (K <= 3)>(wv[nb][j], shift, v, cb);
        read_col(nb, j, wv[nb][j]);                          // the same column of step st + 1
        const half8 b0 = as_half8(v[0], v[1], v[2], v[3]), b1 = as_half8(v[4], v[5], v[6], v[7]);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[mb][nb] = mfma32(a[mb][j][0], b0, acc[mb][nb]);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[mb][nb] = mfma32(a[mb][j][1], b1, acc[mb][nb]);
      }
    park();                                                 // step st + 2 (a clamped copy past the end)
    load_t(st + 3 < s1 ? st + 3 : s1 - 1, tn);
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);  // then VALU
    }
  };

  half8 a0[4][2][2], a1[4][2][2];
  // prologue: step s0's words into wv, step s0 + 1's into the slot, step s0 + 2's in flight in tn
  load_t(s0, tn);
  load_a(s0, a0);
  park();
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int j = 0; j < 2; ++j) read_col(nb, j, wv[nb][j]);
  load_t(s0 + 1 < s1 ? s0 + 1 : s1 - 1, tn);
  park();
  load_t(s0 + 2 < s1 ? s0 + 2 : s1 - 1, tn);
  // Two steps per iteration with the A buffers swapped, so neither is copied.
  // The scheduling barriers keep each A prefetch ahead of the step that precedes its use, so the loads
  // have a whole step of MFMAs to arrive in.
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
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          dst[((mb * 4 + nb) * 4 + q) * 64] =
              (float4v){acc[mb][nb][4 * q], acc[mb][nb][4 * q + 1], acc[mb][nb][4 * q + 2], acc[mb][nb][4 * q + 3]};
  } else {
    // ---- epilogue, one 32-row group at a time
    float sc[4];
    column_scales(p, col0, c, sc);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      float v[4][16];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) v[nb][r] = acc[mb][nb][r];
      epilogue_group(p, v, sc, row0 + 32 * mb, col0, lane);
    }
  }
}

// K-split reduction for a few splits (at most kFewSplits): one wave per (32-row group, 128-column tile),
// four units per workgroup, sums the splits' partials in split order (fixed, so the result is
// deterministic) and applies the output transform.
constexpr int kFewSplits = 3;

__global__ __launch_bounds__(256) void gemm_reduce_wave_kernel(GemmArgs p) {
  const int lane = threadIdx.x & 63;
  const int64_t unit = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (unit >= int64_t(p.ntiles) * kWavesN * 4) return;
  const int lt = int(unit / (kWavesN * 4)), wave = int(unit / 4) % kWavesN, mb = int(unit & 3);
  int mtile, ctile;
  tile_coords(p, p.tile0 + lt, wave, mtile, ctile);
  if (ctile * kCols >= p.OC) return;                        // past the last column block
  const int r0 = mtile * kRows + 32 * mb;
  if (r0 >= p.M) return;                                    // the whole group is past M
  float4v sum[4][4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int q = 0; q < 4; ++q) sum[nb][q] = (float4v){0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < p.splits; ++sp) {
    const float4v* src = p.slab + ((int64_t(sp) * p.ntiles + lt) * kWavesN + wave) * 4096 + mb * 16 * 64 + lane;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) sum[nb][q] += src[(nb * 4 + q) * 64];
  }
  float v[4][16], sc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) v[nb][4 * q + e] = sum[nb][q][e];
  column_scales(p, ctile * kCols, lane & 31, sc);
  epilogue_group(p, v, sc, r0, ctile * kCols, lane);
}

// K-split reduction for more than kFewSplits splits: one workgroup per (32-row group, 128-column tile).  Its four
// waves sum contiguous quarters of the splits, in split order, with the next split's loads in flight while
// one is added; wave 0 then adds the other waves' sums in wave order (a fixed order, so the result is
// deterministic) and applies the output transform.
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmArgs p) {
  __shared__ float4v part[3][16][64];                       // waves 1..3: their sums, 48 KB
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int64_t unit = blockIdx.x;
  if (unit >= int64_t(p.ntiles) * kWavesN * 4) return;     // uniform over the workgroup, as are the next two
  const int lt = int(unit / (kWavesN * 4)), wave = int(unit / 4) % kWavesN, mb = int(unit & 3);
  int mtile, ctile;
  tile_coords(p, p.tile0 + lt, wave, mtile, ctile);
  if (ctile * kCols >= p.OC) return;                        // past the last column block
  const int r0 = mtile * kRows + 32 * mb;
  if (r0 >= p.M) return;                                    // the whole group is past M
  auto first = [&](int ww) { return (ww * p.splits + 3) / 4; };
  const int s0 = first(w), s1 = first(w + 1);
  float4v sum[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) sum[i] = (float4v){0.f, 0.f, 0.f, 0.f};
  // split sp's 16 KB of partials for this group
  auto load = [&](int sp, float4v (&dst)[16]) {
    const float4v* src = p.slab + ((int64_t(sp) * p.ntiles + lt) * kWavesN + wave) * 4096 + mb * 16 * 64 + lane;
#pragma unroll
    for (int i = 0; i < 16; ++i) dst[i] = src[i * 64];
  };
  float4v buf[2][16];
  if (s0 < s1) load(s0, buf[0]);
  for (int sp = s0; sp < s1; sp += 2) {
    if (sp + 1 < s1) load(sp + 1, buf[1]);
#pragma unroll
    for (int i = 0; i < 16; ++i) sum[i] += buf[0][i];
    if (sp + 1 >= s1) break;
    if (sp + 2 < s1) load(sp + 2, buf[0]);
#pragma unroll
    for (int i = 0; i < 16; ++i) sum[i] += buf[1][i];
  }
  if (w > 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) part[w - 1][i][lane] = sum[i];
  }
  __syncthreads();
  if (w > 0) return;
  for (int ww = 1; ww < 4; ++ww)
    if (first(ww) < first(ww + 1))                          // a wave with no split adds nothing
#pragma unroll
      for (int i = 0; i < 16; ++i) sum[i] += part[ww - 1][i][lane];
  float v[4][16], sc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) v[nb][4 * q + e] = sum[nb * 4 + q][e];
  column_scales(p, ctile * kCols, lane & 31, sc);
  epilogue_group(p, v, sc, r0, ctile * kCols, lane);
}

}  // namespace

hipError_t launch_gemm(const void* xf, const int16_t* code, int K, const void* rout, const void* s_out, void* out,
                       int64_t ldo, int64_t col0, int64_t M, int64_t IC, int64_t OC, hipStream_t stream,
                       const float* row_scale, GemmSplit split, float* slab) {
  if ((split.splits > 1 || split.tail_splits > 1) && !slab) return hipErrorInvalidValue;
  GemmArgs a;
  a.xf = (const uint16_t*)xf;
  a.xf_bytes = (M + 31) / 32 * 32 * IC * 2;
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
      const int64_t units = int64_t(ntiles) * kWavesN * 4;   // (32-row group, tile) units
      if (splits <= kFewSplits)                               // a wave per unit
        hipLaunchKernelGGL(gemm_reduce_wave_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, stream, a);
      else                                                    // a workgroup per unit
        hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)units), dim3(256), 0, stream, a);
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
