// Decode-phase kernel (M <= 16): the whole layer -- activation pre-pass, trellis decode, contraction,
// reduction, output Hadamard-128, rout/s_out scales and the bf16 slice write -- in ONE launch that can
// cover several shards of a merged projection ("radiance_escha.py", `escha_linear_into`: the
// prefill/decode choice is made inside the op; `apply`: each shard writes its own column slice).
//
// At decode M the trellis words are the whole cost, so the kernel is shaped around streaming them once:
//   * a block of 8 waves owns one 128-column output block of one shard (one Hadamard-128 block, so the
//     output transform needs no other block) over a range of the input features; two blocks share a CU
//     (the dispatcher deals blocks i and i + 256 to one CU, and shards are laid out heavier K first, so
//     most CUs pair a K=3 block with a K=2 one);
//   * the 8 waves split that feature range; each step's trellis words arrive as coalesced 16-byte loads,
//     pass through the wave's LDS slot, and every lane decodes one tile column in registers
//     (exl3_device.hpp) straight into MFMA B fragments and accumulates [16 rows x 128 cols] in fp32;
//   * while the first words are in flight the block computes its own slice of the rotated activations
//     (x * s_in * rin, Hadamard-128, fp16, permuted order) into LDS -- no separate pre-pass launch and no
//     round trip of the activations through HBM;
//   * the 8 partial accumulators are summed in LDS in a fixed order (deterministic), then each wave
//     takes output rows wave, wave + 8 and applies the output Hadamard, rout and s_out and writes bf16;
//   * when a shard has too few 128-column blocks to fill both block slots of every CU its feature range
//     is split over several blocks (S > 1): each writes its partial rows to the split-K slab with agent-coherent
//     stores, bumps the block counter (agent-scope atomic, no L2-wide fences), and the last one to arrive
//     finishes the block and resets the counter for the next launch or graph replay.  The slab and the
//     counters live in the caller's workspace ("radiance_escha.py", `_ensure_scratch`: split-K partial
//     slab plus block counter, allocated once, never inside the launch).
#include <climits>
#include <utility>

#include "exl3_device.hpp"
#include "exl3_internal.hpp"
#include "k_silu.hpp"

namespace exl3 {

constexpr int kWaves = 8;        // waves per block (two blocks share a CU)
constexpr int kNB = 8;           // tile columns per wave = one 128-column block

struct DecShard {
  const uint32_t* code;
  const uint16_t* xf;            // pre-rotated activations, fragment-major (MR == 0 only)
  const float* sc;               // 8-bit path: row scales of the integer codes in xf (else null)
  const float* part;             // 8-bit path, in-block codes (I8): per-(row, 128-block) max |xh|, [M, IC / 128]
  const uint16_t* s_in;
  const uint16_t* rin;
  const uint16_t* rout;
  const uint16_t* s_out;
  float* slab;                   // [S, M, OC] fp32 (S > 1 only)
  int* counters;                 // [OC / 128] (S > 1 only)
  int64_t col0;
  uint32_t code_bytes;
  int OC, K, S, wg_begin;
};

struct DecArgs {
  const uint16_t* x;             // bf16 [M, IC]
  uint16_t* out;                 // bf16 [M, ldo]
  int64_t ldo;
  int M, IC, n_shards, lds_row;  // lds_row: halves per activation row in LDS (padded)
  int tr_off;                    // byte offset of the per-wave trellis staging slots in LDS
  int wgb[kMaxShards];           // first workgroup of each shard in grid order; INT_MAX past n_shards
  DecShard sh[kMaxShards];
};


// MR: activation rows the fused pre-pass loads (1, 4 or 16).  MR == 0: the activations were rotated once
// for the whole launch by the fragment-major pre-pass (the prefill path's, k_prepass.hip), and each step's
// two A fragments are 16-byte loads from that buffer issued with the step's trellis words.  Then no block
// repeats the rotation, which at M = 8 costs about as much VALU as the decode itself.
// SILU (MR 1 or 4 only): a.x is a dense MLP block's gate_up output [M, 2 IC]; the pre-pass input is
// h = bf16(silu(g) * u), g = a.x[m, k], u = a.x[m, IC + k], formed as the block's activation kernel forms it.
// RG (MR == 0 only): 16-row groups of the launch.  With RG = 2 one launch covers up to 32 rows: every
// decoded tile column feeds the MFMAs of both groups, so the weights are streamed once for 32 rows, and
// each group is reduced exactly as a 16-row launch reduces it (the same bits per row).
// I8 (MR 1 or 4 only): the 8-bit path with the codes formed in the in-block pre-pass.  Each row's scale
// sc = max / 127 comes from the per-(row, block) maxima of sh.part (the values the fragment-major pre-pass
// forms, by the same max and division), the rotated values are quantised as that pre-pass quantises them,
// q = clamp(rne(xh / sc), +-127) in fp32, and stored as fp16 numbers; the epilogue applies the row scale.
template <int K, int SPW, int MR, bool SILU = false, int RG = 1, bool I8 = false>
__device__ __forceinline__ void decode_block(const DecArgs& a, const DecShard& sh, int local, char* lds) {
  constexpr bool kPre = MR == 0;
  static_assert(!SILU || MR == 1 || MR == 4, "the folded activation is for the in-block pre-pass");
  static_assert(!I8 || ((MR == 1 || MR == 4) && !SILU && RG == 1), "in-block codes: 1..4 rows, 16-bit input");
  static_assert(RG == 1 || (RG == 2 && kPre), "two row groups need pre-rotated activations");
  using G = Geom<K>;
  // steps of trellis words in flight per wave: one.  Every block requests its first step at once, so
  // deeper prefetch only queues the first data of late waves behind the early waves' later steps.
  constexpr int kD = 1;
  constexpr int kPB = SPW > 1 ? SPW / 2 : 1;                        // Hadamard blocks per wave (pre-pass)
  static_assert(SPW % 2 == 0, "steps come in Hadamard-block pairs");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int M = a.M;
  const int nblk = sh.OC / kHad;
  const int blk = local % nblk, s = local / nblk;
  const int B = a.IC / kHad;
  const int ba = s * B / sh.S, bb = (s + 1) * B / sh.S;     // Hadamard blocks of this block's k-range
  const int nb = bb - ba;
  // Each wave owns whole Hadamard blocks [hb0, hb1) of that range (two 64-feature steps each): it
  // rotates their activations itself, so no wave waits for another before its main loop.
  const int hb0 = (nb * wave) / kWaves, hb1 = (nb * (wave + 1)) / kWaves;
  const int w_s0 = 2 * hb0, cnt = 2 * (hb1 - hb0);         // cnt <= SPW (planner)
  const uint32_t tpr = uint32_t(sh.OC / kTile);

  uint16_t* xs = reinterpret_cast<uint16_t*>(lds);          // [(M + 1) rows][lds_row] fp16
  const int lrow = a.lds_row;

  // ---- 1. pre-pass inputs of this wave's Hadamard blocks (issued first: they are needed first).
  // Unconditional loads with clamped rows and blocks: a load under a branch would make the compiler
  // wait for the weight stream behind it before the pre-pass can start.
  constexpr int kMR = kPre ? 1 : MR;
  uint32_t xv[kPB][kMR], sv[kPB], rv[kPB];
  uint32_t xu[kPB][SILU ? kMR : 1];   // SILU: the up half (xv holds the gate half)
#pragma unroll
  for (int pb = 0; pb < (kPre ? 0 : kPB); ++pb) {
    const int hb = hb0 + pb < hb1 ? hb0 + pb : (hb1 > hb0 ? hb1 - 1 : 0);
    // lane transforms features f and f + 8 (perm_pair_feature), stored at PERM16 positions 2l, 2l+1
    const int64_t f = int64_t(ba + hb) * kHad + perm_pair_feature(lane);
    sv[pb] = uint32_t(sh.s_in[f]) | (uint32_t(sh.s_in[f + 8]) << 16);
    rv[pb] = uint32_t(sh.rin[f]) | (uint32_t(sh.rin[f + 8]) << 16);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if constexpr (SILU) {
        const uint16_t* gr = a.x + int64_t(m < M ? m : M - 1) * 2 * a.IC + f;
        xv[pb][m] = uint32_t(gr[0]) | (uint32_t(gr[8]) << 16);
        xu[pb][m] = uint32_t(gr[a.IC]) | (uint32_t(gr[a.IC + 8]) << 16);
      } else {
        const uint16_t* xr = a.x + int64_t(m < M ? m : M - 1) * a.IC + f;
        xv[pb][m] = uint32_t(xr[0]) | (uint32_t(xr[8]) << 16);
      }
    }
  }
  // I8: the rows' block maxima (reduced over the wave once the weight stream is requested)
  const int nq = a.IC / kHad;
  float pmax[I8 ? kMR : 1];
#pragma unroll
  for (int m = 0; m < (I8 ? kMR : 0); ++m) {
    const float* pr = sh.part + int64_t(m < M ? m : M - 1) * nq;
    pmax[m] = 0.f;
    for (int b = lane; b < nq; b += 64) pmax[m] = fmaxf(pmax[m], pr[b]);
  }
  __builtin_amdgcn_sched_barrier(0);   // keep these loads ahead of the weight stream

  // ---- 2. the first kD steps of the weight stream, as coalesced 16-byte loads.  One step of this
  // block is 4 tile rows (lane group g) x 8 tiles x 8K words: each lane group reads its tile row's
  // 256K contiguous bytes with K loads of 16 bytes per lane.
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(sh.code), (short)0, (int)sh.code_bytes, kBufferFlags);
  const uint32_t lane_off = uint32_t(g) * tpr * G::kWords * 4u + uint32_t(n) * 16u;
  const uint32_t step_stride = 4u * tpr * G::kWords * 4u;
  const uint32_t base_blk = uint32_t(blk) * kNB * G::kWords * 4u;
  u32x4 tb[kD][K];
  half8 ta[kD][RG][2];   // pre-rotated A fragments of the staged steps (kPre)
  auto load_a = [&](int st, half8 (&dst)[RG][2]) {
    const int step = 2 * ba + (cnt > 0 ? w_s0 + (st < cnt ? st : cnt - 1) : 0);
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {   // 16-row block rg of the fragment-major buffer
      const uint16_t* f = sh.xf + ((int64_t(rg) * (a.IC / 64) + step) * 2 * 512 + lane * 8);
      dst[rg][0] = *reinterpret_cast<const half8*>(f);
      dst[rg][1] = *reinterpret_cast<const half8*>(f + 512);
    }
  };
  auto load_step = [&](int st, u32x4 (&dst)[K]) {
    // Steps past this wave's count (their results are never used) re-read a step of this block's own
    // range, so every address stays inside the tensor: the buffer range check covers only the vector
    // offset, not the scalar one used here.
    const int step = 2 * ba + (cnt > 0 ? w_s0 + (st < cnt ? st : cnt - 1) : 0);
    const uint32_t soff = uint32_t(step) * step_stride + base_blk;
#pragma unroll
    for (int i = 0; i < K; ++i)
      dst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane_off + uint32_t(i * 256), soff, 0));
  };
#pragma unroll
  for (int d = 0; d < kD; ++d) {
    if constexpr (kPre) load_a(d, ta[d]);
    load_step(d, tb[d]);
  }

  // ---- 3. this wave's rotated activations (I8: their codes) into LDS (PERM16 order); its part of row M
  // stays zero
  float rsc[I8 ? kMR : 1];   // I8: the rows' scales (wave-uniform)
#pragma unroll
  for (int m = 0; m < (I8 ? kMR : 0); ++m) {
    float mx = pmax[m];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d, 64));
    rsc[m] = __fdiv_rn(mx, 127.0f);
  }
#pragma unroll
  for (int pb = 0; pb < (kPre ? 0 : kPB); ++pb) {
    if (hb0 + pb < hb1) {
      const float s0 = f16_to_f32(sv[pb] & 0xFFFFu), s1 = f16_to_f32(sv[pb] >> 16);
      const float r0 = f16_to_f32(rv[pb] & 0xFFFFu), r1 = f16_to_f32(rv[pb] >> 16);
      const int kl = (hb0 + pb) * kHad + 2 * lane;          // PERM16 positions 2l, 2l+1 of the block
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        if (m < M) {
          uint32_t xw = xv[pb][m];
          if constexpr (SILU) xw = silu_mul_bf16x2(xv[pb][m], xu[pb][m]);
          float v0 = bf16_to_f32(xw & 0xFFFFu) * s0 * r0;
          float v1 = bf16_to_f32(xw >> 16) * s1 * r1;
          had128_wave_pairs8(v0, v1, lane);
          if constexpr (I8) {
            const float sc = rsc[m];
            auto code = [&](float xv) -> float {
              return sc > 0.f ? fminf(fmaxf(rintf(__fdiv_rn(xv * kInvSqrt128, sc)), -127.f), 127.f) : 0.f;
            };
            *reinterpret_cast<uint32_t*>(xs + m * lrow + kl) = f32x2_to_f16x2(code(v0), code(v1));
          } else {
            *reinterpret_cast<uint32_t*>(xs + m * lrow + kl) = rot_f16x2(v0, v1);
          }
        }
      }
      *reinterpret_cast<uint32_t*>(xs + M * lrow + kl) = 0u;
    }
  }

  // ---- 4. per step: stage the words in this wave's LDS slot, then every lane reads the words of its
  // tile column (column n of tile row g), decodes them into MFMA B operands and accumulates.  Only
  // this wave touches its slot and its slice of xs, so no barrier is needed; LDS operations of one wave
  // complete in order, so the reads of a step see that step's writes and the next step's writes do
  // not overtake this step's reads (lane_exchange_fence keeps the compiler to that order).
  lane_exchange_fence();                                    // the rotated activations above are written
  char* slot = lds + a.tr_off + wave * Slot<K>::kBytes;
  char* my_row = slot + g * Slot<K>::kRowBytes;
  int woff[G::kNW], shift;
  column_word_offsets<K>(n, woff, shift);
  const CodebookRegs cb = codebook_regs();
  float4v acc[RG][kNB];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int j = 0; j < kNB; ++j) acc[rg][j] = (float4v){0.f, 0.f, 0.f, 0.f};
  const uint16_t* xa = xs + (n < M ? n : M) * lrow + 64 * w_s0 + 16 * g;   // row n, or the zero row
#pragma unroll
  for (int st = 0; st < SPW; ++st) {
    if (st < cnt) {
      lane_exchange_fence();                                // the previous step's reads come first
#pragma unroll
      for (int i = 0; i < K; ++i)
        *reinterpret_cast<u32x4*>(my_row + (i * 16 + n) * 16) = tb[st % kD][i];
      lane_exchange_fence();                                // this step's reads see these words
    }
    half8 a0[RG], a1[RG];
    if constexpr (kPre) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        a0[rg] = ta[st % kD][rg][0];
        a1[rg] = ta[st % kD][rg][1];
      }
      load_a(st + kD, ta[st % kD]);
    }
    load_step(st + kD, tb[st % kD]);
    if (st < cnt) {
      if constexpr (!kPre) {
        a0[0] = *reinterpret_cast<const half8*>(xa + 64 * st);
        a1[0] = *reinterpret_cast<const half8*>(xa + 64 * st + 8);
      }
      uint32_t wv[2][G::kNW];
      auto read_col = [&](int j, uint32_t (&dst)[G::kNW]) {
#pragma unroll
        for (int w = 0; w < G::kNW; ++w)
          dst[w] = *reinterpret_cast<const uint32_t*>(my_row + (j * G::kWords + woff[w]) * 4);
      };
      read_col(0, wv[0]);
#pragma unroll
      for (int j = 0; j < kNB; ++j) {
        if (j + 1 < kNB) read_col(j + 1, wv[(j + 1) & 1]);
        uint32_t b[8];
        decode_column<K>(wv[j & 1], shift, b, cb);
        const half8 b0 = as_half8(b[0], b[1], b[2], b[3]), b1 = as_half8(b[4], b[5], b[6], b[7]);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) acc[rg][j] = mfma16(a0[rg], b0, acc[rg][j]);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) acc[rg][j] = mfma16(a1[rg], b1, acc[rg][j]);
      }
    }
  }

  // ---- 5. sum the waves' partials in LDS (fixed order), one 16-row group at a time; wave w finishes
  // rows w and w + kWaves of every group
  const int64_t c0 = int64_t(blk) * kHad + 2 * lane;        // shard-local column of (v0, v1)
  constexpr int kRW = (kDecodeMaxRows + kWaves - 1) / kWaves; // output rows per wave and group
  constexpr int kRT = RG * kRW;                               // output rows per wave
  auto out_row = [&](int t) { return kDecodeMaxRows * (t / kRW) + wave + (t % kRW) * kWaves; };
  float v0[kRT], v1[kRT];
  float* red = reinterpret_cast<float*>(lds);               // [kWaves][rows of the group][128]
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const int Mg = M - kDecodeMaxRows * rg < kDecodeMaxRows ? M - kDecodeMaxRows * rg : kDecodeMaxRows;
    __syncthreads();                                        // xs, or the previous group's partials, are read
#pragma unroll
    for (int j = 0; j < kNB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * g + r;
        if (row < Mg) red[(wave * Mg + row) * kHad + 16 * j + n] = acc[rg][j][r];
      }
    __syncthreads();
#pragma unroll
    for (int tg = 0; tg < kRW; ++tg) {
      const int row = wave + tg * kWaves;                   // within the group
      v0[rg * kRW + tg] = v1[rg * kRW + tg] = 0.f;
      if (row < Mg) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float* p = red + (w * Mg + row) * kHad + 2 * lane;
          v0[rg * kRW + tg] += p[0];
          v1[rg * kRW + tg] += p[1];
        }
      }
    }
  }

  if (sh.S > 1) {
    // ---- 6a. split-K hand-off: coherent partial stores, then one counter bump per block
    const int64_t OC = sh.OC;
#pragma unroll
    for (int t = 0; t < kRT; ++t) {
      const int row = out_row(t);
      if (row < M) {
        float* dst = sh.slab + (int64_t(s) * M + row) * OC + c0;
        __hip_atomic_store(dst, v0[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(dst + 1, v1[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);                          // this wave's partial stores have completed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();                                        // ... and every other wave's
    int* flag = reinterpret_cast<int*>(lds);
    if (threadIdx.x == 0)
      *flag = __hip_atomic_fetch_add(sh.counters + blk, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int old = *flag;
    if (old != sh.S - 1) return;                            // not the last split of this block
#pragma unroll
    for (int t = 0; t < kRT; ++t) {
      const int row = out_row(t);
      if (row < M) {
        v0[t] = v1[t] = 0.f;
        for (int sp = 0; sp < sh.S; ++sp) {
          float* src = sh.slab + (int64_t(sp) * M + row) * OC + c0;
          v0[t] += __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          v1[t] += __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    if (threadIdx.x == 0) __hip_atomic_store(sh.counters + blk, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- 6. output Hadamard-128, (the row scale on the 8-bit path,) rout * s_out, bf16 into the slice
#pragma unroll
  for (int t = 0; t < kRT; ++t) {
    const int row = out_row(t);
    if (row < M) {
      float x0 = v0[t], x1 = v1[t];
      had128_wave(x0, x1, lane);
      if constexpr (I8) {
        float rs = rsc[0];
#pragma unroll
        for (int m = 1; m < kMR; ++m) rs = row == m ? rsc[m] : rs;
        x0 *= rs;
        x1 *= rs;
      } else if (sh.sc) {
        const float rs = sh.sc[row];
        x0 *= rs;
        x1 *= rs;
      }
      x0 = x0 * kInvSqrt128 * f16_to_f32(sh.rout[c0]) * f16_to_f32(sh.s_out[c0]);
      x1 = x1 * kInvSqrt128 * f16_to_f32(sh.rout[c0 + 1]) * f16_to_f32(sh.s_out[c0 + 1]);
      uint16_t* dst = a.out + int64_t(row) * a.ldo + sh.col0 + c0;
      if (((a.ldo | sh.col0) & 1) == 0) {
        *reinterpret_cast<uint32_t*>(dst) = f32_to_bf16(x0) | (f32_to_bf16(x1) << 16);
      } else {
        dst[0] = (uint16_t)f32_to_bf16(x0);
        dst[1] = (uint16_t)f32_to_bf16(x1);
      }
    }
  }
}

template <int KSET, int SPW, int MR, bool SILU = false, int RG = 1, bool I8 = false>
__global__ __launch_bounds__(512, 4) void decode_kernel(DecArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int wg = blockIdx.x;
  // The block's shard, and every kernel argument the block reads, in two batches of scalar loads: the
  // first read of an argument line is a memory round trip, and requested at first use (or through a
  // search loop) they form a chain of them before the first weight load.
  int i = 0;
#pragma unroll
  for (int j = 1; j < kMaxShards; ++j)   // shards are in grid order; +1 when wgb[j] <= wg (scalar ALU only)
    i += int(uint32_t(a.wgb[j] - wg - 1) >> 31);
  const DecShard& sh = a.sh[i];
  asm volatile("" ::"s"(a.x), "s"(a.out), "s"(a.ldo), "s"(a.M), "s"(a.IC), "s"(a.lds_row), "s"(a.tr_off));
  asm volatile("" ::"s"(sh.code), "s"(sh.xf), "s"(sh.sc), "s"(sh.part), "s"(sh.s_in), "s"(sh.rin), "s"(sh.rout),
               "s"(sh.s_out), "s"(sh.slab), "s"(sh.counters), "s"(sh.col0), "s"(sh.code_bytes), "s"(sh.OC),
               "s"(sh.K), "s"(sh.S), "s"(sh.wg_begin));
  const int local = wg - sh.wg_begin;
  if constexpr (KSET >= 1 && KSET <= 8) {
    decode_block<KSET, SPW, MR, SILU, RG, I8>(a, sh, local, lds);
  } else {   // KSET 0: the mixed set {2, 3, 4}
    switch (sh.K) {
      case 2: decode_block<2, SPW, MR, false, RG, I8>(a, sh, local, lds); break;
      case 3: decode_block<3, SPW, MR, false, RG, I8>(a, sh, local, lds); break;
      default: decode_block<4, SPW, MR, false, RG, I8>(a, sh, local, lds); break;
    }
  }
}

// ---------------------------------------------------------------------------------------------------
// Host side: plan and launch
// ---------------------------------------------------------------------------------------------------
namespace {

int spw_variant(int need) { return need <= 2 ? 2 : 4; }
constexpr int kMaxSpw = 4;     // wider variants exceed the 128 registers a 1024-thread block allows

// K whose staging slots size the LDS: the mixed-K launch serves {2, 3, 4} with one layout, so any shard of
// K <= 4 is planned with K = 4's slots (a shard's plan must not depend on the other shards of a call).
int lds_k(int K) { return K <= 4 ? 4 : K; }

size_t tr_offset(int M, int lds_row) { return (size_t(M + 1) * lds_row * 2 + 15) / 16 * 16; }

size_t slot_bytes(int K) { return size_t(4) * (256 * K + 64); }

// LDS of one block: rotated activations, then the waves' trellis staging slots; the reduction buffer
// reuses the same space after the main loop.
size_t lds_bytes_for(int M, int lds_row, int K) {
  const int Mg = M < kDecodeMaxRows ? M : kDecodeMaxRows;   // the reduction runs one 16-row group at a time
  const size_t main = tr_offset(M, lds_row) + size_t(kWaves) * slot_bytes(lds_k(K));
  const size_t red = size_t(kWaves) * Mg * kHad * 4;
  return main > red ? main : red;
}

}  // namespace

// Splits of one shard's feature range.  A function of (M, IC, OC, K) alone -- never of the other shards
// in the call -- so a merged call reduces every shard in the same order as a call of that shard by
// itself and the two agree bit for bit.  Split only as far as needed: until the shard has kFillBlocks blocks
// (C1's 14336-column shards reach it at S = 2: 448 blocks, two per CU), a wave's steps fit the
// largest unrolled variant, and the activation slice fits in LDS.
constexpr int kFillBlocks = 224;

int shard_splits(int64_t M, int B, int nblk, int K) {
  // rows of one 16-row group: a launch of 17..32 rows (two groups) splits a shard exactly as 16 rows do
  const int Mg = int(M < kDecodeMaxRows ? M : kDecodeMaxRows);
  for (int S = 1;; ++S) {
    if (S >= B) return B;
    const int nb_max = (B + S - 1) / S;
    const int spw_need = 2 * ((nb_max + kWaves - 1) / kWaves);   // whole Hadamard blocks per wave
    const bool lds_ok = lds_bytes_for(Mg, kHad * nb_max + 8, K) <= kMaxLds;
    if (spw_need <= kMaxSpw && lds_ok && (nblk * S >= kFillBlocks || nb_max <= kWaves)) return S;
  }
}

bool plan_decode(int64_t M, int64_t IC, int n, const DecShardIn* in, DecPlan* pl, bool pre) {
  if (M < 1 || M > kDecodeLaunchRows || n < 1 || n > kMaxShards) return false;
  const int B = int(IC / kHad);
  int nb_max = 1;
  for (int i = 0; i < n; ++i) {
    pl->S[i] = shard_splits(M, B, int(in[i].OC / kHad), in[i].K);
    const int nb = (B + pl->S[i] - 1) / pl->S[i];
    nb_max = nb > nb_max ? nb : nb_max;
  }
  pl->spw = spw_variant(2 * ((nb_max + kWaves - 1) / kWaves));
  int kmax = 1;
  for (int i = 0; i < n; ++i) kmax = in[i].K > kmax ? in[i].K : kmax;
  pl->pre = pre || M >= kPreRotateRows;
  pl->lds_row = pl->pre ? 0 : kHad * nb_max + 8;
  pl->tr_off = int(tr_offset(int(M), pl->lds_row));
  pl->lds_bytes = lds_bytes_for(int(M), pl->lds_row, kmax);
  if (pl->lds_bytes > kMaxLds) return false;
  // heavier shards (larger K) first: blocks are dispatched in index order
  int order[kMaxShards];
  for (int i = 0; i < n; ++i) order[i] = i;
  for (int i = 1; i < n; ++i)
    for (int j = i; j > 0 && in[order[j]].K > in[order[j - 1]].K; --j) std::swap(order[j], order[j - 1]);
  int wg = 0;
  size_t slab = 0;
  int counters = 0;
  for (int r = 0; r < n; ++r) {
    const int i = order[r];
    const int S = pl->S[i];
    pl->order[r] = i;
    pl->wg_begin[r] = wg;
    wg += int(in[i].OC / kHad) * S;
    if (S > 1) {
      pl->slab_off[r] = slab;
      slab += size_t(S) * size_t(M) * size_t(in[i].OC) * sizeof(float);
      pl->counter_off[r] = counters;
      counters += int(in[i].OC / kHad);
    } else {
      pl->slab_off[r] = 0;
      pl->counter_off[r] = 0;
    }
  }
  pl->wg_total = wg;
  pl->slab_bytes = slab;
  pl->counters = counters;
  bool all_same = true;
  for (int i = 1; i < n; ++i) all_same &= in[i].K == in[0].K;
  bool mixed234 = true;
  for (int i = 0; i < n; ++i) mixed234 &= in[i].K >= 2 && in[i].K <= 4;
  pl->kset = all_same ? in[0].K : (mixed234 ? 0 : -1);
  return counters <= kCounterSlots;
}

template <int KSET, int MR, bool SILU = false, int RG = 1, bool I8 = false>
static void launch_kset_mr(const DecPlan& pl, const DecArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)pl.wg_total), block(kWaves * 64);
  const size_t lds = pl.lds_bytes;
  if (pl.spw <= 2)
    hipLaunchKernelGGL((decode_kernel<KSET, 2, MR, SILU, RG, I8>), grid, block, lds, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<KSET, 4, MR, SILU, RG, I8>), grid, block, lds, stream, a);
}

template <int KSET>
static hipError_t launch_kset(const DecPlan& pl, const DecArgs& a, hipStream_t stream, bool silu, bool i8) {
  // the 8-bit path with in-block codes: launches of 1..4 rows without pre-rotation
  if (i8) {
    if (silu || pl.pre || a.M > 4) return hipErrorInvalidValue;
    if (a.M <= 1)
      launch_kset_mr<KSET, 1, false, 1, true>(pl, a, stream);
    else
      launch_kset_mr<KSET, 4, false, 1, true>(pl, a, stream);
    return hipGetLastError();
  }
  // the folded MLP activation: single-shard launches of 1..4 rows with in-block rotation only
  if (silu) {
    if constexpr (KSET >= 1 && KSET <= 8) {
      if (pl.pre || a.M > 4) return hipErrorInvalidValue;
      if (a.M <= 1)
        launch_kset_mr<KSET, 1, true>(pl, a, stream);
      else
        launch_kset_mr<KSET, 4, true>(pl, a, stream);
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  }
  // activation rows the fused pre-pass loads unconditionally: 1, 4 or 16; 0 = pre-rotated activations
  // (two 16-row groups above 16 rows)
  if (pl.pre && a.M > kDecodeMaxRows)
    launch_kset_mr<KSET, 0, false, 2>(pl, a, stream);
  else if (pl.pre)
    launch_kset_mr<KSET, 0>(pl, a, stream);
  else if (a.M <= 1)
    launch_kset_mr<KSET, 1>(pl, a, stream);
  else if (a.M <= 4)
    launch_kset_mr<KSET, 4>(pl, a, stream);
  else
    launch_kset_mr<KSET, 16>(pl, a, stream);
  return hipGetLastError();
}

hipError_t launch_decode(const DecPlan& pl, const void* x, int64_t M, int64_t IC, int n, const DecShardIn* in,
                         void* out, int64_t ldo, float* slab, int* counters, hipStream_t stream, bool silu, bool i8) {
  if (pl.kset < 0) return hipErrorInvalidValue;
  DecArgs a;
  a.x = (const uint16_t*)x;
  a.out = (uint16_t*)out;
  a.ldo = ldo;
  a.M = (int)M;
  a.IC = (int)IC;
  a.n_shards = n;
  a.lds_row = pl.lds_row;
  a.tr_off = pl.tr_off;
  for (int r = 0; r < kMaxShards; ++r) a.wgb[r] = r < n ? pl.wg_begin[r] : INT_MAX;
  for (int r = 0; r < n; ++r) {
    const DecShardIn& s = in[pl.order[r]];
    DecShard& d = a.sh[r];
    d.code = (const uint32_t*)s.code;
    d.xf = (const uint16_t*)s.xf;
    d.sc = s.sc;
    d.part = s.part;
    if (i8 && !s.part) return hipErrorInvalidValue;
    d.s_in = (const uint16_t*)s.s_in;
    d.rin = (const uint16_t*)s.rin;
    d.rout = (const uint16_t*)s.rout;
    d.s_out = (const uint16_t*)s.s_out;
    d.slab = slab + pl.slab_off[r] / sizeof(float);
    d.counters = counters + pl.counter_off[r];
    d.col0 = s.col0;
    d.code_bytes = uint32_t(IC / 16 * (s.OC / 16) * 32 * s.K);
    d.OC = (int)s.OC;
    d.K = s.K;
    d.S = pl.S[pl.order[r]];
    d.wg_begin = pl.wg_begin[r];
  }
  switch (pl.kset) {
    case 0: return launch_kset<0>(pl, a, stream, silu, i8);
    case 1: return launch_kset<1>(pl, a, stream, silu, i8);
    case 2: return launch_kset<2>(pl, a, stream, silu, i8);
    case 3: return launch_kset<3>(pl, a, stream, silu, i8);
    case 4: return launch_kset<4>(pl, a, stream, silu, i8);
    case 5: return launch_kset<5>(pl, a, stream, silu, i8);
    case 6: return launch_kset<6>(pl, a, stream, silu, i8);
    case 7: return launch_kset<7>(pl, a, stream, silu, i8);
    case 8: return launch_kset<8>(pl, a, stream, silu, i8);
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
