// Device-side building blocks shared by every EXL3 kernel on gfx950 (CDNA4, wave64).
//
//  * the trellis column decode: one lane turns the words of one 16x16 tile column into the 16 fp16
//    weights of that column, packed two per register in the MFMA operand order used everywhere;
//  * the wave-wide Hadamard-128 (two features per lane);
//  * small conversions (bf16/fp16) and the MFMA wrappers.
//
// Trellis layout ("radiance_escha.py", `_TILE = 16`: code is [IC/16, OC/16, 16K]; the kernels see the
// words as little-endian uint32, `process_weights_after_loading`).  In a tile, state i is the 16-bit
// window at stream bit i*K (circular), and lands on in-tile row i % 16 (input feature) and column i / 16
// (output feature).  Column c therefore owns states 16c .. 16c+15, i.e. stream bits [16cK, 16cK + 15K + 16).
//
// Operand order.  A 16x16x32 fp16 MFMA takes 8 k-values per lane.  A lane that decodes tile column c
// produces the 16 k-values (tile rows 0..15) of that column as 8 registers; register p holds
// (row p, row p + 8) in its (low, high) halves.  Registers 0..3 feed one MFMA and 4..7 the next, so the
// k-slots of the two MFMAs visit the tile rows in the order
//     PERM16 = [0, 8, 1, 9, 2, 10, 3, 11 | 4, 12, 5, 13, 6, 14, 7, 15].
// The activation pre-pass stores the rotated activations in that order inside every 16-feature group,
// so A fragments are plain 16-byte loads.  A reduction over k does not care about the order, and the
// same order is used for every K.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace exl3 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kHad = 128;    // "radiance_escha.py" `_HAD`
constexpr int kTile = 16;    // "radiance_escha.py" `_TILE`
constexpr float kInvSqrt128 = 0.08838834764831845f;
// Buffer resource word 3 for raw (untyped) dword loads on gfx9-family parts.
constexpr int kBufferFlags = 0x00020000;

// Position of tile row r inside the permuted 16-group (inverse of PERM16).
__host__ __device__ constexpr int perm16_pos(int r) { return r < 8 ? 2 * r : 2 * (r - 8) + 1; }

// Feature pair a lane transforms when the rotated activations are written in PERM16 order: lane l takes
// features f = 16*(l/8) + l%8 and f + 8 of its 128-block.  PERM16 puts exactly that pair at positions
// 2l, 2l+1, so each lane writes one contiguous 4-byte word.  The Hadamard is unchanged: lane bits 0..2
// are feature bits 0..2, lane bits 3..5 are feature bits 4..6 (monotone), and the in-lane pair is
// feature bit 3 with the lower feature in v0.
__device__ __forceinline__ int perm_pair_feature(int lane) { return 16 * (lane >> 3) + (lane & 7); }

template <int K>
struct Geom {
  static_assert(K >= 1 && K <= 8, "K must be 1..8");
  static constexpr int kWords = 8 * K;                                   // uint32 words per tile
  static constexpr int kSpan = 15 * K + 16;                              // bits a column needs
  static constexpr int kNW = (((K & 1) ? 16 : 0) + kSpan + 31) / 32;      // words loaded per column
  static constexpr int kNR = (kSpan + 31) / 32;                          // words after realignment
};

// Word offsets (within a tile) a lane must load for tile column c, and the column's bit shift in the
// first of them (0, or 16 for odd c when K is odd).
template <int K>
__device__ __forceinline__ void column_word_offsets(int c, int (&woff)[Geom<K>::kNW], int& shift) {
  const int w0 = (c * K) >> 1;
  shift = (K & 1) ? ((c & 1) << 4) : 0;
#pragma unroll
  for (int j = 0; j < Geom<K>::kNW; ++j) {
    int w = w0 + j;
    woff[j] = w >= Geom<K>::kWords ? w - Geom<K>::kWords : w;   // tail-biting wrap
  }
}

// Bits [o, o+16) of the realigned column stream r (valid in the low 16 bits of the result).
template <int K, int O>
__device__ __forceinline__ uint32_t window16(const uint32_t (&r)[Geom<K>::kNR]) {
  constexpr int q = O >> 5, sh = O & 31;
  if constexpr (sh == 0) {
    return r[q];
  } else if constexpr (sh <= 16) {
    return r[q] >> sh;
  } else {
    return __builtin_amdgcn_alignbit(r[q + 1], r[q], sh);
  }
}

// A pointer or size that is the same in every lane of the wave, moved to scalar registers where the
// compiler can see that.  A buffer resource built from a value it must treat as varying across lanes
// (one derived from the wave index, threadIdx.x / 64) is otherwise wrapped, at every buffer access, in a
// loop over the distinct values of the active lanes (four readfirstlane, two compares, an exec-mask loop).
// The builtin takes and returns a signed int: each half goes back through uint32_t before it is widened,
// or a low half with bit 31 set would sign-extend into the high half of the address.
template <class T>
__device__ __forceinline__ T* wave_uniform(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(v))));
  const uint64_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(v >> 32))));
  return reinterpret_cast<T*>(lo | (hi << 32));
}
__device__ __forceinline__ uint32_t wave_uniform(uint32_t x) {
  return uint32_t(__builtin_amdgcn_readfirstlane(int(x)));
}

// A 32-bit constant in a scalar register that the compiler cannot see through.  The asm writes only
// a scalar register: vector outputs of inline asm are avoided, because the compiler inserts no wait
// states around inline asm for the matrix cores, and a vector register it picks for an asm output could
// be one that an MFMA still in flight reads or writes.
template <uint32_t V>
__device__ __forceinline__ uint32_t opaque_sgpr() {
  uint32_t x;
  asm("s_mov_b32 %0, %1" : "=s"(x) : "n"(V));
  return x;
}

// Constants of the codebook held in registers.  gfx9 VOP3 encodings cannot carry literals, so with
// literal operands the compiler splits the mask-and-or into two instructions; opaque register values
// let it select a single v_and_or_b32.  That instruction reads at most one scalar register, so the bias
// must be in a vector register: or-ing in the thread index masked by an opaque zero makes it a per-lane
// value, which the compiler builds (once per kernel) in one of its own choosing.
struct CodebookRegs {
  uint32_t mask;   // 0x8F808F80 (scalar register)
  uint32_t bias;   // 0x30003000 (vector register)
};

__device__ __forceinline__ CodebookRegs codebook_regs() {
  const uint32_t bias = opaque_sgpr<0x30003000u>() | (__builtin_amdgcn_workitem_id_x() & opaque_sgpr<0u>());
  return CodebookRegs{opaque_sgpr<0x8F808F80u>(), bias};
}

// State -> fp16 bit pattern for two states at once:  ((s * 0x9E37) mod 2^16) & 0x8F80 | 0x3000.
__device__ __forceinline__ uint32_t codebook2(uint32_t states, const CodebookRegs& c) {
  u16x2 s = __builtin_bit_cast(u16x2, states);
  s = s * (u16x2){0x9E37, 0x9E37};
  return (__builtin_bit_cast(uint32_t, s) & c.mask) | c.bias;
}

// PAIR64 selects the 64-bit-shift form below.  It saves VALU wherever registers are not scarce; where a
// kernel already fills the register file (the prefill GEMM at K >= 4) the 32-bit form is kept, because the
// aligned register pairs the 64-bit shift needs would spill.
template <int K, int P, bool PAIR64>
__device__ __forceinline__ constexpr bool pair_fits64() {
  constexpr int kA = P * K, kJ = kA >> 5, kSh = kA & 31;
  return PAIR64 && K != 2 && kJ + 1 < Geom<K>::kNR && kSh + 8 * K + 16 <= 64;
}

// q >> D in one v_lshrrev_b64 (full rate on gfx950).  The amount comes from an opaque scalar register:
// with a literal amount the compiler splits the shift into two 32-bit funnel shifts when only some bytes
// of the result are used.
template <int D>
__device__ __forceinline__ uint64_t shr64(uint64_t q) {
  if constexpr (D == 0) return q;
  else return q >> opaque_sgpr<uint32_t(D)>();
}

// Pair P of a tile column: rows (P, P+8).  States p and p+8 start 8K bits (K bytes) apart.  When both fit
// one 64-bit window of the realigned stream, the window q is shifted so that state p sits at bit 0 and one
// byte permute picks bytes (0, 1) and (K, K+1); consecutive pairs of the same window continue from the
// previous pair's shifted q (a shift by K), so every pair costs one shift.  Otherwise each state gets its
// own 32-bit window.
template <int K, int P, bool PAIR64>
__device__ __forceinline__ uint32_t decode_pair(const uint32_t (&r)[Geom<K>::kNR], uint64_t& q, const CodebookRegs& c) {
  constexpr int kA = P * K, kJ = kA >> 5, kSh = kA & 31;
  if constexpr (K == 2) {
    // state p at bit 2p, state p+8 at bit 2p+16: one 32-bit window holds both.
    return codebook2(P == 0 ? r[0] : __builtin_amdgcn_alignbit(r[1], r[0], 2 * P), c);
  } else if constexpr (pair_fits64<K, P, PAIR64>()) {
    constexpr int kAp = (P - 1) * K;
    if constexpr (P > 0 && pair_fits64<K, P - 1, PAIR64>() && (kAp >> 5) == kJ)
      q = shr64<kSh - (kAp & 31)>(q);
    else
      q = shr64<kSh>((uint64_t(r[kJ + 1]) << 32) | r[kJ]);
    constexpr uint32_t kSel = 0x0100u | (uint32_t(K) << 16) | (uint32_t(K + 1) << 24);
    return codebook2(__builtin_amdgcn_perm(uint32_t(q >> 32), uint32_t(q), kSel), c);
  } else {
    const uint32_t lo = window16<K, P * K>(r);
    const uint32_t hi = window16<K, (P + 8) * K>(r);
    return codebook2(__builtin_amdgcn_perm(hi, lo, 0x05040100u), c);   // lo[15:0] | hi[15:0] << 16
  }
}

// Decode one tile column from the words loaded at column_word_offsets: out[p] = (row p, row p+8).
template <int K, bool PAIR64 = true>
__device__ __forceinline__ void decode_column(const uint32_t (&w)[Geom<K>::kNW], int shift, uint32_t (&out)[8],
                                              const CodebookRegs& c) {
  uint32_t r[Geom<K>::kNR];
  if constexpr (K & 1) {
#pragma unroll
    for (int j = 0; j < Geom<K>::kNR; ++j) r[j] = __builtin_amdgcn_alignbit(w[j + 1], w[j], shift);
  } else {
#pragma unroll
    for (int j = 0; j < Geom<K>::kNR; ++j) r[j] = w[j];
  }
  uint64_t q = 0;   // the current 64-bit window, carried from pair to pair
  out[0] = decode_pair<K, 0, PAIR64>(r, q, c);
  out[1] = decode_pair<K, 1, PAIR64>(r, q, c);
  out[2] = decode_pair<K, 2, PAIR64>(r, q, c);
  out[3] = decode_pair<K, 3, PAIR64>(r, q, c);
  out[4] = decode_pair<K, 4, PAIR64>(r, q, c);
  out[5] = decode_pair<K, 5, PAIR64>(r, q, c);
  out[6] = decode_pair<K, 6, PAIR64>(r, q, c);
  out[7] = decode_pair<K, 7, PAIR64>(r, q, c);
}

// Staging of trellis words.  The words of one 64-feature step of a 128-column block are 4 tile rows x
// 8 tiles x 8K words, each tile row 256K contiguous bytes: lane (n, g) loads 16 bytes at n * 16 + i * 256
// of tile row g (i < K), fully coalesced.  A per-wave LDS slot holds that step, each tile row padded by
// 16 words so the four groups of 16 lanes read different banks; lane (n, g) then reads the words of tile
// column n of each tile of row g at column_word_offsets.
template <int K>
struct Slot {
  static constexpr int kRowBytes = 256 * K + 64;
  static constexpr int kBytes = 4 * kRowBytes;
};

// The kernels hand data between the lanes of one wave through LDS without a barrier: staged trellis
// words, rotated activations.  The hardware executes one wave's LDS operations in order, so a lane's
// read after the other lanes' writes sees them; but the compiler sees each lane as a thread of its own,
// for which another lane's store does not exist, so it may reuse a value it loaded earlier from an
// address this lane did not store to, or move this lane's store across loads of the other lanes' data.
// This compiler fence (no instruction) between every write phase and read phase forbids both.
__device__ __forceinline__ void lane_exchange_fence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

__device__ __forceinline__ half8 as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}

__device__ __forceinline__ float4v mfma16(half8 a, half8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------------------------------
// Conversions
// ---------------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {   // round to nearest even; NaN stays NaN
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two values at once with the hardware conversion (round to nearest even, the default rounding mode; fp32
// denormals are kept): the same bits as f32_to_bf16 for every non-NaN input.  lo in bits 0..15.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v){lo, hi}, bf16x2v));
}

// Two values to fp16 at once (hardware conversion, round to nearest even): the same bits as f32_to_f16.
__device__ __forceinline__ uint32_t f32x2_to_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v){lo, hi}, half2v));
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__device__ __forceinline__ uint16_t f32_to_f16(float f) {   // round to nearest even
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// A rotated activation as the MFMAs take it: the fp32 Hadamard output times 1/sqrt(128), rounded to fp32,
// then to fp16 (nearest even).  Every rotation ends in this one sequence, so the pre-pass kernels and the
// decode kernel's in-block rotation give the same bits.  The empty asm statement (no instruction) makes
// the fp32 product a value the compiler cannot look through: otherwise it fuses product and conversion
// into one mixed-precision FMA that rounds once instead of twice, in some kernels and not in others.
__device__ __forceinline__ float rot_scale(float v) {
  float p = v * kInvSqrt128;
  __asm__("" : "+v"(p));
  return p;
}
__device__ __forceinline__ uint16_t rot_f16(float v) { return f32_to_f16(rot_scale(v)); }
__device__ __forceinline__ uint32_t rot_f16x2(float lo, float hi) {
  return f32x2_to_f16x2(rot_scale(lo), rot_scale(hi));
}

// ---------------------------------------------------------------------------------------------------
// Wave-wide orthonormal Hadamard-128: lane l holds features 2l (v0) and 2l+1 (v1) of one 128-block.
// Radix-2 butterflies in natural (Sylvester) order; of each pair the lower feature index takes a + b,
// the upper a - b.  The 1/sqrt(128) normalisation is applied by the caller.
// Partners across lanes come from DPP where the row patterns allow it (lane xor 1, 2 directly; xor 4
// and xor 8 as two mirrors), from ds_swizzle for xor 16 and from ds_bpermute for xor 32.
// ---------------------------------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kQuadXor3 = 0x1B;       // quad_perm [3,2,1,0]
constexpr int kRowMirror = 0x140;     // lane i <- lane 15 - i within each row of 16
constexpr int kRowHalfMirror = 0x141; // lane i <- lane 7 - i within each half-row of 8
constexpr int kRowRor8 = 0x128;       // lane i <- lane (i + 8) mod 16 within each row of 16 (= lane xor 8)

__device__ __forceinline__ float lane_xor4(float v) { return dpp<kRowHalfMirror>(dpp<kQuadXor3>(v)); }   // ^3 ^7
__device__ __forceinline__ float lane_xor8(float v) { return dpp<kRowMirror>(dpp<kRowHalfMirror>(v)); }  // ^7 ^15
__device__ __forceinline__ float lane_xor16(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));  // xor 16 in 32
}

// Butterfly with the partner value p: lower lanes get p + v, upper lanes p - v, written as
// fma(v, +-1, p) (exact: one rounding of the same sum) so the compiler can use v_fmac_f32 on the value the
// lane-exchange move produced.
__device__ __forceinline__ float bfly(float v, float p, bool upper) { return fmaf(v, upper ? -1.0f : 1.0f, p); }

// Lane-pair butterfly over lane bit 4 (resp. 5) for two values X, Y of every lane: after swapping the odd
// rows (halves) of X with the even ones of Y, the lower lane of each pair holds both X values and the
// upper lane both Y values, in the order (lower lane's, upper lane's); both form (a + b, a - b), and
// the same swap puts the four results back in place.
template <bool HALF32>
__device__ __forceinline__ void lane_pair_bfly(float& x, float& y) {
  uint32_t a = __float_as_uint(x), b = __float_as_uint(y);
  auto r = HALF32 ? __builtin_amdgcn_permlane32_swap(a, b, false, false)
                  : __builtin_amdgcn_permlane16_swap(a, b, false, false);
  const float p = __uint_as_float(r[0]), q = __uint_as_float(r[1]);
  auto t = HALF32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(p + q), __float_as_uint(p - q), false, false)
                  : __builtin_amdgcn_permlane16_swap(__float_as_uint(p + q), __float_as_uint(p - q), false, false);
  x = __uint_as_float(t[0]);
  y = __uint_as_float(t[1]);
}

// The same transform for the pre-pass lane layout (perm_pair_feature): lane l holds features
// f = 16*(l/8) + l%8 (v0) and f + 8 (v1).  Stages run in natural feature-bit order 0..6 (lane bits 0..2,
// the in-lane pair, lane bits 3..5), the order of the fragment-major pre-pass, so that the two produce the
// same fp32 sums bit for bit and a row's rotated activations do not depend on which pre-pass ran.
__device__ __forceinline__ void had128_wave_pairs8(float& v0, float& v1, int lane);

__device__ __forceinline__ void had128_wave(float& v0, float& v1, int lane) {
  float a = v0 + v1, b = v0 - v1;
  v0 = bfly(a, dpp<kQuadXor1>(a), lane & 1);
  v1 = bfly(b, dpp<kQuadXor1>(b), lane & 1);
  a = bfly(v0, dpp<kQuadXor2>(v0), lane & 2);
  b = bfly(v1, dpp<kQuadXor2>(v1), lane & 2);
  v0 = bfly(a, lane_xor4(a), lane & 4);
  v1 = bfly(b, lane_xor4(b), lane & 4);
  a = bfly(v0, lane_xor8(v0), lane & 8);
  b = bfly(v1, lane_xor8(v1), lane & 8);
  v0 = bfly(a, lane_xor16(a), lane & 16);
  v1 = bfly(b, lane_xor16(b), lane & 16);
  a = bfly(v0, __shfl_xor(v0, 32, 64), lane & 32);
  b = bfly(v1, __shfl_xor(v1, 32, 64), lane & 32);
  v0 = a;
  v1 = b;
}

__device__ __forceinline__ void had128_wave_pairs8(float& v0, float& v1, int lane) {
  float a = bfly(v0, dpp<kQuadXor1>(v0), lane & 1);   // feature bit 0
  float b = bfly(v1, dpp<kQuadXor1>(v1), lane & 1);
  v0 = bfly(a, dpp<kQuadXor2>(a), lane & 2);          // bit 1
  v1 = bfly(b, dpp<kQuadXor2>(b), lane & 2);
  a = bfly(v0, lane_xor4(v0), lane & 4);              // bit 2
  b = bfly(v1, lane_xor4(v1), lane & 4);
  v0 = a + b;                                          // bit 3: the lane's own pair
  v1 = a - b;
  a = bfly(v0, lane_xor8(v0), lane & 8);              // bit 4
  b = bfly(v1, lane_xor8(v1), lane & 8);
  v0 = bfly(a, lane_xor16(a), lane & 16);             // bit 5
  v1 = bfly(b, lane_xor16(b), lane & 16);
  a = bfly(v0, __shfl_xor(v0, 32, 64), lane & 32);    // bit 6
  b = bfly(v1, __shfl_xor(v1, 32, 64), lane & 32);
  v0 = a;
  v1 = b;
}

// Hadamard-128 over the columns of a 128-column tile held in the accumulators of 32x32 MFMAs:
// v[nb][r] is column 32 nb + (lane & 31) of one of the lane's rows (the rows do not matter).  Radix-2
// butterflies in natural order of the column bits -- lane bits 0..3 by DPP, lane bit 4 by lane-pair swaps,
// nb's two bits in registers -- each stage applied to all 64 values before the next so that the lane
// exchanges of different values fill each other's wait states.  The 1/sqrt(128) is left to the caller.
template <int S>
__device__ __forceinline__ float col_partner(float v) {
  if constexpr (S == 1) return dpp<kQuadXor1>(v);
  else if constexpr (S == 2) return dpp<kQuadXor2>(v);
  else if constexpr (S == 4) return lane_xor4(v);
  else return dpp<kRowRor8>(v);
}

template <int S>
__device__ __forceinline__ void col_stage(float (&v)[4][16], int lane) {
  float q[4][16];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) q[nb][r] = col_partner<S>(v[nb][r]);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) v[nb][r] = bfly(v[nb][r], q[nb][r], lane & S);
}

__device__ __forceinline__ void had128_cols32(float (&v)[4][16], int lane) {
  col_stage<1>(v, lane);
  col_stage<2>(v, lane);
  col_stage<4>(v, lane);
  col_stage<8>(v, lane);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) lane_pair_bfly<false>(v[nb][r], v[nb][r + 1]);
#pragma unroll
  for (int hb = 1; hb < 4; hb <<= 1)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      if (!(nb & hb))
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float lo = v[nb][r], hi = v[nb | hb][r];
          v[nb][r] = lo + hi;
          v[nb | hb][r] = lo - hi;
        }
}

__device__ __forceinline__ float16v mfma32(half8 a, half8 b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

}  // namespace exl3
