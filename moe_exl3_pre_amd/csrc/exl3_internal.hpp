// Internal interface between the C ABI (exl3_api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace exl3 {

constexpr int kCounterSlots = 4096;     // split-K block counters at the head of every workspace
constexpr size_t kCounterBytes = kCounterSlots * sizeof(int);
constexpr size_t kAlign = 256;
constexpr int kMaxShards = 16;
constexpr size_t kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950
constexpr int kDecodeMaxRows = 16;      // rows of one MFMA row group of the decode-phase kernel
constexpr int kDecodeLaunchRows = 32;   // rows one decode-phase launch covers (two groups, pre-rotated)
// Decode-phase launches of at least this many rows take activations rotated once per call by the
// fragment-major pre-pass instead of rotating them in every block.  The separate launch costs ~4 us; the
// in-block rotation grows with the rows (gate_up IC=4096 at M = 4 / 5: 19.0 / 20.9 us in-block against
// 20.0 / 20.3 us pre-rotated, measured on one box).
constexpr int kPreRotateRows = 5;

inline size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }

// One shard as the decode-phase planner sees it.
struct DecShardIn {
  const int16_t* code;
  int64_t OC;
  int K;
  int64_t col0;
  const void *s_in, *rin, *rout, *s_out;
  const void* xf = nullptr;   // decode phase, pre-rotated launches: this shard's fragment-major activations
  const float* sc = nullptr;  // decode phase, 8-bit path: the launch rows' scales (xf then holds the codes)
  const float* part = nullptr;  // decode phase, 8-bit path with in-block codes (1..4 rows): the rows' block maxima
};

struct DecPlan {
  int S[kMaxShards];        // per shard: blocks per 128-column output block along the input features
  int spw;                  // unrolled 64-feature steps per wave (1, 2, 4, 8)
  int lds_row;              // halves per activation row in LDS
  int tr_off;               // LDS byte offset of the trellis staging slots
  size_t lds_bytes;         // dynamic LDS per block
  int kset;                 // kernel K set: 1..8 single K, 0 mixed {2,3,4}, -1 unsupported mix
  bool pre;                 // activations pre-rotated once per launch (M >= kPreRotateRows, or forced)
  int order[kMaxShards];    // shard processed in grid position r
  int wg_begin[kMaxShards];
  size_t slab_off[kMaxShards];
  int counter_off[kMaxShards];
  int wg_total;
  size_t slab_bytes;        // split-K slab (0 when S == 1)
  int counters;             // counter slots used
};

// Plans one decode-phase launch of M <= 32 rows over n shards (above 16 rows with pre-rotated
// activations); false if it cannot be served.  pre: read pre-rotated activations at any M (the 8-bit
// path, whose codes need the row's maximum over all input features first).
bool plan_decode(int64_t M, int64_t IC, int n, const DecShardIn* in, DecPlan* pl, bool pre = false);
// silu: x is a dense MLP block's gate_up output [M, 2 IC] and the activation bf16(silu(g) * u) is formed in the
// in-block pre-pass (one shard, 1..4 rows, no pre-rotation; otherwise hipErrorInvalidValue).
// i8: the 8-bit path with in-block codes (1..4 rows, no pre-rotation; every shard's `part` set).
hipError_t launch_decode(const DecPlan& pl, const void* x, int64_t M, int64_t IC, int n, const DecShardIn* in,
                         void* out, int64_t ldo, float* slab, int* counters, hipStream_t stream, bool silu = false,
                         bool i8 = false);

// permuted: fragment-major, with 16-row fragments (the decode-phase kernel's operand) or with rows32 the
// 32-row fragments of the prefill GEMM (k_gemm.hip), rows past M written as zeros up to the next multiple
// of 16 (32); else natural row-major, rows [M, M_pad) written as zeros.
hipError_t launch_prepass_f16(const void* x, const void* s_in, const void* rin, void* xh, int64_t M, int64_t IC,
                              bool permuted, hipStream_t stream, int64_t M_pad = 0, bool rows32 = false);
// Natural layout: q receives int8 codes.  permuted with f16_codes: the same codes as fp16 numbers in the
// fragment-major layout (16- or, with rows32, 32-row fragments), which needs part, M * (IC / 128) floats of
// scratch.  Other combinations are rejected.
// The per-(row, 128-block) max |xh| of the fragment-major 8-bit pre-pass alone, into part [M, IC / 128]
// (the decode-phase kernel forms the codes of 1..4 rows itself).
hipError_t launch_prepass_amax(const void* x, const void* s_in, const void* rin, float* part, int64_t M, int64_t IC,
                               hipStream_t stream);
hipError_t launch_prepass_i8(const void* x, const void* s_in, const void* rin, void* q, float* scale, int64_t M,
                             int64_t IC, bool permuted, hipStream_t stream, bool f16_codes = false,
                             float* part = nullptr, bool rows32 = false);
hipError_t launch_decode_tiles(void* w, const int16_t* code, int64_t IC, int64_t OC, int K, hipStream_t stream);
// K split of the prefill GEMM.  One wave owns a 128 x 128 output tile, a block is 4 waves (128 rows x 512
// columns) and the chip holds 256 blocks (1024 waves) at a time.  A shard with fewer than 1024 tiles has
// its 64-feature steps split so that about 1024 waves run, each split keeping at least 8 steps (an even
// count), and a second launch sums the splits' partial tiles.  A larger shard whose blocks leave the last
// round of 256 at most half full runs that round's blocks (tail_blocks, the last ones) split
// tail_splits ways instead, so the round takes 1/tail_splits of the time; the other blocks run unsplit.
constexpr int kChipBlocks = 256;

struct GemmSplit {
  int splits;            // 1: no split of the whole shard
  int sps;               // steps per split (the last split may have fewer; every count is even)
  int tail_blocks = 0;   // blocks of the partial last round run split (0: none)
  int tail_splits = 1;
  int tail_sps = 0;
};

inline GemmSplit gemm_split(int64_t M, int64_t IC, int64_t OC) {
  const int64_t steps = IC / 64, tiles = (M + 127) / 128 * (OC / 128);
  int64_t s = tiles > 0 ? 1024 / tiles : 1;
  if (s > steps / 8) s = steps / 8;
  if (s > 1) {
    const int64_t sps = 2 * ((steps + 2 * s - 1) / (2 * s));
    const int64_t n = (steps + sps - 1) / sps;
    if (n > 1) return GemmSplit{int(n), int(sps)};
  }
  GemmSplit g{1, int(steps)};
  const int64_t blocks = (M + 127) / 128 * ((OC + 511) / 512);
  const int64_t r = blocks % kChipBlocks;
  if (blocks > kChipBlocks && r > 0) {
    int64_t ts = kChipBlocks / r;
    if (ts > steps / 8) ts = steps / 8;
    if (ts > 1) {
      const int64_t sps = 2 * ((steps + 2 * ts - 1) / (2 * ts));
      const int64_t n = (steps + sps - 1) / sps;
      if (n > 1) {
        g.tail_blocks = int(r);
        g.tail_splits = int(n);
        g.tail_sps = int(sps);
      }
    }
  }
  return g;
}

// Partial-sum slab of a split GEMM: one 64 KB fp32 tile per (split, block, wave) of the split launch.
inline size_t gemm_slab_bytes(int64_t M, int64_t OC, GemmSplit sp) {
  const size_t blocks = size_t((M + 127) / 128) * size_t((OC + 511) / 512);
  if (sp.splits > 1) return size_t(sp.splits) * blocks * 4 * 65536;
  if (sp.tail_splits > 1) return size_t(sp.tail_splits) * size_t(sp.tail_blocks) * 4 * 65536;
  return 0;
}

// Prefill-phase GEMM of one shard (one wave per 128 x 128 output tile); xf is the pre-pass output in the
// 32-row fragment-major layout (rows padded to 32).  With row_scale (8-bit path) every output row is multiplied
// by row_scale[row] before the output transform.  split.splits > 1 needs slab (gemm_slab_bytes).
hipError_t launch_gemm(const void* xf, const int16_t* code, int K, const void* rout, const void* s_out, void* out,
                       int64_t ldo, int64_t col0, int64_t M, int64_t IC, int64_t OC, hipStream_t stream,
                       const float* row_scale, GemmSplit split, float* slab);

// ---- MoE expert bank
constexpr int kMoeMaxGroups = 64;
constexpr int kMoeMaxExperts = 1024;    // the route sort keeps one slot per thread of one workgroup

struct MoeLaunch {
  const void* x;
  const int32_t* ids;
  const float* wts;
  const int32_t* perm;
  const void *w13, *w2, *w13_suh, *w13_svh, *w2_suh, *w2_svh;
  const int64_t *off_w1, *off_w3, *off_w2;
  void* out;
  // workspace regions
  int32_t* offs;
  int32_t* pslot;
  int32_t* rows;
  int32_t* chunks;          // int32 x 4 per chunk
  int32_t* n_chunks;
  void* xh13;
  void* ah;
  float* o;
  int64_t T;
  int topk, E, H, I, n_groups;
  int g_hi[kMoeMaxGroups];  // exclusive end slot of each group
  int g_k[kMoeMaxGroups];   // k_gu | k_d << 8
  int plan = 0;             // 0: by size, 1: the decode-sized plan (32-row chunks), 2: the prefill plan
};

// The prefill plan (grouped 64-row x 128-column tiles) serves calls with at least this many routed pairs
// per expert on average, when the gathered operands stay under 2 GiB.
constexpr int kMoePrefillPairsPerExpert = 128;
bool moe_prefill_plan(int64_t P, int E, int H, int I, int plan);
// Row pitch (halves) of the per-pair fp16 operands (w1 / w3 rotated activations: n = H; w2's operand:
// n = I).  The expert kernels gather these rows by pair id, one row per lane; at a pitch of a power of two
// every row of a load falls in the same L1 set and the loads serialise on tag conflicts, so each row is
// padded by one 128-byte line.
inline int moe_row_pitch(int n) { return n + 64; }
int64_t moe_max_chunks(int64_t P, int E);
hipError_t launch_moe(const MoeLaunch& m, hipStream_t stream);

// ---- measurement hooks (k_probe.hip): a streaming read and back-to-back MFMAs, for measured peaks
hipError_t launch_probe_read(const void* src, size_t bytes, uint32_t* sink, int blocks, int variant,
                             hipStream_t stream);
hipError_t launch_probe_mfma(float* sink, int kind, int iters, int blocks, hipStream_t stream);

}  // namespace exl3
