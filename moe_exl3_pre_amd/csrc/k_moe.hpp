// Shared by the MoE expert-bank kernels (k_moe.hip: route, rotation, the decode-sized plan and the
// combine; k_moe_tile.hip: the prefill plan's grouped tiles): the launch arguments and the mapping of
// workgroups to chunks.
#pragma once

#include <utility>

#include "exl3_device.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

constexpr int kTileRows = 64;    // rows per chunk of the prefill plan (one tile of rows)

struct MoeArgs {
  const uint16_t* x;        // bf16 [T, H]
  const int32_t* ids;       // [T * topk] logical expert ids
  const float* wts;         // [T * topk]
  const int32_t* perm;      // [E] logical -> slot
  const uint16_t* w13;      // flat int16 banks
  const uint16_t* w2;
  const uint16_t* w13_suh;  // fp16 [E, 2, H]
  const uint16_t* w13_svh;  // fp16 [E, 2, I]
  const uint16_t* w2_suh;   // fp16 [E, I]
  const uint16_t* w2_svh;   // fp16 [E, H]
  const int64_t* off_w1;    // int16-element offsets per slot
  const int64_t* off_w3;
  const int64_t* off_w2;
  uint16_t* out;            // bf16 [T, H]
  // workspace
  int32_t* offs;            // [E + 1] first row of each slot's list
  int32_t* pslot;           // [P] slot of each pair, -1 if dropped (written by the route)
  int32_t* rows;            // [P] pair ids sorted by slot
  int4v* chunks;            // [max_chunks] {slot, first row, rows, k_gu | k_d << 8}
  int32_t* n_chunks;        // [1]
  uint16_t* xh13;           // fp16 [2, P, ldx] rotated activations of w1 (0) and w3 (1), PERM16 order
  uint16_t* ah;             // fp16 [P, ldh] w2's rotated operand, PERM16 order
  float* o;                 // fp32 [P, H] expert outputs
  int T, topk, P, E, H, I, max_chunks;
  int ldx, ldh;             // row pitches of xh13 and ah (moe_row_pitch of H and of I)
  int chunk_rows;           // rows per chunk of a slot's list: 32 (decode-sized plan) or 128 (prefill plan)
  int n_groups;
  int g_hi[kMoeMaxGroups];  // group g covers slots [g_hi[g-1], g_hi[g])
  int g_k[kMoeMaxGroups];   // k_gu | k_d << 8
};

// Chunk c of the launch.  The route stores the table heaviest K group first (heavier groups sit at the end
// of the slot order, so entry 0 is the last slot's last chunk): the entry is requested together with the
// chunk count instead of after it.  Entries from the count up to max_chunks are stale and never used.
__device__ __forceinline__ bool moe_chunk(const MoeArgs& a, int c, int4v& ch) {
  const int n = a.n_chunks[0];
  ch = a.chunks[c < a.max_chunks ? c : a.max_chunks - 1];
  return c < n;
}

// Workgroup -> (chunk, column group).  Workgroups are dealt to the 8 XCDs round-robin (block id mod 8);
// XCD x takes the chunk runs x, x + 8, x + 16, ... of kChunkRun consecutive chunks each, with every column
// group of each chunk.  So the column groups of a chunk share its gathered activations in one L2, and the
// consecutive chunks of one expert mostly share its trellis words there too, while every XCD still gets
// a mix of the K groups.  The launch covers a multiple of 8 kChunkRun chunks (moe_chunk_slots).
constexpr int kChunkRun = 4;

__device__ __forceinline__ void moe_tile(int ncg, int& c, int& cg) {
  const int id = blockIdx.x, x = id & 7, y = id >> 3;
  cg = y % ncg;
  const int i = y / ncg;                                     // this XCD's i-th chunk
  c = ((i / kChunkRun) * 8 + x) * kChunkRun + i % kChunkRun;
}

// Chunk slots a launch covers for at most n chunks: a multiple of 8 kChunkRun, so that moe_tile maps the
// grid onto [0, slots) one to one.
inline int64_t moe_chunk_slots(int64_t n) { return (n + 8 * kChunkRun - 1) / (8 * kChunkRun) * (8 * kChunkRun); }

// KSET 0 covers the mixed set {2, 3, 4} in one launch (one switch per workgroup); KSET k in 1..8 serves
// the chunks of one K and skips the others, so any other mix runs as one launch per distinct K.
template <int KSET, typename F>
__device__ __forceinline__ void moe_dispatch(int k, F&& f) {
  if constexpr (KSET == 0) {
    switch (k) {
      case 2: f(std::integral_constant<int, 2>{}); break;
      case 3: f(std::integral_constant<int, 3>{}); break;
      case 4: f(std::integral_constant<int, 4>{}); break;
      default: break;
    }
  } else {
    if (k == KSET) f(std::integral_constant<int, KSET>{});
  }
}

// The prefill plan's passes (k_moe_tile.hip): pass 0 w13, pass 1 w2, for K set kset (0: {2, 3, 4});
// kslot: the per-wave trellis staging bytes of the set's largest K.
void launch_moe_tile_pass(const MoeArgs& a, int pass, int kset, size_t kslot, int64_t cgroups, hipStream_t stream);

}  // namespace exl3
