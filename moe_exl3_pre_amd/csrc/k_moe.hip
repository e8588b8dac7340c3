// MoE expert-bank forward ("dspark/worker/exl3/bank.py", `Exl3Bank`: one layer's experts in K-sorted
// physical slots, trellis words in two flat int16 banks, w13 = [w1 | w3] per slot; "vLLM PR #190":
// every expert projection is an EXL3 linear with input suh + Hadamard-128 and output Hadamard-128 + svh).
//
//   out[t] = bf16( sum_j topk_w[t, j] * E_{topk_ids[t, j]}(x[t]) ),   E(v) = L_w2( silu(L_w1 v) * L_w3 v )
//
// Four launches, all sized from host-known quantities so the call is graph-capturable:
//   1. route + rotate.  Workgroup 0 sorts the (token, slot) pairs by slot with a counting sort (pair ids
//      ascending inside a slot on the bitmap path; any order on the general path, which no result
//      depends on) and cuts every slot's list into chunks of at most 32 rows.
//      Every other workgroup rotates gathered activations for w1 and w3 of each pair
//      (x[t] * suh, Hadamard-128, fp16, PERM16 order) -- that needs only the pair's slot, not the sort.
//   2. w13.  One workgroup per (chunk, 128-column block of I): two waves stream w1's trellis words and
//      two stream w3's, each decoding tile columns in registers straight into MFMA operands against up
//      to 32 gathered rows.  The epilogue has h1 and h3 of the same 128 intermediate features, so it
//      applies both output Hadamards and svh, forms a = silu(h1) * h3, applies w2's suh and w2's input
//      Hadamard (the same 128-feature block) and writes w2's fp16 operand: the intermediate never goes
//      to HBM in fp32 and needs no pre-pass of its own.
//   3. w2.  One workgroup per (chunk, pair of 128-column blocks of H): same streaming core; output
//      Hadamard and svh; fp32 result per pair.
//   4. combine.  out[t] = sum over j in top-k order, one bf16 rounding.
// Every intermediate is indexed by pair id q = t * topk + j, so only the w13/w2 row lists depend on the
// sort.  Reductions run in a fixed order, so results are deterministic.
#include <type_traits>

#include "exl3_device.hpp"
#include "exl3_internal.hpp"
#include "k_moe.hpp"

namespace exl3 {

constexpr int kMoeRows = 32;          // rows of one chunk: two 16-row MFMA groups per decoded operand
constexpr int kMoeWaves = 4;          // waves per w13 / w2 workgroup: two per half
constexpr int kRedStride = kHad + 4;  // padded fp32 row of the reduction buffers (spreads LDS banks)
constexpr int kRouteThreads = 1024;
static_assert(kMoeMaxExperts <= kRouteThreads && kMoeMaxGroups <= kRouteThreads,
              "the route keeps one slot and one K group per thread");
// w13 / w2 workgroups: the reduction buffer [2 halves][32 rows][kRedStride] and, before it is used, the
// four waves' trellis staging slots share one LDS array
constexpr int kMoeRedFloats = 2 * kMoeRows * kRedStride;
constexpr int kMoeSlotFloats = kMoeWaves * Slot<8>::kBytes / 4;
constexpr int kMoeLdsFloats = kMoeRedFloats > kMoeSlotFloats ? kMoeRedFloats : kMoeSlotFloats;


// Slot of pair q, or -1 when its id is outside [0, E) or the permutation entry is.
__device__ __forceinline__ int pair_slot(const MoeArgs& a, int q) {
  const int e = a.ids[q];
  if (e < 0 || e >= a.E) return -1;
  const int s = a.perm[e];
  return (s >= 0 && s < a.E) ? s : -1;
}

// ---------------------------------------------------------------------------------------------------
// 1a. Route: counting sort of the pairs by slot, done by one workgroup of 1024 threads.
// ---------------------------------------------------------------------------------------------------
// Exclusive scan of v over the block's 1024 threads; returns the prefix and leaves the total in *total.
// tmp holds 48 ints of LDS.
// Inclusive prefix sum over the 64 lanes of a wave with DPP (no LDS round trips): shifts by 1, 2, 4 and 8
// inside each row of 16 lanes, then the last lane of rows 0 and 2 added to rows 1 and 3 and lane 31 added
// to rows 2 and 3.  Lanes without a source lane add the zero old value.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 into rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v);
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kRouteThreads / 64 ? tmp[lane] : 0;
    const int winc = wave_incl_scan(w);
    if (lane < kRouteThreads / 64) tmp[16 + lane] = winc - w;   // exclusive wave offsets
    if (lane == 15) tmp[32] = winc;
  }
  __syncthreads();
  const int r = tmp[16 + wave] + inc - v;
  *total = tmp[32];
  __syncthreads();
  return r;
}

constexpr int kSlotCache = 16384;   // pairs whose slots the route keeps in LDS between its two passes
constexpr int kRouteBatch = 16;     // pairs per thread whose loads the general route issues together

__device__ void moe_route_general(const MoeArgs& a, int* lds) {
  const int tid = threadIdx.x;
  const int E = a.E;
  int* cnt = lds;                 // [E]
  int* next = cnt + E;            // [E] next free row of each slot
  int* perm_l = next + E;         // [E] the slot of each logical expert
  int* tmp = perm_l + E;          // [48]
  int* cache = a.P <= kSlotCache ? tmp + 48 : nullptr;   // [P] slot per pair
  for (int s = tid; s < E; s += kRouteThreads) {
    cnt[s] = 0;
    perm_l[s] = a.perm[s];
  }
  __syncthreads();
  // slots and counts, kRouteBatch pairs per thread at a time: every id of a batch is requested before
  // the first is used, so a batch costs one memory latency, not one per pair
  constexpr int kStride = kRouteThreads * kRouteBatch;
  for (int q0 = 0; q0 < a.P; q0 += kStride) {
    int e[kRouteBatch];
#pragma unroll
    for (int k = 0; k < kRouteBatch; ++k) {
      const int q = q0 + k * kRouteThreads + tid;
      e[k] = q < a.P ? a.ids[q] : -1;
    }
#pragma unroll
    for (int k = 0; k < kRouteBatch; ++k) {
      const int q = q0 + k * kRouteThreads + tid;
      int s = (e[k] >= 0 && e[k] < E) ? perm_l[e[k]] : -1;
      s = (s >= 0 && s < E) ? s : -1;
      if (q < a.P) {
        a.pslot[q] = s;
        if (cache) cache[q] = s;
        if (s >= 0) atomicAdd(&cnt[s], 1);
      }
    }
  }
  __syncthreads();
  // slot offsets and chunk offsets (E <= 1024: one slot per thread)
  const int s = tid;
  const int c = s < E ? cnt[s] : 0;
  int total = 0, chunk_total = 0;
  const int off = block_excl_scan(c, tmp, &total);
  const int nch = (c + a.chunk_rows - 1) / a.chunk_rows;
  const int coff = block_excl_scan(nch, tmp, &chunk_total);
  if (s < E) {
    a.offs[s] = off;
    next[s] = off;
    int gk = 0;
    for (int g = 0; g < a.n_groups; ++g)
      if (s < a.g_hi[g]) {
        gk = a.g_k[g];
        break;
      }
    for (int i = 0; i < nch; ++i) {
      const int r0 = off + i * a.chunk_rows;
      const int nr = c - i * a.chunk_rows < a.chunk_rows ? c - i * a.chunk_rows : a.chunk_rows;
      a.chunks[chunk_total - 1 - (coff + i)] = (int4v){s, r0, nr, gk};   // heaviest first (moe_chunk)
    }
  }
  if (s == 0) {
    a.offs[E] = total;
    a.n_chunks[0] = chunk_total;
  }
  // placement: one LDS atomic per pair on its slot's cursor.  The order inside a slot is whatever the
  // atomics give; nothing depends on it (every row of the w13 / w2 lists is computed on its own and every
  // result is indexed by pair id), so the outputs are the same bits as with a stable order.  The slots
  // come back from the LDS cache or from pslot, which this thread wrote above (the barrier's fence has
  // made those stores visible; no earlier load put their lines in the L1).
  __syncthreads();
  for (int q0 = 0; q0 < a.P; q0 += kStride) {
    int sl[kRouteBatch];
#pragma unroll
    for (int k = 0; k < kRouteBatch; ++k) {
      const int q = q0 + k * kRouteThreads + tid;
      sl[k] = q < a.P ? (cache ? cache[q] : a.pslot[q]) : -1;
    }
#pragma unroll
    for (int k = 0; k < kRouteBatch; ++k)
      if (sl[k] >= 0) a.rows[atomicAdd(&next[sl[k]], 1)] = q0 + k * kRouteThreads + tid;
  }
}

// Fast path of the route when one bit per (slot, pair) and every pair's slot fit in LDS (bitmap_route_fits):
// the pairs set bits of a [slot][P/32] bitmap, one wave per slot turns its row into exclusive popcount
// prefixes, and a pair's position in its slot's list is the number of set bits before it -- the same stable
// order (pair ids ascending inside a slot) without any serial pass.
constexpr int kBitmapWords = 8192;
constexpr int kBitmapSlotCache = 8192;   // pairs whose slots the bitmap route keeps in LDS
static_assert(kBitmapSlotCache % kRouteThreads == 0, "whole batches of expert ids per thread");

__host__ __device__ inline bool bitmap_route_fits(int E, int P) {
  return int64_t(E) * ((P + 31) / 32) <= kBitmapWords && P <= kBitmapSlotCache;
}

__device__ void moe_route_bitmap(const MoeArgs& a, int* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int kW = kRouteThreads / 64;
  // Every kernel argument the route reads is requested here, together: the first read of each argument
  // line is a memory round trip, and requested at first use they would cost one per phase.
  const int* ids = a.ids;
  const int* perm = a.perm;
  int *pslot = a.pslot, *offs = a.offs, *rows = a.rows, *n_chunks = a.n_chunks;
  int4v* chunks = a.chunks;
  const int P = a.P, E = a.E, chunk_rows = a.chunk_rows, n_groups = a.n_groups;
  asm volatile("" ::"s"(ids), "s"(perm), "s"(pslot), "s"(offs), "s"(rows), "s"(n_chunks), "s"(chunks), "s"(P),
               "s"(E), "s"(chunk_rows), "s"(n_groups));
  const int W = (P + 31) / 32;
  uint32_t* bm = reinterpret_cast<uint32_t*>(lds);   // [E][W]
  int* pre = lds + E * W;                             // [E][W] exclusive prefix of popcounts
  int* cnt = pre + E * W;                             // [E]
  int* tmp = cnt + E;                                 // [48]
  int* perm_l = tmp + 48;                             // [E] the slot of each logical expert
  int* grp = perm_l + E;                              // [2][kMoeMaxGroups] the K groups' end slots and K
  int* slot_of = grp + 2 * kMoeMaxGroups;             // [P] (P <= kBitmapSlotCache on this path)
  // The slot table, the group table and (when they fit in LDS) every expert id are requested before the
  // first of them is stored, so the phase waits out one memory latency (E <= kRouteThreads).  The loads
  // are unconditional, with clamped indices: a load under a branch makes the compiler wait for it before
  // the next batch.
  const int pv = perm[tid < E ? tid : E - 1];
  const int gt = tid < kMoeMaxGroups ? tid : kMoeMaxGroups - 1;
  const int gh = a.g_hi[gt], gkv = a.g_k[gt];
  {                                                   // P <= kBitmapSlotCache: one batch, no loop
    constexpr int kIds = kBitmapSlotCache / kRouteThreads;
    int v[kIds];
#pragma unroll
    for (int k = 0; k < kIds; ++k) {
      const int q = k * kRouteThreads + tid;
      v[k] = ids[q < P ? q : P - 1];
    }
#pragma unroll
    for (int k = 0; k < kIds; ++k) {
      const int q = k * kRouteThreads + tid;
      if (q < P) slot_of[q] = v[k];
    }
    if (tid < E) perm_l[tid] = pv;
  }
  if (tid < n_groups) {
    grp[tid] = gh;
    grp[kMoeMaxGroups + tid] = gkv;
  }
  for (int i = tid; i < E * W; i += kRouteThreads) bm[i] = 0u;
  __syncthreads();
  for (int q = tid; q < P; q += kRouteThreads) {
    const int e = slot_of[q];
    int s = (e >= 0 && e < E) ? perm_l[e] : -1;
    s = (s >= 0 && s < E) ? s : -1;
    slot_of[q] = s;
    if (s >= 0) atomicOr(&bm[s * W + (q >> 5)], 1u << (q & 31));
  }
  __syncthreads();
  if (W <= 64) {
    // Rows of up to 64 words: 8 lanes per slot, 8 consecutive words per lane, 8 slots per wave in one
    // pass.  A lane's words take local popcount prefixes; the lane totals are scanned inside each 8-lane
    // segment (DPP shifts by 1, 2 and 4 within the row of 16 lanes, added only from lanes of the same
    // segment).  The prefixes are those of the per-slot scan below.
    const int seg = lane & 7;
    for (int s0 = 8 * wave; s0 < E; s0 += 8 * kW) {
      const int s = s0 + (lane >> 3);
      const int j0 = 8 * seg;
      int pc[8], tot = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pc[i] = tot;
        tot += (s < E && j0 + i < W) ? __popc(bm[s * W + j0 + i]) : 0;
      }
      int inc = tot;
      int t = __builtin_amdgcn_update_dpp(0, inc, 0x111, 0xF, 0xF, false);   // row_shr:1
      inc += seg >= 1 ? t : 0;
      t = __builtin_amdgcn_update_dpp(0, inc, 0x112, 0xF, 0xF, false);       // row_shr:2
      inc += seg >= 2 ? t : 0;
      t = __builtin_amdgcn_update_dpp(0, inc, 0x114, 0xF, 0xF, false);       // row_shr:4
      inc += seg >= 4 ? t : 0;
      const int ex = inc - tot;
      if (s < E) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (j0 + i < W) pre[s * W + j0 + i] = ex + pc[i];
        if (seg == 7) cnt[s] = inc;
      }
    }
  } else {
    for (int s = wave; s < E; s += kW) {
      int carry = 0;
      for (int j0 = 0; j0 < W; j0 += 64) {
        const int j = j0 + lane;
        const int v = j < W ? __popc(bm[s * W + j]) : 0;
        const int inc = wave_incl_scan(v);
        if (j < W) pre[s * W + j] = carry + inc - v;
        carry += __builtin_amdgcn_readlane(inc, 63);
      }
      if (lane == 0) cnt[s] = carry;
    }
  }
  __syncthreads();
  const int s = tid;
  const int c = s < E ? cnt[s] : 0;
  int total = 0, chunk_total = 0;
  const int off = block_excl_scan(c, tmp, &total);
  const int nch = (c + chunk_rows - 1) / chunk_rows;
  const int coff = block_excl_scan(nch, tmp, &chunk_total);
  int gk = 0;
  if (s < E) {
    cnt[s] = off;                                     // from here on: first row of the slot
    for (int g = 0; g < n_groups; ++g)
      if (s < grp[g]) {
        gk = grp[kMoeMaxGroups + g];
        break;
      }
  }
  __syncthreads();
  // The route's global stores all come after its last barrier: a store still in flight at a barrier makes
  // the compiler wait for it there as soon as a register it reads is reused.
  for (int q = tid; q < P; q += kRouteThreads) {
    const int sl = slot_of[q];                       // this thread wrote it above
    pslot[q] = sl;
    if (sl >= 0) {
      const int w = sl * W + (q >> 5);
      rows[cnt[sl] + pre[w] + __popc(bm[w] & ((1u << (q & 31)) - 1u))] = q;
    }
  }
  if (s < E) {
    offs[s] = off;
    for (int i = 0; i < nch; ++i) {
      const int r0 = off + i * chunk_rows;
      const int nr = c - i * chunk_rows < chunk_rows ? c - i * chunk_rows : chunk_rows;
      chunks[chunk_total - 1 - (coff + i)] = (int4v){s, r0, nr, gk};   // heaviest first (moe_chunk)
    }
  }
  if (s == 0) {
    offs[E] = total;
    n_chunks[0] = chunk_total;
  }
}

__device__ void moe_route(const MoeArgs& a, int* lds) {
  if (bitmap_route_fits(a.E, a.P))
    moe_route_bitmap(a, lds);
  else
    moe_route_general(a, lds);
}

// ---------------------------------------------------------------------------------------------------
// 1b. Rotation of gathered activations for w1 and w3.  One wave per (token, 128-block, two groups of 8
// rows), the rows being the token's (pair, projection) combinations (pair j = row / 2, projection row % 2):
// lane (n, g) holds row n's features 16g .. 16g+15 of the block (the x chunk is the same for every row,
// the sign vector is the pair's expert's).  Hadamard-128: register butterflies over feature bits 0..3,
// a row-rotate DPP exchange over bit 4 (lane bit 3) and lane-pair swaps over bits 5 and 6 (lane bits 4
// and 5), then each lane writes its 16-group as 32 contiguous bytes of the PERM16 layout.  Two groups per
// wave: the token's x chunk is loaded once, and the launch's workgroups (every one of which reserves the
// route's LDS) stay within what the chip holds at once (at top-8 one group per wave would need 513).
// ---------------------------------------------------------------------------------------------------
constexpr int kRotGroups = 2;   // groups of 8 rows one rotation wave transforms

inline int64_t moe_rotate_units(int64_t T, int H, int topk) {
  const int nrh = (topk + 3) / 4;                          // groups of 8 rows: 2 * topk rows per token
  return T * (H / kHad) * ((nrh + kRotGroups - 1) / kRotGroups);
}

__device__ void moe_rotate(const MoeArgs& a, int64_t unit) {
  const int lane = threadIdx.x & 63, n = lane & 7, g = lane >> 3;
  const int nblk = a.H / kHad;
  const int nrh = (a.topk + 3) / 4;                        // groups of 8 rows: 2 * topk rows per token
  const int nru = (nrh + kRotGroups - 1) / kRotGroups;     // this wave: groups kRotGroups * ru + k
  const int64_t tb = unit / nru;
  const int ru = int(unit % nru);
  const int t = int(tb / nblk), hb = int(tb % nblk);
  if (t >= a.T) return;
  const int f = hb * kHad + 16 * g;
  const u32x4* xp = reinterpret_cast<const u32x4*>(a.x + int64_t(t) * a.H + f);
  const u32x4 xv[2] = {xp[0], xp[1]};                      // the token's chunk serves every group
  // every group's sign-scale chunk is loaded before any arithmetic (the wave is latency-bound otherwise)
  int jj[kRotGroups], sl[kRotGroups];
  u32x4 sv[kRotGroups][2];
  const int proj = n & 1;
#pragma unroll
  for (int k = 0; k < kRotGroups; ++k) {
    const int rh = ru * kRotGroups + k;
    jj[k] = rh * 4 + (n >> 1);
    sl[k] = rh < nrh && jj[k] < a.topk ? pair_slot(a, t * a.topk + jj[k]) : -1;
    const int sc = sl[k] < 0 ? 0 : sl[k];
    const u32x4* sp = reinterpret_cast<const u32x4*>(a.w13_suh + int64_t(sc * 2 + proj) * a.H + f);
    sv[k][0] = sp[0];
    sv[k][1] = sp[1];
  }
#pragma unroll
  for (int k = 0; k < kRotGroups; ++k) {
    if (ru * kRotGroups + k >= nrh) break;                 // wave-uniform
    float v[16];
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int sh = (w & 1) * 16;
      v[w] = bf16_to_f32((xv[w >> 3][(w >> 1) & 3] >> sh) & 0xFFFFu) *
             f16_to_f32(uint16_t(sv[k][w >> 3][(w >> 1) & 3] >> sh));
    }
#pragma unroll
    for (int b = 1; b < 16; b <<= 1)                       // feature bits 0..3
#pragma unroll
      for (int w = 0; w < 16; ++w)
        if (!(w & b)) {
          const float lo = v[w], hi = v[w | b];
          v[w] = lo + hi;
          v[w | b] = lo - hi;
        }
    float q[16];
#pragma unroll
    for (int w = 0; w < 16; ++w) q[w] = dpp<kRowRor8>(v[w]);  // bit 4: lane xor 8 within each row of 16
#pragma unroll
    for (int w = 0; w < 16; ++w) v[w] = bfly(v[w], q[w], lane & 8);
#pragma unroll
    for (int w = 0; w < 16; w += 2) lane_pair_bfly<false>(v[w], v[w + 1]);   // bit 5: lane bit 4
#pragma unroll
    for (int w = 0; w < 16; w += 2) lane_pair_bfly<true>(v[w], v[w + 1]);    // bit 6: lane bit 5
    if (sl[k] >= 0) {
      const int64_t qi = int64_t(t) * a.topk + jj[k];
      u32x4* dst = reinterpret_cast<u32x4*>(a.xh13 + (int64_t(proj) * a.P + qi) * a.ldx + f);
      u32x4 o0, o1;                                        // PERM16: positions (2i, 2i+1) hold features (i, i+8)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o0[i] = rot_f16x2(v[i], v[i + 8]);
        o1[i] = rot_f16x2(v[i + 4], v[i + 12]);
      }
      dst[0] = o0;
      dst[1] = o1;
    }
  }
}

__global__ __launch_bounds__(kRouteThreads, 8) void moe_route_rotate_kernel(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) int route_lds[];
  if (blockIdx.x == 0) {
    // the route is the launch's long pole: its waves take issue priority over the rotation waves
    // sharing their CU
    __builtin_amdgcn_s_setprio(3);
    moe_route(a, route_lds);
    return;
  }
  const int64_t unit = int64_t(blockIdx.x - 1) * (kRouteThreads / 64) + (threadIdx.x >> 6);
  moe_rotate(a, unit);
}

// ---------------------------------------------------------------------------------------------------
// Streaming core: one wave accumulates rows x [128 columns] over its 64-feature steps [st0, st0 + nst)
// of one expert projection.  Each step's trellis words arrive as K coalesced 16-byte loads per lane
// (PD steps in flight), are staged in the wave's LDS slot, and every lane then reads its tile column's
// words from there (one column ahead) and decodes them into MFMA operands.  The A fragments of the next
// step are loaded one step ahead.  Loads are unconditional with clamped steps (every address stays
// inside the tensor); only the arithmetic and the staging are predicated.  LDS operations of one wave
// complete in order, so a step's reads see that step's writes.
// ---------------------------------------------------------------------------------------------------
template <int K>
__device__ __forceinline__ void moe_accumulate(const uint16_t* code, uint32_t code_bytes, int tpr, int blk,
                                               const uint16_t* arow0, const uint16_t* arow1, int st0, int nst,
                                               bool two, char* slot, float4v (&acc0)[8], float4v (&acc1)[8]) {
  using G = Geom<K>;
  constexpr int PD = K <= 3 ? 2 : 1;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  int woff[G::kNW], shift;
  column_word_offsets<K>(n, woff, shift);
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(wave_uniform(code)), (short)0,
                                        (int)wave_uniform(code_bytes), kBufferFlags);
  const uint32_t lane_off = uint32_t(g) * uint32_t(tpr) * G::kWords * 4u + uint32_t(n) * 16u;
  const uint32_t step_stride = 4u * uint32_t(tpr) * G::kWords * 4u;
  const uint32_t base_blk = uint32_t(blk) * 8u * G::kWords * 4u;
  const int last = st0 + (nst > 0 ? nst - 1 : 0);
  char* my_row = slot + g * Slot<K>::kRowBytes;

  u32x4 tb[PD][K];
  half8 A[2][2][2];   // [ring][row group][k half]
  auto load_step = [&](int st, u32x4 (&dst)[K]) {
    const uint32_t soff = uint32_t(st < last ? st : last) * step_stride + base_blk;
#pragma unroll
    for (int i = 0; i < K; ++i)
      dst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane_off + uint32_t(i * 256), soff, 0));
  };
  auto load_a = [&](int st, half8 (&dst)[2][2]) {
    const int o = 64 * (st < last ? st : last);
    dst[0][0] = *reinterpret_cast<const half8*>(arow0 + o);
    dst[0][1] = *reinterpret_cast<const half8*>(arow0 + o + 8);
    dst[1][0] = *reinterpret_cast<const half8*>(arow1 + o);
    dst[1][1] = *reinterpret_cast<const half8*>(arow1 + o + 8);
  };
  auto read_col = [&](int j, uint32_t (&dst)[G::kNW]) {
#pragma unroll
    for (int w = 0; w < G::kNW; ++w) dst[w] = *reinterpret_cast<const uint32_t*>(my_row + (j * G::kWords + woff[w]) * 4);
  };
  load_a(st0, A[0]);
#pragma unroll
  for (int p = 0; p < PD; ++p) load_step(st0 + p, tb[p]);
  __builtin_amdgcn_sched_barrier(0);

  const CodebookRegs cb = codebook_regs();
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    acc0[j] = (float4v){0.f, 0.f, 0.f, 0.f};
    acc1[j] = (float4v){0.f, 0.f, 0.f, 0.f};
  }
  for (int s = 0; s < nst; s += 2) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int st = s + p;
      load_a(st0 + st + 1, A[(p + 1) & 1]);
      const bool live = st < nst;
      if (live) {
        lane_exchange_fence();                              // the previous step's reads come first
#pragma unroll
        for (int i = 0; i < K; ++i) *reinterpret_cast<u32x4*>(my_row + (i * 16 + n) * 16) = tb[p % PD][i];
        lane_exchange_fence();                              // this step's reads see these words
      }
      load_step(st0 + st + PD, tb[p % PD]);
      if (live) {
        uint32_t wv[2][G::kNW];
        read_col(0, wv[0]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (j + 1 < 8) read_col(j + 1, wv[(j + 1) & 1]);
          uint32_t b[8];
          decode_column<K>(wv[j & 1], shift, b, cb);
          const half8 b0 = as_half8(b[0], b[1], b[2], b[3]);
          const half8 b1 = as_half8(b[4], b[5], b[6], b[7]);
          acc0[j] = mfma16(A[p][0][0], b0, acc0[j]);
          acc0[j] = mfma16(A[p][0][1], b1, acc0[j]);
          if (two) {
            acc1[j] = mfma16(A[p][1][0], b0, acc1[j]);
            acc1[j] = mfma16(A[p][1][1], b1, acc1[j]);
          }
        }
      }
    }
  }
}

// Fixed-order sum of the two waves of one half into red [32][kRedStride]: wave 0 stores, wave 1 adds.
__device__ __forceinline__ void moe_reduce(float* red, int wq, bool two, const float4v (&acc0)[8],
                                           const float4v (&acc1)[8]) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  for (int turn = 0; turn < 2; ++turn) {
    if (wq == turn) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* p0 = red + (4 * g + r) * kRedStride + 16 * j + n;
          float* p1 = red + (16 + 4 * g + r) * kRedStride + 16 * j + n;
          if (turn == 0) {
            *p0 = acc0[j][r];
            if (two) *p1 = acc1[j][r];
          } else {
            *p0 += acc0[j][r];
            if (two) *p1 += acc1[j][r];
          }
        }
    }
    __syncthreads();
  }
}

template <int K>
__device__ __forceinline__ void moe_w13_block(const MoeArgs& a, const int4v ch, int cb, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = wave >> 1, wq = wave & 1, n = lane & 15, g = lane >> 4;
  const int slot = ch[0], row0 = ch[1], nrows = ch[2];
  const bool two = nrows > 16;
  const int NS = a.H / 64;
  const int st0 = NS * wq / 2, st1 = NS * (wq + 1) / 2;
  const int64_t off = h == 0 ? a.off_w1[slot] : a.off_w3[slot];
  const uint16_t* A = a.xh13 + int64_t(h) * a.P * a.ldx;
  const int r0 = a.rows[row0 + (n < nrows ? n : nrows - 1)];
  const int r1 = a.rows[row0 + (16 + n < nrows ? 16 + n : nrows - 1)];
  float4v acc0[8], acc1[8];
  moe_accumulate<K>(a.w13 + off, uint32_t(int64_t(a.H) * a.I * K / 8), a.I / 16, cb, A + int64_t(r0) * a.ldx + 16 * g,
                    A + int64_t(r1) * a.ldx + 16 * g, st0, st1 - st0, two,
                    reinterpret_cast<char*>(red) + wave * Slot<K>::kBytes, acc0, acc1);
  __syncthreads();                               // the staging slots share LDS with the reduction buffer
  moe_reduce(red + h * kMoeRows * kRedStride, wq, two, acc0, acc1);

  // epilogue: lane l owns intermediate features f, f + 8 of this block (PERM16 positions 2l, 2l+1)
  const int f = perm_pair_feature(lane);
  const int64_t col = int64_t(cb) * kHad + f;
  const uint16_t* svh1 = a.w13_svh + (int64_t(slot) * 2 + 0) * a.I + col;
  const uint16_t* svh3 = a.w13_svh + (int64_t(slot) * 2 + 1) * a.I + col;
  const uint16_t* suh2 = a.w2_suh + int64_t(slot) * a.I + col;
  const float s1a = f16_to_f32(svh1[0]), s1b = f16_to_f32(svh1[8]);
  const float s3a = f16_to_f32(svh3[0]), s3b = f16_to_f32(svh3[8]);
  const float u2a = f16_to_f32(suh2[0]), u2b = f16_to_f32(suh2[8]);
  for (int r = wave; r < nrows; r += kMoeWaves) {
    const float* p1 = red + r * kRedStride;
    const float* p3 = red + (kMoeRows + r) * kRedStride;
    float h1a = p1[f], h1b = p1[f + 8], h3a = p3[f], h3b = p3[f + 8];
    had128_wave(h1a, h1b, lane);
    had128_wave(h3a, h3b, lane);
    h1a *= kInvSqrt128 * s1a;
    h1b *= kInvSqrt128 * s1b;
    h3a *= kInvSqrt128 * s3a;
    h3b *= kInvSqrt128 * s3b;
    float va = h1a / (1.0f + __expf(-h1a)) * h3a * u2a;
    float vb = h1b / (1.0f + __expf(-h1b)) * h3b * u2b;
    had128_wave(va, vb, lane);
    uint16_t* dst = a.ah + int64_t(a.rows[row0 + r]) * a.ldh + int64_t(cb) * kHad + 2 * lane;
    *reinterpret_cast<uint32_t*>(dst) = rot_f16x2(va, vb);
  }
}

template <int K>
__device__ __forceinline__ void moe_w2_block(const MoeArgs& a, const int4v ch, int cbp, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = wave >> 1, wq = wave & 1, n = lane & 15, g = lane >> 4;
  const int slot = ch[0], row0 = ch[1], nrows = ch[2];
  const bool two = nrows > 16;
  const int nblk = a.H / kHad;
  const int cb = 2 * cbp + h;
  const bool active = cb < nblk;                 // an odd last column block leaves half 1 idle
  const int NS = a.I / 64;
  const int st0 = NS * wq / 2, st1 = active ? NS * (wq + 1) / 2 : st0;
  const int r0 = a.rows[row0 + (n < nrows ? n : nrows - 1)];
  const int r1 = a.rows[row0 + (16 + n < nrows ? 16 + n : nrows - 1)];
  float4v acc0[8], acc1[8];
  moe_accumulate<K>(a.w2 + a.off_w2[slot], uint32_t(int64_t(a.I) * a.H * K / 8), a.H / 16, active ? cb : 0,
                    a.ah + int64_t(r0) * a.ldh + 16 * g, a.ah + int64_t(r1) * a.ldh + 16 * g, st0, st1 - st0, two,
                    reinterpret_cast<char*>(red) + wave * Slot<K>::kBytes, acc0, acc1);
  __syncthreads();                               // the staging slots share LDS with the reduction buffer
  float* rh = red + h * kMoeRows * kRedStride;
  moe_reduce(rh, wq, two, acc0, acc1);
  if (!active) return;
  const int64_t c0 = int64_t(cb) * kHad + 2 * lane;
  const float sa = f16_to_f32(a.w2_svh[int64_t(slot) * a.H + c0]);
  const float sb = f16_to_f32(a.w2_svh[int64_t(slot) * a.H + c0 + 1]);
  for (int r = wq; r < nrows; r += 2) {
    float v0 = rh[r * kRedStride + 2 * lane], v1 = rh[r * kRedStride + 2 * lane + 1];
    had128_wave(v0, v1, lane);
    float* dst = a.o + int64_t(a.rows[row0 + r]) * a.H + c0;
    *reinterpret_cast<float2*>(dst) = make_float2(v0 * kInvSqrt128 * sa, v1 * kInvSqrt128 * sb);
  }
}

template <int KSET>
__global__ __launch_bounds__(kMoeWaves * 64, 3) void moe_w13_kernel(MoeArgs a) {
  __shared__ __attribute__((aligned(16))) float red[kMoeLdsFloats];
  int c, cb;
  moe_tile(a.I / kHad, c, cb);
  int4v ch;
  if (!moe_chunk(a, c, ch)) return;
  moe_dispatch<KSET>(ch[3] & 0xFF, [&](auto k) { moe_w13_block<decltype(k)::value>(a, ch, cb, red); });
}

template <int KSET>
__global__ __launch_bounds__(kMoeWaves * 64) void moe_w2_kernel(MoeArgs a) {
  __shared__ __attribute__((aligned(16))) float red[kMoeLdsFloats];
  int c, cbp;
  moe_tile((a.H / kHad + 1) / 2, c, cbp);
  int4v ch;
  if (!moe_chunk(a, c, ch)) return;
  moe_dispatch<KSET>(ch[3] >> 8, [&](auto k) { moe_w2_block<decltype(k)::value>(a, ch, cbp, red); });
}

// ---------------------------------------------------------------------------------------------------
// 4. Combine: one thread per (token, 4 columns); sum over j in top-k order in fp32, one bf16 rounding.
// ---------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void moe_combine_kernel(MoeArgs a) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int per_row = a.H / 4;
  if (i >= int64_t(a.T) * per_row) return;
  const int t = int(i / per_row), c = int(i % per_row) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  constexpr int kB = 8;   // terms whose loads are issued together
  for (int j0 = 0; j0 < a.topk; j0 += kB) {
    float w[kB];
    float4 v[kB];
    // Every term's row, slot and weight are requested before any is used: the loads are unconditional
    // (q < P, always inside the workspace and the weight array), and the selections come after them.  A
    // dropped pair's row was never written and is replaced by exact zeros.
    float4 raw[kB];
    int sl[kB];
    float wv[kB];
#pragma unroll
    for (int r = 0; r < kB; ++r) {
      const int j = j0 + r < a.topk ? j0 + r : a.topk - 1;
      const int q = t * a.topk + j;
      raw[r] = *reinterpret_cast<const float4*>(a.o + int64_t(q) * a.H + c);
      sl[r] = a.pslot[q];
      wv[r] = a.wts[q];
    }
#pragma unroll
    for (int r = 0; r < kB; ++r) {
      const bool use = j0 + r < a.topk && sl[r] >= 0;
      w[r] = use ? wv[r] : 0.f;
      v[r] = use ? raw[r] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int r = 0; r < kB; ++r) {   // top-k order; a dropped term adds exactly zero
      acc.x += w[r] * v[r].x;
      acc.y += w[r] * v[r].y;
      acc.z += w[r] * v[r].z;
      acc.w += w[r] * v[r].w;
    }
  }
  const uint32_t lo = f32_to_bf16(acc.x) | (f32_to_bf16(acc.y) << 16);
  const uint32_t hi = f32_to_bf16(acc.z) | (f32_to_bf16(acc.w) << 16);
  *reinterpret_cast<uint2*>(a.out + int64_t(t) * a.H + c) = make_uint2(lo, hi);
}

// ---------------------------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------------------------
int64_t moe_max_chunks(int64_t P, int E) { return (P + kMoeRows - 1) / kMoeRows + E; }

bool moe_prefill_plan(int64_t P, int E, int H, int I, int plan) {
  const bool fits = P * int64_t(moe_row_pitch(H > I ? H : I)) * 2 < (int64_t(1) << 31);
  if (plan == 1 || !fits) return false;
  return plan == 2 || P >= int64_t(kMoePrefillPairsPerExpert) * E;
}

static size_t moe_slot_bytes(unsigned ks) {   // staging slot of the largest K in the bit set
  int kmax = 1;
  for (int k = 1; k <= 8; ++k)
    if (ks & (1u << k)) kmax = k;
  return size_t(4) * (256 * kmax + 64);
}

static size_t moe_route_lds_bytes(int E, int P) {
  const size_t words = size_t(E) * ((P + 31) / 32);
  if (bitmap_route_fits(E, P)) return (2 * words + 2 * E + 48 + 2 * kMoeMaxGroups + size_t(P)) * sizeof(int);
  return size_t(3 * E + 48 + (P <= kSlotCache ? P : 0)) * sizeof(int);
}

hipError_t launch_moe(const MoeLaunch& m, hipStream_t stream) {
  MoeArgs a;
  a.x = (const uint16_t*)m.x;
  a.ids = m.ids;
  a.wts = m.wts;
  a.perm = m.perm;
  a.w13 = (const uint16_t*)m.w13;
  a.w2 = (const uint16_t*)m.w2;
  a.w13_suh = (const uint16_t*)m.w13_suh;
  a.w13_svh = (const uint16_t*)m.w13_svh;
  a.w2_suh = (const uint16_t*)m.w2_suh;
  a.w2_svh = (const uint16_t*)m.w2_svh;
  a.off_w1 = m.off_w1;
  a.off_w3 = m.off_w3;
  a.off_w2 = m.off_w2;
  a.out = (uint16_t*)m.out;
  a.offs = m.offs;
  a.pslot = m.pslot;
  a.rows = m.rows;
  a.chunks = (int4v*)m.chunks;
  a.n_chunks = m.n_chunks;
  a.xh13 = (uint16_t*)m.xh13;
  a.ah = (uint16_t*)m.ah;
  a.o = m.o;
  a.T = int(m.T);
  a.topk = m.topk;
  a.P = int(m.T * m.topk);
  a.E = m.E;
  a.H = m.H;
  a.I = m.I;
  a.max_chunks = int(moe_max_chunks(a.P, m.E));
  a.ldx = moe_row_pitch(a.H);
  a.ldh = moe_row_pitch(a.I);
  a.n_groups = m.n_groups;
  for (int g = 0; g < kMoeMaxGroups; ++g) {
    a.g_hi[g] = g < m.n_groups ? m.g_hi[g] : 0;
    a.g_k[g] = g < m.n_groups ? m.g_k[g] : 0;
  }
  const bool prefill = moe_prefill_plan(a.P, a.E, a.H, a.I, m.plan);
  a.chunk_rows = prefill ? kTileRows : kMoeRows;
  const int64_t rot_units = moe_rotate_units(a.T, a.H, a.topk);
  const int64_t rot_blocks = (rot_units + kRouteThreads / 64 - 1) / (kRouteThreads / 64);
  hipLaunchKernelGGL(moe_route_rotate_kernel, dim3(unsigned(1 + rot_blocks)), dim3(kRouteThreads),
                     moe_route_lds_bytes(a.E, a.P), stream, a);
  // chunk slots of the grid (moe_tile); the prefill plan's chunks of kTileRows number at most P / kTileRows + E
  const int64_t nch = prefill ? (int64_t(a.P) + kTileRows - 1) / kTileRows + a.E : a.max_chunks;
  const int64_t cgroups = moe_chunk_slots(nch);
  const dim3 g13(unsigned(cgroups * (a.I / kHad))), g2(unsigned(cgroups * ((a.H / kHad + 1) / 2)));
  for (int pass = 0; pass < 2; ++pass) {
    // the K values of this projection, as a bit set
    unsigned ks = 0;
    for (int g = 0; g < m.n_groups; ++g) ks |= 1u << (pass == 0 ? (m.g_k[g] & 0xFF) : (m.g_k[g] >> 8));
    auto go = [&](auto kset) {
      constexpr int KS = decltype(kset)::value;
      if (prefill) {
        // (chunk, column group) tiles; chunk groups of 8 as in moe_tile, and the chunks past the
        // route's count exit at once
        launch_moe_tile_pass(a, pass, KS, KS == 0 ? moe_slot_bytes(0x1Cu) : moe_slot_bytes(1u << KS), cgroups, stream);
      } else if (pass == 0) {
        hipLaunchKernelGGL(moe_w13_kernel<KS>, g13, dim3(kMoeWaves * 64), 0, stream, a);
      } else {
        hipLaunchKernelGGL(moe_w2_kernel<KS>, g2, dim3(kMoeWaves * 64), 0, stream, a);
      }
    };
    if ((ks & ~0x1Cu) == 0) {
      go(std::integral_constant<int, 0>{});
    } else {
      if (ks & (1u << 1)) go(std::integral_constant<int, 1>{});
      if (ks & (1u << 2)) go(std::integral_constant<int, 2>{});
      if (ks & (1u << 3)) go(std::integral_constant<int, 3>{});
      if (ks & (1u << 4)) go(std::integral_constant<int, 4>{});
      if (ks & (1u << 5)) go(std::integral_constant<int, 5>{});
      if (ks & (1u << 6)) go(std::integral_constant<int, 6>{});
      if (ks & (1u << 7)) go(std::integral_constant<int, 7>{});
      if (ks & (1u << 8)) go(std::integral_constant<int, 8>{});
    }
  }
  const int64_t comb = (int64_t(a.T) * (a.H / 4) + 255) / 256;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(unsigned(comb)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace exl3
